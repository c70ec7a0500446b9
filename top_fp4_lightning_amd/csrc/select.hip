// Exact top-k selection (k <= 2048) over rows of fp32 values, ranked by (value desc, index asc).
//
// Every element gets a unique 64-bit composite c = (key << 32) | ~pos, where key is the fp32
// bit pattern mapped to an order-preserving uint32 and pos the element's reported index; -inf
// and NaN never enter the selection. The top k are exactly the elements with c >= T. T is found
// by radix passes of 11 bits over the composites of a short candidate list: a lower bound of the
// k-th key, taken from wavefront maxima, admits a few percent of a row as candidates (details
// above the candidate filter below).
//
// The winners are written in ascending position order (the natural order for gathering the
// selected keys afterwards):
//  - rows of at most 16384 values: one block per row (256, 512 or 1024 threads), 16 values per
//    thread in registers (one launch); the candidates sit in LDS in slot order and the winners
//    are written in that order, which is position order when the optional block map is
//    ascending (as the pool and this function produce);
//  - longer rows (candidate pool over 2^17 block maxima, full score rows): three launches over
//    chunks of 4096 values (bound, collect, finish; ordered by kernel boundaries, no cross-block
//    fences or waits); the finishing block orders the winners by position.
// A row may also be read through a pool's block list from a full score row (map_values): slot
// 8i + r holds the value at position 8 * block_i + r, so the top-k restricted to the pooled
// blocks needs neither a masked copy of the row nor the long-row launches.
#include "internal.h"

namespace fp4idx {
namespace {

constexpr int kSmallRow = 16384;
constexpr int kPadBins = kHistBins + kHistBins / 32;
constexpr int64_t kBitmapMax = (int64_t)1 << 18;  // pool rows up to this many blocks use the bitmap

__device__ __forceinline__ int hidx(int b) { return b + (b >> 5); }

// order-preserving key of a float; -0 and +0 share the key of +0 (equal values tie, and ties go
// to the lower index)
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    u = u == 0x80000000u ? 0u : u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}
// finite or +inf; excludes -inf (0x007fffff) and NaN (keys above +inf's 0xff800000)
__device__ __forceinline__ bool eligible(uint32_t k) { return k > 0x007fffffu && k <= 0xff800000u; }
__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t pos) {
    return ((uint64_t)key << 32) | (uint64_t)(~pos);
}
__device__ __forceinline__ uint32_t comp_pos(uint64_t c) { return ~(uint32_t)c; }
__device__ __forceinline__ uint32_t comp_key(uint64_t c) { return (uint32_t)(c >> 32); }

__host__ __device__ inline size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline int64_t row_cap(const SelectArgs& a) {
    if (a.map_values) return a.map_width * kBlock;
    return a.pool_mode ? (a.max_n + kBlock - 1) / kBlock : a.max_n;
}

struct RowInfo {
    int64_t len;  // values in this row
    int64_t pin;  // pinned element (pool mode) or -1
    int64_t n;    // visible positions of the score row (map_values)
};

__device__ __forceinline__ RowInfo row_info(const SelectArgs& a, int64_t t) {
    int64_t n = a.nv ? (int64_t)a.nv[t] : a.max_n;
    n = n < 0 ? 0 : (n > a.max_n ? a.max_n : n);
    RowInfo ri;
    ri.n = n;
    if (a.map_values) {
        int64_t c = a.map_count[t / a.map_group];
        c = c < 0 ? 0 : (c > a.map_width ? a.map_width : c);
        ri.len = c * kBlock;
        ri.pin = -1;
    } else if (a.pool_mode) {
        ri.len = (n + kBlock - 1) / kBlock;
        ri.pin = (a.pin && n > 0) ? (n - 1) / kBlock : -1;
    } else {
        ri.len = n;
        ri.pin = -1;
    }
    return ri;
}

__device__ __constant__ int kShift[6] = {53, 42, 31, 20, 9, 0};
__device__ __constant__ int kWidth[6] = {11, 11, 11, 11, 11, 9};

struct Sel {
    int digit;
    uint32_t above;
};

// ---- wave-private histograms: hw[wave][1024] words, two 16-bit bins per word ----
template <int NT>
struct Hist {
    static constexpr int kWaves = NT / 64;
    uint32_t hw[kWaves][kHistBins / 2];
    uint32_t h[kPadBins];  // summed histogram, bin b at hidx(b)
};

template <int NT>
__device__ __forceinline__ void hist_clear_own(Hist<NT>& H) {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < kHistBins / 2 / 64; ++i) H.hw[w][l + 64 * i] = 0u;
}

// Histogram increments from the active lanes of a wavefront. When every active lane hits the
// same bin (rows of ties, or a pass over bits the candidates share) one lane adds the count:
// same-address atomics from a whole wavefront would otherwise serialise.
template <int NT>
__device__ __forceinline__ void hist_add(Hist<NT>& H, uint32_t digit) {
    uint32_t* hw = H.hw[threadIdx.x >> 6];
    const uint64_t act = __ballot(1);
    const uint32_t d0 = __builtin_amdgcn_readfirstlane(digit);
    if (__ballot(digit == d0) == act) {
        if ((uint32_t)(threadIdx.x & 63) == (uint32_t)(__ffsll((unsigned long long)act) - 1))
            atomicAdd(&hw[d0 >> 1], (uint32_t)__popcll(act) << (16 * (d0 & 1)));
    } else {
        atomicAdd(&hw[digit >> 1], 1u << (16 * (digit & 1)));
    }
}

__device__ __forceinline__ void bin_add(uint32_t* h, uint32_t bin) {
    const uint64_t act = __ballot(1);
    const uint32_t b0 = __builtin_amdgcn_readfirstlane(bin);
    if (__ballot(bin == b0) == act) {
        if ((uint32_t)(threadIdx.x & 63) == (uint32_t)(__ffsll((unsigned long long)act) - 1)) atomicAdd(&h[b0], (uint32_t)__popcll(act));
    } else {
        atomicAdd(&h[bin], 1u);
    }
}

template <int NT>
__device__ __forceinline__ void hist_reduce(Hist<NT>& H) {
    for (int b = threadIdx.x; b < kHistBins; b += NT) {
        uint32_t s = 0;
#pragma unroll
        for (int w = 0; w < Hist<NT>::kWaves; ++w) s += (H.hw[w][b >> 1] >> (16 * (b & 1))) & 0xffffu;
        H.h[hidx(b)] = s;
    }
}

// Threshold digit of the padded histogram h: the largest d with sum_{b >= d} h[b] >= need
// (d = -1 when the total is below need); `above` = count in bins above d. Computed by one whole
// wavefront (lane l owns bins [32l, 32l + 32)); every lane returns the result.
__device__ Sel wave_threshold(const uint32_t* h, uint32_t need) {
    const int lane = threadIdx.x & 63;
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) s += h[33 * lane + j];
    uint32_t suf = s;  // inclusive suffix sum over lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_down(suf, off);
        if (lane + off < 64) suf += o;
    }
    const uint32_t total = __shfl(suf, 0);
    if (total < need) return Sel{-1, total};
    const uint64_t own = __ballot(suf - s < need && need <= suf);
    const int L = __ffsll((unsigned long long)own) - 1;
    const uint32_t aboveL = __shfl(suf - s, L);
    const uint32_t v = lane < 32 ? h[33 * L + lane] : 0u;
    uint32_t vs = v;  // inclusive suffix over lanes 0..31
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) {
        const uint32_t o = __shfl_down(vs, off);
        if (lane + off < 32) vs += o;
    }
    const bool hit = lane < 32 && aboveL + vs >= need && aboveL + vs - v < need;
    const uint64_t hm = __ballot(hit);
    const int J = __ffsll((unsigned long long)hm) - 1;
    return Sel{32 * L + J, aboveL + __shfl(vs - v, J)};
}

// the same, computed by wave 0 for the whole block; ends with a barrier
__device__ void block_threshold(const uint32_t* h, uint32_t need, Sel& sel) {
    if (threadIdx.x < 64) {
        const Sel r = wave_threshold(h, need);
        if (threadIdx.x == 0) sel = r;
    }
    __syncthreads();
}

// One radix pass over the elements delivered by `each` (a callable that invokes its argument
// on every composite of this thread); returns true and sets T when the selection is complete.
template <int NT, class Each>
__device__ bool radix_pass(Each each, int p, uint32_t& need, uint64_t& prefix, uint64_t& mask, uint64_t& T,
                           Hist<NT>& H, Sel& sel) {
    const int shf = kShift[p];
    const uint64_t dm = ((uint64_t)1 << kWidth[p]) - 1;
    __syncthreads();
    hist_clear_own(H);
    each([&](uint64_t c) {
        if (c != 0 && ((c ^ prefix) & mask) == 0) hist_add(H, (uint32_t)((c >> shf) & dm));
    });
    __syncthreads();
    hist_reduce(H);
    __syncthreads();
    block_threshold(H.h, need, sel);
    const int d = sel.digit;
    const uint32_t above = sel.above;
    if (d < 0) {  // fewer than `need` present: take every eligible element
        T = 1ull;
        return true;
    }
    if (H.h[hidx(d)] == need - above) {
        T = prefix | ((uint64_t)d << shf);
        return true;
    }
    need -= above;
    prefix |= (uint64_t)d << shf;
    mask |= dm << shf;
    if (p == 5) {
        T = prefix;
        return true;
    }
    return false;
}

__device__ __forceinline__ uint64_t cmpx(uint64_t v, uint64_t p, bool keep_min) {
    return keep_min ? (v < p ? v : p) : (v < p ? p : v);
}

// ascending bitonic sort of s[0..N) (N a power of two <= 2048) by NT threads; element i lives in
// thread i % NT, register slot i / NT.
template <int NT>
__device__ void block_sort(uint64_t* s, int N) {
    constexpr int Q = kMaxK / NT;
    const int tid = threadIdx.x;
    uint64_t v[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) v[q] = tid + q * NT < N ? s[tid + q * NT] : 0ull;
    for (int size = 2; size <= N; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride >= NT) {
                const int qs = stride / NT;
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    if (q & qs) continue;
                    const int i = tid + q * NT;
                    const bool up = (i & size) == 0;
                    const uint64_t x = v[q], y = v[q | qs];
                    v[q] = cmpx(x, y, up);
                    v[q | qs] = cmpx(x, y, !up);
                }
            } else if (stride >= 64) {
                __syncthreads();
#pragma unroll
                for (int q = 0; q < Q; ++q)
                    if (tid + q * NT < N) s[tid + q * NT] = v[q];
                __syncthreads();
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    const int i = tid + q * NT;
                    if (i < N) {
                        const int j = i ^ stride;
                        v[q] = cmpx(v[q], s[j], (i < j) == ((i & size) == 0));
                    }
                }
            } else {
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    const int i = tid + q * NT;
                    const uint64_t p = __shfl_xor(v[q], stride);
                    const int j = i ^ stride;
                    if (i < N) v[q] = cmpx(v[q], p, (i < j) == ((i & size) == 0));
                }
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < Q; ++q)
        if (tid + q * NT < N) s[tid + q * NT] = v[q];
    __syncthreads();
}

__device__ __forceinline__ void write_one(const SelectArgs& a, int64_t t, int slot, uint64_t c) {
    a.out_idx[t * a.out_stride + slot] = (int32_t)comp_pos(c);
    if (a.out_val && !a.pool_mode) a.out_val[t * a.out_stride + slot] = key_value(comp_key(c));
}

__device__ __forceinline__ void write_pad(const SelectArgs& a, int64_t t, uint32_t cnt) {
    for (int i = (int)cnt + threadIdx.x; i < a.pad_to; i += blockDim.x) {
        a.out_idx[t * a.out_stride + i] = -1;
        if (a.out_val && !a.pool_mode) a.out_val[t * a.out_stride + i] = -INFINITY;
    }
    if (a.out_count && threadIdx.x == 0) a.out_count[t] = (int32_t)cnt;
}

// ---------------------------------------------------------------- candidate filter and list radix
// Rows are read as runs of 8 consecutive slots: in a block of NT threads, thread tid holds the
// values of slots c0 + 8 * (tid + r * NT) + e (run r < 2, e < 8) as floats in registers, -inf
// past the row and +inf for the pinned block, plus the position of each run's first slot (block
// map entry * 8, or the slot itself). Work per value is a handful of instructions:
//  1. A lower bound T0 of the k-th largest key. A wavefront with at least R eligible lanes
//     contributes the R-th largest of its lanes' maxima; when the contributing wavefronts number
//     at least k / R, at least k values lie at or above the smallest contribution, T0.
//     (Without enough contributions T0 = 0 and every eligible value is a candidate.)
//  2. The values at or above T0 (a few percent of a row) become candidates, stored as
//     (value bits, ~position).
//  3. Radix passes over the candidates find T: the first digit starts below the bits that T0 and
//     the row maximum share; passes stop when the threshold digit holds exactly the elements
//     still needed, or at most 64 of them, which are then ranked against each other in parallel.
//  4. The candidates >= T are the winners.
constexpr int kRuns = 2;
constexpr int kRunSlots = 8 * kRuns;  // values per thread
constexpr int kSelRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format, range checked

// inclusive prefix over the 64 lanes of a wavefront with lane moves inside the data-parallel-
// primitive network: shifts by 1, 2, 4, 8 within each row of 16 lanes, then row 0's last lane
// into row 1 (and row 2's into row 3), then lane 31 into rows 2 and 3
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_or_zero(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, true);
}
__device__ __forceinline__ uint32_t wave_incl_add(uint32_t v) {
    v += dpp_or_zero<0x111, 0xF>(v);
    v += dpp_or_zero<0x112, 0xF>(v);
    v += dpp_or_zero<0x114, 0xF>(v);
    v += dpp_or_zero<0x118, 0xF>(v);
    v += dpp_or_zero<0x142, 0xA>(v);
    v += dpp_or_zero<0x143, 0xC>(v);
    return v;
}
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t wave_incl_max(uint32_t v) {
    v = umax(v, dpp_or_zero<0x111, 0xF>(v));
    v = umax(v, dpp_or_zero<0x112, 0xF>(v));
    v = umax(v, dpp_or_zero<0x114, 0xF>(v));
    v = umax(v, dpp_or_zero<0x118, 0xF>(v));
    v = umax(v, dpp_or_zero<0x142, 0xA>(v));
    v = umax(v, dpp_or_zero<0x143, 0xC>(v));
    return v;
}

// exclusive prefix of one value per thread over the block, and the block total, with one
// barrier: wavefront totals go to wsum, and every thread adds up the totals it needs. wsum must
// not be rewritten before every thread has passed the next barrier (callers alternate buffers).
template <int NT>
__device__ __forceinline__ uint32_t block_scan(uint32_t x, uint32_t* wsum, uint32_t& total) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint32_t v = wave_incl_add(x);
    if (lane == 63) wsum[w] = v;
    __syncthreads();
    uint32_t pre = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const uint32_t u = wsum[i];
        tot += u;
        pre += i < w ? u : 0u;
    }
    total = tot;
    return pre + v - x;
}

__device__ __forceinline__ uint64_t list_entry(float v, uint32_t pos) {
    return ((uint64_t)__float_as_uint(v) << 32) | (uint64_t)(~pos);
}
__device__ __forceinline__ uint64_t entry_composite(uint64_t x) {
    return ((uint64_t)order_key(__uint_as_float((uint32_t)(x >> 32))) << 32) | (x & 0xffffffffull);
}

// the 8 values of a run at byte offset off; values past the descriptor's range read as 0 (the
// compiler merges the eight dword loads into two 16-byte loads)
__device__ __forceinline__ void load_run(__amdgpu_buffer_rsrc_t rv, uint32_t off, float (&v)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rv, (int)(off + 4u * e), 0, 0));
}

template <int NT>
__device__ __forceinline__ void chunk_load(const SelectArgs& a, int64_t t, const RowInfo& ri, int64_t c0,
                                           float (&v)[kRuns][8], uint32_t (&pb)[kRuns]) {
    const int64_t rem64 = ri.len - c0;
    const int rem = rem64 < (int64_t)(kRunSlots * NT) ? (int)rem64 : kRunSlots * NT;
    const int tid = threadIdx.x;
    if (a.map_values) {
        // block ids, then the 8 values of each block from the score row; ids outside the row's
        // blocks and positions past n_t read as -inf (the loads are issued unconditionally, range
        // checked by the descriptors, and the invalid ones replaced afterwards)
        const int32_t* mrow = a.map + (t / a.map_group) * a.map_stride + c0 / kBlock;
        const __amdgpu_buffer_rsrc_t rm =
            __builtin_amdgcn_make_buffer_rsrc((void*)mrow, 0, ((rem + kBlock - 1) / kBlock) * 4, kSelRsrcWord3);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a.vals + t * a.stride), 0, (int)(ri.n * 4), kSelRsrcWord3);
        const uint32_t nb = (uint32_t)((ri.n + kBlock - 1) / kBlock), n = (uint32_t)ri.n;
        bool okb[kRuns];
#pragma unroll
        for (int r = 0; r < kRuns; ++r) {
            const uint32_t id = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rm, (tid + r * NT) * 4, 0, 0);
            okb[r] = id < nb;
            pb[r] = okb[r] ? id * (uint32_t)kBlock : 0u;
        }
#pragma unroll
        for (int r = 0; r < kRuns; ++r) load_run(rv, pb[r] * 4u, v[r]);
#pragma unroll
        for (int r = 0; r < kRuns; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (!(okb[r] && pb[r] + (uint32_t)e < n)) v[r][e] = -INFINITY;
    } else {
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a.vals + t * a.stride + c0), 0, rem * 4, kSelRsrcWord3);
#pragma unroll
        for (int r = 0; r < kRuns; ++r) load_run(rv, (uint32_t)(8 * (tid + r * NT)) * 4u, v[r]);
    }
    if (a.map && !a.map_values) {
        const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a.map + t * a.map_stride + c0 / kBlock), 0, ((rem + kBlock - 1) / kBlock) * 4, kSelRsrcWord3);
#pragma unroll
        for (int r = 0; r < kRuns; ++r)
            pb[r] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rm, (tid + r * NT) * 4, 0, 0) * (uint32_t)kBlock;
    } else if (!a.map_values) {
#pragma unroll
        for (int r = 0; r < kRuns; ++r) pb[r] = (uint32_t)(c0 + 8 * (tid + r * NT));
    }
#pragma unroll
    for (int r = 0; r < kRuns; ++r) {
        const int nvalid = rem - 8 * (tid + r * NT);
        if (nvalid < 8) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (e >= nvalid) v[r][e] = -INFINITY;
        }
    }
    if (ri.pin >= c0 && ri.pin < c0 + rem) {  // the block of the newest position counts as +inf
        const int p = (int)(ri.pin - c0);
        const int pr = p >> 3;
        if (pr % NT == tid) {
#pragma unroll
            for (int r = 0; r < kRuns; ++r)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (pr / NT == r && (p & 7) == e) v[r][e] = INFINITY;
        }
    }
}

// key of the thread's M-th largest eligible value (ties count separately); 0 when the thread holds
// fewer than M eligible values. Keys, not floats, so that -inf and NaN are never counted.
template <int M>
__device__ __forceinline__ uint32_t lane_mth(const float (&v)[kRuns][8]) {
    uint32_t m[M];
#pragma unroll
    for (int i = 0; i < M; ++i) m[i] = 0u;
#pragma unroll
    for (int r = 0; r < kRuns; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t k = order_key(v[r][e]);
            uint32_t x = eligible(k) ? k : 0u;
#pragma unroll
            for (int i = 0; i < M; ++i) {  // insert x into the descending m[0..M)
                const uint32_t hi = max(m[i], x);
                x = min(m[i], x);
                m[i] = hi;
            }
        }
    return m[M - 1];
}

// key of the thread's largest value; 0 when the thread holds no eligible value
__device__ __forceinline__ uint32_t lane_max(const float (&v)[kRuns][8]) {
    float fm = v[0][0];
#pragma unroll
    for (int r = 0; r < kRuns; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) fm = fmaxf(fm, v[r][e]);
    const uint32_t k = order_key(fm);
    return eligible(k) ? k : 0u;
}

// the R-th largest lo key of the wavefront's lanes, to its top 16 bits (0 when fewer than R
// lanes hold an eligible value)
__device__ __forceinline__ uint32_t wave_rth(uint32_t lo, uint32_t R) {
    uint32_t t = 0u;
    for (int b = 31; b >= 16; --b) {
        const uint32_t tr = t | (1u << b);
        if ((uint32_t)__popcll(__ballot(lo >= tr)) >= R) t = tr;
    }
    return t;
}

// For t = wave_rth(lo, R) the R-th largest lane key lies in t's 16-bit bucket: the bucket's
// smallest key is at least t and at most that key, and equal to it when the bucket holds a single
// value, as on rows of tied values. Valid in lane 63; 0 stays 0.
__device__ __forceinline__ uint32_t bucket_floor(uint32_t lo, uint32_t t) {
    const uint32_t m = ~wave_incl_max(t && (lo >> 16) == (t >> 16) ? ~lo : 0u);
    return t ? m : 0u;
}

// R for a row of `waves` wavefronts of which at least `waves / share` contribute
__device__ __forceinline__ uint32_t bound_rank(uint32_t k, int64_t waves, int share) {
    const int64_t r = waves > 0 ? ((int64_t)share * k + waves - 1) / waves : 64;
    return (uint32_t)(r < 1 ? 1 : (r > 64 ? 64 : r));
}

template <int NT>
struct RadixShared {
    uint32_t wsum[2][NT / 64];
    uint32_t red[2][NT / 64];
    int digit;
    uint32_t above, nfin;
    uint64_t T;
    uint64_t fin[64];
    uint32_t rk[64];
};

constexpr uint32_t kInfKey = 0xff800000u;  // order key of +inf

// T for the candidates L[0 .. C) (C > k, at least k of them with keys >= T0); hist holds two
// 2048-bin scratch histograms (passes alternate between them, so that clearing the next one
// needs no barrier of its own). Called by the whole block; contains barriers. +inf entries (the
// pinned block, +inf values) are counted first and kept out of the passes. Each pass splits the
// composite range [rlo, rhi) that holds the threshold into 2048 equal bins of 2^sh (the first
// range runs from T0 to the largest finite key, so that its bins spread the candidates thinly);
// a bin whose entries all win ends the search, and a bin of at most 64 entries is ranked directly.
template <int NT>
__device__ uint64_t list_radix(const uint64_t* L, uint32_t C, uint32_t k, uint32_t T0, uint32_t* hist,
                               RadixShared<NT>& S) {
    constexpr int NW = NT / 64;
    constexpr int B = kHistBins / NT;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (tid == 0) {
        S.digit = 0;
        S.above = 0u;
        S.T = 1ull;
        S.nfin = 0u;
    }
    if (tid < 64) S.rk[tid] = 0u;
    for (int b = tid; b < kHistBins; b += NT) hist[b] = 0u;  // the first pass's histogram
    uint32_t km = 0u, ni = 0u;
    for (uint32_t i = tid; i < C; i += NT) {
        const uint32_t kk = order_key(__uint_as_float((uint32_t)(L[i] >> 32)));
        if (kk >= kInfKey)
            ++ni;
        else
            km = kk > km ? kk : km;
    }
    km = wave_incl_max(km);
    ni = wave_incl_add(ni);
    if (lane == 63) {
        S.red[0][w] = km;
        S.red[1][w] = ni;
    }
    __syncthreads();
    km = 0u;
    ni = 0u;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        km = S.red[0][i] > km ? S.red[0][i] : km;
        ni += S.red[1][i];
    }
    uint32_t need = k;
    uint64_t rlo, rhi;  // the threshold composite lies in [rlo, rhi)
    if (ni >= need) {   // among the +inf entries: positions decide
        rlo = (uint64_t)kInfKey << 32;
        rhi = rlo + (1ull << 32);
    } else {
        need -= ni;
        rlo = (uint64_t)T0 << 32;
        rhi = ((uint64_t)km + 1ull) << 32;  // km < kInfKey: no overflow
    }
    int sb = 0;
    for (int pass = 0;; ++pass) {
        // the fewest bits per bin that cover the range with 2048 bins
        const uint64_t span1 = rhi - rlo - 1ull;
        const int bits = span1 ? 64 - __clzll((long long)span1) : 0;
        const int sh = bits > 11 ? bits - 11 : 0;
        uint32_t* h = hist + (pass & 1) * kHistBins;
        for (uint32_t i = tid; i < C; i += NT) {
            const uint64_t x = entry_composite(L[i]);
            if (x >= rlo && x < rhi) bin_add(h, (uint32_t)((x - rlo) >> sh));
        }
        __syncthreads();
        // every thread is past the previous pass's reads of the other histogram: clear it for
        // the next pass (two more barriers separate this from the next pass's adds)
        for (int b = tid; b < kHistBins; b += NT) hist[((pass + 1) & 1) * kHistBins + b] = 0u;
        {  // threshold digit: thread tid owns bins kHistBins - 1 - (B * tid + j), j < B
            uint32_t c[B], sum = 0;
#pragma unroll
            for (int j = 0; j < B; ++j) {
                c[j] = h[kHistBins - 1 - (B * tid + j)];
                sum += c[j];
            }
            uint32_t tot;
            const uint32_t ex = block_scan<NT>(sum, S.wsum[sb], tot);
            sb ^= 1;
            if (ex < need && need <= ex + sum) {
                uint32_t acc = ex;
#pragma unroll
                for (int j = 0; j < B; ++j) {
                    if (acc + c[j] >= need) {
                        S.digit = kHistBins - 1 - (B * tid + j);
                        S.above = acc;
                        break;
                    }
                    acc += c[j];
                }
            }
            __syncthreads();
        }
        const int d = S.digit;
        const uint32_t above = S.above;
        const uint32_t on = h[d];
        const uint64_t blo = rlo + ((uint64_t)d << sh);
        if (on == need - above) return blo;
        need -= above;
        const uint64_t bhi = blo + (1ull << sh);  // blo < rhi <= 0xff80000100000000, sh <= 53: no overflow
        rlo = blo;
        rhi = bhi < rhi ? bhi : rhi;
        if (on <= 64 || sh == 0) break;
    }
    // the few elements in the bin, ranked against each other (counters cleared at the start)
    for (uint32_t i = tid; i < C; i += NT) {
        const uint64_t x = entry_composite(L[i]);
        if (x >= rlo && x < rhi) {
            const uint32_t f = atomicAdd(&S.nfin, 1u);
            if (f < 64u) S.fin[f] = x;
        }
    }
    __syncthreads();
    const uint32_t nf = S.nfin < 64u ? S.nfin : 64u;
    constexpr int per = (64 + NW - 1) / NW;
    if ((uint32_t)lane < nf) {
        const uint64_t xi = S.fin[lane];
        uint32_t rank = 0;
#pragma unroll
        for (int jj = 0; jj < per; ++jj) {
            const uint32_t j = (uint32_t)(w * per + jj);
            if (j < nf && S.fin[j] > xi) ++rank;
        }
        if (rank) atomicAdd(&S.rk[lane], rank);
    }
    __syncthreads();
    if ((uint32_t)tid < nf && S.rk[tid] == need - 1) S.T = S.fin[tid];
    __syncthreads();
    return S.T;
}

// ---------------------------------------------------------------- rows of <= 16 * NT values
// One block per row, all four steps in registers and LDS. When R > 128 would be needed or the
// candidates overflow the list, the radix passes run over the registers instead (wave-private
// histograms) and the winners are compacted from the registers.
template <int NT, bool WIDE>
struct SmallShared {
    // candidate list capacity. WIDE (launched when k needs more than 64 values per wavefront and
    // the row is longer than the narrow list) keeps three times as many entries, enough for the
    // looser bound of k = 2048 on a full row; the narrow list keeps the output step short
    static constexpr int kCap = (WIDE ? 12 : 4) * NT;
    union {
        Hist<NT> H;  // register passes
        struct {
            uint64_t list[kCap];
            uint32_t hist[2 * kHistBins];
        } L;
    };
    RadixShared<NT> R;
    uint32_t wt0[NT / 64];   // each wavefront's contribution to T0
    uint32_t wout[NT / 64];  // scan buffer of the output step
    Sel sel;
};

template <int NT, bool WIDE>
__global__ __launch_bounds__(NT) void select_small_kernel(SelectArgs a) {
    constexpr int NW = NT / 64;
    constexpr int kCap = SmallShared<NT, WIDE>::kCap;
    __shared__ SmallShared<NT, WIDE> S;
    const int64_t t = blockIdx.x;
    const RowInfo ri = row_info(a, t);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    float v[kRuns][8];
    uint32_t pb[kRuns];
    chunk_load<NT>(a, t, ri, 0, v, pb);

    // 1. T0 (every wavefront must contribute here). Each wavefront needs R values at or above
    // its contribution: the R-th largest of its lanes' maxima, or in the wide form for
    // 64 < R <= 128 the ceil(R / 4)-th largest of its lanes' fourth-largest values (four values
    // per such lane; a middle lane's fourth value bounds tighter than the lowest lane's second)
    const uint32_t R = ((uint32_t)a.k + NW - 1) / NW;
    const uint32_t t0w = R <= 64 ? wave_rth(lane_max(v), R)
                                 : (WIDE && R <= 128 ? wave_rth(lane_mth<4>(v), (R + 3) / 4) : 0u);
    if (lane == 0) S.wt0[w] = t0w;
    __syncthreads();
    uint32_t T0 = S.wt0[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) T0 = S.wt0[i] < T0 ? S.wt0[i] : T0;
    const float fT = T0 ? key_value(T0) : -__FLT_MAX__;  // v >= fT: exactly the values with key >= T0

    // 2. candidates: counts per run, packed, one scan gives slot-order offsets
    uint32_t cr[kRuns];
#pragma unroll
    for (int r = 0; r < kRuns; ++r) {
        cr[r] = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) cr[r] += v[r][e] >= fT ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t ex = block_scan<NT>(cr[0] | (cr[1] << 16), S.R.wsum[0], tot);
    const uint32_t C = (tot & 0xffffu) + (tot >> 16);
    const uint32_t k = (uint32_t)a.k;
    uint64_t T = 1ull;  // every candidate
    uint32_t cnt;
    // Too many candidates: most of them tie (rows of equal values, a zero query). Each round
    // takes M, the smallest candidate's key, and counts the values strictly above it. Fewer than k
    // above it: M is the k-th value, and the winners are every value above it and the first ones
    // equal to it in slot order. Otherwise the next round looks at the values above M. A row left
    // unresolved (more levels of ties, or few enough values above M) takes the register passes.
    // The rounds keep their own copies so that the common path below stays as it is.
    if (__builtin_expect(C > (uint32_t)kCap && T0 != 0u, 0)) {
        float fL = fT;
        uint32_t exL = ex, totL = tot;
        for (int round = 0; round < 3; ++round) {
            uint32_t mk = 0xffffffffu;
#pragma unroll
            for (int r = 0; r < kRuns; ++r)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (v[r][e] >= fL) mk = min(mk, order_key(v[r][e]));
            const uint32_t wmax = wave_incl_max(~mk);  // the minimum as the maximum of complements
            if (lane == 63) S.R.red[0][w] = wmax;
            __syncthreads();
            uint32_t nmin = 0u;
#pragma unroll
            for (int i = 0; i < NW; ++i) nmin = S.R.red[0][i] > nmin ? S.R.red[0][i] : nmin;
            const uint32_t M = ~nmin;
            const float fM = key_value(M);
            uint32_t gr[kRuns];
#pragma unroll
            for (int r = 0; r < kRuns; ++r) {
                gr[r] = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) gr[r] += v[r][e] > fM ? 1u : 0u;
            }
            uint32_t totg;
            const uint32_t exg = block_scan<NT>(gr[0] | (gr[1] << 16), S.R.wsum[(round + 1) & 1], totg);
            const uint32_t Cg = (totg & 0xffffu) + (totg >> 16);
            if (Cg < k) {
                const uint32_t m = k - Cg;
                uint32_t gb[kRuns] = {exg & 0xffffu, (totg & 0xffffu) + (exg >> 16)};
                uint32_t tb[kRuns] = {(exL & 0xffffu) - (exg & 0xffffu),
                                      ((totL & 0xffffu) - (totg & 0xffffu)) + (exL >> 16) - (exg >> 16)};
#pragma unroll
                for (int r = 0; r < kRuns; ++r)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint64_t c = composite(order_key(v[r][e]), pb[r] + (uint32_t)e);
                        if (v[r][e] > fM) {
                            write_one(a, t, (int)(gb[r] + (tb[r] < m ? tb[r] : m)), c);
                            ++gb[r];
                        } else if (v[r][e] >= fL) {
                            if (tb[r] < m) write_one(a, t, (int)(gb[r] + tb[r]), c);
                            ++tb[r];
                        }
                    }
                write_pad(a, t, k);
                return;
            }
            if (Cg <= (uint32_t)kCap) break;
            fL = key_value(M + 1u);
            exL = exg;
            totL = totg;
        }
        __syncthreads();
    }
    if (C <= (uint32_t)kCap) {
        uint32_t o[kRuns] = {ex & 0xffffu, (tot & 0xffffu) + (ex >> 16)};
#pragma unroll
        for (int r = 0; r < kRuns; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (v[r][e] >= fT) S.L.list[o[r]++] = list_entry(v[r][e], pb[r] + (uint32_t)e);
        __syncthreads();
        // 3. radix passes over the list
        if (C > k) T = list_radix<NT>(S.L.list, C, k, T0, S.L.hist, S.R);
        // 4. list entries >= T, in list order: thread tid takes entries [Q * tid, Q * tid + Q)
        constexpr int Q = kCap / NT;
        uint64_t x[Q];
        uint32_t wm = 0, c = 0;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const uint32_t i = (uint32_t)(Q * tid + q);
            x[q] = i < C ? entry_composite(S.L.list[i]) : 0ull;
            const bool win = i < C && x[q] >= T;
            wm |= (win ? 1u : 0u) << q;
            c += win ? 1u : 0u;
        }
        uint32_t slot = block_scan<NT>(c, S.wout, cnt);
#pragma unroll
        for (int q = 0; q < Q; ++q)
            if ((wm >> q) & 1u) {
                if (slot < k) write_one(a, t, (int)slot, x[q]);
                ++slot;
            }
    } else {
        // register passes over the composites
        auto each = [&](auto&& f) {
#pragma unroll
            for (int r = 0; r < kRuns; ++r)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t kk = order_key(v[r][e]);
                    f(eligible(kk) ? composite(kk, pb[r] + (uint32_t)e) : 0ull);
                }
        };
        uint32_t need = k;
        uint64_t prefix = 0ull, mask = 0ull;
        for (int p = 0; p < 6; ++p)
            if (radix_pass<NT>(each, p, need, prefix, mask, T, S.H, S.sel)) break;
        uint32_t wr[kRuns] = {0, 0};
#pragma unroll
        for (int r = 0; r < kRuns; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t kk = order_key(v[r][e]);
                if (eligible(kk) && composite(kk, pb[r] + (uint32_t)e) >= T) wr[r] |= 1u << e;
            }
        __syncthreads();
        uint32_t tot2;
        const uint32_t ex2 = block_scan<NT>((uint32_t)__popc(wr[0]) | ((uint32_t)__popc(wr[1]) << 16), S.R.wsum[0],
                                            tot2);
        uint32_t o[kRuns] = {ex2 & 0xffffu, (tot2 & 0xffffu) + (ex2 >> 16)};
        cnt = (tot2 & 0xffffu) + (tot2 >> 16);
#pragma unroll
        for (int r = 0; r < kRuns; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if ((wr[r] >> e) & 1u) {
                    if (o[r] < k) write_one(a, t, (int)o[r], composite(order_key(v[r][e]), pb[r] + (uint32_t)e));
                    ++o[r];
                }
    }
    write_pad(a, t, cnt < k ? cnt : k);
}

// ---------------------------------------------------------------- longer rows
// Three launches over chunks of 4096 values (256 threads), ordered by kernel boundaries:
//   bound   - per chunk, for two ranks (R1 for every wavefront of the row contributing, R2 = 2 R1
//             for half of them, as in rows that are mostly -inf): the smallest contribution of
//             its wavefronts and their number, written to the chunk's slot of the workspace (no
//             atomics);
//   collect - every block reduces its row's chunk slots to T0 and appends its values at or above
//             T0 to the row's candidate list (one reservation atomic per block);
//   finish  - one block per row stages the candidates in LDS (when they fit), runs the radix
//             passes, orders the winners by position (LDS bitmap for pool block ids, else a
//             bitonic sort), writes them and clears the row's candidate count.
constexpr int kLargeThreads = 256;
constexpr int kChunk = kLargeThreads * kRunSlots;
constexpr int kFinishThreads = 1024;
constexpr int kFinishCap = 8192;  // candidates staged in LDS by the finishing block

struct ChunkBound {
    uint32_t t0[2];     // smallest contribution for R1, R2 (0xffffffff when none)
    uint32_t waves[2];  // contributing wavefronts
};

struct RowState {
    uint32_t n_cand;
    uint32_t t0;
    uint32_t pad[30];  // one 128-byte line per row
};

struct WsView {
    RowState* st;       // [nq]
    ChunkBound* bound;  // [nq][chunks]
    uint64_t* cand;     // [nq][cap]
    uint32_t* ties;     // [nq][chunks * kChunk / 32]: pool rows' values equal to the bound, as bits
    int64_t cap;
    int64_t chunks;
};

__host__ __device__ inline WsView ws_view(void* ws, int32_t nq, int64_t cap) {
    WsView v;
    v.cap = cap > 0 ? cap : 1;
    v.chunks = (v.cap + kChunk - 1) / kChunk;
    char* p = (char*)ws;
    v.st = (RowState*)p;
    p += align_up((size_t)nq * sizeof(RowState));
    v.bound = (ChunkBound*)p;
    p += align_up((size_t)nq * (size_t)v.chunks * sizeof(ChunkBound));
    v.cand = (uint64_t*)p;
    p += align_up((size_t)nq * (size_t)v.cap * 8);
    v.ties = (uint32_t*)p;
    return v;
}

__global__ __launch_bounds__(kLargeThreads) void select_bound_kernel(SelectArgs a, WsView ws) {
    constexpr int NW = kLargeThreads / 64;
    __shared__ uint32_t wt[2][NW];
    const int64_t t = blockIdx.y;
    const RowInfo ri = row_info(a, t);
    const int64_t c0 = (int64_t)blockIdx.x * kChunk;
    if (c0 >= ri.len) return;  // uniform per block
    float v[kRuns][8];
    uint32_t pb[kRuns];
    chunk_load<kLargeThreads>(a, t, ri, c0, v, pb);
    const uint32_t lm = lane_max(v);
    const int64_t chunks = (ri.len + kChunk - 1) / kChunk;
    // bucket floors: a row whose values tie at the bound then has the tied key itself as its bound
    // (the finishing block resolves such ties by position without a radix pass)
    const uint32_t t1 = bucket_floor(lm, wave_rth(lm, bound_rank((uint32_t)a.k, chunks * NW, 1)));
    const uint32_t t2 = bucket_floor(lm, wave_rth(lm, bound_rank((uint32_t)a.k, chunks * NW, 2)));
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 63) {
        wt[0][w] = t1;
        wt[1][w] = t2;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        ChunkBound cb{{0xffffffffu, 0xffffffffu}, {0u, 0u}};
#pragma unroll
        for (int i = 0; i < NW; ++i) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
                if (wt[j][i]) {
                    cb.t0[j] = wt[j][i] < cb.t0[j] ? wt[j][i] : cb.t0[j];
                    ++cb.waves[j];
                }
        }
        ws.bound[t * ws.chunks + blockIdx.x] = cb;
    }
}

// T0 of row t from its chunk bounds, by the whole block
template <int NT>
__device__ __forceinline__ uint32_t row_bound(const SelectArgs& a, const WsView& ws, int64_t t, int64_t chunks,
                                              uint32_t* red) {
    constexpr int NW = NT / 64;
    uint32_t t0[2] = {0xffffffffu, 0xffffffffu}, nw[2] = {0u, 0u};
    for (int64_t c = threadIdx.x; c < chunks; c += NT) {
        const ChunkBound cb = ws.bound[t * ws.chunks + c];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            t0[j] = cb.t0[j] < t0[j] ? cb.t0[j] : t0[j];
            nw[j] += cb.waves[j];
        }
    }
    // wavefront reductions (min as the max of complements), then across wavefronts
    const uint32_t r0 = wave_incl_max(~t0[0]), r1 = wave_incl_max(~t0[1]), r2 = wave_incl_add(nw[0]),
                   r3 = wave_incl_add(nw[1]);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 63) {
        red[w] = r0;
        red[NW + w] = r1;
        red[2 * NW + w] = r2;
        red[3 * NW + w] = r3;
    }
    __syncthreads();
    uint32_t n0 = 0u, n1 = 0u, c0 = 0u, c1 = 0u;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        n0 = red[i] > n0 ? red[i] : n0;
        n1 = red[NW + i] > n1 ? red[NW + i] : n1;
        c0 += red[2 * NW + i];
        c1 += red[3 * NW + i];
    }
    const int64_t waves = chunks * (kLargeThreads / 64);
    const uint64_t k = (uint64_t)a.k;
    if ((uint64_t)c0 * bound_rank(a.k, waves, 1) >= k) return ~n0;
    if ((uint64_t)c1 * bound_rank(a.k, waves, 2) >= k) return ~n1;
    return 0u;
}

__global__ __launch_bounds__(kLargeThreads) void select_collect_kernel(SelectArgs a, WsView ws) {
    constexpr int NW = kLargeThreads / 64;
    __shared__ uint32_t red[4 * NW];
    __shared__ uint32_t wsum[NW];
    __shared__ uint32_t base;
    const int64_t t = blockIdx.y;
    const RowInfo ri = row_info(a, t);
    const int64_t c0 = (int64_t)blockIdx.x * kChunk;
    if (c0 >= ri.len) return;  // uniform per block
    float v[kRuns][8];
    uint32_t pb[kRuns];
    chunk_load<kLargeThreads>(a, t, ri, c0, v, pb);
    const int64_t chunks = (ri.len + kChunk - 1) / kChunk;
    const uint32_t T0 = row_bound<kLargeThreads>(a, ws, t, chunks, red);
    if (blockIdx.x == 0 && threadIdx.x == 0) ws.st[t].t0 = T0;
    const float fT = T0 ? key_value(T0) : -__FLT_MAX__;
    // Pool rows (block maxima) keep the values equal to the bound out of the list, as bits by block
    // id: on rows of tied maxima (a zero query) the list stays short, and the finishing block takes
    // the ties it needs by block id. The chunk's words are written whole, ties or not.
    const bool split = a.pool_mode && T0 != 0u;
    uint32_t c = 0;
    uint32_t tm[kRuns] = {0u, 0u};
#pragma unroll
    for (int r = 0; r < kRuns; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const bool tie = split && v[r][e] == fT;  // -0 is +0 and NaN never equal: the key equals T0
            tm[r] |= (tie ? 1u : 0u) << e;
            c += v[r][e] >= fT && !tie ? 1u : 0u;
        }
    if (split) {
        // run r of thread tid is byte tid % 4 of word (c0 + 8 (tid + r NT)) / 32: four lanes per word
        const int tid = threadIdx.x;
        uint32_t* trow = ws.ties + t * ws.chunks * (kChunk / 32);
#pragma unroll
        for (int r = 0; r < kRuns; ++r) {
            uint32_t wb = tm[r] << (8 * (tid & 3));
            wb |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)wb, 0xB1, 0xF, 0xF, false);  // lane ^ 1
            wb |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)wb, 0x4E, 0xF, 0xF, false);  // lane ^ 2
            if ((tid & 3) == 0) trow[(c0 + 8 * (tid + r * kLargeThreads)) >> 5] = wb;
        }
    }
    uint32_t tot;
    uint32_t o = block_scan<kLargeThreads>(c, wsum, tot);
    if (threadIdx.x == 0) base = tot ? atomicAdd(&ws.st[t].n_cand, tot) : 0u;
    __syncthreads();
    uint64_t* out = ws.cand + t * ws.cap + base;
#pragma unroll
    for (int r = 0; r < kRuns; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (v[r][e] >= fT && !((tm[r] >> e) & 1u)) out[o++] = list_entry(v[r][e], pb[r] + (uint32_t)e);
}

__global__ __launch_bounds__(kFinishThreads) void select_finish_kernel(SelectArgs a, WsView ws) {
    __shared__ uint64_t list[kFinishCap];
    __shared__ uint32_t hist[2 * kHistBins];
    __shared__ RadixShared<kFinishThreads> S;
    __shared__ uint64_t out[kMaxK];
    __shared__ uint32_t bits[kBitmapMax / 32];
    const int64_t t = blockIdx.x;
    const uint32_t C = ws.st[t].n_cand, T0 = ws.st[t].t0;
    const uint32_t k = (uint32_t)a.k;
    const uint64_t* gc = ws.cand + t * ws.cap;
    const uint64_t* L = gc;
    const RowInfo ri = row_info(a, t);
    // pool ids leave through an LDS bitmap of the row's blocks: cleared before the first barrier
    const bool bitmap = a.pool_mode && ri.len <= kBitmapMax;
    const int words = bitmap ? (int)((ri.len + 31) / 32) : 0;
    for (int i = threadIdx.x; i < words; i += kFinishThreads) bits[i] = 0u;
    if (C <= (uint32_t)kFinishCap) {
        for (uint32_t i = threadIdx.x; i < C; i += kFinishThreads) list[i] = gc[i];
        L = list;
    }
    __syncthreads();
    // Pool rows with fewer than k list entries above the bound (T0 != 0): the bound is the k-th
    // value, and the winners are every list entry and the first k - C values equal to the bound,
    // taken by block id from the tie bitmap the collecting blocks wrote.
    const bool ties = bitmap && T0 != 0u && C < k;
    if (ties) {
        for (uint32_t i = threadIdx.x; i < C; i += kFinishThreads) {
            const uint32_t pos = comp_pos(entry_composite(L[i]));
            atomicOr(&bits[pos >> 5], 1u << (pos & 31));
        }
        const uint32_t* trow = ws.ties + t * ws.chunks * (kChunk / 32);
        const uint32_t m = k - C;
        const int per = (words + kFinishThreads - 1) / kFinishThreads;
        const int w0 = threadIdx.x * per;
        uint32_t mine = 0;
        for (int q = 0; q < per; ++q)
            if (w0 + q < words) mine += (uint32_t)__popc(trow[w0 + q]);
        uint32_t nt;
        uint32_t base = block_scan<kFinishThreads>(mine, S.wsum[1], nt);  // also orders the ORs above
        for (int q = 0; q < per && w0 + q < words && base < m; ++q) {
            uint32_t b = trow[w0 + q];
            const uint32_t c = (uint32_t)__popc(b);
            if (base + c > m) {  // keep the lowest m - base bits
                for (uint32_t drop = base + c - m; drop; --drop) b &= ~(1u << (31 - __clz(b)));
            }
            atomicOr(&bits[w0 + q], b);
            base += c;
        }
        __syncthreads();
    }
    const uint64_t T = (!ties && C > k) ? list_radix<kFinishThreads>(L, C, k, T0, hist, S) : 1ull;
    if (bitmap) {
        // the winners are the entries at or above T: exactly min(C, k) of them, since T is the
        // k-th largest of distinct composites (or 1, every entry, when C <= k); with ties they are
        // in the bitmap already
        if (!ties) {
            for (uint32_t i = threadIdx.x; i < C; i += kFinishThreads) {
                const uint64_t x = entry_composite(L[i]);
                if (x >= T) {
                    const uint32_t pos = comp_pos(x);
                    atomicOr(&bits[pos >> 5], 1u << (pos & 31));
                }
            }
        }
        __syncthreads();
        if (threadIdx.x == 0) ws.st[t].n_cand = 0u;  // cleared for the next call
        // ascending block ids through the bitmap and a block-wide prefix sum
        const int per = (words + kFinishThreads - 1) / kFinishThreads;
        const int w0 = threadIdx.x * per;
        uint32_t mine = 0;
        for (int q = 0; q < per; ++q)
            if (w0 + q < words) mine += (uint32_t)__popc(bits[w0 + q]);
        uint32_t nall;
        uint32_t base = block_scan<kFinishThreads>(mine, S.wsum[0], nall);
        for (int q = 0; q < per; ++q) {
            if (w0 + q >= words) break;
            uint32_t b = bits[w0 + q];
            while (b) {
                const int bit = __ffs(b) - 1;
                b &= b - 1;
                a.out_idx[t * a.out_stride + base] = (w0 + q) * 32 + bit;
                ++base;
            }
        }
        write_pad(a, t, ties ? k : (C < k ? C : k));
        return;
    }
    // the winners, gathered in rounds of 8 consecutive entries per thread
    constexpr int Q = 8;
    uint32_t nw = 0;
    int sb = 0;
    for (uint32_t i0 = 0; i0 < C; i0 += Q * kFinishThreads) {
        uint64_t x[Q];
        uint32_t wm = 0, c = 0;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const uint32_t i = i0 + Q * threadIdx.x + q;
            x[q] = i < C ? entry_composite(L[i]) : 0ull;
            const bool win = i < C && x[q] >= T;
            wm |= (win ? 1u : 0u) << q;
            c += win ? 1u : 0u;
        }
        __syncthreads();  // the scan buffer of two rounds ago is free
        uint32_t tot;
        uint32_t slot = nw + block_scan<kFinishThreads>(c, S.wsum[sb], tot);
        sb ^= 1;
#pragma unroll
        for (int q = 0; q < Q; ++q)
            if ((wm >> q) & 1u) {
                if (slot < (uint32_t)kMaxK) out[slot] = x[q];
                ++slot;
            }
        nw += tot;
    }
    __syncthreads();
    if (threadIdx.x == 0) ws.st[t].n_cand = 0u;  // cleared for the next call
    const uint32_t cnt = nw < k ? nw : k;
    {
        // ascending position: sort (pos, key) pairs
        int N = 1;
        while (N < (int)cnt) N <<= 1;
        for (int i = threadIdx.x; i < N; i += kFinishThreads)
            out[i] = i < (int)cnt ? (((uint64_t)comp_pos(out[i]) << 32) | comp_key(out[i])) : ~0ull;
        __syncthreads();
        block_sort<kFinishThreads>(out, N);
        for (int i = threadIdx.x; i < (int)cnt; i += kFinishThreads) {
            const uint64_t pk = out[i];
            a.out_idx[t * a.out_stride + i] = (int32_t)(uint32_t)(pk >> 32);
            if (a.out_val && !a.pool_mode) a.out_val[t * a.out_stride + i] = key_value((uint32_t)pk);
        }
    }
    write_pad(a, t, cnt);
}

}  // namespace

size_t select_workspace_bytes(int32_t nq, int64_t cap, int32_t k) {
    (void)k;
    if (nq <= 0 || cap < 0) return 0;
    if (cap <= kSmallRow) return 256;
    const WsView v = ws_view(nullptr, nq, cap);
    return align_up((size_t)nq * sizeof(RowState)) + align_up((size_t)nq * (size_t)v.chunks * sizeof(ChunkBound)) +
           align_up((size_t)nq * (size_t)v.cap * 8) + align_up((size_t)nq * (size_t)v.chunks * (kChunk / 32) * 4);
}

size_t select_counter_bytes(int32_t nq) { return nq > 0 ? (size_t)nq * sizeof(RowState) : 0; }

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
    if (a.nq <= 0) return hipSuccess;
    const int64_t cap = row_cap(a);
    if (cap <= kSmallRow) {
        // the block holds 16 values per thread, and T0 needs k <= NT (k <= 2 NT with the lanes'
        // fourth-largest values, in the wide 1024-thread form) to bound the candidates
        const dim3 grid((unsigned)a.nq);
        const int64_t per_thread = (cap + 8 * kRuns - 1) / (8 * kRuns);
        const int64_t nt = per_thread > a.k ? per_thread : a.k;
        if (nt <= 256)
            hipLaunchKernelGGL((select_small_kernel<256, false>), grid, dim3(256), 0, stream, a);
        else if (nt <= 512)
            hipLaunchKernelGGL((select_small_kernel<512, false>), grid, dim3(512), 0, stream, a);
        else if (a.k <= 1024 || cap <= SmallShared<1024, false>::kCap)  // the narrow list holds such a row whole
            hipLaunchKernelGGL((select_small_kernel<1024, false>), grid, dim3(1024), 0, stream, a);
        else
            hipLaunchKernelGGL((select_small_kernel<1024, true>), grid, dim3(1024), 0, stream, a);
        return hipGetLastError();
    }
    const WsView v = ws_view(a.ws, a.nq, cap);
    hipLaunchKernelGGL(select_bound_kernel, dim3((unsigned)v.chunks, (unsigned)a.nq), dim3(kLargeThreads), 0, stream,
                       a, v);
    hipLaunchKernelGGL(select_collect_kernel, dim3((unsigned)v.chunks, (unsigned)a.nq), dim3(kLargeThreads), 0,
                       stream, a, v);
    hipLaunchKernelGGL(select_finish_kernel, dim3((unsigned)a.nq), dim3(kFinishThreads), 0, stream, a, v);
    return hipGetLastError();
}

}  // namespace fp4idx
