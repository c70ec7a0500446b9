// Exact top-k selection (k <= 2048) over rows of fp32 values, ranked by (value desc, index asc).
//
// Keys: the fp32 bit pattern mapped to an order-preserving uint32; a 64-bit composite
// (key << 32) | ~index is unique per element and orders exactly like (value desc, index asc).
// -inf and NaN are not eligible.
//
//  1. clear   : zero the per-row histograms and counters in the workspace.
//  2. hist    : histogram of the top 11 key bits per row (LDS, then global atomics).
//  3. filter  : each block recomputes the threshold digit from the row histogram; elements above
//               it are certainly selected ("sure"), elements on it are candidates. Appends use
//               one atomic per wavefront (ballot + popcount).
//  4. finish  : one block per row runs radix passes over the candidates' remaining 53 composite
//               bits until exactly k are chosen, then bitonic-sorts the k composites in LDS and
//               writes indices (and values).
// Pool mode (candidate pool of the hierarchical indexer): values are block maxima, the block of
// position n-1 is pinned to +inf, and the kept block ids are written in ascending order.
#include "internal.h"

namespace fp4idx {
namespace {

struct RowCtl {
    uint32_t sure;
    uint32_t cand;
    int32_t thr_bin;
    uint32_t total;
};

constexpr int kChunk = 4096;  // elements per block in hist / filter
constexpr int kFinishThreads = 1024;

__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}
// finite or +inf; excludes -inf (0x007fffff) and NaN (keys above +inf's 0xff800000)
__device__ __forceinline__ bool eligible(uint32_t k) { return k > 0x007fffffu && k <= 0xff800000u; }

struct WsView {
    uint32_t* hist;  // [nq][2048]
    RowCtl* ctl;     // [nq]
    uint64_t* sel;   // [nq][k]
    uint64_t* cand;  // [nq][cap]
    int64_t cap;
};

__host__ __device__ inline size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline WsView ws_view(void* ws, int32_t nq, int64_t cap, int32_t k) {
    char* p = (char*)ws;
    WsView v;
    v.hist = (uint32_t*)p;
    p += align_up((size_t)nq * kHistBins * 4);
    v.ctl = (RowCtl*)p;
    p += align_up((size_t)nq * sizeof(RowCtl));
    v.sel = (uint64_t*)p;
    p += align_up((size_t)nq * k * 8);
    v.cand = (uint64_t*)p;
    v.cap = cap;
    return v;
}

struct RowInfo {
    int64_t len;  // values in this row
    int64_t pin;  // pinned element (pool mode) or -1
};

__device__ __forceinline__ RowInfo row_info(const SelectArgs& a, int64_t t) {
    int64_t n = a.nv ? (int64_t)a.nv[t] : a.max_n;
    n = n < 0 ? 0 : (n > a.max_n ? a.max_n : n);
    RowInfo ri;
    if (a.pool_mode) {
        ri.len = (n + kBlock - 1) / kBlock;
        ri.pin = n > 0 ? (n - 1) / kBlock : -1;
    } else {
        ri.len = n;
        ri.pin = -1;
    }
    return ri;
}

__device__ __forceinline__ uint32_t key_at(const SelectArgs& a, int64_t t, int64_t i, const RowInfo& ri) {
    if (i == ri.pin) return 0xff800000u;  // +inf
    return order_key(a.vals[t * a.stride + i]);
}

__device__ __forceinline__ uint32_t pos_at(const SelectArgs& a, int64_t t, int64_t i) {
    if (a.map) return (uint32_t)(a.map[t * a.map_stride + (i >> 3)] * kBlock + (int32_t)(i & 7));
    return (uint32_t)i;
}

__global__ void select_clear_kernel(uint32_t* hist, RowCtl* ctl, int32_t nq) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nh = (int64_t)nq * kHistBins;
    if (i < nh) hist[i] = 0u;
    if (i < nq) ctl[i] = RowCtl{0u, 0u, -1, 0u};
}

__global__ __launch_bounds__(256) void select_hist_kernel(SelectArgs a, WsView v) {
    __shared__ uint32_t h[kHistBins];
    const int64_t t = blockIdx.y;
    const RowInfo ri = row_info(a, t);
    const int64_t c0 = (int64_t)blockIdx.x * kChunk;
    if (c0 >= ri.len) return;  // uniform per block
    for (int b = threadIdx.x; b < kHistBins; b += blockDim.x) h[b] = 0u;
    __syncthreads();
    const int64_t c1 = c0 + kChunk < ri.len ? c0 + kChunk : ri.len;
    for (int64_t i = c0 + threadIdx.x; i < c1; i += blockDim.x) {
        const uint32_t k = key_at(a, t, i, ri);
        if (eligible(k)) atomicAdd(&h[k >> 21], 1u);
    }
    __syncthreads();
    for (int b = threadIdx.x; b < kHistBins; b += blockDim.x)
        if (h[b]) atomicAdd(&v.hist[t * kHistBins + b], h[b]);
}

// threshold digit of a 2048-bin histogram: the largest d with sum_{b >= d} h[b] >= need;
// returns -1 (and *above = total) when the total is below need. 256 threads, 8 bins each.
__device__ int find_threshold(const uint32_t* h, uint32_t need, uint32_t* above, uint32_t* total, uint32_t* scratch,
                              int* result) {
    const int tid = threadIdx.x;
    uint32_t part = 0;
    for (int b = 0; b < 8; ++b) part += h[tid * 8 + b];
    scratch[tid] = part;
    if (tid == 0) *result = -1;
    __syncthreads();
    // suffix sums over the 256 partials (inclusive), Hillis-Steele
    for (int off = 1; off < 256; off <<= 1) {
        uint32_t x = (tid + off < 256) ? scratch[tid + off] : 0u;
        __syncthreads();
        scratch[tid] += x;
        __syncthreads();
    }
    uint32_t cum = scratch[tid] - part;  // elements in bins above this thread's range
    const uint32_t tot = scratch[0];
    for (int b = tid * 8 + 7; b >= tid * 8; --b) {
        if (cum < need && cum + h[b] >= need) {
            *result = b;
            *above = cum;
        }
        cum += h[b];
    }
    __syncthreads();
    if (*result < 0 && tid == 0) *above = tot;
    *total = tot;
    __syncthreads();
    return *result;
}

__device__ __forceinline__ uint32_t wave_append(bool pred, uint32_t* counter) {
    const uint64_t m = __ballot(pred);
    if (m == 0) return 0;
    const int lane = threadIdx.x & 63;
    const int leader = __ffsll((unsigned long long)m) - 1;
    uint32_t base = 0;
    if (lane == leader) base = atomicAdd(counter, (uint32_t)__popcll(m));
    base = __shfl(base, leader);
    return base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
}

__global__ __launch_bounds__(256) void select_filter_kernel(SelectArgs a, WsView v) {
    __shared__ uint32_t h[kHistBins];
    __shared__ uint32_t scratch[256];
    __shared__ uint32_t above, total;
    __shared__ int thr;
    const int64_t t = blockIdx.y;
    const RowInfo ri = row_info(a, t);
    const int64_t c0 = (int64_t)blockIdx.x * kChunk;
    if (c0 >= ri.len && blockIdx.x != 0) return;
    for (int b = threadIdx.x; b < kHistBins; b += blockDim.x) h[b] = v.hist[t * kHistBins + b];
    __syncthreads();
    const int b1 = find_threshold(h, (uint32_t)a.k, &above, &total, scratch, &thr);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        v.ctl[t].thr_bin = b1;
        v.ctl[t].total = total;
    }
    const int64_t c1 = c0 + kChunk < ri.len ? c0 + kChunk : ri.len;
    // iterate in wave-uniform trip counts so that ballots see the whole wave
    for (int64_t i0 = c0; i0 < c1; i0 += blockDim.x) {
        const int64_t i = i0 + threadIdx.x;
        uint32_t k = 0;
        if (i < c1) k = key_at(a, t, i, ri);
        const bool ok = i < c1 && eligible(k);
        const int bin = (int)(k >> 21);
        const bool sure = ok && bin > b1;
        const bool cand = ok && bin == b1;
        const uint32_t ps = wave_append(sure, &v.ctl[t].sure);
        const uint32_t pc = wave_append(cand, &v.ctl[t].cand);
        if (sure || cand) {
            const uint64_t comp = ((uint64_t)k << 32) | (uint64_t)(~pos_at(a, t, i));
            if (sure) v.sel[t * a.k + ps] = comp;
            else if ((int64_t)pc < v.cap) v.cand[t * v.cap + pc] = comp;
        }
    }
}

__global__ __launch_bounds__(kFinishThreads) void select_finish_kernel(SelectArgs a, WsView v) {
    __shared__ uint64_t keep[kMaxK];
    __shared__ uint32_t h[kHistBins];
    __shared__ uint32_t scratch[256];
    __shared__ uint32_t nkeep, above, total;
    __shared__ int thr;
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const RowCtl ctl = v.ctl[t];
    const uint32_t nsure = ctl.sure;
    uint32_t ncand = ctl.cand;
    if ((int64_t)ncand > v.cap) ncand = (uint32_t)v.cap;
    for (uint32_t i = tid; i < nsure; i += blockDim.x) keep[i] = v.sel[t * a.k + i];
    if (tid == 0) nkeep = nsure;
    __syncthreads();
    uint32_t need = ctl.thr_bin >= 0 ? (uint32_t)a.k - nsure : 0u;
    const uint64_t* cand = v.cand + t * v.cap;
    // composite bits below the top 11 (which all candidates share): digits 52..42, 41..31,
    // 30..20, 19..9, 8..0
    uint64_t prefix = 0, mask = 0;
    const int shifts[5] = {42, 31, 20, 9, 0};
    const int widths[5] = {11, 11, 11, 11, 9};
    for (int p = 0; p < 5 && need > 0; ++p) {
        const int sh = shifts[p];
        const uint64_t dm = ((uint64_t)1 << widths[p]) - 1;
        for (int b = tid; b < kHistBins; b += blockDim.x) h[b] = 0u;
        __syncthreads();
        for (uint32_t i = tid; i < ncand; i += blockDim.x) {
            const uint64_t c = cand[i];
            if (((c ^ prefix) & mask) == 0) atomicAdd(&h[(c >> sh) & dm], 1u);
        }
        __syncthreads();
        // threshold digit with 256 threads over 2048 bins
        int d = -1;
        if (tid < 256) {
            uint32_t part = 0;
            for (int b = 0; b < 8; ++b) part += h[tid * 8 + b];
            scratch[tid] = part;
            if (tid == 0) thr = -1;
        }
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            uint32_t x = 0;
            if (tid < 256) x = (tid + off < 256) ? scratch[tid + off] : 0u;
            __syncthreads();
            if (tid < 256) scratch[tid] += x;
            __syncthreads();
        }
        if (tid < 256) {
            uint32_t cum = scratch[tid];
            uint32_t part = 0;
            for (int b = 0; b < 8; ++b) part += h[tid * 8 + b];
            cum -= part;
            for (int b = tid * 8 + 7; b >= tid * 8; --b) {
                if (cum < need && cum + h[b] >= need) {
                    thr = b;
                    above = cum;
                }
                cum += h[b];
            }
        }
        __syncthreads();
        d = thr;  // always found: candidates matching the prefix number at least `need`
        const bool take_eq = (h[d] == need - above);
        for (uint32_t i = tid; i < ncand; i += blockDim.x) {
            const uint64_t c = cand[i];
            if (((c ^ prefix) & mask) != 0) continue;
            const int dig = (int)((c >> sh) & dm);
            if (dig > d || (take_eq && dig == d)) {
                const uint32_t slot = atomicAdd(&nkeep, 1u);
                if (slot < kMaxK) keep[slot] = c;
            }
        }
        __syncthreads();
        if (take_eq) need = 0;
        else {
            need -= above;
            prefix |= (uint64_t)d << sh;
            mask |= dm << sh;
        }
        __syncthreads();
    }
    const uint32_t cnt = nkeep < (uint32_t)a.k ? nkeep : (uint32_t)a.k;
    // sort: descending composite (rank order) or, in pool mode, ascending block id
    int N = 1;
    while (N < (int)cnt) N <<= 1;
    for (int i = tid; i < N; i += blockDim.x) {
        if (i >= (int)cnt) keep[i] = a.pool_mode ? ~0ull : 0ull;
        else if (a.pool_mode) keep[i] = (uint64_t)(uint32_t)(~(uint32_t)keep[i]);
    }
    __syncthreads();
    for (int size = 2; size <= N; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < N / 2; i += blockDim.x) {
                const int lo = 2 * stride * (i / stride) + (i % stride);
                const int hi = lo + stride;
                const bool up = (lo & size) == 0;
                const uint64_t x = keep[lo], y = keep[hi];
                if ((x > y) == up) {
                    keep[lo] = y;
                    keep[hi] = x;
                }
            }
            __syncthreads();
        }
    }
    int32_t* oi = a.out_idx + t * a.out_stride;
    for (int i = tid; i < a.pad_to; i += blockDim.x) {
        if (i < (int)cnt) {
            if (a.pool_mode) {
                oi[i] = (int32_t)keep[i];
            } else {
                const uint64_t c = keep[N - 1 - i];
                oi[i] = (int32_t)(~(uint32_t)c);
                if (a.out_val) a.out_val[t * a.out_stride + i] = key_value((uint32_t)(c >> 32));
            }
        } else {
            oi[i] = -1;
            if (a.out_val && !a.pool_mode) a.out_val[t * a.out_stride + i] = -INFINITY;
        }
    }
    if (a.out_count && tid == 0) a.out_count[t] = (int32_t)cnt;
}

}  // namespace

size_t select_workspace_bytes(int32_t nq, int64_t cap, int32_t k) {
    if (nq <= 0 || cap < 0 || k <= 0) return 0;
    return align_up((size_t)nq * kHistBins * 4) + align_up((size_t)nq * sizeof(RowCtl)) +
           align_up((size_t)nq * k * 8) + align_up((size_t)nq * (size_t)(cap > 0 ? cap : 1) * 8);
}

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
    if (a.nq <= 0) return hipSuccess;
    const int64_t cap = a.pool_mode ? (a.max_n + kBlock - 1) / kBlock : a.max_n;
    const WsView v = ws_view(a.ws, a.nq, cap > 0 ? cap : 1, a.k);
    const int64_t nclear = (int64_t)a.nq * kHistBins;
    hipLaunchKernelGGL(select_clear_kernel, dim3((unsigned)((nclear + 255) / 256)), dim3(256), 0, stream, v.hist,
                       v.ctl, a.nq);
    const int64_t gx = cap > 0 ? (cap + kChunk - 1) / kChunk : 1;
    hipLaunchKernelGGL(select_hist_kernel, dim3((unsigned)gx, (unsigned)a.nq), dim3(256), 0, stream, a, v);
    hipLaunchKernelGGL(select_filter_kernel, dim3((unsigned)gx, (unsigned)a.nq), dim3(256), 0, stream, a, v);
    hipLaunchKernelGGL(select_finish_kernel, dim3((unsigned)a.nq), dim3(kFinishThreads), 0, stream, a, v);
    return hipGetLastError();
}

}  // namespace fp4idx
