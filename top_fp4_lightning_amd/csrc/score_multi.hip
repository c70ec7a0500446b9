// Many-query indexer scan on gfx950 (chunked prefill, speculative decode): every query of a group
// shares one key range; scores and / or block-8 maxima as in the single-query scan.
#include "score_common.h"

#include <type_traits>

namespace fp4idx {
namespace {

// Many queries sharing one key range (chunked prefill, speculative decode).
//
// Work unit: a tile of 32 keys against all 32 heads of one query as two
// V_MFMA_SCALE_F32_32X32X64_F8F6F4 ops (the second accumulating onto the first). Lane l supplies
// row / column l % 32 and, in op k (k = 0, 1), the FP4 block 2 * (l / 32) + k: so op 0 contracts
// blocks 0 and 2, op 1 blocks 1 and 3, and a lane reads the 32 contiguous code bytes of its key's
// half row plus the two scale bytes of that half (selected per op by the scale byte-select).
// Output: lane l holds key l % 32 for the 16 heads 8 * (j / 4) + 4 * (l / 32) + j % 4
// (j = 0..15). On this chip a 32x32x64 op overlaps the ReLU epilogue better than two
// 16x16x128 ops and leaves half the matrix instructions.
//
// When scores are written, the head sum is taken in the same order as the single-query scan, so
// both paths give bit-identical scores: each lane keeps the two 8-head chains (4g .. 4g+3,
// 16+4g .. 16+4g+3) for g = l / 32 and g + 2, adds them, and one cross-half add completes the key.
// The block-maxima-only form (chunked prefill, speculative verification) sums a lane's 16 heads
// in one chain instead: one vector instruction fewer per tile on a kernel bound by vector issue,
// and a different rounding of the same exact per-head dots (fp32 sums of 32 terms, well inside the
// scores' 1e-5 tolerance).
//
// Each wave keeps QW queries in registers and applies every tile it loads to all of them; the
// four waves of a block take consecutive queries and the same key chunk. Grid: x = query tiles
// of 4*QW queries (fastest, so that concurrently running blocks share a key chunk in L2),
// y = key chunks of KT*64 keys, z = groups. SCORES / BMAX select the outputs at compile time.
// Steps whose 64 keys are visible to every query of the wave run without masks; the remaining
// steps run a masked copy.
typedef float v16f __attribute__((ext_vector_type(16)));

struct QRegs32 {
    v4i a[2];     // op k: this lane's FP4 block 2 * (l / 32) + k of head l % 32
    int sc;       // byte k: that block's UE8M0 scale
    float w[16];  // weights of the output rows held by this lane
};

__device__ __forceinline__ void load_query32(const uint8_t* __restrict__ q_codes,
                                             const uint8_t* __restrict__ q_scales, const float* __restrict__ w,
                                             int64_t t, int lane, QRegs32& q) {
    const int head = lane & 31, h = lane >> 5;
    const uint8_t* row = q_codes + (t * kHeads + head) * kRowBytes + 32 * h;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint4 c = *reinterpret_cast<const uint4*>(row + 16 * k);
        q.a[k] = v4i{(int)c.x, (int)c.y, (int)c.z, (int)c.w};
    }
    const uint8_t* srow = q_scales + (t * kHeads + head) * kGroups + 2 * h;
    q.sc = (int)srow[0] | ((int)srow[1] << 8);
#pragma unroll
    for (int j = 0; j < 16; ++j) q.w[j] = w[t * kHeads + 8 * (j / 4) + 4 * h + (j % 4)];
}

struct KTile32 {
    v4i b[2];
    int sc;
};

__device__ __forceinline__ v16f mfma_tile32(const QRegs32& q, const KTile32& kt) {
    v16f z;
#pragma unroll
    for (int j = 0; j < 16; ++j) z[j] = 0.0f;
    const v16f t =
        __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(q.a[0]), widen(kt.b[0]), z, 4, 4, 0, q.sc, 0, kt.sc);
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(q.a[1]), widen(kt.b[1]), t, 4, 4, 1, q.sc, 1, kt.sc);
}

// this lane's partial. SAME_ORDER: chain over rows j = 0-3, 8-11 plus chain over rows 4-7, 12-15
// (the single-query scan's order); otherwise one chain over the 16 rows
template <bool SAME_ORDER>
__device__ __forceinline__ float lane_partial32(const QRegs32& q, const v16f& o) {
    if constexpr (SAME_ORDER) {
        float pa = 0.0f, pb = 0.0f;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pa = fmaf(q.w[8 * b + i], relu(o[8 * b + i]), pa);
                pb = fmaf(q.w[8 * b + 4 + i], relu(o[8 * b + 4 + i]), pb);
            }
        return pa + pb;
    } else {
        float p = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) p = fmaf(q.w[j], relu(o[j]), p);
        return p;
    }
}

// two tiles' partials -> in lane l the score of key l of the 64-key step
__device__ __forceinline__ float combine2(float p0, float p1) {
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Keys are staged in LDS once per block, two 64-key steps at a time: per step 4 KiB of codes
// (16-byte chunks XOR-swizzled so that eight consecutive keys fall on distinct bank groups for
// the operand reads) and 256 bytes of scales. The staging uses direct-to-LDS buffer loads (no
// registers in between), three buffers deep: while block s is scored, the loads of blocks s + 1
// and s + 2 are in flight. One barrier per staged block, after each wave has waited for its own
// loads of block s, publishes block s and frees the buffer of block s - 1 for the next issue.
// Control flow around the barriers is uniform per block.
//
// Block maxima: after a step, all eight lanes of a key block hold its maximum, and lane 8g stores
// that of block g (eight consecutive floats per step and query): no per-step bookkeeping on the
// vector pipe, which bounds this kernel.
constexpr int kStepKeys = 64;
constexpr int kStageSteps = 2;                      // 64-key steps per staged block (one barrier)
constexpr int kStageCodes = kStepKeys * kRowBytes;  // bytes of codes per step
constexpr int kBufs = 3;  // staged blocks in LDS: kBufs - 1 in flight while one is scored

struct StageBuf {
    alignas(16) uint8_t codes[kBufs][kStageSteps][kStageCodes];
    alignas(16) uint32_t scales[kBufs][kStageSteps * kStepKeys];
};

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// wait until at most N of this wave's vector-memory loads are outstanding (loads complete in
// order, so every load issued before the last N has landed, in LDS for the direct loads)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS byte offset of 16-byte chunk p (0..3) of key kk (0..63) of a step
__device__ __forceinline__ uint32_t stage_chunk(int kk, int p) {
    return (uint32_t)(kk * 4 + (p ^ ((kk >> 1) & 3))) * 16u;
}

template <int QW, int KT, bool SCORES, bool BMAX>
__global__ __launch_bounds__(256) void score_multi_kernel(ScoreArgs a) {
    __shared__ StageBuf sb;
    const int lane = threadIdx.x & 63;
    // wave index as a uniform value: query bounds, key range and descriptors stay scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t g0 = (int64_t)blockIdx.z * a.group;  // first query of the group
    const int64_t qb0 = g0 + (int64_t)blockIdx.x * 4 * QW;  // first query of the block
    const int64_t qw0 = qb0 + (int64_t)wave * QW;
    const int64_t g_end = g0 + a.group;
    const int e_begin = (int)blockIdx.y * (KT * kStepKeys);  // key ranges are below 2^24

    // visible-key counts: the block's maximum bounds the staging (uniform per block), the wave's
    // bounds decide which steps it scores and which run masked (uniform per wave)
    auto nvis = [&](int64_t qq) -> int {
        int64_t n = qq < g_end ? (int64_t)a.n_vis[qq] : 0;
        return (int)(n < 0 ? 0 : (n > a.max_n ? a.max_n : n));
    };
    int nb_max = 0;
#pragma unroll
    for (int i = 0; i < 4 * QW; ++i) {
        const int n = nvis(qb0 + i);
        nb_max = n > nb_max ? n : nb_max;
    }
    if (e_begin >= nb_max) return;  // uniform per block
    // queries of this wave inside the group: the last wave of a group may hold fewer than QW, or
    // none (it still stages keys for the block but scores nothing)
    const int qv = (int)(g_end - qw0 < 0 ? 0 : (g_end - qw0 < QW ? g_end - qw0 : QW));
    int nq_[QW];
    int nmax = 0, nmin = INT32_MAX;
#pragma unroll
    for (int i = 0; i < QW; ++i) {
        nq_[i] = nvis(qw0 + i);
        nmax = nq_[i] > nmax ? nq_[i] : nmax;
        if (i < qv) nmin = nq_[i] < nmin ? nq_[i] : nmin;
    }
    const int e_stop = e_begin + KT * kStepKeys < nb_max ? e_begin + KT * kStepKeys : nb_max;
    const int n_steps = (e_stop - e_begin + kStepKeys - 1) / kStepKeys;

    QRegs32 q[QW];
#pragma unroll
    for (int i = 0; i < QW; ++i)
        load_query32(a.q_codes, a.q_scales, a.w, qw0 + i < g_end ? qw0 + i : g0, lane, q[i]);
    const KeyRange kr = key_range(a.k_codes, a.k_scales, a.k_base[g0], nb_max);
    const int h = lane >> 5, c = lane & 31;
    // per-query output rows; a query past the group has n = 0 and never stores
    float* srow[QW];
    float* brow[QW];
#pragma unroll
    for (int i = 0; i < QW; ++i) {
        const int64_t qq = qw0 + i < g_end ? qw0 + i : g0;
        srow[i] = SCORES ? a.scores + qq * a.score_stride : nullptr;
        brow[i] = BMAX ? a.block_max + qq * a.bm_stride : nullptr;
    }

    // Staging with direct-to-LDS loads: lane l of a wave's load lands at the instruction's LDS base
    // + 16 l (4 l for a word), so each lane fetches the global chunk that belongs at its LDS slot.
    // Per staged block every wave issues kStageSteps + 1 loads: for each step its 1 KiB of the
    // codes (slots 64 wave .. 64 wave + 63, i.e. keys 16 wave .. 16 wave + 15, with the XOR swizzle
    // undone on the global side), and the 64 scale words of step wave % 2 (waves 2 and 3 repeat
    // waves 0 and 1 with the same bytes, so that all waves count the same loads).
    constexpr int kLoadsPerStage = kStageSteps + 1;
    auto stage_issue = [&](int sg) {
        const int buf = sg % kBufs;
        const uint32_t e0 = (uint32_t)(e_begin + sg * kStageSteps * kStepKeys);
        const int slot = 64 * wave + lane;
        const int kk = slot >> 2;
        const int p = (slot & 3) ^ ((kk >> 1) & 3);
#pragma unroll
        for (int ss = 0; ss < kStageSteps; ++ss)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                kr.codes, (lds_void_ptr)&sb.codes[buf][ss][1024 * wave], 16,
                (e0 + (uint32_t)(ss * kStepKeys + kk)) * kRowBytes + (uint32_t)p * 16u, 0, 0, kReuse);
        const int ss = wave & 1;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kr.scales, (lds_void_ptr)&sb.scales[buf][ss * kStepKeys], 4,
                                                 (e0 + (uint32_t)(ss * kStepKeys + lane)) * kGroups, 0, 0, kReuse);
    };
    // operands of tile u (keys 32u .. 32u + 31) of step ss of buffer buf
    auto read_tiles = [&](int buf, int ss, KTile32 (&t)[2]) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int kk = 32 * u + c;
#pragma unroll
            for (int k = 0; k < 2; ++k)
                t[u].b[k] = *reinterpret_cast<const v4i*>(
                    __builtin_assume_aligned(&sb.codes[buf][ss][stage_chunk(kk, 2 * h + k)], 16));
            t[u].sc = (int)reinterpret_cast<const uint16_t*>(&sb.scales[buf][ss * kStepKeys + kk])[h];
        }
    };

    // the wave scores steps 0 .. last (its queries see keys below nmax)
    const int last = (nmax - e_begin + kStepKeys - 1) / kStepKeys < n_steps
                         ? (nmax - e_begin + kStepKeys - 1) / kStepKeys - 1
                         : n_steps - 1;
    // lane 8g of a step stores the maximum of block g, through a buffer descriptor of the query's
    // row: the lane's byte offset is fixed, the step's (8 blocks a step) is a scalar
    const bool bm_lane = (lane & 7) == 0;
    __amdgpu_buffer_rsrc_t bm_rsrc[QW];
#pragma unroll
    for (int i = 0; i < QW; ++i)
        bm_rsrc[i] = __builtin_amdgcn_make_buffer_rsrc(BMAX ? (void*)brow[i] : (void*)a.k_codes, 0,
                                                       BMAX ? (int)(((nq_[i] + kBlock - 1) / kBlock) * 4) : 0,
                                                       kRsrcWord3);
    const int bm_voff = ((e_begin >> 3) + (lane >> 3)) * 4;
    // score rows the same way: lane l stores key e0 + l, keys past the query's count are dropped
    __amdgpu_buffer_rsrc_t sc_rsrc[QW];
#pragma unroll
    for (int i = 0; i < QW; ++i)
        sc_rsrc[i] = __builtin_amdgcn_make_buffer_rsrc(SCORES ? (void*)srow[i] : (void*)a.k_codes, 0,
                                                       SCORES ? nq_[i] * 4 : 0, kRsrcWord3);
    const int sc_voff = (e_begin + lane) * 4;

    // score step `it` for every query; MASKED steps drop keys past each query's count
    auto step = [&](const KTile32 (&t)[2], int it, auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        const int e0 = e_begin + it * kStepKeys;
        const int el = e0 + lane;
#pragma unroll
        for (int i = 0; i < QW; ++i) {
            if (i >= qv) break;  // uniform per wave
            const v16f o0 = mfma_tile32(q[i], t[0]);
            const v16f o1 = mfma_tile32(q[i], t[1]);
            const float sc = combine2(lane_partial32<SCORES>(q[i], o0), lane_partial32<SCORES>(q[i], o1));
            const bool valid = !MASKED || el < nq_[i];
            if (SCORES)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), sc_rsrc[i], sc_voff, it * kStepKeys * 4, 0);
            if (BMAX) {
                // every lane of a block holds its maximum; one lane per block stores it (the
                // block is visible when its first key is)
                float m = max8(valid ? sc : -INFINITY);
                asm volatile("" : "+v"(m));  // the whole maximum in every lane, before the store branch
                if (bm_lane)  // blocks past the query's visible ones fall outside the descriptor
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m), bm_rsrc[i], bm_voff,
                                                          it * (kStepKeys / kBlock) * 4, 0);
            }
            // one query's matrix results live at a time: keeps the wave within the register
            // budget of four waves per SIMD (other waves hide the matrix latency)
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    const int n_stages = (n_steps + kStageSteps - 1) / kStageSteps;
    for (int sg = 0; sg < kBufs - 1 && sg < n_stages; ++sg) stage_issue(sg);
    // staged block sg lives in buffer sg % kBufs: the loop is unrolled over the buffers, so that
    // each copy reads its buffer at fixed LDS offsets (immediates of the operand reads)
#pragma nounroll
    for (int sg0 = 0; sg0 < n_stages; sg0 += kBufs) {
#pragma unroll
        for (int buf = 0; buf < kBufs; ++buf) {
            const int sg = sg0 + buf;
            if (sg >= n_stages) break;  // uniform per block
            // staged blocks issued after this one so far: their loads may stay in flight
            const int younger = (n_stages - 1 < sg + kBufs - 2 ? n_stages - 1 : sg + kBufs - 2) - sg;
            if (kBufs >= 4 && younger >= 2)
                wait_vm<2 * kLoadsPerStage>();
            else if (younger >= 1)
                wait_vm<kLoadsPerStage>();
            else
                wait_vm<0>();
            // every wave's loads of block sg have landed, and every wave is done with block sg - 1,
            // whose buffer the next issue overwrites
            __syncthreads();
            if (sg + kBufs - 1 < n_stages) stage_issue(sg + kBufs - 1);
#pragma unroll
            for (int ss = 0; ss < kStageSteps; ++ss) {
                const int it = sg * kStageSteps + ss;
                if (it <= last) {  // uniform per wave
                    KTile32 t[2];
                    read_tiles(buf, ss, t);
                    if (e_begin + (it + 1) * kStepKeys <= nmin)
                        step(t, it, std::false_type{});
                    else
                        step(t, it, std::true_type{});
                }
            }
        }
    }
}

// queries per wave in the many-query scan: two keep a wave within 128 registers, i.e. four
// waves per SIMD, which hide the matrix-result latency of each other
constexpr int kMultiQ = 2;
constexpr int kMultiIters = 32;  // 64-key steps per block (2048 keys)

}  // namespace

hipError_t launch_score_multi(const ScoreArgs& a, hipStream_t stream) {
    if (a.nq <= 0 || a.max_n <= 0) return hipSuccess;
    const int64_t qtile = 4 * kMultiQ;
    const int64_t gx = (a.group + qtile - 1) / qtile;
    const int64_t gy = (a.max_n + kMultiIters * 64 - 1) / (kMultiIters * 64);
    const int64_t gz = a.nq / a.group;
    const dim3 grid((unsigned)gx, (unsigned)gy, (unsigned)gz);
    if (a.scores && a.block_max)
        hipLaunchKernelGGL((score_multi_kernel<kMultiQ, kMultiIters, true, true>), grid, dim3(256), 0, stream, a);
    else if (a.scores)
        hipLaunchKernelGGL((score_multi_kernel<kMultiQ, kMultiIters, true, false>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((score_multi_kernel<kMultiQ, kMultiIters, false, true>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace fp4idx
