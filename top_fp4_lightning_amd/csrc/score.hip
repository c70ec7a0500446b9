// Indexer scoring on gfx950: scaled-FP4 MFMA for the per-head dots, fused ReLU-weighted head sum,
// block-8 maxima.
//
// Work unit: one wave scores 64 keys per step as four tiles of 16 keys. For a tile, two
// V_MFMA_SCALE_F32_16X16X128_F8F6F4 ops (FP4 x FP4, one per half of the 32 heads) contract all
// 128 dims at once: A = the query (16 heads x 128), B = 16 keys x 128. Operand lane layout
// (verified on the hardware): lane l holds row/column l % 16 and the 32-element K-block l / 16,
// i.e. 16 code bytes, plus that block's E8M0 scale byte. So a tile's B operand is the 1 KiB of
// codes of 16 consecutive keys read with one 128-bit load per lane (fully coalesced), and the
// query stays in registers for the whole scan. Output: lane l holds key l % 16 for heads
// 4 * (l / 16) + i (i = 0..3) of each half. Each lane sums ReLU(d) * w over its 8 heads; the
// four lane rows are then combined for four tiles at once with two permlane32 swaps and one
// permlane16 swap, which leaves the score of key l of the 64-key step in lane l.
//
// The four scale bytes of a step's key l arrive as one 32-bit load in lane l and reach the tile
// lanes through ds_bpermute. The scan gives each wavefront one step (eight wavefronts per SIMD
// keep the loads in flight); the gather's long form keeps the next step's loads in flight while
// the current step computes.
//
// The scale-FP4 MFMA aligns the four 32-element block sums of a dot to the largest block exponent
// (also when that block sums to zero): the dot is exact when the block exponent sums of the pair
// span at most 14 (measured), which rotated activations meet with a wide margin; the head sum is
// fp32.
#include "score_common.h"

namespace fp4idx {
namespace {

struct QRegs {
    v4i a[2];       // heads 0-15 and 16-31: this lane's 32-element block of head (l % 16) + 16h
    int sc[2];      // its UE8M0 scale byte
    float w[2][4];  // weights of output heads 16h + 4 * (l / 16) + i
};

__device__ __forceinline__ void load_query(const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales,
                                           const float* __restrict__ w, int64_t t, int lane, QRegs& q) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int head = 16 * h + r;
        const uint4 c = *reinterpret_cast<const uint4*>(q_codes + ((t * kHeads + head) * kRowBytes + g * 16));
        q.a[h] = v4i{(int)c.x, (int)c.y, (int)c.z, (int)c.w};
        q.sc[h] = (int)q_scales[(t * kHeads + head) * kGroups + g];
#pragma unroll
        for (int i = 0; i < 4; ++i) q.w[h][i] = w[t * kHeads + 16 * h + 4 * g + i];
    }
}

constexpr uint32_t kAbsent = 0x3ffffffu;  // a key index past every range: its loads read zeros

// B operand of one tile
struct KTile {
    v4i b;
    int sc;
};

// A 64-key step's operands: per tile u, this lane's 16 code bytes of key 16u + l % 16 (group
// l / 16); and one 32-bit word per lane holding all four scale bytes of the step's key l. One
// dword load per lane replaces four byte loads (one per tile) and leaves the memory pipeline a
// quarter of the scale instructions; tile u's scale byte then comes from lane 16u + l % 16.
struct KStep {
    v4i b[4];
    uint32_t sw;
};

template <int POLICY>
__device__ __forceinline__ v4i load_codes(const KeyRange& kr, uint32_t e, int g) {
    const auto c =
        __builtin_amdgcn_raw_buffer_load_b128(kr.codes, e * (uint32_t)kRowBytes + (uint32_t)g * 16u, 0, POLICY);
    return v4i{(int)c[0], (int)c[1], (int)c[2], (int)c[3]};
}

template <int POLICY>
__device__ __forceinline__ uint32_t load_scale_word(const KeyRange& kr, uint32_t e) {
    return __builtin_amdgcn_raw_buffer_load_b32(kr.scales, e * (uint32_t)kGroups, 0, POLICY);
}

// tile u of a step: the codes, and the scale byte of group g of key 16u + r taken from that key's lane
__device__ __forceinline__ KTile step_tile(const KStep& ks, int u, int r, int g) {
    KTile kt;
    kt.b = ks.b[u];
    kt.sc = (int)(((uint32_t)__builtin_amdgcn_ds_bpermute((16 * u + r) * 4, (int)ks.sw) >> (8 * g)) & 0xffu);
    return kt;
}

struct TileOut {
    v4f d[2];
};

__device__ __forceinline__ void mfma_tile(const QRegs& q, const KTile& kt, TileOut& o) {
    const v4f z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 2; ++h)
        o.d[h] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(widen(q.a[h]), widen(kt.b), z, 4, 4, 0, q.sc[h], 0,
                                                                  kt.sc);
}

// this lane's partial score: sum over its 8 heads of w * ReLU(d), fixed order
__device__ __forceinline__ float lane_partial(const QRegs& q, const TileOut& o) {
    float p = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) p = fmaf(q.w[h][i], relu(o.d[h][i]), p);
    return p;
}

// combine the four 16-lane rows for four tiles: returns in lane l the score of key l of the step
__device__ __forceinline__ float combine4(float p0, float p1, float p2, float p3) {
    // permlane32_swap(x, y): x' = [x.lo, y.lo], y' = [x.hi, y.hi] (32-lane halves)
    auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p2), false, false);
    auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p1), __float_as_uint(p3), false, false);
    const float u = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);  // lanes 0-31: tile 0, 32-63: tile 2
    const float v = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);  // lanes 0-31: tile 1, 32-63: tile 3
    // permlane16_swap(x, y): x' = [x.r0, y.r0, x.r2, y.r2], y' = [x.r1, y.r1, x.r3, y.r3]
    auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(u), __float_as_uint(v), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// --------------------------------------------------------------------------------------------
// Full-layer scan, one query per key range. Grid: x = chunks of 4 waves x ITERS x 64 keys,
// y = queries. Keys past n_t are not scored (their loads read zeros).
template <int ITERS>
__global__ __launch_bounds__(256) void score_full_kernel(ScoreArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t t = blockIdx.y;
    int64_t n = a.n_vis[t];
    n = n < 0 ? 0 : (n > a.max_n ? a.max_n : n);
    const int64_t e_begin = ((int64_t)blockIdx.x * 4 + wave) * (ITERS * 64);
    if (e_begin >= n) return;

    QRegs q;
    load_query(a.q_codes, a.q_scales, a.w, t, lane, q);
    const KeyRange kr = key_range(a.k_codes, a.k_scales, a.k_base[t], n);
    const int g = lane >> 4, r = lane & 15;
    float* bm_row = a.block_max ? a.block_max + t * a.bm_stride : nullptr;
    float* sc_row = a.scores ? a.scores + t * a.score_stride : nullptr;

    auto load_step = [&](int64_t e0, KStep& ks) {
#pragma unroll
        for (int u = 0; u < 4; ++u) ks.b[u] = load_codes<kStream>(kr, (uint32_t)(e0 + 16 * u + r), g);
        ks.sw = load_scale_word<kStream>(kr, (uint32_t)(e0 + lane));
    };
    KStep cur, nxt;
    load_step(e_begin, cur);
    for (int it = 0; it < ITERS; ++it) {
        const int64_t e0 = e_begin + (int64_t)it * 64;
        if (e0 >= n) break;
        if (it + 1 < ITERS) load_step(e0 + 64, nxt);
        float p[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            TileOut o;
            mfma_tile(q, step_tile(cur, u, r, g), o);
            p[u] = lane_partial(q, o);
            if (a.head_dots) {
                const int64_t e = e0 + 16 * u + r;
                if (e < n) {
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            a.head_dots[(t * kHeads + 16 * h + 4 * g + i) * a.score_stride + e] = o.d[h][i];
                }
            }
        }
        const float s = combine4(p[0], p[1], p[2], p[3]);
        const int64_t e = e0 + lane;
        const bool valid = e < n;
        if (sc_row && valid) sc_row[e] = s;
        if (bm_row) {
            const float m = max8(valid ? s : -INFINITY);
            if ((lane & 7) == 0 && valid) bm_row[e >> 3] = m;
        }
        cur = nxt;
    }
}

// --------------------------------------------------------------------------------------------
// Pool gather: slot 8i + r of query t is position 8 * blocks[t][i] + r. Every slot in
// [0, 8 * max_blocks) is written (-inf when absent). Grid: x = chunks of slots, y = queries.
template <int ITERS>
__global__ __launch_bounds__(256) void score_gather_kernel(GatherArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t t = blockIdx.y;
    const int64_t slots = (int64_t)a.max_blocks * kBlock;
    const int64_t s_begin = ((int64_t)blockIdx.x * 4 + wave) * (ITERS * 64);
    const int g = lane >> 4, r = lane & 15;
    const int32_t* blk = a.blocks + t * a.blocks_stride;

    // Block ids of one 64-slot step: the four tiles' slots of this lane and the lane's own output
    // slot, read unconditionally (clamped to the row) so that the four key loads of a step are
    // issued back to back instead of each waiting on its own id. The first step's ids and the
    // query need only the kernel arguments and are requested before the query's count and
    // length, so that the kernel's start is two memory round trips before the key loads, not
    // three. (Waves past the slots, in the last block, run with every slot absent and store
    // nothing.)
    auto step_ids = [&](int64_t s0, int32_t (&b)[5]) {
#pragma unroll
        for (int u = 0; u < 5; ++u) {
            const int64_t i = (s0 + (u < 4 ? 16 * u + r : lane)) >> 3;
            b[u] = blk[i < a.max_blocks ? i : a.max_blocks - 1];
        }
    };
    int32_t bc[5];
    step_ids(s_begin, bc);
    QRegs q;
    load_query(a.q_codes, a.q_scales, a.w, t, lane, q);
    int64_t cnt = a.block_count[t];
    cnt = cnt < 0 ? 0 : (cnt > a.max_blocks ? a.max_blocks : cnt);
    int64_t n = a.n_vis[t];
    n = n < 0 ? 0 : (n > kMaxScanKeys ? kMaxScanKeys : n);
    const KeyRange kr = key_range(a.k_codes, a.k_scales, a.k_base[t], n);

    // key indices of a step's slots; absent slots (past the slots, the count or the row, negative
    // ids, positions >= n) map to kAbsent
    auto step_positions = [&](int64_t s0, const int32_t (&b)[5], uint32_t (&pos)[5]) {
#pragma unroll
        for (int u = 0; u < 5; ++u) {
            const int64_t s = s0 + (u < 4 ? 16 * u + r : lane);
            const int64_t e = (int64_t)b[u] * kBlock + (s & 7);
            // bitwise, not short-circuit: no branch for the compiler to sink the id loads into
            const bool ok = (s < slots) & ((s >> 3) < cnt) & (b[u] >= 0) & (e < n);
            pos[u] = ok ? (uint32_t)e : kAbsent;
        }
    };

    // a lane's own slot (pos[4]) is slot 16u + r of tile u for the lanes that read its scale byte
    auto load_step = [&](const uint32_t (&pos)[5], KStep& ks) {
#pragma unroll
        for (int u = 0; u < 4; ++u) ks.b[u] = load_codes<kReuse>(kr, pos[u], g);
        ks.sw = load_scale_word<kReuse>(kr, pos[4]);
    };
    uint32_t pc[5], pn[5] = {kAbsent, kAbsent, kAbsent, kAbsent, kAbsent};
    KStep cur, nxt;
    step_positions(s_begin, bc, pc);
    load_step(pc, cur);
    for (int it = 0; it < ITERS; ++it) {
        const int64_t s0 = s_begin + (int64_t)it * 64;
        if (s0 >= slots) break;
        if (it + 1 < ITERS) {
            int32_t bn[5];
            step_ids(s0 + 64, bn);
            step_positions(s0 + 64, bn, pn);
            load_step(pn, nxt);
        }
        float p[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            TileOut o;
            mfma_tile(q, step_tile(cur, u, r, g), o);
            p[u] = lane_partial(q, o);
            if (a.head_dots && pc[u] != kAbsent) {
                const int64_t s = s0 + 16 * u + r;
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        a.head_dots[(t * kHeads + 16 * h + 4 * g + i) * a.score_stride + s] = o.d[h][i];
            }
        }
        const float sc = combine4(p[0], p[1], p[2], p[3]);
        const int64_t s = s0 + lane;
        if (s < slots) a.scores[t * a.score_stride + s] = pc[4] != kAbsent ? sc : -INFINITY;
        cur = nxt;
#pragma unroll
        for (int u = 0; u < 5; ++u) pc[u] = pn[u];
    }
}

// One 64-key step per wavefront (256 keys per block): the kernel then fits in 64 registers, eight
// wavefronts per SIMD keep the most key loads in flight, and it streams at the rate of a plain read
constexpr int kScanIters = 1;
// Pool gather: one 64-slot step per wavefront when the launch is small (a decode step: the latency
// of a few short-lived waves), several steps when it is large (prefill: the query is loaded once
// per wavefront and the next step's keys are in flight while the current step computes).
constexpr int kGatherIters = 1;
constexpr int kGatherItersMany = 4;
constexpr int64_t kGatherManySlots = (int64_t)1 << 22;  // slots per launch from which the long form runs
}  // namespace

hipError_t launch_score_full(const ScoreArgs& a, hipStream_t stream) {
    if (a.nq <= 0 || a.max_n <= 0) return hipSuccess;
    if (a.group > 1 && a.head_dots == nullptr) return launch_score_multi(a, stream);
    const int64_t per_block = 4 * kScanIters * 64;
    const int64_t gx = (a.max_n + per_block - 1) / per_block;
    hipLaunchKernelGGL(score_full_kernel<kScanIters>, dim3((unsigned)gx, (unsigned)a.nq), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_score_gather(const GatherArgs& a, hipStream_t stream) {
    if (a.nq <= 0 || a.max_blocks <= 0) return hipSuccess;
    const int64_t slots = (int64_t)a.max_blocks * kBlock;
    if ((int64_t)a.nq * slots >= kGatherManySlots) {
        const int64_t per_block = 4 * kGatherItersMany * 64;
        const int64_t gx = (slots + per_block - 1) / per_block;
        hipLaunchKernelGGL(score_gather_kernel<kGatherItersMany>, dim3((unsigned)gx, (unsigned)a.nq), dim3(256), 0,
                           stream, a);
    } else {
        const int64_t per_block = 4 * kGatherIters * 64;
        const int64_t gx = (slots + per_block - 1) / per_block;
        hipLaunchKernelGGL(score_gather_kernel<kGatherIters>, dim3((unsigned)gx, (unsigned)a.nq), dim3(256), 0,
                           stream, a);
    }
    return hipGetLastError();
}

}  // namespace fp4idx
