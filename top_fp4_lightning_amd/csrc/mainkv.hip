// Main-KV FP4 codec on gfx950: rows of 512 values stored as E2M1 codes with one E4M3 scale per
// 16 values and no global scale (256 + 32 bytes per entry), and the gather of the selected
// entries dequantised to bf16 for core attention ("DeepSeek-V4.1 model structure (3)",
// sections "the scale format decides precision" and "removing the global scale still leaves
// enough range").
//
// Both kernels are HBM-bound streams: one wavefront per row / selected entry, lane l owning the
// 8 values 8l .. 8l + 7 (16 bytes of bf16, one dword of codes, half a scale group).
//
// Quantisation decides every code by exact comparisons: the scale s is an E4M3 value (at most
// 4 significant bits), so 6 * s and the E2M1 midpoints t * s (t = 0.25 .. 5, at most 3 bits) are
// exact in fp32 and |x| is compared with them directly; no division is rounded.
#include "internal.h"

namespace fp4idx {
namespace {

constexpr int kMkvDim = 512;
constexpr int kMkvGroup = 16;
constexpr int kMkvCodeBytes = kMkvDim / 2;            // 256
constexpr int kMkvScales = kMkvDim / kMkvGroup;       // 32
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// E4M3 ("fn" variant: exponent bias 7, exponent field 0 subnormal, no infinities) byte -> value
__device__ __forceinline__ float e4m3_value(uint32_t b) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    const float mag = e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
    return (b & 0x80u) ? -mag : mag;
}

// smallest positive-byte E4M3 value s with 6 * s >= a (a >= 0 finite); bytes 0x00 .. 0x7e are
// ascending in value, so a binary search over them; saturates at 0x7e (448)
__device__ __forceinline__ uint32_t e4m3_scale_for(float a) {
    uint32_t lo = 0, hi = 0x7e;  // invariant: the answer is in [lo, hi]
#pragma unroll
    for (int it = 0; it < 7; ++it) {
        const uint32_t mid = (lo + hi) >> 1;
        if (6.0f * e4m3_value(mid) >= a)
            hi = mid;
        else
            lo = mid + 1;
    }
    return lo < 0x7e ? lo : 0x7e;
}

// E2M1 code of x for scale s > 0: the number of midpoints below |x|, a tie going to the even
// code (the midpoints 0.75, 1.75 and 3.5 lie below an even code: >=, the others: >)
__device__ __forceinline__ uint32_t e2m1_code(float x, float s) {
    const float a = fabsf(x);
    uint32_t c = (a > 0.25f * s) + (a >= 0.75f * s) + (a > 1.25f * s) + (a >= 1.75f * s) + (a > 2.5f * s) +
                 (a >= 3.5f * s) + (a > 5.0f * s);
    return (c != 0 && __float_as_uint(x) >> 31) ? (c | 8u) : c;
}

__device__ __forceinline__ float bf16f(uint32_t h) { return __uint_as_float(h << 16); }

__global__ __launch_bounds__(256) void quantize_kv_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;  // uniform per wave
    const uint4 v = *reinterpret_cast<const uint4*>(x + r * kMkvDim + 8 * lane);
    float f[8];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16f(w[i] & 0xffffu);
        f[2 * i + 1] = bf16f(w[i] >> 16);
    }
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(f[i]));
    // the group of 16 is this lane and its neighbour (lane ^ 1)
    a = fmaxf(a, __shfl_xor(a, 1));
    const uint32_t sb = e4m3_scale_for(a);
    const float s = e4m3_value(sb);
    uint32_t word = 0;
    if (s > 0.0f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) word |= e2m1_code(f[i], s) << (4 * i);
    }
    reinterpret_cast<uint32_t*>(codes + r * kMkvCodeBytes)[lane] = word;
    if ((lane & 1) == 0) scales[r * kMkvScales + (lane >> 1)] = (uint8_t)sb;
}

// E2M1 nibble -> value (sign bit 3; magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6)
__device__ __forceinline__ float e2m1_value(uint32_t n) {
    const uint32_t m = n & 7u;
    const uint32_t bits = m >= 2 ? ((((m >> 1) + 126u) << 23) | ((m & 1u) << 22)) : (m == 1 ? 0x3f000000u : 0u);
    return __uint_as_float(bits | ((n & 8u) << 28));
}

// one wavefront per selected entry; EPW consecutive entries of one query per wavefront, their
// loads issued before any is used. Grid: x = chunks of 4 * EPW entries, y = queries.
template <int EPW>
__global__ __launch_bounds__(256) void gather_kv_kernel(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ scales,
                                                        const int64_t* __restrict__ kv_base,
                                                        const int32_t* __restrict__ n_vis,
                                                        const int32_t* __restrict__ idx, int64_t idx_stride,
                                                        int32_t k, uint16_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t t = blockIdx.y;
    // the wave's first entry, uniform across the wave
    const int i0 = __builtin_amdgcn_readfirstlane(((int)blockIdx.x * 4 + (int)(threadIdx.x >> 6)) * EPW);
    if (i0 >= k) return;
    const int64_t base = kv_base[t];
    const int64_t n = n_vis[t];
    const int32_t* sel = idx + t * idx_stride;
    // all EPW positions first (clamped to the row), so that no row load waits on the next position
    int64_t pos[EPW];
#pragma unroll
    for (int j = 0; j < EPW; ++j) {
        const int i = i0 + j;
        pos[j] = sel[i < k ? i : k - 1];
        if (i >= k) pos[j] = -1;
    }
    uint32_t cw[EPW], sb[EPW];
    bool ok[EPW];
#pragma unroll
    for (int j = 0; j < EPW; ++j) {
        const int64_t p = pos[j];
        ok[j] = p >= 0 && p < n;
        cw[j] = 0;
        sb[j] = 0;
        if (ok[j]) {
            const int64_t row = base + p;
            cw[j] = reinterpret_cast<const uint32_t*>(codes + row * kMkvCodeBytes)[lane];
            sb[j] = scales[row * kMkvScales + (lane >> 1)];
        }
    }
    uint16_t* orow = out + (t * k + i0) * (int64_t)kMkvDim;
#pragma unroll
    for (int j = 0; j < EPW; ++j) {
        if (i0 + j >= k) continue;
        uint32_t o[4] = {0u, 0u, 0u, 0u};
        if (ok[j]) {
            const float s = e4m3_value(sb[j]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // products of an E2M1 value and an E4M3 scale have at most 6 significant bits:
                // exact in bf16, so the top half of the fp32 pattern is the bf16 value
                const uint32_t lo = __float_as_uint(e2m1_value(cw[j] >> (8 * i)) * s) >> 16;
                const uint32_t hi = __float_as_uint(e2m1_value(cw[j] >> (8 * i + 4)) * s) >> 16;
                o[i] = lo | (hi << 16);
            }
        }
        // the rows go to core attention, not back through this kernel: stream them past the caches
        __builtin_nontemporal_store(v4u{o[0], o[1], o[2], o[3]},
                                    reinterpret_cast<v4u*>(orow + j * kMkvDim + 8 * lane));
    }
}

constexpr int kGatherEPW = 4;  // entries per wavefront (2 and 4 measured equal, 8 and 16 slower)

}  // namespace

hipError_t launch_quantize_kv(const uint16_t* x, int64_t rows, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    const int64_t blocks = (rows + 3) / 4;
    hipLaunchKernelGGL(quantize_kv_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, rows, codes, scales);
    return hipGetLastError();
}

hipError_t launch_gather_kv(const uint8_t* codes, const uint8_t* scales, const int64_t* kv_base, const int32_t* n_vis,
                            int32_t nq, const int32_t* idx, int64_t idx_stride, int32_t k, uint16_t* out,
                            hipStream_t stream) {
    if (nq <= 0 || k <= 0) return hipSuccess;
    const int per_block = 4 * kGatherEPW;
    const dim3 grid((unsigned)((k + per_block - 1) / per_block), (unsigned)nq);
    hipLaunchKernelGGL(gather_kv_kernel<kGatherEPW>, grid, dim3(256), 0, stream, codes, scales, kv_base, n_vis, idx,
                       idx_stride, k, out);
    return hipGetLastError();
}

}  // namespace fp4idx
