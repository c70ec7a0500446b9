// Random-Hadamard rotation + MXFP4 quantisation of 128-dim rows (indexer queries and keys).
//
// Rotation: sign flip, then the Sylvester Walsh-Hadamard transform computed as a fast transform
// in fp64 (every partial sum of bf16 inputs is exact), then fl32(S) * fl32(2^-3.5) in fp32.
// Scale: smallest e with 6 * 2^e >= group max (the ideal max/6 rounded up to a power of two).
// Codes: E2M1 by threshold comparison on y / 2^e (nearest, ties to the even mantissa bit).
// Layout: 16 lanes per row (lane i owns elements 8i .. 8i+7), or a wavefront per row (elements
// 2i, 2i+1) for small launches.
#include "internal.h"

namespace fp4idx {
namespace {

// Partner exchange inside each 16-lane row through the data-parallel-primitive network (a few
// cycles, no LDS round trip): the value of lane li ^ M. M = 1, 2: quad permutations; M = 8: a
// rotation of the row by 8; M = 4: a shift by 4 up or down, chosen by the lane's bit 2.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
template <int M>
__device__ __forceinline__ uint32_t xor_lane32(uint32_t v, int li) {
    if constexpr (M == 1) return dpp32<0xB1>(v);   // quad_perm [1,0,3,2]
    if constexpr (M == 2) return dpp32<0x4E>(v);   // quad_perm [2,3,0,1]
    if constexpr (M == 8) return dpp32<0x128>(v);  // row_ror:8
    if constexpr (M == 4) {
        const uint32_t up = dpp32<0x104>(v);  // row_shl:4, the value of lane li + 4
        const uint32_t dn = dpp32<0x114>(v);  // row_shr:4, the value of lane li - 4
        return (li & 4) ? dn : up;
    }
    if constexpr (M == 32) {
        // swap of the two 32-lane halves: the first result holds (low, low), the second (high, high)
        const auto sw = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (li & 32) ? sw[0] : sw[1];
    }
    if constexpr (M == 16) {
        // swap of neighbouring 16-lane rows: the first result holds rows (0, 0, 2, 2), the
        // second rows (1, 1, 3, 3)
        const auto sw = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (li & 16) ? sw[0] : sw[1];
    }
    return v;
}
template <int M>
__device__ __forceinline__ double xor_lane(double v, int li) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = xor_lane32<M>((uint32_t)b, li), hi = xor_lane32<M>((uint32_t)(b >> 32), li);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
template <int M>
__device__ __forceinline__ float xor_lanef(float v, int li) {
    return __uint_as_float(xor_lane32<M>(__float_as_uint(v), li));
}

// E2M1 code (0..7) of a magnitude v in [0, 6]: nearest grid value, ties to even mantissa
__device__ __forceinline__ uint32_t e2m1_mag_code(float a) {
    uint32_t c;
    if (a <= 0.25f) c = 0;
    else if (a < 0.75f) c = 1;
    else if (a <= 1.25f) c = 2;
    else if (a < 1.75f) c = 3;
    else if (a <= 2.5f) c = 4;
    else if (a < 3.5f) c = 5;
    else if (a <= 5.0f) c = 6;
    else c = 7;
    return c;
}

// one butterfly stage over lane bit M (element-index bit M * EPL)
template <int M, int EPL>
__device__ __forceinline__ void lane_stage(double (&v)[EPL], int li) {
    const bool upper = (li & M) != 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const double p = xor_lane<M>(v[i], li);
        v[i] = upper ? (p - v[i]) : (v[i] + p);
    }
}

// LPR lanes per row, EPL = 128 / LPR consecutive elements per lane: 16 lanes (8 elements) for
// large launches (fewer instructions per row), 64 lanes (2 elements) for small ones (the query
// rows of a decode step: the least dependent work per lane, so the shortest path through the
// kernel).
template <int LPR>
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                       const int8_t* __restrict__ signs, uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
    constexpr int EPL = kDim / LPR;      // elements per lane
    constexpr int GL = 32 / EPL;         // lanes per 32-element scale group
    const int li = threadIdx.x & (LPR - 1);
    const int64_t row = (int64_t)blockIdx.x * (256 / LPR) + (threadIdx.x / LPR);
    const bool live = row < rows;  // dead lanes still join the lane exchanges of their row group

    uint32_t words[EPL / 2] = {};
    uint32_t sw[EPL >= 4 ? EPL / 4 : 1];
    if constexpr (EPL == 8) {
        if (live) {
            const uint4 raw = *reinterpret_cast<const uint4*>(x + row * kDim + li * 8);
            words[0] = raw.x; words[1] = raw.y; words[2] = raw.z; words[3] = raw.w;
        }
        const uint2 sg = *reinterpret_cast<const uint2*>(signs + li * 8);
        sw[0] = sg.x;
        sw[1] = sg.y;
    } else if constexpr (EPL == 4) {
        if (live) {
            const uint2 raw = *reinterpret_cast<const uint2*>(x + row * kDim + li * 4);
            words[0] = raw.x; words[1] = raw.y;
        }
        sw[0] = *reinterpret_cast<const uint32_t*>(signs + li * 4);
    } else {
        if (live) words[0] = *reinterpret_cast<const uint32_t*>(x + row * kDim + li * 2);
        sw[0] = *reinterpret_cast<const uint16_t*>(signs + li * 2);
    }

    double v[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        uint32_t h = (i & 1) ? (words[i >> 1] >> 16) : (words[i >> 1] & 0xffffu);
        float f = __uint_as_float(h << 16);
        int s = (int)(int8_t)((sw[i >> 2] >> (8 * (i & 3))) & 0xffu);
        v[i] = (double)f * (double)s;
    }
    // butterflies over the element-index bits inside the lane
#pragma unroll
    for (int b = 1; b < EPL; b <<= 1) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            if (!(i & b)) {
                double p = v[i], q = v[i | b];
                v[i] = p + q;
                v[i | b] = p - q;
            }
        }
    }
    // butterflies over the lane bits (element-index bits EPL .. 64)
    lane_stage<1, EPL>(v, li);
    lane_stage<2, EPL>(v, li);
    lane_stage<4, EPL>(v, li);
    lane_stage<8, EPL>(v, li);
    if constexpr (LPR >= 32) lane_stage<16, EPL>(v, li);
    if constexpr (LPR >= 64) lane_stage<32, EPL>(v, li);
    const float inv = 0x1.6a09e6p-4f;  // fl32(2^-3.5)
    float y[EPL];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        float s32 = (float)v[i];
        y[i] = s32 * inv;
        amax = fmaxf(amax, fabsf(y[i]));
    }
    // group of 32 = GL consecutive lanes
    amax = fmaxf(amax, xor_lanef<1>(amax, li));
    amax = fmaxf(amax, xor_lanef<2>(amax, li));
    if constexpr (GL >= 8) amax = fmaxf(amax, xor_lanef<4>(amax, li));
    if constexpr (GL >= 16) amax = fmaxf(amax, xor_lanef<8>(amax, li));

    int e = -127;
    if (amax > 0.0f) {
        int E;
        const float m = frexpf(amax, &E);  // amax = m * 2^E, 0.5 <= m < 1 (exact, subnormals too)
        e = (m <= 0.75f) ? E - 3 : E - 2;
        e = e < -127 ? -127 : (e > 127 ? 127 : e);
    }
    // y / 2^e in fp32: exact whenever the result is at least 2^-126, and a smaller magnitude
    // encodes to 0 however it rounds; |y / 2^e| <= 6 by the choice of e
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const float vd = ldexpf(y[i], -e);
        uint32_t c = e2m1_mag_code(fabsf(vd));
        if (c != 0 && vd < 0.0f) c |= 8u;
        packed |= c << (4 * i);
    }
    if (live) {
        if constexpr (EPL == 8)
            *reinterpret_cast<uint32_t*>(codes + row * kRowBytes + li * 4) = packed;
        else if constexpr (EPL == 4)
            *reinterpret_cast<uint16_t*>(codes + row * kRowBytes + li * 2) = (uint16_t)packed;
        else
            codes[row * kRowBytes + li] = (uint8_t)packed;
        if (li % GL == 0) scales[row * kGroups + li / GL] = (uint8_t)(e + 127);
    }
}

// launches up to this many rows take a whole wavefront per row (two elements per lane: the
// shortest path through the kernel; 32 lanes per row measured 1.5 us slower per decode step)
constexpr int64_t kSmallQuantRows = 4096;
constexpr int kSmallQuantLanes = 64;

}  // namespace

hipError_t launch_quantize(const uint16_t* x, int64_t rows, const int8_t* signs, uint8_t* codes, uint8_t* scales,
                           hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    if (rows <= kSmallQuantRows) {
        constexpr int L = kSmallQuantLanes;
        const int64_t blocks = (rows + 256 / L - 1) / (256 / L);
        hipLaunchKernelGGL(quantize_kernel<L>, dim3((unsigned)blocks), dim3(256), 0, stream, x, rows, signs, codes,
                           scales);
    } else {
        const int64_t blocks = (rows + 15) / 16;
        hipLaunchKernelGGL(quantize_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, stream, x, rows, signs, codes,
                           scales);
    }
    return hipGetLastError();
}

}  // namespace fp4idx
