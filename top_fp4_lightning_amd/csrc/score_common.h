// Helpers shared by the indexer scoring kernels (single-query scan, pool gather, many-query
// scan): range-checked key descriptors, ReLU on the bit pattern, block-8 maxima across lanes.
//
// Keys are read with buffer loads through a descriptor that spans exactly one query's (or one
// group's) key range: reads past the range return zeros (zero codes contribute nothing), so
// there are no per-lane branches around loads and offsets are 32-bit.
#pragma once

#include "internal.h"

namespace fp4idx {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format, range checked

// FP4 operands occupy the low four registers of the instruction's 8-register operand
__device__ __forceinline__ v8i widen(v4i x) { return v8i{x[0], x[1], x[2], x[3], 0, 0, 0, 0}; }

// one query's (or group's) key rows [base, base + n) as two range-checked buffers
struct KeyRange {
    __amdgpu_buffer_rsrc_t codes;
    __amdgpu_buffer_rsrc_t scales;
};

__device__ __forceinline__ KeyRange key_range(const uint8_t* k_codes, const uint8_t* k_scales, int64_t base,
                                              int64_t n) {
    KeyRange r;
    r.codes = __builtin_amdgcn_make_buffer_rsrc((void*)(k_codes + base * kRowBytes), 0, (int)(n * kRowBytes),
                                                kRsrcWord3);
    r.scales = __builtin_amdgcn_make_buffer_rsrc((void*)(k_scales + base * kGroups), 0, (int)(n * kGroups),
                                                 kRsrcWord3);
    return r;
}

// cache policy of key loads: kStream marks them non-temporal (a scan reads each key once and
// should not displace reusable lines), kReuse keeps the default policy (pooled keys are re-read by
// later layers, prefill keys by other query tiles)
constexpr int kReuse = 0;
constexpr int kStream = 2;

// ReLU on the fp32 bit pattern: as a signed integer every negative float (and -0) is below 0,
// every positive float keeps its bits; one integer max, no NaN canonicalisation
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// lane move inside the data-parallel-primitive network (no LDS round trip)
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// maximum over each aligned group of 8 lanes, in all 8 lanes (the scoring sources are built
// without NaN semantics, so each step is one max with the lane move folded in)
__device__ __forceinline__ float max8(float v) {
    v = fmaxf(v, dpp_mov<0xB1>(v));   // quad_perm [1,0,3,2]: partner lane ^ 1
    v = fmaxf(v, dpp_mov<0x4E>(v));   // quad_perm [2,3,0,1]: partner lane ^ 2
    v = fmaxf(v, dpp_mov<0x141>(v));  // row_half_mirror: lane i <-> 7 - i, i.e. the other quad
    return v;
}

}  // namespace
}  // namespace fp4idx
