// Internal declarations of libfp4idx (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4idx {

constexpr int kHeads = 32;
constexpr int kDim = 128;
constexpr int kRowBytes = 64;   // E2M1 codes of one 128-dim row
constexpr int kGroups = 4;      // UE8M0 scales per row (groups of 32)
constexpr int kBlock = 8;       // positions per pool block
constexpr int kMaxK = 2048;
constexpr int kHistBins = 2048; // 11-bit radix digits
// Largest key range one query may scan: key offsets inside a range are 32-bit byte offsets
// (64 B per key) in buffer descriptors.
constexpr int64_t kMaxScanKeys = (int64_t)1 << 24;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// ---- launches (each returns the HIP error of its launch) ----
hipError_t launch_quantize(const uint16_t* x, int64_t rows, const int8_t* signs, uint8_t* codes, uint8_t* scales,
                           hipStream_t stream);

struct ScoreArgs {
    const uint8_t* k_codes;
    const uint8_t* k_scales;
    const int64_t* k_base;
    const int32_t* n_vis;
    int32_t nq;
    int32_t group;
    int64_t max_n;
    const uint8_t* q_codes;
    const uint8_t* q_scales;
    const float* w;
    float* scores;
    int64_t score_stride;
    float* block_max;
    int64_t bm_stride;
    float* head_dots;
};
hipError_t launch_score_full(const ScoreArgs& a, hipStream_t stream);
// many queries per key range (group > 1, no per-head output): the scan above dispatches to it
hipError_t launch_score_multi(const ScoreArgs& a, hipStream_t stream);

struct GatherArgs {
    const uint8_t* k_codes;
    const uint8_t* k_scales;
    const int64_t* k_base;
    const int32_t* n_vis;
    int32_t nq;
    const int32_t* blocks;
    int64_t blocks_stride;
    const int32_t* block_count;
    int32_t max_blocks;
    const uint8_t* q_codes;
    const uint8_t* q_scales;
    const float* w;
    float* scores;
    int64_t score_stride;
    float* head_dots;
};
hipError_t launch_score_gather(const GatherArgs& a, hipStream_t stream);

// Radix selection shared by idx_topk and idx_build_pool.
struct SelectArgs {
    // values: row t has n_t = min(max(nv[t], 0), max_n) values at vals[t * stride + i]
    const float* vals;
    int64_t stride;
    const int32_t* nv;       // may be null (every row has max_n values)
    int32_t nq;
    int64_t max_n;
    int32_t k;
    // pool mode: vals are block maxima, nv are visible positions, the row holds ceil(n_t / 8)
    // values and the block of position n_t - 1 is pinned to +inf; output ascending block ids
    bool pool_mode;
    bool pin;  // pool mode: pin the block of position n_t - 1 (the candidate pool); false ranks raw maxima
    // optional slot -> position map (top-k over pool-order scores)
    const int32_t* map;
    int64_t map_stride;
    // map_values: the map indexes a full score row instead. Row t then holds
    // 8 * min(map_count[t / map_group], map_width) slots, slot s is the value at position
    // p = map[t / map_group][s / 8] * 8 + s % 8 of vals row t, and -inf where p >= n_t or the
    // block id lies outside [0, ceil(n_t / 8))
    bool map_values;
    const int32_t* map_count;
    int32_t map_group;
    int64_t map_width;
    // outputs
    int32_t* out_idx;
    int64_t out_stride;
    float* out_val;          // may be null
    int32_t* out_count;      // may be null
    int32_t pad_to;          // out_idx entries in [count, pad_to) are set to -1
    void* ws;
};
size_t select_workspace_bytes(int32_t nq, int64_t max_n, int32_t k);
// bytes at the start of a selection workspace that hold the per-row counters of rows 0 .. nq - 1
// (zero before a call, restored to zero by it); the rest is written before it is read
size_t select_counter_bytes(int32_t nq);

// training form of the pool: -inf outside the pooled blocks, in place
hipError_t launch_mask_pool(float* scores, int64_t score_stride, const int32_t* n_vis, int32_t nq, int64_t max_n,
                            const int32_t* pool_blocks, int64_t pool_stride, const int32_t* pool_count,
                            int32_t group, hipStream_t stream);

// main-KV codec: rows of 512 values, E2M1 codes with an E4M3 scale per 16 values
hipError_t launch_quantize_kv(const uint16_t* x, int64_t rows, uint8_t* codes, uint8_t* scales, hipStream_t stream);
hipError_t launch_gather_kv(const uint8_t* codes, const uint8_t* scales, const int64_t* kv_base, const int32_t* n_vis,
                            int32_t nq, const int32_t* idx, int64_t idx_stride, int32_t k, uint16_t* out,
                            hipStream_t stream);
hipError_t launch_select(const SelectArgs& a, hipStream_t stream);

}  // namespace fp4idx
