// C-ABI entry points of libfp4idx: host-side validation, then asynchronous launches.
// Every check runs before the first HIP call, so argument errors never touch the device.
#include <stdarg.h>
#include <stdio.h>
#include <mutex>
#include <string>

#include "../../include/fp4idx.h"
#include "internal.h"

using namespace fp4idx;

// ---- scratch of idx_build_pool_noalloc, for callers that cannot allocate ----
// The selection workspace lives in this file-scope device array: one copy on every GPU the
// library runs on, held until the process ends, shared by every call on that GPU (calls that
// overlap on one GPU race). On the host, `scratch` is only a stand-in for the device symbol and is
// never passed to a kernel or a copy: its device address is resolved once per device with
// hipGetSymbolAddress and kept in g_scratch.
constexpr size_t kScratchBytes = (size_t)80 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

thread_local std::string g_last_error;

idx_status fail(idx_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

idx_status ok() {
    g_last_error.clear();
    return IDX_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

idx_status hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(IDX_EHIP, "%s: HIP launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

#define REQUIRE(cond, st, ...)                   \
    do {                                          \
        if (!(cond)) return fail(st, __VA_ARGS__); \
    } while (0)

constexpr int64_t kMaxRows = (int64_t)1 << 36;
constexpr int64_t kMaxN = (int64_t)1 << 30;
constexpr int32_t kMaxQueries = 65535;  // grid y dimension
constexpr int64_t kMaxPoolScoreN = (int64_t)1 << 28;  // a score row read through a pool: below 2^30 bytes

size_t ws_bytes_for(int32_t op, int32_t nq, int64_t max_n, int32_t k) {
    if (nq < 0 || max_n < 0 || max_n > kMaxN || k < 1 || k > kMaxK) return 0;
    if (op == IDX_OP_BUILD_POOL) return select_workspace_bytes(nq, (max_n + kBlock - 1) / kBlock, k);
    if (op == IDX_OP_TOPK) return select_workspace_bytes(nq, max_n, k);
    return 0;
}


// Validation shared by the two pool entry points; fills the selection arguments (all but the
// workspace).
idx_status pool_args(const char* fn, const float* block_max, int64_t bm_stride, const int32_t* n_vis, int32_t nq,
                     int64_t max_n, int32_t topk_blocks, int32_t block, int32_t* pool_blocks, int64_t pool_stride,
                     int32_t* pool_count, bool pin, SelectArgs& a) {
    REQUIRE(block == kBlock, IDX_EUNSUPPORTED, "%s: block=%d (only 8 is implemented)", fn, block);
    REQUIRE(topk_blocks >= 1 && topk_blocks <= kMaxK, IDX_EUNSUPPORTED, "%s: topk_blocks=%d out of [1, 2048]", fn,
            topk_blocks);
    REQUIRE(nq >= 0 && nq <= kMaxQueries, IDX_EUNSUPPORTED, "%s: nq=%d out of [0, 65535]", fn, nq);
    REQUIRE(max_n >= 0 && max_n <= kMaxN, IDX_EINVAL, "%s: max_n=%lld out of [0, 2^30]", fn, (long long)max_n);
    if (nq == 0) return ok();
    REQUIRE(block_max && n_vis && pool_blocks && pool_count, IDX_EINVAL, "%s: null pointer", fn);
    REQUIRE(bm_stride >= (max_n + kBlock - 1) / kBlock, IDX_EINVAL, "%s: bm_stride < ceil(max_n/8)", fn);
    REQUIRE(pool_stride >= topk_blocks, IDX_EINVAL, "%s: pool_stride=%lld < topk_blocks=%d", fn,
            (long long)pool_stride, topk_blocks);
    REQUIRE(aligned(block_max, 4) && aligned(n_vis, 4) && aligned(pool_blocks, 4) && aligned(pool_count, 4),
            IDX_EALIGN, "%s: misaligned pointer", fn);
    a.vals = block_max;
    a.stride = bm_stride;
    a.nv = n_vis;
    a.nq = nq;
    a.max_n = max_n;
    a.k = topk_blocks;
    a.pool_mode = true;
    a.pin = pin;
    a.out_idx = pool_blocks;
    a.out_stride = pool_stride;
    a.out_count = pool_count;
    a.pad_to = topk_blocks;
    return ok();
}


constexpr int kMaxDevices = 64;
struct DeviceScratch {
    void* ptr;             // device address of this device's `scratch`
    int32_t rows_cleared;  // per-row counters [0, rows_cleared) known to be zero
};
std::mutex g_scratch_mu;
DeviceScratch g_scratch[kMaxDevices];

__global__ void clear_bytes_kernel(uint8_t* p, size_t bytes) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < bytes; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

// This device's scratch address; on first use and whenever a call needs the counters of more rows
// than any call before it, those counters are cleared on `stream` (a fill kernel, no memset) before
// the call's own kernels. Every selection call restores the counters it uses to zero.
idx_status device_scratch(int32_t nq, hipStream_t stream, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(IDX_EHIP, "idx_build_pool_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    REQUIRE(dev >= 0 && dev < kMaxDevices, IDX_EUNSUPPORTED, "idx_build_pool_noalloc: device %d above %d", dev,
            kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    DeviceScratch& ds = g_scratch[dev];
    if (!ds.ptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(IDX_EHIP, "idx_build_pool_noalloc: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        ds.ptr = p;
        ds.rows_cleared = 0;
    }
    if (nq > ds.rows_cleared) {
        const size_t from = select_counter_bytes(ds.rows_cleared), to = select_counter_bytes(nq);
        const size_t bytes = to - from;
        const unsigned blocks = (unsigned)((bytes + 255) / 256 < 1024 ? (bytes + 255) / 256 : 1024);
        hipLaunchKernelGGL(clear_bytes_kernel, dim3(blocks), dim3(256), 0, stream, (uint8_t*)ds.ptr + from, bytes);
        e = hipGetLastError();
        if (e != hipSuccess) return fail(IDX_EHIP, "idx_build_pool_noalloc: clear: %s", hipGetErrorString(e));
        ds.rows_cleared = nq;
    }
    *out = ds.ptr;
    return ok();
}

}  // namespace

extern "C" {

int32_t idx_abi_version(void) { return IDX_ABI_VERSION; }

const char* idx_last_error(void) { return g_last_error.c_str(); }

size_t idx_workspace_size(int32_t op, int32_t nq, int64_t max_n, int32_t k) {
    return ws_bytes_for(op, nq, max_n, k);
}

idx_status idx_quantize_q(const uint16_t* x_bf16, int64_t rows, const int8_t* signs, uint8_t* codes,
                          uint8_t* scales, void* stream) {
    REQUIRE(rows >= 0 && rows <= kMaxRows, IDX_EINVAL, "idx_quantize_q: rows=%lld out of [0, 2^36]", (long long)rows);
    if (rows == 0) return ok();
    REQUIRE(x_bf16 && signs && codes && scales, IDX_EINVAL, "idx_quantize_q: null pointer");
    REQUIRE(aligned(x_bf16, 16) && aligned(codes, 16) && aligned(signs, 16) && aligned(scales, 4), IDX_EALIGN,
            "idx_quantize_q: x, codes and signs must be 16-byte aligned, scales 4-byte aligned");
    return hip_status(launch_quantize(x_bf16, rows, signs, codes, scales, (hipStream_t)stream), "idx_quantize_q");
}

idx_status idx_score_full(const uint8_t* k_codes, const uint8_t* k_scales, const int64_t* k_base,
                          const int32_t* n_vis, int32_t nq, int32_t group, int64_t max_n, const uint8_t* q_codes,
                          const uint8_t* q_scales, const float* w, float* scores, int64_t score_stride,
                          float* block_max, int64_t bm_stride, float* head_dots, void* stream) {
    REQUIRE(nq >= 0 && nq <= kMaxQueries, IDX_EUNSUPPORTED, "idx_score_full: nq=%d out of [0, 65535]", nq);
    REQUIRE(max_n >= 0 && max_n <= kMaxScanKeys, IDX_EUNSUPPORTED, "idx_score_full: max_n=%lld out of [0, 2^24]",
            (long long)max_n);
    REQUIRE(group >= 1 && (nq == 0 || nq % group == 0), IDX_EINVAL, "idx_score_full: group=%d must divide nq=%d",
            group, nq);
    REQUIRE(scores || block_max || head_dots, IDX_EINVAL, "idx_score_full: no output requested");
    if (nq == 0 || max_n == 0) return ok();
    REQUIRE(k_codes && k_scales && k_base && n_vis && q_codes && q_scales && w, IDX_EINVAL,
            "idx_score_full: null input pointer");
    REQUIRE(aligned(k_codes, 16) && aligned(q_codes, 16) && aligned(k_scales, 4) && aligned(q_scales, 4) &&
                aligned(w, 4) && aligned(k_base, 8) && aligned(n_vis, 4),
            IDX_EALIGN, "idx_score_full: misaligned input pointer");
    if (scores || head_dots)
        REQUIRE(score_stride >= max_n, IDX_EINVAL, "idx_score_full: score_stride=%lld < max_n=%lld",
                (long long)score_stride, (long long)max_n);
    if (block_max)
        REQUIRE(bm_stride >= (max_n + kBlock - 1) / kBlock, IDX_EINVAL,
                "idx_score_full: bm_stride=%lld < ceil(max_n/8)", (long long)bm_stride);
    REQUIRE((!scores || aligned(scores, 4)) && (!block_max || aligned(block_max, 4)) &&
                (!head_dots || aligned(head_dots, 4)),
            IDX_EALIGN, "idx_score_full: misaligned output pointer");
    ScoreArgs a{k_codes, k_scales, k_base, n_vis, nq, group, max_n, q_codes, q_scales, w,
                scores, score_stride, block_max, bm_stride, head_dots};
    return hip_status(launch_score_full(a, (hipStream_t)stream), "idx_score_full");
}

idx_status idx_build_pool(const float* block_max, int64_t bm_stride, const int32_t* n_vis, int32_t nq,
                          int64_t max_n, int32_t topk_blocks, int32_t block, int32_t* pool_blocks,
                          int64_t pool_stride, int32_t* pool_count, void* ws, size_t ws_bytes, void* stream) {
    SelectArgs a{};
    const idx_status st = pool_args("idx_build_pool", block_max, bm_stride, n_vis, nq, max_n, topk_blocks, block,
                                    pool_blocks, pool_stride, pool_count, true, a);
    if (st != IDX_OK || nq == 0) return st;
    const size_t need = ws_bytes_for(IDX_OP_BUILD_POOL, nq, max_n, topk_blocks);
    REQUIRE(ws && ws_bytes >= need, IDX_EWORKSPACE, "idx_build_pool: workspace %zu bytes, need %zu", ws_bytes, need);
    REQUIRE(aligned(ws, 16), IDX_EALIGN, "idx_build_pool: misaligned workspace");
    a.ws = ws;
    return hip_status(launch_select(a, (hipStream_t)stream), "idx_build_pool");
}

idx_status idx_build_pool_noalloc(const float* block_max, int64_t bm_stride, const int32_t* n_vis, int32_t nq,
                                  int64_t max_n, int32_t topk_blocks, int32_t block, int32_t* pool_blocks,
                                  int64_t pool_stride, int32_t* pool_count, void* stream) {
    SelectArgs a{};
    const idx_status st = pool_args("idx_build_pool_noalloc", block_max, bm_stride, n_vis, nq, max_n, topk_blocks,
                                    block, pool_blocks, pool_stride, pool_count, true, a);
    if (st != IDX_OK || nq == 0) return st;
    const size_t need = ws_bytes_for(IDX_OP_BUILD_POOL, nq, max_n, topk_blocks);
    REQUIRE(need <= kScratchBytes, IDX_EUNSUPPORTED,
            "idx_build_pool_noalloc: nq=%d rows of max_n=%lld positions need %zu bytes of scratch, above the "
            "library's fixed %zu",
            nq, (long long)max_n, need, kScratchBytes);
    void* ptr = nullptr;
    const idx_status sst = device_scratch(nq, (hipStream_t)stream, &ptr);
    if (sst != IDX_OK) return sst;
    a.ws = ptr;
    return hip_status(launch_select(a, (hipStream_t)stream), "idx_build_pool_noalloc");
}

idx_status idx_top_blocks(const float* block_max, int64_t bm_stride, const int32_t* n_vis, int32_t nq, int64_t max_n,
                          int32_t k, int32_t block, int32_t* blocks, int64_t blocks_stride, int32_t* count, void* ws,
                          size_t ws_bytes, void* stream) {
    SelectArgs a{};
    const idx_status st = pool_args("idx_top_blocks", block_max, bm_stride, n_vis, nq, max_n, k, block, blocks,
                                    blocks_stride, count, false, a);
    if (st != IDX_OK || nq == 0) return st;
    const size_t need = ws_bytes_for(IDX_OP_BUILD_POOL, nq, max_n, k);
    REQUIRE(ws && ws_bytes >= need, IDX_EWORKSPACE, "idx_top_blocks: workspace %zu bytes, need %zu", ws_bytes, need);
    REQUIRE(aligned(ws, 16), IDX_EALIGN, "idx_top_blocks: misaligned workspace");
    a.ws = ws;
    return hip_status(launch_select(a, (hipStream_t)stream), "idx_top_blocks");
}

idx_status idx_score_pool_gather(const uint8_t* k_codes, const uint8_t* k_scales, const int64_t* k_base,
                                 const int32_t* n_vis, int32_t nq, const int32_t* blocks, int64_t blocks_stride,
                                 const int32_t* block_count, int32_t max_blocks, int32_t block,
                                 const uint8_t* q_codes, const uint8_t* q_scales, const float* w, float* scores,
                                 int64_t score_stride, float* head_dots, void* stream) {
    REQUIRE(block == kBlock, IDX_EUNSUPPORTED, "idx_score_pool_gather: block=%d (only 8 is implemented)", block);
    REQUIRE(nq >= 0 && nq <= kMaxQueries, IDX_EUNSUPPORTED, "idx_score_pool_gather: nq=%d out of [0, 65535]", nq);
    REQUIRE(max_blocks >= 0 && max_blocks <= (1 << 20), IDX_EINVAL,
            "idx_score_pool_gather: max_blocks=%d out of [0, 2^20]", max_blocks);
    if (nq == 0 || max_blocks == 0) return ok();
    REQUIRE(k_codes && k_scales && k_base && n_vis && blocks && block_count && q_codes && q_scales && w && scores,
            IDX_EINVAL, "idx_score_pool_gather: null pointer");
    REQUIRE(blocks_stride >= max_blocks, IDX_EINVAL, "idx_score_pool_gather: blocks_stride < max_blocks");
    REQUIRE(score_stride >= (int64_t)max_blocks * kBlock, IDX_EINVAL,
            "idx_score_pool_gather: score_stride < 8 * max_blocks");
    REQUIRE(aligned(k_codes, 16) && aligned(q_codes, 16) && aligned(k_scales, 4) && aligned(q_scales, 4) &&
                aligned(w, 4) && aligned(k_base, 8) && aligned(n_vis, 4) && aligned(blocks, 4) &&
                aligned(block_count, 4) && aligned(scores, 4) && (!head_dots || aligned(head_dots, 4)),
            IDX_EALIGN, "idx_score_pool_gather: misaligned pointer");
    GatherArgs a{k_codes, k_scales, k_base, n_vis, nq, blocks, blocks_stride, block_count, max_blocks,
                 q_codes, q_scales, w, scores, score_stride, head_dots};
    return hip_status(launch_score_gather(a, (hipStream_t)stream), "idx_score_pool_gather");
}

idx_status idx_topk(const float* scores, int64_t score_stride, const int32_t* n_valid, int32_t nq, int64_t max_n,
                    int32_t k, const int32_t* blocks, int64_t blocks_stride, int32_t block, int32_t* out_idx,
                    int64_t out_stride, float* out_val, void* ws, size_t ws_bytes, void* stream) {
    REQUIRE(k >= 1 && k <= kMaxK, IDX_EUNSUPPORTED, "idx_topk: k=%d out of [1, 2048]", k);
    REQUIRE(nq >= 0 && nq <= kMaxQueries, IDX_EUNSUPPORTED, "idx_topk: nq=%d out of [0, 65535]", nq);
    REQUIRE(max_n >= 0 && max_n <= kMaxN, IDX_EINVAL, "idx_topk: max_n=%lld out of [0, 2^30]", (long long)max_n);
    if (blocks) REQUIRE(block == kBlock, IDX_EUNSUPPORTED, "idx_topk: block=%d (only 8 is implemented)", block);
    if (nq == 0) return ok();
    REQUIRE(scores && out_idx, IDX_EINVAL, "idx_topk: null pointer");
    REQUIRE(score_stride >= max_n, IDX_EINVAL, "idx_topk: score_stride < max_n");
    REQUIRE(out_stride >= k, IDX_EINVAL, "idx_topk: out_stride < k");
    if (blocks)
        REQUIRE(blocks_stride >= (max_n + kBlock - 1) / kBlock, IDX_EINVAL, "idx_topk: blocks_stride < ceil(max_n/8)");
    const size_t need = ws_bytes_for(IDX_OP_TOPK, nq, max_n, k);
    REQUIRE(ws && ws_bytes >= need, IDX_EWORKSPACE, "idx_topk: workspace %zu bytes, need %zu", ws_bytes, need);
    REQUIRE(aligned(ws, 16) && aligned(scores, 4) && aligned(out_idx, 4) && (!out_val || aligned(out_val, 4)) &&
                (!n_valid || aligned(n_valid, 4)) && (!blocks || aligned(blocks, 4)),
            IDX_EALIGN, "idx_topk: misaligned pointer");
    SelectArgs a{};
    a.vals = scores;
    a.stride = score_stride;
    a.nv = n_valid;
    a.nq = nq;
    a.max_n = max_n;
    a.k = k;
    a.pool_mode = false;
    a.map = blocks;
    a.map_stride = blocks_stride;
    a.out_idx = out_idx;
    a.out_stride = out_stride;
    a.out_val = out_val;
    a.out_count = nullptr;
    a.pad_to = k;
    a.ws = ws;
    return hip_status(launch_select(a, (hipStream_t)stream), "idx_topk");
}

idx_status idx_topk_pool(const float* scores, int64_t score_stride, const int32_t* n_vis, int32_t nq, int64_t max_n,
                         const int32_t* pool_blocks, int64_t pool_stride, const int32_t* pool_count,
                         int32_t max_blocks, int32_t group, int32_t block, int32_t k, int32_t* out_idx,
                         int64_t out_stride, float* out_val, void* stream) {
    REQUIRE(k >= 1 && k <= kMaxK, IDX_EUNSUPPORTED, "idx_topk_pool: k=%d out of [1, 2048]", k);
    REQUIRE(nq >= 0 && nq <= kMaxQueries, IDX_EUNSUPPORTED, "idx_topk_pool: nq=%d out of [0, 65535]", nq);
    REQUIRE(max_n >= 0 && max_n <= kMaxPoolScoreN, IDX_EUNSUPPORTED, "idx_topk_pool: max_n=%lld out of [0, 2^28]",
            (long long)max_n);
    REQUIRE(block == kBlock, IDX_EUNSUPPORTED, "idx_topk_pool: block=%d (only 8 is implemented)", block);
    REQUIRE(max_blocks >= 0 && max_blocks <= kMaxK, IDX_EUNSUPPORTED, "idx_topk_pool: max_blocks=%d out of [0, 2048]",
            max_blocks);
    REQUIRE(group >= 1 && (nq == 0 || nq % group == 0), IDX_EINVAL, "idx_topk_pool: group=%d must divide nq=%d",
            group, nq);
    if (nq == 0) return ok();
    REQUIRE(scores && n_vis && pool_blocks && pool_count && out_idx, IDX_EINVAL, "idx_topk_pool: null pointer");
    REQUIRE(score_stride >= max_n, IDX_EINVAL, "idx_topk_pool: score_stride=%lld < max_n=%lld",
            (long long)score_stride, (long long)max_n);
    REQUIRE(pool_stride >= max_blocks, IDX_EINVAL, "idx_topk_pool: pool_stride=%lld < max_blocks=%d",
            (long long)pool_stride, max_blocks);
    REQUIRE(out_stride >= k, IDX_EINVAL, "idx_topk_pool: out_stride < k");
    REQUIRE(aligned(scores, 4) && aligned(n_vis, 4) && aligned(pool_blocks, 4) && aligned(pool_count, 4) &&
                aligned(out_idx, 4) && (!out_val || aligned(out_val, 4)),
            IDX_EALIGN, "idx_topk_pool: pointers must be 4-byte aligned");
    SelectArgs a{};
    a.vals = scores;
    a.stride = score_stride;
    a.nv = n_vis;
    a.nq = nq;
    a.max_n = max_n;
    a.k = k;
    a.pool_mode = false;
    a.map = pool_blocks;
    a.map_stride = pool_stride;
    a.map_values = true;
    a.map_count = pool_count;
    a.map_group = group;
    a.map_width = max_blocks;
    a.out_idx = out_idx;
    a.out_stride = out_stride;
    a.out_val = out_val;
    a.out_count = nullptr;
    a.pad_to = k;
    a.ws = nullptr;
    return hip_status(launch_select(a, (hipStream_t)stream), "idx_topk_pool");
}

idx_status idx_quantize_kv(const uint16_t* x_bf16, int64_t rows, uint8_t* codes, uint8_t* scales, void* stream) {
    REQUIRE(rows >= 0 && rows <= (int64_t)1 << 31, IDX_EINVAL, "idx_quantize_kv: rows=%lld out of [0, 2^31]",
            (long long)rows);
    if (rows == 0) return ok();
    REQUIRE(x_bf16 && codes && scales, IDX_EINVAL, "idx_quantize_kv: null pointer");
    REQUIRE(aligned(x_bf16, 16) && aligned(codes, 4) && aligned(scales, 1), IDX_EALIGN,
            "idx_quantize_kv: x must be 16-byte aligned, codes 4-byte aligned");
    return hip_status(launch_quantize_kv(x_bf16, rows, codes, scales, (hipStream_t)stream), "idx_quantize_kv");
}

idx_status idx_gather_kv(const uint8_t* codes, const uint8_t* scales, const int64_t* kv_base, const int32_t* n_vis,
                         int32_t nq, const int32_t* idx, int64_t idx_stride, int32_t k, uint16_t* out,
                         void* stream) {
    REQUIRE(nq >= 0 && k >= 0, IDX_EINVAL, "idx_gather_kv: nq=%d, k=%d must be >= 0", nq, k);
    REQUIRE(nq <= kMaxQueries, IDX_EUNSUPPORTED, "idx_gather_kv: nq=%d above 65535", nq);
    REQUIRE((int64_t)nq * k <= (int64_t)1 << 31, IDX_EUNSUPPORTED, "idx_gather_kv: nq * k above 2^31");
    if (nq == 0 || k == 0) return ok();
    REQUIRE(codes && scales && kv_base && n_vis && idx && out, IDX_EINVAL, "idx_gather_kv: null pointer");
    REQUIRE(idx_stride >= k, IDX_EINVAL, "idx_gather_kv: idx_stride=%lld < k=%d", (long long)idx_stride, k);
    REQUIRE(aligned(codes, 4) && aligned(kv_base, 8) && aligned(n_vis, 4) && aligned(idx, 4) && aligned(out, 16),
            IDX_EALIGN, "idx_gather_kv: codes, n_vis and idx must be 4-byte, kv_base 8-byte, out 16-byte aligned");
    return hip_status(launch_gather_kv(codes, scales, kv_base, n_vis, nq, idx, idx_stride, k, out, (hipStream_t)stream),
                      "idx_gather_kv");
}

idx_status idx_mask_pool(float* scores, int64_t score_stride, const int32_t* n_vis, int32_t nq, int64_t max_n,
                         const int32_t* pool_blocks, int64_t pool_stride, const int32_t* pool_count, int32_t group,
                         int32_t block, void* stream) {
    REQUIRE(nq >= 0 && nq <= kMaxQueries, IDX_EUNSUPPORTED, "idx_mask_pool: nq=%d out of [0, 65535]", nq);
    REQUIRE(max_n >= 0 && max_n <= kMaxN, IDX_EUNSUPPORTED, "idx_mask_pool: max_n=%lld out of [0, 2^30]",
            (long long)max_n);
    REQUIRE(block == kBlock, IDX_EUNSUPPORTED, "idx_mask_pool: block=%d (only %d)", block, kBlock);
    REQUIRE(group >= 1 && (nq == 0 || nq % group == 0), IDX_EINVAL, "idx_mask_pool: group=%d must divide nq=%d",
            group, nq);
    if (nq == 0 || max_n == 0) return ok();
    REQUIRE(scores && n_vis && pool_blocks && pool_count, IDX_EINVAL, "idx_mask_pool: null pointer");
    REQUIRE(score_stride >= max_n, IDX_EINVAL, "idx_mask_pool: score_stride=%lld < max_n", (long long)score_stride);
    REQUIRE(pool_stride >= 0, IDX_EINVAL, "idx_mask_pool: negative pool_stride");
    REQUIRE(aligned(scores, 4) && aligned(n_vis, 4) && aligned(pool_blocks, 4) && aligned(pool_count, 4), IDX_EALIGN,
            "idx_mask_pool: pointers must be 4-byte aligned");
    return hip_status(launch_mask_pool(scores, score_stride, n_vis, nq, max_n, pool_blocks, pool_stride, pool_count,
                                       group, (hipStream_t)stream),
                      "idx_mask_pool");
}

}  // extern "C"
