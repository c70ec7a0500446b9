// The candidate pool in its training form ("DeepSeek-V4.1 model structure (3)", sections "three
// details of the pool in the code" and "the pool also acts in training"): a Reindex layer that
// scores every visible position sets the positions outside the pooled blocks to -inf before its
// top-512. In place over a score row; one block per chunk of 16384 positions marks its 2048
// block ids from the pool list in an LDS bitmap, then streams the chunk.
#include "internal.h"

namespace fp4idx {
namespace {

constexpr int kMaskThreads = 256;
constexpr int kMaskChunk = 16384;                 // positions per block
constexpr int kMaskBlocks = kMaskChunk / kBlock;  // pool blocks per chunk: 2048 bits
constexpr int kMaskWords = kMaskBlocks / 32;

__global__ __launch_bounds__(kMaskThreads) void mask_pool_kernel(float* __restrict__ scores, int64_t score_stride,
                                                                 const int32_t* __restrict__ n_vis, int64_t max_n,
                                                                 const int32_t* __restrict__ pool_blocks,
                                                                 int64_t pool_stride,
                                                                 const int32_t* __restrict__ pool_count, int32_t group) {
    __shared__ uint32_t keep[kMaskWords];
    const int64_t t = blockIdx.y;
    int64_t n = n_vis[t];
    n = n < 0 ? 0 : (n > max_n ? max_n : n);
    const int64_t s0 = (int64_t)blockIdx.x * kMaskChunk;
    if (s0 >= n) return;  // uniform per block
    const int64_t b0 = s0 / kBlock;
    for (int i = threadIdx.x; i < kMaskWords; i += kMaskThreads) keep[i] = 0u;
    __syncthreads();
    const int64_t p = t / group;
    int64_t cnt = pool_count[p];
    cnt = cnt < 0 ? 0 : (cnt > pool_stride ? pool_stride : cnt);
    const int32_t* pool = pool_blocks + p * pool_stride;
    for (int64_t i = threadIdx.x; i < cnt; i += kMaskThreads) {
        const int64_t b = (int64_t)pool[i] - b0;
        if (b >= 0 && b < kMaskBlocks) atomicOr(&keep[b >> 5], 1u << (b & 31));
    }
    __syncthreads();
    float* row = scores + t * score_stride;
    const int64_t end = s0 + kMaskChunk < n ? s0 + kMaskChunk : n;
    for (int64_t s = s0 + threadIdx.x; s < end; s += kMaskThreads) {
        const int64_t b = s / kBlock - b0;
        if (((keep[b >> 5] >> (b & 31)) & 1u) == 0) row[s] = -INFINITY;
    }
}

}  // namespace

hipError_t launch_mask_pool(float* scores, int64_t score_stride, const int32_t* n_vis, int32_t nq, int64_t max_n,
                            const int32_t* pool_blocks, int64_t pool_stride, const int32_t* pool_count,
                            int32_t group, hipStream_t stream) {
    if (nq <= 0 || max_n <= 0) return hipSuccess;
    const dim3 grid((unsigned)((max_n + kMaskChunk - 1) / kMaskChunk), (unsigned)nq);
    hipLaunchKernelGGL(mask_pool_kernel, grid, dim3(kMaskThreads), 0, stream, scores, score_stride, n_vis, max_n,
                       pool_blocks, pool_stride, pool_count, group);
    return hipGetLastError();
}

}  // namespace fp4idx
