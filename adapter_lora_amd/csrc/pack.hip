// Load-time packing of one adapter into its slot of the rank-grouped table
// ("vLLM-Ascend dynamic LoRA operator" walkthrough: section 2.1 lays the
// weights out once at load time; section 4.3 pads the rank to a multiple of
// 16 with zero A rows and zero B columns).  Pure copies; element bits are
// moved unchanged, padding is written as zero bits.
#include "common.hpp"
#include "kernels.hpp"

namespace mlora {

template <typename E>
__global__ void k_pack_A(const E* __restrict__ src, E* __restrict__ dst, int K, int n_sl, int r,
                         int rp) {
    const int64_t total = (int64_t)n_sl * rp * K;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t row = i / K;
        const int k = (int)(i - row * K);
        const int s = (int)(row / rp);
        const int j = (int)(row - (int64_t)s * rp);
        dst[i] = (j < r) ? src[((int64_t)s * r + j) * K + k] : E(0);
    }
}

template <typename E>
__global__ void k_pack_B(const E* __restrict__ src, E* __restrict__ dst, int64_t N, int r,
                         int rp) {
    const int64_t total = N * rp;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t n = i / rp;
        const int j = (int)(i - n * rp);
        dst[i] = (j < r) ? src[n * r + j] : E(0);
    }
}

// Embedding adapters (SGLang "LoRA Layers" page: A (rank, vocab) is read by
// an embedding lookup): A is stored transposed, [vocab, rp] row-major, so the
// lookup of a token reads one contiguous row of rp values.
template <typename E>
__global__ void k_pack_A_T(const E* __restrict__ src, E* __restrict__ dst, int vocab, int r,
                           int rp) {
    const int64_t total = (int64_t)vocab * rp;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t t = i / rp;
        const int j = (int)(i - t * rp);
        dst[i] = (j < r) ? src[(int64_t)j * vocab + t] : E(0);
    }
}

static unsigned blocks_for(int64_t n) {
    int64_t b = (n + 255) / 256;
    if (b > 8192) b = 8192;
    if (b < 1) b = 1;
    return (unsigned)b;
}

hipError_t launch_pack_adapter(int dtype, int K, int64_t N, int n_sl, int rank, int rank_pad,
                               const void* A_src, const void* B_src, void* A_dst, void* B_dst,
                               hipStream_t st) {
    const int64_t na = (int64_t)n_sl * rank_pad * K;
    const int64_t nb = N * rank_pad;
    if (dtype == LORA_BF16) {
        hipLaunchKernelGGL(k_pack_A<uint16_t>, dim3(blocks_for(na)), dim3(256), 0, st,
                           (const uint16_t*)A_src, (uint16_t*)A_dst, K, n_sl, rank, rank_pad);
        hipLaunchKernelGGL(k_pack_B<uint16_t>, dim3(blocks_for(nb)), dim3(256), 0, st,
                           (const uint16_t*)B_src, (uint16_t*)B_dst, N, rank, rank_pad);
    } else {
        hipLaunchKernelGGL(k_pack_A<uint32_t>, dim3(blocks_for(na)), dim3(256), 0, st,
                           (const uint32_t*)A_src, (uint32_t*)A_dst, K, n_sl, rank, rank_pad);
        hipLaunchKernelGGL(k_pack_B<uint32_t>, dim3(blocks_for(nb)), dim3(256), 0, st,
                           (const uint32_t*)B_src, (uint32_t*)B_dst, N, rank, rank_pad);
    }
    return hipGetLastError();
}

hipError_t launch_pack_embedding_adapter(int dtype, int vocab, int64_t emb, int rank,
                                         int rank_pad, const void* A_src, const void* B_src,
                                         void* A_dst, void* B_dst, hipStream_t st) {
    const int64_t na = (int64_t)vocab * rank_pad;
    const int64_t nb = emb * rank_pad;
    if (dtype == LORA_BF16) {
        hipLaunchKernelGGL(k_pack_A_T<uint16_t>, dim3(blocks_for(na)), dim3(256), 0, st,
                           (const uint16_t*)A_src, (uint16_t*)A_dst, vocab, rank, rank_pad);
        hipLaunchKernelGGL(k_pack_B<uint16_t>, dim3(blocks_for(nb)), dim3(256), 0, st,
                           (const uint16_t*)B_src, (uint16_t*)B_dst, emb, rank, rank_pad);
    } else {
        hipLaunchKernelGGL(k_pack_A_T<uint32_t>, dim3(blocks_for(na)), dim3(256), 0, st,
                           (const uint32_t*)A_src, (uint32_t*)A_dst, vocab, rank, rank_pad);
        hipLaunchKernelGGL(k_pack_B<uint32_t>, dim3(blocks_for(nb)), dim3(256), 0, st,
                           (const uint32_t*)B_src, (uint32_t*)B_dst, emb, rank, rank_pad);
    }
    return hipGetLastError();
}

}  // namespace mlora
