// Streaming reference kernel for the benchmark's practical ceiling: reads
// `rd_bytes` and writes `wr_bytes` (a prefix of what it read) with nothing
// else in the way, so that a kernel of the path can be compared with the
// fastest plain transfer of the same byte mix and launch shape on the same
// GPU.  Not part of the library's C ABI (include/mlora.h); built into its own
// shared object for bench.py.
//
// Thread t of a grid of T threads reads the 16-byte words t, t + T, ...,
// t + (U-1) T of each pass (coalesced: consecutive threads read consecutive
// words), all U loads issued before the first is used, and writes back the
// words of the pass that fall below `wr_words`.  Past the end the index is
// clamped, so every load is unconditional.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;

template <int U>
__global__ __launch_bounds__(kThreads) void k_stream(const uint4* __restrict__ src, int64_t rd_words,
                                                     uint4* __restrict__ dst, int64_t wr_words) {
    const int64_t T = (int64_t)gridDim.x * kThreads;
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    for (int64_t base = t; base < rd_words; base += T * U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + u * T;
            v[u] = src[i < rd_words ? i : rd_words - 1];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + u * T;
            if (i < wr_words) dst[i] = v[u];
        }
    }
}

template <int U>
hipError_t launch(const void* src, int64_t rd_words, void* dst, int64_t wr_words, int grid,
                  hipStream_t st) {
    if (grid <= 0) {
        const int64_t per = (int64_t)kThreads * U;
        grid = (int)((rd_words + per - 1) / per);
    }
    hipLaunchKernelGGL(k_stream<U>, dim3(grid), dim3(kThreads), 0, st,
                       reinterpret_cast<const uint4*>(src), rd_words, reinterpret_cast<uint4*>(dst),
                       wr_words);
    return hipGetLastError();
}

}  // namespace

extern "C" {

// Returns 0 on success, 1 for a bad argument, 2 for a launch error.
//   src  device, rd_bytes readable (16-byte aligned, rd_bytes % 16 == 0, > 0);
//   dst  device, wr_bytes writable (wr_bytes <= rd_bytes, % 16 == 0);
//   grid workgroups of 256 threads (0: one pass, grid = rd_words / (256 U));
//   unroll U in {1, 2, 4, 8, 16}: loads in flight per thread.
int mlora_stream(const void* src, int64_t rd_bytes, void* dst, int64_t wr_bytes, int grid,
                 int unroll, hipStream_t stream) {
    if (!src || rd_bytes <= 0 || rd_bytes % 16 || wr_bytes < 0 || wr_bytes % 16 ||
        wr_bytes > rd_bytes || (wr_bytes > 0 && !dst) || grid < 0)
        return 1;
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u) return 1;
    const int64_t rw = rd_bytes / 16, ww = wr_bytes / 16;
    hipError_t e;
    switch (unroll) {
        case 1: e = launch<1>(src, rw, dst, ww, grid, stream); break;
        case 2: e = launch<2>(src, rw, dst, ww, grid, stream); break;
        case 4: e = launch<4>(src, rw, dst, ww, grid, stream); break;
        case 8: e = launch<8>(src, rw, dst, ww, grid, stream); break;
        case 16: e = launch<16>(src, rw, dst, ww, grid, stream); break;
        default: return 1;
    }
    return e == hipSuccess ? 0 : 2;
}

}  // extern "C"
