// Dense multi-LoRA shrink and expand over a segment table
// ("vLLM-Ascend dynamic LoRA operator" walkthrough, section 2.3: per segment
// X_seg A_i^T, then S B_i^T added to the y_base rows of the segment's tokens;
// every segment is served by one launch).
//
// Work units never straddle a segment: a segment of m_s tokens is cut into
// ceil(m_s / 64) row tiles, and each launch's grid enumerates
// (row tile, K chunk) for the shrink or (row tile, 256-column tile) for the
// expand.  Which segment a row tile belongs to is found on the device from
// seg_indptr by a wavefront prefix scan (section 2.4 asks for the "which
// block, which segment, which rank" mapping to be settled outside the inner
// loops; here it is settled once per workgroup, before any data moves).
#include "common.hpp"
#include "kernels.hpp"
#include "tiles.hpp"

namespace mlora {

constexpr int kRowTile = 64;

struct UnitInfo {
    int seg;      // segment index, -1 if the unit does not exist
    int pbeg;     // first sorted position of the tile
    int n;        // rows in the tile
};

// Wave 0 finds row tile u; result broadcast through LDS.
__device__ __forceinline__ UnitInfo find_row_tile(const LinearArgs& a, int u, int* sh) {
    if (threadIdx.x < kWave) {
        const int lane = lane_id();
        const int nseg = a.num_segments[0];
        int run = 0, found = -1, pbeg = 0, nr = 0;
        for (int s0 = 0; s0 < nseg && found < 0; s0 += kWave) {
            const int s = s0 + lane;
            int b = 0, e = 0, t = 0;
            if (s < nseg) {
                b = a.seg_indptr[s];
                e = a.seg_indptr[s + 1];
                t = (e - b + kRowTile - 1) / kRowTile;
            }
            int inc = t;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const int v = __shfl_up(inc, o, kWave);
                if (lane >= o) inc += v;
            }
            const int excl = run + inc - t;
            const bool mine = (s < nseg) && u >= excl && u < excl + t;
            const unsigned long long bal = __ballot(mine);
            if (bal) {
                const int src = __ffsll((unsigned long long)bal) - 1;
                found = __shfl(s, src, kWave);
                const int mt = u - __shfl(excl, src, kWave);
                pbeg = __shfl(b, src, kWave) + mt * kRowTile;
                nr = min(kRowTile, __shfl(e, src, kWave) - pbeg);
            }
            run += __shfl(inc, kWave - 1, kWave);
        }
        if (lane == 0) {
            sh[0] = found;
            sh[1] = pbeg;
            sh[2] = nr;
        }
    }
    __syncthreads();
    return UnitInfo{sh[0], sh[1], sh[2]};
}

// ---------------------------------------------------------------------------
// shrink: P[c][p][col] partial sums (p = sorted position, col = sl*r_max + j)
// ---------------------------------------------------------------------------
template <typename T, int NCB>
__global__ __launch_bounds__(kTileThreads) void k_shrink_dense(LinearArgs a, const T* __restrict__ x,
                                                                int64_t ldx, float* __restrict__ P,
                                                                int C) {
    __shared__ int sh[4];
    __shared__ int s_in[kRowTile], s_out[kRowTile];
    const int u = blockIdx.x / C;
    const int c = blockIdx.x % C;
    const UnitInfo ui = find_row_tile(a, u, sh);
    if (ui.seg < 0) return;
    const int id = a.req_to_lora[ui.seg];
    const int rp = a.rank[id];
    for (int i = threadIdx.x; i < ui.n; i += kTileThreads) {
        s_in[i] = a.sorted_idx[ui.pbeg + i];
        s_out[i] = ui.pbeg + i;
    }
    __syncthreads();
    const RowSet rs{ui.n, kRowTile, s_in, s_out};
    const int k0 = c * kKChunk;
    const int k1 = min(a.K, k0 + kKChunk);
    float* Pc = P + (int64_t)c * a.M * a.cols;
    const T* A = reinterpret_cast<const T*>(a.A) + a.a_off[id];
    if constexpr (sizeof(T) == 2) {
        shrink_tile_bf16<NCB>(rs, reinterpret_cast<const uint16_t*>(x), ldx,
                              reinterpret_cast<const uint16_t*>(A), a.K, rp, a.r_max, k0, k1,
                              Pc, a.cols);
    } else {
        shrink_tile_simple<T>(rs, x, ldx, A, a.K, a.n_sl, rp, a.r_max, k0, k1, Pc, a.cols);
    }
}

// S[p][:] = sum_c P[c][p][:] for every sorted position with an adapter
__global__ void k_reduce_partials(const float* __restrict__ P, int C, int64_t cstride,
                                  float* __restrict__ S, int cols,
                                  const int32_t* __restrict__ seg_indptr,
                                  const int32_t* __restrict__ num_segments) {
    const int m_valid = seg_indptr[num_segments[0]];
    const int64_t total4 = (int64_t)m_valid * cols / 4;   // cols is a multiple of 16
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total4; i += stride) {
        float4 acc = reinterpret_cast<const float4*>(P)[i];
        for (int c = 1; c < C; ++c) {
            const float4 v = reinterpret_cast<const float4*>(P + c * cstride)[i];
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        reinterpret_cast<float4*>(S)[i] = acc;
    }
}

// ---------------------------------------------------------------------------
// expand: y[sorted_idx[p], n] += S[p, sl, :rp] . B_i[n, :rp]
// ---------------------------------------------------------------------------
struct TileMap {
    int n_tiles;
    int tile_start[LORA_MAX_SLICES + 1];
};

__device__ __forceinline__ void tile_cols(const LinearArgs& a, const TileMap& tm, int t, int* sl,
                                          int* n0, int* n1) {
    int s = 0;
    while (s + 1 < a.n_sl && t >= tm.tile_start[s + 1]) ++s;
    *sl = s;
    *n0 = (int)(a.slice_off[s] + (int64_t)(t - tm.tile_start[s]) * kNTile);
    *n1 = (int)min((int64_t)*n0 + kNTile, a.slice_off[s + 1]);
}

template <typename T>
__global__ __launch_bounds__(kTileThreads) void k_expand_dense(LinearArgs a, TileMap tm,
                                                                const float* __restrict__ S,
                                                                T* __restrict__ y, int64_t ldy) {
    __shared__ int sh[4];
    __shared__ int s_in[kRowTile], s_out[kRowTile];
    const int u = blockIdx.x / tm.n_tiles;
    const int t = blockIdx.x % tm.n_tiles;
    const UnitInfo ui = find_row_tile(a, u, sh);
    if (ui.seg < 0) return;
    const int id = a.req_to_lora[ui.seg];
    const int rp = a.rank[id];
    if (rp == 0) return;
    for (int i = threadIdx.x; i < ui.n; i += kTileThreads) {
        s_in[i] = ui.pbeg + i;
        s_out[i] = a.sorted_idx[ui.pbeg + i];
    }
    __syncthreads();
    int sl, n0, n1;
    tile_cols(a, tm, t, &sl, &n0, &n1);
    const RowSet rs{ui.n, kRowTile, s_in, s_out};
    const T* B = reinterpret_cast<const T*>(a.B) + a.b_off[id];
    if constexpr (sizeof(T) == 2) {
        expand_tile_bf16(rs, S, a.cols, sl * a.r_max, reinterpret_cast<const uint16_t*>(B), rp, n0,
                         n1, reinterpret_cast<uint16_t*>(y), ldy);
    } else {
        expand_tile_simple<T>(rs, S, a.cols, sl * a.r_max, B, rp, n0, n1, y, ldy);
    }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
static int row_tiles_max(const LinearArgs& a) { return a.M / kRowTile + a.s_max; }

TileMap make_tile_map(const LinearArgs& a) {
    TileMap tm{};
    int t = 0;
    for (int s = 0; s < a.n_sl; ++s) {
        tm.tile_start[s] = t;
        const int64_t n = a.slice_off[s + 1] - a.slice_off[s];
        t += (int)((n + kNTile - 1) / kNTile);
    }
    tm.tile_start[a.n_sl] = t;
    tm.n_tiles = t;
    return tm;
}

template <typename T, int NCB>
static void launch_shrink_ncb(const LinearArgs& a, const void* x, int64_t ldx, float* P, int C,
                              hipStream_t st) {
    const unsigned grid = (unsigned)(row_tiles_max(a) * C);
    hipLaunchKernelGGL((k_shrink_dense<T, NCB>), dim3(grid), dim3(kTileThreads), 0, st, a,
                       reinterpret_cast<const T*>(x), ldx, P, C);
}

template <typename T>
static hipError_t launch_shrink_t(const LinearArgs& a, const void* x, int64_t ldx, float* P,
                                  int C, hipStream_t st) {
    const int ncb = a.cols / 16;
    switch (ncb) {
#define MLORA_NCB(n) case n: launch_shrink_ncb<T, n>(a, x, ldx, P, C, st); break;
        MLORA_NCB(1) MLORA_NCB(2) MLORA_NCB(3) MLORA_NCB(4) MLORA_NCB(5) MLORA_NCB(6)
        MLORA_NCB(7) MLORA_NCB(8) MLORA_NCB(9) MLORA_NCB(10) MLORA_NCB(11) MLORA_NCB(12)
        MLORA_NCB(13) MLORA_NCB(14) MLORA_NCB(15) MLORA_NCB(16)
#undef MLORA_NCB
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_shrink(const LinearArgs& a, const void* x, int64_t ldx, float* S, void* ws,
                         hipStream_t st) {
    const int C = kchunks(a.K);
    const LinearWs L = linear_ws_layout(a.M, a.K, a.cols, a.L, a.n_sl);
    float* P = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + L.partial);
    hipError_t e = (a.dtype == LORA_BF16) ? launch_shrink_t<uint16_t>(a, x, ldx, P, C, st)
                                          : launch_shrink_t<float>(a, x, ldx, P, C, st);
    if (e != hipSuccess) return e;
    int64_t total4 = (int64_t)a.M * a.cols / 4;
    int64_t blocks = (total4 + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(k_reduce_partials, dim3((unsigned)blocks), dim3(256), 0, st, P, C,
                       (int64_t)a.M * a.cols, S, a.cols, a.seg_indptr, a.num_segments);
    return hipGetLastError();
}

hipError_t launch_expand(const LinearArgs& a, const float* S, void* y, int64_t ldy,
                         hipStream_t st) {
    const TileMap tm = make_tile_map(a);
    const unsigned grid = (unsigned)(row_tiles_max(a) * tm.n_tiles);
    if (a.dtype == LORA_BF16) {
        hipLaunchKernelGGL(k_expand_dense<uint16_t>, dim3(grid), dim3(kTileThreads), 0, st, a, tm,
                           S, reinterpret_cast<uint16_t*>(y), ldy);
    } else {
        hipLaunchKernelGGL(k_expand_dense<float>, dim3(grid), dim3(kTileThreads), 0, st, a, tm, S,
                           reinterpret_cast<float*>(y), ldy);
    }
    return hipGetLastError();
}

}  // namespace mlora
