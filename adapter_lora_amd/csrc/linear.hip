// Dense multi-LoRA shrink and expand over the tile schedule
// ("vLLM-Ascend dynamic LoRA operator" walkthrough, section 2.3: per segment
// X_seg A_i^T, then S B_i^T added to the y_base rows of the segment's tokens;
// every segment is served by one launch; section 2.4: the block -> segment ->
// rank mapping is settled before the product kernels run).
//
// A work unit is one 64-row tile of the schedule (tiles never straddle a
// segment) and either a (K chunk, S column group) for the shrink or a run of
// 256-column output tiles inside one slice for the expand.  A workgroup
// learns everything about its tile with independent loads issued together
// (tile descriptor, the tile's 64 token indices, and for tables of up to 256
// slots every slot's rank and weight offset), so its data loads start after
// one memory round trip.
#include "common.hpp"
#include "kernels.hpp"
#include "tiles.hpp"
#include "tile_view.hpp"

namespace mlora {

// ---------------------------------------------------------------------------
// shrink: P[c][p][col] partial sums (p = sorted position, col = sl*r_max + j)
// unit = (tile, K chunk c, column group cg of 64 S columns)
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kTileThreads) void k_shrink_dense(LinearArgs a, const T* __restrict__ x,
                                                                int64_t ldx, float* __restrict__ P,
                                                                int C, int G, int units) {
    __shared__ int s_in[kRowTile], s_out[kRowTile];
    const int u = (int)blockIdx.x;
    if (u >= units) return;
    const int tile = u / (C * G);
    const int c = (u / G) % C;
    const int cg = u % G;
    const TileView v = tile_view(a, tile, true);
    if (v.seg < 0) return;
    if (threadIdx.x < kRowTile) {
        s_in[threadIdx.x] = v.row;
        s_out[threadIdx.x] = (int)threadIdx.x < v.n ? v.pbeg + (int)threadIdx.x : -1;
    }
    __syncthreads();
    const RowSet rs{v.n, kRowTile, s_in, s_out};
    float* Pc = P + (int64_t)c * a.M * a.cols;
    const T* A = reinterpret_cast<const T*>(a.A) + v.off;
    if constexpr (sizeof(T) == 2) {
        __shared__ uint4 sXA[kShrinkLds / 16];
        const int k0 = c * kShrinkK;
        const int k1 = min(a.K, k0 + kShrinkK);
        shrink_group_bf16(rs, 0, reinterpret_cast<const uint16_t*>(x), ldx,
                          reinterpret_cast<const uint16_t*>(A), a.K, a.n_sl, v.rp, a.r_max, cg,
                          k0, k1, Pc, a.cols, sXA);
    } else {
        const int k0 = c * kKChunk;
        const int k1 = min(a.K, k0 + kKChunk);
        shrink_tile_simple<T>(rs, x, ldx, A, a.K, a.n_sl, v.rp, a.r_max, k0, k1, Pc, a.cols);
    }
}

// S[p][:] = sum_c P[c][p][:] for every sorted position with an adapter, the
// chunks added in order c = 0, 1, ...  A thread issues the loads of up to
// kReduceBatch chunks before it adds any of them (a loop that adds as it
// loads waits out one memory round trip per chunk).  The rows are bounded by
// M, so no load waits for the number of rows with an adapter; that count
// only gates the stores.
constexpr int kReduceBatch = 8;

__global__ void k_reduce_partials(const float* __restrict__ P, int C, int64_t cstride,
                                  float* __restrict__ S, int cols, int M,
                                  const int32_t* __restrict__ seg_indptr,
                                  const int32_t* __restrict__ num_segments) {
    const int64_t total4 = (int64_t)M * cols / 4;          // cols is a multiple of 16
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const float4* P4 = reinterpret_cast<const float4*>(P);
    const int64_t c4 = cstride / 4;
    const int m_valid = seg_indptr[num_segments[0]];
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total4; i += stride) {
        float4 acc = P4[i];
        for (int c0 = 1; c0 < C; c0 += kReduceBatch) {
            float4 v[kReduceBatch];
#pragma unroll
            for (int q = 0; q < kReduceBatch; ++q) v[q] = P4[min(c0 + q, C - 1) * c4 + i];
#pragma unroll
            for (int q = 0; q < kReduceBatch; ++q) {
                if (c0 + q < C) {
                    acc.x += v[q].x; acc.y += v[q].y; acc.z += v[q].z; acc.w += v[q].w;
                }
            }
        }
        if (i * 4 / cols < m_valid) reinterpret_cast<float4*>(S)[i] = acc;
    }
}

// ---------------------------------------------------------------------------
// expand: y[sorted_idx[p], n] += S[p, sl, :rp] . B_i[n, :rp]
// unit = (tile, group g of up to `tpw` consecutive 256-column tiles of one slice)
// ---------------------------------------------------------------------------
struct GroupMap {
    int n_groups;                              // groups per row tile, all slices
    int tpw;                                   // 256-column tiles per group
    int group_start[LORA_MAX_SLICES + 1];      // first group of each slice
};

template <typename T>
__global__ __launch_bounds__(kTileThreads) __attribute__((amdgpu_waves_per_eu(3))) void k_expand_dense(LinearArgs a, GroupMap gm,
                                                                const float* __restrict__ S,
                                                                T* __restrict__ y, int64_t ldy,
                                                                int units) {
    __shared__ int s_in[kRowTile], s_out[kRowTile];
    const int u = (int)blockIdx.x;
    if (u >= units) return;
    const int tile = u / gm.n_groups;
    const int g = u % gm.n_groups;
    const TileView v = tile_view(a, tile, false);
    if (v.seg < 0 || v.rp == 0) return;
    if (threadIdx.x < kRowTile) {
        s_in[threadIdx.x] = (int)threadIdx.x < v.n ? v.pbeg + (int)threadIdx.x : -1;
        s_out[threadIdx.x] = v.row;
    }
    __syncthreads();
    int sl = 0;
    while (sl + 1 < a.n_sl && g >= gm.group_start[sl + 1]) ++sl;
    const int64_t nb = a.slice_off[sl] + (int64_t)(g - gm.group_start[sl]) * gm.tpw * kNTile;
    const int n_begin = (int)nb;
    const int n_end = (int)min(nb + (int64_t)gm.tpw * kNTile, a.slice_off[sl + 1]);
    const RowSet rs{v.n, kRowTile, s_in, s_out};
    const T* B = reinterpret_cast<const T*>(a.B) + v.off;
    if constexpr (sizeof(T) == 2) {
        __shared__ uint4 lds[kExpandLds / 16];
        expand_rows_bf16(rs, S, a.cols, sl * a.r_max, reinterpret_cast<const uint16_t*>(B), v.rp,
                         n_begin, n_end, reinterpret_cast<uint16_t*>(y), ldy, lds);
    } else {
        for (int n0 = n_begin; n0 < n_end; n0 += kNTile)
            expand_tile_simple<T>(rs, S, a.cols, sl * a.r_max, B, v.rp, n0, min(n0 + kNTile, n_end),
                                  y, ldy);
    }
}

// Pipelined bf16 expand: unit = (tile, run of gm.tpw 128-column tiles of one
// slice); see expand_pipe_bf16.
__global__ __launch_bounds__(kTileThreads) __attribute__((amdgpu_waves_per_eu(3))) void k_expand_pipe(
    LinearArgs a, GroupMap gm, const float* __restrict__ S, uint16_t* __restrict__ y, int64_t ldy,
    int units) {
    __shared__ int s_in[kRowTile], s_out[kRowTile];
    const int u = (int)blockIdx.x;
    if (u >= units) return;
    const int tile = u / gm.n_groups;
    const int g = u % gm.n_groups;
    const TileView v = tile_view(a, tile, false);
    if (v.seg < 0 || v.rp == 0) return;
    if (threadIdx.x < kRowTile) {
        s_in[threadIdx.x] = (int)threadIdx.x < v.n ? v.pbeg + (int)threadIdx.x : -1;
        s_out[threadIdx.x] = v.row;
    }
    __syncthreads();
    int sl = 0;
    while (sl + 1 < a.n_sl && g >= gm.group_start[sl + 1]) ++sl;
    const int64_t nb = a.slice_off[sl] + (int64_t)(g - gm.group_start[sl]) * gm.tpw * kPCols;
    const int n_begin = (int)nb;
    const int n_end = (int)min(nb + (int64_t)gm.tpw * kPCols, a.slice_off[sl + 1]);
    const RowSet rs{v.n, kRowTile, s_in, s_out};
    // the rank and the B block are the same for every lane (buffer resources
    // are built from scalar registers)
    const int rp = __builtin_amdgcn_readfirstlane(v.rp);
    const int64_t off = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(v.off >> 32)) << 32) |
                                  (uint32_t)__builtin_amdgcn_readfirstlane((int)v.off));
    const uint16_t* B = reinterpret_cast<const uint16_t*>(a.B) + off;
    __shared__ uint4 lds[kPipeLds / 16];
    expand_pipe_bf16(rs, v.n, S, a.cols, sl * a.r_max, B, (int)a.slice_off[a.n_sl], rp, n_begin,
                     n_end, y, ldy, lds);
}

// ---------------------------------------------------------------------------
// embedding lookup (SGLang "LoRA Layers" page, the embedding's A side):
// S[p][j] = A_i[j, t] for the token t at sorted position p, read from the
// transposed table row A_i^T[t] (rp contiguous values); zero past rp and for
// token ids outside [0, vocab).  unit = one tile of the schedule; thread
// (row, q) covers rank positions 16q .. 16q+15 of one row.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kTileThreads) void k_embed_shrink(LinearArgs a,
                                                                const int32_t* __restrict__ tokens,
                                                                float* __restrict__ S, int units) {
    const int tile = (int)blockIdx.x;
    if (tile >= units) return;
    const TileView v = tile_view(a, tile, true);
    if (v.seg < 0) return;
    const int row = threadIdx.x / 4, q = threadIdx.x % 4;
    const int m = __shfl(v.row, row, kWave);          // every wave holds the tile's 64 rows
    if (row >= v.n || q * 16 >= a.r_max) return;
    const int vocab = a.K;
    const int tok = tokens[m];
    const bool on = q * 16 < v.rp && tok >= 0 && tok < vocab;
    const T* src = reinterpret_cast<const T*>(a.A) + v.off + (int64_t)(on ? tok : 0) * v.rp + q * 16;
    float vals[16];
    if constexpr (sizeof(T) == 2) {
        const uint4 lo = ld16_if(src, on, src), hi = ld16_if(src + 8, on, src);
        const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            vals[2 * i] = __uint_as_float(w[i] << 16);
            vals[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 f = ldf4_if(src + 4 * i, on, src);
            vals[4 * i] = f.x; vals[4 * i + 1] = f.y; vals[4 * i + 2] = f.z; vals[4 * i + 3] = f.w;
        }
    }
    float4* dst = reinterpret_cast<float4*>(S + (int64_t)(v.pbeg + row) * a.cols + q * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        dst[i] = make_float4(vals[4 * i], vals[4 * i + 1], vals[4 * i + 2], vals[4 * i + 3]);
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
static unsigned grid_of(int units) { return (unsigned)(units > 0 ? units : 1); }

hipError_t launch_shrink(const LinearArgs& a, const void* x, int64_t ldx, float* S, void* ws,
                         hipStream_t st) {
    const bool bf16 = a.dtype == LORA_BF16;
    const int C = bf16 ? (a.K + kShrinkK - 1) / kShrinkK : kchunks(a.K);
    const int G = bf16 ? (a.cols + kGroupCols - 1) / kGroupCols : 1;
    const int units = a.max_tiles * C * G;
    const LinearWs L = linear_ws_layout(a.M, a.K, a.cols);
    float* P = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + L.partial);
    if (bf16)
        hipLaunchKernelGGL(k_shrink_dense<uint16_t>, dim3(grid_of(units)), dim3(kTileThreads), 0, st,
                           a, reinterpret_cast<const uint16_t*>(x), ldx, P, C, G, units);
    else
        hipLaunchKernelGGL(k_shrink_dense<float>, dim3(grid_of(units)), dim3(kTileThreads), 0, st,
                           a, reinterpret_cast<const float*>(x), ldx, P, C, G, units);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int64_t total4 = (int64_t)a.M * a.cols / 4;
    int64_t blocks = (total4 + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(k_reduce_partials, dim3((unsigned)blocks), dim3(256), 0, st, P, C,
                       (int64_t)a.M * a.cols, S, a.cols, a.M, a.seg_indptr, a.num_segments);
    return hipGetLastError();
}

// One 256-column tile per workgroup: a workgroup walks its tiles one after
// another without overlapping them, so spreading tiles over more workgroups
// (three resident per CU) hides more latency.  The pipelined expand takes
// runs of `tpw` 128-column tiles.
static GroupMap make_group_map(const LinearArgs& a, int tpw = 1, int tile_cols = kNTile) {
    GroupMap gm{};
    gm.tpw = tpw;
    int g = 0;
    for (int s = 0; s < a.n_sl; ++s) {
        gm.group_start[s] = g;
        const int t = (int)((a.slice_off[s + 1] - a.slice_off[s] + tile_cols - 1) / tile_cols);
        g += (t + tpw - 1) / tpw;
    }
    gm.group_start[a.n_sl] = g;
    gm.n_groups = g;
    return gm;
}

hipError_t launch_embedding_shrink(const LinearArgs& a, const int32_t* tokens, float* S,
                                   hipStream_t st) {
    const int units = a.max_tiles;
    if (a.dtype == LORA_BF16)
        hipLaunchKernelGGL(k_embed_shrink<uint16_t>, dim3(grid_of(units)), dim3(kTileThreads), 0,
                           st, a, tokens, S, units);
    else
        hipLaunchKernelGGL(k_embed_shrink<float>, dim3(grid_of(units)), dim3(kTileThreads), 0, st,
                           a, tokens, S, units);
    return hipGetLastError();
}

// The pipelined bf16 expand addresses y and B through buffer resources with
// 32-bit byte offsets, so it serves outputs whose rows span less than 2 GiB
// (M * ldy * 2 bytes) and B blocks under 2 GiB; larger ones take the
// one-tile-per-workgroup kernel.  Its runs are as short as keeps every unit
// resident at once (three workgroups per CU on 256 CUs): a second, partial
// round of workgroups costs more than shorter pipelines save (stacked QKV:
// 24.3 us for the delta kernels with runs of 2 tiles against 26.1 us
// unpipelined; stacked gate/up, runs of 6, 39.4 against 44.2, where runs of
// 5, 920 units, took 43.6).  When the schedule's tiles are nearly full (at
// least 48 rows on average) a unit carries enough traffic that two per CU
// keep the memory system as busy, and longer runs win (2048-token prefill:
// runs of 3, 440 units, 28.6 us against 29.4 with runs of 2 and 30.9
// unpipelined).
constexpr int kResidentExpandUnits = 3 * 256;
constexpr int kFullTileExpandUnits = 2 * 256;

hipError_t launch_expand(const LinearArgs& a, const float* S, void* y, int64_t ldy,
                         hipStream_t st) {
    if (a.dtype == LORA_BF16 && (int64_t)a.M * ldy * 2 <= 0x7fffffff &&
        a.slice_off[a.n_sl] * a.r_max * 2 <= 0x7fffffff) {
        const bool full = (int64_t)a.M >= (int64_t)48 * a.max_tiles;
        const int budget = max(1, (full ? kFullTileExpandUnits : kResidentExpandUnits) /
                                      max(1, a.max_tiles));                      // runs per tile
        const int tiles = make_group_map(a, 1, kPCols).n_groups;                  // 128-column tiles
        int t = (tiles + budget - 1) / budget;
        GroupMap gp = make_group_map(a, t, kPCols);
        while (gp.n_groups > budget && gp.n_groups > a.n_sl) gp = make_group_map(a, ++t, kPCols);
        const int units = a.max_tiles * gp.n_groups;
        hipLaunchKernelGGL(k_expand_pipe, dim3(grid_of(units)), dim3(kTileThreads), 0, st, a, gp, S,
                           reinterpret_cast<uint16_t*>(y), ldy, units);
        return hipGetLastError();
    }
    const GroupMap gm = make_group_map(a);
    const int units = a.max_tiles * gm.n_groups;
    if (a.dtype == LORA_BF16) {
        hipLaunchKernelGGL(k_expand_dense<uint16_t>, dim3(grid_of(units)), dim3(kTileThreads), 0, st,
                           a, gm, S, reinterpret_cast<uint16_t*>(y), ldy, units);
    } else {
        hipLaunchKernelGGL(k_expand_dense<float>, dim3(grid_of(units)), dim3(kTileThreads), 0, st, a,
                           gm, S, reinterpret_cast<float*>(y), ldy, units);
    }
    return hipGetLastError();
}

}  // namespace mlora
