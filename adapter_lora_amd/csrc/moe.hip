// LoRA on a Mixture-of-Experts MLP (SGLang "LoRA + MoE" page):
//   * alignment: one padded list of (token, expert) pairs per adapter, sorted
//     by expert ("MoE LoRA Alignment");
//   * stage 1.5: cache1 += gate/up delta, before the activation;
//   * stage 2: silu_and_mul;
//   * stage 3.5: cache3 += down delta, before the reduce;
//   * the final top-k weighted reduce.
// The deltas run the same MFMA shrink / expand tiles as the dense path, with
// a unit = (adapter, block of block_size_m aligned pairs) that reads the
// weights of the block's expert.
#include "common.hpp"
#include "kernels.hpp"
#include "tiles.hpp"

namespace mlora {

// ---------------------------------------------------------------- alignment
constexpr int kAlignThreads = 256;
constexpr int kAlignWaves = kAlignThreads / kWave;
constexpr int kMaxExperts = 256;

__global__ __launch_bounds__(kAlignThreads) void k_moe_align(
    const int32_t* __restrict__ topk_ids, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ adapter_enabled, int M, int topk, int E,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ expert_ids,
    int32_t* __restrict__ ntpp, int mtp, int bs) {
    __shared__ int cnt[kMaxExperts];
    __shared__ int base[kMaxExperts];
    __shared__ int wcnt[kAlignWaves][kMaxExperts];
    __shared__ int total_sh;
    const int l = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int P = M * topk;
    const int nblk = mtp / bs;
    int32_t* row = sorted_ids + (int64_t)l * mtp;
    int32_t* erow = expert_ids + (int64_t)l * nblk;
    const bool on = adapter_enabled[l] != 0;

    for (int e = tid; e < kMaxExperts; e += kAlignThreads) {
        cnt[e] = 0;
        for (int w = 0; w < kAlignWaves; ++w) wcnt[w][e] = 0;
    }
    __syncthreads();
    if (on) {
        for (int f = tid; f < P; f += kAlignThreads) {
            const int e = topk_ids[f];
            if (ids[f / topk] == l && e >= 0 && e < E) atomicAdd(&cnt[e], 1);
        }
    }
    __syncthreads();
    if (wave == 0) {
        int run = 0;
        for (int e0 = 0; e0 < E; e0 += kWave) {
            const int e = e0 + lane;
            const int c = (e < E) ? cnt[e] : 0;
            const int pad = (c + bs - 1) / bs * bs;
            int inc = pad;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const int v = __shfl_up(inc, o, kWave);
                if (lane >= o) inc += v;
            }
            if (e < E) base[e] = run + inc - pad;
            run += __shfl(inc, kWave - 1, kWave);
        }
        if (lane == 0) {
            total_sh = run;
            ntpp[l] = run;
        }
    }
    __syncthreads();
    const int total = total_sh;
    // expert id per block; sentinels in padding slots and the tail
    for (int b = tid; b < nblk; b += kAlignThreads) erow[b] = -1;
    __syncthreads();
    for (int e = 0; e < E; ++e) {
        const int c = cnt[e];
        if (c == 0) continue;
        const int pad = (c + bs - 1) / bs * bs;
        for (int b = base[e] / bs + tid; b < (base[e] + pad) / bs; b += kAlignThreads) erow[b] = e;
        for (int i = base[e] + c + tid; i < base[e] + pad; i += kAlignThreads) row[i] = P;
    }
    for (int i = total + tid; i < mtp; i += kAlignThreads) row[i] = P;
    if (!on) return;
    // stable scatter of the adapter's pairs, in increasing f, into their bucket
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 1;
    const unsigned long long lt = (1ull << lane) - 1ull;
    for (int f0 = 0; f0 < P; f0 += kAlignThreads) {
        const int f = f0 + tid;
        int e = 0;
        bool act = false;
        if (f < P) {
            e = topk_ids[f];
            act = ids[f / topk] == l && e >= 0 && e < E;
        }
        unsigned long long peers = __ballot(act);
        for (int i = 0; i < nbits; ++i) {
            const bool bit = (e >> i) & 1;
            const unsigned long long bb = __ballot(bit);
            peers &= bit ? bb : ~bb;
        }
        const int rank_w = __popcll(peers & lt);
        const bool leader = act && rank_w == 0;
        if (leader) wcnt[wave][e] = __popcll(peers);
        __syncthreads();
        if (act) {
            int pos = base[e] + rank_w;
            for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
            row[pos] = f;
        }
        __syncthreads();
        if (leader) {
            atomicAdd(&base[e], __popcll(peers));   // one leader per wave and expert
            wcnt[wave][e] = 0;
        }
        __syncthreads();
    }
}

hipError_t launch_moe_align(const int32_t* topk_ids, const int32_t* ids,
                            const int32_t* adapter_enabled, int M, int topk, int E, int L,
                            int32_t* sorted_token_ids, int32_t* expert_ids, int32_t* ntpp,
                            int max_tokens_padded, int block_size_m, hipStream_t st) {
    hipLaunchKernelGGL(k_moe_align, dim3(L), dim3(kAlignThreads), 0, st, topk_ids, ids,
                       adapter_enabled, M, topk, E, sorted_token_ids, expert_ids, ntpp,
                       max_tokens_padded, block_size_m);
    return hipGetLastError();
}

// ---------------------------------------------------------------- deltas
// Weight slot of adapter l and expert e in a [L, E, ...] stack; an outer
// (hidden-side) stack shared by the experts has one slot per adapter.
__device__ __forceinline__ int64_t moe_slot(const MoeArgs& a, bool outer, int l, int e) {
    return (outer && a.shared_outer) ? (int64_t)l : (int64_t)l * a.E + e;
}

// Units are numbered block-major (block b of every adapter, then block b + 1):
// an adapter's used blocks are a prefix of its list, so the units with work
// take the lowest workgroup ids and the idle ones (blocks past an adapter's
// padded length) come last instead of holding dispatch slots among them.
struct MoeUnit {
    bool ok;
    int e;
    int n;     // rows to process: 1 + the last real row of the block
};

// Stage the rows of block b of adapter l.  `shrink` selects the row roles:
// shrink: in = source row of the activation, out = P/S row (l*mtp + pos);
// expand: in = S row, out = cache row f.
// Every index load is issued at once (indices clamped, not tested), so the
// unit is known after one memory round trip.  Padding rows (sentinels) read
// and write nothing; rows past the block's last real row are not visited.
__device__ __forceinline__ MoeUnit moe_unit(const MoeArgs& a, int which, bool shrink, int l, int b,
                                            int* s_in, int* s_out, int* s_wlast) {
    const int bs = a.block_size_m;                // <= blockDim.x; s_wlast: one int per wave
    const int P = a.M * a.topk;
    const int i = threadIdx.x;
    const int pos = b * bs + min(i, bs - 1);
    const int en = a.adapter_enabled[l];
    const int np = a.ntpp[l];
    const int e = a.expert_ids[(int64_t)l * (a.max_tokens_padded / bs) + b];
    const int f = a.sorted_token_ids[(int64_t)l * a.max_tokens_padded + pos];
    if (!en || b * bs >= np || e < 0 || e >= a.E) return MoeUnit{false, -1, 0};
    const bool real = i < bs && f >= 0 && f < P;
    if (i < bs) {
        const int srow = l * a.max_tokens_padded + pos;
        const int src = which == 0 ? f / a.topk : f;
        if (shrink) {
            s_in[i] = real ? src : -1;
            s_out[i] = real ? srow : -1;
        } else {
            s_in[i] = real ? srow : -1;
            s_out[i] = real ? f : -1;
        }
    }
    const unsigned long long bal = __ballot(real);
    if (lane_id() == 0) s_wlast[i / kWave] = bal ? (i / kWave) * kWave + 63 - __clzll(bal) : -1;
    __syncthreads();
    int last = -1;
#pragma unroll
    for (int w = 0; w < (int)(blockDim.x / kWave); ++w) last = max(last, s_wlast[w]);
    return MoeUnit{true, e, last + 1};
}

template <typename T>
__global__ __launch_bounds__(kTileThreads) void k_moe_shrink(MoeArgs a, int which,
                                                              const T* __restrict__ in,
                                                              int64_t ld_in, float* __restrict__ P,
                                                              int C, int K, int units) {
    __shared__ int s_in[kMaxRowTile], s_out[kMaxRowTile];
    const int unit = (int)blockIdx.x;
    if (unit >= units) return;
    const int blk = unit / C;
    const int c = unit % C;
    const int l = blk % a.L, b = blk / a.L;
    __shared__ int s_wlast[kTileWaves];
    const MoeUnit mu = moe_unit(a, which, true, l, b, s_in, s_out, s_wlast);
    if (!mu.ok) return;
    const int64_t ew = moe_slot(a, which == 0, l, mu.e);
    const T* A = reinterpret_cast<const T*>(which == 0 ? a.A_gu : a.A_d) + ew * a.r * K;
    const RowSet rs{mu.n, a.block_size_m, s_in, s_out};
    const int rows = a.L * a.max_tokens_padded;
    float* Pc = P + (int64_t)c * rows * a.r;
    if constexpr (sizeof(T) == 2) {
        __shared__ uint4 sXA[kShrinkLds / 16];
        const int k0 = c * kShrinkK;
        const int k1 = min(K, k0 + kShrinkK);
        for (int r0 = 0; r0 < rs.n; r0 += 64)
            shrink_group_bf16(rs, r0, reinterpret_cast<const uint16_t*>(in), ld_in,
                              reinterpret_cast<const uint16_t*>(A), K, 1, a.r, a.r, 0, k0, k1, Pc,
                              a.r, sXA);
    } else {
        const int k0 = c * kKChunk;
        const int k1 = min(K, k0 + kKChunk);
        shrink_tile_simple<T>(rs, in, ld_in, A, K, 1, a.r, a.r, k0, k1, Pc, a.r);
    }
}

// bf16 shrink for sparse blocks: unit = (aligned block, K chunk of 1024, 16
// S columns).  With kNW waves, wave w takes K values [w 1024 / kNW, (w + 1)
// 1024 / kNW) of the chunk in 32 / kNW steps of v_mfma_f32_16x16x32_bf16,
// with 16 of the block's rows as the first operand and the unit's 16 A rows
// (kept in registers for every row group) as the second; the waves'
// partials are added in LDS in a fixed order.  Only real rows are visited,
// 16 at a time, so a block of ~16 real rows costs one MFMA chain per wave
// instead of a 64-row tile.  The partial goes to P (float) or, with a
// nonzero tag, into P's tagged exchange slot for the expand units of the
// same launch.  red: kNW * 256 floats of LDS.
constexpr int kNarrowK = 1024;

template <int kNW>
__device__ __forceinline__ void moe_shrink_unit(const MoeArgs& a, int which,
                                                const uint16_t* __restrict__ in, int64_t ld_in,
                                                float* __restrict__ P, int C, int G, int K,
                                                int unit, int* s_in, int* s_out, int* s_wlast,
                                                float* red, uint32_t tag) {
    constexpr int kNS = 32 / kNW;                 // MFMA steps per wave
    const int blk = unit / (C * G);
    const int c = (unit / G) % C;
    const int cb = unit % G;
    const int l = blk % a.L, b = blk / a.L;
    const MoeUnit mu = moe_unit(a, which, true, l, b, s_in, s_out, s_wlast);
    if (!mu.ok) return;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int lr = lane % 16, lq = lane / 16;
    const int64_t ew = moe_slot(a, which == 0, l, mu.e);
    const uint16_t* A = reinterpret_cast<const uint16_t*>(which == 0 ? a.A_gu : a.A_d) +
                        (ew * a.r + cb * 16 + lr) * K;
    const int kw = c * kNarrowK + wave * (32 * kNS) + lq * 8;   // this lane's first K value
    uint4 av[kNS];
#pragma unroll
    for (int kk = 0; kk < kNS; ++kk) av[kk] = ld16_if(A + kw + kk * 32, kw + kk * 32 < K, A);
    const int64_t cs = (int64_t)a.L * a.max_tokens_padded * a.r;
    for (int r0 = 0; r0 < mu.n; r0 += 16) {
        const int i = r0 + lr;
        const int xr = i < mu.n ? s_in[i] : -1;
        const uint16_t* xp = in + (int64_t)(xr < 0 ? 0 : xr) * ld_in;
        uint4 xv[kNS];
#pragma unroll
        for (int kk = 0; kk < kNS; ++kk)
            xv[kk] = ld16_if(xp + kw + kk * 32, xr >= 0 && kw + kk * 32 < K, in);
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < kNS; ++kk) acc = mfma_bf16(xv[kk], av[kk], acc);
        // acc[q]: block row r0 + 4 lq + q, S column cb*16 + lr
#pragma unroll
        for (int q = 0; q < 4; ++q) red[(wave * 16 + lq * 4 + q) * 16 + lr] = acc[q];
        __syncthreads();
        if (threadIdx.x < 256) {
            const int row = threadIdx.x / 16, col = threadIdx.x % 16;
            const int orow = r0 + row < mu.n ? s_out[r0 + row] : -1;
            if (orow >= 0) {
                float sum[kNW];
#pragma unroll
                for (int w = 0; w < kNW; ++w) sum[w] = red[(w * 16 + row) * 16 + col];
                // pairwise, in a fixed order
#pragma unroll
                for (int h = 1; h < kNW; h *= 2)
#pragma unroll
                    for (int w = 0; w + h < kNW; w += 2 * h) sum[w] += sum[w + h];
                const int64_t at = (int64_t)c * cs + (int64_t)orow * a.r + cb * 16 + col;
                if (tag != 0u)
                    slot_put(reinterpret_cast<slot_t*>(P) + at, sum[0], tag);
                else
                    P[at] = sum[0];
            }
        }
        __syncthreads();     // red is rewritten by the next row group
    }
}

// S rows of the aligned positions that exist (pos < ntpp[l]), the K chunks
// added in order; all of a batch's chunk loads are issued before any is added
// (one memory round trip per batch, not per chunk).  Padding positions
// (sentinel pairs) are read along but not stored: their S rows are never used.
constexpr int kMoeReduceBatch = 8;

__global__ void k_moe_reduce(const float* __restrict__ P, int C, int64_t cstride,
                             float* __restrict__ S, int r, int mtp,
                             const int32_t* __restrict__ ntpp,
                             const int32_t* __restrict__ sorted_ids, int npairs) {
    const int l = blockIdx.y;
    const int n = ntpp[l];
    const int64_t row0 = (int64_t)l * mtp;
    const int total4 = n * r / 4;
    const float4* P4 = reinterpret_cast<const float4*>(P);
    const int64_t c4 = cstride / 4;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total4; i += gridDim.x * blockDim.x) {
        const int64_t idx = row0 * r / 4 + i;
        const int f = sorted_ids[row0 + i * 4 / r];
        float4 acc = P4[idx];
        for (int c0 = 1; c0 < C; c0 += kMoeReduceBatch) {
            float4 v[kMoeReduceBatch];
#pragma unroll
            for (int q = 0; q < kMoeReduceBatch; ++q) v[q] = P4[min(c0 + q, C - 1) * c4 + idx];
#pragma unroll
            for (int q = 0; q < kMoeReduceBatch; ++q) {
                if (c0 + q < C) {
                    acc.x += v[q].x; acc.y += v[q].y; acc.z += v[q].z; acc.w += v[q].w;
                }
            }
        }
        if (f >= 0 && f < npairs) reinterpret_cast<float4*>(S)[idx] = acc;
    }
}

// fp32 expand: unit = (aligned block, 256 output columns), S from the reduce.
template <typename T>
__global__ __launch_bounds__(kTileThreads) void k_moe_expand(MoeArgs a, int which,
                                                              const float* __restrict__ S,
                                                              T* __restrict__ out, int64_t ld_out,
                                                              int N, int n_groups, int units) {
    __shared__ int s_in[kMaxRowTile], s_out[kMaxRowTile];
    __shared__ int s_wlast[kTileWaves];
    const int unit = (int)blockIdx.x;
    if (unit >= units) return;
    const int blk = unit / n_groups;
    const int g = unit % n_groups;
    const int l = blk % a.L, b = blk / a.L;
    const MoeUnit mu = moe_unit(a, which, false, l, b, s_in, s_out, s_wlast);
    if (!mu.ok) return;
    const int64_t ew = moe_slot(a, which == 1, l, mu.e);
    const T* B = reinterpret_cast<const T*>(which == 0 ? a.B_gu : a.B_d) + ew * (int64_t)N * a.r;
    const RowSet rs{mu.n, a.block_size_m, s_in, s_out};
    const int n0 = g * kNTile;
    expand_tile_simple<T>(rs, S, a.r, 0, B, a.r, n0, min(N, n0 + kNTile), out, ld_out);
}

template <int kSteps, bool kWide>
__global__ __launch_bounds__(kWide ? kWideThreads : kTileThreads)
__attribute__((amdgpu_waves_per_eu(kWide ? (kSteps == 1 ? 4 : 2) : 3))) void k_moe_delta(
    MoeArgs a, int which, const uint16_t* __restrict__ in, int64_t ld_in, float* __restrict__ P,
    int C, int G, int K, int nprod, uint16_t* __restrict__ out, int64_t ld_out, int N,
    int n_groups, int units, int* err, WaitCtl wc) {
    constexpr int kThreads = kWide ? kWideThreads : kTileThreads;
    constexpr int kNW = kThreads / kWave;
    static_assert(kNW * 256 * 4 <= (kWide ? kWideLds : kExpandLds), "shrink scratch must fit");
    __shared__ int s_in[kMaxRowTile], s_out[kMaxRowTile];
    __shared__ int s_wlast[kNW];
    __shared__ uint4 lds[(kWide ? kWideLds : kExpandLds) / 16];
    const uint32_t tag = launch_tag();
    if ((int)blockIdx.x < nprod) {
        moe_shrink_unit<kNW>(a, which, in, ld_in, P, C, G, K, (int)blockIdx.x, s_in, s_out,
                             s_wlast, reinterpret_cast<float*>(lds), tag);
        return;
    }
    const int unit = (int)blockIdx.x - nprod;
    if (unit >= units) return;
    const int blk = unit / n_groups;
    const int g = unit % n_groups;
    const int l = blk % a.L, b = blk / a.L;
    const MoeUnit mu = moe_unit(a, which, false, l, b, s_in, s_out, s_wlast);
    if (!mu.ok) return;
    const int64_t ew = moe_slot(a, which == 1, l, mu.e);
    const uint16_t* B =
        reinterpret_cast<const uint16_t*>(which == 0 ? a.B_gu : a.B_d) + ew * (int64_t)N * a.r;
    const RowSet rs{mu.n, a.block_size_m, s_in, s_out};
    const SChunks sc{C, (int64_t)a.L * a.max_tokens_padded * a.r, tag ^ wc.poll_xor, err,
                     wc.max_spin};
    if constexpr (kWide) {
        const int n0 = g * kWideCols;
        expand_rows_wide<kSteps>(rs, reinterpret_cast<const slot_t*>(P), a.r, 0, B, a.r, n0, min(N, n0 + kWideCols), out,
                                    ld_out, lds, sc);
    } else {
        const int n0 = g * kNTile;
        expand_rows_bf16<true, kSteps>(rs, P, a.r, 0, B, a.r, n0, min(N, n0 + kNTile), out, ld_out,
                                    lds, sc);
    }
}

template <int kSteps>
static void launch_moe_delta_bf16(const MoeArgs& a, int which, const uint16_t* in, int64_t ld_in,
                                  float* P, int C, int G, int K, int nprod, uint16_t* out,
                                  int64_t ld_out, int N, int nblk, int* err, hipStream_t st) {
    // wide 16 x 1024 tiles when the output is wide enough that 64 x 256 tiles
    // would need many rounds of mostly idle workgroups (the gate/up output)
    if (N >= 2 * kWideCols * 4) {
        const int wg = (N + kWideCols - 1) / kWideCols;
        const int units = a.L * nblk * wg;
        hipLaunchKernelGGL((k_moe_delta<kSteps, true>), dim3((unsigned)(nprod + units)),
                           dim3(kWideThreads), 0, st, a, which, in, ld_in, P, C, G, K, nprod, out,
                           ld_out, N, wg, units, err, wait_ctl());
    } else {
        const int ng = (N + kNTile - 1) / kNTile;
        const int units = a.L * nblk * ng;
        hipLaunchKernelGGL((k_moe_delta<kSteps, false>), dim3((unsigned)(nprod + units)),
                           dim3(kTileThreads), 0, st, a, which, in, ld_in, P, C, G, K, nprod, out,
                           ld_out, N, ng, units, err, wait_ctl());
    }
}

template <typename T>
static hipError_t moe_delta_t(const MoeArgs& a, int which, const void* in, int64_t ld_in,
                              void* out, int64_t ld_out, void* ws, hipStream_t st) {
    const int K = which == 0 ? a.H : a.I;
    const int N = which == 0 ? 2 * a.I : a.H;
    const int nblk = a.max_tokens_padded / a.block_size_m;
    const MoeWs W = moe_ws_layout(a.L, a.max_tokens_padded, a.r, a.H > a.I ? a.H : a.I);
    float* P = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + W.partial);
    if constexpr (sizeof(T) == 2) {
        // one launch; P holds the partials as tagged exchange slots (8 bytes each)
        const int C = (K + kNarrowK - 1) / kNarrowK;
        const int G = a.r / 16;
        const int nprod = a.L * nblk * C * G;
        int* err = &reinterpret_cast<WsHeader*>(reinterpret_cast<char*>(ws) + W.header)->error;
        const uint16_t* xin = reinterpret_cast<const uint16_t*>(in);
        uint16_t* o = static_cast<uint16_t*>(out);
        // rank <= 32: one 32-wide MFMA step, half the B operands in registers
        if (a.r <= 32)
            launch_moe_delta_bf16<1>(a, which, xin, ld_in, P, C, G, K, nprod, o, ld_out, N, nblk,
                                     err, st);
        else
            launch_moe_delta_bf16<2>(a, which, xin, ld_in, P, C, G, K, nprod, o, ld_out, N, nblk,
                                     err, st);
        return hipGetLastError();
    } else {
        // fp32: shrink into K-chunk partials, reduce into S, expand
        const int C = kchunks(K);
        float* S = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + W.S);
        const int units = a.L * nblk * C;
        hipLaunchKernelGGL((k_moe_shrink<T>), dim3((unsigned)(units > 0 ? units : 1)),
                           dim3(kTileThreads), 0, st, a, which, reinterpret_cast<const T*>(in),
                           ld_in, P, C, K, units);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t cstride = (int64_t)a.L * a.max_tokens_padded * a.r;
        int rb = (a.max_tokens_padded * a.r / 4 + 255) / 256;
        if (rb < 1) rb = 1;
        hipLaunchKernelGGL(k_moe_reduce, dim3((unsigned)rb, (unsigned)a.L), dim3(256), 0, st, P, C,
                           cstride, S, a.r, a.max_tokens_padded, a.ntpp, a.sorted_token_ids,
                           a.M * a.topk);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int n_groups = (N + kNTile - 1) / kNTile;
        const int units2 = a.L * nblk * n_groups;
        hipLaunchKernelGGL((k_moe_expand<T>), dim3((unsigned)(units2 > 0 ? units2 : 1)),
                           dim3(kTileThreads), 0, st, a, which, S, reinterpret_cast<T*>(out),
                           ld_out, N, n_groups, units2);
        return hipGetLastError();
    }
}

hipError_t launch_moe_delta(const MoeArgs& a, int which, const void* in, int64_t ld_in,
                            void* out, int64_t ld_out, void* ws, hipStream_t st) {
    return a.dtype == LORA_BF16 ? moe_delta_t<uint16_t>(a, which, in, ld_in, out, ld_out, ws, st)
                                : moe_delta_t<float>(a, which, in, ld_in, out, ld_out, ws, st);
}

// ---------------------------------------------------------------- silu_and_mul
__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

__global__ void k_silu_mul_bf16(const uint16_t* __restrict__ c1, int64_t ld1,
                                uint16_t* __restrict__ c2, int64_t ld2, int P, int I) {
    const int per_row = I / 8;
    const int64_t total = (int64_t)P * per_row;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t f = i / per_row;
        const int j = (int)(i - f * per_row) * 8;
        float g[8], u[8];
        Io<uint16_t>::ld8(c1 + f * ld1 + j, g);
        Io<uint16_t>::ld8(c1 + f * ld1 + I + j, u);
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            w[q] = f32_to_bf16(silu_f(g[2 * q]) * u[2 * q]) |
                   (f32_to_bf16(silu_f(g[2 * q + 1]) * u[2 * q + 1]) << 16);
        *reinterpret_cast<uint4*>(c2 + f * ld2 + j) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

__global__ void k_silu_mul_f32(const float* __restrict__ c1, int64_t ld1, float* __restrict__ c2,
                               int64_t ld2, int P, int I) {
    const int64_t total = (int64_t)P * I;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t f = i / I;
        const int j = (int)(i - f * I);
        c2[f * ld2 + j] = silu_f(c1[f * ld1 + j]) * c1[f * ld1 + I + j];
    }
}

hipError_t launch_silu_and_mul(int dtype, const void* c1, int64_t ld1, void* c2, int64_t ld2,
                               int P, int I, hipStream_t st) {
    // bf16: one 16-byte piece per thread, 512-thread workgroups (9.2 against
    // 9.5 us with 256 for the 512 x 14336 activation; more pieces per thread
    // and non-temporal loads were slower)
    const int threads = dtype == LORA_BF16 ? 512 : 256;
    const int64_t work = dtype == LORA_BF16 ? (int64_t)P * I / 8 : (int64_t)P * I;
    int64_t blocks = (work + threads - 1) / threads;
    if (blocks > 16384) blocks = 16384;
    if (blocks < 1) blocks = 1;
    if (dtype == LORA_BF16)
        hipLaunchKernelGGL(k_silu_mul_bf16, dim3((unsigned)blocks), dim3(threads), 0, st,
                           (const uint16_t*)c1, ld1, (uint16_t*)c2, ld2, P, I);
    else
        hipLaunchKernelGGL(k_silu_mul_f32, dim3((unsigned)blocks), dim3(threads), 0, st,
                           (const float*)c1, ld1, (float*)c2, ld2, P, I);
    return hipGetLastError();
}

// ---------------------------------------------------------------- top-k reduce
template <typename T>
__global__ void k_topk_reduce(const T* __restrict__ c3, int64_t ld3, const float* __restrict__ w,
                              T* __restrict__ out, int64_t ldo, int M, int topk, int H) {
    const int per_row = H / 8;
    const int64_t total = (int64_t)M * per_row;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t m = i / per_row;
        const int h = (int)(i - m * per_row) * 8;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int k = 0; k < topk; ++k) {
            const float wk = w[m * topk + k];
            float v[8];
            Io<T>::ld8(c3 + (m * topk + k) * ld3 + h, v);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += wk * v[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) Io<T>::st(out + m * ldo + h + e, acc[e]);
    }
}

hipError_t launch_topk_reduce(int dtype, const void* c3, int64_t ld3, const float* w, void* out,
                              int64_t ldo, int M, int topk, int H, hipStream_t st) {
    int64_t blocks = ((int64_t)M * H / 8 + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    if (blocks < 1) blocks = 1;
    if (dtype == LORA_BF16)
        hipLaunchKernelGGL(k_topk_reduce<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, st,
                           (const uint16_t*)c3, ld3, w, (uint16_t*)out, ldo, M, topk, H);
    else
        hipLaunchKernelGGL(k_topk_reduce<float>, dim3((unsigned)blocks), dim3(256), 0, st,
                           (const float*)c3, ld3, w, (float*)out, ldo, M, topk, H);
    return hipGetLastError();
}

}  // namespace mlora
