// The base layer and its LoRA delta in one product (Ascend walkthrough,
// section 1.1: y = x W^T + (x A^T) B^T; SGLang "LoRA Layers" page, structure
// diagram: base_output + lora_delta):
//     y[m, n] = sum_k x[m, k] W[n, k] + sum_{j < rp} S[p, sl, j] B_i[n, j]
// with S = x A_i^T from lora_shrink (fp32, sorted rows).  y is written once;
// there is no read-modify-write of a separately stored base output.
//
// Work unit = (128 consecutive sorted positions, 256 output columns of one
// slice); the rows of a unit may belong to several segments and to tokens
// without an adapter.  Four waves, one per SIMD; wave w owns columns
// [64 w, 64 w + 64) of the unit for all 128 rows: 4 x 2 blocks of
// v_mfma_f32_32x32x16_bf16 (the 32 x 32 form keeps the matrix unit busy from
// a single wave), K in stages of 64.
//
// Both operands are staged through an LDS ring of three stages (48 KB each:
// 128 x rows and 256 W rows of 128 bytes).  Global loads read whole 128-byte
// row segments (eight lanes per row), two stages ahead in registers; a stage
// is written to the ring two stages before its use, so the next stage is
// always readable and each wave fetches its first operands while it
// multiplies the last K step of the current one.  One barrier per stage.
// 16-byte chunks of a row are XOR-swizzled so that the operand reads (32 rows,
// one chunk) and the staging writes (8 rows, 8 chunks) hit distinct banks.
// The stage count is rounded up to even: stages past K meet x values cleared
// to zero.  Every load is issued on every path (past the end from clamped
// addresses), so the number of loads in flight is the same everywhere and the
// compiler's waits keep the newer stage in flight.
//
// Epilogue: the unit's S values and the B operands of its first two
// segments are loaded during the last two stages, which need no global loads
// or LDS writes of their own.  The S values go to LDS once as a bf16 hi / lo
// pair; each segment that meets the unit's rows (and has a nonzero rank)
// then multiplies its rows of them, selected by a mask on the operand, with
// the adapter's B rows on the same MFMA blocks.  One bf16 rounding, staged
// through LDS so that each output row is written in 16-byte pieces by token
// index.
#include "common.hpp"
#include "kernels.hpp"

namespace mlora {

constexpr int kGM = 128;                 // rows per unit
constexpr int kGN = 256;                 // columns per unit
constexpr int kGK = 64;                  // K per stage
constexpr int kGRing = 3;                // LDS stages
constexpr int kGStage = (kGM + kGN) * 8; // uint4 per stage (48 KB)
constexpr int kGThreads = 256;
constexpr int kGRB = kGM / 32;           // 32-row blocks per wave
constexpr int kGCB = 2;                  // 32-column blocks per wave
constexpr int kGXL = kGM / 32;           // x rows loaded per thread and stage
constexpr int kGWL = kGN / 32;           // W rows loaded per thread and stage
constexpr int kSLD = LORA_MAX_RANK + 8;  // bf16 row stride of the staged S
static_assert(kGM * kSLD * 2 * 2 <= kGRing * kGStage * 16, "staged S must fit the ring");
static_assert(4 * kGM * 72 * 2 <= kGRing * kGStage * 16, "staged output must fit the ring");

// Position of 16-byte chunk c of row r (rows of 128 bytes): the chunk is
// permuted by (r ^ (r / 8)) % 8, which gives 8 consecutive rows distinct
// chunks within 128 bytes of banks and 16 consecutive rows distinct
// 16-byte bank groups within 256 bytes.
__device__ __forceinline__ int gsw(int r, int c) { return r * 8 + (c ^ ((r ^ (r >> 3)) & 7)); }

struct GemmParams {
    LinearArgs a;
    const uint16_t* x;
    int64_t ldx;
    const uint16_t* W;
    int64_t ldw;
    uint16_t* y;
    int64_t ldy;
    const float* S;              // fp32 [M][cols], sorted rows
    int col_tiles;               // 256-column tiles over all slices
    int tile_start[LORA_MAX_SLICES + 1];
    int nk2;                     // stages, rounded up to even
    int seg_stride;              // ceil((L + 1) / 64): first-round search stride
};

__global__ __launch_bounds__(kGThreads, 1) void k_gemm_lora(GemmParams p) {
    __shared__ uint4 smem[kGRing * kGStage];
    __shared__ int s_tok[kGM];
    const LinearArgs& a = p.a;
    const int u = (int)blockIdx.x;
    const int rt = u / p.col_tiles;
    const int ct = u % p.col_tiles;
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int lr = lane % 32, lh = lane / 32;
    const int p0 = rt * kGM;
    const int rows = min(kGM, a.M - p0);
    const int K = a.K;

    // first round of the segment search, needed only by the epilogue:
    // lane j holds seg_indptr[j * stride] (entries past the segments hold
    // the number of tokens with an adapter)
    const int L = a.L;
    const int srch1 = a.seg_indptr[min(lane * p.seg_stride, L)];
    const int m_valid = a.seg_indptr[L];
    const int nseg = a.num_segments[0];
    // with fewer than 64 adapter slots the stride is 1 and lane j holds
    // segment start j; with it, lane j also loads segment j's adapter and
    // slot j's rank and B offset, so the unit's segments need no further
    // round of loads
    const bool quick = L < kWave;
    const int lq = min(lane, max(L - 1, 0));
    const int q_id = a.req_to_lora[lq];
    const int q_rk = a.rank[lq];
    const int64_t q_bo = a.b_off[lq];

    if (tid < kGM) {
        int m = tid < rows ? a.sorted_idx[p0 + tid] : -1;
        // (checked builds) a token index outside the batch is never stored
        if (table_fault(a.err, tid < rows && (m < 0 || m >= a.M))) {
            if (tid < rows && (m < 0 || m >= a.M)) m = -1;
        }
        s_tok[tid] = m;
    }

    // ---- columns of the unit (one slice)
    int sl = 0;
    while (sl + 1 < a.n_sl && ct >= p.tile_start[sl + 1]) ++sl;
    const int n0 = (int)(a.slice_off[sl] + (int64_t)(ct - p.tile_start[sl]) * kGN);
    const int n1 = (int)min((int64_t)n0 + kGN, a.slice_off[sl + 1]);

    // ---- staging: thread t loads 16-byte chunk t % 8 of rows t / 8 + 32 i
    const int tr = tid / 8, tc = tid % 8;
    const uint16_t* xrow[kGXL];
#pragma unroll
    for (int i = 0; i < kGXL; ++i) {
        const int m = a.sorted_idx[p0 + min(tr + 32 * i, rows - 1)];
        xrow[i] = p.x + (int64_t)((kTableChecks && (m < 0 || m >= a.M)) ? 0 : m) * p.ldx;
    }
    const uint16_t* wrow[kGWL];
#pragma unroll
    for (int i = 0; i < kGWL; ++i)
        wrow[i] = p.W + (int64_t)min(n0 + tr + 32 * i, n1 - 1) * p.ldw;

    uint4 rs[2][kGXL + kGWL];   // stages in flight (stage s in slot s % 2)
    auto kx = [&](int s) { return min(s * kGK + tc * 8, K - 8); };
    auto gload = [&](int s, int slot) {
        const int k = kx(s);
#pragma unroll
        for (int i = 0; i < kGXL; ++i) rs[slot][i] = ld16(xrow[i] + k);
#pragma unroll
        for (int i = 0; i < kGWL; ++i) rs[slot][kGXL + i] = ld16(wrow[i] + k);
    };
    auto lstore = [&](int s, int slot) {
        // x values past K are cleared; W there meets only those zeros
        const uint32_t m = opaque_mask(s * kGK + tc * 8 < K);
        uint4* st = smem + (s % kGRing) * kGStage;
#pragma unroll
        for (int i = 0; i < kGXL; ++i) {
            const uint4 v = rs[slot][i];
            st[gsw(tr + 32 * i, tc)] = make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
        }
#pragma unroll
        for (int i = 0; i < kGWL; ++i) st[kGM * 8 + gsw(tr + 32 * i, tc)] = rs[slot][kGXL + i];
    };
    // one load or one LDS write of the twelve per thread and stage
    // (i < 4: x rows, else W rows); `i` is a literal at every call
    auto gload1 = [&](int s, int slot, int i) {
        rs[slot][i] = ld16((i < kGXL ? xrow[i] : wrow[i - kGXL]) + kx(s));
    };
    auto lstore1 = [&](int s, int slot, int i) {
        uint4* st = smem + (s % kGRing) * kGStage;
        if (i < kGXL) {
            const uint32_t m = opaque_mask(s * kGK + tc * 8 < K);
            const uint4 v = rs[slot][i];
            st[gsw(tr + 32 * i, tc)] = make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
        } else {
            st[kGM * 8 + gsw(tr + 32 * (i - kGXL), tc)] = rs[slot][i];
        }
    };
    // MFMA operands of K step t (16 wide) of stage s
    struct Ops {
        uint4 a[kGRB];
        uint4 b[kGCB];
    };
    auto oread = [&](int s, int t) {
        const uint4* st = smem + (s % kGRing) * kGStage;
        Ops o;
#pragma unroll
        for (int rb = 0; rb < kGRB; ++rb) o.a[rb] = st[gsw(rb * 32 + lr, 2 * t + lh)];
#pragma unroll
        for (int cb = 0; cb < kGCB; ++cb)
            o.b[cb] = st[kGM * 8 + gsw(wave * 64 + cb * 32 + lr, 2 * t + lh)];
        return o;
    };

    // one of the six operand reads of K step t (j < 4: x rows, else W rows)
    auto oread1 = [&](Ops& o, int s, int t, int j) {
        const uint4* st = smem + (s % kGRing) * kGStage;
        if (j < kGRB) o.a[j] = st[gsw(j * 32 + lr, 2 * t + lh)];
        else o.b[j - kGRB] = st[kGM * 8 + gsw(wave * 64 + (j - kGRB) * 32 + lr, 2 * t + lh)];
    };

    f32x16_t acc[kGRB][kGCB];
#pragma unroll
    for (int rb = 0; rb < kGRB; ++rb)
#pragma unroll
        for (int cb = 0; cb < kGCB; ++cb)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[rb][cb][q] = 0.f;
    auto mfma1 = [&](const Ops& o, int i) {
        const int rb = i / kGCB, cb = i % kGCB;
        acc[rb][cb] = mfma32_bf16(o.a[rb], o.b[cb], acc[rb][cb]);
    };

    // prologue: stages 0 and 1 in LDS, stages 2 and 3 in flight, the first
    // operands of stage 0 read
    gload(0, 0);
    gload(1, 1);
    lstore(0, 0);
    gload(2, 0);
    lstore(1, 1);
    gload(3, 1);
    __syncthreads();
    Ops o0 = oread(0, 0);

    // the unit's first two segments (start, end, rank, B offset; rank 0:
    // none), for the B operands loaded during the last two stages
    int sfirst = 0;
    int pk_beg[2] = {0, 0}, pk_end[2] = {0, 0}, pk_rp[2] = {0, 0};
    int64_t pk_bo[2] = {0, 0};
    if (quick && p0 < m_valid) {
        sfirst = 63 - __clzll((long long)__ballot(lane <= L && srch1 <= p0));
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int sj = sfirst + j;
            if (sj >= nseg) break;
            pk_beg[j] = __builtin_amdgcn_readlane(srch1, sj);
            pk_end[j] = __builtin_amdgcn_readlane(srch1, sj + 1);
            const int id = __builtin_amdgcn_readlane(q_id, sj);
            if (pk_beg[j] < p0 + rows && id >= 0 && id < L) {
                pk_rp[j] = __builtin_amdgcn_readlane(q_rk, id);
                pk_bo[j] = readlane64(q_bo, id);
            }
        }
    }

    // stage ks; `slot` (ks & 1) is a literal at every call.  The ring slot of
    // stage ks + 2 was last read (stage ks - 1) before the previous barrier;
    // stage ks + 1 was written a stage ago, before that barrier.  With one
    // wave per SIMD, anything issued between MFMAs would leave the matrix
    // unit idle, so each MFMA (32 cycles) is followed by at most one LDS write
    // or one global load, and one operand read for the next K step, in a
    // fixed order: the writes of stage ks + 2 during the first two K steps,
    // the loads of stage ks + 4 (into the registers just written out) during
    // the last two.
    //
    // `mode` (a literal at every call): 0 = as above; 1 = no global loads
    // (stages ks + 4 do not exist); 2 = MFMAs and operand reads only (the
    // last two stages: nothing left to write, no barrier); 3 = the same
    // without the reads for a next stage.
    auto step = [&](int ks, int slot, int mode) {
        Ops o1, o2, o3;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            mfma1(o0, i);
            if (i < 6) oread1(o1, ks, 1, i);
            if (i < 6 && mode < 2) lstore1(ks + 2, slot, i);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            mfma1(o1, i);
            if (i < 6) oread1(o2, ks, 2, i);
            if (i < 6 && mode < 2) lstore1(ks + 2, slot, 6 + i);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            mfma1(o2, i);
            if (i < 6) oread1(o3, ks, 3, i);
            if (i < 6 && mode == 0) gload1(ks + 4, slot, i);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            mfma1(o3, i);
            if (i < 6 && mode < 3) oread1(o0, ks + 1, 0, i);
            if (i < 6 && mode == 0) gload1(ks + 4, slot, 6 + i);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (mode < 2) __syncthreads();
    };
    int ks = 0;
    for (; ks + 4 < p.nk2; ks += 2) {
        step(ks, 0, 0);
        step(ks + 1, 1, 0);
    }
    if (p.nk2 >= 4) {
        step(ks, 0, 1);
        step(ks + 1, 1, 1);
        ks += 2;
    }

    // ---- LoRA operands, loaded during the last two stages: the unit's S
    // values for this slice, the same for every segment (thread t: row t / 2,
    // rank positions 32 (t % 2) + 4 e, clamped into the row; positions past a
    // segment's rank are never multiplied), and the B operands of the first
    // two segments (rank steps t < rp / 16, as below)
    const bool lora = p0 < m_valid && a.r_max > 0;
    float4 sv[8];
    uint4 pb[2][kGCB][4];
    if (lora) {
        const int srow = min(p0 + tid / 2, a.M - 1);
        const float* sp = p.S + (int64_t)srow * a.cols + sl * a.r_max;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            sv[e] = *reinterpret_cast<const float4*>(sp + min((tid % 2) * 32 + 4 * e, a.r_max - 4));
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (pk_rp[j] == 0) continue;
            const int rp = pk_rp[j];
            const uint16_t* Bt = reinterpret_cast<const uint16_t*>(a.B) + pk_bo[j];
#pragma unroll
            for (int cb = 0; cb < kGCB; ++cb) {
                const int n = min(n0 + wave * 64 + cb * 32 + lr, n1 - 1);
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    pb[j][cb][t] = ld16(Bt + (int64_t)n * rp + min(t * 16, rp - 16) + lh * 8);
            }
        }
    }
    step(ks, 0, 2);
    step(ks + 1, 1, 3);
    __syncthreads();     // every wave is done with the ring

    // ---- LoRA epilogue: the unit's S values as a bf16 hi / lo pair in LDS,
    // then one pass per segment that meets the unit's rows, its S rows picked
    // by a row mask on the operand
    if (lora) {
        uint16_t* sHi = reinterpret_cast<uint16_t*>(smem);   // the ring is free now
        uint16_t* sLo = sHi + kGM * kSLD;
        {
            const int row = tid / 2, j0 = (tid % 2) * 32;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float f[4] = {sv[e].x, sv[e].y, sv[e].z, sv[e].w};
                uint32_t h[4], l[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    h[q] = f32_to_bf16(f[q]);
                    l[q] = f32_to_bf16(f[q] - bf16_to_f32(h[q]));
                }
                *reinterpret_cast<uint2*>(sHi + row * kSLD + j0 + 4 * e) =
                    make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
                *reinterpret_cast<uint2*>(sLo + row * kSLD + j0 + 4 * e) =
                    make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
            }
        }
        __syncthreads();
        // segment of sorted position p0: the last s with seg_indptr[s] <= p0
        int s0 = sfirst;
        if (!quick) {
            const uint64_t b1 = __ballot(lane * p.seg_stride <= L && srch1 <= p0);
            const int lo = (63 - __clzll((long long)b1)) * p.seg_stride;
            const int v2 = a.seg_indptr[min(lo + lane, L)];
            const uint64_t b2 = __ballot(lane < p.seg_stride && lo + lane <= L && v2 <= p0);
            s0 = lo + 63 - __clzll((long long)b2);
        }
        for (int s = s0; s < nseg; ++s) {
            const int k = quick ? s - s0 : 2;       // 0, 1: the prefetched segments
            int beg, end, rp;
            int64_t bo = 0;
            uint4 bop[kGCB][4];
            if (k == 0) {
                beg = pk_beg[0]; end = pk_end[0]; rp = pk_rp[0];
            } else if (k == 1) {
                beg = pk_beg[1]; end = pk_end[1]; rp = pk_rp[1];
            } else {
                beg = a.seg_indptr[s];
                end = a.seg_indptr[s + 1];
                const int id = a.req_to_lora[s];
                const bool id_ok = id >= 0 && id < L;   // never index past the table
                table_fault(a.err, beg < p0 + rows && !id_ok);
                rp = (beg < p0 + rows && id_ok) ? a.rank[id] : 0;
                bo = id_ok ? a.b_off[id] : 0;
            }
            if (beg >= p0 + rows) break;
            if (rp == 0) continue;
            if (k == 0) {
#pragma unroll
                for (int cb = 0; cb < kGCB; ++cb)
#pragma unroll
                    for (int t = 0; t < 4; ++t) bop[cb][t] = pb[0][cb][t];
            } else if (k == 1) {
#pragma unroll
                for (int cb = 0; cb < kGCB; ++cb)
#pragma unroll
                    for (int t = 0; t < 4; ++t) bop[cb][t] = pb[1][cb][t];
            } else {
                const uint16_t* Bt = reinterpret_cast<const uint16_t*>(a.B) + bo;
#pragma unroll
                for (int cb = 0; cb < kGCB; ++cb) {
                    const int n = min(n0 + wave * 64 + cb * 32 + lr, n1 - 1);
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        bop[cb][t] = ld16(Bt + (int64_t)n * rp + min(t * 16, rp - 16) + lh * 8);
                }
            }
            const int r0 = max(beg - p0, 0), r1 = min(end - p0, rows);
#pragma unroll
            for (int rb = 0; rb < kGRB; ++rb) {
                if (rb * 32 + 32 <= r0 || rb * 32 >= r1) continue;
                const int row = rb * 32 + lr;
                const uint32_t m = opaque_mask(row >= r0 && row < r1);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    if (t * 16 >= rp) continue;
                    const int o = row * kSLD + t * 16 + lh * 8;
                    const uint4 h0 = *reinterpret_cast<const uint4*>(sHi + o);
                    const uint4 l0 = *reinterpret_cast<const uint4*>(sLo + o);
                    const uint4 h = make_uint4(h0.x & m, h0.y & m, h0.z & m, h0.w & m);
                    const uint4 l = make_uint4(l0.x & m, l0.y & m, l0.z & m, l0.w & m);
#pragma unroll
                    for (int cb = 0; cb < kGCB; ++cb) {
                        acc[rb][cb] = mfma32_bf16(h, bop[cb][t], acc[rb][cb]);
                        acc[rb][cb] = mfma32_bf16(l, bop[cb][t], acc[rb][cb]);
                    }
                }
            }
        }
        __syncthreads();     // the output staging below reuses the S rows' LDS
    }

    // ---- store through LDS (the ring is free: every wave has passed the last
    // barrier): each wave stages its 128 x 64 block as bf16, rows of 72
    // values, then writes whole 16-byte row pieces.  acc[rb][cb][q] is row
    // 32 rb + 8 (q / 4) + 4 lh + q % 4, column 64 w + 32 cb + lr.  A wave reads
    // back only what it wrote itself, so no barrier is needed.
    {
        constexpr int OLD = 72;
        uint16_t* so = reinterpret_cast<uint16_t*>(smem) + wave * kGM * OLD;
#pragma unroll
        for (int rb = 0; rb < kGRB; ++rb)
#pragma unroll
            for (int cb = 0; cb < kGCB; ++cb)
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    so[(rb * 32 + (q / 4) * 8 + lh * 4 + q % 4) * OLD + cb * 32 + lr] =
                        (uint16_t)f32_to_bf16(acc[rb][cb][q]);
        const int c = lane % 8;
        const int n = n0 + wave * 64 + c * 8;       // slices are multiples of 8 wide
#pragma unroll
        for (int j = 0; j < kGM / 8; ++j) {
            const int row = j * 8 + lane / 8;
            const int m = s_tok[row];
            const uint4 v = *reinterpret_cast<const uint4*>(so + row * OLD + c * 8);
            if (m >= 0 && n < n1) *reinterpret_cast<uint4*>(p.y + (int64_t)m * p.ldy + n) = v;
        }
    }
}

hipError_t launch_gemm_lora(const LinearArgs& a, const void* x, int64_t ldx, const void* W,
                            int64_t ldw, const float* S, void* y, int64_t ldy, hipStream_t st) {
    GemmParams p{};
    p.a = a;
    p.x = static_cast<const uint16_t*>(x);
    p.ldx = ldx;
    p.W = static_cast<const uint16_t*>(W);
    p.ldw = ldw;
    p.y = static_cast<uint16_t*>(y);
    p.ldy = ldy;
    p.S = S;
    int t = 0;
    for (int s = 0; s < a.n_sl; ++s) {
        p.tile_start[s] = t;
        t += (int)((a.slice_off[s + 1] - a.slice_off[s] + kGN - 1) / kGN);
    }
    p.tile_start[a.n_sl] = t;
    p.col_tiles = t;
    const int nk = (a.K + kGK - 1) / kGK;
    p.nk2 = (nk + 1) / 2 * 2;
    p.seg_stride = (a.L + 1 + kWave - 1) / kWave;
    const int row_units = (a.M + kGM - 1) / kGM;
    const unsigned grid = (unsigned)(row_units * p.col_tiles);
    hipLaunchKernelGGL(k_gemm_lora, dim3(grid), dim3(kGThreads), 0, st, p);
    return hipGetLastError();
}

}  // namespace mlora
