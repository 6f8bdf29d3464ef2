// Work-unit tiles shared by the dense multi-LoRA kernels and the MoE-LoRA
// kernels.  A unit owns up to RT gathered rows that all use one adapter
// (one expert for MoE) and either
//   * a K chunk of the shrink product  P[c][row][col] = sum_k x[row, k] A[col, k]
//     (partial sums over the chunk; a reduce step adds the chunks), or
//   * a 256-column tile of the expand product  y[row, n] += sum_j S[row, j] B[n, j].
//
// Both run on bf16 MFMA (v_mfma_f32_16x16x32_bf16).  Operand layout of one
// 16x16x32 step for lane l: A-operand row (l % 16), eight consecutive K
// values starting at 8*(l / 16); B-operand column (l % 16), the same eight
// K values; result rows 4*(l / 16) + q, q = 0..3, column l % 16.  Both
// products read their operands K-contiguous straight from the row-major
// tables (x and A rows for the shrink, B rows and S rows for the expand), so
// no transposes are made anywhere.
//
// The expand feeds S to the MFMA as a bf16 pair (hi = rne(S), lo = rne(S - hi)),
// two MFMAs per step, which keeps the product within ~2^-16 of fp32.
#pragma once

#include "common.hpp"

namespace mlora {

// Split 8 fp32 values into bf16 hi / lo parts (8 each).
__device__ __forceinline__ void split_hi_lo(const float* v, uint4& hi, uint4& lo) {
    uint32_t h[8], l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        h[i] = f32_to_bf16(v[i]);
        l[i] = f32_to_bf16(v[i] - bf16_to_f32(h[i]));
    }
    hi = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                    h[6] | (h[7] << 16));
    lo = make_uint4(l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16),
                    l[6] | (l[7] << 16));
}

constexpr int kTileThreads = 256;

// Work units are numbered by blockIdx directly.  The hardware hands
// consecutive workgroups to the 8 XCDs round robin, which spreads the units
// that find no work (tiles past the schedule, empty MoE blocks) evenly over
// the XCDs; grouping consecutive units on one XCD for L2 reuse left half of
// the XCDs idle when the empty units were contiguous.
constexpr int kTileWaves = kTileThreads / kWave;
constexpr int kMaxRowTile = 256;

// Rows of one unit, staged in LDS by the unit decoder.
struct RowSet {
    int n;                   // rows in this unit (<= RT)
    int RT;                  // row tile (multiple of 16, <= kMaxRowTile)
    const int* in_row;       // LDS [RT]: input row index, -1 = padding row
    const int* out_row;      // LDS [RT]: output row index, -1 = padding row
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// ---------------------------------------------------------------------------
// shrink unit: P[out_row][cg*64 + c] = sum_{k0 <= k < k1} x[in_row, k] A[row(c), k]
// for the 64 S columns of column group cg and up to 64 rows (k1 - k0 <= 512).
//   S column block cbg (16 columns) = slice sl = cbg / (r_max/16), block
//   jj = cbg % (r_max/16); it is active when jj < rp/16 and then reads
//   adapter rows sl*rp + jj*16 .. +16; inactive blocks store zeros (rank
//   padding).
// The A chunk (up to 64 rows x 512 K, 64 KB) goes to LDS with direct
// global->LDS loads: one wave instruction moves one 1 KB row segment, lane l
// fetching the 16-byte chunk that belongs at its LDS position (chunk q of row
// r sits at position q ^ (r & 15), so the MFMA operand reads of 16
// consecutive rows hit 64 distinct banks).  No registers hold A on the way.
// Each wave keeps its 16 x rows for the chunk in registers; the x loads are
// issued together with the A loads, so a unit costs one memory round trip.
// ---------------------------------------------------------------------------
constexpr int kShrinkK = 512;
// the A chunk is staged one row per direct-load instruction (64 lanes x 16 B)
static_assert(kShrinkK * 2 == kWave * 16, "an A row of the K chunk is one wave's direct load");
constexpr int kGroupCols = 64;
constexpr int kShrinkLds = kGroupCols * kShrinkK * 2;   // bytes: the A chunk

__device__ __forceinline__ int swz(int r, int q) { return r * (kShrinkK / 8) + (q ^ (r & 15)); }

// The MFMA steps of one shrink unit over the first NB column blocks.  There
// is no branch in the loop and each step's LDS operand reads are issued one
// step ahead of its MFMAs, so operand reads and matrix work overlap (a branch
// per block inside the loop makes every MFMA wait out its own LDS read).
template <int NB>
__device__ __forceinline__ void shrink_mfma_steps(const uint4* __restrict__ sA, const uint4* xv,
                                                  f32x4_t* acc, int lr, int lq) {
    constexpr int KS = kShrinkK / 32;
    uint4 b[2][NB];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) b[0][cb] = sA[swz(cb * 16 + lr, lq)];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        if (kk + 1 < KS) {
#pragma unroll
            for (int cb = 0; cb < NB; ++cb)
                b[(kk + 1) & 1][cb] = sA[swz(cb * 16 + lr, (kk + 1) * 4 + lq)];
        }
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) acc[cb] = mfma_bf16(xv[kk], b[kk & 1][cb], acc[cb]);
    }
}

__device__ __forceinline__ void shrink_group_bf16(const RowSet& rs, int r0,
                                                  const uint16_t* __restrict__ x, int64_t ldx,
                                                  const uint16_t* __restrict__ A, int K, int n_sl,
                                                  int rp, int r_max, int cg, int k0, int k1,
                                                  float* __restrict__ P, int pld,
                                                  uint4* __restrict__ sA) {
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int bps = r_max / 16;
    const int nbr = rp / 16;
    const int lr = lane % 16;
    const int lq = lane / 16;                 // 16-byte chunk within a 32-wide K step
    const int rows = min(64, rs.n - r0);
    const int nq = (k1 - k0) / 8;             // valid 16-byte chunks per row segment
    bool act[4];
    int arow[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const int cbg = cg * 4 + cb;
        const int sl = cbg / bps, jj = cbg % bps;
        act[cb] = sl < n_sl && jj < nbr;
        arow[cb] = sl * rp + jj * 16;
    }
    const bool any = act[0] || act[1] || act[2] || act[3];
    // 1. A rows 16w .. 16w+15 of the group (column block w), one row per
    //    instruction; chunks past k1 repeat the row's last valid chunk (their
    //    x partners are zero)
    if (act[wave]) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = wave * 16 + i;
            const int q = min(lane ^ i, nq - 1);     // chunk stored at position `lane`
            const uint16_t* src = A + (int64_t)(arow[wave] + i) * K + k0 + q * 8;
            __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(sA + r * (kShrinkK / 8)), 16, 0, 0);
        }
    }
    // 2. this wave's 16 x rows (rows 16w + lr), chunks kk*4 + lq
    const int rg = wave;
    uint4 xv[kShrinkK / 32];
    {
        const int i = rg * 16 + lr;
        const int xr = (i < rows) ? rs.in_row[r0 + i] : -1;
        const uint16_t* xp = x + (int64_t)(xr < 0 ? 0 : xr) * ldx + k0 + lq * 8;
#pragma unroll
        for (int kk = 0; kk < kShrinkK / 32; ++kk)
            xv[kk] = ld16_if(xp + kk * 32, any && xr >= 0 && kk * 4 + lq < nq, x);
    }
    __builtin_amdgcn_s_waitcnt(0);    // direct-to-LDS loads are tracked by vmcnt only
    __syncthreads();
    f32x4_t acc[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (any && rg * 16 < rows) {
        // active blocks are a prefix for one slice (rank blocks 0 .. rp/16-1);
        // other patterns run all four and drop the blocks without A rows
        const int mask = (act[0] ? 1 : 0) | (act[1] ? 2 : 0) | (act[2] ? 4 : 0) | (act[3] ? 8 : 0);
        if (mask == 1) {
            shrink_mfma_steps<1>(sA, xv, acc, lr, lq);
        } else if (mask == 3) {
            shrink_mfma_steps<2>(sA, xv, acc, lr, lq);
        } else if (mask == 7) {
            shrink_mfma_steps<3>(sA, xv, acc, lr, lq);
        } else {
            shrink_mfma_steps<4>(sA, xv, acc, lr, lq);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
                if (!act[cb]) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
        const int row = rg * 16 + lq * 4 + qq;
        const int orow = (row < rows) ? rs.out_row[r0 + row] : -1;
        if (orow < 0) continue;
        float* pp = P + (int64_t)orow * pld + cg * kGroupCols + lr;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
            if (cg * kGroupCols + cb * 16 < pld) pp[cb * 16] = acc[cb][qq];
    }
    __syncthreads();     // sA is reused by the next row block
}

// ---------------------------------------------------------------------------
// expand: y[out_row, n] += sum_{j < rp} S[srow, sc0 + j] * B[n, j] for
// n in [n_begin, n_end), walked in 64-row x 256-column tiles.  S rows come
// from rs.in_row (index into S), y rows from rs.out_row.
// ---------------------------------------------------------------------------
// One 64-row x 256-column output tile, y staged in LDS as bf16.
//   1. the y tile is copied into LDS with direct global->LDS loads (no
//      registers; one wave instruction moves two rows x 512 bytes, lane l
//      fetching the 16-byte chunk that belongs at its LDS position: chunk q
//      of row r sits at position q ^ (r & 15)); S rows are loaded and split
//      into bf16 hi / lo parts in LDS; the B operands of the wave's 64
//      columns go to registers — all before anything waits;
//   2. wave w runs the MFMAs for columns n0 + 64w .. +64 of all 64 rows and
//      adds each 16 x 16 result into the LDS tile (one rounding per element);
//   3. the tile is written back row-major (2 rows x 512 bytes per instruction).
// 16-byte store marked non-temporal (streamed past the caches' retention):
// the expand's y tiles are written once and not read again by the kernel.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st_nt16(void* p, const uint4& v) {
    const u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}

constexpr int kYRowBytes = kNTile * 2;                       // 512
constexpr int kSLds = LORA_MAX_RANK + 8;                     // bf16 row stride of staged S
constexpr int kExpandLds = 64 * kYRowBytes + 2 * 64 * kSLds * 2;   // bytes

__device__ __forceinline__ int ypos(int r, int q) { return r * (kYRowBytes / 16) + (q ^ (r & 15)); }

// Partial sums of S handed to the expand instead of S itself: the S value
// at an offset is the sum of `C` chunk partials `cs` slots apart, added in
// chunk order, each a tagged exchange slot of the launch with tag `tag`.
struct SChunks {
    int C;
    int64_t cs;
    uint32_t tag;     // what a full slot carries (the launch's tag, XOR the wait control's)
    int* err;         // sticky error word for a wait that runs out (may be null)
    int max_spin;     // polls before a wait gives up
};

// Sum of chunks [c0, c1) of one float4 of S held in tagged exchange slots,
// in chunk order; each chunk's four slots are polled (kSlotBatch chunks
// together) until they carry the launch's tag.  A wait that runs out sets
// `timeout` and leaves the missing partials out.
template <int kSlotBatch>
__device__ __forceinline__ float4 slot_range_sum(const slot_t* p, SChunks sc, int c0, int c1,
                                                 bool& timeout) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int cb = c0; cb < c1; cb += kSlotBatch) {
        slot_t w[kSlotBatch][4];
        for (int spin = 0;; ++spin) {
            bool all = true;
#pragma unroll
            for (int q = 0; q < kSlotBatch; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    w[q][e] = cb + q < c1 ? slot_load(p + (int64_t)(cb + q) * sc.cs + e)
                                          : ((slot_t)sc.tag << 32);
#pragma unroll
            for (int q = 0; q < kSlotBatch; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) all = all && slot_full(w[q][e], sc.tag);
            if (all) break;
            if (timeout || spin >= sc.max_spin) {
                timeout = true;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
#pragma unroll
        for (int q = 0; q < kSlotBatch; ++q) {
            if (cb + q >= c1) continue;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = slot_full(w[q][e], sc.tag) ? __uint_as_float((uint32_t)w[q][e]) : 0.f;
            acc.x += v[0]; acc.y += v[1]; acc.z += v[2]; acc.w += v[3];
        }
    }
    return acc;
}

// Stage `nrows` S rows into LDS as bf16 hi / lo pairs: rank positions
// 0..rp-1 summed from their chunk partials in tagged exchange slots, zero
// past rp and for missing rows.  Called by every thread of the block; at
// most 4 nthreads (row, float4) pairs (nrows * rp / 4).
//
// A poll is a round trip to the point where the workgroups of all XCDs
// meet, so the chunks are split over the threads rather than walked by one:
// with `items` (row, float4) pairs for the tile's rows, G = threads / items
// groups of consecutive chunks (at least 1, at most C, and no more than the
// scratch holds) are polled at once,
// task (g, item) adding group g's chunks.  The task sums meet in LDS (sHi /
// sLo serve as the scratch) and are added in group order.  The positions
// past rp are then cleared.  kNRows rows, kThreads threads; a thread polls
// kBatch chunks at a time (fewer registers for the wide tile).
template <int kNRows, int kThreads, int kBatch>
__device__ __forceinline__ void stage_s_slots(const RowSet& rs, int r0, int rows,
                                              const slot_t* __restrict__ S, int sld, int sc0,
                                              SChunks sc, int rp, uint16_t* __restrict__ sHi,
                                              uint16_t* __restrict__ sLo) {
    constexpr int nrows = kNRows, nthreads = kThreads;
    constexpr int kPer = (kNRows * LORA_MAX_RANK / 4 + kThreads - 1) / kThreads;  // items per thread
    constexpr int kCap = kNRows * kSLds / 4;      // float4 that sHi and sLo hold together
    static_assert(kNRows * LORA_MAX_RANK / 4 <= kCap, "one task per item must fit");
    const int wa = rp / 4;                        // float4 per row below rp
    const int tid = (int)threadIdx.x;
    const int items = rows * wa;
    const int G = max(1, min(sc.C, min(nthreads, kCap) / max(items, 1)));
    const int per = (sc.C + G - 1) / G;
    float4* part = reinterpret_cast<float4*>(sHi);   // G * items <= kCap float4
    bool timeout = false;
    for (int t = tid; t < G * items; t += nthreads) {
        const int g = t / items, it = t % items;
        const int row = it / wa, j = (it % wa) * 4;
        const int sr = rs.in_row[r0 + row];
        const int c0 = g * per, c1 = min(sc.C, c0 + per);
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        if (sr >= 0 && c0 < c1)
            acc = slot_range_sum<kBatch>(S + (int64_t)sr * sld + sc0 + j, sc, c0, c1, timeout);
        part[t] = acc;
    }
    if (timeout && sc.err != nullptr) atomicOr(sc.err, kErrSpin);
    __syncthreads();
    float4 sum[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int i = tid + k * nthreads;
        sum[k] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i < items) {
            sum[k] = part[i];
            for (int g = 1; g < G; ++g) {
                const float4 v = part[g * items + i];
                sum[k].x += v.x; sum[k].y += v.y; sum[k].z += v.z; sum[k].w += v.w;
            }
        }
    }
    __syncthreads();                              // the scratch is overwritten below
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int i = tid + k * nthreads;
        if (i >= nrows * wa) break;
        const int row = i / wa, j = (i % wa) * 4;
        const float v[4] = {sum[k].x, sum[k].y, sum[k].z, sum[k].w};   // zero past `items`
        uint32_t h[2], l[2];
#pragma unroll
        for (int q = 0; q < 4; q += 2) {
            const uint32_t h0 = f32_to_bf16(v[q]), h1 = f32_to_bf16(v[q + 1]);
            h[q / 2] = h0 | (h1 << 16);
            l[q / 2] = f32_to_bf16(v[q] - bf16_to_f32(h0)) |
                       (f32_to_bf16(v[q + 1] - bf16_to_f32(h1)) << 16);
        }
        *reinterpret_cast<uint2*>(sHi + row * kSLds + j) = make_uint2(h[0], h[1]);
        *reinterpret_cast<uint2*>(sLo + row * kSLds + j) = make_uint2(l[0], l[1]);
    }
    const int wz = LORA_MAX_RANK / 4 - wa;        // float4 per row past rp
    for (int i = tid; i < nrows * wz; i += nthreads) {
        const int row = i / wz, j = rp + (i % wz) * 4;
        *reinterpret_cast<uint2*>(sHi + row * kSLds + j) = make_uint2(0u, 0u);
        *reinterpret_cast<uint2*>(sLo + row * kSLds + j) = make_uint2(0u, 0u);
    }
}

// kSlots: S arrives as chunk partials in tagged exchange slots written by
// the same launch, polled until they carry its tag (stage_s_slots).
// kSteps: 32-wide rank steps the code is built for; 1 needs rp <= 32 and
// keeps half the B operands out of registers (the MoE launches, whose rank
// is known at launch, pick it; the dense launches mix ranks up to 64).
template <bool kSlots = false, int kSteps = 2>
__device__ __forceinline__ void expand_tile_bf16(const RowSet& rs, int r0, int rows,
                                                 const float* __restrict__ S, int sld, int sc0,
                                                 const uint16_t* __restrict__ B, int rp, int n0,
                                                 int n1, uint16_t* __restrict__ y, int64_t ldy_,
                                                 uint4* __restrict__ ytile,
                                                 uint16_t* __restrict__ sHi,
                                                 uint16_t* __restrict__ sLo, SChunks sc = {1, 0, 0u, nullptr, kMaxSpin}) {
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int lr = lane % 16;
    const int lq = lane / 16;
    const int nsteps = (rp + 31) / 32;
    const int nw = n0 + wave * 64;
    const int nchunks = (n1 - n0) / 8;                // valid 16-byte chunks per row
    // 0. S rows first (thread t: row t / 4, rank positions 16 (t % 4) .. +16):
    //    their hi / lo split waits only for them, while the y tile and the B
    //    operands issued after them are still arriving (loads complete in
    //    order; measured 0.1-0.5 us per launch on the dense workloads)
    const int srow = tid / 4, sqt = tid % 4;
    float4 sv_early[4];
    if constexpr (!kSlots) {
        const int sr = srow < rows ? rs.in_row[r0 + srow] : -1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = sqt * 16 + e * 4;
            sv_early[e] = ldf4_if(S + (int64_t)sr * sld + sc0 + j, sr >= 0 && j < rp, S);
        }
    }
    // 1a. y tile -> LDS: wave w moves rows 16w .. 16w+15, two rows per instruction
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = wave * 16 + 2 * i + lane / 32;
        const int pos = lane % 32;
        const int q = pos ^ (r & 15);
        const int yr = r < rows ? rs.out_row[r0 + r] : -1;
        const bool ok = yr >= 0 && q < nchunks;
        const uint16_t* src = ok ? y + (int64_t)yr * ldy_ + n0 + q * 8 : y;
        __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(ytile + (wave * 16 + 2 * i) * (kYRowBytes / 16)),
                                         16, 0, 0);
    }
    // 1b. B operands: rows nw + 16*nb + lr, 8 rank values at st*32 + lq*8
    uint4 bop[4][kSteps];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        const int n = nw + nb * 16 + lr;
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
            const int j = st * 32 + lq * 8;
            // columns clamped (those past n1 are never written back); rank
            // positions past rp meet zero S values.  The dense launches skip
            // the loads past rp (a rank <= 32 segment needs no second step:
            // 30.8 against 31.2 us for the 2048-token prefill's delta
            // kernels, no spill); the MoE expand keeps clamped loads (62.2
            // against 64.2 us with skipped ones)
            if constexpr (kSlots) {
                bop[nb][st] = ld16(B + (int64_t)min(n, n1 - 1) * rp + min(j, rp - 8));
            } else {
                bop[nb][st] = make_uint4(0, 0, 0, 0);
                if (j < rp) bop[nb][st] = ld16(B + (int64_t)min(n, n1 - 1) * rp + j);
            }
        }
    }
    if constexpr (kSlots) {
        stage_s_slots<64, kTileThreads, 4>(rs, r0, rows, reinterpret_cast<const slot_t*>(S),
                                           sld, sc0, sc, rp, sHi, sLo);
    } else {
        // 1c. S rows (loaded at step 0) split into hi / lo in LDS; positions
        //     past rp are written as zeros, so the MFMA operand reads below
        //     need no mask
        {
            const int row = srow, qt = sqt;
            float4 sv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) sv[e] = sv_early[e];
            uint32_t h[8], l[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float v[4] = {sv[e].x, sv[e].y, sv[e].z, sv[e].w};
#pragma unroll
                for (int q = 0; q < 4; q += 2) {
                    const uint32_t h0 = f32_to_bf16(v[q]), h1 = f32_to_bf16(v[q + 1]);
                    const uint32_t l0 = f32_to_bf16(v[q] - bf16_to_f32(h0));
                    const uint32_t l1 = f32_to_bf16(v[q + 1] - bf16_to_f32(h1));
                    h[e * 2 + q / 2] = h0 | (h1 << 16);
                    l[e * 2 + q / 2] = l0 | (l1 << 16);
                }
            }
            uint4* hp = reinterpret_cast<uint4*>(sHi + row * kSLds + qt * 16);
            uint4* lp = reinterpret_cast<uint4*>(sLo + row * kSLds + qt * 16);
            hp[0] = make_uint4(h[0], h[1], h[2], h[3]);
            hp[1] = make_uint4(h[4], h[5], h[6], h[7]);
            lp[0] = make_uint4(l[0], l[1], l[2], l[3]);
            lp[1] = make_uint4(l[4], l[5], l[6], l[7]);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);    // direct-to-LDS loads are tracked by vmcnt only
    __syncthreads();
    // 2. MFMA; each 16 x 16 result is added into the LDS tile
    if (nw < n1) {
        // S operands of the next row group are read while this one's MFMAs run
        uint4 shi[kSteps], slo[kSteps], nhi[kSteps], nlo[kSteps];
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
            shi[st] = ld16(sHi + lr * kSLds + st * 32 + lq * 8);
            slo[st] = ld16(sLo + lr * kSLds + st * 32 + lq * 8);
        }
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            if (rg * 16 >= rows) break;
            if (rg < 3) {
#pragma unroll
                for (int st = 0; st < kSteps; ++st) {
                    nhi[st] = ld16(sHi + ((rg + 1) * 16 + lr) * kSLds + st * 32 + lq * 8);
                    nlo[st] = ld16(sLo + ((rg + 1) * 16 + lr) * kSLds + st * 32 + lq * 8);
                }
            }
            const int r = rg * 16 + lr;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < kSteps; ++st) {
                    if (st < nsteps) {
                        acc = mfma_bf16(bop[nb][st], shi[st], acc);
                        acc = mfma_bf16(bop[nb][st], slo[st], acc);
                    }
                }
                // acc[e]: column c + e, row r, where c = wave*64 + nb*16 + lq*4
                const int c = wave * 64 + nb * 16 + lq * 4;
                uint2* yp = reinterpret_cast<uint2*>(ytile + ypos(r, c / 8)) + ((c / 4) & 1);
                const uint2 old = *yp;
                uint2 nv;
                nv.x = f32_to_bf16(__uint_as_float(old.x << 16) + acc[0]) |
                       (f32_to_bf16(__uint_as_float(old.x & 0xffff0000u) + acc[1]) << 16);
                nv.y = f32_to_bf16(__uint_as_float(old.y << 16) + acc[2]) |
                       (f32_to_bf16(__uint_as_float(old.y & 0xffff0000u) + acc[3]) << 16);
                *yp = nv;
            }
#pragma unroll
            for (int st = 0; st < kSteps; ++st) {
                shi[st] = nhi[st];
                slo[st] = nlo[st];
            }
        }
    }
    __syncthreads();
    // 3. row-major write-back: thread t covers rows t/32 + 8i, chunk t % 32
    //    (non-temporal stores: 31.2 against 31.7 us for the 2048-token
    //    prefill's delta kernels, same box; no change on the stacked layers,
    //    slightly slower on the MoE's wide tiles, which keep ordinary stores)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = tid / 32 + 8 * i;
        const int q = tid % 32;
        const int yr = r < rows ? rs.out_row[r0 + r] : -1;
        if (yr >= 0 && q < nchunks)
            st_nt16(y + (int64_t)yr * ldy_ + n0 + q * 8, ytile[ypos(r, q)]);
    }
    __syncthreads();     // the LDS tile is reused by the next tile
}

// All rows of rs over columns [n_begin, n_end), one 64 x 256 tile at a time.
template <bool kSlots = false, int kSteps = 2>
__device__ __forceinline__ void expand_rows_bf16(const RowSet& rs, const float* __restrict__ S,
                                                 int sld, int sc0,
                                                 const uint16_t* __restrict__ B, int rp,
                                                 int n_begin, int n_end,
                                                 uint16_t* __restrict__ y, int64_t ldy_,
                                                 uint4* __restrict__ lds, SChunks sc = {1, 0, 0u, nullptr, kMaxSpin}) {
    for (int r0 = 0; r0 < rs.n; r0 += 64) {
        const int rows = min(64, rs.n - r0);
        for (int n0 = n_begin; n0 < n_end; n0 += kNTile)
            expand_tile_bf16<kSlots, kSteps>(rs, r0, rows, S, sld, sc0, B, rp, n0, min(n0 + kNTile, n_end),
                                   y, ldy_, lds,
                                   reinterpret_cast<uint16_t*>(lds + 64 * kYRowBytes / 16),
                                   reinterpret_cast<uint16_t*>(lds + 64 * kYRowBytes / 16) +
                                       64 * kSLds,
                                   sc);
    }
}

// ---------------------------------------------------------------------------
// Pipelined expand over a run of 64-row x 128-column tiles of one row tile:
// S is staged once for the whole run, and while tile k's products are folded
// into LDS and written back, tile k+1's y values and B operands are already
// on their way into registers, so a workgroup's loads, matrix work and stores
// overlap instead of running as three phases one after another.  The y tiles
// alternate between two LDS buffers (a buffer is refilled two tiles after its
// write-back read it out, with two barriers in between).
//   thread t: y rows t/16 + 16 i (i = 0..3), 16-byte chunk t % 16 of the tile
//   wave w:   columns 32w .. 32w+31 of the tile (two 16-column blocks)
// y and B go through buffer resources: y based at the run's first column
// (row byte offsets below 2^31), B at the adapter's block of nb_rows x rp
// values (under 2 GiB); the launcher checks both bounds.
// ---------------------------------------------------------------------------
constexpr int kPCols = 128;
constexpr int kPRowChunks = kPCols / 8;                              // 16
constexpr int kPipeLds = 2 * 64 * kPCols * 2 + 2 * 64 * kSLds * 2;   // bytes

__device__ __forceinline__ int ppos(int r, int q) { return r * kPRowChunks + (q ^ (r & 15)); }

// y values are read once and written back once: loaded non-temporal (the
// cache policy's nt bit), as they are stored, they stay out of the way of
// the B rows that later tiles of the same adapter read again (2048-token
// prefill delta kernels 26.4 against 28.6 us; stacked QKV 23.3 against
// 24.2; gate/up 37.1 against 39.0.  Non-temporal loads with plain stores:
// 29.9, 24.1 and 39.2 us)
__device__ __forceinline__ uint4 buf_ld16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4_vt v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void expand_pipe_bf16(const RowSet& rs, int rows,
                                                 const float* __restrict__ S, int sld, int sc0,
                                                 const uint16_t* __restrict__ B, int nb_rows,
                                                 int rp, int n_begin, int n_end,
                                                 uint16_t* __restrict__ y, int64_t ldy_,
                                                 uint4* __restrict__ lds) {
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int lr = lane % 16;
    const int lq = lane / 16;
    const int nsteps = (rp + 31) / 32;
    uint4* ybuf = lds;                                           // [2][64 * kPRowChunks]
    uint16_t* sHi = reinterpret_cast<uint16_t*>(lds + 2 * 64 * kPRowChunks);
    uint16_t* sLo = sHi + 64 * kSLds;
    // S rows first (thread t: row t / 4, rank positions 16 (t % 4) .. +16)
    const int srow = tid / 4, sqt = tid % 4;
    float4 sv[4];
    {
        const int sr = srow < rows ? rs.in_row[srow] : -1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = sqt * 16 + e * 4;
            sv[e] = ldf4_if(S + (int64_t)sr * sld + sc0 + j, sr >= 0 && j < rp, S);
        }
    }
    const int wq = tid % 16;
    const __amdgpu_buffer_rsrc_t yr = buf_rsrc(y + n_begin, 0x7fffffffu);
    const __amdgpu_buffer_rsrc_t br = buf_rsrc(B, (uint32_t)nb_rows * (uint32_t)rp * 2u);
    uint32_t yoff[4];                                             // row byte offsets, kBufOff if none
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = tid / 16 + 16 * i;
        const int row = r < rows ? rs.out_row[r] : -1;
        yoff[i] = row >= 0 ? (uint32_t)((int64_t)row * ldy_ * 2) : kBufOff;
    }
    // the loads of the tile at column n0 (none past n_end)
    auto load_y = [&](int n0, uint4 (&yv)[4]) {
        const int nch = (min(n0 + kPCols, n_end) - n0) / 8;
        const uint32_t c = (uint32_t)(n0 - n_begin) * 2u + (uint32_t)wq * 16u;
#pragma unroll
        for (int i = 0; i < 4; ++i) yv[i] = buf_ld16_nt(yr, wq < nch ? yoff[i] + c : kBufOff);
    };
    auto load_b = [&](int n0, uint4 (&bv)[2][2]) {
        const int n1 = min(n0 + kPCols, n_end);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int n = min(n0 + wave * 32 + nb * 16 + lr, n1 - 1);
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const int j = st * 32 + lq * 8;
                // rank positions past rp read zeros (their S values are zero
                // too, and 0 * NaN would not be)
                bv[nb][st] = buf_ld16(br, (j < rp && n0 < n_end) ? (uint32_t)(n * rp + j) * 2u
                                                                  : kBufOff);
            }
        }
    };
    uint4 yv[4], bA[2][2], bB[2][2];
    load_y(n_begin, yv);
    load_b(n_begin, bA);
    // S split into bf16 hi / lo in LDS, zero past rp
    {
        uint32_t h[8], l[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float v[4] = {sv[e].x, sv[e].y, sv[e].z, sv[e].w};
#pragma unroll
            for (int q = 0; q < 4; q += 2) {
                const uint32_t h0 = f32_to_bf16(v[q]), h1 = f32_to_bf16(v[q + 1]);
                h[e * 2 + q / 2] = h0 | (h1 << 16);
                l[e * 2 + q / 2] = f32_to_bf16(v[q] - bf16_to_f32(h0)) |
                                   (f32_to_bf16(v[q + 1] - bf16_to_f32(h1)) << 16);
            }
        }
        uint4* hp = reinterpret_cast<uint4*>(sHi + srow * kSLds + sqt * 16);
        uint4* lp = reinterpret_cast<uint4*>(sLo + srow * kSLds + sqt * 16);
        hp[0] = make_uint4(h[0], h[1], h[2], h[3]);
        hp[1] = make_uint4(h[4], h[5], h[6], h[7]);
        lp[0] = make_uint4(l[0], l[1], l[2], l[3]);
        lp[1] = make_uint4(l[4], l[5], l[6], l[7]);
    }
    // one tile: its y values (in yv) into LDS buffer `buf`, the next tile's
    // loads issued (y into the freed yv, B into bn; past the run they read
    // nothing), products folded in with bc, write-back
    auto tile = [&](int n0, int buf, const uint4 (&bc)[2][2], uint4 (&bn)[2][2]) {
        const int n1 = min(n0 + kPCols, n_end);
        const int nch = (n1 - n0) / 8;
        uint4* yt = ybuf + buf * (64 * kPRowChunks);
#pragma unroll
        for (int i = 0; i < 4; ++i) yt[ppos(tid / 16 + 16 * i, wq)] = yv[i];
        load_y(n0 + kPCols, yv);
        load_b(n0 + kPCols, bn);
        __syncthreads();
        const int cw = wave * 32;
        if (n0 + cw < n1) {
            uint4 shi[2], slo[2], nhi[2], nlo[2];
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                shi[st] = ld16(sHi + lr * kSLds + st * 32 + lq * 8);
                slo[st] = ld16(sLo + lr * kSLds + st * 32 + lq * 8);
            }
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                if (rg * 16 >= rows) break;
                if (rg < 3) {
#pragma unroll
                    for (int st = 0; st < 2; ++st) {
                        nhi[st] = ld16(sHi + ((rg + 1) * 16 + lr) * kSLds + st * 32 + lq * 8);
                        nlo[st] = ld16(sLo + ((rg + 1) * 16 + lr) * kSLds + st * 32 + lq * 8);
                    }
                }
                const int r = rg * 16 + lr;
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int st = 0; st < 2; ++st) {
                        if (st < nsteps) {
                            acc = mfma_bf16(bc[nb][st], shi[st], acc);
                            acc = mfma_bf16(bc[nb][st], slo[st], acc);
                        }
                    }
                    // acc[e]: tile column c + e, row r
                    const int c = cw + nb * 16 + lq * 4;
                    uint2* yp = reinterpret_cast<uint2*>(yt + ppos(r, c / 8)) + ((c / 4) & 1);
                    const uint2 old = *yp;
                    uint2 nv;
                    nv.x = f32_to_bf16(__uint_as_float(old.x << 16) + acc[0]) |
                           (f32_to_bf16(__uint_as_float(old.x & 0xffff0000u) + acc[1]) << 16);
                    nv.y = f32_to_bf16(__uint_as_float(old.y << 16) + acc[2]) |
                           (f32_to_bf16(__uint_as_float(old.y & 0xffff0000u) + acc[3]) << 16);
                    *yp = nv;
                }
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    shi[st] = nhi[st];
                    slo[st] = nlo[st];
                }
            }
        }
        __syncthreads();
        const uint32_t c = (uint32_t)(n0 - n_begin) * 2u + (uint32_t)wq * 16u;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            buf_st16_nt(yt[ppos(tid / 16 + 16 * i, wq)], yr, wq < nch ? yoff[i] + c : kBufOff);
    };
    // two tiles per trip so the B register sets alternate without copies
    for (int n0 = n_begin;;) {
        tile(n0, 0, bA, bB);
        n0 += kPCols;
        if (n0 >= n_end) break;
        tile(n0, 1, bB, bA);
        n0 += kPCols;
        if (n0 >= n_end) break;
    }
}

// ---------------------------------------------------------------------------
// plain vector-ALU versions (any storage type); used for fp32 storage
// ---------------------------------------------------------------------------
// Wide expand tile for sparse row blocks (MoE): up to 32 rows (two groups of
// 16) x 1024 columns, 512 threads.  Wave w owns columns n0 + 128w .. +128 as
// 8 blocks of 16.  The same three phases as the 64 x 256 tile (y tile
// straight into LDS, MFMA results folded into it, row-major write-back), but
// a unit with few rows carries four times the columns, so an MoE block of
// about 16 real rows needs a quarter of the workgroups; a block of 17-32
// rows is one pass (its y rows, S rows and B operands loaded once).
// ---------------------------------------------------------------------------
constexpr int kWideThreads = 512;
constexpr int kWideCols = 1024;
constexpr int kWideRows = 32;                                       // rows per pass (2 groups of 16)
constexpr int kWideRowChunks = kWideCols / 8;                       // 128 chunks of 16 bytes
constexpr int kWideLds = kWideRows * kWideCols * 2 + 2 * kWideRows * kSLds * 2;   // bytes

__device__ __forceinline__ int wpos(int r, int q) { return r * kWideRowChunks + (q ^ r); }

template <int kSteps>
__device__ __forceinline__ void expand_wide_bf16(const RowSet& rs, int r0, int rows,
                                                 const slot_t* __restrict__ S, int sld, int sc0,
                                                 const uint16_t* __restrict__ B, int rp, int n0,
                                                 int n1, uint16_t* __restrict__ y, int64_t ldy_,
                                                 uint4* __restrict__ ytile,
                                                 uint16_t* __restrict__ sHi,
                                                 uint16_t* __restrict__ sLo, SChunks sc = {1, 0, 0u, nullptr, kMaxSpin}) {
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;                 // 0..7
    const int lr = lane % 16;
    const int lq = lane / 16;
    const int nsteps = kSteps == 1 ? 1 : (rp + 31) / 32;
    const int nw = n0 + wave * 128;
    const int nchunks = (n1 - n0) / 8;            // valid 16-byte chunks per row
    // 1a. y rows -> LDS: one wave instruction per half row (1 KB), rows past
    //     `rows` skipped; position p of row r holds chunk p ^ r
    constexpr int kHalves = kWideRows * 2 / (kWideThreads / kWave);   // per wave
#pragma unroll
    for (int i = 0; i < kHalves; ++i) {
        const int k = wave * kHalves + i;
        const int r = k / 2, h = k % 2;
        if (r >= rows) break;                     // wave-uniform
        const int q = (h * 64 + lane) ^ r;
        const int yr = rs.out_row[r0 + r];
        const bool ok = yr >= 0 && q < nchunks;
        const uint16_t* src = ok ? y + (int64_t)yr * ldy_ + n0 + q * 8 : y;
        __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(ytile + r * kWideRowChunks + h * 64), 16, 0,
                                         0);
    }
    // 1b. B operands: rows nw + 16 nb + lr (clamped; see expand_tile_bf16)
    uint4 bop[8][kSteps];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
        const int n = min(nw + nb * 16 + lr, n1 - 1);
        bop[nb][0] = ld16(B + (int64_t)n * rp + min(lq * 8, rp - 8));
        if constexpr (kSteps > 1) bop[nb][1] = make_uint4(0, 0, 0, 0);
    }
    if constexpr (kSteps > 1) {
        if (nsteps > 1) {
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const int n = min(nw + nb * 16 + lr, n1 - 1);
                bop[nb][1] = ld16(B + (int64_t)n * rp + min(32 + lq * 8, rp - 8));
            }
        }
    }
    // 1c. S rows summed from the shrink part's tagged slots
    stage_s_slots<kWideRows, kWideThreads, 2>(rs, r0, rows, S, sld, sc0, sc, rp, sHi, sLo);
    __builtin_amdgcn_s_waitcnt(0);    // direct-to-LDS loads are tracked by vmcnt only
    __syncthreads();
    // 2. MFMA, one 16-row group after the other; each 16 x 16 result is
    //    added into the tile
#pragma unroll 1
    for (int rg = 0; rg < kWideRows / 16; ++rg) {
        if (rg * 16 >= rows || nw >= n1) break;
        const int row = rg * 16 + lr;
        uint4 shi[kSteps], slo[kSteps];
        shi[0] = ld16(sHi + row * kSLds + lq * 8);
        slo[0] = ld16(sLo + row * kSLds + lq * 8);
        if constexpr (kSteps > 1) {
            shi[1] = slo[1] = make_uint4(0, 0, 0, 0);
            if (nsteps > 1) {
                shi[1] = ld16(sHi + row * kSLds + 32 + lq * 8);
                slo[1] = ld16(sLo + row * kSLds + 32 + lq * 8);
            }
        }
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
            // acc[e]: column c + e of row `row`, where c = 128 wave + 16 nb + 4 lq
            const int c = wave * 128 + nb * 16 + lq * 4;
            uint2* yp = reinterpret_cast<uint2*>(ytile + wpos(row, c / 8)) + ((c / 4) & 1);
            const uint2 old = *yp;
            f32x4_t acc = {__uint_as_float(old.x << 16), __uint_as_float(old.x & 0xffff0000u),
                           __uint_as_float(old.y << 16), __uint_as_float(old.y & 0xffff0000u)};
            acc = mfma_bf16(bop[nb][0], shi[0], acc);
            acc = mfma_bf16(bop[nb][0], slo[0], acc);
            if constexpr (kSteps > 1) {
                if (nsteps > 1) {
                    acc = mfma_bf16(bop[nb][1], shi[1], acc);
                    acc = mfma_bf16(bop[nb][1], slo[1], acc);
                }
            }
            uint2 nv;
            nv.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
            nv.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
            *yp = nv;
        }
    }
    __syncthreads();
    // 3. row-major write-back: a wave instruction stores 64 chunks of one row
#pragma unroll 2
    for (int i = 0; i < kWideRows * kWideRowChunks / kWideThreads; ++i) {
        const int idx = i * kWideThreads + tid;
        const int r = idx / kWideRowChunks, q = idx % kWideRowChunks;
        const int yr = r < rows ? rs.out_row[r0 + r] : -1;
        if (yr >= 0 && q < nchunks)
            *reinterpret_cast<uint4*>(y + (int64_t)yr * ldy_ + n0 + q * 8) = ytile[wpos(r, q)];
    }
    __syncthreads();     // the LDS tile is reused by the next row group
}

// All rows of rs (kWideRows at a time) over columns [n0, min(n0 + 1024, n_end)).
template <int kSteps>
__device__ __forceinline__ void expand_rows_wide(const RowSet& rs, const slot_t* __restrict__ S,
                                                 int sld, int sc0,
                                                 const uint16_t* __restrict__ B, int rp, int n0,
                                                 int n1, uint16_t* __restrict__ y, int64_t ldy_,
                                                 uint4* __restrict__ lds, SChunks sc = {1, 0, 0u, nullptr, kMaxSpin}) {
    uint16_t* sHi = reinterpret_cast<uint16_t*>(lds + kWideRows * kWideRowChunks);
    uint16_t* sLo = sHi + kWideRows * kSLds;
    for (int r0 = 0; r0 < rs.n; r0 += kWideRows)
        expand_wide_bf16<kSteps>(rs, r0, min(kWideRows, rs.n - r0), S, sld, sc0, B, rp, n0, n1, y,
                                 ldy_, lds, sHi, sLo, sc);
}

// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void shrink_tile_simple(const RowSet& rs, const T* __restrict__ x,
                                                   int64_t ldx, const T* __restrict__ A, int K,
                                                   int n_sl, int rp, int r_max, int k0, int k1,
                                                   float* __restrict__ P, int pld) {
    const int cols = n_sl * r_max;
    const int total = rs.n * cols;
    for (int e = threadIdx.x; e < total; e += kTileThreads) {
        const int i = e / cols, col = e % cols;
        const int orow = rs.out_row[i];
        if (orow < 0) continue;
        const int sl = col / r_max, j = col % r_max;
        float acc = 0.f;
        const int xr = rs.in_row[i];
        if (j < rp && xr >= 0) {
            const T* xp = x + (int64_t)xr * ldx;
            const T* ap = A + (int64_t)(sl * rp + j) * K;
            for (int k = k0; k < k1; ++k) acc += Io<T>::ld(xp + k) * Io<T>::ld(ap + k);
        }
        P[(int64_t)orow * pld + col] = acc;
    }
}

template <typename T>
__device__ __forceinline__ void expand_tile_simple(const RowSet& rs, const float* __restrict__ S,
                                                   int sld, int sc0, const T* __restrict__ B,
                                                   int rp, int n0, int n1, T* __restrict__ y,
                                                   int64_t ldy_) {
    const int w = n1 - n0;
    const int total = rs.n * w;
    for (int e = threadIdx.x; e < total; e += kTileThreads) {
        const int i = e / w, n = n0 + e % w;
        const int yr = rs.out_row[i], sr = rs.in_row[i];
        if (yr < 0 || sr < 0) continue;
        const float* sp = S + (int64_t)sr * sld + sc0;
        const T* bp = B + (int64_t)n * rp;
        float acc = 0.f;
        for (int j = 0; j < rp; ++j) acc += sp[j] * Io<T>::ld(bp + j);
        T* yp = y + (int64_t)yr * ldy_ + n;
        Io<T>::st(yp, Io<T>::ld(yp) + acc);
    }
}

}  // namespace mlora
