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

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_bf16(const uint4& a, const uint4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

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

// Workgroup ids are handed to the 8 XCDs round robin; renumber them so that
// consecutive work units (which share input rows) run on the same XCD and
// meet in its L2.  grid must be a multiple of 8.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_unit(int b, int grid) {
    return (b % kXcds) * (grid / kXcds) + b / kXcds;
}
constexpr int kTileWaves = kTileThreads / kWave;
constexpr int kMaxRowTile = 256;

// Rows of one unit, staged in LDS by the unit decoder.
struct RowSet {
    int n;                   // rows in this unit (<= RT)
    int RT;                  // row tile (multiple of 16, <= kMaxRowTile)
    const int* in_row;       // LDS [RT]: input row index, -1 = padding row
    const int* out_row;      // LDS [RT]: output row index, -1 = padding row
};

// ---------------------------------------------------------------------------
// shrink unit: P[out_row][cg*64 + c] = sum_{k0 <= k < k1} x[in_row, k] A[row(c), k]
// for the 64 S columns of column group cg (k1 - k0 <= 512).
//   S column block cbg (16 columns) = slice sl = cbg / (r_max/16), block
//   jj = cbg % (r_max/16); it is active when jj < rp/16 and then reads
//   adapter rows sl*rp + jj*16 .. +16; inactive blocks store zeros (rank
//   padding).
// The group's A chunk (64 rows x 512 K, 64 KB) is staged in LDS with every
// load issued at once; row r's 16-byte chunk q lives at chunk q ^ (r & 15),
// so the MFMA operand reads of 16 consecutive rows hit 64 distinct banks.
// Each wave keeps its 16 x rows for the whole chunk in registers (16 loads
// in flight per lane), so a unit costs one memory round trip.
// ---------------------------------------------------------------------------
constexpr int kShrinkK = 512;
constexpr int kGroupCols = 64;
constexpr int kShrinkLds = kGroupCols * kShrinkK * 2;   // bytes

__device__ __forceinline__ int swz(int r, int q) { return r * (kShrinkK / 8) + (q ^ (r & 15)); }

__device__ __forceinline__ void shrink_group_bf16(const RowSet& rs, const uint16_t* __restrict__ x,
                                                  int64_t ldx, const uint16_t* __restrict__ A,
                                                  int K, int n_sl, int rp, int r_max, int cg,
                                                  int k0, int k1, float* __restrict__ P, int pld,
                                                  uint4* __restrict__ sA) {
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int bps = r_max / 16;
    const int nbr = rp / 16;
    const int lr = lane % 16;
    const int lq = lane / 16;                 // 16-byte chunk within a 32-wide K step
    const uint4 z = make_uint4(0, 0, 0, 0);
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
    // x rows of this wave's first row group: loads issued together with the
    // A chunk's, before anything waits
    const int rg0 = wave;
    uint4 xv[kShrinkK / 32];
    auto load_x = [&](int rg) {
        const int i = rg * 16 + lr;
        const int xr = (i < rs.n) ? rs.in_row[i] : -1;
        const uint16_t* xp = x + (int64_t)(xr < 0 ? 0 : xr) * ldx + lq * 8;
#pragma unroll
        for (int kk = 0; kk < kShrinkK / 32; ++kk) {
            const int k = k0 + kk * 32;
            xv[kk] = ld16_if(xp + k, any && xr >= 0 && k + lq * 8 < k1, x);
        }
    };
    // 1. A chunk -> registers -> LDS.  Thread t covers chunk (t % 64) of rows
    //    t / 64 + 4 i, i = 0..15 (a wavefront reads one 1 KB row segment).
    if (any) {
        uint4 av[16];
        const int q = tid % 64;
        const int k = k0 + q * 8;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = i * 4 + tid / 64;
            const int cb = r / 16;
            av[i] = ld16_if(A + (int64_t)(arow[cb] + r % 16) * K + k, act[cb] && k < k1, A);
        }
        if (rg0 * 16 < rs.n) load_x(rg0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = i * 4 + tid / 64;
            sA[swz(r, q)] = av[i];
        }
    }
    __syncthreads();
    for (int rg = rg0; rg * 16 < rs.n; rg += kTileWaves) {
        f32x4_t acc[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (any) {
            if (rg != rg0) load_x(rg);
#pragma unroll
            for (int kk = 0; kk < kShrinkK / 32; ++kk) {
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    if (act[cb]) {
                        const uint4 b = sA[swz(cb * 16 + lr, kk * 4 + lq)];
                        acc[cb] = mfma_bf16(xv[kk], b, acc[cb]);
                    }
                }
            }
        }
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const int row = rg * 16 + lq * 4 + qq;
            const int orow = (row < rs.n) ? rs.out_row[row] : -1;
            if (orow < 0) continue;
            float* pp = P + (int64_t)orow * pld + cg * kGroupCols + lr;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
                if (cg * kGroupCols + cb * 16 < pld) pp[cb * 16] = acc[cb][qq];
        }
    }
}

// ---------------------------------------------------------------------------
// expand: y[out_row, n] += sum_{j < rp} S[srow, sc0 + j] * B[n, j] for
// n in [n_begin, n_end), walked in 256-column tiles; in a tile wave w owns
// columns n0 + 64w .. +64.  S rows come from rs.in_row (index into S), y rows
// from rs.out_row.  Per block of 64 rows, S is staged once in LDS as bf16 hi /
// lo parts; per column tile every wave has its B operands and all of its y
// values in flight before the MFMAs.
// ---------------------------------------------------------------------------
constexpr int kSLds = LORA_MAX_RANK + 8;       // bf16 row stride of the staged S
constexpr int kExpandLds = 2 * 64 * kSLds * 2;  // bytes (hi and lo)

// Column tile operands of one wave: B rows nw + 16*nb + lr (2 K steps of 32)
// and the y values (4 row groups x 4 column blocks, 4 values each).
struct ExpandOps {
    uint4 bop[4][2];
    uint2 yv[4][4];
};

__device__ __forceinline__ void expand_load(ExpandOps& o, const uint16_t* __restrict__ B, int rp,
                                            int nsteps, int nw, int n1, const int* yrow,
                                            const uint16_t* __restrict__ y, int64_t ldy_) {
    const int lane = lane_id();
    const int lr = lane % 16;
    const int lk = (lane / 16) * 8;
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        const int n = nw + nb * 16 + lr;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const int j = st * 32 + lk;
            o.bop[nb][st] = ld16_if(B + (int64_t)n * rp + j, st < nsteps && n < n1 && j < rp, B);
        }
    }
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int n = nw + nb * 16 + (lane / 16) * 4;
            o.yv[rg][nb] = ld8_if(y + (int64_t)yrow[rg] * ldy_ + n, yrow[rg] >= 0 && n < n1, y);
        }
    }
}

__device__ __forceinline__ void expand_compute(const ExpandOps& o, int rows, int nsteps, int rp,
                                               int nw, int n1, const int* yrow,
                                               const uint16_t* __restrict__ sHi,
                                               const uint16_t* __restrict__ sLo,
                                               uint16_t* __restrict__ y, int64_t ldy_) {
    const int lane = lane_id();
    const int lr = lane % 16;
    const int lk = (lane / 16) * 8;
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
        if (rg * 16 >= rows) break;
        uint4 shi[2], slo[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const int j = st * 32 + lk;
            const bool jin = st < nsteps && j < rp;
            shi[st] = ld16_if(sHi + (rg * 16 + lr) * kSLds + j, jin, sHi);
            slo[st] = ld16_if(sLo + (rg * 16 + lr) * kSLds + j, jin, sLo);
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                if (st < nsteps) {
                    acc = mfma_bf16(o.bop[nb][st], shi[st], acc);
                    acc = mfma_bf16(o.bop[nb][st], slo[st], acc);
                }
            }
            // acc[q] = delta for column nw + 16*nb + 4*(lane/16) + q, token row lr
            const int n = nw + nb * 16 + (lane / 16) * 4;
            if (yrow[rg] >= 0 && n < n1) {
                const uint2 old = o.yv[rg][nb];
                uint2 nv;
                nv.x = f32_to_bf16(__uint_as_float(old.x << 16) + acc[0]) |
                       (f32_to_bf16(__uint_as_float(old.x & 0xffff0000u) + acc[1]) << 16);
                nv.y = f32_to_bf16(__uint_as_float(old.y << 16) + acc[2]) |
                       (f32_to_bf16(__uint_as_float(old.y & 0xffff0000u) + acc[3]) << 16);
                *reinterpret_cast<uint2*>(y + (int64_t)yrow[rg] * ldy_ + n) = nv;
            }
        }
    }
}

// Per block of 64 rows: the first column tile's B / y loads and the S rows are
// issued together; S is converted into LDS; then column tile k is computed
// while the loads of tile k + 1 are already in flight.
__device__ __forceinline__ void expand_rows_bf16(const RowSet& rs, const float* __restrict__ S,
                                                 int sld, int sc0,
                                                 const uint16_t* __restrict__ B, int rp,
                                                 int n_begin, int n_end,
                                                 uint16_t* __restrict__ y, int64_t ldy_,
                                                 uint16_t* __restrict__ sHi,
                                                 uint16_t* __restrict__ sLo) {
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int lr = lane % 16;
    const int nsteps = (rp + 31) / 32;
    for (int r0 = 0; r0 < rs.n; r0 += 64) {
        const int rows = min(64, rs.n - r0);
        int yrow[4];
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) yrow[rg] = (rg * 16 + lr < rows) ? rs.out_row[r0 + rg * 16 + lr] : -1;
        ExpandOps cur, nxt;
        expand_load(cur, B, rp, nsteps, n_begin + wave * 64, min(n_begin + kNTile, n_end), yrow, y, ldy_);
        // S rows -> LDS (hi / lo): thread t covers row t / 4, quarter t % 4
        {
            const int row = threadIdx.x / 4, qt = threadIdx.x % 4;
            const int sr = row < rows ? rs.in_row[r0 + row] : -1;
            const int per = rp / 4;                       // 4..16, a multiple of 4
            float4 sv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sv[e] = ldf4_if(S + (int64_t)sr * sld + sc0 + qt * per + e * 4, sr >= 0 && e * 4 < per, S);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (e * 4 >= per) break;
                const float v[4] = {sv[e].x, sv[e].y, sv[e].z, sv[e].w};
                uint32_t h[4], l[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    h[q] = f32_to_bf16(v[q]);
                    l[q] = f32_to_bf16(v[q] - bf16_to_f32(h[q]));
                }
                const int j = qt * per + e * 4;
                *reinterpret_cast<uint2*>(sHi + row * kSLds + j) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
                *reinterpret_cast<uint2*>(sLo + row * kSLds + j) = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
            }
        }
        __syncthreads();
        for (int n0 = n_begin; n0 < n_end; n0 += kNTile) {
            const int n1 = min(n0 + kNTile, n_end);
            const int nn = n0 + kNTile;
            if (nn < n_end)
                expand_load(nxt, B, rp, nsteps, nn + wave * 64, min(nn + kNTile, n_end), yrow, y, ldy_);
            const int nw = n0 + wave * 64;
            if (nw < n1) expand_compute(cur, rows, nsteps, rp, nw, n1, yrow, sHi, sLo, y, ldy_);
            cur = nxt;
        }
        __syncthreads();     // S of the next row block overwrites sHi / sLo
    }
}

// ---------------------------------------------------------------------------
// plain vector-ALU versions (any storage type); used for fp32 storage
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
