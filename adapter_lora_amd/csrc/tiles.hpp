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
// for the 64 S columns of column group cg and up to 64 rows (k1 - k0 <= 512).
//   S column block cbg (16 columns) = slice sl = cbg / (r_max/16), block
//   jj = cbg % (r_max/16); it is active when jj < rp/16 and then reads
//   adapter rows sl*rp + jj*16 .. +16; inactive blocks store zeros (rank
//   padding).
// Both operand chunks (64 x rows and 64 A rows, 512 K values each: 2 x 64 KB)
// are loaded row-major — a wavefront reads one contiguous 1 KB row segment
// per instruction — with all 32 loads of a thread in flight at once, and
// staged in LDS; row r's 16-byte chunk q lives at chunk q ^ (r & 15), so the
// MFMA operand reads of 16 consecutive rows hit 64 distinct banks.
// ---------------------------------------------------------------------------
constexpr int kShrinkK = 512;
constexpr int kGroupCols = 64;
constexpr int kShrinkLds = 2 * kGroupCols * kShrinkK * 2;   // bytes: x chunk + A chunk

__device__ __forceinline__ int swz(int r, int q) { return r * (kShrinkK / 8) + (q ^ (r & 15)); }

__device__ __forceinline__ void shrink_group_bf16(const RowSet& rs, int r0,
                                                  const uint16_t* __restrict__ x, int64_t ldx,
                                                  const uint16_t* __restrict__ A, int K, int n_sl,
                                                  int rp, int r_max, int cg, int k0, int k1,
                                                  float* __restrict__ P, int pld,
                                                  uint4* __restrict__ sX, uint4* __restrict__ sA) {
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int bps = r_max / 16;
    const int nbr = rp / 16;
    const int lr = lane % 16;
    const int lq = lane / 16;                 // 16-byte chunk within a 32-wide K step
    const int rows = min(64, rs.n - r0);
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
    if (any) {
        // thread t covers chunk (t % 64) of rows t / 64 + 4 i, i = 0..15
        const int q = tid % 64;
        const int k = k0 + q * 8;
        uint4 av[16], xv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = i * 4 + tid / 64;
            const int cb = r / 16;
            av[i] = ld16_if(A + (int64_t)(arow[cb] + r % 16) * K + k, act[cb] && k < k1, A);
            const int xr = r < rows ? rs.in_row[r0 + r] : -1;
            xv[i] = ld16_if(x + (int64_t)xr * ldx + k, xr >= 0 && k < k1, x);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = i * 4 + tid / 64;
            sA[swz(r, q)] = av[i];
            sX[swz(r, q)] = xv[i];
        }
    }
    __syncthreads();
    // wave w: rows 16w .. 16w+15, the group's 4 column blocks
    const int rg = wave;
    f32x4_t acc[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (any && rg * 16 < rows) {
#pragma unroll
        for (int kk = 0; kk < kShrinkK / 32; ++kk) {
            const uint4 a = sX[swz(rg * 16 + lr, kk * 4 + lq)];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                if (act[cb]) {
                    const uint4 b = sA[swz(cb * 16 + lr, kk * 4 + lq)];
                    acc[cb] = mfma_bf16(a, b, acc[cb]);
                }
            }
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
    __syncthreads();     // sX / sA are reused by the next row block
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
constexpr int kYRowBytes = kNTile * 2;                       // 512
constexpr int kSLds = LORA_MAX_RANK + 8;                     // bf16 row stride of staged S
constexpr int kExpandLds = 64 * kYRowBytes + 2 * 64 * kSLds * 2;   // bytes

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ int ypos(int r, int q) { return r * (kYRowBytes / 16) + (q ^ (r & 15)); }

__device__ __forceinline__ void expand_tile_bf16(const RowSet& rs, int r0, int rows,
                                                 const float* __restrict__ S, int sld, int sc0,
                                                 const uint16_t* __restrict__ B, int rp, int n0,
                                                 int n1, uint16_t* __restrict__ y, int64_t ldy_,
                                                 uint4* __restrict__ ytile,
                                                 uint16_t* __restrict__ sHi,
                                                 uint16_t* __restrict__ sLo) {
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int lr = lane % 16;
    const int lq = lane / 16;
    const int nsteps = (rp + 31) / 32;
    const int nw = n0 + wave * 64;
    const int nchunks = (n1 - n0) / 8;                // valid 16-byte chunks per row
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
    uint4 bop[4][2];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        const int n = nw + nb * 16 + lr;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const int j = st * 32 + lq * 8;
            bop[nb][st] = ld16_if(B + (int64_t)n * rp + j, st < nsteps && n < n1 && j < rp, B);
        }
    }
    // 1c. S rows: thread t covers row t / 4, quarter t % 4 of rp
    {
        const int row = tid / 4, qt = tid % 4;
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
    __builtin_amdgcn_s_waitcnt(0);    // direct-to-LDS loads are tracked by vmcnt only
    __syncthreads();
    // 2. MFMA; each 16 x 16 result is added into the LDS tile
    if (nw < n1) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            if (rg * 16 >= rows) break;
            uint4 shi[2], slo[2];
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const int j = st * 32 + lq * 8;
                const bool jin = st < nsteps && j < rp;
                shi[st] = ld16_if(sHi + (rg * 16 + lr) * kSLds + j, jin, sHi);
                slo[st] = ld16_if(sLo + (rg * 16 + lr) * kSLds + j, jin, sLo);
            }
            const int r = rg * 16 + lr;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < 2; ++st) {
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
        }
    }
    __syncthreads();
    // 3. row-major write-back: thread t covers rows t/32 + 8i, chunk t % 32
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = tid / 32 + 8 * i;
        const int q = tid % 32;
        const int yr = r < rows ? rs.out_row[r0 + r] : -1;
        if (yr >= 0 && q < nchunks)
            *reinterpret_cast<uint4*>(y + (int64_t)yr * ldy_ + n0 + q * 8) = ytile[ypos(r, q)];
    }
    __syncthreads();     // the LDS tile is reused by the next tile
}

// All rows of rs over columns [n_begin, n_end), one 64 x 256 tile at a time.
__device__ __forceinline__ void expand_rows_bf16(const RowSet& rs, const float* __restrict__ S,
                                                 int sld, int sc0,
                                                 const uint16_t* __restrict__ B, int rp,
                                                 int n_begin, int n_end,
                                                 uint16_t* __restrict__ y, int64_t ldy_,
                                                 uint4* __restrict__ lds) {
    for (int r0 = 0; r0 < rs.n; r0 += 64) {
        const int rows = min(64, rs.n - r0);
        for (int n0 = n_begin; n0 < n_end; n0 += kNTile)
            expand_tile_bf16(rs, r0, rows, S, sld, sc0, B, rp, n0, min(n0 + kNTile, n_end), y,
                             ldy_, lds, reinterpret_cast<uint16_t*>(lds + 64 * kYRowBytes / 16),
                             reinterpret_cast<uint16_t*>(lds + 64 * kYRowBytes / 16) + 64 * kSLds);
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
