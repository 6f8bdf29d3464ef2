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
// shrink: partial S over one K chunk for NCB column blocks of 16
//   block cb: slice sl = cb / bps, j-block jj = cb % bps (bps = r_max/16);
//   active when jj < rp/16, reads adapter rows sl*rp + jj*16 .. +16;
//   inactive blocks store zeros (rank padding beyond the adapter's rank).
// ---------------------------------------------------------------------------
template <int NCB>
__device__ __forceinline__ void shrink_tile_bf16(const RowSet& rs, const uint16_t* __restrict__ x,
                                                 int64_t ldx, const uint16_t* __restrict__ A,
                                                 int K, int rp, int r_max, int k0, int k1,
                                                 float* __restrict__ P, int pld) {
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int bps = r_max / 16;
    const int nbr = rp / 16;
    const int lr = lane % 16;
    const int lk = (lane / 16) * 8;
    for (int rg = wave; rg * 16 < rs.RT; rg += kTileWaves) {
        if (rg * 16 >= rs.n) break;
        const int i = rg * 16 + lr;
        const int xr = (i < rs.n) ? rs.in_row[i] : -1;
        const uint16_t* xp = x + (int64_t)(xr < 0 ? 0 : xr) * ldx + lk;
        const uint16_t* ap[NCB];
        bool act[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int sl = cb / bps, jj = cb % bps;
            act[cb] = jj < nbr;
            ap[cb] = A + (int64_t)(sl * rp + (act[cb] ? jj : 0) * 16 + lr) * K + lk;
        }
        f32x4_t acc[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const uint4 z = make_uint4(0, 0, 0, 0);
        int k = nbr > 0 ? k0 : k1;     // rank-0 slot: only the zero stores below
        for (; k + 64 <= k1; k += 64) {
            const uint4 xa0 = xr >= 0 ? ld16(xp + k) : z;
            const uint4 xa1 = xr >= 0 ? ld16(xp + k + 32) : z;
            uint4 b0[NCB], b1[NCB];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                b0[cb] = act[cb] ? ld16(ap[cb] + k) : z;
                b1[cb] = act[cb] ? ld16(ap[cb] + k + 32) : z;
            }
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                if (act[cb]) {
                    acc[cb] = mfma_bf16(xa0, b0[cb], acc[cb]);
                    acc[cb] = mfma_bf16(xa1, b1[cb], acc[cb]);
                }
            }
        }
        for (; k < k1; k += 32) {
            // K is a multiple of 8: lanes whose 8 values fall past k1 load zeros
            const bool kin = k + lk < k1;
            const uint4 xa = (xr >= 0 && kin) ? ld16(xp + k) : z;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                if (act[cb]) {
                    const uint4 bb = kin ? ld16(ap[cb] + k) : z;
                    acc[cb] = mfma_bf16(xa, bb, acc[cb]);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = rg * 16 + (lane / 16) * 4 + q;
            const int orow = (row < rs.n) ? rs.out_row[row] : -1;
            if (orow < 0) continue;
            float* pp = P + (int64_t)orow * pld + lr;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) pp[cb * 16] = acc[cb][q];
        }
    }
}

// ---------------------------------------------------------------------------
// expand: y[out_row, n] += sum_{j < rp} S[srow, sc0 + j] * B[n, j] for
// n in [n0, n1) (n1 - n0 <= 256); wave w owns columns n0 + 64w .. +64.
// S rows come from rs.in_row (index into S), y rows from rs.out_row.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ float ldy(const T* p);
template <>
__device__ __forceinline__ float ldy<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

__device__ __forceinline__ void expand_tile_bf16(const RowSet& rs, const float* __restrict__ S,
                                                 int sld, int sc0,
                                                 const uint16_t* __restrict__ B, int rp, int n0,
                                                 int n1, uint16_t* __restrict__ y, int64_t ldy_) {
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int lr = lane % 16;
    const int lk = (lane / 16) * 8;
    const int nw = n0 + wave * 64;
    if (nw >= n1) return;
    const uint4 z = make_uint4(0, 0, 0, 0);
    const int nsteps = (rp + 31) / 32;
    // B operands for the wave's 4 column blocks: rows nw + 16*nb + lr
    uint4 bop[4][2];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        const int n = nw + nb * 16 + lr;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const int j = st * 32 + lk;
            bop[nb][st] = (st < nsteps && n < n1 && j < rp) ? ld16(B + (int64_t)n * rp + j) : z;
        }
    }
    for (int rg = 0; rg * 16 < rs.n; ++rg) {
        const int i = rg * 16 + lr;                     // this lane's S row (operand column)
        const int sr = (i < rs.n) ? rs.in_row[i] : -1;
        uint4 shi[2], slo[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const int j = st * 32 + lk;
            float v[8];
            if (st < nsteps && sr >= 0 && j < rp) {
                const float4 a = *reinterpret_cast<const float4*>(S + (int64_t)sr * sld + sc0 + j);
                const float4 b = *reinterpret_cast<const float4*>(S + (int64_t)sr * sld + sc0 + j + 4);
                v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
                v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = 0.f;
            }
            split_hi_lo(v, shi[st], slo[st]);
        }
        // output rows handled by this lane: tokens rg*16 + lr; columns 4*(lane/16)+q
        const int yr = (i < rs.n) ? rs.out_row[i] : -1;
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
            // acc[q] = delta for column nw + 16*nb + 4*(lane/16) + q, token row i
            const int n = nw + nb * 16 + (lane / 16) * 4;
            if (yr >= 0 && n < n1) {
                uint16_t* yp = y + (int64_t)yr * ldy_ + n;
                const uint2 old = *reinterpret_cast<const uint2*>(yp);
                const float o0 = __uint_as_float(old.x << 16);
                const float o1 = __uint_as_float(old.x & 0xffff0000u);
                const float o2 = __uint_as_float(old.y << 16);
                const float o3 = __uint_as_float(old.y & 0xffff0000u);
                uint2 nv;
                nv.x = f32_to_bf16(o0 + acc[0]) | (f32_to_bf16(o1 + acc[1]) << 16);
                nv.y = f32_to_bf16(o2 + acc[2]) | (f32_to_bf16(o3 + acc[3]) << 16);
                *reinterpret_cast<uint2*>(yp) = nv;
            }
        }
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
