// lora_build_segments: token clustering by adapter id into a segment table
// ("vLLM-Ascend dynamic LoRA operator" walkthrough, section 2.3: equal ids
// made contiguous; a segment is an id plus a contiguous range of tokens).
//
// One workgroup runs a stable counting sort:
//   1. histogram of bucket ids in LDS (bucket L = no adapter);
//   2. one wavefront scans the histogram into bucket bases and compacts the
//      non-empty adapter buckets into (req_to_lora, seg_indptr);
//   3. tokens are scattered tile by tile in token order: inside a wavefront
//      equal buckets are found with one ballot per id bit, so a token's rank
//      among its equals is a popcount; earlier wavefronts' counts per bucket
//      come from a small LDS table.  Order inside a bucket is token order.
// It also writes the tile schedule the shrink / expand kernels run on (the
// walkthrough's section 2.4: which block, which segment, which rank is worked
// out before the product kernels start): every segment is cut into tiles of
// 64 sorted positions, and each tile records its segment, adapter, first
// position, row count and its 64 token indices, so a product workgroup finds
// everything about its rows in one memory round trip.
#include "common.hpp"
#include "kernels.hpp"
#include "wave_groups.hpp"

namespace mlora {

constexpr int kSegThreads = 1024;
constexpr int kSegWaves = kSegThreads / kWave;
constexpr int kCachedTiles = 8;

__global__ __launch_bounds__(kSegThreads) void k_build_segments(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ enabled, int M, int L,
    int32_t* __restrict__ sorted_idx, int32_t* __restrict__ seg_indptr,
    int32_t* __restrict__ req_to_lora, int32_t* __restrict__ num_segments,
    int32_t* __restrict__ tile_info, int32_t* __restrict__ tile_rows,
    int32_t* __restrict__ num_tiles, int max_tiles) {
    extern __shared__ int lds[];
    const int NB = L + 1;
    int* count = lds;                    // [NB]
    int* base = count + NB;              // [NB]  running output position per bucket
    int* bstart = base + NB;             // [NB]  first sorted position of bucket b
    int* btile = bstart + NB;            // [NB]  first tile of bucket b's segment
    int* stile = btile + NB;             // [NB]  first tile of segment s (stile[nseg] = total)
    int* sbucket = stile + NB;           // [NB]  adapter id of segment s
    int* wcnt = sbucket + NB;            // [kSegWaves][NB] per-tile, per-wave bucket counts
    __shared__ int s_segs, s_tiles;
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;

    for (int i = tid; i < NB * (6 + kSegWaves); i += kSegThreads) lds[i] = 0;
    __syncthreads();
    // bucket L collects tokens without an (enabled) adapter
    auto bucket_of = [&](int v) {
        const bool in = v >= 0 && v < L;
        return (in && (!enabled || enabled[v] != 0)) ? v : L;
    };

    // bucket of each of this thread's tokens; the first kCachedTiles tiles stay
    // in registers for the scatter (their loads are issued together)
    int bk[kCachedTiles];
#pragma unroll
    for (int i = 0; i < kCachedTiles; ++i) {
        const int m = i * kSegThreads + tid;
        int b = L;
        if (m < M) b = bucket_of(ids[m]);
        bk[i] = b;
    }
    const int nbits = 32 - __clz(L);          // enough bits for buckets 0..L
    const unsigned long long lt = (1ull << lane) - 1ull;
    // lanes of this wavefront (with a token) whose bucket equals b: one
    // ballot per bucket bit
    auto peers_of = [&](int b, bool act) {
        unsigned long long pe = __ballot(act);
        for (int i = 0; i < nbits; ++i) {
            const bool bit = (b >> i) & 1;
            const unsigned long long bb = __ballot(bit);
            pe &= bit ? bb : ~bb;
        }
        return pe;
    };
    // histogram: one LDS atomic per distinct bucket and wavefront (a batch
    // of contiguous segments gives most wavefronts a single bucket)
    auto count_tile = [&](int t0, int b) {
        const bool act = t0 + tid < M;
        const unsigned long long pe = peers_of(b, act);
        if (act && __popcll(pe & lt) == 0) atomicAdd(&count[b], __popcll(pe));
    };
#pragma unroll
    for (int i = 0; i < kCachedTiles; ++i) {
        if (i * kSegThreads >= M) break;
        count_tile(i * kSegThreads, bk[i]);
    }
    for (int t0 = kCachedTiles * kSegThreads; t0 < M; t0 += kSegThreads)
        count_tile(t0, t0 + tid < M ? bucket_of(ids[t0 + tid]) : L);
    __syncthreads();

    if (wave == 0) {
        int run = 0, segs = 0, trun = 0;
        for (int b0 = 0; b0 < NB; b0 += kWave) {
            const int b = b0 + lane;
            const int c = (b < NB) ? count[b] : 0;
            const bool present = (b < L) && (c > 0);
            const int nt = present ? (c + kRowTileRows - 1) / kRowTileRows : 0;
            int inc = c, tinc = nt;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const int t = __shfl_up(inc, o, kWave);
                const int u = __shfl_up(tinc, o, kWave);
                if (lane >= o) {
                    inc += t;
                    tinc += u;
                }
            }
            const int excl = run + inc - c;
            const int texcl = trun + tinc - nt;
            if (b < NB) {
                base[b] = excl;
                bstart[b] = excl;
                btile[b] = texcl;
            }
            const unsigned long long bal = __ballot(present);
            const int s = segs + __popcll(bal & ((1ull << lane) - 1ull));
            if (present) {
                req_to_lora[s] = b;
                seg_indptr[s + 1] = excl + c;
                stile[s] = texcl;
                sbucket[s] = b;
            }
            run += __shfl(inc, kWave - 1, kWave);
            trun += __shfl(tinc, kWave - 1, kWave);
            segs += __popcll(bal);
        }
        const int m_valid = run - count[L];
        if (lane == 0) {
            seg_indptr[0] = 0;
            num_segments[0] = segs;
            num_tiles[0] = trun;
            stile[segs] = trun;
            s_segs = segs;
            s_tiles = trun;
        }
        for (int s = segs + 1 + lane; s <= L; s += kWave) seg_indptr[s] = m_valid;
        for (int s = segs + lane; s < L; s += kWave) req_to_lora[s] = -1;
    }
    __syncthreads();

    // tile schedule: per 64-row tile its segment, adapter, first position and
    // row count; rows past the count are marked -1 in tile_rows
    {
        const int segs = s_segs;
        const int tiles = min(s_tiles, max_tiles);
        for (int t = tid; t < tiles; t += kSegThreads) {
            int lo = 0, hi = segs - 1;                 // last s with stile[s] <= t
            while (lo < hi) {
                const int mid = (lo + hi + 1) / 2;
                if (stile[mid] <= t) lo = mid; else hi = mid - 1;
            }
            const int b = sbucket[lo];
            const int i = t - stile[lo];
            const int beg = bstart[b] + i * kRowTileRows;
            const int n = min(kRowTileRows, count[b] - i * kRowTileRows);
            tile_info[t * 4 + 0] = lo;
            tile_info[t * 4 + 1] = b;
            tile_info[t * 4 + 2] = beg;
            tile_info[t * 4 + 3] = n;
            for (int r = n; r < kRowTileRows; ++r) tile_rows[t * kRowTileRows + r] = -1;
        }
    }

    // one tile of kSegThreads tokens in token order; b = this thread's bucket
    auto scatter_tile = [&](int t0, int b) {
        const int m = t0 + tid;
        const bool act = m < M;
        const unsigned long long peers = peers_of(b, act);
        const int rank_w = __popcll(peers & lt);
        const bool leader = act && rank_w == 0;
        if (leader) wcnt[wave * NB + b] = __popcll(peers);
        __syncthreads();
        if (act) {
            // earlier wavefronts' tokens of the bucket (all reads issued together)
            int pos = base[b] + rank_w;
#pragma unroll
            for (int w = 0; w < kSegWaves; ++w) pos += w < wave ? wcnt[w * NB + b] : 0;
            sorted_idx[pos] = m;
            if (b < L) {
                const int rel = pos - bstart[b];
                const int t = btile[b] + rel / kRowTileRows;
                if (t < max_tiles) tile_rows[t * kRowTileRows + rel % kRowTileRows] = m;
            }
        }
        __syncthreads();
        if (leader) {
            atomicAdd(&base[b], __popcll(peers));
            wcnt[wave * NB + b] = 0;
        }
        __syncthreads();
    };
#pragma unroll
    for (int i = 0; i < kCachedTiles; ++i) {
        if (i * kSegThreads >= M) break;
        scatter_tile(i * kSegThreads, bk[i]);
    }
    for (int t0 = kCachedTiles * kSegThreads; t0 < M; t0 += kSegThreads) {
        int b = L;
        if (t0 + tid < M) b = bucket_of(ids[t0 + tid]);
        scatter_tile(t0, b);
    }
}

// ---------------------------------------------------------------------------
// Small batches (M <= 64, the decode case): one wavefront, no LDS and no
// barriers (wave_groups.hpp: bitonic sort of (bucket, token) keys across the
// 64 lanes, segment starts from neighbour comparisons, segment numbers from
// popcounts).  Every segment has at most 64 rows, so it is exactly one tile
// of the schedule.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kWave) void k_build_segments_wave(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ enabled, int M, int L,
    int32_t* __restrict__ sorted_idx, int32_t* __restrict__ seg_indptr,
    int32_t* __restrict__ req_to_lora, int32_t* __restrict__ num_segments,
    int32_t* __restrict__ tile_info, int32_t* __restrict__ tile_rows,
    int32_t* __restrict__ num_tiles) {
    const int b = M > 0 ? token_bucket(load_token(ids, enabled, M, L), enabled, L) : L;
    const WaveGroups g = wave_group(b, M, L);
    write_wave_segments(g, M, L, sorted_idx, seg_indptr, req_to_lora, num_segments, tile_info,
                        tile_rows, num_tiles);
}

hipError_t launch_build_segments(const int32_t* ids, const int32_t* enabled, int M, int L,
                                 int32_t* sorted_idx, int32_t* seg_indptr, int32_t* req_to_lora,
                                 int32_t* num_segments, int32_t* tile_info, int32_t* tile_rows,
                                 int32_t* num_tiles, int max_tiles, hipStream_t st) {
    if (M <= kWave) {
        hipLaunchKernelGGL(k_build_segments_wave, dim3(1), dim3(kWave), 0, st, ids, enabled, M, L,
                           sorted_idx, seg_indptr, req_to_lora, num_segments, tile_info,
                           tile_rows, num_tiles);
        return hipGetLastError();
    }
    const size_t lds = (size_t)(L + 1) * (6 + kSegWaves) * sizeof(int);
    hipLaunchKernelGGL(k_build_segments, dim3(1), dim3(kSegThreads), lds, st, ids, enabled, M, L,
                       sorted_idx, seg_indptr, req_to_lora, num_segments, tile_info, tile_rows,
                       num_tiles, max_tiles);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// zero fill (workspace initialisation; a kernel rather than a memset so that
// it can sit inside a captured graph)
// ---------------------------------------------------------------------------
__global__ void k_fill_zero(uint4* __restrict__ p, size_t n16, uint8_t* __restrict__ tail,
                            size_t ntail) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        p[i] = make_uint4(0, 0, 0, 0);
    if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
    if (bytes == 0) return hipSuccess;
    const size_t n16 = bytes / 16;
    const size_t ntail = bytes - n16 * 16;
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks == 0) blocks = 1;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, st, (uint4*)p, n16,
                       (uint8_t*)p + n16 * 16, ntail);
    return hipGetLastError();
}

}  // namespace mlora
