// lora_build_segments: token clustering by adapter id into a segment table
// ("vLLM-Ascend dynamic LoRA operator" walkthrough, section 2.3: equal ids
// made contiguous; a segment is an id plus a contiguous range of tokens).
//
// One workgroup of 16 wavefronts runs a stable counting sort.  Wavefront w
// owns a contiguous chunk of the tokens (a multiple of 64, in passes of 64):
//   1. every id load is issued at once (the first kCachedPasses passes stay in
//      registers), together with the adapter mask, which goes to LDS, so a
//      token's bucket (its id, or L for none or a disabled adapter) costs no
//      dependent global load;
//   2. each wavefront counts its chunk per bucket into its own LDS row: inside
//      a pass equal buckets are found with one ballot per id bit, and the
//      first lane of each group adds the group's size;
//   3. per bucket, the rows are turned into exclusive offsets across the
//      wavefronts; one wavefront scans the bucket totals into bucket bases and
//      compacts the non-empty adapter buckets into (req_to_lora, seg_indptr);
//   4. each wavefront scatters its chunk with no further barrier: a token's
//      position is its bucket's base, plus its wavefront's offset, plus the
//      equal tokens of its earlier passes (kept in the same row), plus its
//      rank inside its pass (a popcount).  Order inside a bucket is token
//      order.
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
constexpr int kCachedPasses = 8;   // tokens per wavefront kept in registers: 8 x 64

// LDS words of the block builder for L adapter slots
inline size_t build_segments_lds(int L) {
    return ((size_t)(L + 1) * (kSegWaves + 5) + (size_t)L) * sizeof(int);
}

__global__ __launch_bounds__(kSegThreads) void k_build_segments(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ enabled, int M, int L,
    int32_t* __restrict__ sorted_idx, int32_t* __restrict__ seg_indptr,
    int32_t* __restrict__ req_to_lora, int32_t* __restrict__ num_segments,
    int32_t* __restrict__ tile_info, int32_t* __restrict__ tile_rows,
    int32_t* __restrict__ num_tiles, int max_tiles) {
    extern __shared__ int lds[];
    const int NB = L + 1;
    int* row = lds;                      // [kSegWaves][NB] per-wavefront bucket counts, then offsets
    int* total = row + kSegWaves * NB;   // [NB]  tokens per bucket
    int* bstart = total + NB;            // [NB]  first sorted position of bucket b
    int* btile = bstart + NB;            // [NB]  first tile of bucket b's segment
    int* stile = btile + NB;             // [NB]  first tile of segment s (stile[nseg] = total)
    int* sbucket = stile + NB;           // [NB]  adapter id of segment s
    int* en = sbucket + NB;              // [L]   adapter mask
    __shared__ int s_segs, s_tiles;
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;

    // chunk of this wavefront: [c0, c1), passes of 64 tokens
    const int per = (M + kSegThreads - 1) / kSegThreads;      // passes per wavefront
    const int c0 = min(M, wave * per * kWave);
    const int c1 = min(M, c0 + per * kWave);

    // 1. every load at once: the cached passes' ids (index clamped into the
    //    batch, so no load is conditional) and the mask
    int idc[kCachedPasses];
#pragma unroll
    for (int i = 0; i < kCachedPasses; ++i) idc[i] = ids[min(c0 + i * kWave + lane, M - 1)];
    const int e = (enabled && tid < L) ? enabled[tid] : 1;
    for (int i = tid; i < kSegWaves * NB; i += kSegThreads) row[i] = 0;
    for (int i = tid; i < L; i += kSegThreads) en[i] = (i == tid) ? e : (enabled ? enabled[i] : 1);
    __syncthreads();

    // the mask entry is read at a clamped index, so the lookups of several
    // passes do not wait for one another
    auto bucket_of = [&](int v) {
        const bool in = v >= 0 && v < L;
        const int on = en[in ? v : 0];
        return (in && on != 0) ? v : L;
    };
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
    int* my = row + wave * NB;
    // bucket of pass i's token (L past the chunk); passes past the cached
    // ones load their ids again
    auto pass_bucket = [&](int i) {
        const int m = c0 + i * kWave + lane;
        return m < c1 ? bucket_of(ids[m]) : L;
    };
    int bk[kCachedPasses];
#pragma unroll
    for (int i = 0; i < kCachedPasses; ++i) {
        const int v = idc[i];
        const bool in = v >= 0 && v < L;
        const int on = en[in ? v : 0];            // unconditional: the reads overlap
        bk[i] = (c0 + i * kWave + lane < c1 && in && on != 0) ? v : L;
    }

    // 2. counts of this wavefront's chunk per bucket (wave-private row; the
    //    first lane of each group of equal buckets adds the group's size)
    auto count_pass = [&](int i, int b) {
        const bool act = c0 + i * kWave + lane < c1;
        const unsigned long long pe = peers_of(b, act);
        if (act && __popcll(pe & lt) == 0) my[b] += __popcll(pe);
    };
#pragma unroll
    for (int i = 0; i < kCachedPasses; ++i)
        if (c0 + i * kWave < c1) count_pass(i, bk[i]);
    for (int i = kCachedPasses; c0 + i * kWave < c1; ++i) count_pass(i, pass_bucket(i));
    __syncthreads();

    // 3a. per bucket: the wavefront rows become exclusive offsets (all 16
    //     counts read before any is rewritten, so the reads overlap)
    for (int b = tid; b < NB; b += kSegThreads) {
        int c[kSegWaves];
#pragma unroll
        for (int w = 0; w < kSegWaves; ++w) c[w] = row[w * NB + b];
        int run = 0;
#pragma unroll
        for (int w = 0; w < kSegWaves; ++w) {
            row[w * NB + b] = run;
            run += c[w];
        }
        total[b] = run;
    }
    __syncthreads();

    // 3b. bucket bases, segments and tile numbers (one wavefront)
    if (wave == 0) {
        int run = 0, segs = 0, trun = 0;
        for (int b0 = 0; b0 < NB; b0 += kWave) {
            const int b = b0 + lane;
            const int c = (b < NB) ? total[b] : 0;
            const bool present = (b < L) && (c > 0);
            const int nt = present ? (c + kRowTileRows - 1) / kRowTileRows : 0;
            const int inc = wave_incl_scan(c), tinc = wave_incl_scan(nt);
            const int excl = run + inc - c;
            const int texcl = trun + tinc - nt;
            if (b < NB) {
                bstart[b] = excl;
                btile[b] = texcl;
            }
            const unsigned long long bal = __ballot(present);
            const int s = segs + __popcll(bal & lt);
            if (present) {
                req_to_lora[s] = b;
                seg_indptr[s + 1] = excl + c;
                stile[s] = texcl;
                sbucket[s] = b;
            }
            run += __builtin_amdgcn_readlane(inc, kWave - 1);
            trun += __builtin_amdgcn_readlane(tinc, kWave - 1);
            segs += __popcll(bal);
        }
        const int m_valid = run - total[L];
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
    // row count; rows past the count are marked -1 in tile_rows.  One
    // wavefront per tile, lane r for row r: the tile's segment is the last s
    // with stile[s] <= t, found by a ballot (64 segments at a time past 64).
    {
        const int segs = s_segs;
        const int tiles = min(s_tiles, max_tiles);
        // up to 64 segments: lane s holds segment s's first tile, adapter,
        // first position and size, read once per wavefront, so a tile costs
        // a ballot and four readlanes instead of a chain of LDS reads
        const bool in_regs = segs <= kWave;
        int g_st = 0, g_b = 0, g_beg = 0, g_n = 0;
        if (in_regs && lane < segs) {
            g_st = stile[lane];
            g_b = sbucket[lane];
            g_beg = bstart[g_b];
            g_n = total[g_b];
        }
        for (int t = wave; in_regs && t < tiles; t += kSegWaves) {
            const unsigned long long bl = __ballot(lane < segs && g_st <= t);
            const int s = 63 - __clzll(bl);        // stile[0] = 0 <= t: never empty
            const int b = __builtin_amdgcn_readlane(g_b, s);
            const int i = t - __builtin_amdgcn_readlane(g_st, s);
            const int beg = __builtin_amdgcn_readlane(g_beg, s) + i * kRowTileRows;
            const int n = min(kRowTileRows, __builtin_amdgcn_readlane(g_n, s) - i * kRowTileRows);
            if (lane < 4) tile_info[t * 4 + lane] = lane == 0 ? s : lane == 1 ? b : lane == 2 ? beg : n;
            if (lane >= n) tile_rows[t * kRowTileRows + lane] = -1;
        }
        for (int t = wave; !in_regs && t < tiles; t += kSegWaves) {
            int s = 0;
            for (int s0 = 0; s0 < segs; s0 += kWave) {
                const bool le = s0 + lane < segs && stile[s0 + lane] <= t;
                const unsigned long long bl = __ballot(le);
                if (bl) s = s0 + 63 - __clzll(bl);
            }
            const int b = sbucket[s];
            const int i = t - stile[s];
            const int beg = bstart[b] + i * kRowTileRows;
            const int n = min(kRowTileRows, total[b] - i * kRowTileRows);
            if (lane < 4) tile_info[t * 4 + lane] = lane == 0 ? s : lane == 1 ? b : lane == 2 ? beg : n;
            if (lane >= n) tile_rows[t * kRowTileRows + lane] = -1;
        }
    }

    // 4. scatter, pass by pass in token order; the wavefront's row now holds,
    //    per bucket, the sorted offset of its next token inside the bucket
    auto scatter_pass = [&](int i, int b) {
        const int m = c0 + i * kWave + lane;
        const bool act = m < c1;
        const unsigned long long peers = peers_of(b, act);
        const int rank_w = __popcll(peers & lt);
        if (act) {
            const int pos = bstart[b] + my[b] + rank_w;
            sorted_idx[pos] = m;
            if (b < L) {
                const int rel = pos - bstart[b];
                const int t = btile[b] + rel / kRowTileRows;
                if (t < max_tiles) tile_rows[t * kRowTileRows + rel % kRowTileRows] = m;
            }
        }
        // every lane has read its offset before the group's first lane moves it
        __builtin_amdgcn_wave_barrier();
        if (act && rank_w == 0) my[b] += __popcll(peers);
        __builtin_amdgcn_wave_barrier();
    };
#pragma unroll
    for (int i = 0; i < kCachedPasses; ++i)
        if (c0 + i * kWave < c1) scatter_pass(i, bk[i]);
    for (int i = kCachedPasses; c0 + i * kWave < c1; ++i) scatter_pass(i, pass_bucket(i));
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
    const size_t lds = build_segments_lds(L);
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
