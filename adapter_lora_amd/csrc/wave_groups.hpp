// Grouping of a small batch (M <= 64 tokens) by adapter id inside one
// wavefront ("vLLM-Ascend dynamic LoRA operator" walkthrough, section 2.3:
// equal ids made contiguous, one segment per id).  Token m (lane m) has a
// bucket: its adapter id, or L for "no adapter".  The sorted order is by
// bucket and, inside a bucket, by token (a stable order); token m's sorted
// position is the number of tokens with a smaller bucket plus the number of
// earlier tokens with the same bucket.  Both counts come from ballots, one
// per bit of the bucket from the highest down: after the bits above bit i,
// each lane knows which lanes still agree with it (`eq`) and which were
// already found smaller (`less`).  A single forward lane permute then puts
// every token at its sorted position.  Segment starts are the sorted
// positions whose bucket differs from the left neighbour's, and segment
// numbers are popcounts of the start mask, so any segment's bounds are found
// with one ballot.  No LDS and no barriers: every wavefront that needs the
// grouping computes it itself.
#pragma once

#include "common.hpp"

namespace mlora {

struct WaveGroups {
    int key;                   // lane p: (bucket << 6) | token at sorted position p; INT_MAX past M
    unsigned long long smask;  // bit p: a segment starts at sorted position p
    int nseg;                  // segments (adapters with at least one token)
    int mvalid;                // tokens with an adapter
};

// mask of bits 0..p (p in 0..63)
__device__ __forceinline__ unsigned long long bits_upto(int p) {
    return p >= kWave - 1 ? ~0ull : ((2ull << p) - 1ull);
}

// `bucket` is lane m's bucket (0..L-1, or L for none); lanes >= M are ignored.
__device__ __forceinline__ WaveGroups wave_group(int bucket, int M, int L) {
    const int lane = lane_id();
    const bool valid = lane < M;
    const unsigned long long vmask = __ballot(valid);
    unsigned long long less = 0ull, eq = vmask;
    const int nbits = 32 - __clz(L);          // bits of the buckets 0..L
    for (int i = nbits - 1; i >= 0; --i) {
        const bool bit = (bucket >> i) & 1;
        const unsigned long long B = __ballot(valid && bit);
        less |= bit ? (eq & ~B) : 0ull;
        eq &= bit ? B : ~B;
    }
    // lanes >= M keep their own position: the valid tokens fill 0 .. M-1
    const int pos = valid ? __popcll(less) + __popcll(eq & ((1ull << lane) - 1ull)) : lane;
    const int mine = valid ? (bucket << 6) | lane : 0x7fffffff;
    const int key = __builtin_amdgcn_ds_permute(pos * 4, mine);
    const int b = key >> 6;
    const bool has = lane < M && b < L;
    const int prev = __shfl_up(b, 1, kWave);
    const bool start = has && (lane == 0 || prev != b);
    WaveGroups g;
    g.key = key;
    g.smask = __ballot(start);
    g.nseg = __popcll(g.smask);
    g.mvalid = __popcll(__ballot(has));
    return g;
}

// Segment s of a grouping: first sorted position, token count and adapter
// id (wave-uniform).  A segment past the last one gives n = 0, id = -1.
__device__ __forceinline__ void wave_segment(const WaveGroups& g, int s, int* p0, int* n, int* id) {
    const int lane = lane_id();
    const bool start = (g.smask >> lane) & 1ull;
    const int segno = __popcll(g.smask & bits_upto(lane)) - 1;
    const unsigned long long hit = __ballot(start && segno == s);
    if (hit == 0ull) {
        *p0 = 0;
        *n = 0;
        *id = -1;
        return;
    }
    const int p = __ffsll((long long)hit) - 1;
    const unsigned long long above = g.smask & ~bits_upto(p);
    const int p1 = above ? __ffsll((long long)above) - 1 : g.mvalid;
    *p0 = p;
    *n = p1 - p;
    *id = __builtin_amdgcn_readlane(g.key, p) >> 6;
}

// Bucket of token `lane` (lanes >= M read token M - 1 and are ignored):
// its id when that lies in [0, L) and the adapter is enabled, else L.
// `enabled` may be null (every adapter enabled).  Split in two so that a
// caller can issue other loads between them: load_token() issues the id
// load and, for L <= 256, one mask load per 64 slots and lane;
// token_bucket() picks the token's mask entry by lane shuffle (a dependent
// load only for larger tables).  M >= 1.
struct TokenLoad {
    int v;
    int e[4];
};

__device__ __forceinline__ TokenLoad load_token(const int32_t* __restrict__ ids,
                                                const int32_t* __restrict__ enabled, int M, int L) {
    const int lane = lane_id();
    TokenLoad t;
    t.v = ids[min(lane, M - 1)];
#pragma unroll
    for (int q = 0; q < 4; ++q) t.e[q] = 1;
    if (enabled && L <= 4 * kWave) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (q * kWave < L) t.e[q] = enabled[min(q * kWave + lane, L - 1)];
    }
    return t;
}

__device__ __forceinline__ int token_bucket(const TokenLoad& t, const int32_t* __restrict__ enabled,
                                            int L) {
    const bool in = t.v >= 0 && t.v < L;
    if (!enabled) return in ? t.v : L;
    int on;
    if (L <= 4 * kWave) {
        const int vv = in ? t.v : 0;
        const int src = vv % kWave, q = vv / kWave;
        on = __shfl(t.e[0], src, kWave);
#pragma unroll
        for (int k = 1; k < 4; ++k)
            if (k * kWave < L) {
                const int ek = __shfl(t.e[k], src, kWave);
                on = q == k ? ek : on;
            }
    } else {
        on = in ? enabled[t.v] : 0;
    }
    return (in && on != 0) ? t.v : L;
}

// Segment table and tile schedule of a grouping, written by one wavefront
// in the layout lora_build_segments produces (every segment of a batch of
// at most 64 tokens is exactly one 64-row tile).
__device__ __forceinline__ void write_wave_segments(const WaveGroups& g, int M, int L,
                                                    int32_t* __restrict__ sorted_idx,
                                                    int32_t* __restrict__ seg_indptr,
                                                    int32_t* __restrict__ req_to_lora,
                                                    int32_t* __restrict__ num_segments,
                                                    int32_t* __restrict__ tile_info,
                                                    int32_t* __restrict__ tile_rows,
                                                    int32_t* __restrict__ num_tiles) {
    const int lane = lane_id();
    const int m = g.key & 63;
    const int b = g.key >> 6;
    const bool start = (g.smask >> lane) & 1ull;
    const unsigned long long le = bits_upto(lane);
    const unsigned long long above = g.smask & ~le;
    const int n_here = (above ? __ffsll((long long)above) - 1 : g.mvalid) - lane;
    if (lane < M) sorted_idx[lane] = m;
    if (start) {
        const int s = __popcll(g.smask & le) - 1;
        req_to_lora[s] = b;
        seg_indptr[s] = lane;
        tile_info[s * 4 + 0] = s;
        tile_info[s * 4 + 1] = b;
        tile_info[s * 4 + 2] = lane;
        tile_info[s * 4 + 3] = n_here;
    }
    // rows of tile s: sorted positions p0 .. p0 + n - 1, then -1
    unsigned long long rest = g.smask;
    for (int s = 0; s < g.nseg; ++s) {
        const int p0 = __ffsll((long long)rest) - 1;
        rest &= rest - 1;
        const int n = __shfl(n_here, p0, kWave);
        const int r = __shfl(m, min(p0 + lane, kWave - 1), kWave);
        tile_rows[s * kWave + lane] = lane < n ? r : -1;
    }
    for (int s = g.nseg + lane; s <= L; s += kWave) seg_indptr[s] = g.mvalid;
    for (int s = g.nseg + lane; s < L; s += kWave) req_to_lora[s] = -1;
    if (lane == 0) {
        num_segments[0] = g.nseg;
        num_tiles[0] = g.nseg;
    }
}

}  // namespace mlora
