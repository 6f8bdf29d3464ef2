// Fused decode: y[m] += (x[m] A_i^T) B_i^T for a small batch (M <= 64) in a
// single launch ("vLLM-Ascend dynamic LoRA operator" walkthrough: section 2.1
// fused operator — look up A/B by id, two low-rank products, add to the base
// rows; section 2.2 — S accumulated in fp32; section 1.2 — at decode every
// token may use a different adapter, so the work is a gather-GEMV whose cost
// is reading each touched adapter's A and B once).
//
// The launch has two groups of workgroups:
//   producers  (blockIdx <  grid1): unit = (segment, 16 rows of A, 512-wide K
//              chunk).  Lanes stream one row of A chunk each 1 KB at a time
//              (coalesced 16-byte loads), dot it with the segment's token rows
//              and reduce across the wavefront with DPP lane swaps.  Each
//              partial sum goes into a tagged 64-bit exchange slot.
//   consumers  (blockIdx >= grid1): unit = (segment, 256 output columns of a
//              slice), thread t owning column n0 + t.  A thread first loads its
//              column's B row (rp contiguous values) and the y values it will
//              update, and only then waits for the segment's slots (one set
//              per launch, shared by every consumer of the segment and
//              tagged with the launch's own tag); the K-chunk
//              partials are summed in a fixed order into LDS (S stays on chip,
//              as a bf16 hi / lo pair for bf16 data) and each thread dots its B
//              row with every token's S row, read from LDS as a broadcast.  No
//              cross-lane reduction is needed on this side.
// Consumers only wait on producers, which never wait, and producers have the
// lower workgroup ids, so they are dispatched first; every wait is also
// bounded (kMaxSpin polls) and reports a device error instead of hanging.
#include "common.hpp"
#include "kernels.hpp"
#include "wave_groups.hpp"

namespace mlora {

constexpr int kDecThreads = 256;

// B rows loaded non-temporal (the cache policy's nt bit) by the one-tile
// consumers: each consumer reads its tile's B block once, and the hint keeps
// it from displacing what the rest of the launch reads again (decode step
// 8.70 against 8.95 us).  The lookup consumers of the embedding read plain
// (9.4 against 7.7 us with the hint), and so do the pipelined multi-tile
// consumers (LM head 18.9 against 18.4 us).
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}
constexpr int kDecWaves = kDecThreads / kWave;

struct DecodeParams {
    LinearArgs a;
    const void* x;
    int64_t ldx;
    void* y;
    int64_t ldy;
    int* err;
    slot_t* slots;     // [C][64][a.cols]: K chunk, sorted position, S column
    int C;
    int jb_max;        // n_sl * r_max / 16
    int grid1;
    int n_tiles;
    int tile_start[LORA_MAX_SLICES + 1];
    int G;             // 256-column tiles per consumer (consecutive, one slice)
    int n_groups;      // consumers per segment, all slices
    int group_start[LORA_MAX_SLICES + 1];
    const int32_t* ids;      // non-null: segments grouped on chip from the ids
    const int32_t* enabled;  // adapter mask for that grouping (may be null)
    SegOut out;              // segment table written by the last workgroup (ids mode)
    int writer;              // 1 when the last workgroup writes `out`
    int by_slot;             // ids mode with L <= M: producers numbered over the used slots
    const int32_t* tokens;   // non-null: embedding lookup, S rows read from the
                             // transposed A table by token id (a.K = vocab); no producers
    WaitCtl wc;              // the consumers' bounded waits
    int pipe;                // bf16 consumers walk their tiles pipelined (dec_consumer_run)
};

// ---------------------------------------------------------------- shared view
// Everything a workgroup needs to know about segment s, fetched with
// independent loads so that the index lookups cost one memory round trip:
// either the segment table's entries for s and the whole sorted token list
// (M <= 64, one entry per lane), or, in ids mode, every token's id (the
// grouping is then computed in registers, wave_groups.hpp); and, for tables
// of up to 256 slots, every slot's rank and weight offset (picked by lane
// shuffle once the id is known).
struct SegView {
    int nseg, id, rp, p0, ms;
    int tl;                    // lane t < ms: the segment's t-th token (sorted order)
    int64_t off;
    int tok;                   // lane t < ms: token id of the segment's t-th token (embedding lookup)
    int64_t off2;              // the adapter's A offset as well (embedding lookup)
};

// Exchange slot of K chunk c, sorted position pos and S column col
// (slice sl, rank index j: col = sl * r_max + j).
__device__ __forceinline__ slot_t* slot_at(const DecodeParams& p, int c, int pos, int col) {
    return p.slots + ((int64_t)c * LORA_DECODE_MAX_M + pos) * p.a.cols + col;
}

// The arguments the segment view reads first, passed ahead of the parameter
// block as separate scalar kernel arguments: the view's loads then start
// without waiting for the loads of the (600-byte) parameter block, which
// measured 0.3-0.5 us earlier on the decode workload.
struct ViewArgs {
    const int32_t* ids;        // null: segments come from the table in the parameter block
    const int32_t* rank;
    const int64_t* offs;       // a_off for producers, b_off for consumers
    int M, L;
    const int32_t* tokens;     // embedding lookup: token ids (else null)
    const int64_t* offs2;      // embedding lookup: a_off (else null)
};

__device__ __forceinline__ SegView seg_view(const DecodeParams& p, const ViewArgs& va, int s) {
    const LinearArgs& a = p.a;
    const int lane = lane_id();
    const int64_t* offs = va.offs;
    const int M = va.M, L = va.L;
    SegView v;
    TokenLoad tl;
    int p1 = 0;
    const int tk = va.tokens ? va.tokens[min(lane, M - 1)] : 0;
    if (va.ids) {
        tl = load_token(va.ids, p.enabled, M, L);
    } else {
        v.nseg = a.num_segments[0];
        v.id = a.req_to_lora[s];
        v.p0 = a.seg_indptr[s];
        p1 = a.seg_indptr[s + 1];
        // indices are clamped rather than tested, so every load is
        // unconditional and all of them are in flight together
        v.tl = a.sorted_idx[min(lane, M - 1)];
    }
    int rk[4];
    int64_t of[4], of2[4];
    const bool small = L <= 4 * kWave;
    if (small) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (q * kWave < L) {            // one load per 64 slots and lane
                const int j = min(q * kWave + lane, L - 1);
                rk[q] = va.rank[j];
                of[q] = offs[j];
                of2[q] = va.offs2 ? va.offs2[j] : 0;
            } else {
                rk[q] = 0;
                of[q] = 0;
                of2[q] = 0;
            }
        }
    }
    if (va.ids) {
        const WaveGroups g = wave_group(token_bucket(tl, p.enabled, L), M, L);
        int n;
        wave_segment(g, s, &v.p0, &n, &v.id);
        v.nseg = g.nseg;
        v.tl = g.key & 63;
        p1 = v.p0 + n;
    }
    // lane t: token at sorted position p0 + t
    v.tl = __shfl(v.tl, (v.p0 + lane) & (kWave - 1), kWave);
    const int id = (v.id < 0 || v.id >= L) ? 0 : v.id;   // never index past the table
    if (small) {
        // id is the same in every lane: the entry is read with readlane
        const int q = id / kWave, src = id % kWave;
        const int r_sel = q == 0 ? rk[0] : q == 1 ? rk[1] : q == 2 ? rk[2] : rk[3];
        const int64_t o_sel = q == 0 ? of[0] : q == 1 ? of[1] : q == 2 ? of[2] : of[3];
        v.rp = __builtin_amdgcn_readlane(r_sel, src);
        const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)o_sel, src);
        const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)o_sel >> 32), src);
        v.off = (int64_t)(((uint64_t)hi << 32) | lo);
        const int64_t o2 = q == 0 ? of2[0] : q == 1 ? of2[1] : q == 2 ? of2[2] : of2[3];
        const uint32_t lo2 = __builtin_amdgcn_readlane((uint32_t)o2, src);
        const uint32_t hi2 = __builtin_amdgcn_readlane((uint32_t)((uint64_t)o2 >> 32), src);
        v.off2 = (int64_t)(((uint64_t)hi2 << 32) | lo2);
    } else {
        v.rp = va.rank[id];
        v.off = offs[id];
        v.off2 = va.offs2 ? va.offs2[id] : 0;
    }
    // token id of the segment's t-th token (lane t reads token tl of lane t)
    v.tok = va.tokens ? __shfl(tk, v.tl & (kWave - 1), kWave) : 0;
    v.ms = p1 - v.p0;
    if (kTableChecks && !va.ids && s < v.nseg) {
        // a segment of the table must name a slot and lie inside the batch
        const bool seg_ok = v.id >= 0 && v.id < L && v.p0 >= 0 && v.ms >= 0 && p1 <= M;
        const bool tok_ok = lane >= v.ms || (v.tl >= 0 && v.tl < M);
        if (table_fault(p.err, !(seg_ok && tok_ok))) v.id = -1;
    }
    return v;
}

// Slot mode (ids mode with L <= M <= 64, so that the launch has units for
// every slot): units are numbered compactly over the slots the batch uses.
// Every workgroup loads the ids and, one slot per lane, every slot's rank and
// weight offset in one batch of loads; from the token buckets it knows which
// slots have tokens, and a prefix sum over the slots gives each working unit
// its slot.  Producer unit u is the u-th of the (16-row A block, K chunk)
// pairs of the used slots in slot order, so the working producers take the
// lowest workgroup ids, one per compute unit while there are at most 256 of
// them: a second producer on a compute unit queues its weight loads behind
// the first one's (measured: the producers of the last used slots, which had
// landed on compute units already holding working producers, finished about
// 1 us after the rest).  Units past the work exit at once.  Consumer units
// stay numbered slot-major (consumer unit u serves slot u / n_groups): a
// consumer needs only its own slot's rank and offset, two scalar loads, and
// the compact numbering's extra reductions delayed the B loads of the
// wide-output consumers.  The weight loads are issued before the slot's token
// list (slot_tokens) is formed.
struct SlotTable {
    int rk;             // lane s < L: rank of slot s
    int64_t off;        // lane s < L: weight offset of slot s
    uint64_t used;      // bit s: slot s has a token and a non-zero rank
};

__device__ __forceinline__ SlotTable slot_table_load(const ViewArgs& va) {
    const int j = min(lane_id(), va.L - 1);
    return SlotTable{va.rank[j], va.offs[j], 0ull};
}

// b: this lane's token bucket (L for none).  Slots are at most 64 here.
__device__ __forceinline__ void slot_table_used(SlotTable& t, int b, int M, int L) {
    const int lane = lane_id();
    const bool in = lane < M && b < L;
    const uint32_t lo = wave_or(in && b < 32 ? 1u << (b & 31) : 0u);
    const uint32_t hi = wave_or(in && b >= 32 ? 1u << (b & 31) : 0u);
    const uint64_t has = ((uint64_t)hi << 32) | lo;
    t.used = __ballot(lane < L && ((has >> lane) & 1ull) && t.rk > 0);
}

__device__ __forceinline__ void slot_pick(const SlotTable& t, int s, SegView& v) {
    v.id = s;
    v.rp = __builtin_amdgcn_readlane(t.rk, s);
    v.off = readlane64(t.off, s);
}

// Producer unit u: slot, 16-row block jb and K chunk c; false past the work.
__device__ __forceinline__ bool slot_producer(const SlotTable& t, int u, int per_block, SegView& v,
                                              int* jb, int* c, int C) {
    const int lane = lane_id();
    const int units = ((t.used >> lane) & 1ull) ? (t.rk / 16) * per_block : 0;
    const int incl = wave_incl_scan(units);
    const unsigned long long past = __ballot(incl > u);
    if (past == 0ull) return false;
    const int s = __ffsll((long long)past) - 1;
    const int n = __builtin_amdgcn_readlane(units, s);
    const int local = u - (__builtin_amdgcn_readlane(incl, s) - n);
    if (local < 0 || local >= n) return false;    // never taken when the scan is right
    slot_pick(t, s, v);
    *jb = local / C;
    *c = local % C;
    return true;
}

// The token list of slot s (b: this lane's token bucket) without grouping
// the whole batch: one ballot marks the slot's tokens, and one lane permute
// puts the t-th of them (ascending token index: the stable order) in lane t.
// The first sorted position is the number of tokens with a smaller bucket.
__device__ __forceinline__ void slot_tokens(int b, int M, SegView& v) {
    const int lane = lane_id();
    const bool valid = lane < M;
    const unsigned long long mine = __ballot(valid && b == v.id);
    v.p0 = __popcll(__ballot(valid && b < v.id));
    v.ms = __popcll(mine);
    const int below = __popcll(mine & ((1ull << lane) - 1ull));
    const bool in = (mine >> lane) & 1ull;
    // members go to lanes 0 .. ms-1 in order, the others to ms .. 63
    const int dst = in ? below : v.ms + (lane - below);
    v.tl = __builtin_amdgcn_ds_permute(dst * 4, lane);
}

// ---------------------------------------------------------------- producers
// Unit = (segment, 16 rows of A, K chunk of 512 x dec_steps values).  Wave w owns rows
// 4w..4w+3; per step a lane loads 8 consecutive K values of each row (one
// 16-byte load, 1 KB contiguous per row and wave) and of each token row, and
// accumulates row x token partial dot products in fp32.  One wavefront
// reduction per (row, token) at the end.
constexpr int kTokGroup = 4;                    // token rows accumulated together

// 8 consecutive elements kept in their storage form (one or two 16-byte words)
template <typename T> struct Raw8 { uint4 q[sizeof(T) / 2]; };

template <typename T>
__device__ __forceinline__ Raw8<T> ld_raw8_if(const T* p, bool ok, const T* safe) {
    Raw8<T> r;
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 2); ++i) r.q[i] = ld16_if(p + i * (16 / (int)sizeof(T)), ok, safe);
    return r;
}

template <typename T>
__device__ __forceinline__ void raw_to_f(const Raw8<T>& r, float* o) {
    if constexpr (sizeof(T) == 2) {
        const uint32_t w[4] = {r.q[0].x, r.q[0].y, r.q[0].z, r.q[0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    } else {
        o[0] = __uint_as_float(r.q[0].x); o[1] = __uint_as_float(r.q[0].y);
        o[2] = __uint_as_float(r.q[0].z); o[3] = __uint_as_float(r.q[0].w);
        o[4] = __uint_as_float(r.q[1].x); o[5] = __uint_as_float(r.q[1].y);
        o[6] = __uint_as_float(r.q[1].z); o[7] = __uint_as_float(r.q[1].w);
    }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// c + sum of 8 products; bf16 pairs go through v_dot2_f32_bf16 (products of
// two bf16 values are exact in fp32, the sums are fp32)
template <typename T>
__device__ __forceinline__ float dot8(const Raw8<T>& a, const Raw8<T>& b, float c) {
    if constexpr (sizeof(T) == 2) {
        c = dot2_bf16(a.q[0].x, b.q[0].x, c);
        c = dot2_bf16(a.q[0].y, b.q[0].y, c);
        c = dot2_bf16(a.q[0].z, b.q[0].z, c);
        c = dot2_bf16(a.q[0].w, b.q[0].w, c);
        return c;
    } else {
        float af[8], bf[8];
        raw_to_f(a, af);
        raw_to_f(b, bf);
#pragma unroll
        for (int e = 0; e < 8; ++e) c += af[e] * bf[e];
        return c;
    }
}

// wave steps of 512 K values per producer unit (1024 K values)
// K values; A stays in registers for the whole unit
template <typename T> constexpr int dec_steps() { return 2; }

template <typename T>
__device__ __forceinline__ void dec_produce(const DecodeParams& p, const ViewArgs& va, int unit,
                                            uint32_t tag) {
    constexpr int ST = dec_steps<T>();
    const LinearArgs& a = p.a;
    const int per_s = p.jb_max * p.C;
    int s = unit / per_s;
    int jb = (unit % per_s) / p.C;
    int c = unit % p.C;
    SegView v;
    int b = 0;
    if (p.by_slot) {
        const TokenLoad tl = load_token(va.ids, p.enabled, va.M, va.L);
        SlotTable st = slot_table_load(va);
        b = token_bucket(tl, p.enabled, va.L);
        slot_table_used(st, b, va.M, va.L);
        if (!slot_producer(st, unit, a.n_sl * p.C, v, &jb, &c, p.C)) return;
        s = v.id;
    } else {
        v = seg_view(p, va, s);
        if (s >= v.nseg || v.id < 0) return;
    }
    const int nb = v.rp / 16;
    if (nb == 0 || jb >= nb * a.n_sl) return;
    const int sl = jb / nb, jj = jb % nb;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int kbase = c * ST * 512 + lane * 8;
    const T* A = reinterpret_cast<const T*>(a.A) + v.off +
                 (int64_t)(sl * v.rp + jj * 16 + wave * 4) * a.K;
    // A rows of every step, issued together
    Raw8<T> ar[ST][4];
#pragma unroll
    for (int st = 0; st < ST; ++st) {
        const int k = kbase + st * 512;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ar[st][i] = ld_raw8_if(A + (int64_t)i * a.K + k, k < a.K, A);
        }
    }
    if (p.by_slot) slot_tokens(b, va.M, v);
    const T* X = reinterpret_cast<const T*>(p.x);
    for (int t0 = 0; t0 < v.ms; t0 += kTokGroup) {
        float acc[kTokGroup][4];
#pragma unroll
        for (int u = 0; u < kTokGroup; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[u][i] = 0.f;
        int mrow[kTokGroup];
#pragma unroll
        for (int u = 0; u < kTokGroup; ++u) mrow[u] = __shfl(v.tl, (t0 + u) & (kWave - 1), kWave);
#pragma unroll
        for (int st = 0; st < ST; ++st) {
            const int k = kbase + st * 512;
            Raw8<T> xr[kTokGroup];
#pragma unroll
            for (int u = 0; u < kTokGroup; ++u) {
                xr[u] = ld_raw8_if(X + (int64_t)mrow[u] * p.ldx + k, k < a.K && t0 + u < v.ms, X);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int u = 0; u < kTokGroup; ++u) acc[u][i] = dot8<T>(ar[st][i], xr[u], acc[u][i]);
            }
        }
#pragma unroll
        for (int u = 0; u < kTokGroup; ++u) {
            if (t0 + u >= v.ms) break;
            // rows 0..3 summed over the wavefront (DPP row sums, then the four
            // row totals); lane i < 4 writes row i
            const float r0 = wave_total(acc[u][0]), r1 = wave_total(acc[u][1]);
            const float r2 = wave_total(acc[u][2]), r3 = wave_total(acc[u][3]);
            const float tot = lane == 0 ? r0 : lane == 1 ? r1 : lane == 2 ? r2 : r3;
            if (lane < 4)
                slot_put(slot_at(p, c, v.p0 + t0 + u, sl * a.r_max + jj * 16 + wave * 4 + lane), tot,
                         tag);
        }
    }
}

// bf16 producers on MFMA.  Same unit; wave w takes K values
// [256 w, 256 w + 256) of the chunk in 8 steps of v_mfma_f32_16x16x32_bf16
// with the segment's tokens (up to 16 at a time, missing ones zero) as the
// first operand and the unit's 16 A rows as the second, so the reduction
// over K happens inside the matrix core.  The four waves' 16 x 16 partials
// are added in LDS in a fixed order and written to the exchange slots.
__device__ __forceinline__ void dec_produce_mfma(const DecodeParams& p, const ViewArgs& va, int unit,
                                                 float* red, uint32_t tag) {
    const LinearArgs& a = p.a;
    const int per_s = p.jb_max * p.C;
    int s = unit / per_s;
    int jb = (unit % per_s) / p.C;
    int c = unit % p.C;
    SegView v;
    int b = 0;
    if (p.by_slot) {
        const TokenLoad tl = load_token(va.ids, p.enabled, va.M, va.L);
        SlotTable st = slot_table_load(va);
        b = token_bucket(tl, p.enabled, va.L);
        slot_table_used(st, b, va.M, va.L);
        if (!slot_producer(st, unit, a.n_sl * p.C, v, &jb, &c, p.C)) return;
        s = v.id;
    } else {
        v = seg_view(p, va, s);
        if (s >= v.nseg || v.id < 0) return;
    }
    const int nb = v.rp / 16;
    if (nb == 0 || jb >= nb * a.n_sl) return;
    const int sl = jb / nb, jj = jb % nb;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int lr = lane % 16, lq = lane / 16;
    const int kw = c * 1024 + wave * 256 + lq * 8;          // this lane's first K value
    const uint16_t* A = reinterpret_cast<const uint16_t*>(a.A) + v.off +
                        (int64_t)(sl * v.rp + jj * 16 + lr) * a.K;
    const uint16_t* X = reinterpret_cast<const uint16_t*>(p.x);
    uint4 av[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) av[kk] = ld16_if(A + kw + kk * 32, kw + kk * 32 < a.K, A);
    if (p.by_slot) slot_tokens(b, va.M, v);
    for (int t0 = 0; t0 < v.ms; t0 += 16) {
        const int nt = min(16, v.ms - t0);
        const int m = __shfl(v.tl, t0 + min(lr, nt - 1), kWave);
        const uint16_t* xp = X + (int64_t)m * p.ldx;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        uint4 xv[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) xv[kk] = ld16_if(xp + kw + kk * 32, lr < nt && kw + kk * 32 < a.K, X);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) acc = mfma_bf16(xv[kk], av[kk], acc);
        // acc[q]: token 4 lq + q, A row lr
#pragma unroll
        for (int q = 0; q < 4; ++q) red[(wave * 16 + lq * 4 + q) * 16 + lr] = acc[q];
        __syncthreads();
        {
            const int tok = threadIdx.x / 16, row = threadIdx.x % 16;
            if (tok < nt) {
                const float sum = (red[(0 * 16 + tok) * 16 + row] + red[(1 * 16 + tok) * 16 + row]) +
                                  (red[(2 * 16 + tok) * 16 + row] + red[(3 * 16 + tok) * 16 + row]);
                // one slot, read by every consumer of the slice
                slot_put(slot_at(p, c, v.p0 + t0 + tok, sl * a.r_max + jj * 16 + row), sum, tag);
            }
        }
        __syncthreads();     // red is rewritten by the next token group
    }
}

// ---------------------------------------------------------------- consumers
constexpr int kPollBatch = 8;    // exchange slots polled together

// S of a segment's tokens for slice sl: each element is the sum of its
// K-chunk partials in chunk order, polled kPollBatch exchange slots at a
// time until each carries the launch's tag; written to LDS (bf16 tables: as
// a hi / lo pair, rows of LORA_MAX_RANK values).  False when a wait ran out
// (the error word is set by the caller).
template <typename T>
__device__ __forceinline__ bool collect_S(const DecodeParams& p, const SegView& v, int sl,
                                          uint32_t tag, uint4* lds) {
    constexpr int SLD = LORA_MAX_RANK;
    const int rp = v.rp;
    uint16_t* sHi = reinterpret_cast<uint16_t*>(lds);
    uint16_t* sLo = sHi + LORA_DECODE_MAX_M * SLD;
    float* sS = reinterpret_cast<float*>(lds);
    const int64_t cstride = (int64_t)LORA_DECODE_MAX_M * p.a.cols;
    bool ok = true;
    const uint32_t want = tag ^ p.wc.poll_xor;
    for (int e = threadIdx.x; e < v.ms * rp; e += kDecThreads) {
        const int t = e / rp, j = e % rp;
        const slot_t* sp = slot_at(p, 0, v.p0 + t, sl * p.a.r_max + j);
        float acc = 0.f;
        for (int c0 = 0; c0 < p.C; c0 += kPollBatch) {
            slot_t w[kPollBatch];
            for (int spin = 0;; ++spin) {
                bool all = true;
#pragma unroll
                for (int q = 0; q < kPollBatch; ++q)
                    w[q] = c0 + q < p.C ? slot_load(sp + (c0 + q) * cstride) : ((slot_t)want << 32);
#pragma unroll
                for (int q = 0; q < kPollBatch; ++q) all = all && slot_full(w[q], want);
                if (all) break;
                if (!ok || spin >= p.wc.max_spin) {
                    ok = false;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
#pragma unroll
            for (int q = 0; q < kPollBatch; ++q)
                if (c0 + q < p.C && slot_full(w[q], want)) acc += __uint_as_float((uint32_t)w[q]);
        }
        if constexpr (sizeof(T) == 2) {
            const uint32_t h = f32_to_bf16(acc);
            sHi[t * SLD + j] = (uint16_t)h;
            sLo[t * SLD + j] = (uint16_t)f32_to_bf16(acc - bf16_to_f32(h));
        } else {
            sS[t * SLD + j] = acc;
        }
    }
    return ok;
}

// `first`: the consumer's first tile (find the tokens, collect S, which then
// stays in LDS for its later tiles).
template <typename T, int RCAP>
__device__ __forceinline__ void dec_consume(const DecodeParams& p, SegView& v, int b, int sl,
                                            int n0, int n1, uint4* lds, bool first,
                                            uint32_t tag) {
    constexpr int EPC = 16 / (int)sizeof(T);   // elements per 16-byte chunk
    constexpr int CPR = RCAP / EPC;            // 16-byte chunks of a B row
    constexpr int SLD = LORA_MAX_RANK;         // row stride of S in LDS (elements)
    const LinearArgs& a = p.a;
    const int rp = v.rp;
    const int tid = threadIdx.x;
    const T* B = reinterpret_cast<const T*>(a.B) + v.off;
    T* Y = reinterpret_cast<T*>(p.y);
    // thread t owns output column n0 + t and keeps that column's B row
    // (rank values 0..rp-1) in registers; rows and columns that do not exist
    // are clamped into range and their results never stored
    const int n_out = n0 + tid;
    const bool nin = n_out < n1;
    const int n_ld = min(n_out, n1 - 1);
    // 1. B row and the y values this thread will update, issued before any wait
    uint4 brow[CPR];
#pragma unroll
    for (int q = 0; q < CPR; ++q) {
        const T* src = B + (int64_t)n_ld * rp + min(q * EPC, rp - EPC);
        brow[q] = p.tokens ? ld16(src) : ld16_nt(src);
    }
    if (first && p.by_slot) slot_tokens(b, a.M, v);   // b: this lane's token bucket
    float yv[kTokGroup];
#pragma unroll
    for (int u = 0; u < kTokGroup; ++u) {
        const int m = __builtin_amdgcn_readlane(v.tl, min(u, v.ms - 1));
        yv[u] = Io<T>::ld(Y + (int64_t)m * p.ldy + n_ld);
    }
    // 2. S of the segment's tokens for this slice: sum of the K-chunk partials,
    //    polled kPollBatch slots at a time, into LDS (bf16: as a hi / lo pair)
    uint16_t* sHi = reinterpret_cast<uint16_t*>(lds);
    uint16_t* sLo = sHi + LORA_DECODE_MAX_M * SLD;
    float* sS = reinterpret_cast<float*>(lds);
    bool ok = true;
    if (first && p.tokens) {
        // embedding lookup: the S row of sorted position p0 + t is row `tok`
        // of the adapter's transposed A table; wave w takes tokens w, w + 4, ...
        // (the token is wave-uniform, so it is read with readlane)
        const T* At = reinterpret_cast<const T*>(a.A) + v.off2;
        const int lane = lane_id();
        for (int t = tid / kWave; t < v.ms; t += kDecWaves) {
            const int tok = __builtin_amdgcn_readlane(v.tok, t);
            const bool on = tok >= 0 && tok < a.K;
            if (lane < rp) {
                const float val = on ? Io<T>::ld(At + (int64_t)tok * rp + lane) : 0.f;
                if constexpr (sizeof(T) == 2) {
                    sHi[t * SLD + lane] = (uint16_t)f32_to_bf16(val);   // exact: val is bf16
                    sLo[t * SLD + lane] = 0;
                } else {
                    sS[t * SLD + lane] = val;
                }
            }
        }
    }
    if (first) {
        if (!p.tokens) ok = collect_S<T>(p, v, sl, tag, lds);
        if (!ok) atomicOr(p.err, kErrSpin);
        __syncthreads();
    }
    // 3. delta of column n for each token: B row . S row (read by every lane
    //    at the same LDS address, a broadcast)
    auto delta = [&](int t) {
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < CPR; ++q) {
            if (q * EPC >= rp) break;
            if constexpr (sizeof(T) == 2) {
                const uint4 h = *reinterpret_cast<const uint4*>(sHi + t * SLD + q * 8);
                const uint4 l = *reinterpret_cast<const uint4*>(sLo + t * SLD + q * 8);
                acc = dot2_bf16(brow[q].x, h.x, acc);
                acc = dot2_bf16(brow[q].y, h.y, acc);
                acc = dot2_bf16(brow[q].z, h.z, acc);
                acc = dot2_bf16(brow[q].w, h.w, acc);
                acc = dot2_bf16(brow[q].x, l.x, acc);
                acc = dot2_bf16(brow[q].y, l.y, acc);
                acc = dot2_bf16(brow[q].z, l.z, acc);
                acc = dot2_bf16(brow[q].w, l.w, acc);
            } else {
                const float4 sv = *reinterpret_cast<const float4*>(sS + t * SLD + q * 4);
                acc += __uint_as_float(brow[q].x) * sv.x + __uint_as_float(brow[q].y) * sv.y +
                       __uint_as_float(brow[q].z) * sv.z + __uint_as_float(brow[q].w) * sv.w;
            }
        }
        return acc;
    };
    //    The first kTokGroup tokens take every prefetched y value before the
    //    first store: the wait for a load counts the stores issued after it,
    //    so a store in between would add its whole latency to the next token.
    //    A looked-up token outside the vocabulary has no delta: its row is
    //    not stored at all.
    auto row_on = [&](int t) {
        if (!p.tokens) return true;
        const int tok = __builtin_amdgcn_readlane(v.tok, t);
        return tok >= 0 && tok < a.K;
    };
    float res[kTokGroup];
#pragma unroll
    for (int u = 0; u < kTokGroup; ++u) {
        if (u >= v.ms) break;
        res[u] = yv[u] + delta(u);
    }
#pragma unroll
    for (int u = 0; u < kTokGroup; ++u) {
        if (u >= v.ms) break;
        const int m = __builtin_amdgcn_readlane(v.tl, u);
        if (nin && row_on(u)) Io<T>::st(Y + (int64_t)m * p.ldy + n_out, res[u]);
    }
    for (int t = kTokGroup; t < v.ms; ++t) {
        const int m = __builtin_amdgcn_readlane(v.tl, t);
        const float old = Io<T>::ld(Y + (int64_t)m * p.ldy + n_ld);
        const float r = old + delta(t);
        if (nin && row_on(t)) Io<T>::st(Y + (int64_t)m * p.ldy + n_out, r);
    }
}

// bf16 consumers for ranks above 16: the deltas of 16 tokens x 64 columns
// per wave as blocks of v_mfma_f32_16x16x32_bf16, the first operand the
// tokens' S rows (hi / lo pair from LDS, zero past the tokens and past rp),
// the second the wave's B rows (lane l: column 16 cb + l % 16, rank values
// 32 t + 8 (l / 16) .. + 8).  acc[cb][q] is token 16 tb + 4 (l / 16) + q of
// column n0 + 64 w + 16 cb + l % 16.  For a segment with several tokens this
// replaces 2 rp dot products per token and column by a few MFMAs per wave.
template <int RCAP>
__device__ __forceinline__ void dec_consume_mfma(const DecodeParams& p, SegView& v, int b, int sl,
                                                 int n0, int n1, uint4* lds, bool first,
                                                 uint32_t tag) {
    constexpr int NT = RCAP / 32;              // 32-wide rank steps
    constexpr int SLD = LORA_MAX_RANK;
    const LinearArgs& a = p.a;
    const int rp = v.rp;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int lr = lane % 16, lq = lane / 16;
    const uint16_t* B = reinterpret_cast<const uint16_t*>(a.B) + v.off;
    uint16_t* Y = reinterpret_cast<uint16_t*>(p.y);
    // 1. B operands (clamped into the row and the slice: positions past rp
    //    meet zero S values, columns past n1 are never stored), then the y
    //    values of the first 16 tokens, issued before any wait
    uint4 bop[4][NT];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const int n = min(n0 + wave * 64 + cb * 16 + lr, n1 - 1);
#pragma unroll
        for (int t = 0; t < NT; ++t) bop[cb][t] = ld16_nt(B + (int64_t)n * rp + min(t * 32 + lq * 8, rp - 8));
    }
    if (first && p.by_slot) slot_tokens(b, a.M, v);   // b: this lane's token bucket
    auto token_row = [&](int u) {                  // the segment's u-th token
        return __shfl(v.tl, min(u, v.ms - 1), kWave);
    };
    float yv[4][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int m = token_row(lq * 4 + q);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int n = min(n0 + wave * 64 + cb * 16 + lr, n1 - 1);
            yv[cb][q] = bf16_to_f32(Y[(int64_t)m * p.ldy + n]);
        }
    }
    // 2. S of the segment's tokens (first tile only; it stays in LDS)
    if (first) {
        const bool ok = collect_S<uint16_t>(p, v, sl, tag, lds);
        if (!ok) atomicOr(p.err, kErrSpin);
        __syncthreads();
    }
    // 3. deltas, 16 tokens at a time, and the y update
    const uint16_t* sHi = reinterpret_cast<const uint16_t*>(lds);
    const uint16_t* sLo = sHi + LORA_DECODE_MAX_M * SLD;
    for (int tb = 0; tb * 16 < v.ms; ++tb) {
        f32x4_t acc[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t * 32 >= rp) break;
            const int row = tb * 16 + lr, k = t * 32 + lq * 8;
            const uint32_t m = opaque_mask(row < v.ms && k < rp);
            const uint4 h0 = *reinterpret_cast<const uint4*>(sHi + min(row, LORA_DECODE_MAX_M - 1) * SLD + min(k, SLD - 8));
            const uint4 l0 = *reinterpret_cast<const uint4*>(sLo + min(row, LORA_DECODE_MAX_M - 1) * SLD + min(k, SLD - 8));
            const uint4 h = make_uint4(h0.x & m, h0.y & m, h0.z & m, h0.w & m);
            const uint4 l = make_uint4(l0.x & m, l0.y & m, l0.z & m, l0.w & m);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                acc[cb] = mfma_bf16(h, bop[cb][t], acc[cb]);
                acc[cb] = mfma_bf16(l, bop[cb][t], acc[cb]);
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int u = tb * 16 + lq * 4 + q;
            const int m = token_row(u);
            if (u >= v.ms) continue;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const int n = n0 + wave * 64 + cb * 16 + lr;
                if (n >= n1) continue;
                uint16_t* yp = Y + (int64_t)m * p.ldy + n;
                const float old = tb == 0 ? yv[cb][q] : bf16_to_f32(*yp);
                *yp = (uint16_t)f32_to_bf16(old + acc[cb][q]);
            }
        }
    }
}

// ---------------------------------------------------------------- pipelined runs
// bf16 consumers that walk several tiles (the vocabulary-wide LM head): while
// tile k's deltas are formed and stored, tile k+1's B operands and y values
// are already loading into a second register set.  B and y go through buffer
// resources (an offset past the resource reads zeros and drops a store), so a
// tile's loads and stores are all issued without a branch and the compiler's
// memory-counter waits are exact: waiting for tile k+1's loads does not also
// wait for tile k's stores.  A run past its last tile loads nothing.  The
// MFMA form walks 128-column half tiles (wave w: 32 columns), so that two
// register sets take what one 256-column set did.  Tokens past the first 16
// (MFMA form) or kTokGroup (dot-product form) of a segment take ordinary
// loads and stores after the pipelined part.  Requires y rows within 2 GiB
// of p.y (M * ldy * 2 bytes) and B blocks under 2 GiB (checked by the
// launcher).
struct DecBuf {
    __amdgpu_buffer_rsrc_t b, y;
    int rp, ldy;
};

__device__ __forceinline__ uint32_t y_off(const DecBuf& d, int m, int n, bool on) {
    return on ? (uint32_t)(m * d.ldy + n) * 2u : kBufOff;
}

template <int NT> struct MfmaTile {
    uint4 b[2][NT];
    float y[2][4];
};

template <int NT>
__device__ __forceinline__ void mfma_tile_b(const DecBuf& d, int n0, int n1, bool on,
                                            MfmaTile<NT>& R) {
    const int lane = lane_id(), wave = threadIdx.x / kWave, lr = lane % 16, lq = lane / 16;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const int n = min(n0 + wave * 32 + cb * 16 + lr, n1 - 1);
#pragma unroll
        for (int t = 0; t < NT; ++t)
            R.b[cb][t] = buf_ld16(d.b, on ? (uint32_t)(n * d.rp + min(t * 32 + lq * 8, d.rp - 8)) * 2u
                                          : kBufOff);
    }
}

template <int NT>
__device__ __forceinline__ void mfma_tile_y(const DecBuf& d, const SegView& v, int n0, int n1,
                                            bool on, MfmaTile<NT>& R) {
    const int lane = lane_id(), wave = threadIdx.x / kWave, lr = lane % 16, lq = lane / 16;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int m = __shfl(v.tl, min(lq * 4 + q, v.ms - 1), kWave);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const int n = min(n0 + wave * 32 + cb * 16 + lr, n1 - 1);
            R.y[cb][q] = bf16_to_f32(buf_ld_u16(d.y, y_off(d, m, n, on)));
        }
    }
}

template <int NT>
__device__ __forceinline__ void mfma_tile_out(const DecodeParams& p, const DecBuf& d,
                                              const SegView& v, int n0, int n1, const uint4* lds,
                                              const MfmaTile<NT>& R) {
    constexpr int SLD = LORA_MAX_RANK;
    const int lane = lane_id(), wave = threadIdx.x / kWave, lr = lane % 16, lq = lane / 16;
    const uint16_t* sHi = reinterpret_cast<const uint16_t*>(lds);
    const uint16_t* sLo = sHi + LORA_DECODE_MAX_M * SLD;
    uint16_t* Y = reinterpret_cast<uint16_t*>(p.y);
    for (int tb = 0; tb * 16 < v.ms; ++tb) {
        f32x4_t acc[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t * 32 >= d.rp) break;
            const int row = tb * 16 + lr, k = t * 32 + lq * 8;
            const uint32_t m = opaque_mask(row < v.ms && k < d.rp);
            const uint4 h0 = *reinterpret_cast<const uint4*>(sHi + min(row, LORA_DECODE_MAX_M - 1) * SLD + min(k, SLD - 8));
            const uint4 l0 = *reinterpret_cast<const uint4*>(sLo + min(row, LORA_DECODE_MAX_M - 1) * SLD + min(k, SLD - 8));
            const uint4 h = make_uint4(h0.x & m, h0.y & m, h0.z & m, h0.w & m);
            const uint4 l = make_uint4(l0.x & m, l0.y & m, l0.z & m, l0.w & m);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                acc[cb] = mfma_bf16(h, R.b[cb][t], acc[cb]);
                acc[cb] = mfma_bf16(l, R.b[cb][t], acc[cb]);
            }
        }
        if (tb == 0) {
            // the first 16 tokens: y values from registers, every store issued
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int u = lq * 4 + q;
                const int m = __shfl(v.tl, min(u, v.ms - 1), kWave);
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    const int n = n0 + wave * 32 + cb * 16 + lr;
                    buf_st_u16((uint16_t)f32_to_bf16(R.y[cb][q] + acc[cb][q]), d.y,
                               y_off(d, m, n, u < v.ms && n < n1));
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int u = tb * 16 + lq * 4 + q;
                const int m = __shfl(v.tl, min(u, v.ms - 1), kWave);
                if (u >= v.ms) continue;
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    const int n = n0 + wave * 32 + cb * 16 + lr;
                    if (n >= n1) continue;
                    uint16_t* yp = Y + (int64_t)m * p.ldy + n;
                    *yp = (uint16_t)f32_to_bf16(bf16_to_f32(*yp) + acc[cb][q]);
                }
            }
        }
    }
}

// dot-product form (ranks up to 16): thread t owns column n0 + t
template <int CPR> struct DotTile {
    uint4 b[CPR];
    float y[kTokGroup];
};

template <int CPR>
__device__ __forceinline__ void dot_tile_b(const DecBuf& d, int n0, int n1, bool on, DotTile<CPR>& R) {
    const int n = min(n0 + (int)threadIdx.x, n1 - 1);
#pragma unroll
    for (int q = 0; q < CPR; ++q)
        R.b[q] = buf_ld16(d.b, on ? (uint32_t)(n * d.rp + min(q * 8, d.rp - 8)) * 2u : kBufOff);
}

template <int CPR>
__device__ __forceinline__ void dot_tile_y(const DecBuf& d, const SegView& v, int n0, int n1,
                                           bool on, DotTile<CPR>& R) {
    const int n = min(n0 + (int)threadIdx.x, n1 - 1);
#pragma unroll
    for (int u = 0; u < kTokGroup; ++u) {
        const int m = __builtin_amdgcn_readlane(v.tl, min(u, v.ms - 1));
        R.y[u] = bf16_to_f32(buf_ld_u16(d.y, y_off(d, m, n, on)));
    }
}

template <int CPR>
__device__ __forceinline__ void dot_tile_out(const DecodeParams& p, const DecBuf& d,
                                             const SegView& v, int n0, int n1, const uint4* lds,
                                             const DotTile<CPR>& R) {
    constexpr int SLD = LORA_MAX_RANK;
    const uint16_t* sHi = reinterpret_cast<const uint16_t*>(lds);
    const uint16_t* sLo = sHi + LORA_DECODE_MAX_M * SLD;
    uint16_t* Y = reinterpret_cast<uint16_t*>(p.y);
    const int n_out = n0 + (int)threadIdx.x;
    const bool nin = n_out < n1;
    const int n_ld = min(n_out, n1 - 1);
    auto delta = [&](int t) {
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < CPR; ++q) {
            if (q * 8 >= d.rp) break;
            const uint4 h = *reinterpret_cast<const uint4*>(sHi + t * SLD + q * 8);
            const uint4 l = *reinterpret_cast<const uint4*>(sLo + t * SLD + q * 8);
            acc = dot2_bf16(R.b[q].x, h.x, acc);
            acc = dot2_bf16(R.b[q].y, h.y, acc);
            acc = dot2_bf16(R.b[q].z, h.z, acc);
            acc = dot2_bf16(R.b[q].w, h.w, acc);
            acc = dot2_bf16(R.b[q].x, l.x, acc);
            acc = dot2_bf16(R.b[q].y, l.y, acc);
            acc = dot2_bf16(R.b[q].z, l.z, acc);
            acc = dot2_bf16(R.b[q].w, l.w, acc);
        }
        return acc;
    };
#pragma unroll
    for (int u = 0; u < kTokGroup; ++u) {
        const int m = __builtin_amdgcn_readlane(v.tl, min(u, v.ms - 1));
        const float r = R.y[u] + delta(min(u, v.ms - 1));
        buf_st_u16((uint16_t)f32_to_bf16(r), d.y, y_off(d, m, n_out, nin && u < v.ms));
    }
    for (int t = kTokGroup; t < v.ms; ++t) {
        const int m = __builtin_amdgcn_readlane(v.tl, t);
        const float old = bf16_to_f32(Y[(int64_t)m * p.ldy + n_ld]);
        const float r = old + delta(t);
        if (nin) Y[(int64_t)m * p.ldy + n_out] = (uint16_t)f32_to_bf16(r);
    }
}

// The run over the columns [c0, c1) of slice sl in tiles of kW columns.
// The first two tiles' loads are issued before the wait for S (B first, then
// the segment's tokens are found and the y values loaded); afterwards tile
// k+2's loads go out as soon as tile k's deltas are stored, into the
// register set tile k used.  Two tiles per trip, so the sets alternate
// without copies.
template <int kW, typename Tile, typename LoadB, typename LoadY, typename Out>
__device__ __forceinline__ void dec_run(const DecodeParams& p, SegView& v, int b, int sl, int c0,
                                        int c1, uint4* lds, uint32_t tag, LoadB load_b,
                                        LoadY load_y, Out out) {
    const LinearArgs& a = p.a;
    Tile R0, R1;
    auto hi = [&](int n0) { return min(n0 + kW, c1); };
    load_b(c0, hi(c0), true, R0);
    load_b(c0 + kW, hi(c0 + kW), c0 + kW < c1, R1);
    if (p.by_slot) slot_tokens(b, a.M, v);
    load_y(c0, hi(c0), true, R0);
    load_y(c0 + kW, hi(c0 + kW), c0 + kW < c1, R1);
    const bool ok = collect_S<uint16_t>(p, v, sl, tag, lds);
    if (!ok) atomicOr(p.err, kErrSpin);
    __syncthreads();
    for (int n0 = c0;;) {
        out(n0, hi(n0), R0);
        const int n2 = n0 + 2 * kW;
        load_b(n2, hi(n2), n2 < c1, R0);
        load_y(n2, hi(n2), n2 < c1, R0);
        n0 += kW;
        if (n0 >= c1) break;
        out(n0, hi(n0), R1);
        const int n3 = n0 + 2 * kW;
        load_b(n3, hi(n3), n3 < c1, R1);
        load_y(n3, hi(n3), n3 < c1, R1);
        n0 += kW;
        if (n0 >= c1) break;
    }
}

__device__ __forceinline__ void dec_consumer_run(const DecodeParams& p, SegView& v, int b, int sl,
                                                 int tb, int te, uint4* lds, uint32_t tag) {
    const LinearArgs& a = p.a;
    // the rank and the B block are the same in every lane (buffer resources
    // are built from scalar registers)
    const int rp = __builtin_amdgcn_readfirstlane(v.rp);
    const int64_t off = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(v.off >> 32)) << 32) |
                                  (uint32_t)__builtin_amdgcn_readfirstlane((int)v.off));
    const uint32_t b_bytes = (uint32_t)a.slice_off[a.n_sl] * (uint32_t)rp * 2u;
    const DecBuf d{buf_rsrc(reinterpret_cast<const uint16_t*>(a.B) + off, b_bytes),
                   buf_rsrc(p.y, 0x7fffffffu), rp, (int)p.ldy};
    const int c0 = (int)(a.slice_off[sl] + (int64_t)(tb - p.tile_start[sl]) * kNTile);
    const int c1 = (int)min(a.slice_off[sl] + (int64_t)(te - p.tile_start[sl]) * kNTile,
                            a.slice_off[sl + 1]);
    if (rp <= 16) {
        dec_run<kNTile, DotTile<2>>(
            p, v, b, sl, c0, c1, lds, tag,
            [&](int n0, int n1, bool on, DotTile<2>& R) { dot_tile_b<2>(d, n0, n1, on, R); },
            [&](int n0, int n1, bool on, DotTile<2>& R) { dot_tile_y<2>(d, v, n0, n1, on, R); },
            [&](int n0, int n1, const DotTile<2>& R) { dot_tile_out<2>(p, d, v, n0, n1, lds, R); });
    } else if (rp <= 32) {
        dec_run<kNTile / 2, MfmaTile<1>>(
            p, v, b, sl, c0, c1, lds, tag,
            [&](int n0, int n1, bool on, MfmaTile<1>& R) { mfma_tile_b<1>(d, n0, n1, on, R); },
            [&](int n0, int n1, bool on, MfmaTile<1>& R) { mfma_tile_y<1>(d, v, n0, n1, on, R); },
            [&](int n0, int n1, const MfmaTile<1>& R) { mfma_tile_out<1>(p, d, v, n0, n1, lds, R); });
    } else {
        dec_run<kNTile / 2, MfmaTile<2>>(
            p, v, b, sl, c0, c1, lds, tag,
            [&](int n0, int n1, bool on, MfmaTile<2>& R) { mfma_tile_b<2>(d, n0, n1, on, R); },
            [&](int n0, int n1, bool on, MfmaTile<2>& R) { mfma_tile_y<2>(d, v, n0, n1, on, R); },
            [&](int n0, int n1, const MfmaTile<2>& R) { mfma_tile_out<2>(p, d, v, n0, n1, lds, R); });
    }
}

// Ids mode: an id outside [-1, L) is treated as "no adapter" and reported in
// the error word (one wavefront).
__device__ __forceinline__ void report_bad_ids(const DecodeParams& p, const int32_t* ids, int M,
                                               int L) {
    if (!ids || !p.err) return;
    const int lane = lane_id();
    const int id = ids[min(lane, M - 1)];
    if (__ballot(lane < M && (id < -1 || id >= L)) != 0ull && lane == 0) atomicOr(p.err, kErrBadId);
}

// Consumer unit u: segment (or slot) u / n_groups, and G consecutive
// 256-column tiles of one slice; S is collected once, on the first tile.
template <typename T>
__device__ __forceinline__ void dec_consumer(const DecodeParams& p, const ViewArgs& va, int u,
                                             uint4* lds, uint32_t tag) {
    const LinearArgs& a = p.a;
    const int s = u / p.n_groups;
    const int g = u % p.n_groups;
    SegView v;
    int b = 0;
    if (p.by_slot) {
        // consumer units keep the slot-major numbering: slot s's rank and
        // offset are two scalar loads issued with the ids, and one ballot
        // tells whether any token uses it
        const TokenLoad tl = load_token(va.ids, p.enabled, va.M, va.L);
        v.id = s;
        v.rp = va.rank[s];
        v.off = va.offs[s];
        b = token_bucket(tl, p.enabled, va.L);
        if (v.rp == 0 || __ballot(lane_id() < va.M && b == s) == 0ull) return;
    } else {
        v = seg_view(p, va, s);
        if (s >= v.nseg || v.id < 0 || v.rp == 0) return;
    }
    int sl = 0;
    while (sl + 1 < a.n_sl && g >= p.group_start[sl + 1]) ++sl;
    const int tb = p.tile_start[sl] + (g - p.group_start[sl]) * p.G;
    const int te = min(tb + p.G, p.tile_start[sl + 1]);
    if constexpr (sizeof(T) == 2) {
        if (p.pipe && !p.tokens) {
            dec_consumer_run(p, v, b, sl, tb, te, lds, tag);
            return;
        }
    }
    for (int t = tb; t < te; ++t) {
        const int n0 = (int)(a.slice_off[sl] + (int64_t)(t - p.tile_start[sl]) * kNTile);
        const int n1 = (int)min((int64_t)n0 + kNTile, a.slice_off[sl + 1]);
        const bool first = t == tb;
        if (v.rp <= 16)
            dec_consume<T, 16>(p, v, b, sl, n0, n1, lds, first, tag);
        else if constexpr (sizeof(T) == 2) {
            if (p.tokens) {
                if (v.rp <= 32) dec_consume<T, 32>(p, v, b, sl, n0, n1, lds, first, tag);
                else dec_consume<T, 64>(p, v, b, sl, n0, n1, lds, first, tag);
            } else if (v.rp <= 32) {
                dec_consume_mfma<32>(p, v, b, sl, n0, n1, lds, first, tag);
            } else {
                dec_consume_mfma<64>(p, v, b, sl, n0, n1, lds, first, tag);
            }
        } else if (v.rp <= 32)
            dec_consume<T, 32>(p, v, b, sl, n0, n1, lds, first, tag);
        else
            dec_consume<T, 64>(p, v, b, sl, n0, n1, lds, first, tag);
    }
}

template <typename T>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(3))) void k_decode_fused(const int32_t* __restrict__ ids,
                                                             const int32_t* __restrict__ rank,
                                                             const int64_t* __restrict__ a_off,
                                                             const int64_t* __restrict__ b_off,
                                                             int M, int L, DecodeParams p) {
    __shared__ uint4 lds[LORA_DECODE_MAX_M * LORA_MAX_RANK * 4 / 16];   // the segment's S
    if (p.writer && blockIdx.x == gridDim.x - 1) {
        // ids mode: the segment table for later calls on the same batch
        if (threadIdx.x < kWave) {
            const LinearArgs& a = p.a;
            const int b = token_bucket(load_token(p.ids, p.enabled, a.M, a.L), p.enabled, a.L);
            const WaveGroups g = wave_group(b, a.M, a.L);
            write_wave_segments(g, a.M, a.L, p.out.sorted_idx, p.out.seg_indptr,
                                p.out.req_to_lora, p.out.num_segments, p.out.tile_info,
                                p.out.tile_rows, p.out.num_tiles);
            report_bad_ids(p, ids, M, L);
        }
        return;
    }
    const uint32_t tag = launch_tag();
    if ((int)blockIdx.x < p.grid1) {
        const ViewArgs va{ids, rank, a_off, M, L, nullptr, nullptr};
        if constexpr (sizeof(T) == 2)
            dec_produce_mfma(p, va, blockIdx.x, reinterpret_cast<float*>(lds), tag);
        else
            dec_produce<T>(p, va, blockIdx.x, tag);
    } else {
        const ViewArgs va{ids, rank, b_off, M, L, p.tokens, p.tokens ? a_off : nullptr};
        dec_consumer<T>(p, va, blockIdx.x - p.grid1, lds, tag);
    }
    // without a table writer, the first workgroup checks the ids once its
    // own work is done (off the path of its weight loads)
    if (!p.writer && blockIdx.x == 0 && threadIdx.x < kWave) report_bad_ids(p, ids, M, L);
}

static hipError_t launch_decode(DecodeParams& p, unsigned grid, hipStream_t st) {
    const LinearArgs& a = p.a;
    if (a.dtype == LORA_BF16) {
        hipLaunchKernelGGL(k_decode_fused<uint16_t>, dim3(grid), dim3(kDecThreads), 0, st, p.ids,
                           a.rank, a.a_off, a.b_off, a.M, a.L, p);
    } else {
        hipLaunchKernelGGL(k_decode_fused<float>, dim3(grid), dim3(kDecThreads), 0, st, p.ids,
                           a.rank, a.a_off, a.b_off, a.M, a.L, p);
    }
    return hipGetLastError();
}

// Tiles of 256 columns per slice, and consumers of G consecutive tiles of
// one slice each.
static void set_tiles(DecodeParams& p, int G) {
    const LinearArgs& a = p.a;
    int t = 0, g = 0;
    for (int s = 0; s < a.n_sl; ++s) {
        p.tile_start[s] = t;
        p.group_start[s] = g;
        const int nt = (int)((a.slice_off[s + 1] - a.slice_off[s] + kNTile - 1) / kNTile);
        t += nt;
        g += (nt + G - 1) / G;
    }
    p.tile_start[a.n_sl] = t;
    p.group_start[a.n_sl] = g;
    p.n_tiles = t;
    p.G = G;
    p.n_groups = g;
}

hipError_t launch_embedding_decode(const LinearArgs& a, const int32_t* ids,
                                   const int32_t* enabled, const int32_t* tokens,
                                   const SegOut& out, void* y, int64_t ldy, hipStream_t st) {
    DecodeParams p{};
    p.wc = wait_ctl();
    p.a = a;
    p.y = y;
    p.ldy = ldy;
    p.ids = ids;
    p.enabled = ids ? enabled : nullptr;
    p.out = out;
    p.writer = (ids && out.sorted_idx) ? 1 : 0;
    p.tokens = tokens;
    p.C = 0;
    p.jb_max = a.cols / 16;
    p.grid1 = 0;                        // consumers only: S comes from the lookup
    set_tiles(p, 1);
    return launch_decode(p, (unsigned)(a.s_max * p.n_groups + p.writer), st);
}

// Launch size past which consumers take several tiles.  The bf16 kernel
// keeps three workgroups per CU resident (768), but a consumer's tiles run one
// after another (about 3 µs each on the LM head), so sizing the groups to
// stay resident (7 tiles each) measured slower, 33.7 µs, than letting a second
// round of 3-tile consumers start as the first ones finish, 22 µs.
constexpr int kResident = 1536;

hipError_t launch_decode_fused(const LinearArgs& a, const int32_t* ids, const int32_t* enabled,
                               const SegOut& out, const void* x, int64_t ldx, void* y,
                               int64_t ldy, void* ws, int32_t* err, hipStream_t st) {
    DecodeParams p{};
    p.wc = wait_ctl();
    p.a = a;
    p.ids = ids;
    p.enabled = ids ? enabled : nullptr;
    p.out = out;
    p.writer = (ids && out.sorted_idx) ? 1 : 0;
    p.x = x;
    p.ldx = ldx;
    p.y = y;
    p.ldy = ldy;
    p.by_slot = (ids && a.L <= a.s_max) ? 1 : 0;
    const LinearWs L = linear_ws_layout(a.M, a.K, a.cols);
    char* base = reinterpret_cast<char*>(ws);
    p.err = err ? err : &reinterpret_cast<WsHeader*>(base + L.header)->error;
    p.slots = reinterpret_cast<slot_t*>(base + L.slots);
    static_assert(512 * dec_steps<uint16_t>() == kDecKChunk && 512 * dec_steps<float>() == kDecKChunk,
                  "producer K chunk");
    p.C = (a.K + kDecKChunk - 1) / kDecKChunk;
    p.jb_max = a.cols / 16;
    p.grid1 = a.s_max * p.jb_max * p.C;
    // Consumers wait for their producers, so a consumer that is not resident
    // yet starts only when an earlier one has finished.  Wide outputs (a
    // vocabulary-sized LM head) therefore give each consumer G tiles, enough
    // to keep the launch within kResident workgroups; S is collected once per
    // consumer.
    set_tiles(p, 1);
    const int room = kResident - p.grid1 - p.writer;
    const int cons = a.s_max * p.n_tiles;
    if (cons > room) set_tiles(p, room > 0 ? (cons + room - 1) / room : p.n_tiles);
    // Consumers of several tiles walk them pipelined (LM head, 32000 columns,
    // three tiles per consumer: 18.2 against 20.7 µs); one-tile consumers keep
    // the branchy form, which issues only the stores of real tokens (decode:
    // 8.95 against 9.5 µs pipelined).
    p.pipe = (p.G > 1 && (int64_t)a.M * ldy * 2 <= 0x7fffffff &&
              a.slice_off[a.n_sl] * a.r_max * 2 <= 0x7fffffff) ? 1 : 0;
    return launch_decode(p, (unsigned)(p.grid1 + a.s_max * p.n_groups + p.writer), st);
}

}  // namespace mlora
