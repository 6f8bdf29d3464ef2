// Internal launch interface between the C ABI layer (api.cpp) and the
// kernels.  Host and device visible; no HIP types beyond hipStream_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mlora.h"
#include "common.hpp"
#include <cstdlib>

namespace mlora {

// The wait control the launches pass (see WaitCtl): the checked library
// reads MLORA_DEBUG_WAIT_FAULT once.
inline WaitCtl wait_ctl() {
#ifdef MLORA_DEBUG
    static const bool fault = [] {
        const char* e = std::getenv("MLORA_DEBUG_WAIT_FAULT");
        return e != nullptr && e[0] == '1';
    }();
    if (fault) return WaitCtl{0x80000000u, 64};
#endif
    return WaitCtl{0u, kMaxSpin};
}


// Dense multi-LoRA call description (validated by api.cpp).
struct LinearArgs {
    int dtype;
    int K;
    int n_sl;
    int L;
    int r_max;      // padded rank bound (multiple of 16)
    int M;
    int s_max;      // segment bound: min(L, M)
    int cols;       // n_sl * r_max: width of one S row
    int64_t slice_off[LORA_MAX_SLICES + 1];
    const void* A;
    const void* B;
    const int64_t* a_off;
    const int64_t* b_off;
    const int32_t* rank;
    const int32_t* sorted_idx;
    const int32_t* seg_indptr;
    const int32_t* req_to_lora;
    const int32_t* num_segments;
    const int32_t* tile_info;   // [max_tiles][4]: segment, adapter, first position, rows
    const int32_t* tile_rows;   // [max_tiles][64]: token index per row, -1 past the rows
    const int32_t* num_tiles;
    int max_tiles;
    int* err;                   // workspace error word (null: none); table checks report here
};

// K columns handled by one shrink work unit (fused decode and MFMA shrink).
constexpr int kKChunk = 512;
// Output columns handled by one expand work unit.
constexpr int kNTile = 256;

inline int kchunks(int K) { return (K + kKChunk - 1) / kKChunk; }

inline int ntiles_total(const LinearArgs& a) {
    int t = 0;
    for (int s = 0; s < a.n_sl; ++s) {
        const int64_t n = a.slice_off[s + 1] - a.slice_off[s];
        t += (int)((n + kNTile - 1) / kNTile);
    }
    return t;
}

// K columns handled by one fused-decode producer unit.
constexpr int kDecKChunk = 1024;

// Workspace layout (bytes from the start), see api.cpp.
struct LinearWs {
    size_t header;      // WsHeader
    size_t slots;       // slot_t[Cd][64][cols] (decode exchange: K chunk, sorted position, S column)
    size_t partial;     // float[C][M][cols]   (MFMA shrink partial sums)
    size_t S;           // float[M][cols]      (S between shrink and expand)
    size_t total;
};

LinearWs linear_ws_layout(int M, int K, int cols);

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);

// rows per tile of the tile schedule
constexpr int kRowTileRows = 64;

// `enabled` (device [L], may be null): a token whose adapter is disabled is
// treated like a token without an adapter.
hipError_t launch_build_segments(const int32_t* ids, const int32_t* enabled, int M, int L,
                                 int32_t* sorted_idx, int32_t* seg_indptr, int32_t* req_to_lora,
                                 int32_t* num_segments, int32_t* tile_info, int32_t* tile_rows,
                                 int32_t* num_tiles, int max_tiles, hipStream_t st);

hipError_t launch_pack_adapter(int dtype, int K, int64_t N, int n_sl, int rank, int rank_pad,
                               const void* A_src, const void* B_src, void* A_dst, void* B_dst,
                               hipStream_t st);

// Embedding adapter: A stored transposed ([vocab, rank_pad]), B as usual.
hipError_t launch_pack_embedding_adapter(int dtype, int vocab, int64_t emb, int rank,
                                         int rank_pad, const void* A_src, const void* B_src,
                                         void* A_dst, void* B_dst, hipStream_t st);

// Segment table outputs of the single-launch decode (all null: not written).
struct SegOut {
    int32_t* sorted_idx;
    int32_t* seg_indptr;
    int32_t* req_to_lora;
    int32_t* num_segments;
    int32_t* tile_info;
    int32_t* tile_rows;
    int32_t* num_tiles;
};

// Fused decode (M <= LORA_DECODE_MAX_M).  With `ids` null the segments come
// from the table in `a`; otherwise every workgroup groups the batch from
// `ids` (and `enabled`, may be null) on chip and one extra workgroup writes
// the segment table into `out` when out.sorted_idx is not null.
// `err`: where errors are reported (null: the workspace's own error word).
hipError_t launch_decode_fused(const LinearArgs& a, const int32_t* ids, const int32_t* enabled,
                               const SegOut& out, const void* x, int64_t ldx, void* y,
                               int64_t ldy, void* ws, int32_t* err, hipStream_t st);

// Checks and launch of the single-launch decode on an exchange workspace
// `ws` known to be large enough (api.cpp); errors go to `err` (null: the
// workspace's own error word).
lora_status fused_decode(const lora_weights_t* w, const int32_t* ids,
                         const int32_t* adapter_enabled, const void* x, int64_t ldx, int32_t M,
                         void* y, int64_t ldy, int32_t* sorted_idx, int32_t* seg_indptr,
                         int32_t* req_to_lora, int32_t* num_segments, int32_t* tile_info,
                         int32_t* tile_rows, int32_t* num_tiles, int32_t max_tiles, void* ws,
                         int32_t* err, hipStream_t stream);

// Device address of the current GPU's fixed decode scratch
// (LORA_NOALLOC_SCRATCH_BYTES, noalloc.hip), looked up once per device.
hipError_t noalloc_scratch(void** out);

// Single-launch embedding decode (M <= LORA_DECODE_MAX_M): the fused decode
// kernel's consumers only, with S rows looked up from the transposed A table
// by token id; segments grouped from `ids` on chip (table written to `out`
// when out.sorted_idx is not null).
hipError_t launch_embedding_decode(const LinearArgs& a, const int32_t* ids,
                                   const int32_t* enabled, const int32_t* tokens,
                                   const SegOut& out, void* y, int64_t ldy, hipStream_t st);

// S (fp32 [M][cols], sorted rows) from x; `ws` holds the partial sums.
hipError_t launch_shrink(const LinearArgs& a, const void* x, int64_t ldx, float* S, void* ws,
                         hipStream_t st);

hipError_t launch_expand(const LinearArgs& a, const float* S, void* y, int64_t ldy,
                         hipStream_t st);

// y = x W^T + S B_i^T per row tile (bf16 MFMA; S fp32 [M][cols], sorted rows).
hipError_t launch_gemm_lora(const LinearArgs& a, const void* x, int64_t ldx, const void* W,
                            int64_t ldw, const float* S, void* y, int64_t ldy, hipStream_t st);

// Embedding lookup: S (fp32 [M][r_max], sorted rows) = rows of the
// transposed A table selected by token id (a.K is the vocabulary).
hipError_t launch_embedding_shrink(const LinearArgs& a, const int32_t* tokens, float* S,
                                   hipStream_t st);

// MoE
struct MoeArgs {
    int dtype;
    int L, E, H, I, r;
    int shared_outer;   // gate_up A and down B: one slot per adapter, shared by the experts
    int M, topk;
    int max_tokens_padded, block_size_m;
    const void* A_gu;
    const void* B_gu;
    const void* A_d;
    const void* B_d;
    const int32_t* adapter_enabled;
    const int32_t* sorted_token_ids;
    const int32_t* expert_ids;
    const int32_t* ntpp;
};

struct MoeWs {
    size_t header;
    size_t partial;     // fp32 [C][L*max_tokens_padded][r], or (bf16) tagged slots [C1024][...][r]
    size_t S;           // float[L*max_tokens_padded][r]
    size_t total;
};

MoeWs moe_ws_layout(int L, int max_tokens_padded, int r, int Kmax);

hipError_t launch_moe_align(const int32_t* topk_ids, const int32_t* ids,
                            const int32_t* adapter_enabled, int M, int topk, int E, int L,
                            int32_t* sorted_token_ids, int32_t* expert_ids, int32_t* ntpp,
                            int max_tokens_padded, int block_size_m, hipStream_t st);

// which = 0: gate/up (x rows = f / topk, K = H, N = 2I); 1: down (rows = f, K = I, N = H)
hipError_t launch_moe_delta(const MoeArgs& a, int which, const void* in, int64_t ld_in,
                            void* out, int64_t ld_out, void* ws, hipStream_t st);

hipError_t launch_silu_and_mul(int dtype, const void* c1, int64_t ld1, void* c2, int64_t ld2,
                               int P, int I, hipStream_t st);

hipError_t launch_topk_reduce(int dtype, const void* c3, int64_t ld3, const float* w, void* out,
                              int64_t ldo, int M, int topk, int H, hipStream_t st);

}  // namespace mlora
