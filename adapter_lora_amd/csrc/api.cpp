// C ABI entry points: argument checks, workspace layout, launches.
// Nothing here allocates device memory or synchronises (except
// lora_read_device_error, which is documented to synchronise).
#include <dlfcn.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../include/mlora.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace mlora;

namespace {

constexpr size_t kAlign = 256;
inline size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

lora_status from_hip(hipError_t e) { return e == hipSuccess ? LORA_OK : LORA_HIP_ERROR; }

// The sticky error word of a linear workspace (its first word).
int* ws_error(void* workspace) { return &reinterpret_cast<WsHeader*>(workspace)->error; }

// roctx ranges around the entry points that launch work, for profiler
// timelines (rocprofv3 --marker-trace).  Off unless MLORA_ROCTX=1 when the
// first call is made; the roctx library is then looked up at run time, so
// the library has no link dependency on it and a call pays one branch when
// ranges are off.
struct Roctx {
    int (*push)(const char*) = nullptr;
    int (*pop)() = nullptr;
    Roctx() {
        const char* on = getenv("MLORA_ROCTX");
        if (!on || strcmp(on, "1") != 0) return;
        void* h = dlopen("librocprofiler-sdk-roctx.so.1", RTLD_NOW | RTLD_LOCAL);
        if (!h) h = dlopen("libroctx64.so.4", RTLD_NOW | RTLD_LOCAL);
        if (!h) return;
        push = reinterpret_cast<int (*)(const char*)>(dlsym(h, "roctxRangePushA"));
        pop = reinterpret_cast<int (*)()>(dlsym(h, "roctxRangePop"));
        if (!push || !pop) push = nullptr, pop = nullptr;
    }
};

const Roctx& roctx() {
    static const Roctx r;
    return r;
}

class Range {
  public:
    explicit Range(const char* name) : on_(roctx().push != nullptr) {
        if (on_) roctx().push(name);
    }
    ~Range() {
        if (on_) roctx().pop();
    }
    Range(const Range&) = delete;
    Range& operator=(const Range&) = delete;

  private:
    bool on_;
};

int64_t n_total(const lora_weights_t* w) { return w->slice_offsets[w->n_slices]; }

lora_status check_weights(const lora_weights_t* w) {
    if (!w) return LORA_INVALID_ARG;
    if (w->dtype != LORA_F32 && w->dtype != LORA_BF16) return LORA_INVALID_ARG;
    if (w->K <= 0 || w->K % 8 != 0) return LORA_INVALID_ARG;
    if (w->n_slices < 1 || w->n_slices > LORA_MAX_SLICES) return LORA_INVALID_ARG;
    if (w->L < 1 || w->L > LORA_MAX_ADAPTERS) return LORA_INVALID_ARG;
    if (w->r_max < LORA_RANK_ALIGN || w->r_max > LORA_MAX_RANK || w->r_max % LORA_RANK_ALIGN)
        return LORA_INVALID_ARG;
    if (w->slice_offsets[0] != 0) return LORA_INVALID_ARG;
    for (int s = 0; s < w->n_slices; ++s) {
        const int64_t n = w->slice_offsets[s + 1] - w->slice_offsets[s];
        if (n <= 0 || n % 8 != 0) return LORA_INVALID_ARG;
    }
    if (n_total(w) > INT32_MAX) return LORA_UNSUPPORTED;
    if (!w->A || !w->B || !w->a_off || !w->b_off || !w->rank) return LORA_INVALID_ARG;
    if (!aligned16(w->A) || !aligned16(w->B)) return LORA_INVALID_ARG;
    return LORA_OK;
}

lora_status check_segments(const lora_segments_t* seg, const lora_weights_t* w, int M) {
    if (!seg || !seg->sorted_idx || !seg->seg_indptr || !seg->req_to_lora || !seg->num_segments ||
        !seg->tile_info || !seg->tile_rows || !seg->num_tiles)
        return LORA_INVALID_ARG;
    if (seg->L != w->L) return LORA_INVALID_ARG;
    if (seg->max_tiles < lora_tile_capacity(M, w->L)) return LORA_INVALID_ARG;
    return LORA_OK;
}

lora_status check_rows(const void* p, int64_t ld, int64_t width) {
    if (!p || !aligned16(p)) return LORA_INVALID_ARG;
    if (ld < width || ld % 8 != 0) return LORA_INVALID_ARG;
    return LORA_OK;
}

LinearArgs make_args(const lora_weights_t* w, const lora_segments_t* seg, int M) {
    LinearArgs a{};
    a.dtype = w->dtype;
    a.K = w->K;
    a.n_sl = w->n_slices;
    a.L = w->L;
    a.r_max = w->r_max;
    a.M = M;
    a.s_max = std::min(w->L, M);
    a.cols = w->n_slices * w->r_max;
    for (int s = 0; s <= w->n_slices; ++s) a.slice_off[s] = w->slice_offsets[s];
    a.A = w->A;
    a.B = w->B;
    a.a_off = w->a_off;
    a.b_off = w->b_off;
    a.rank = w->rank;
    a.sorted_idx = seg->sorted_idx;
    a.seg_indptr = seg->seg_indptr;
    a.req_to_lora = seg->req_to_lora;
    a.num_segments = seg->num_segments;
    a.tile_info = seg->tile_info;
    a.tile_rows = seg->tile_rows;
    a.num_tiles = seg->num_tiles;
    a.max_tiles = seg->max_tiles;
    return a;
}

LinearWs layout_for(const lora_weights_t* w, int M) {
    return linear_ws_layout(M, w->K, w->n_slices * w->r_max);
}

}  // namespace

namespace mlora {

// header | decode slots [Cd][64][cols] | shrink partials [C][M][cols] |
// S [M][cols], with Cd = ceil(K / kDecKChunk) and C = ceil(K / kKChunk).
// The header and decode region do not depend on M, so calls of any M may
// share one workspace.
LinearWs linear_ws_layout(int M, int K, int cols) {
    LinearWs ws{};
    const size_t C = (size_t)kchunks(K);
    const size_t Cd = (size_t)((K + kDecKChunk - 1) / kDecKChunk);
    size_t off = 0;
    ws.header = off;
    off += up(sizeof(WsHeader));
    ws.slots = off;
    off += up(Cd * LORA_DECODE_MAX_M * (size_t)cols * sizeof(slot_t));
    ws.partial = off;
    off += up(C * (size_t)M * cols * sizeof(float));
    ws.S = off;
    off += up((size_t)M * cols * sizeof(float));
    ws.total = off;
    return ws;
}

MoeWs moe_ws_layout(int L, int mtp, int r, int Kmax) {
    MoeWs ws{};
    // partials: fp32 values per K chunk of kKChunk (fp32 path), or 8-byte
    // tagged exchange slots per K chunk of 1024 (bf16 path)
    const size_t C = (size_t)kchunks(Kmax);
    const size_t C8 = (size_t)(Kmax + 1023) / 1024;
    const size_t rows = (size_t)L * mtp;
    size_t off = 0;
    ws.header = off;
    off += up(sizeof(WsHeader));
    ws.partial = off;
    off += up(std::max(C * sizeof(float), C8 * sizeof(uint64_t)) * rows * r);
    ws.S = off;
    off += up(rows * r * sizeof(float));
    ws.total = off;
    return ws;
}

// Host-side checks of the single-launch decode's arguments other than the
// workspace (w already checked, 0 <= M <= LORA_DECODE_MAX_M).
lora_status fused_decode_check(const lora_weights_t* w, const int32_t* ids, const void* x,
                               int64_t ldx, int32_t M, void* y, int64_t ldy, int32_t* sorted_idx,
                               int32_t* seg_indptr, int32_t* req_to_lora, int32_t* num_segments,
                               int32_t* tile_info, int32_t* tile_rows, int32_t* num_tiles,
                               int32_t max_tiles) {
    lora_status st;
    if (sorted_idx) {
        if (!seg_indptr || !req_to_lora || !num_segments || !tile_info || !tile_rows || !num_tiles)
            return LORA_INVALID_ARG;
        if (max_tiles < lora_tile_capacity(M, w->L)) return LORA_INVALID_ARG;
    }
    if (M == 0) return LORA_OK;
    if (!ids) return LORA_INVALID_ARG;
    if ((st = check_rows(x, ldx, w->K)) != LORA_OK) return st;
    return check_rows(y, ldy, n_total(w));
}

// Launch of the single-launch decode (arguments checked by
// fused_decode_check), shared by lora_fused_decode and its allocation-free
// form; `ws` is an exchange workspace already known to be large enough and
// errors go to `err` (null: the workspace's own error word).
lora_status fused_decode(const lora_weights_t* w, const int32_t* ids,
                         const int32_t* adapter_enabled, const void* x, int64_t ldx, int32_t M,
                         void* y, int64_t ldy, int32_t* sorted_idx, int32_t* seg_indptr,
                         int32_t* req_to_lora, int32_t* num_segments, int32_t* tile_info,
                         int32_t* tile_rows, int32_t* num_tiles, int32_t max_tiles, void* ws,
                         int32_t* err, hipStream_t stream) {
    const bool table = sorted_idx != nullptr;
    if (M == 0) {
        if (!table) return LORA_OK;
        return from_hip(launch_build_segments(nullptr, nullptr, 0, w->L, sorted_idx, seg_indptr,
                                              req_to_lora, num_segments, tile_info, tile_rows,
                                              num_tiles, max_tiles, stream));
    }
    // segment-table fields of the args are unused in ids mode
    lora_segments_t none{};
    LinearArgs a = make_args(w, &none, M);
    const SegOut out{sorted_idx, seg_indptr, req_to_lora, num_segments, tile_info, tile_rows,
                     num_tiles};
    return from_hip(launch_decode_fused(a, ids, adapter_enabled, out, x, ldx, y, ldy, ws, err,
                                        stream));
}

}  // namespace mlora

extern "C" {

int32_t lora_abi_version(void) { return MLORA_ABI_VERSION; }

const char* lora_status_string(lora_status s) {
    switch (s) {
        case LORA_OK: return "ok";
        case LORA_INVALID_ARG: return "invalid argument";
        case LORA_UNSUPPORTED: return "unsupported shape or option";
        case LORA_HIP_ERROR: return "HIP launch error";
    }
    return "unknown status";
}

size_t lora_workspace_size(const lora_weights_t* w, int32_t M) {
    if (check_weights(w) != LORA_OK || M < 0) return 0;
    return layout_for(w, M).total;
}

lora_status lora_workspace_init(void* workspace, size_t bytes, hipStream_t stream) {
    const Range range("lora_workspace_init");
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1))) return LORA_INVALID_ARG;
    return from_hip(launch_fill_zero(workspace, bytes, stream));
}

lora_status lora_read_device_error(void* workspace, int32_t* out, hipStream_t stream) {
    const Range range("lora_read_device_error");
    if (!workspace || !out) return LORA_INVALID_ARG;
    int v = 0;
    hipError_t e = hipMemcpyAsync(&v, workspace, sizeof(int), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return LORA_HIP_ERROR;
    *out = v;
    if (v != 0) {
        e = launch_fill_zero(workspace, sizeof(int), stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return LORA_HIP_ERROR;
    }
    return LORA_OK;
}

lora_status lora_table_plan(int32_t L, const int32_t* ranks, int32_t n_slices, int32_t K,
                            int64_t N_total, int32_t* rank_pad, int64_t* a_off, int64_t* b_off,
                            int64_t* a_elems, int64_t* b_elems) {
    if (L < 1 || L > LORA_MAX_ADAPTERS || !ranks || !rank_pad || !a_off || !b_off || !a_elems ||
        !b_elems)
        return LORA_INVALID_ARG;
    if (n_slices < 1 || n_slices > LORA_MAX_SLICES || K <= 0 || K % 8 || N_total <= 0 ||
        N_total % 8)
        return LORA_INVALID_ARG;
    for (int i = 0; i < L; ++i)
        if (ranks[i] < 0 || ranks[i] > LORA_MAX_RANK) return LORA_INVALID_ARG;
    for (int i = 0; i < L; ++i)
        rank_pad[i] = (ranks[i] + LORA_RANK_ALIGN - 1) / LORA_RANK_ALIGN * LORA_RANK_ALIGN;
    // rank-group major: every slot of padded rank 16, then 32, 48, 64; slots
    // in index order inside a group
    int64_t ao = 0, bo = 0;
    for (int rp = LORA_RANK_ALIGN; rp <= LORA_MAX_RANK; rp += LORA_RANK_ALIGN) {
        for (int i = 0; i < L; ++i) {
            if (rank_pad[i] != rp) continue;
            a_off[i] = ao;
            b_off[i] = bo;
            ao += (int64_t)n_slices * rp * K;
            bo += N_total * rp;
        }
    }
    for (int i = 0; i < L; ++i)
        if (rank_pad[i] == 0) a_off[i] = b_off[i] = 0;
    *a_elems = ao;
    *b_elems = bo;
    return LORA_OK;
}

lora_status lora_pack_adapter(int32_t dtype, int32_t K, int64_t N_total, int32_t n_slices,
                              int32_t rank, int32_t rank_pad, const void* A_src,
                              const void* B_src, void* A_dst, void* B_dst, hipStream_t stream) {
    const Range range("lora_pack_adapter");
    if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_INVALID_ARG;
    if (K <= 0 || N_total <= 0 || n_slices < 1 || n_slices > LORA_MAX_SLICES) return LORA_INVALID_ARG;
    if (rank < 0 || rank > LORA_MAX_RANK) return LORA_INVALID_ARG;
    if (rank_pad != (rank + LORA_RANK_ALIGN - 1) / LORA_RANK_ALIGN * LORA_RANK_ALIGN)
        return LORA_INVALID_ARG;
    if (rank == 0) return LORA_OK;
    if (!A_src || !B_src || !A_dst || !B_dst) return LORA_INVALID_ARG;
    return from_hip(launch_pack_adapter(dtype, K, N_total, n_slices, rank, rank_pad, A_src, B_src,
                                        A_dst, B_dst, stream));
}

int32_t lora_tile_capacity(int32_t M, int32_t L) {
    if (M < 0 || L < 1) return 0;
    return M / LORA_TILE_ROWS + std::min(L, M);
}

lora_status lora_build_segments(const int32_t* ids, const int32_t* adapter_enabled, int32_t M,
                                int32_t L, int32_t* sorted_idx, int32_t* seg_indptr,
                                int32_t* req_to_lora, int32_t* num_segments, int32_t* tile_info,
                                int32_t* tile_rows, int32_t* num_tiles, int32_t max_tiles,
                                hipStream_t stream) {
    const Range range("lora_build_segments");
    if (M < 0 || M > (1 << 24) || L < 1 || L > LORA_MAX_ADAPTERS) return LORA_INVALID_ARG;
    if (!seg_indptr || !req_to_lora || !num_segments || !num_tiles) return LORA_INVALID_ARG;
    if (max_tiles < lora_tile_capacity(M, L)) return LORA_INVALID_ARG;
    if (M > 0 && (!ids || !sorted_idx || !tile_info || !tile_rows)) return LORA_INVALID_ARG;
    return from_hip(launch_build_segments(ids, adapter_enabled, M, L, sorted_idx, seg_indptr,
                                          req_to_lora, num_segments, tile_info, tile_rows,
                                          num_tiles, max_tiles, stream));
}

lora_status lora_shrink(const lora_weights_t* w, const void* x, int64_t ldx, int32_t M,
                        const lora_segments_t* seg, float* S, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
    const Range range("lora_shrink");
    lora_status st = check_weights(w);
    if (st != LORA_OK) return st;
    if (M < 0 || M > (1 << 24)) return LORA_INVALID_ARG;
    if ((st = check_segments(seg, w, M)) != LORA_OK) return st;
    if (M == 0) return LORA_OK;
    if ((st = check_rows(x, ldx, w->K)) != LORA_OK) return st;
    if (!S || !aligned16(S)) return LORA_INVALID_ARG;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
        return LORA_INVALID_ARG;
    if (workspace_bytes < layout_for(w, M).total) return LORA_INVALID_ARG;
    LinearArgs a = make_args(w, seg, M);
    a.err = ws_error(workspace);
    return from_hip(launch_shrink(a, x, ldx, S, workspace, stream));
}

lora_status lora_expand_add(const lora_weights_t* w, const float* S, int32_t M,
                            const lora_segments_t* seg, void* y, int64_t ldy,
                            hipStream_t stream) {
    const Range range("lora_expand_add");
    lora_status st = check_weights(w);
    if (st != LORA_OK) return st;
    if (M < 0 || M > (1 << 24)) return LORA_INVALID_ARG;
    if ((st = check_segments(seg, w, M)) != LORA_OK) return st;
    if (M == 0) return LORA_OK;
    if (!S || !aligned16(S)) return LORA_INVALID_ARG;
    if ((st = check_rows(y, ldy, n_total(w))) != LORA_OK) return st;
    const LinearArgs a = make_args(w, seg, M);
    return from_hip(launch_expand(a, S, y, ldy, stream));
}

lora_status lora_shrink_expand_add(const lora_weights_t* w, const void* x, int64_t ldx,
                                   int32_t M, const lora_segments_t* seg, void* y, int64_t ldy,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const Range range("lora_shrink_expand_add");
    lora_status st = check_weights(w);
    if (st != LORA_OK) return st;
    if (M < 0 || M > (1 << 24)) return LORA_INVALID_ARG;
    if ((st = check_segments(seg, w, M)) != LORA_OK) return st;
    if (M == 0) return LORA_OK;
    if ((st = check_rows(x, ldx, w->K)) != LORA_OK) return st;
    if ((st = check_rows(y, ldy, n_total(w))) != LORA_OK) return st;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
        return LORA_INVALID_ARG;
    const LinearWs L = layout_for(w, M);
    if (workspace_bytes < L.total) return LORA_INVALID_ARG;
    LinearArgs a = make_args(w, seg, M);
    a.err = ws_error(workspace);
    if (M <= LORA_DECODE_MAX_M)
        return from_hip(launch_decode_fused(a, nullptr, nullptr, SegOut{}, x, ldx, y, ldy,
                                            workspace, nullptr, stream));
    float* S = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + L.S);
    hipError_t e = launch_shrink(a, x, ldx, S, workspace, stream);
    if (e != hipSuccess) return LORA_HIP_ERROR;
    return from_hip(launch_expand(a, S, y, ldy, stream));
}

lora_status lora_linear_fused(const lora_weights_t* w, const void* W, int64_t ldw,
                              const void* x, int64_t ldx, int32_t M, const lora_segments_t* seg,
                              void* y, int64_t ldy, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    const Range range("lora_linear_fused");
    lora_status st = check_weights(w);
    if (st != LORA_OK) return st;
    if (w->dtype != LORA_BF16) return LORA_UNSUPPORTED;
    if (M < 0 || M > (1 << 24)) return LORA_INVALID_ARG;
    if ((st = check_segments(seg, w, M)) != LORA_OK) return st;
    if (M == 0) return LORA_OK;
    if ((st = check_rows(W, ldw, w->K)) != LORA_OK) return st;
    if ((st = check_rows(x, ldx, w->K)) != LORA_OK) return st;
    if ((st = check_rows(y, ldy, n_total(w))) != LORA_OK) return st;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
        return LORA_INVALID_ARG;
    const LinearWs L = layout_for(w, M);
    if (workspace_bytes < L.total) return LORA_INVALID_ARG;
    LinearArgs a = make_args(w, seg, M);
    a.err = ws_error(workspace);
    float* S = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + L.S);
    hipError_t e = launch_shrink(a, x, ldx, S, workspace, stream);
    if (e != hipSuccess) return LORA_HIP_ERROR;
    return from_hip(launch_gemm_lora(a, x, ldx, W, ldw, S, y, ldy, stream));
}

lora_status lora_fused_decode(const lora_weights_t* w, const int32_t* ids,
                              const int32_t* adapter_enabled, const void* x, int64_t ldx,
                              int32_t M, void* y, int64_t ldy, int32_t* sorted_idx,
                              int32_t* seg_indptr, int32_t* req_to_lora, int32_t* num_segments,
                              int32_t* tile_info, int32_t* tile_rows, int32_t* num_tiles,
                              int32_t max_tiles, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    const Range range("lora_fused_decode");
    lora_status st = check_weights(w);
    if (st != LORA_OK) return st;
    if (M < 0) return LORA_INVALID_ARG;
    if (M > LORA_DECODE_MAX_M) return LORA_UNSUPPORTED;
    if ((st = fused_decode_check(w, ids, x, ldx, M, y, ldy, sorted_idx, seg_indptr, req_to_lora,
                                 num_segments, tile_info, tile_rows, num_tiles, max_tiles)) !=
        LORA_OK)
        return st;
    if (M > 0 && (!workspace || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) ||
                  workspace_bytes < layout_for(w, M).total))
        return LORA_INVALID_ARG;
    return fused_decode(w, ids, adapter_enabled, x, ldx, M, y, ldy, sorted_idx, seg_indptr,
                        req_to_lora, num_segments, tile_info, tile_rows, num_tiles, max_tiles,
                        workspace, nullptr, stream);
}

lora_status lora_fused_decode_noalloc(const lora_weights_t* w, const int32_t* ids,
                                      const int32_t* adapter_enabled, const void* x, int64_t ldx,
                                      int32_t M, void* y, int64_t ldy, int32_t* sorted_idx,
                                      int32_t* seg_indptr, int32_t* req_to_lora,
                                      int32_t* num_segments, int32_t* tile_info,
                                      int32_t* tile_rows, int32_t* num_tiles, int32_t max_tiles,
                                      int32_t* error_word, hipStream_t stream) {
    const Range range("lora_fused_decode_noalloc");
    lora_status st = check_weights(w);
    if (st != LORA_OK) return st;
    if (M < 0) return LORA_INVALID_ARG;
    if (M > LORA_DECODE_MAX_M) return LORA_UNSUPPORTED;
    // header and exchange slots (M plays no part) must fit the fixed array
    if (layout_for(w, 0).total > (size_t)LORA_NOALLOC_SCRATCH_BYTES) return LORA_UNSUPPORTED;
    if ((st = fused_decode_check(w, ids, x, ldx, M, y, ldy, sorted_idx, seg_indptr, req_to_lora,
                                 num_segments, tile_info, tile_rows, num_tiles, max_tiles)) !=
        LORA_OK)
        return st;
    void* scratch = nullptr;
    if (M > 0 && noalloc_scratch(&scratch) != hipSuccess) return LORA_HIP_ERROR;
    return fused_decode(w, ids, adapter_enabled, x, ldx, M, y, ldy, sorted_idx, seg_indptr,
                        req_to_lora, num_segments, tile_info, tile_rows, num_tiles, max_tiles,
                        scratch, error_word, stream);
}

lora_status lora_pack_embedding_adapter(int32_t dtype, int32_t vocab, int64_t emb, int32_t rank,
                                        int32_t rank_pad, const void* A_src, const void* B_src,
                                        void* A_dst, void* B_dst, hipStream_t stream) {
    const Range range("lora_pack_embedding_adapter");
    if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_INVALID_ARG;
    if (vocab <= 0 || vocab % 8 || emb <= 0 || emb % 8) return LORA_INVALID_ARG;
    if (rank < 0 || rank > LORA_MAX_RANK) return LORA_INVALID_ARG;
    if (rank_pad != (rank + LORA_RANK_ALIGN - 1) / LORA_RANK_ALIGN * LORA_RANK_ALIGN)
        return LORA_INVALID_ARG;
    if (rank == 0) return LORA_OK;
    if (!A_src || !B_src || !A_dst || !B_dst) return LORA_INVALID_ARG;
    return from_hip(launch_pack_embedding_adapter(dtype, vocab, emb, rank, rank_pad, A_src, B_src,
                                                  A_dst, B_dst, stream));
}

lora_status lora_embedding_shrink(const lora_weights_t* w, const int32_t* tokens, int32_t M,
                                  const lora_segments_t* seg, float* S, hipStream_t stream) {
    const Range range("lora_embedding_shrink");
    lora_status st = check_weights(w);
    if (st != LORA_OK) return st;
    if (w->n_slices != 1) return LORA_INVALID_ARG;
    if (M < 0 || M > (1 << 24)) return LORA_INVALID_ARG;
    if ((st = check_segments(seg, w, M)) != LORA_OK) return st;
    if (M == 0) return LORA_OK;
    if (!tokens || !S || !aligned16(S)) return LORA_INVALID_ARG;
    const LinearArgs a = make_args(w, seg, M);
    return from_hip(launch_embedding_shrink(a, tokens, S, stream));
}

lora_status lora_embedding_decode(const lora_weights_t* w, const int32_t* ids,
                                  const int32_t* adapter_enabled, const int32_t* tokens,
                                  int32_t M, void* y, int64_t ldy, int32_t* sorted_idx,
                                  int32_t* seg_indptr, int32_t* req_to_lora,
                                  int32_t* num_segments, int32_t* tile_info, int32_t* tile_rows,
                                  int32_t* num_tiles, int32_t max_tiles, hipStream_t stream) {
    const Range range("lora_embedding_decode");
    lora_status st = check_weights(w);
    if (st != LORA_OK) return st;
    if (w->n_slices != 1) return LORA_INVALID_ARG;
    if (M < 0) return LORA_INVALID_ARG;
    if (M > LORA_DECODE_MAX_M) return LORA_UNSUPPORTED;
    const bool table = sorted_idx != nullptr;
    if (table) {
        if (!seg_indptr || !req_to_lora || !num_segments || !tile_info || !tile_rows || !num_tiles)
            return LORA_INVALID_ARG;
        if (max_tiles < lora_tile_capacity(M, w->L)) return LORA_INVALID_ARG;
    }
    if (M == 0) {
        if (!table) return LORA_OK;
        return from_hip(launch_build_segments(nullptr, nullptr, 0, w->L, sorted_idx, seg_indptr,
                                              req_to_lora, num_segments, tile_info, tile_rows,
                                              num_tiles, max_tiles, stream));
    }
    if (!ids || !tokens) return LORA_INVALID_ARG;
    if ((st = check_rows(y, ldy, n_total(w))) != LORA_OK) return st;
    lora_segments_t none{};
    const LinearArgs a = make_args(w, &none, M);
    const SegOut out{sorted_idx, seg_indptr, req_to_lora, num_segments, tile_info, tile_rows,
                     num_tiles};
    return from_hip(launch_embedding_decode(a, ids, adapter_enabled, tokens, out, y, ldy, stream));
}

// ------------------------------------------------------------------ MoE
int32_t lora_moe_align_capacity(int32_t M, int32_t topk, int32_t E, int32_t block_size_m) {
    if (M < 0 || topk < 1 || E < 1 || block_size_m < 1) return 0;
    const int64_t cap = (int64_t)M * topk + (int64_t)E * (block_size_m - 1);
    const int64_t r = (cap + block_size_m - 1) / block_size_m * block_size_m;
    return r > INT32_MAX ? 0 : (int32_t)r;
}

static lora_status check_align(const lora_moe_align_t* al, int M, int topk, int E) {
    if (!al || !al->sorted_token_ids || !al->expert_ids || !al->ntpp) return LORA_INVALID_ARG;
    const int bs = al->block_size_m;
    if (bs < 16 || bs > 256 || bs % 16) return LORA_INVALID_ARG;
    if (al->max_tokens_padded % bs) return LORA_INVALID_ARG;
    if (al->max_tokens_padded < lora_moe_align_capacity(M, topk, E, bs)) return LORA_INVALID_ARG;
    return LORA_OK;
}

static lora_status check_moe_weights(const lora_moe_weights_t* w) {
    if (!w) return LORA_INVALID_ARG;
    if (w->dtype != LORA_F32 && w->dtype != LORA_BF16) return LORA_INVALID_ARG;
    if (w->L < 1 || w->L > LORA_MAX_ADAPTERS || w->E < 1 || w->E > 256) return LORA_INVALID_ARG;
    if (w->H <= 0 || w->H % 8 || w->I <= 0 || w->I % 8) return LORA_INVALID_ARG;
    if (w->r < LORA_RANK_ALIGN || w->r > LORA_MAX_RANK || w->r % LORA_RANK_ALIGN) return LORA_INVALID_ARG;
    if (!w->A_gu || !w->B_gu || !w->A_d || !w->B_d || !w->adapter_enabled) return LORA_INVALID_ARG;
    if (!aligned16(w->A_gu) || !aligned16(w->B_gu) || !aligned16(w->A_d) || !aligned16(w->B_d))
        return LORA_INVALID_ARG;
    return LORA_OK;
}

lora_status lora_moe_align(const int32_t* topk_ids, const int32_t* ids,
                           const int32_t* adapter_enabled, int32_t M, int32_t topk, int32_t E,
                           int32_t L, int32_t block_size_m, int32_t max_tokens_padded,
                           int32_t* sorted_token_ids, int32_t* expert_ids, int32_t* ntpp,
                           hipStream_t stream) {
    const Range range("lora_moe_align");
    if (M < 0 || topk < 1 || topk > 16 || E < 1 || E > 256 || L < 1 || L > LORA_MAX_ADAPTERS)
        return LORA_INVALID_ARG;
    if ((int64_t)M * topk > (1 << 24)) return LORA_INVALID_ARG;
    if (!adapter_enabled) return LORA_INVALID_ARG;
    if (M > 0 && (!topk_ids || !ids)) return LORA_INVALID_ARG;
    const lora_moe_align_t out{sorted_token_ids, expert_ids, ntpp, max_tokens_padded,
                               block_size_m};
    lora_status st = check_align(&out, M, topk, E);
    if (st != LORA_OK) return st;
    return from_hip(launch_moe_align(topk_ids, ids, adapter_enabled, M, topk, E, L,
                                     sorted_token_ids, expert_ids, ntpp, max_tokens_padded,
                                     block_size_m, stream));
}

size_t lora_moe_workspace_size(const lora_moe_weights_t* w, int32_t max_tokens_padded) {
    if (check_moe_weights(w) != LORA_OK || max_tokens_padded < 0) return 0;
    return moe_ws_layout(w->L, max_tokens_padded, w->r, std::max(w->H, w->I)).total;
}

static MoeArgs make_moe(const lora_moe_weights_t* w, int M, int topk, const lora_moe_align_t* al) {
    MoeArgs a{};
    a.dtype = w->dtype;
    a.L = w->L; a.E = w->E; a.H = w->H; a.I = w->I; a.r = w->r;
    a.shared_outer = w->shared_outer != 0;
    a.M = M; a.topk = topk;
    a.max_tokens_padded = al->max_tokens_padded;
    a.block_size_m = al->block_size_m;
    a.A_gu = w->A_gu; a.B_gu = w->B_gu; a.A_d = w->A_d; a.B_d = w->B_d;
    a.adapter_enabled = w->adapter_enabled;
    a.sorted_token_ids = al->sorted_token_ids;
    a.expert_ids = al->expert_ids;
    a.ntpp = al->ntpp;
    return a;
}

static lora_status moe_delta(const lora_moe_weights_t* w, int which, const void* in, int64_t ld_in,
                             int32_t M, int32_t topk, const lora_moe_align_t* al, void* out,
                             int64_t ld_out, void* ws, size_t ws_bytes, hipStream_t stream) {
    lora_status st = check_moe_weights(w);
    if (st != LORA_OK) return st;
    if (M < 0 || topk < 1 || topk > 16 || (int64_t)M * topk > (1 << 24)) return LORA_INVALID_ARG;
    if ((st = check_align(al, M, topk, w->E)) != LORA_OK) return st;
    if (M == 0) return LORA_OK;
    const int K = which == 0 ? w->H : w->I;
    const int N = which == 0 ? 2 * w->I : w->H;
    if ((st = check_rows(in, ld_in, K)) != LORA_OK) return st;
    if ((st = check_rows(out, ld_out, N)) != LORA_OK) return st;
    if (!ws || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1))) return LORA_INVALID_ARG;
    if (ws_bytes < lora_moe_workspace_size(w, al->max_tokens_padded)) return LORA_INVALID_ARG;
    const MoeArgs a = make_moe(w, M, topk, al);
    return from_hip(launch_moe_delta(a, which, in, ld_in, out, ld_out, ws, stream));
}

lora_status lora_moe_gate_up_add(const lora_moe_weights_t* w, const void* x, int64_t ldx,
                                 int32_t M, int32_t topk, const lora_moe_align_t* align,
                                 void* cache1, int64_t ld1, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    const Range range("lora_moe_gate_up_add");
    return moe_delta(w, 0, x, ldx, M, topk, align, cache1, ld1, workspace, workspace_bytes, stream);
}

lora_status lora_moe_down_add(const lora_moe_weights_t* w, const void* cache2, int64_t ld2,
                              int32_t M, int32_t topk, const lora_moe_align_t* align,
                              void* cache3, int64_t ld3, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    const Range range("lora_moe_down_add");
    return moe_delta(w, 1, cache2, ld2, M, topk, align, cache3, ld3, workspace, workspace_bytes,
                     stream);
}

lora_status lora_moe_silu_and_mul(int32_t dtype, const void* cache1, int64_t ld1, void* cache2,
                                  int64_t ld2, int32_t P, int32_t I, hipStream_t stream) {
    const Range range("lora_moe_silu_and_mul");
    if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_INVALID_ARG;
    if (P < 0 || I <= 0 || I % 8) return LORA_INVALID_ARG;
    if (P == 0) return LORA_OK;
    lora_status st = check_rows(cache1, ld1, 2 * (int64_t)I);
    if (st != LORA_OK) return st;
    if ((st = check_rows(cache2, ld2, I)) != LORA_OK) return st;
    return from_hip(launch_silu_and_mul(dtype, cache1, ld1, cache2, ld2, P, I, stream));
}

lora_status lora_moe_topk_reduce(int32_t dtype, const void* cache3, int64_t ld3,
                                 const float* topk_weights, void* out, int64_t ldo, int32_t M,
                                 int32_t topk, int32_t H, hipStream_t stream) {
    const Range range("lora_moe_topk_reduce");
    if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_INVALID_ARG;
    if (M < 0 || topk < 1 || topk > 16 || H <= 0 || H % 8) return LORA_INVALID_ARG;
    if (M == 0) return LORA_OK;
    if (!topk_weights) return LORA_INVALID_ARG;
    lora_status st = check_rows(cache3, ld3, H);
    if (st != LORA_OK) return st;
    if ((st = check_rows(out, ldo, H)) != LORA_OK) return st;
    return from_hip(launch_topk_reduce(dtype, cache3, ld3, topk_weights, out, ldo, M, topk, H,
                                       stream));
}

}  // extern "C"
