// Device helpers shared by the gfx950 kernels: storage conversion, 16-byte
// vector loads, wavefront reductions, and the tagged fp32 exchange slots
// through which workgroups of one launch hand partial sums to each other.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mlora.h"

namespace mlora {

constexpr int kWave = 64;

// ----------------------------------------------------------------------------
// storage types: float (fp32) and uint16_t holding bfloat16 bits
// ----------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Round to nearest, ties to even.  NaNs stay NaN (quiet bit set).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

template <typename T> struct Io;

template <> struct Io<float> {
    static constexpr int kPer16B = 4;
    __device__ static float ld(const float* p) { return *p; }
    __device__ static void st(float* p, float v) { *p = v; }
    // 8 consecutive elements -> floats
    __device__ static void ld8(const float* p, float* o) {
        const float4 a = *reinterpret_cast<const float4*>(p);
        const float4 b = *reinterpret_cast<const float4*>(p + 4);
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
};

template <> struct Io<uint16_t> {
    static constexpr int kPer16B = 8;
    __device__ static float ld(const uint16_t* p) { return bf16_to_f32(*p); }
    __device__ static void st(uint16_t* p, float v) { *p = (uint16_t)f32_to_bf16(v); }
    __device__ static void ld8(const uint16_t* p, float* o) {
        const uint4 a = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};

// ----------------------------------------------------------------------------
// masked vector loads without branches: the load always happens, from `p`
// when `ok` and otherwise from `safe` (any readable address, e.g. the start
// of the same tensor), and the result is cleared with a bitwise AND whose
// mask the compiler cannot see through.  With a visible condition the
// compiler turns "load, then select on ok" back into a load under an
// exec-mask branch followed by a wait for it, which serialises the loads
// that were meant to be in flight together.
// ----------------------------------------------------------------------------
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ uint32_t opaque_mask(bool ok) {
    uint32_t m = ok ? 0xffffffffu : 0u;
    asm("" : "+v"(m));     // not volatile: equal masks may still be shared
    return m;
}

__device__ __forceinline__ uint4 ld16_if(const void* p, bool ok, const void* safe) {
    const uint4 v = *reinterpret_cast<const uint4*>(ok ? p : safe);
    const uint32_t m = opaque_mask(ok);
    return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

__device__ __forceinline__ uint2 ld8_if(const void* p, bool ok, const void* safe) {
    const uint2 v = *reinterpret_cast<const uint2*>(ok ? p : safe);
    const uint32_t m = opaque_mask(ok);
    return make_uint2(v.x & m, v.y & m);
}

__device__ __forceinline__ float4 ldf4_if(const float* p, bool ok, const float* safe) {
    const uint4 v = ld16_if(p, ok, safe);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                       __uint_as_float(v.w));
}

// ----------------------------------------------------------------------------
// Raw buffer access (gfx9 buffer resource, stride 0): an access at a byte
// offset at or past the resource's size reads zeros and writes nothing, so
// rows and columns outside a tile need neither a branch nor a mask.  With
// every load and store of a loop issued unconditionally the compiler's
// memory counter waits are exact: waiting for one load does not wait for the
// stores and loads issued after it.
// ----------------------------------------------------------------------------
typedef unsigned int u32x4_vt __attribute__((ext_vector_type(4)));
constexpr uint32_t kBufOff = 0x80000000u;         // an offset past every resource used here

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4_vt v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint16_t buf_ld_u16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ void buf_st_u16(uint16_t v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}
// non-temporal (the cache policy's nt bit)
__device__ __forceinline__ void buf_st16_nt(const uint4& v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4_vt w = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, 2);
}

// ----------------------------------------------------------------------------
// bf16 MFMA, 16 x 16 output, K = 32 (v_mfma_f32_16x16x32_bf16).  Lane l
// supplies row (l % 16) of the first operand and column (l % 16) of the
// second, eight consecutive K values starting at 8 * (l / 16) for both; it
// receives rows 4 * (l / 16) + q, q = 0..3, of column l % 16 of the result.
// ----------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_bf16(const uint4& a, const uint4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// bf16 MFMA, 32 x 32 output, K = 16 (v_mfma_f32_32x32x16_bf16).  Lane l
// supplies row (l % 32) of the first operand and column (l % 32) of the
// second, eight consecutive K values starting at 8 * (l / 32) for both; it
// receives rows 8 * (q / 4) + 4 * (l / 32) + q % 4, q = 0..15, of column
// l % 32 of the result.  Issued back to back from one wave per SIMD on 2-8
// accumulators, this form kept the matrix unit near its peak in a probe; the
// 16 x 16 form on 4-16 accumulators did not (0.9-1.5 PFLOP/s).
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16_t mfma32_bf16(const uint4& a, const uint4& b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// ----------------------------------------------------------------------------
// wavefront reductions
// ----------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// 64-bit value of lane `l` (wave-uniform l), as two 32-bit readlanes.
__device__ __forceinline__ int64_t readlane64(int64_t v, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), l);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Sum over each row of 16 lanes, left in every lane of the row, with DPP
// lane swaps (VALU only: swap neighbours, swap pairs, mirror half rows, mirror
// rows).  Fixed order, so the result is deterministic.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xF, 0xF, false));
}

__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_move<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_move<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_move<0x141>(v);   // row_half_mirror
    v += dpp_move<0x140>(v);   // row_mirror
    return v;
}

// Integer forms with the DPP controls as template arguments: lanes a control
// leaves out (row / bank masks) or whose source lies outside the row read 0.
template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF>
__device__ __forceinline__ int dpp_int(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, BANK_MASK, true);
}

// OR over the whole wavefront (wave-uniform): within rows of 16 lanes by
// DPP swaps and mirrors, then the four row results by readlane.
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
    int x = (int)v;
    x |= dpp_int<0xB1>(x);     // quad_perm [1,0,3,2]
    x |= dpp_int<0x4E>(x);     // quad_perm [2,3,0,1]
    x |= dpp_int<0x141>(x);    // row_half_mirror
    x |= dpp_int<0x140>(x);    // row_mirror
    return (uint32_t)(__builtin_amdgcn_readlane(x, 15) | __builtin_amdgcn_readlane(x, 31) |
                      __builtin_amdgcn_readlane(x, 47) | __builtin_amdgcn_readlane(x, 63));
}

// Inclusive prefix sum over the wavefront's lanes (lane i: v_0 + ... + v_i),
// the DPP sequence for GFX9: shifts of 1..3 inside each row, then of 4 and 8
// into the upper banks, then the last lane of a row broadcast into the rows
// above it (rows 1 and 3, then rows 2 and 3).
__device__ __forceinline__ int wave_incl_scan(int v) {
    int x = v + dpp_int<0x111>(v);                 // row_shr:1
    x += dpp_int<0x112>(v);                        // row_shr:2
    x += dpp_int<0x113>(v);                        // row_shr:3
    x += dpp_int<0x114, 0xF, 0xE>(x);              // row_shr:4, banks 1-3
    x += dpp_int<0x118, 0xF, 0xC>(x);              // row_shr:8, banks 2-3
    x += dpp_int<0x142, 0xA>(x);                   // row_bcast:15, rows 1 and 3
    x += dpp_int<0x143, 0xC>(x);                   // row_bcast:31, rows 2 and 3
    return x;
}

// Sum over the whole wavefront, returned as a wave-uniform value.
__device__ __forceinline__ float wave_total(float v) {
    v = row16_sum(v);
    const int b = __builtin_bit_cast(int, v);
    return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 15)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 31))) +
           (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 47)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 63)));
}

// ----------------------------------------------------------------------------
// tagged exchange slots
//
// A slot is one 64-bit word {fp32 value (low), tag (high)} written and read
// with single 64-bit relaxed atomics at agent scope, so the value and its tag
// always travel together: no fence is needed to order data before a flag.
// The tag identifies the launch (launch_tag below): a slot counts as full
// for a launch only when it carries that launch's tag, so slots are never
// emptied after use, and values left by earlier launches (or by a launch
// that gave up waiting) are simply ignored.  Tag 0 never matches, so a
// zeroed workspace holds no full slot.
// ----------------------------------------------------------------------------
typedef unsigned long long slot_t;

__device__ __forceinline__ void slot_put(slot_t* s, float v, uint32_t tag) {
    const slot_t w = ((slot_t)tag << 32) | (slot_t)__float_as_uint(v);
    __hip_atomic_store(s, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ slot_t slot_load(const slot_t* s) {
    return __hip_atomic_load(s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool slot_full(slot_t w, uint32_t tag) { return (uint32_t)(w >> 32) == tag; }

// The dispatch's packet index on its hardware queue (a user SGPR set by the
// command processor for every dispatch, graph replays included).
extern "C" __device__ uint64_t mlora_dispatch_id() __asm("llvm.amdgcn.dispatch.id");

// Tag of this launch: the dispatch index mixed with the queue's address,
// reduced to [1, 2^32 - 1].  Consecutive dispatches on one queue get
// different tags (for 2^32 - 1 dispatches), and equal dispatch indices on two
// queues get different tags unless the two queue addresses happen to
// collide in 32 bits.  Wave-uniform; scalar arithmetic only.
__device__ __forceinline__ uint32_t launch_tag() {
    const uint64_t id = mlora_dispatch_id();
    const uint64_t q = (uint64_t)(uintptr_t)__builtin_amdgcn_queue_ptr() >> 6;
    const uint64_t h = id + q * 0x9E3779B97F4A7C15ull;
    return (uint32_t)(h % 0xffffffffull) + 1u;
}

__device__ __forceinline__ int atomic_add_agent(int* p, int v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void atomic_store_agent(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workspace header shared by every kernel that uses a workspace (256 bytes).
struct WsHeader {
    int error;        // sticky error bits (LORA_DEVERR_*), first word: read by the host
    int pad[63];
};
static_assert(sizeof(WsHeader) == 256, "workspace header size");

constexpr int kErrSpin = LORA_DEVERR_WAIT;
constexpr int kErrBadId = LORA_DEVERR_BAD_ID;

// Device-side checks of the segment table handed to the table-form calls,
// compiled in only when the library is built with MLORA_DEBUG.
#ifdef MLORA_DEBUG
constexpr bool kTableChecks = true;
#else
constexpr bool kTableChecks = false;
#endif

// Wave-uniform call: true when any lane found a bad entry, which is then
// reported once in `err` (may be null).
__device__ __forceinline__ bool table_fault(int* err, bool bad) {
    if (!kTableChecks) return false;
    const bool any = __ballot(bad) != 0ull;
    if (any && err && lane_id() == 0) atomicOr(err, LORA_DEVERR_TABLE);
    return any;
}
constexpr int kMaxSpin = 1 << 20;

// Control of the bounded waits on exchange slots: a poll expects the
// launch's tag XOR poll_xor, and a wait gives up after max_spin polls.  The
// launches pass {0, kMaxSpin}, except in the checked library (MLORA_DEBUG)
// run with MLORA_DEBUG_WAIT_FAULT=1 in the environment: then every poll
// misses and gives up after 64 tries, which exercises the LORA_DEVERR_WAIT
// path with kernels that still end normally.
struct WaitCtl {
    uint32_t poll_xor;
    int max_spin;
};

}  // namespace mlora
