// gdn_internal.h -- shared internals of libgdn: block-record layout, small device
// helpers and the launcher declarations.  Not part of the public ABI (include/gdn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stddef.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

// ---------------------------------------------------------------------------
// Block record.  gdn_verify_block writes it, gdn_commit consumes it.
//
//   [0, 256)            RecHeader (one per record)
//   ctrl                RecCtrl[B]                  per-instance error bits
//   flags               uint32 [B][H][kCommitSlices] pending-block flags, one per
//                                                   commit workgroup
//   G                   fp32 [B][T][H]              log-decay prefix sums of the block
//   delta               fp32 [B][T][H][dv]          the block's delta rows
//   kcopy               in_dt [B][T][H][dk]         the block's keys
//
// Each section starts on a 256-byte boundary.  Since the verify never writes S,
// S itself is the block checkpoint; with delta and k the commit rebuilds
//   S_n = exp(G_n) S + sum_{j<=n} exp(G_n - G_j) delta_j k_j^T.
// Every commit workgroup owns one flag, which the verify sets and the commit
// checks and clears, so the commit needs no coordination between workgroups.
// ---------------------------------------------------------------------------
constexpr uint32_t kRecMagic = 0x52444E47u;   // "GDNR": header written by a verify
constexpr uint32_t kRecValid = 0x444C4156u;   // "VALD": a block is pending for that workgroup
constexpr int kCommitRows = 32;               // value rows per commit workgroup
constexpr int kCommitSlices = 4;              // flags per (instance, head): 128 / kCommitRows

struct RecHeader {
    uint32_t magic;
    int32_t T, B, H, dk, dv, in_dt;
    uint32_t reserved[9];
};
static_assert(sizeof(RecHeader) == 64, "record header is 64 bytes");

struct RecCtrl {
    uint32_t err;    // GDN_REC_* bits left by the last commit attempt
    uint32_t pad[3];
};
static_assert(sizeof(RecCtrl) == 16, "record control word is 16 bytes");

struct RecLayout {
    size_t ctrl, flags, G, delta, kcopy, total;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline RecLayout rec_layout(int B, int T, int H, int dk, int dv, int esize) {
    RecLayout r;
    r.ctrl = 256;
    r.flags = r.ctrl + align256(size_t(B) * sizeof(RecCtrl));
    r.G = r.flags + align256(size_t(B) * H * kCommitSlices * sizeof(uint32_t));
    r.delta = r.G + align256(size_t(B) * T * H * sizeof(float));
    r.kcopy = r.delta + align256(size_t(B) * T * H * dv * sizeof(float));
    r.total = r.kcopy + align256(size_t(B) * T * H * dk * esize);
    return r;
}

inline int esize_of(gdn_in_dtype dt) { return dt == GDN_IN_BF16 ? 2 : 4; }

// ---------------------------------------------------------------------------
// Device helpers.
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte accesses for the recurrent state, which each
// pass reads once and writes once: they should not displace reused data from
// the caches, and they reach a higher HBM rate than plain accesses.
__device__ inline float4 ld_stream(const float *p) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ inline void st_stream(float *p, const float4 &v) {
    __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4 *>(p));
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ inline uint4 ld_stream_u4(const void *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ inline float bf16_bits_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Split eight fp32 values into high and low bf16 parts, both rounded to nearest
// even: hi = bf16(x), lo = bf16(x - hi), so x = hi + lo + r with
// |r| <= 2^-17 |x| (outside the subnormal range).  Two values are converted per
// instruction; hi is widened back from its packed bits (a shift for the low
// half, a mask for the high half) instead of being converted again.
__device__ inline void split8_bf16(const float (&x)[8], bf16x8 &hi, bf16x8 &lo) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t u = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{x[2 * i], x[2 * i + 1]}), bf16x2));
        h[i] = u;
        const float h0 = __uint_as_float(u << 16), h1 = __uint_as_float(u & 0xffff0000u);
        l[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{x[2 * i] - h0, x[2 * i + 1] - h1}), bf16x2));
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// Load 8 consecutive input elements (16 B of bf16 or 32 B of fp32) as fp32.
template <typename TIn> struct In8;
template <> struct In8<float> {
    float4 a, b;
    __device__ inline void load(const float *p) {
        a = *reinterpret_cast<const float4 *>(p);
        b = *reinterpret_cast<const float4 *>(p + 4);
    }
    __device__ inline void store_raw(float *p) const {
        *reinterpret_cast<float4 *>(p) = a;
        *reinterpret_cast<float4 *>(p + 4) = b;
    }
    __device__ inline float get(int e) const {
        return e < 4 ? (&a.x)[e] : (&b.x)[e - 4];
    }
};
template <> struct In8<__hip_bfloat16> {
    uint4 raw;
    __device__ inline void load(const __hip_bfloat16 *p) { raw = *reinterpret_cast<const uint4 *>(p); }
    __device__ inline void store_raw(__hip_bfloat16 *p) const { *reinterpret_cast<uint4 *>(p) = raw; }
    __device__ inline float get(int e) const {
        const uint32_t w = (&raw.x)[e >> 1];
        return bf16_bits_to_f32(uint16_t((e & 1) ? (w >> 16) : (w & 0xffffu)));
    }
};

template <typename TIn> __device__ inline float load1(const TIn *p);
template <> __device__ inline float load1<float>(const float *p) { return *p; }
template <> __device__ inline float load1<__hip_bfloat16>(const __hip_bfloat16 *p) {
    return bf16_bits_to_f32(*reinterpret_cast<const uint16_t *>(p));
}

// ---------------------------------------------------------------------------
// Asynchronous global -> LDS copies.
// ---------------------------------------------------------------------------
// global_load_lds_dwordx4: lane l's 16 bytes from `src` land at LDS byte
// lds_base + 16 l (each lane gathers from its own address).  Issued through
// inline asm so that the compiler, which cannot count these copies precisely,
// does not wait for all of them before every LDS read; the kernels wait for
// them explicitly (s_waitcnt vmcnt) before reading what they copied.
__device__ inline void dma16(const void *src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(src)
                 : "memory", "m0");
}

// 4 bytes per lane (global_load_lds_dword): lane l's word lands at lds_base + 4 l.
__device__ inline void dma4(const void *src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(src)
                 : "memory", "m0");
}

// The same with a uniform 64-bit base in SGPRs and a 32-bit per-lane byte
// offset (the saddr form): no per-lane 64-bit address arithmetic.
// dma16 for data read once (a streaming, non-temporal load).
__device__ inline void dma16_nt(const void *src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(__builtin_amdgcn_readfirstlane(lds_base)),
                 "v"(src)
                 : "memory", "m0");
}
__device__ inline void dma16s(const void *sbase, uint32_t voff, uint32_t lds_base) {
    // Both are wave-uniform by contract; readfirstlane keeps them in SGPRs where
    // the compiler cannot prove it (free when they already are).
    // (readfirstlane returns int: both halves go back through uint32_t before
    // widening, or a low word with bit 31 set would sign-extend over the high.)
    const uint64_t sb = reinterpret_cast<uint64_t>(sbase);
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(sb >> 32)));
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(sb & 0xffffffffu)));
    const uint64_t sbu = (uint64_t(hi) << 32) | uint64_t(lo);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(__builtin_amdgcn_readfirstlane(lds_base)),
                 "v"(voff), "s"(sbu)
                 : "memory", "m0");
}

// dma16s for data read once (a streaming, non-temporal load).
__device__ inline void dma16s_nt(const void *sbase, uint32_t voff, uint32_t lds_base) {
    const uint64_t sb = reinterpret_cast<uint64_t>(sbase);
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(sb >> 32)));
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(sb & 0xffffffffu)));
    const uint64_t sbu = (uint64_t(hi) << 32) | uint64_t(lo);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(__builtin_amdgcn_readfirstlane(lds_base)),
                 "v"(voff), "s"(sbu)
                 : "memory", "m0");
}

__device__ inline uint32_t lds_addr(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void *)p));
}


// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector memory
// operations are outstanding, leaving the other counters unconstrained.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// ---------------------------------------------------------------------------
// Launchers (one per kernel family); each returns a hipError_t.
// ---------------------------------------------------------------------------
hipError_t launch_verify(const float *S, const void *q, const void *k, const void *v,
                         const float *g, const float *beta, int T, gdn_in_dtype dt,
                         const gdn_shape &shp, float *o, void *record, hipStream_t stream);

hipError_t launch_commit(float *S, void *record, const int32_t *n_accepted, int32_t *pos,
                         const gdn_shape &shp, hipStream_t stream);

hipError_t launch_commit_verify(float *S, void *record_prev, const int32_t *n_accepted, int32_t *pos,
                                const void *q, const void *k, const void *v, const float *g,
                                const float *beta, int T, gdn_in_dtype dt, const gdn_shape &shp, float *o,
                                void *record_next, hipStream_t stream);

hipError_t launch_prefill(float *S, const void *q, const void *k, const void *v,
                          const float *g, const float *beta, int L, gdn_in_dtype dt,
                          const gdn_shape &shp, float *o, void *ws, size_t ws_bytes,
                          hipStream_t stream);

// Workspace bytes the two-pass prefill schedule uses for this shape and prompt
// length (0 when the one-pass schedule is the faster one).
size_t prefill_workspace_bytes(const gdn_shape &shp, int L);
size_t accept_workspace_bytes(int B, int T, int V, bool sampled);
// Size of the library's own scratch for gdn_accept_sampled_noalloc (per device).
constexpr size_t kAcceptScratchBytes = size_t(1) << 20;
hipError_t launch_accept_sampled_noalloc(const void *tgt, const void *drf, gdn_in_dtype dt, const int32_t *drafts,
                                         const float *u_acc, const float *u_samp, float inv_tau, int B, int T, int V,
                                         int32_t *n_out, int32_t *next, hipStream_t st);
size_t attn_workspace_bytes(const gdn_attn_shape &s, int T);
hipError_t launch_mixer_verify(const float *S, const gdn_mixer_inputs &in, int T, const gdn_shape &shp, float *y,
                               void *record, hipStream_t stream);
hipError_t launch_mixer_commit_verify(float *S, void *record_prev, const int32_t *n_accepted, int32_t *pos,
                                      const gdn_mixer_inputs &in, int T, const gdn_shape &shp, float *y,
                                      void *record_next, hipStream_t stream);
hipError_t launch_attn_verify(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                              const int32_t *ctx, int T, float scale, const gdn_attn_shape &s, float *o, void *ws,
                              hipStream_t st);
hipError_t launch_accept_greedy(const void *tgt, gdn_in_dtype dt, const int32_t *drafts, int B, int T, int V,
                                int32_t *n_out, int32_t *next, void *ws, hipStream_t st);
hipError_t launch_accept_sampled(const void *tgt, const void *drf, gdn_in_dtype dt, const int32_t *drafts,
                                 const float *u_acc, const float *u_samp, float inv_tau, int B, int T, int V,
                                 int32_t *n_out, int32_t *next, void *ws, hipStream_t st);
hipError_t launch_history_rewind(void *hist, const void *rows, const int32_t *n, int B, int W, int T, int C,
                                 gdn_in_dtype dt, hipStream_t st);

}  // namespace gdn
