// verify.hip -- the verify kernel: outputs of a T-row speculative block from the
// checkpoint state, without writing the state.
//
// A workgroup owns one (instance, head); each of its waves owns 64 value rows,
// whose dv x dk fp32 state is read from HBM exactly once, into registers, and
// never written (the value-column partition of the lithos-metal README, "How it
// works", region table, "GDN mixer" row).  At 128 state registers per lane and
// three waves per SIMD, the 96 MiB state of a 48-layer, 32-head batch is resident
// in the register files at once: every load is issued up front, in one round.  The
// block coefficients depend only on q and k, which arrive first, so they are
// ready before the state is.
//
// Instead of stepping the state T times in registers (about 3T FMA per state
// element), the block is solved in its UT form with chunk = T.  With
// G_t = g_1 + ... + g_t, gamma_t = exp(G_t) and Gamma_tj = exp(G_t - G_j):
//
//   delta_t = beta_t (v_t - gamma_t S k_t) - sum_{j<t} beta_t Gamma_tj (k_t.k_j) delta_j
//   o_t     = gamma_t S q_t + sum_{j<=t} Gamma_tj (q_t.k_j) delta_j
//
// so the state enters only through the 2T projections [K;Q] S^T, one dense
// (2T x dk) x (dk x dv) contraction per head, on MFMA; the VALU is left with
// O(T^2) work per value row.  For bf16 inputs the rows of [K;Q] are exact bf16
// operands and the fp32 state is split into a high and a low bf16 part (two
// v_mfma_f32_16x16x32_bf16 per 32 keys; the dropped residual is below 2^-17 of
// each state element).  For fp32 inputs the contraction runs on fp32 MFMA
// (v_mfma_f32_16x16x4_f32).  The Gram matrix [K;Q] K^T is built the same way
// while the state is still arriving.
#include "gdn_internal.h"

namespace gdn {
namespace {

__device__ inline float comp(const float4 &v, int c) {
    return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
}

// Split eight fp32 values (two float4) into high and low bf16 parts; products
// with exact bf16 operands are exact in the fp32 MFMA accumulator.
__device__ inline void split_bf16(const float4 &a, const float4 &b, bf16x8 &hi, bf16x8 &lo) {
    const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    split8_bf16(x, hi, lo);
}

// bf16 X rows are 2 dk bytes, unpadded, with their 16-byte pieces in swizzled
// order (slot = piece ^ xswz(x)), so that 16 consecutive rows read at one piece
// hit distinct banks.
template <int DK>
__device__ inline int xswz(int x) {
    return DK == 128 ? (x & 15) : ((x >> 1) & 7);
}
template <int DK>
__device__ inline int xoff(int x, int piece) {  // byte offset of piece `piece` of row x
    return x * (2 * DK) + ((piece ^ xswz<DK>(x)) << 4);
}

// A operand row x of the bf16 X for key block p: keys 32p + 8lg .. 32p + 8lg + 7,
// one 16-byte piece (the keys a lane holds in its state registers for that block).
template <int DK>
__device__ inline bf16x8 xrow_bf16(const uint8_t *Xb, int x, int p, int lg) {
    return *reinterpret_cast<const bf16x8 *>(Xb + xoff<DK>(x, 4 * p + lg));
}

// The state's lane layout.  In registers, lane (lr, lg) of a wave holds row lr of
// a 16-row tile at keys 32c + 8lg + {0..7} for each 32-key block c (float4 2c and
// 2c + 1): the B-operand layout of the bf16 MFMA, c being the contraction block.
// In memory, a copy instruction covers 8 rows x 128 bytes: copy (rg, c) of lane l
// is row 8rg + (l & 7), bytes 128c + 16(l >> 3) of the row.  Whole 128-byte lines
// per instruction stream at the copy rate; the 16 rows x 64 bytes that the
// register layout would read directly reached only about three quarters of it on
// the same in-place stream (both measured).  Lane l holds its own row in copy rg
// = (l & 15) / 8 and the row of lane l ^ 8 in the other, at the key quad that lane
// needs: one DPP move (row_ror:8 with a bank mask) per register puts every quad
// in place, and the inverse moves restore the copy layout before a store.
constexpr int kRor8 = 0x128;   // DPP row_ror:8 (lane l reads lane l ^ 8 of its row)
__device__ inline float dpp_ror8(float old, float src, int bank_mask_hi) {
    // bank_mask_hi: lanes 8..15 of each row (true) or lanes 0..7 (false) take src.
    return bank_mask_hi
               ? __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), kRor8, 0xf, 0xc, false))
               : __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), kRor8, 0xf, 0x3, false));
}
// Copy layout (a = copy rg 0, c = copy rg 1 of one 128-byte block) <-> register
// layout (keys + 0..3, keys + 4..7), in place.
// Both directions are the same exchange: lanes 8..15 of a row take the first
// register from the second of lane l ^ 8, lanes 0..7 the second from the first.
__device__ inline void swap_quads(float &a, float &c) {
    const float t = a;
    a = dpp_ror8(a, c, true);
    c = dpp_ror8(c, t, false);
}
__device__ inline void swap_quads(float4 &a, float4 &c) {
    swap_quads(a.x, c.x);
    swap_quads(a.y, c.y);
    swap_quads(a.z, c.z);
    swap_quads(a.w, c.w);
}
// Raw buffer accesses: the descriptor's fourth word for gfx9-family targets, and
// the cache-policy bit of a streaming (non-temporal) access.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kBufferNt = 2;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// Key of component e of state register m of lane group lg (KM registers a row).
__device__ inline int skey(int m, int lg) { return 32 * (m >> 1) + 8 * lg + 4 * (m & 1); }

// The GDN mixer around the recurrence (MIX): the kernel builds q, k, v and the
// gates itself from the layer's raw in-projection rows, and applies the gated
// RMS norm to its outputs.  Per token: a width-4 causal filter over the filter
// history and the block (per channel), SiLU; q and k L2-normalised per head, q
// scaled by 1/sqrt(dk), value head h reading q/k head h / (H / Hk); q, k, v
// rounded to bf16; beta = sigmoid(b), g = -exp(A_log) softplus(a + dt_bias);
// after the recurrence y = o / sqrt(mean(o^2) + eps) * norm_w * SiLU(z).
struct MixArgs {
    const __hip_bfloat16 *x;     // raw rows [B][T][conv_dim], channels q | k | v
    const __hip_bfloat16 *hist;  // filter history [B][3][conv_dim], oldest first
    const float *conv_w;         // [conv_dim][4]
    const float *a, *bg;         // gate pre-activations [B][T][H]
    const float *A_log, *dt_bias;  // [H]
    const __hip_bfloat16 *z;     // output gate [B][T][H][dv]
    const float *norm_w;         // [dv]
    int Hk;                      // q/k heads
};
constexpr float kMixEps = 1e-6f;

// SiLU per element of the mixer, in about a dozen instructions and within about
// 1 ulp: e^-x from the hardware exp2 with the rounding error of -x log2(e)
// (carried in two parts) folded back in to first order, and the reciprocal of
// 1 + e^-x from the hardware estimate refined by one Newton step.  q, k and v
// are rounded to bf16 afterwards: a smaller error moves fewer of them across a
// rounding boundary.  x is clamped at -40 (where x sigmoid(x) is below 2e-16 in
// size) so that no step meets an infinity.
__device__ inline float silu(float x) {
    constexpr float kL2e = 1.44269504f, kL2eLo = 1.925963e-8f, kLn2 = 0.693147181f;
    const float xc = fmaxf(x, -40.f);
    const float t = -xc * kL2e;
    const float lo = fmaf(-xc, kL2eLo, fmaf(-xc, kL2e, -t));   // -xc log2(e) - t
    const float d = 1.f + __builtin_amdgcn_exp2f(t) * fmaf(lo, kLn2, 1.f);
    float r = __builtin_amdgcn_rcpf(d);
    r *= fmaf(-d, r, 2.f);
    return x * r;
}
// 1 / sqrt(a) for a > 0: the hardware estimate and one Newton step.
__device__ inline float rsqrt_nr(float a) {
    const float r = __builtin_amdgcn_rsqf(a);
    return r * fmaf(-0.5f * a * r, r, 1.5f);
}
__device__ inline float softplusf(float x) { return x > 20.f ? x : log1pf(expf(x)); }
__device__ inline uint32_t ldbits(const __hip_bfloat16 *p, size_t i) {
    return reinterpret_cast<const uint16_t *>(p)[i];
}
// Sum over the wave, returned (uniform) to every lane, all in DPP: within each
// row of 16 lanes swap neighbours, swap pairs, mirror within 8 and within 16
// (every lane then holds its row's sum); then lane 15 of rows 0 and 2 is added
// into rows 1 and 3 (row_bcast:15), and lane 31 into rows 2 and 3
// (row_bcast:31), so lane 63 holds the total, read out once.  No LDS round trips,
// unlike a shuffle tree.
template <int CTRL, int ROWS = 0xf> __device__ inline float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xf, false));
}
__device__ inline float wave_sum(float v) {
    v = dpp_add<0xB1>(v);          // quad_perm [1,0,3,2]
    v = dpp_add<0x4E>(v);          // quad_perm [2,3,0,1]
    v = dpp_add<0x141>(v);         // row_half_mirror
    v = dpp_add<0x140>(v);         // row_mirror
    v = dpp_add<0x142, 0xa>(v);    // row_bcast:15 into rows 1 and 3
    v = dpp_add<0x143, 0xc>(v);    // row_bcast:31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// X rows: 0..TM-1 hold k_1..k_TM, TM..2TM-1 hold q_1..q_TM (TM = 8 MT); rows of
// t >= T repeat row T (bf16: finite data nothing reads the results of) or are
// zero (fp32).  MT = number of 16-row MFMA tiles of X (1 for T <= 8, 2 for
// T <= 16).
//
// FUSED: first commit the block pending in record `rprev` at n_acc[b] rows, as
// the commit kernel does (same checks, error bits, flags and pos), applying the
// rank-n update to each state tile as it arrives and writing S_n back; then
// verify the new block from S_n.  Each (instance, head) reads its state once.
//
// NT = 16-row tiles per wave: 4 (a workgroup covers a head's dv rows), or 1 for
// few heads (a workgroup covers 32 rows, dv / 32 workgroups per head, each
// computing the head's block coefficients itself): four times the workgroups,
// a quarter of the state per wave.
//
// MIX: q, k, v and the gates come from the mixer's raw inputs (`mix`) instead of
// q, k, v, g, beta, and the outputs are the gated RMS norm of the recurrence's.
// Occupancy: three waves a SIMD (168 VGPRs) hold the 48-layer state in one round
// of register-resident slices; fp32 inputs (the small-shape path: 8-element
// operand rows and fp32 MFMA operands take more registers) get two (256 VGPRs),
// which keeps them free of scratch spills.
template <typename TIn>
constexpr int verify_waves_per_eu() {
    return sizeof(TIn) == 4 ? 2 : 3;
}

template <int DK, int DV, typename TIn, int MT, bool FUSED, int NT, bool MIX = false>
__global__ __launch_bounds__(DV) __attribute__((amdgpu_waves_per_eu(verify_waves_per_eu<TIn>()))) void verify_kernel(
    float *__restrict__ S, const TIn *__restrict__ q, const TIn *__restrict__ k,
    const TIn *__restrict__ v, const float *__restrict__ g, const float *__restrict__ beta,
    int T, int B, int H, float *__restrict__ o, uint8_t *__restrict__ rec, uint8_t *__restrict__ rprev,
    const int32_t *__restrict__ n_acc, int32_t *__restrict__ pos, MixArgs mix) {
    constexpr int NW = DV / 64;      // waves per workgroup
    constexpr int NTH = 64 * NW;     // threads
    constexpr int RW = 16 * NT;      // value rows per wave
    constexpr int RS = NW * RW;      // value rows per workgroup
    constexpr int SLICES = DV / RS;  // workgroups per head
    constexpr int KM = DK / 16;      // 16-key groups (4 keys per lane group)
    constexpr int XR = 16 * MT;      // rows of X
    constexpr int XS = DK + 4;       // LDS row stride of the fp32 X, floats
    constexpr int TM = 8 * MT;       // largest T for this instantiation
    constexpr int KH = KM / NW;      // key groups per wave for the Gram matrix
    constexpr bool kBf16 = sizeof(TIn) == 2;
    // fp32 inputs: staging pieces per thread (8 elements each).
    constexpr int NCH = (2 * TM * DK / 8 + NTH - 1) / NTH;
    constexpr int NVP = (TM * DV / 8 + NTH - 1) / NTH;
    // bf16 inputs: 1 KiB copy blocks of K (and of Q) and of V.
    constexpr int NBK = TM * DK * 2 / 1024, NBV = TM * DV * 2 / 1024;
    constexpr int NSTATE = NT * KM;  // state loads per thread
    static_assert(NW * 64 == DV && KH * NW == KM && SLICES * RS == DV && RS % kCommitRows == 0, "shape");
    static_assert(!kBf16 || (NBK >= 1 && NBV >= 1 && NSTATE <= 63), "copy blocks");
    static_assert(!MIX || (kBf16 && DK == 128 && DV == 128 && NT == 4), "the mixer: bf16, d = 128, whole heads");

    __shared__ __attribute__((aligned(16))) float X[kBf16 ? 4 : XR * XS];
    __shared__ __attribute__((aligned(16))) uint8_t Xb[kBf16 ? XR * 2 * DK : 16];
    __shared__ __attribute__((aligned(16))) uint8_t Vb[kBf16 ? TM * DV * 2 : 16];   // bf16 [TM][DV]
    __shared__ __attribute__((aligned(16))) float Vs[kBf16 ? 4 : TM * DV];          // fp32 [TM][DV]
    __shared__ __attribute__((aligned(16))) float P[XR][RS + 1];   // [K;Q] S^T: rows x, columns value row (local)
    __shared__ float gpart[NW][XR][XR + 1];       // per-wave partial Gram matrices
    __shared__ float coefM[TM][TM + 1], coefN[TM][TM + 1];
    __shared__ float Gs[TM], gam[TM], bs[TM];
    __shared__ __attribute__((aligned(16))) float graw[64], braw[64];  // g_t, beta_t (t clamped)
    // FUSED: the first (up to) 8 replayed rows of the pending block: delta (then
    // exp(G_n - G_j) delta), its keys (in the pending record's dtype) and G.
    constexpr int CR = 8;
    __shared__ __attribute__((aligned(16))) float cdraw[FUSED ? CR * DV : 4];
    __shared__ __attribute__((aligned(16))) uint8_t kraw[FUSED ? CR * DK * 4 : 16];
    __shared__ __attribute__((aligned(16))) float gprev[FUSED ? 64 : 4];

    const int bh = blockIdx.x / SLICES, slice = blockIdx.x - bh * SLICES;
    const int b = bh / H, h = bh - b * H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int rbase = slice * RS;                 // first value row of the workgroup
    const int fl0 = rbase / kCommitRows;          // its first pending flag (commit slice)
    const RecLayout RL = rec_layout(B, T, H, DK, DV, int(sizeof(TIn)));

    // FUSED: the pending block's status (uniform over the workgroup).  cn rows
    // are committed when ok; cerr is the instance's error bit otherwise.
    int cn = 0, Tp = 1, esp = 2;
    bool cok = false;
    uint32_t cerr = 0;
    RecLayout RLp{};
    if constexpr (FUSED) {
        const RecHeader *hp = reinterpret_cast<const RecHeader *>(rprev);
        if (hp->magic != kRecMagic) {
            cerr = GDN_REC_NO_BLOCK;
        } else {
            Tp = hp->T;
            const int ipd = hp->in_dt;
            if (hp->B != B || hp->H != H || hp->dk != DK || hp->dv != DV || Tp < 1 || Tp > GDN_T_MAX ||
                (ipd != GDN_IN_F32 && ipd != GDN_IN_BF16)) {
                cerr = b < hp->B ? uint32_t(GDN_REC_SHAPE) : 0u;
            } else {
                esp = ipd == GDN_IN_BF16 ? 2 : 4;
                RLp = rec_layout(B, Tp, H, DK, DV, esp);
                const uint32_t *fl = reinterpret_cast<const uint32_t *>(rprev + RLp.flags) + size_t(bh) * kCommitSlices;
                bool valid = true;
#pragma unroll
                for (int sl = 0; sl < RS / kCommitRows; ++sl) valid = valid && fl[fl0 + sl] == kRecValid;
                const int n = n_acc[b];
                if (!valid) {
                    cerr = GDN_REC_NO_BLOCK;
                } else if (n < 0 || n > Tp) {
                    cerr = GDN_REC_N_RANGE;
                } else {
                    cok = true;
                    cn = n;
                }
            }
        }
        cn = __builtin_amdgcn_readfirstlane(cn);
        if (cn > 0) {
            // Copy rows j < min(cn, CR) of delta (DV floats each) and of the keys
            // (DK elements each), clamped to row cn - 1, and G_1..G_Tp.
            const int nr = min(cn, CR);
            const uint8_t *dsrc = rprev + RLp.delta;
            const uint8_t *ksrc = rprev + RLp.kcopy;
            const uint32_t lcd = lds_addr(cdraw), lk = lds_addr(kraw);
            constexpr int DBLK = CR * DV * 4 / 1024;
#pragma unroll
            for (int jj = 0; jj < (DBLK + NW - 1) / NW; ++jj) {
                const int blk = jj * NW + w;
                if (DBLK % NW == 0 || blk < DBLK) {
                    const int byte = blk * 1024 + 16 * lane, j = byte / (4 * DV), pc = byte % (4 * DV);
                    dma16(dsrc + ((size_t(b) * Tp + min(j, nr - 1)) * H + h) * DV * 4 + pc, lcd + blk * 1024);
                }
            }
            const int krow = DK * esp, kblk = CR * krow / 1024;  // 2 or 4 blocks (dk = 128)
            for (int blk = w; blk < kblk; blk += NW) {
                const int byte = blk * 1024 + 16 * lane, j = byte / krow, pc = byte % krow;
                dma16(ksrc + ((size_t(b) * Tp + min(j, nr - 1)) * H + h) * krow + pc, lk + blk * 1024);
            }
            if (w == 0)
                dma4(rprev + RLp.G + ((size_t(b) * Tp + min(lane, Tp - 1)) * H + h) * 4, lds_addr(gprev));
        }
    }

    // Loads, in the order they are consumed; every address is valid (clamped) and
    // no loaded register is touched until it is used, so all of them are in
    // flight together.
    // 1. Gates, copied into LDS (lane t of wave 0 copies g_t and beta_t): a
    //    register load would be sunk by the compiler to its use, behind a wait for
    //    the state.
    [[maybe_unused]] float alog = 0.f, dtb = 0.f;
    if constexpr (MIX) {
        // Raw a_t and b_t (activated once they land, after the state loads are
        // issued).
        if (w == 0) {
            const size_t gi = size_t(b * T + min(lane, T - 1)) * H + h;
            dma4(mix.a + gi, lds_addr(graw));
            dma4(mix.bg + gi, lds_addr(braw));
        }
        alog = mix.A_log[h];
        dtb = mix.dt_bias[h];
    } else if (w == 0) {
        const size_t gi = size_t(b * T + min(lane, T - 1)) * H + h;
        dma4(g + gi, lds_addr(graw));
        dma4(beta + gi, lds_addr(braw));
    }
    // 2. The block's keys, queries and values.  bf16: copied straight into LDS
    //    (1 KiB blocks, round robin over the waves); fp32: 8-element pieces into
    //    registers, staged below.
    In8<TIn> xin[kBf16 ? 1 : NCH], vin[kBf16 ? 1 : NVP];
    // MIX: the head's raw rows (its q, k and v channel segments, 256 bytes each,
    // of the 3 history rows and of the TM block rows, the latter clamped to row
    // T - 1) are copied into LDS, the history rows into Xb and the block rows
    // into P: both are free until the filter has read them (Xb is written after
    // the norm barrier, P in the tile loop).  Thread c later builds channel c of
    // q, k and v for every token.  Its filter taps, and the output gate and norm
    // weight of value row c, are register loads, issued here too; the gates are
    // pinned (an empty asm that claims to change them) in the epilogue.
    [[maybe_unused]] float4 mwt[MIX ? 3 : 1];
    [[maybe_unused]] uint32_t zr[MIX ? TM : 1];
    [[maybe_unused]] float nwr = 0.f;
    constexpr int kRawRow = 3 * 256;    // bytes of a raw row's three segments (dk = dv = 128)
    static_assert(!MIX || TM * kRawRow <= int(sizeof(P)), "block rows fit P");
    static_assert(!MIX || 3 * kRawRow <= XR * 2 * DK, "history rows fit Xb");
    if constexpr (MIX) {
        const int grp = H / mix.Hk, hk = h / grp, c = tid;
        const size_t cdim = size_t(2 * mix.Hk * DK + H * DV);
        const size_t seg0 = size_t(hk) * DK, seg1 = size_t(mix.Hk + hk) * DK, seg2 = size_t(2 * mix.Hk) * DK + size_t(h) * DV;
        // 16-byte piece p of the raw rows: row p / 48, segment (p % 48) / 16,
        // elements 8 (p % 16) ..; 64 pieces per copy instruction.
        constexpr int NPH = 3 * 48;                   // history pieces
        constexpr int NJH = (NPH + 63) / 64, NJX = TM * 48 / 64;   // copy instructions
        const uint32_t lh = lds_addr(Xb), lp = lds_addr(&P[0][0]);
#pragma unroll
        for (int jj = 0; jj < (NJH + NJX + NW - 1) / NW; ++jj) {
            const int j = jj * NW + w;                 // history blocks first, then block rows
            const bool hist = j < NJH;
            const int p = 64 * (hist ? j : j - NJH) + lane, pr = p % 48, u = pr / 16;
            const size_t off = (u == 0 ? seg0 : u == 1 ? seg1 : seg2) + 8 * (pr % 16);
            if (hist) {
                if (p < NPH) dma16(mix.hist + (size_t(b) * 3 + p / 48) * cdim + off, lh + j * 1024);
            } else if (j < NJH + NJX) {
                dma16(mix.x + (size_t(b) * T + min(p / 48, T - 1)) * cdim + off, lp + (j - NJH) * 1024);
            }
        }
        mwt[0] = *reinterpret_cast<const float4 *>(mix.conv_w + (seg0 + c) * 4);
        mwt[1] = *reinterpret_cast<const float4 *>(mix.conv_w + (seg1 + c) * 4);
        mwt[2] = *reinterpret_cast<const float4 *>(mix.conv_w + (seg2 + c) * 4);
        const int i = rbase + RW * w + lane;   // the thread's value row in the epilogue
#pragma unroll
        for (int t = 0; t < TM; ++t) zr[t] = ldbits(mix.z, (size_t(b * T + min(t, T - 1)) * H + h) * DV + i);
        nwr = mix.norm_w[i];
    } else if constexpr (kBf16) {
        const uint32_t lx = lds_addr(Xb), lv = lds_addr(Vb);
        // Block j of K (of Q) holds rows 1024 j / (2 dk) ..; wave w copies blocks
        // w, w + NW, ...  Lane l's piece sits at LDS row r, slot s and comes from
        // token row min(r, T - 1), piece s ^ xswz(row of X).
#pragma unroll
        for (int jj = 0; jj < (NBK + NW - 1) / NW; ++jj) {
            const int j = jj * NW + w;
            if (NBK % NW == 0 || j < NBK) {
                const int byte = j * 1024 + 16 * lane, r = byte / (2 * DK), slot = (byte % (2 * DK)) >> 4;
                const size_t row = (size_t(b * T + min(r, T - 1)) * H + h) * DK;
                dma16(k + row + 8 * (slot ^ xswz<DK>(r)), lx + j * 1024);
                dma16(q + row + 8 * (slot ^ xswz<DK>(TM + r)), lx + TM * 2 * DK + j * 1024);
            }
        }
#pragma unroll
        for (int jj = 0; jj < (NBV + NW - 1) / NW; ++jj) {
            const int j = jj * NW + w;
            if (NBV % NW == 0 || j < NBV) {
                const int byte = j * 1024 + 16 * lane, t = byte / (2 * DV), piece = (byte % (2 * DV)) >> 4;
                dma16(v + (size_t(b * T + min(t, T - 1)) * H + h) * DV + 8 * piece, lv + j * 1024);
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            const int c = min(tid + u * NTH, 2 * T * DK / 8 - 1);
            const int e = c * 8, r = e / DK, col = e - r * DK;
            const bool isk = r < T;
            const int t = isk ? r : r - T;
            xin[u].load((isk ? k : q) + (size_t(b * T + t) * H + h) * DK + col);
        }
#pragma unroll
        for (int u = 0; u < NVP; ++u) {
            const int c = min(tid + u * NTH, T * DV / 8 - 1);
            const int e = c * 8, t = e / DV, col = e - t * DV;
            vin[u].load(v + (size_t(b * T + t) * H + h) * DV + col);
        }
    }
    // Compiler-only barrier: keep the loads above ahead of the state loads, so
    // consuming them never waits for the state.
    asm volatile("" ::: "memory");
    // 3. The wave's state rows, 16-row tile by tile (tile nt: rows RW w + 16nt ..,
    //    copies in the whole-line layout, put into the register layout before use).
    //    The plain verify issues all four tiles at once; the fused kernel keeps two
    //    tiles in flight and issues the next after writing one back, so that its
    //    reads and write-backs share the memory system instead of queueing as a
    //    read phase followed by a write phase.
    constexpr int NPRE = (FUSED || MIX) ? (NT < 2 ? NT : 2) : NT;   // tiles loaded up front
    constexpr int NEARLY = FUSED ? (NPRE < 1 ? NPRE : 1) : 0;          // tiles committed before the Gram
    // The copies go through a buffer descriptor over the wave's RW rows (in scalar
    // registers): lane l's byte offset (row l & 7 of the tile, 16 bytes l >> 3 of a
    // line) in one register and the copy's constant offset in a scalar one, where
    // 64-bit lane addresses would take two registers per copy.
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        S + (size_t(bh) * DV + rbase + RW * w) * DK, 0, RW * DK * 4, kBufferWord3);
    const uint32_t soff = uint32_t(((lane & 7) * DK + 4 * (lane >> 3)) * 4);
    auto scopy = [](int nt, int rg, int c) { return uint32_t(((16 * nt + 8 * rg) * DK + 32 * c) * 4); };
    float4 sreg[NT][KM];
    auto load_tile = [&](int nt) {
#pragma unroll
        for (int c = 0; c < KM / 2; ++c)
#pragma unroll
            for (int rg = 0; rg < 2; ++rg)
                sreg[nt][2 * c + rg] = __builtin_bit_cast(
                    float4, __builtin_amdgcn_raw_buffer_load_b128(srs, soff, scopy(nt, rg, c), kBufferNt));
    };
    auto store_copy = [&](int nt, int rg, int c, const float4 &val) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, val), srs, soff, scopy(nt, rg, c), kBufferNt);
    };
    // The tile's registers into the register layout, once they have landed.
    auto fix_tile = [&](int nt) {
#pragma unroll
        for (int c = 0; c < KM / 2; ++c) {
            swap_quads(sreg[nt][2 * c], sreg[nt][2 * c + 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
#pragma unroll
    for (int nt = 0; nt < NPRE; ++nt) load_tile(nt);

    TIn *kcopy = reinterpret_cast<TIn *>(rec + RL.kcopy);
    // The LDS copies were issued before the NPRE KM state loads; loads complete in
    // order, so once at most that many are outstanding the copies have landed.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(NPRE * KM));
    asm volatile("" ::: "memory");
    if constexpr (MIX) {
        __shared__ float nrm[2][NW][TM];
        const int c = tid;
        __syncthreads();   // every wave's raw-row copies have landed
        asm volatile("" : "+v"(alog), "+v"(dtb));
        if (w == 0) {   // the gates; wave 0 copied them and is their only reader until a barrier
            graw[lane] = -expf(alog) * softplusf(graw[lane] + dtb);
            braw[lane] = 1.f / (1.f + expf(-braw[lane]));   // once per token: the library forms
        }
        float y[3][TM];
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            float xr[TM + 3];
#pragma unroll
            for (int r = 0; r < TM + 3; ++r) {
                const uint8_t *row = r < 3 ? Xb + r * kRawRow : reinterpret_cast<const uint8_t *>(&P[0][0]) + (r - 3) * kRawRow;
                xr[r] = bf16_bits_to_f32(*reinterpret_cast<const uint16_t *>(row + u * 256 + 2 * c));
            }
#pragma unroll
            for (int t = 0; t < TM; ++t)
                y[u][t] = silu(mwt[u].x * xr[t] + mwt[u].y * xr[t + 1] + mwt[u].z * xr[t + 2] + mwt[u].w * xr[t + 3]);
        }
        // L2 norms of q and k per token over the head's dk channels (two waves).
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const float sq = wave_sum(y[0][t] * y[0][t]), sk = wave_sum(y[1][t] * y[1][t]);
            if (lane == 0) {
                nrm[0][w][t] = sq;
                nrm[1][w][t] = sk;
            }
        }
        __syncthreads();
        const float qs = 1.f / sqrtf(float(DK));   // a constant
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int j = 0; j < NW; ++j) {
                sq += nrm[0][j][t];
                sk += nrm[1][j][t];
            }
            const __bf16 qv = static_cast<__bf16>(y[0][t] * (rsqrt_nr(sq + kMixEps) * qs));
            const __bf16 kv = static_cast<__bf16>(y[1][t] * rsqrt_nr(sk + kMixEps));
            const int piece = c >> 3, e2 = (c & 7) * 2;
            *reinterpret_cast<__bf16 *>(Xb + xoff<DK>(t, piece) + e2) = kv;
            *reinterpret_cast<__bf16 *>(Xb + xoff<DK>(TM + t, piece) + e2) = qv;
            reinterpret_cast<__bf16 *>(Vb)[t * DV + c] = static_cast<__bf16>(y[2][t]);
        }
    }
    if constexpr (!kBf16) {
        // Stage X and V (fp32); the piece index is clamped exactly as for the
        // loads: a thread past the end rewrites the last piece with the same data.
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            const int c = min(tid + u * NTH, 2 * T * DK / 8 - 1);
            const int e = c * 8, r = e / DK, col = e - r * DK;
            const int x = r < T ? r : TM + (r - T);
            *reinterpret_cast<float4 *>(X + x * XS + col) =
                make_float4(xin[u].get(0), xin[u].get(1), xin[u].get(2), xin[u].get(3));
            *reinterpret_cast<float4 *>(X + x * XS + col + 4) =
                make_float4(xin[u].get(4), xin[u].get(5), xin[u].get(6), xin[u].get(7));
            if (r < T) xin[u].store_raw(kcopy + (size_t(b * T + r) * H + h) * DK + col);
        }
#pragma unroll
        for (int u = 0; u < NVP; ++u) {
            const int c = min(tid + u * NTH, T * DV / 8 - 1);
            const int e = c * 8, t = e / DV, col = e - t * DV;
            *reinterpret_cast<float4 *>(Vs + t * DV + col) =
                make_float4(vin[u].get(0), vin[u].get(1), vin[u].get(2), vin[u].get(3));
            *reinterpret_cast<float4 *>(Vs + t * DV + col + 4) =
                make_float4(vin[u].get(4), vin[u].get(5), vin[u].get(6), vin[u].get(7));
        }
        for (int idx = tid; idx < 2 * (TM - T) * DK; idx += NTH) {
            const int rr = idx / DK, x = rr < TM - T ? T + rr : TM + T + (rr - (TM - T));
            X[x * XS + idx % DK] = 0.f;
        }
    }
    __syncthreads();
    float gam_n = 1.f;
    if constexpr (FUSED) {
        if (cn > 0) {
            // exp(G_n - G_j) delta_j for the wave's own value rows (lane < RW:
            // row rbase + RW w + lane; wave w is the only reader of them).
            const float Gn = gprev[cn - 1];
            gam_n = expf(Gn);
            if (lane < RW) {
                const int row = rbase + RW * w + lane;
#pragma unroll
                for (int j = 0; j < CR; ++j)
                    if (j < cn) cdraw[j * DV + row] *= expf(Gn - gprev[j]);
            }
        }
    }
    // [K;Q] S^T of state tile nt (register layout) into P.  bf16 inputs: the fp32
    // state is split into bf16 high and low parts against the exact bf16 X (two
    // bf16 MFMAs per 32 keys); fp32 inputs: fp32 MFMA.  The contraction slots visit
    // the same keys in A and B.
    auto products = [&](int nt) {
        f32x4 acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (kBf16) {
#pragma unroll
            for (int p = 0; p < KM / 2; ++p) {
                bf16x8 shi, slo;
                split_bf16(sreg[nt][2 * p], sreg[nt][2 * p + 1], shi, slo);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const bf16x8 a = xrow_bf16<DK>(Xb, 16 * mt + lr, p, lg);
                    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, shi, acc[mt], 0, 0, 0);
                    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, slo, acc[mt], 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int m = 0; m < KM; ++m) {
                float4 a[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    a[mt] = *reinterpret_cast<const float4 *>(X + (16 * mt + lr) * XS + skey(m, lg));
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(comp(a[mt], c), comp(sreg[nt][m], c),
                                                                       acc[mt], 0, 0, 0);
            }
        }
        // Lane (lr, lg) of a 16x16 result tile holds rows 4lg..4lg+3 of column lr.
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) P[16 * mt + 4 * lg + r][RW * w + 16 * nt + lr] = acc[mt][r];
    };
    // FUSED: the commit of state tile nt (in registers), its write-back, and the
    // load of the tile NPRE ahead.  Needs only the pending block's rows, so the
    // first NEARLY tiles are committed before this block's Gram matrix and
    // coefficients, and the state keeps streaming meanwhile.
    auto commit_tile = [&](int nt) {
        fix_tile(nt);
        if (cn > 0) {
            // S_n = exp(G_n) S + sum_{j < n} exp(G_n - G_j) delta_j k_j^T for this
            // tile (row RW w + 16nt + lr, keys skey(m, lg) + {0..3}), written back.
            const int row = rbase + RW * w + 16 * nt + lr;
#pragma unroll
            for (int m = 0; m < KM; ++m) {
                sreg[nt][m].x *= gam_n;
                sreg[nt][m].y *= gam_n;
                sreg[nt][m].z *= gam_n;
                sreg[nt][m].w *= gam_n;
            }
            auto add_row = [&](float c, const float4 (&kv)[KM]) {
#pragma unroll
                for (int m = 0; m < KM; ++m) {
                    sreg[nt][m].x += c * kv[m].x;
                    sreg[nt][m].y += c * kv[m].y;
                    sreg[nt][m].z += c * kv[m].z;
                    sreg[nt][m].w += c * kv[m].w;
                }
            };
            const int nr = min(cn, CR);
            if (esp == 2) {
                // bf16 keys: a lane's 8 keys of block c are consecutive, one 16-byte
                // read, unpacked at the update.
#pragma unroll 1
                for (int j = 0; j < nr; ++j) {
                    uint4 kr[KM / 2];
#pragma unroll
                    for (int c = 0; c < KM / 2; ++c)
                        kr[c] = *reinterpret_cast<const uint4 *>(kraw + (j * DK + skey(2 * c, lg)) * 2);
                    const float cj = cdraw[j * DV + row];
#pragma unroll
                    for (int c = 0; c < KM / 2; ++c) {
                        float4 &lo = sreg[nt][2 * c], &hi = sreg[nt][2 * c + 1];
                        lo.x += cj * __uint_as_float(kr[c].x << 16);
                        lo.y += cj * __uint_as_float(kr[c].x & 0xffff0000u);
                        lo.z += cj * __uint_as_float(kr[c].y << 16);
                        lo.w += cj * __uint_as_float(kr[c].y & 0xffff0000u);
                        hi.x += cj * __uint_as_float(kr[c].z << 16);
                        hi.y += cj * __uint_as_float(kr[c].z & 0xffff0000u);
                        hi.z += cj * __uint_as_float(kr[c].w << 16);
                        hi.w += cj * __uint_as_float(kr[c].w & 0xffff0000u);
                    }
                }
            } else {
#pragma unroll 1
                for (int j = 0; j < nr; ++j) {
                    float4 kv[KM];
#pragma unroll
                    for (int m = 0; m < KM; ++m)
                        kv[m] = *reinterpret_cast<const float4 *>(kraw + (j * DK + skey(m, lg)) * 4);
                    add_row(cdraw[j * DV + row], kv);
                }
            }
            // Rows past CR (blocks longer than 8): straight from the record.
#pragma unroll 1
            for (int j = CR; j < cn; ++j) {
                const size_t rj = (size_t(b) * Tp + j) * H + h;
                const float c = expf(gprev[cn - 1] - reinterpret_cast<const float *>(rprev + RLp.G)[rj]) *
                                reinterpret_cast<const float *>(rprev + RLp.delta)[rj * DV + row];
                float4 kv[KM];
#pragma unroll
                for (int m = 0; m < KM; ++m) {
                    const int key = skey(m, lg);
                    if (esp == 2) {
                        const uint2 r2 = *reinterpret_cast<const uint2 *>(rprev + RLp.kcopy + (rj * DK + key) * 2);
                        kv[m] = make_float4(__uint_as_float(r2.x << 16), __uint_as_float(r2.x & 0xffff0000u),
                                            __uint_as_float(r2.y << 16), __uint_as_float(r2.y & 0xffff0000u));
                    } else {
                        kv[m] = *reinterpret_cast<const float4 *>(rprev + RLp.kcopy + (rj * DK + key) * 4);
                    }
                }
                add_row(c, kv);
            }
            // Stored in the copy layout: swapped, stored and swapped back in place.
#pragma unroll
            for (int c = 0; c < KM / 2; ++c) {
                swap_quads(sreg[nt][2 * c], sreg[nt][2 * c + 1]);
                store_copy(nt, 0, c, sreg[nt][2 * c]);
                store_copy(nt, 1, c, sreg[nt][2 * c + 1]);
                swap_quads(sreg[nt][2 * c], sreg[nt][2 * c + 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (nt + NPRE < NT) load_tile(nt + NPRE);
    };
    if constexpr (FUSED) {
#pragma unroll
        for (int nt = 0; nt < NEARLY; ++nt) commit_tile(nt);
    }
    if (w == 0) {
        // Log-decay prefix sums over the block, in one fixed order (a wave scan);
        // the commit reuses the stored values.  Read by the coefficients after
        // the barrier that follows the Gram matrix.
        const float gv = graw[lane], bv = braw[lane];
        float Gp = lane < T ? gv : 0.f;
#pragma unroll
        for (int off = 1; off < TM; off <<= 1) {
            const float y = __shfl_up(Gp, off, 64);
            if (lane >= off) Gp += y;
        }
        if (lane < T) {
            Gs[lane] = Gp;
            gam[lane] = expf(Gp);
            bs[lane] = bv;
            if (slice == 0) reinterpret_cast<float *>(rec + RL.G)[size_t(b * T + lane) * H + h] = Gp;
        }
    }
    if (kBf16 && slice == 0) {
        // The block's keys into the record, from the LDS copy (unswizzled).
        for (int c = tid; c < T * DK / 8; c += NTH) {
            const int r = c / (DK / 8), piece = c - r * (DK / 8);
            *reinterpret_cast<uint4 *>(kcopy + (size_t(b * T + r) * H + h) * DK + 8 * piece) =
                *reinterpret_cast<const uint4 *>(Xb + xoff<DK>(r, piece));
        }
    }

    // Gram matrix X X^T, each wave over its share of the keys, while the state is
    // still arriving: exact on bf16 MFMA for bf16 rows, fp32 MFMA otherwise.
    // Contraction slots visit keys 32p + 8lg + {0..7} (bf16), or 16m + 4lg + c
    // (fp32), in A and B alike.
    {
        f32x4 gacc[MT][MT];
#pragma unroll
        for (int m1 = 0; m1 < MT; ++m1)
#pragma unroll
            for (int m2 = 0; m2 < MT; ++m2) gacc[m1][m2] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (kBf16) {
#pragma unroll
            for (int pp = 0; pp < KH / 2; ++pp) {
                const int p = w * (KH / 2) + pp;
                bf16x8 a[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) a[mt] = xrow_bf16<DK>(Xb, 16 * mt + lr, p, lg);
#pragma unroll
                for (int m1 = 0; m1 < MT; ++m1)
#pragma unroll
                    for (int m2 = 0; m2 < MT; ++m2)
                        gacc[m1][m2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m1], a[m2], gacc[m1][m2], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int mm = 0; mm < KH; ++mm) {
                const int m = w * KH + mm;
                float4 a[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    a[mt] = *reinterpret_cast<const float4 *>(X + (16 * mt + lr) * XS + 16 * m + 4 * lg);
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int m1 = 0; m1 < MT; ++m1)
#pragma unroll
                        for (int m2 = 0; m2 < MT; ++m2)
                            gacc[m1][m2] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                comp(a[m1], c), comp(a[m2], c), gacc[m1][m2], 0, 0, 0);
            }
        }
#pragma unroll
        for (int m1 = 0; m1 < MT; ++m1)
#pragma unroll
            for (int m2 = 0; m2 < MT; ++m2)
#pragma unroll
                for (int r = 0; r < 4; ++r) gpart[w][16 * m1 + 4 * lg + r][16 * m2 + lr] = gacc[m1][m2][r];
    }
    __syncthreads();
    // Block coefficients (shared by every value row of the head):
    //   coefM[t][j] = beta_t Gamma_tj k_t.k_j (j < t),  coefN[t][j] = Gamma_tj q_t.k_j (j <= t).
    for (int idx = tid; idx < TM * TM; idx += NTH) {
        const int t = idx / TM, j = idx - t * TM;
        if (t < T && j <= t) {
            float kk = 0.f, qk = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
                kk += gpart[ww][t][j];
                qk += gpart[ww][TM + t][j];
            }
            const float dec = expf(Gs[t] - Gs[j]);
            coefM[t][j] = j < t ? bs[t] * dec * kk : 0.f;
            coefN[t][j] = dec * qk;
        }
    }
    __syncthreads();

    // The products tile by tile as the state arrives.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        if constexpr (FUSED) {
            if (nt >= NEARLY) commit_tile(nt);
        } else {
            fix_tile(nt);
            if constexpr (MIX) {
                if (nt + NPRE < NT) load_tile(nt + NPRE);
            }
        }
        products(nt);
    }
    // P columns RW w .. RW w + RW - 1 are this wave's own; its LDS operations
    // complete in order, and the compiler-only barrier keeps the compiler from
    // reordering them.
    asm volatile("" ::: "memory");

    // Value rows (one per lane, lane < RW of each wave): forward substitution for
    // delta, then outputs.
    float oo[MIX ? TM : 1];
    if (lane < RW) {
        const int li = RW * w + lane, i = rbase + li;
        float *Drec = reinterpret_cast<float *>(rec + RL.delta);
        float d[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            if (t < T) {
                float vt;
                if constexpr (kBf16)
                    vt = bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(Vb)[t * DV + i]);
                else
                    vt = Vs[t * DV + i];
                float dt = bs[t] * (vt - gam[t] * P[t][li]);
#pragma unroll
                for (int j = 0; j < t; ++j) dt -= coefM[t][j] * d[j];
                d[t] = dt;
                float ot = gam[t] * P[TM + t][li];
#pragma unroll
                for (int j = 0; j <= t; ++j) ot += coefN[t][j] * d[j];
                const size_t idx = (size_t(b * T + t) * H + h) * DV + i;
                // Streaming stores help the plain verify and cost the fused kernel
                // (measured), whose state write-backs are streaming already.
                if constexpr (MIX)
                    oo[t] = ot;
                else if constexpr (FUSED)
                    o[idx] = ot;
                else
                    __builtin_nontemporal_store(ot, o + idx);
                if constexpr (FUSED)
                    Drec[idx] = dt;
                else
                    __builtin_nontemporal_store(dt, Drec + idx);
            }
        }
    }

    if constexpr (MIX) {
        // Gated RMS norm over the head's dv outputs of each token: every lane holds
        // one value row (the workgroup covers the head).
        __shared__ float osq[NW][TM];
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const float s2 = wave_sum(t < T ? oo[t] * oo[t] : 0.f);
            if (lane == 0) osq[w][t] = s2;
        }
        __syncthreads();
        const int i = rbase + RW * w + lane;
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            if (t < T) {
                float s2 = 0.f;
#pragma unroll
                for (int j = 0; j < NW; ++j) s2 += osq[j][t];
                const size_t idx = (size_t(b * T + t) * H + h) * DV + i;
                o[idx] = oo[t] * rsqrt_nr(s2 * (1.f / float(DV)) + kMixEps) * nwr * silu(__uint_as_float(zr[t] << 16));
            }
        }
    }

    if constexpr (FUSED) {
        // Retire the committed block (every thread read the flags above, before
        // the barriers since) or report why nothing was committed.
        if (cok && tid < RS / kCommitRows)
            reinterpret_cast<uint32_t *>(rprev + RLp.flags)[size_t(bh) * kCommitSlices + fl0 + tid] = 0u;
        if (tid == 0 && h == 0 && slice == 0) {
            if (cok && pos) pos[b] += cn;
            if (cerr) atomicOr(&reinterpret_cast<RecCtrl *>(rprev + 256)[b].err, cerr);
        }
    }

    // Mark the block pending for every commit workgroup of this head, clear the
    // instance's error bits; the header describes the record.
    if (tid < RS / kCommitRows)
        reinterpret_cast<uint32_t *>(rec + RL.flags)[size_t(bh) * kCommitSlices + fl0 + tid] = kRecValid;
    if (tid == 0 && h == 0 && slice == 0) reinterpret_cast<RecCtrl *>(rec + RL.ctrl)[b].err = 0u;
    if (tid == 0 && bh == 0 && slice == 0) {
        RecHeader *hd = reinterpret_cast<RecHeader *>(rec);
        hd->T = T;
        hd->B = B;
        hd->H = H;
        hd->dk = DK;
        hd->dv = DV;
        hd->in_dt = kBf16 ? GDN_IN_BF16 : GDN_IN_F32;
        hd->magic = kRecMagic;
    }
}

constexpr unsigned kFewVerifyHeads = 256;  // fewer (instance, head) pairs: 4x the workgroups

template <int DK, int DV, typename TIn, bool FUSED>
hipError_t launch_t(float *S, const void *q, const void *k, const void *v, const float *g,
                    const float *beta, int T, const gdn_shape &s, float *o, void *rec, void *rprev,
                    const int32_t *n_acc, int32_t *pos, hipStream_t st) {
    const unsigned heads = unsigned(s.B) * unsigned(s.H);
    const dim3 block(DV);
    auto *qq = static_cast<const TIn *>(q);
    auto *kk = static_cast<const TIn *>(k);
    auto *vv = static_cast<const TIn *>(v);
    auto *rr = static_cast<uint8_t *>(rec);
    auto *rp = static_cast<uint8_t *>(rprev);
    // Few heads (fewer workgroups than compute units): 32 value rows per
    // workgroup; otherwise a whole head per workgroup.
    if (heads < kFewVerifyHeads) {
        constexpr int NTF = 128 / DV;  // tiles per wave for 32-row workgroups
        static_assert(NTF * 16 * (DV / 64) == 32, "few-heads workgroups cover 32 value rows");
        const dim3 grid(heads * unsigned(DV / 32));
        if (T <= 8)
            hipLaunchKernelGGL((verify_kernel<DK, DV, TIn, 1, FUSED, NTF>), grid, block, 0, st, S, qq, kk, vv, g,
                               beta, T, s.B, s.H, o, rr, rp, n_acc, pos, MixArgs{});
        else
            hipLaunchKernelGGL((verify_kernel<DK, DV, TIn, 2, FUSED, NTF>), grid, block, 0, st, S, qq, kk, vv, g,
                               beta, T, s.B, s.H, o, rr, rp, n_acc, pos, MixArgs{});
    } else {
        const dim3 grid(heads);
        if (T <= 8)
            hipLaunchKernelGGL((verify_kernel<DK, DV, TIn, 1, FUSED, 4>), grid, block, 0, st, S, qq, kk, vv, g,
                               beta, T, s.B, s.H, o, rr, rp, n_acc, pos, MixArgs{});
        else
            hipLaunchKernelGGL((verify_kernel<DK, DV, TIn, 2, FUSED, 4>), grid, block, 0, st, S, qq, kk, vv, g,
                               beta, T, s.B, s.H, o, rr, rp, n_acc, pos, MixArgs{});
    }
    return hipGetLastError();
}

template <bool FUSED>
hipError_t launch_any(float *S, const void *q, const void *k, const void *v, const float *g, const float *beta,
                      int T, gdn_in_dtype dt, const gdn_shape &s, float *o, void *rec, void *rprev,
                      const int32_t *n_acc, int32_t *pos, hipStream_t st) {
#define GDN_VERIFY_LAUNCH(DK_, DV_)                                                                        \
    if (s.dk == DK_ && s.dv == DV_)                                                                       \
        return dt == GDN_IN_BF16                                                                          \
                   ? launch_t<DK_, DV_, __hip_bfloat16, FUSED>(S, q, k, v, g, beta, T, s, o, rec, rprev,  \
                                                               n_acc, pos, st)                            \
                   : launch_t<DK_, DV_, float, FUSED>(S, q, k, v, g, beta, T, s, o, rec, rprev, n_acc,    \
                                                      pos, st);
    GDN_VERIFY_LAUNCH(128, 128)
    GDN_VERIFY_LAUNCH(128, 64)
    GDN_VERIFY_LAUNCH(64, 128)
    GDN_VERIFY_LAUNCH(64, 64)
#undef GDN_VERIFY_LAUNCH
    return hipErrorInvalidValue;
}

template <bool FUSED>
hipError_t launch_mix_t(float *S, const MixArgs &m, int T, const gdn_shape &s, float *o, void *rec, void *rprev,
                        const int32_t *n_acc, int32_t *pos, hipStream_t st) {
    using bf = __hip_bfloat16;
    const dim3 grid(unsigned(s.B) * unsigned(s.H)), block(128);
    auto *rr = static_cast<uint8_t *>(rec);
    auto *rp = static_cast<uint8_t *>(rprev);
    const bf *none = nullptr;
    const float *nonef = nullptr;
    if (T <= 8)
        hipLaunchKernelGGL((verify_kernel<128, 128, bf, 1, FUSED, 4, true>), grid, block, 0, st, S, none, none, none,
                           nonef, nonef, T, s.B, s.H, o, rr, rp, n_acc, pos, m);
    else
        hipLaunchKernelGGL((verify_kernel<128, 128, bf, 2, FUSED, 4, true>), grid, block, 0, st, S, none, none, none,
                           nonef, nonef, T, s.B, s.H, o, rr, rp, n_acc, pos, m);
    return hipGetLastError();
}

MixArgs mix_args(const gdn_mixer_inputs &in) {
    MixArgs m;
    m.x = static_cast<const __hip_bfloat16 *>(in.x);
    m.hist = static_cast<const __hip_bfloat16 *>(in.history);
    m.conv_w = in.conv_w;
    m.a = in.a;
    m.bg = in.b;
    m.A_log = in.A_log;
    m.dt_bias = in.dt_bias;
    m.z = static_cast<const __hip_bfloat16 *>(in.z);
    m.norm_w = in.norm_w;
    m.Hk = in.Hk;
    return m;
}

}  // namespace

hipError_t launch_mixer_verify(const float *S, const gdn_mixer_inputs &in, int T, const gdn_shape &shp, float *y,
                               void *record, hipStream_t stream) {
    return launch_mix_t<false>(const_cast<float *>(S), mix_args(in), T, shp, y, record, nullptr, nullptr, nullptr,
                               stream);
}

hipError_t launch_mixer_commit_verify(float *S, void *record_prev, const int32_t *n_accepted, int32_t *pos,
                                      const gdn_mixer_inputs &in, int T, const gdn_shape &shp, float *y,
                                      void *record_next, hipStream_t stream) {
    return launch_mix_t<true>(S, mix_args(in), T, shp, y, record_next, record_prev, n_accepted, pos, stream);
}

hipError_t launch_verify(const float *S, const void *q, const void *k, const void *v,
                         const float *g, const float *beta, int T, gdn_in_dtype dt,
                         const gdn_shape &shp, float *o, void *record, hipStream_t stream) {
    // The plain verify never writes S.
    return launch_any<false>(const_cast<float *>(S), q, k, v, g, beta, T, dt, shp, o, record, nullptr, nullptr,
                             nullptr, stream);
}

hipError_t launch_commit_verify(float *S, void *record_prev, const int32_t *n_accepted, int32_t *pos,
                                const void *q, const void *k, const void *v, const float *g,
                                const float *beta, int T, gdn_in_dtype dt, const gdn_shape &shp, float *o,
                                void *record_next, hipStream_t stream) {
    return launch_any<true>(S, q, k, v, g, beta, T, dt, shp, o, record_next, record_prev, n_accepted, pos,
                            stream);
}

}  // namespace gdn
