// prefill.hip -- chunked prefill of the gated delta rule in UT / WY form.
//
// Long prompts are where prefill time goes (devdoido audit, "What does
// long-context prefill cost on Apple silicon?").  The prompt is cut into chunks of
// C = 64 tokens; only the fp32 state crosses chunk boundaries.  Within a chunk,
// with the log-decay prefix G_t (restarted per chunk), gamma_t = exp(G_t),
// Gamma_tj = exp(G_t - G_j) and e_t = exp(G_last - G_t):
//
//   A   = strictly-lower(beta_t Gamma_tj k_t.k_j),   Linv = (I + A)^{-1}
//   R   = diag(beta) (V - diag(gamma) K S^T)
//   D   = Linv R                                 (the chunk's delta rows)
//   O   = diag(gamma) Q S^T + lower-incl(Gamma o Q K^T) D
//   S  <- gamma_last S + D^T diag(e) K
//
// (the chunkwise form of Gated DeltaNet, ICLR 2025).  Every product is a dense
// contraction and runs on bf16 MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulate).
// q, k, v are bf16 and enter exactly; fp32 operands (S, R, D, Linv, the decayed
// Gram matrices) are split into a high and a low bf16 part, x = hi + lo with
// |x - hi - lo| <= 2^-17 |x|, and multiplied as hi*hi + hi*lo + lo*hi (the
// split-bf16 scheme of Henry, Tang & Heinecke, ARITH 2019).
//
// Rows of S never interact, so slices of the value index are independent; a
// workgroup owns RS = 16 * NWS value rows of one (instance, head), holds their
// state in registers and walks the chunks in order, wave w owning 16 rows.  Per
// chunk, the state-independent quantities (gates, Gram matrices, Linv, P) are
// built in LDS, then each wave runs the state-coupled products for its rows.
// MFMA results feed the next MFMA straight from registers: a 16x16 result tile
// holds rows 4*(lane/16)+r of column lane%16, which is the layout of a B operand
// whose contraction index runs over those rows.
//
// Two schedules:
//  - one pass (many heads): one workgroup per head builds and consumes each
//    chunk's quantities itself;
//  - two phases (few heads, where the chunk scan's latency dominates): a prep
//    builds Linv, P and the gates of every chunk in parallel into a
//    workspace, and a scan walks the chunks doing only state-coupled work,
//    with the next chunk's operands copied into LDS one chunk ahead.  The
//    chunks are cut into segments and each segment's prep runs beside the
//    previous segment's scan, on the compute units the scan leaves idle.
#include <algorithm>

#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int C = GDN_PREFILL_CHUNK;


__device__ inline f32x4 mma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

struct Split8 {
    bf16x8 hi, lo;
};

__device__ inline Split8 split8(const float (&x)[8]) {
    Split8 s;
    split8_bf16(x, s.hi, s.lo);
    return s;
}

__device__ inline bf16x8 cat4(const bf16x4 &a, const bf16x4 &b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// x * y with both split: hi*hi + hi*lo + lo*hi.
__device__ inline f32x4 mma3(const Split8 &a, const Split8 &b, f32x4 c) {
    c = mma(a.hi, b.hi, c);
    c = mma(a.hi, b.lo, c);
    return mma(a.lo, b.hi, c);
}

template <int DK>
struct alignas(16) Smem {
    __bf16 Ks[C][DK + 8];   // keys, row-major [t][key]
    __bf16 Qs[C][DK + 8];   // queries, row-major
    __bf16 Kt[DK][C + 8];   // keys, transposed [key][t]
    float Am[C][C + 4];     // strictly-lower(beta_t Gamma_tj k_t.k_j)
    float Tm[C][C + 4];     // Linv = (I + A)^{-1}
    float Pm[C][C + 4];     // lower-incl(Gamma_tj q_t.k_j)
    float gam[C], ee[C], bet[C], G[C];
    // Linv and P split into bf16 high and low parts: the A operands of the
    // state-coupled products, ready to use.
    __bf16 LiH[C][C + 8], LiL[C][C + 8], PH[C][C + 8], PL[C][C + 8];
};

// LDS of the prep kernel: Linv and the inverse's scratch reuse the keys' and
// queries' space once the Gram matrices are built, so two workgroups fit on a CU.
template <int DK>
struct alignas(16) PrepSmem {
    union {
        struct {
            __bf16 Ks[C][DK + 8];
            __bf16 Qs[C][DK + 8];
        };
        struct {
            float Tm[C][C + 4];
            float Inv[4 * 2 * 320];   // the inverse's scratch (4 waves x 2 matrices)
        };
    };
    float Am[C][C + 4];
    float Pm[C][C + 4];
    float gam[C], ee[C], bet[C], G[C];
};

// Workspace record of one (instance, head, chunk) in the two-phase schedule.
// Linv and P as bf16 (hi, lo) pairs: four [C][C] bf16 arrays, then gam, ee, bet.
constexpr size_t kPrepMatBytes = 4 * C * C * sizeof(__bf16);
constexpr size_t kPrepBytes = (kPrepMatBytes + 3 * C * sizeof(float) + 255) & ~size_t(255);
constexpr int kFewHeads = 256;  // fewer (instance, head) pairs than this: two phases

// Keys and queries of one chunk as raw 16-byte pieces: piece u of thread tid is
// row t = (tid + u NT) / (DK / 8), columns col .. col + 7.
template <int DK, int NT>
struct ChunkKQ {
    static constexpr int NLD = C * DK / 8 / NT;
    static_assert(NLD >= 1 && NLD * NT * 8 == C * DK, "staging tiling");
    uint4 kv[NLD], qv[NLD];
    // Rows past the prompt read the last valid row (always a valid address); they
    // are zeroed when stored, never here, so nothing waits on these loads early.
    // kStream: streaming loads, for rows nothing reads again soon (the one-pass
    // kernel; the two-phase prep's rows are read again by the scan).
    template <bool kStream = false>
    __device__ inline void load(const __hip_bfloat16 *k, const __hip_bfloat16 *q, size_t row0, int n,
                                int H, int h, int tid) {
#pragma unroll
        for (int u = 0; u < NLD; ++u) {
            const int idx = tid + u * NT;
            const int t = idx / (DK / 8), col = (idx - t * (DK / 8)) * 8;
            const size_t off = ((row0 + min(t, n - 1)) * H + h) * DK + col;
            kv[u] = kStream ? ld_stream_u4(k + off) : *reinterpret_cast<const uint4 *>(k + off);
            qv[u] = kStream ? ld_stream_u4(q + off) : *reinterpret_cast<const uint4 *>(q + off);
        }
    }
    // kTrans: also write the transposed keys (the state update's A operand).
    template <bool kTrans = true, typename SM>
    __device__ inline void store(SM &sm, int n, int tid) const {
#pragma unroll
        for (int u = 0; u < NLD; ++u) {
            const int idx = tid + u * NT;
            const int t = idx / (DK / 8), col = (idx - t * (DK / 8)) * 8;
            const uint4 z = make_uint4(0u, 0u, 0u, 0u);
            const uint4 kk = t < n ? kv[u] : z, qq = t < n ? qv[u] : z;
            *reinterpret_cast<uint4 *>(&sm.Ks[t][col]) = kk;
            *reinterpret_cast<uint4 *>(&sm.Qs[t][col]) = qq;
            if constexpr (kTrans) {
                const __bf16 *kh = reinterpret_cast<const __bf16 *>(&kk);
#pragma unroll
                for (int e = 0; e < 8; ++e) sm.Kt[col + e][t] = kh[e];
            }
        }
    }
};

// Gates of one chunk (wave 0, lane t): log-decay prefix sum G, gamma = exp(G),
// e = exp(G_last - G), beta; rows past the prompt get g = beta = e = 0.
template <typename SM>
__device__ inline void chunk_gates(SM &sm, float gt, float bt, int n, int lane) {
    if (lane >= n) {
        gt = 0.f;
        bt = 0.f;
    }
    float Gp = gt;  // inclusive prefix sum over the chunk
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(Gp, off, 64);
        if (lane >= off) Gp += y;
    }
    const float Glast = __shfl(Gp, n - 1, 64);
    sm.G[lane] = Gp;
    sm.gam[lane] = __expf(Gp);
    sm.ee[lane] = lane < n ? __expf(Glast - Gp) : 0.f;
    sm.bet[lane] = bt;
}

// 16x16 fp32 operands of the inverse, by where they live.  RowMat: row-major
// fp32 in LDS, element (r, c) at p[r * ld + c] (16-byte aligned rows and
// column bases).  ColMat: a wave's scratch matrix, stored transposed, element
// (r, c) at p[20 c + r].
struct RowMat {
    const float *p;
    int ld;
};
struct ColMat {
    const float *p;
};

// The four values a lane contributes over the four k-steps of a product: k-step
// s takes contraction index 4 lg + s from lane group lg, so a lane's A values
// are A(lr, 4 lg .. 4 lg + 3) and its B values B(4 lg .. 4 lg + 3, lr); where
// those are consecutive in memory (A row-major, B stored transposed) they come
// in one 16-byte read.
__device__ inline float4 a_vals(const RowMat &m, int lr, int lg) {
    return *reinterpret_cast<const float4 *>(m.p + lr * m.ld + 4 * lg);
}
__device__ inline float4 a_vals(const ColMat &m, int lr, int lg) {
    return make_float4(m.p[20 * (4 * lg) + lr], m.p[20 * (4 * lg + 1) + lr], m.p[20 * (4 * lg + 2) + lr],
                       m.p[20 * (4 * lg + 3) + lr]);
}
__device__ inline float4 b_vals(const RowMat &m, int lr, int lg) {
    return make_float4(m.p[(4 * lg) * m.ld + lr], m.p[(4 * lg + 1) * m.ld + lr], m.p[(4 * lg + 2) * m.ld + lr],
                       m.p[(4 * lg + 3) * m.ld + lr]);
}
__device__ inline float4 b_vals(const ColMat &m, int lr, int lg) {
    return *reinterpret_cast<const float4 *>(m.p + 20 * lr + 4 * lg);
}

// One 16x16 fp32 product on the fp32 MFMA, d + A B.  The result is in the D
// layout: lane (lr, lg) holds rows 4lg .. 4lg + 3 of column lr.
template <typename MA, typename MB>
__device__ inline f32x4 mm16(const MA &a, const MB &b, f32x4 d, int lr, int lg) {
    const float4 av = a_vals(a, lr, lg), bv = b_vals(b, lr, lg);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(av.x, bv.x, d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(av.y, bv.y, d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(av.z, bv.z, d, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x4f32(av.w, bv.w, d, 0, 0, 0);
}

// A D-layout tile into a wave's scratch matrix, stored transposed (column c at
// 20 c): one 16-byte write per lane; read back as a ColMat.
__device__ inline void scr_put(float *m, const f32x4 &d, int lr, int lg) {
    *reinterpret_cast<float4 *>(m + 20 * lr + 4 * lg) = make_float4(d[0], d[1], d[2], d[3]);
}

// Linv = (I + A)^{-1} for the chunk's strictly lower A (fp32 [C][C + 4] in LDS)
// into Tm's lower block triangle, on the fp32 MFMA; waves 0..3 take part, and
// any further waves run `side` meanwhile.
// Diagonal 16x16 blocks: with N strictly lower, N^16 = 0 and
//   (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8),
// three squarings and three products, one wave per block, its intermediates in
// its own two scratch matrices (scr: 4 x 2 x 320 floats).  Off-diagonal blocks
// by 2x2 blocking: X_10 = -X_11 A_10 X_00 and X_32 = -X_33 A_32 X_22 complete the
// inverses X_A, X_B of the two 32x32 diagonal blocks, and the lower-left 32x32
// block is -X_B A_BA X_A.
// Every product of lower-triangular factors keeps exact zeros above the
// diagonal and ones on it, so the diagonal blocks need no masking.  Tm may be
// Am itself: each block is read before it is overwritten.
template <typename MA, typename MT, typename Side>
__device__ inline void tri_inverse(const MA &Am, MT &Tm, float *scr, int w, int lane, Side &&side) {
    const int lr = lane & 15, lg = lane >> 4;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    constexpr int LD = C + 4;
    const auto A = [&](int bi, int bj) { return RowMat{&Am[16 * bi][16 * bj], LD}; };
    const auto X = [&](int bi, int bj) { return RowMat{&Tm[16 * bi][16 * bj], LD}; };
    if (w >= 4) side();   // waves past the fourth: independent work, if any
    if (w < 4) {
        const int b0 = 16 * w;
        float *s0 = scr + w * 640, *s1 = s0 + 320;
        const RowMat N = A(w, w);
        const f32x4 p1 = mm16(N, N, z, lr, lg);                       // N^2
        scr_put(s0, p1, lr, lg);
        const f32x4 p2 = mm16(ColMat{s0}, ColMat{s0}, z, lr, lg);     // N^4
        const f32x4 y = mm16(N, ColMat{s0}, z, lr, lg);               // N^3
        f32x4 x;                                                       // (I - N)(I + N^2)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 4 * lg + r;
            x[r] = (row == lr ? 1.f : 0.f) - Am[b0 + row][b0 + lr] + p1[r] - y[r];
        }
        scr_put(s0, p2, lr, lg);                                       // (this wave's reads of N^2 came first)
        scr_put(s1, x, lr, lg);
        const f32x4 p3 = mm16(ColMat{s0}, ColMat{s0}, z, lr, lg);     // N^8
        x = mm16(ColMat{s1}, ColMat{s0}, x, lr, lg);                  // X (I + N^4)
        scr_put(s0, p3, lr, lg);
        scr_put(s1, x, lr, lg);
        x = mm16(ColMat{s1}, ColMat{s0}, x, lr, lg);                  // X (I + N^8)
#pragma unroll
        for (int r = 0; r < 4; ++r) Tm[b0 + 4 * lg + r][b0 + lr] = x[r];
    }
    __syncthreads();
    // The off-diagonal block inside each 32x32 diagonal block: X_10 and X_32.
    if (w < 2) {
        const int j = 2 * w, i = j + 1;
        float *s0 = scr + w * 640;
        scr_put(s0, mm16(A(i, j), X(j, j), z, lr, lg), lr, lg);
        const f32x4 x = mm16(X(i, i), ColMat{s0}, z, lr, lg);
#pragma unroll
        for (int r = 0; r < 4; ++r) Tm[16 * i + 4 * lg + r][16 * j + lr] = -x[r];
    }
    __syncthreads();
    // The lower-left 32x32 block: with X_A, X_B the inverses of the two diagonal
    // 32x32 blocks and A_BA the lower-left block of A, it is -X_B (A_BA X_A).
    // Y = A_BA X_A, block (p, q) on wave 2 (p - 2) + q ...
    if (w < 4) {
        const int p = 2 + (w >> 1), q = w & 1;
        f32x4 y = mm16(A(p, 1), X(1, q), z, lr, lg);
        if (q == 0) y = mm16(A(p, 0), X(0, 0), y, lr, lg);
        scr_put(scr + w * 640, y, lr, lg);
    }
    __syncthreads();
    // ... then X_ij = -sum_{m=2}^{i} X_im Y_mj, block (i, j) on wave 2 (i - 2) + j.
    if (w < 4) {
        const int i = 2 + (w >> 1), j = w & 1;
        f32x4 x = mm16(X(i, 2), ColMat{scr + j * 640}, z, lr, lg);
        if (i == 3) x = mm16(X(3, 3), ColMat{scr + (2 + j) * 640}, x, lr, lg);
#pragma unroll
        for (int r = 0; r < 4; ++r) Tm[16 * i + 4 * lg + r][16 * j + lr] = -x[r];
    }
    __syncthreads();
}

// Gram matrices and Linv of the staged chunk (all NWS >= 4 waves; barriers
// inside).  On entry Ks, Qs and the gates are in LDS; on exit Pm and Tm hold P
// and Linv in their lower block triangles (diagonal blocks included, zero above
// the diagonal within them); the strictly upper blocks are never written.  scr:
// 10 KiB of LDS for the inverse, free until the chunk's products; `side` runs on
// waves past the fourth during the inverse, after the Gram matrices.
template <int DK, int NWS, typename SM, typename Side>
__device__ inline void chunk_prep(SM &sm, int tid, int w, int lane, float *scr, Side &&side) {
    constexpr int KB = DK / 32;
    constexpr int NT = 64 * NWS;
    const int lr = lane & 15, lg = lane >> 4;
    // Gram tiles: A from K K^T, P from Q K^T (lower tiles only).
    for (int qi = w; qi < 20; qi += NWS) {
        const bool isq = qi >= 10;
        const int p = isq ? qi - 10 : qi;
        const int tt = p >= 6 ? 3 : p >= 3 ? 2 : p >= 1 ? 1 : 0;
        const int jt = p - tt * (tt + 1) / 2;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const bf16x8 a = isq ? *reinterpret_cast<const bf16x8 *>(&sm.Qs[16 * tt + lr][32 * kb + 8 * lg])
                                 : *reinterpret_cast<const bf16x8 *>(&sm.Ks[16 * tt + lr][32 * kb + 8 * lg]);
            const bf16x8 bk = *reinterpret_cast<const bf16x8 *>(&sm.Ks[16 * jt + lr][32 * kb + 8 * lg]);
            acc = mma(a, bk, acc);
        }
        const int j = 16 * jt + lr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * tt + 4 * lg + r;
            const float dec = __expf(sm.G[t] - sm.G[j]);
            if (isq)
                sm.Pm[t][j] = j <= t ? dec * acc[r] : 0.f;
            else
                sm.Am[t][j] = j < t ? sm.bet[t] * dec * acc[r] : 0.f;
        }
    }
    __syncthreads();
    tri_inverse(sm.Am, sm.Tm, scr, w, lane, side);
}

// Eight elements (row t, columns j8 .. j8 + 7) of Linv and of P, split into bf16
// high and low parts; zero in the strictly upper blocks, which chunk_prep leaves
// unwritten.
template <typename SM>
__device__ inline void split_mats8(const SM &sm, int t, int j8, Split8 &ls, Split8 &ps) {
    float a[8], p8[8];
    *reinterpret_cast<float4 *>(a) = *reinterpret_cast<const float4 *>(&sm.Tm[t][j8]);
    *reinterpret_cast<float4 *>(a + 4) = *reinterpret_cast<const float4 *>(&sm.Tm[t][j8 + 4]);
    *reinterpret_cast<float4 *>(p8) = *reinterpret_cast<const float4 *>(&sm.Pm[t][j8]);
    *reinterpret_cast<float4 *>(p8 + 4) = *reinterpret_cast<const float4 *>(&sm.Pm[t][j8 + 4]);
    if ((j8 >> 4) > (t >> 4)) {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = p8[e] = 0.f;
    }
    ls = split8(a);
    ps = split8(p8);
}

// The state-coupled products' A operands in LDS: Linv (kP false) or P (kP true)
// split, by threads t0, t0 + nt, ...; zero in the strictly upper blocks.
template <bool kP, int DK>
__device__ inline void split_mat(Smem<DK> &sm, int t0, int nt) {
    for (int idx = t0; idx < C * C / 8; idx += nt) {
        const int t = idx / (C / 8), j8 = (idx - t * (C / 8)) * 8;
        float a[8];
        const float *src = kP ? &sm.Pm[t][j8] : &sm.Tm[t][j8];
        *reinterpret_cast<float4 *>(a) = *reinterpret_cast<const float4 *>(src);
        *reinterpret_cast<float4 *>(a + 4) = *reinterpret_cast<const float4 *>(src + 4);
        if ((j8 >> 4) > (t >> 4)) {
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] = 0.f;
        }
        const Split8 sp = split8(a);
        *reinterpret_cast<bf16x8 *>(kP ? &sm.PH[t][j8] : &sm.LiH[t][j8]) = sp.hi;
        *reinterpret_cast<bf16x8 *>(kP ? &sm.PL[t][j8] : &sm.LiL[t][j8]) = sp.lo;
    }
}

// Scheduling fences between the steps of chunk_state (compiler-only; no
// instruction is emitted).  They keep the scheduler from hoisting the next
// step's LDS operands, and the registers they hold, over the current step: a
// gain where the chunk's own prep shares the kernel, a loss in the scan kernel,
// whose prefetch needs the freedom.
template <bool F>
__device__ inline void step_fence() {
    if constexpr (F) asm volatile("" ::: "memory");
}
template <bool F>
__device__ inline void sched_fence() {
    if constexpr (F) __builtin_amdgcn_sched_barrier(0);
}

// State-coupled products of one chunk for one wave's 16 value rows (value row
// irow = this lane's column).  vv[tt][r] = v[t][irow] for t = 16 tt + 4 lg + r
// (0 past the prompt); obase points at o for the chunk's first token and this
// lane's value row, ostride is one token.
template <int DK, bool F>
__device__ inline void chunk_state(const Smem<DK> &sm, float (&st)[DK / 16][4], const float (&vv)[4][4],
                                   int n, int lane, float *__restrict__ obase, size_t ostride) {
    constexpr int KT = DK / 16, KB = DK / 32;
    const int lr = lane & 15, lg = lane >> 4;
    // The contraction over keys visits, for block p and lane group lg, keys
    // 32p + 4lg + {0..3} and 32p + 16 + 4lg + {0..3}: the keys this lane holds
    // in st[2p] and st[2p+1].  Products are formed in an order that keeps few
    // values live: K S^T and Q S^T first (the split state then dies), then D, then
    // the outputs and the state update.
    f32x4 X[4], Y[4];
    {
        Split8 sB[KB];
#pragma unroll
        for (int p = 0; p < KB; ++p) {
            const float x[8] = {st[2 * p][0], st[2 * p][1], st[2 * p][2], st[2 * p][3],
                                st[2 * p + 1][0], st[2 * p + 1][1], st[2 * p + 1][2], st[2 * p + 1][3]};
            sB[p] = split8(x);
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            X[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
            Y[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int t = 16 * tt + lr;
#pragma unroll
            for (int p = 0; p < KB; ++p) {
                const bf16x8 ka = cat4(*reinterpret_cast<const bf16x4 *>(&sm.Ks[t][32 * p + 4 * lg]),
                                       *reinterpret_cast<const bf16x4 *>(&sm.Ks[t][32 * p + 16 + 4 * lg]));
                const bf16x8 qa = cat4(*reinterpret_cast<const bf16x4 *>(&sm.Qs[t][32 * p + 4 * lg]),
                                       *reinterpret_cast<const bf16x4 *>(&sm.Qs[t][32 * p + 16 + 4 * lg]));
                X[tt] = mma(ka, sB[p].hi, X[tt]);
                X[tt] = mma(ka, sB[p].lo, X[tt]);
                Y[tt] = mma(qa, sB[p].hi, Y[tt]);
                Y[tt] = mma(qa, sB[p].lo, Y[tt]);
            }
            sched_fence<F>();
        }
    }
    step_fence<F>();
    // R = diag(beta) (V - diag(gamma) K S^T), rows t = 16 tt + 4 lg + r, split as the
    // B operand of D = Linv R.
    Split8 rB[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int tt = 2 * p + (e >> 2), r = e & 3, tr = 16 * tt + 4 * lg + r;
            x[e] = sm.bet[tr] * (vv[tt][r] - sm.gam[tr] * X[tt][r]);
        }
        rB[p] = split8(x);
    }
    // D = Linv R (Linv is lower triangular: only blocks p <= tt / 2).
    f32x4 D[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        D[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int t = 16 * tt + lr;
#pragma unroll
        for (int p = 0; p <= tt / 2; ++p) {
            Split8 a;
            a.hi = cat4(*reinterpret_cast<const bf16x4 *>(&sm.LiH[t][32 * p + 4 * lg]),
                        *reinterpret_cast<const bf16x4 *>(&sm.LiH[t][32 * p + 16 + 4 * lg]));
            a.lo = cat4(*reinterpret_cast<const bf16x4 *>(&sm.LiL[t][32 * p + 4 * lg]),
                        *reinterpret_cast<const bf16x4 *>(&sm.LiL[t][32 * p + 16 + 4 * lg]));
            D[tt] = mma3(a, rB[p], D[tt]);
        }
        sched_fence<F>();
    }
    step_fence<F>();
    // D split twice: as is (for P D) and scaled by e (for the state update).
    Split8 dB[2], eB[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        float x[8], y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int tt = 2 * p + (e >> 2), r = e & 3, tr = 16 * tt + 4 * lg + r;
            x[e] = D[tt][r];
            y[e] = sm.ee[tr] * D[tt][r];
        }
        dB[p] = split8(x);
        eB[p] = split8(y);
    }
    step_fence<F>();
    // O = diag(gamma) Q S^T + P D.
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int t = 16 * tt + lr;
        f32x4 Ot = Y[tt];
#pragma unroll
        for (int r = 0; r < 4; ++r) Ot[r] *= sm.gam[16 * tt + 4 * lg + r];
#pragma unroll
        for (int p = 0; p <= tt / 2; ++p) {
            Split8 a;
            a.hi = cat4(*reinterpret_cast<const bf16x4 *>(&sm.PH[t][32 * p + 4 * lg]),
                        *reinterpret_cast<const bf16x4 *>(&sm.PH[t][32 * p + 16 + 4 * lg]));
            a.lo = cat4(*reinterpret_cast<const bf16x4 *>(&sm.PL[t][32 * p + 4 * lg]),
                        *reinterpret_cast<const bf16x4 *>(&sm.PL[t][32 * p + 16 + 4 * lg]));
            Ot = mma3(a, dB[p], Ot);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tr = 16 * tt + 4 * lg + r;
            if (tr < n) __builtin_nontemporal_store(Ot[r], obase + size_t(tr) * ostride);
        }
        sched_fence<F>();
    }
    step_fence<F>();
    // S <- gamma_last S + K^T diag(e) D; the result tiles over keys match st[][].
    const float glast = sm.gam[n - 1];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        f32x4 U = {0.f, 0.f, 0.f, 0.f};
        const int key = 16 * kt + lr;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const bf16x8 ka = cat4(*reinterpret_cast<const bf16x4 *>(&sm.Kt[key][32 * p + 4 * lg]),
                                   *reinterpret_cast<const bf16x4 *>(&sm.Kt[key][32 * p + 16 + 4 * lg]));
            U = mma(ka, eB[p].hi, U);
            U = mma(ka, eB[p].lo, U);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) st[kt][r] = glast * st[kt][r] + U[r];
        sched_fence<F>();
    }
}

// v[t][irow] for the lane's rows t = 16 tt + 4 lg + r of a chunk (raw bf16 bits;
// rows past the prompt read the last valid row and are masked at use).
struct ChunkV {
    uint16_t raw[4][4];
    __device__ inline void load(const __hip_bfloat16 *v, size_t row0, int n, int H, int h, int DV,
                                int irow, int lg) {
        const uint16_t *vb = reinterpret_cast<const uint16_t *>(v);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * tt + 4 * lg + r;
                raw[tt][r] = __builtin_nontemporal_load(vb + ((row0 + min(t, n - 1)) * H + h) * DV + irow);
            }
    }
    __device__ inline void get(float (&vv)[4][4], int n, int lg) const {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * tt + 4 * lg + r;
                vv[tt][r] = t < n ? bf16_bits_to_f32(raw[tt][r]) : 0.f;
            }
    }
};

// ---------------------------------------------------------------------------
// One pass: one workgroup per (instance, head), NWS waves of 16 value rows.
// ---------------------------------------------------------------------------
template <int DK, int DV, int NWS>
__global__ __launch_bounds__(64 * NWS) void prefill_kernel(
    float *__restrict__ S, const __hip_bfloat16 *__restrict__ q, const __hip_bfloat16 *__restrict__ k,
    const __hip_bfloat16 *__restrict__ v, const float *__restrict__ g, const float *__restrict__ beta,
    int L, int H, float *__restrict__ o) {
    constexpr int RS = 16 * NWS;       // value rows per workgroup
    constexpr int SLICES = DV / RS;
    constexpr int KT = DK / 16;
    constexpr int NT = 64 * NWS;
    static_assert(SLICES * RS == DV, "tiling");

    __shared__ Smem<DK> sm;

    const int wg = blockIdx.x;
    const int bh = wg / SLICES, slice = wg - bh * SLICES;
    const int b = bh / H, h = bh - b * H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int irow = slice * RS + w * 16 + lr;  // value row of this lane's column

    // State slice in registers: st[kt][r] = S[irow][16 kt + 4 lg + r].
    float *Srow = S + (size_t(bh) * DV + irow) * DK;
    float st[KT][4];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        const float4 s4 = *reinterpret_cast<const float4 *>(Srow + 16 * kt + 4 * lg);
        st[kt][0] = s4.x;
        st[kt][1] = s4.y;
        st[kt][2] = s4.z;
        st[kt][3] = s4.w;
    }

    const int nchunks = (L + C - 1) / C;
    for (int c = 0; c < nchunks; ++c) {
        const int c0 = c * C;
        const int n = min(C, L - c0);
        const size_t row0 = size_t(b) * L + c0;  // (b, c0) token row
        {
            ChunkKQ<DK, NT> kq;
            kq.template load<true>(k, q, row0, n, H, h, tid);
            const size_t gi = (row0 + min(lane, n - 1)) * H + h;
            const float gt = g[gi], bt = beta[gi];
            kq.store(sm, n, tid);
            if (w == 0) chunk_gates(sm, gt, bt, n, lane);
        }
        __syncthreads();
        // The inverse's scratch: the split operands' space, rewritten below.
        chunk_prep<DK, NWS>(sm, tid, w, lane, reinterpret_cast<float *>(&sm.LiH[0][0]), [] {});
        split_mat<true>(sm, tid, NT);
        split_mat<false>(sm, tid, NT);
        __syncthreads();
        ChunkV cv;
        cv.load(v, row0, n, H, h, DV, irow, lg);
        float vv[4][4];
        cv.get(vv, n, lg);
        chunk_state<DK, true>(sm, st, vv, n, lane, o + (row0 * H + h) * DV + irow, size_t(H) * DV);
        __syncthreads();  // the next chunk overwrites the shared buffers
    }

#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
        *reinterpret_cast<float4 *>(Srow + 16 * kt + 4 * lg) =
            make_float4(st[kt][0], st[kt][1], st[kt][2], st[kt][3]);
}

// ---------------------------------------------------------------------------
// Two-phase schedule, prep: a workgroup builds Linv, P and the gates of one
// (instance, head, chunk) and writes them to that chunk's workspace record,
// with NWS >= 4 waves.
// ---------------------------------------------------------------------------
template <int DK, int NWS>
__device__ __forceinline__ void prep_unit(PrepSmem<DK> &sm, const __hip_bfloat16 *__restrict__ q,
                                 const __hip_bfloat16 *__restrict__ k, const float *__restrict__ g,
                                 const float *__restrict__ beta, int L, int H, int nchunks,
                                 uint8_t *__restrict__ ws, int bh, int c) {
    constexpr int NT = 64 * NWS;
    const int b = bh / H, h = bh - b * H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c0 = c * C, n = min(C, L - c0);
    const size_t row0 = size_t(b) * L + c0;
    {
        ChunkKQ<DK, NT> kq;
        kq.load(k, q, row0, n, H, h, tid);
        const size_t gi = (row0 + min(lane, n - 1)) * H + h;
        const float gt = g[gi], bt = beta[gi];
        kq.template store<false>(sm, n, tid);
        if (w == 0) chunk_gates(sm, gt, bt, n, lane);
    }
    __syncthreads();
    chunk_prep<DK, NWS>(sm, tid, w, lane, sm.Inv, [] {});
    // Linv hi, Linv lo, P hi, P lo as dense bf16 [C][C], then gam, ee, bet.
    uint8_t *out = ws + (size_t(bh) * nchunks + c) * kPrepBytes;
    for (int idx = tid; idx < C * C / 8; idx += NT) {
        const int t = idx / (C / 8), j8 = (idx - t * (C / 8)) * 8;
        Split8 ls, ps;
        split_mats8(sm, t, j8, ls, ps);
        __bf16 *o16 = reinterpret_cast<__bf16 *>(out) + t * C + j8;
        *reinterpret_cast<bf16x8 *>(o16) = ls.hi;
        *reinterpret_cast<bf16x8 *>(o16 + C * C) = ls.lo;
        *reinterpret_cast<bf16x8 *>(o16 + 2 * C * C) = ps.hi;
        *reinterpret_cast<bf16x8 *>(o16 + 3 * C * C) = ps.lo;
    }
    if (tid < C) {
        float *gout = reinterpret_cast<float *>(out + kPrepMatBytes);
        gout[tid] = sm.gam[tid];
        gout[C + tid] = sm.ee[tid];
        gout[2 * C + tid] = sm.bet[tid];
    }
}

// ---------------------------------------------------------------------------
// Two phases, scan: one workgroup per (instance, head, 32 value rows) walks
// a range of chunks doing only the state-coupled products.  Each chunk's operands
// (keys, queries, Linv and P split, the gates, the workgroup's value columns)
// are copied global -> LDS asynchronously one chunk ahead, into the other half
// of a double buffer, so the walk waits on memory once per chunk at most.
// ---------------------------------------------------------------------------

// Operand mapping of the scan.  The 16 rows of result tile tt (a 16x16 MFMA
// tile over tokens) are the tokens tau(tt, m) = 32 (tt/2) + 8 (m/4) + 4 (tt%2) +
// m%4, m = 0..15, and the contraction slots of block p for lane group lg are the
// 8 consecutive indices 32p + 8lg .. + 7.  A D-layout lane (lr, lg) of tiles 2p
// and 2p + 1 then holds exactly tokens 32p + 8lg .. + 7 (4 from each tile), the
// slots of a B operand over tokens; and every A operand is one 16-byte LDS
// read.  The state is kept the same way over keys: st[kt][r] is key
// 32 (kt/2) + 8 lg + 4 (kt%2) + r of value row irow.
__device__ inline int tau(int tt, int m) { return 32 * (tt >> 1) + 8 * (m >> 2) + 4 * (tt & 1) + (m & 3); }

// LDS layouts.  Rows of keys/queries (256 B at dk = 128, 128 B at dk = 64) and
// of the [C][C] matrices (128 B) keep their 16-byte pieces in an XOR-swizzled
// order, slot = piece ^ swz(row), chosen so that the A-operand row reads (16
// rows 8 (m/4) + m%4 apart, one piece each) and the transposed reads of the
// state update (4 consecutive rows x 4 pieces) hit distinct banks.
__device__ inline int swz16(int t) { return ((t & 3) << 2) | ((t >> 3) & 3); }        // 16 pieces a row
__device__ inline int swz8(int t) { return (((t >> 1) & 1) << 2) | ((t >> 3) & 3); }   // 8 pieces a row
template <int DK>
__device__ inline int kq_off(int t, int piece) {  // byte offset of a key/query piece
    if constexpr (DK == 128)
        return t * 256 + ((piece ^ swz16(t)) << 4);
    else
        return t * 128 + ((piece ^ swz8(t)) << 4);
}
__device__ inline int mat_off(int arr, int t, int piece) {  // byte offset in the matrices
    return arr * (C * C * 2) + t * 128 + ((piece ^ swz8(t)) << 4);
}

constexpr int kOStride = 36;  // floats per output staging row (16-byte aligned, fewer conflicts)

template <int DK>
struct alignas(16) ScanLds {
    uint8_t K[2][C * DK * 2];
    uint8_t Q[2][C * DK * 2];
    uint8_t M[2][4 * C * C * 2];   // Linv hi, Linv lo, P hi, P lo
    uint8_t V[2][C * 32 * 2];      // the workgroup's 32 value columns, [t][32] bf16
    float G[2][256];               // gamma, e, beta (3 x 64), padded to 1 KiB
    float O[C * kOStride];         // output staging: token rows, the 32 value columns
    // Partial K S^T exchange between the two key halves (4 waves x 4 tiles x 64
    // lanes x 4); at dk = 128 the current stage's Q buffer, dead by then, holds it.
    float Xch[DK == 128 ? 4 : 4 * 4 * 64 * 4];
};

typedef short v4s __attribute__((ext_vector_type(4)));

template <int V>
struct IntC {
    static constexpr int value = V;
};

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// i % 4 of the 8 bytes addressed by lane 4 e + i / 4, for e = 0..3.  With lane
// j addressing row r0 + j / 4 at column c(j % 4) .. + 3 of a row-major 16-bit
// matrix, lane i receives rows r0 .. r0 + 3 of column c(i / 4) + i % 4.
__device__ inline bf16x4 read_tr(const uint8_t *p) {
    const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)p);
    return __builtin_bit_cast(bf16x4, r);
}

__device__ inline bf16x8 lds16(const uint8_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// Wave (g, kh) of a scan workgroup owns value rows 16 g .. 16 g + 15 (of the
// workgroup's 32) and keys 64 kh .. 64 kh + 63 of their state; of the output
// tiles it finalises tt = kh and kh + 2, i.e. tokens 32p + 8a + 4kh + r.

// Store a chunk's finished outputs (64 tokens x the workgroup's 32 value
// columns, every wave's, after a barrier) from the staging buffer: wave w takes
// tokens 16w .. 16w + 15 as whole 128-byte rows, 8 a store (tokens < n).  Whole
// lines: half-line streaming stores of the same bytes drain markedly slower.
// obase points at o for the chunk's first token and the workgroup's first value
// column; ostride is one token.
template <int DK>
__device__ inline void scan_store_o(const ScanLds<DK> &sm, int n, int lane, int w,
                                    float *__restrict__ obase, size_t ostride) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = 16 * w + 8 * i + (lane >> 3);
        const int col = 4 * (lane & 7);
        const float4 v4 = *reinterpret_cast<const float4 *>(&sm.O[row * kOStride + col]);
        if (row < n) st_stream(obase + size_t(row) * ostride + col, v4);
    }
}

// State-coupled products of one chunk (the products of chunk_state) for wave
// (g, KH), from LDS stage SG, in the operand mapping above.  st holds the
// wave's quarter of the state: st[kt][r] is key 32 (KT/2) + 8 lg + 4 (KT%2) + r
// of value row irow, KT = 4 KH + kt (dk = 128; dk = 64: 2 KH + kt).  The pair
// (g, 0), (g, 1) exchanges partial K S^T and Q S^T through LDS, with the
// workgroup's barriers between.  Outputs stay in the staging buffer.
//
// Every LDS operand is read in two batches ahead of its use: the key, query,
// value and gate operands first, then (while the partial products run) the
// Linv, P and transposed-key operands, so the wave waits on LDS latency about
// twice per chunk rather than once per operand.  Stage and key half are
// compile-time, so every LDS address is a per-lane base plus a constant.
template <int DK, int SG, int KH>
__device__ __forceinline__ void scan_chunk(ScanLds<DK> &sm, float (&st)[DK / 32][4], int n, int lane, int g) {
    constexpr int KTH = DK / 32;   // 16-key state tiles per key half
    constexpr int KBH = DK / 64;   // 32-key contraction blocks per key half
    const int lr = lane & 15, lg = lane >> 4;
    const uint8_t *Kc = sm.K[SG], *Qc = sm.Q[SG], *Mc = sm.M[SG];
    const float *Gc = sm.G[SG];
    float *xch = DK == 128 ? reinterpret_cast<float *>(sm.Q[SG]) : sm.Xch;

    // Batch 1: keys and queries over this wave's keys (A operands of K S^T and
    // Q S^T), the workgroup's value columns (transposed) and the gates.  Lane
    // (lr, lg) of tile 2p + hh holds tokens t0 + r, t0 = 32p + 8lg + 4hh.
    bf16x8 ka[4][KBH], qa[4][KBH];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int t = tau(tt, lr);
#pragma unroll
        for (int p = 0; p < KBH; ++p) {
            const int piece = 4 * (KBH * KH + p) + lg;
            ka[tt][p] = lds16(Kc + kq_off<DK>(t, piece));
            qa[tt][p] = lds16(Qc + kq_off<DK>(t, piece));
        }
    }
    float4 ga[2][2], be[2][2], ee[2][2];
    bf16x4 vt[2][2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int t0 = 32 * p + 8 * lg + 4 * hh;
            vt[p][hh] = read_tr(sm.V[SG] + (t0 + (lr >> 2)) * 64 + 32 * g + 8 * (lr & 3));
            ga[p][hh] = *reinterpret_cast<const float4 *>(Gc + t0);
            ee[p][hh] = *reinterpret_cast<const float4 *>(Gc + 64 + t0);
            be[p][hh] = *reinterpret_cast<const float4 *>(Gc + 128 + t0);
        }
    const float glast = Gc[n - 1];
    __builtin_amdgcn_sched_barrier(0);

    // Partial X = K S^T and Y = Q S^T over this wave's keys.
    f32x4 X[4], Y[4];
    {
        Split8 sB[KBH];
#pragma unroll
        for (int p = 0; p < KBH; ++p) {
            const float x[8] = {st[2 * p][0], st[2 * p][1], st[2 * p][2], st[2 * p][3],
                                st[2 * p + 1][0], st[2 * p + 1][1], st[2 * p + 1][2], st[2 * p + 1][3]};
            sB[p] = split8(x);
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            X[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
            Y[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < KBH; ++p) {
                X[tt] = mma(ka[tt][p], sB[p].hi, X[tt]);
                X[tt] = mma(ka[tt][p], sB[p].lo, X[tt]);
                Y[tt] = mma(qa[tt][p], sB[p].hi, Y[tt]);
                Y[tt] = mma(qa[tt][p], sB[p].lo, Y[tt]);
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // Batch 2: Linv tiles (tt, p <= tt/2) for D, P tiles of this wave's output
    // tiles tt = KH + 2hh (p <= hh), and K^T for the state update: tile kt's A
    // operand is K^T at keys 32 (KT/2) + 8 (lr/4) + 4 (KT%2) + lr%4 (row lr) and
    // tokens 32p + 8lg + {0..7} (slots), two transposed reads of 4 token rows.
    Split8 li[6], pm[3];
    bf16x8 kt_a[KTH][2];
#pragma unroll
    for (int tt = 0, u = 0; tt < 4; ++tt) {
        const int t = tau(tt, lr);
#pragma unroll
        for (int p = 0; p <= tt / 2; ++p, ++u) {
            li[u].hi = lds16(Mc + mat_off(0, t, 4 * p + lg));
            li[u].lo = lds16(Mc + mat_off(1, t, 4 * p + lg));
        }
    }
#pragma unroll
    for (int hh = 0, u = 0; hh < 2; ++hh) {
        const int t = tau(KH + 2 * hh, lr);
#pragma unroll
        for (int p = 0; p <= hh; ++p, ++u) {
            pm[u].hi = lds16(Mc + mat_off(2, t, 4 * p + lg));
            pm[u].lo = lds16(Mc + mat_off(3, t, 4 * p + lg));
        }
    }
#pragma unroll
    for (int kt = 0; kt < KTH; ++kt) {
        const int KTg = KTH * KH + kt;
        const int piece = 4 * (KTg >> 1) + (lr & 3), h8 = (KTg & 1) << 3;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int ta = 32 * p + 8 * lg + (lr >> 2);
            kt_a[kt][p] = cat4(read_tr(Kc + kq_off<DK>(ta, piece) + h8), read_tr(Kc + kq_off<DK>(ta + 4, piece) + h8));
        }
    }

    // Exchange: every wave is done reading Q (the exchange space at dk = 128);
    // each wave posts its partial X, and its partial Y of the tiles its partner
    // finalises into those tiles' output staging slots.
    __syncthreads();
    {
        float *mine = xch + (2 * g + KH) * 1024 + lane * 4;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
            *reinterpret_cast<float4 *>(mine + tt * 256) = make_float4(X[tt][0], X[tt][1], X[tt][2], X[tt][3]);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            constexpr int o = 1 - KH;
            const int tt = o + 2 * hh, t0 = 32 * hh + 8 * lg + 4 * o;
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.O[(t0 + r) * kOStride + 16 * g + lr] = Y[tt][r];
        }
    }
    __syncthreads();
    {
        const float *theirs = xch + (2 * g + (1 - KH)) * 1024 + lane * 4;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const float4 o4 = *reinterpret_cast<const float4 *>(theirs + tt * 256);
            X[tt][0] += o4.x;
            X[tt][1] += o4.y;
            X[tt][2] += o4.z;
            X[tt][3] += o4.w;
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int tt = KH + 2 * hh, t0 = 32 * hh + 8 * lg + 4 * KH;
#pragma unroll
            for (int r = 0; r < 4; ++r) Y[tt][r] += sm.O[(t0 + r) * kOStride + 16 * g + lr];
        }
    }
    // R = diag(beta) (V - diag(gamma) X).
    Split8 rB[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        float x[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                x[4 * hh + r] = (&be[p][hh].x)[r] *
                                (static_cast<float>(vt[p][hh][r]) - (&ga[p][hh].x)[r] * X[2 * p + hh][r]);
        rB[p] = split8(x);
    }
    // D = Linv R (Linv is lower triangular: p <= tt / 2).
    f32x4 D[4];
#pragma unroll
    for (int tt = 0, u = 0; tt < 4; ++tt) {
        D[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p <= tt / 2; ++p, ++u) D[tt] = mma3(li[u], rB[p], D[tt]);
    }
    // D split twice: as is (for P D) and scaled by e (for the state update).
    Split8 dB[2], eB[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        float x[8], y[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                x[4 * hh + r] = D[2 * p + hh][r];
                y[4 * hh + r] = (&ee[p][hh].x)[r] * D[2 * p + hh][r];
            }
        dB[p] = split8(x);
        eB[p] = split8(y);
    }
    // S <- gamma_last S + K^T diag(e) D over this wave's keys.
#pragma unroll
    for (int kt = 0; kt < KTH; ++kt) {
        f32x4 U = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            U = mma(kt_a[kt][p], eB[p].hi, U);
            U = mma(kt_a[kt][p], eB[p].lo, U);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) st[kt][r] = glast * st[kt][r] + U[r];
    }
    // O = diag(gamma) Y + P D for this wave's tiles KH and KH + 2, into staging.
#pragma unroll
    for (int hh = 0, u = 0; hh < 2; ++hh) {
        const int tt = KH + 2 * hh, t0 = 32 * hh + 8 * lg + 4 * KH;
        f32x4 Ot = Y[tt];
#pragma unroll
        for (int r = 0; r < 4; ++r) Ot[r] *= (&ga[hh][KH].x)[r];
#pragma unroll
        for (int p = 0; p <= hh; ++p, ++u) Ot = mma3(pm[u], dB[p], Ot);
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.O[(t0 + r) * kOStride + 16 * g + lr] = Ot[r];
    }
}

template <int DK, int DV>
__device__ __forceinline__ void scan_role(ScanLds<DK> &sm, int wg, int nscan, float *__restrict__ S,
                                          const __hip_bfloat16 *__restrict__ q,
                                          const __hip_bfloat16 *__restrict__ k,
                                          const __hip_bfloat16 *__restrict__ v, int L, int H, int nchunks,
                                          int cbeg, int cend, const uint8_t *__restrict__ ws,
                                          float *__restrict__ o) {
    constexpr int RS = 32;                  // value rows per workgroup
    constexpr int NW = 4;                   // waves: 2 row groups x 2 key halves
    constexpr int SLICES = DV / RS;
    constexpr int KTH = DK / 32;            // 16-key state tiles per wave
    constexpr int NKQ = C * DK * 2 / 1024;  // 1 KiB blocks of a key or query chunk
    static_assert(SLICES * RS == DV && NKQ % NW == 0, "tiling");

    // Workgroup i runs on XCD i % 8.  The SLICES workgroups of one head read the
    // same keys, queries and chunk matrices, so they are placed on one XCD, where
    // its L2 serves the repeats: within each group of 8 SLICES workgroups, XCD x
    // takes head 8 g + x, slice = position / 8.  A ragged last group maps linearly.
    const int grp = 8 * SLICES;
    int bh, slice;
    if (wg < nscan / grp * grp) {
        const int g0 = wg / grp, r = wg - g0 * grp;
        bh = 8 * g0 + (r & 7);
        slice = r >> 3;
    } else {
        bh = wg / SLICES;
        slice = wg - bh * SLICES;
    }
    const int b = bh / H, h = bh - b * H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = w >> 1, kh = w & 1;        // row group, key half
    const int irow = slice * RS + 16 * g + lr;

    // State quarter in registers: st[kt][r] = S[irow][32 (KT/2) + 8 lg + 4 (KT%2) + r],
    // KT = KTH kh + kt.
    float *Srow = S + (size_t(bh) * DV + irow) * DK;
    float st[KTH][4];
#pragma unroll
    for (int kt = 0; kt < KTH; ++kt) {
        const int KT = KTH * kh + kt;
        const float4 s4 = *reinterpret_cast<const float4 *>(Srow + 32 * (KT >> 1) + 8 * lg + 4 * (KT & 1));
        st[kt][0] = s4.x;
        st[kt][1] = s4.y;
        st[kt][2] = s4.z;
        st[kt][3] = s4.w;
    }

    const __hip_bfloat16 *kb = k + (size_t(b) * L * H + h) * DK;   // token row t at + t H DK
    const __hip_bfloat16 *qb = q + (size_t(b) * L * H + h) * DK;
    const __hip_bfloat16 *vb = v + (size_t(b) * L * H + h) * DV + slice * RS;
    const uint8_t *wsh = ws + size_t(bh) * nchunks * kPrepBytes;
    const size_t kstride = size_t(H) * DK, vstride = size_t(H) * DV;

    // Copy chunk cn's operands into stage cn & 1.  Wave w takes the 1 KiB blocks
    // w, w + 4, ...  Full chunks use uniform bases and per-lane offsets computed
    // once; a partial last chunk clamps each lane's row to the last token (finite
    // data that beta = e = 0 cancels; those outputs are not stored).
    constexpr int RPB = 1024 / (2 * DK);      // key rows per 1 KiB block
    const uint32_t kstride_b = uint32_t(kstride) * 2, vstride_b = uint32_t(vstride) * 2;
    auto kq_piece = [&](int blk) {           // swizzled piece of this lane in K/Q block blk
        const int row = blk * RPB + lane / (64 / RPB), slot = lane % (64 / RPB);
        return DK == 128 ? (slot ^ swz16(row)) : (slot ^ swz8(row));
    };
    uint32_t vo_kq[NKQ / NW], vo_m[32 / NW];
#pragma unroll
    for (int u = 0; u < NKQ / NW; ++u)
        vo_kq[u] = uint32_t(lane / (64 / RPB)) * kstride_b + 16u * uint32_t(kq_piece(NW * u + w));
#pragma unroll
    for (int u = 0; u < 32 / NW; ++u) {
        const int blk = NW * u + w, mrow = (blk & 7) * 8 + (lane >> 3);  // row of the block in its matrix
        vo_m[u] = uint32_t(lane >> 3) * 128u + 16u * uint32_t((lane & 7) ^ swz8(mrow));
    }
    const uint32_t vo_v = uint32_t(lane >> 2) * vstride_b + 16u * uint32_t(lane & 3);
    const uint32_t vo_g = 16u * uint32_t(min(lane, 3 * C / 4 - 1));
    auto issue = [&](int cn) {
        const int s = (cn - cbeg) & 1, c0 = cn * C;
        const uint8_t *rec = wsh + size_t(cn) * kPrepBytes;
        const uint32_t lk = lds_addr(sm.K[s]), lq = lds_addr(sm.Q[s]), lm = lds_addr(sm.M[s]),
                       lv = lds_addr(sm.V[s]);
        if (c0 + C <= L) {
            const uint8_t *kc = reinterpret_cast<const uint8_t *>(kb + size_t(c0) * kstride);
            const uint8_t *qc = reinterpret_cast<const uint8_t *>(qb + size_t(c0) * kstride);
            const uint8_t *vc = reinterpret_cast<const uint8_t *>(vb + size_t(c0) * vstride);
#pragma unroll
            for (int u = 0; u < NKQ / NW; ++u) {
                const int blk = NW * u + w;
                const size_t boff = size_t(blk * RPB) * kstride_b;
                dma16s(kc + boff, vo_kq[u], lk + blk * 1024);
                dma16s(qc + boff, vo_kq[u], lq + blk * 1024);
            }
            dma16s(vc + size_t(16 * w) * vstride_b, vo_v, lv + w * 1024);
        } else {
#pragma unroll
            for (int u = 0; u < NKQ / NW; ++u) {
                const int blk = NW * u + w, row = blk * RPB + lane / (64 / RPB);
                const size_t off = size_t(min(c0 + row, L - 1)) * kstride + 8 * kq_piece(blk);
                dma16(kb + off, lk + blk * 1024);
                dma16(qb + off, lq + blk * 1024);
            }
            const int row = 16 * w + (lane >> 2);
            dma16(vb + size_t(min(c0 + row, L - 1)) * vstride + 8 * (lane & 3), lv + w * 1024);
        }
#pragma unroll
        for (int u = 0; u < 32 / NW; ++u) {
            const int blk = NW * u + w;
            dma16s(rec + blk * 1024, vo_m[u], lm + blk * 1024);
        }
        if (w == 0) dma16s(rec + kPrepMatBytes, vo_g, lds_addr(sm.G[s]));
    };

    // Outputs of chunk c leave through the staging buffer at the top of chunk
    // c + 1, so the wait at the top of each chunk finds the stores long done.
    float *ob = o + (size_t(b) * L * H + h) * DV + slice * RS;
    const size_t ostride = size_t(H) * DV;
    // One step per chunk; the loop is unrolled over the two LDS stages so that
    // stage and key half are compile-time inside scan_chunk.
    auto step = [&](int c, auto stage) __attribute__((always_inline)) {
        constexpr int SG = decltype(stage)::value;
        const int c0 = c * C, n = min(C, L - c0);
        // This chunk's copies (issued one chunk ago) have landed, for every wave,
        // and every wave is done with the buffers the next copies overwrite.
        __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) expcnt(7) lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (c > cbeg) scan_store_o<DK>(sm, C, lane, w, ob + size_t(c0 - C) * ostride, ostride);
        if (c + 1 < cend) issue(c + 1);
        asm volatile("" ::: "memory");
        if (kh)
            scan_chunk<DK, SG, 1>(sm, st, n, lane, g);
        else
            scan_chunk<DK, SG, 0>(sm, st, n, lane, g);
    };
    issue(cbeg);
    for (int c = cbeg; c < cend; c += 2) {
        step(c, IntC<0>{});
        if (c + 1 < cend) step(c + 1, IntC<1>{});
    }
    // The last chunk's outputs, once every wave has staged its part.
    __syncthreads();
    scan_store_o<DK>(sm, min(C, L - (cend - 1) * C), lane, w, ob + size_t(cend - 1) * C * ostride, ostride);

#pragma unroll
    for (int kt = 0; kt < KTH; ++kt) {
        const int KT = KTH * kh + kt;
        *reinterpret_cast<float4 *>(Srow + 32 * (KT >> 1) + 8 * lg + 4 * (KT & 1)) =
            make_float4(st[kt][0], st[kt][1], st[kt][2], st[kt][3]);
    }
}

template <int DK>
union FusedLds {
    PrepSmem<DK> prep;
    ScanLds<DK> scan;
};

// Prep records of chunks [pbeg, pend) for every (instance, head): unit u =
// chunk-relative index * heads + head, workgroup u % nprep; NWS waves a unit.
template <int DK, int NWS>
__device__ __forceinline__ void prep_role(PrepSmem<DK> &sm, int wg, int nprep, const __hip_bfloat16 *__restrict__ q,
                                          const __hip_bfloat16 *__restrict__ k, const float *__restrict__ g,
                                          const float *__restrict__ beta, int L, int H, int heads, int nchunks,
                                          int pbeg, int pend, uint8_t *__restrict__ ws) {
    const int units = heads * (pend - pbeg);
    for (int u = wg; u < units; u += nprep) {
        const int c = pbeg + u / heads, bh = u % heads;
        __syncthreads();  // the previous unit's LDS reads are done
        prep_unit<DK, NWS>(sm, q, k, g, beta, L, H, nchunks, ws, bh, c);
    }
}

// One stage of the pipelined two-phase schedule: workgroups [0, nprep) build
// the prep records of chunks [pbeg, pend) while workgroups [nprep, nprep +
// nscan) scan chunks [cbeg, cend), whose records an earlier launch built.  The
// two roles share nothing, so no workgroup waits on another; the prep runs on
// the compute units the scan leaves idle.
template <int DK, int DV>
__global__ __launch_bounds__(256) void prefill_stage_kernel(
    float *__restrict__ S, const __hip_bfloat16 *__restrict__ q, const __hip_bfloat16 *__restrict__ k,
    const __hip_bfloat16 *__restrict__ v, const float *__restrict__ g, const float *__restrict__ beta, int L,
    int H, int heads, int nchunks, int cbeg, int cend, int pbeg, int pend, int nprep, int nscan,
    uint8_t *__restrict__ ws, float *__restrict__ o) {
    __shared__ FusedLds<DK> sm;
    const int wg = blockIdx.x;
    if (wg < nprep)
        prep_role<DK, 4>(sm.prep, wg, nprep, q, k, g, beta, L, H, heads, nchunks, pbeg, pend, ws);
    else
        scan_role<DK, DV>(sm.scan, wg - nprep, nscan, S, q, k, v, L, H, nchunks, cbeg, cend, ws, o);
}

// Prep records of chunks [pbeg, pend) on the whole chip (two workgroups a
// compute unit: this kernel needs only the prep's LDS).  Nothing runs beside
// it, so each unit takes 8 waves (the Gram tiles and the split spread over
// twice the waves; the inverse keeps its 4): the unit's latency is the launch's.
template <int DK>
__global__ __launch_bounds__(512) void prefill_prep_kernel(
    const __hip_bfloat16 *__restrict__ q, const __hip_bfloat16 *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, int L, int H, int heads, int nchunks, int pbeg, int pend,
    uint8_t *__restrict__ ws) {
    __shared__ PrepSmem<DK> sm;
    prep_role<DK, 8>(sm, blockIdx.x, gridDim.x, q, k, g, beta, L, H, heads, nchunks, pbeg, pend, ws);
}

// ---------------------------------------------------------------------------
// One pass, many heads (dv = 128): one workgroup of 4 waves per (instance, head),
// wave w owning value rows 32 w .. 32 w + 31 over all keys, so the state-coupled
// products need no exchange between waves.  76 KB of LDS, so two heads share a
// compute unit and one head's chunk chain runs in the other's latency shadows.
// Per chunk:
//   P0  K and Q copied global -> LDS (swizzled rows), gates by wave 0;
//   P1  Gram tiles: A = strictly-lower(beta Gamma K K^T) in fp32, P = lower-incl
//       (Gamma Q K^T) split into bf16 hi/lo straight from the MFMA tiles (a row
//       band of each per wave); Y = Q S^T for the wave's 32 rows;
//   P2  the chunk's values copied into Q's space; Linv = (I + A)^{-1} in place
//       over A;
//   P3  Linv split into bf16 hi/lo, in place over A (read, barrier, write);
//   P4  X = K S^T, R (values by transposed LDS reads), D = Linv R,
//       O = diag(gamma) Y + P D and S <- gamma_last S + K^T diag(e) D.
// Operands follow the scan's mapping (tau token order, st[kt][r] = key
// 32 (kt/2) + 8 lg + 4 (kt%2) + r), with two 16-row tiles per wave.
// ---------------------------------------------------------------------------
template <int DK>
struct alignas(16) PassLds {
    uint8_t K[C * DK * 2];
    union {
        uint8_t Q[C * DK * 2];         // queries (P0 - P1)
        uint8_t V[C * 128 * 2];        // then the chunk's values, [t][dv = 128] (P2 - P4)
    };
    uint8_t PM[2 * C * C * 2];         // P hi, P lo
    union {
        float A[C][C + 4];             // A, then Linv in place (P1 - P3)
        uint8_t Li[2 * C * C * 2];     // Linv hi, Linv lo (P3 - P4)
    };
    float scr[4 * 640];                // the inverse's scratch
    float G[C], gam[C], ee[C], bet[C];
};

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

template <int DK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefill_pass_kernel(
    float *__restrict__ S, const __hip_bfloat16 *__restrict__ q, const __hip_bfloat16 *__restrict__ k,
    const __hip_bfloat16 *__restrict__ v, const float *__restrict__ g, const float *__restrict__ beta, int L,
    int H, float *__restrict__ o) {
    constexpr int DV = 128, NW = 4;
    constexpr int KT = DK / 16, KB = DK / 32;
    constexpr int NKQ = C * DK * 2 / 1024;   // 1 KiB blocks of a key or query chunk
    constexpr int RPB = 1024 / (2 * DK);     // rows per block
    static_assert(NKQ % NW == 0, "every wave copies the same number of blocks");
    __shared__ PassLds<DK> sm;

    const int bh = blockIdx.x, b = bh / H, h = bh - b * H;
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Value rows: lane column lr of row tile rt is row 32 w + 2 lr + rt, so a
    // lane's two rows are adjacent (one 8-byte output store per token).
    int irow[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) irow[rt] = 32 * w + 2 * lr + rt;

    // State: st[rt][kt][r] = S[irow[rt]][32 (kt/2) + 8 lg + 4 (kt%2) + r].
    float st[2][KT][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const float *Srow = S + (size_t(bh) * DV + irow[rt]) * DK;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            const float4 s4 = *reinterpret_cast<const float4 *>(Srow + 32 * (kt >> 1) + 8 * lg + 4 * (kt & 1));
            st[rt][kt][0] = s4.x;
            st[rt][kt][1] = s4.y;
            st[rt][kt][2] = s4.z;
            st[rt][kt][3] = s4.w;
        }
    }
    const size_t kstride = size_t(H) * DK, vstride = size_t(H) * DV;
    const uint32_t kstride_b = uint32_t(kstride) * 2;
    const __hip_bfloat16 *kb = k + (size_t(b) * L * H + h) * DK;
    const __hip_bfloat16 *qb = q + (size_t(b) * L * H + h) * DK;
    const uint16_t *vbase = reinterpret_cast<const uint16_t *>(v) + (size_t(b) * L * H + h) * DV;
    auto kq_piece = [&](int blk) {
        const int row = blk * RPB + lane / (64 / RPB), slot = lane % (64 / RPB);
        return DK == 128 ? (slot ^ swz16(row)) : (slot ^ swz8(row));
    };
    uint32_t vo_kq[NKQ / NW];
#pragma unroll
    for (int u = 0; u < NKQ / NW; ++u)
        vo_kq[u] = uint32_t(lane / (64 / RPB)) * kstride_b + 16u * uint32_t(kq_piece(NW * u + w));
    const uint32_t lk = lds_addr(sm.K), lq = lds_addr(sm.Q), lv = lds_addr(sm.V);
    const uint32_t vstride_b = uint32_t(vstride) * 2;
    // V copies: lane l fills LDS slot l % 16 of row l / 16 of a 4-row block; rows
    // keep their 16-byte pieces in the order slot = piece ^ vswz(row), vswz(row) =
    // 4 ((row / 8) % 4), so the reads of rows 8 apart (one per lane group) hit
    // different banks.  Block blk's rows share row / 8 = blk / 2.
    auto vswz = [](int row) { return 4 * ((row >> 3) & 3); };
    uint32_t vo_v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
        vo_v[u] = uint32_t(lane >> 4) * vstride_b + 16u * uint32_t((lane & 15) ^ vswz(4 * (NW * u + w)));

    // Per-lane LDS offsets of the P4 operands (aKQ, aM, aTR, set per chunk).  In
    // the tau order a result tile's token is t = T(tt) + tl, T(tt) = 32 (tt/2) +
    // 4 (tt%2) a constant and tl = 8 (lr/4) + lr%4 the lane's part, and every
    // swizzle term depends on tl alone: an operand address is a per-lane offset
    // (one per contraction block) plus a compile-time constant, which the LDS
    // instructions take as their immediate offset.  Likewise the K^T reads of the
    // state update (rows ta = 32 p + 8 lg + lr/4, + 4; piece 4 (kt/2) + lr%4):
    // the swizzle of ta depends on tal = 8 lg + lr/4 alone.
    auto Tc = [](int tt) { return 32 * (tt >> 1) + 4 * (tt & 1); };

    const int nchunks = (L + C - 1) / C;
    for (int c = 0; c < nchunks; ++c) {
        const int c0 = c * C, n = min(C, L - c0);
        const size_t row0 = size_t(b) * L + c0;
        // The lane index made opaque per chunk: the per-lane addresses below are
        // recomputed each chunk (a few VALU) rather than held across the loop.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int lr = ln & 15, lg = ln >> 4;
        const int irow[2] = {32 * w + 2 * lr, 32 * w + 2 * lr + 1};
        const int tl = 8 * (lr >> 2) + (lr & 3), tal = 8 * lg + (lr >> 2);
        uint32_t aKQ[KB], aM[2], aTR[KT / 2];
#pragma unroll
        for (int p = 0; p < KB; ++p) aKQ[p] = kq_off<DK>(tl, 4 * p + lg);
#pragma unroll
        for (int p = 0; p < 2; ++p) aM[p] = mat_off(0, tl, 4 * p + lg);
#pragma unroll
        for (int kk = 0; kk < KT / 2; ++kk) aTR[kk] = kq_off<DK>(tal, 4 * kk + (lr & 3));
        // P0: gates' inputs, the chunk's keys and queries into LDS.
        float gt = 0.f, bt = 0.f;
        if (w == 0) {
            const size_t gi = (row0 + min(ln, n - 1)) * H + h;
            gt = g[gi];
            bt = beta[gi];
        }
        asm volatile("" ::: "memory");
        if (n == C) {
            const uint8_t *kc = reinterpret_cast<const uint8_t *>(kb + size_t(c0) * kstride);
            const uint8_t *qc = reinterpret_cast<const uint8_t *>(qb + size_t(c0) * kstride);
#pragma unroll
            for (int u = 0; u < NKQ / NW; ++u) {
                const int blk = NW * u + w;
                const size_t boff = size_t(blk * RPB) * kstride_b;
                dma16s_nt(kc + boff, vo_kq[u], lk + blk * 1024);
                dma16s_nt(qc + boff, vo_kq[u], lq + blk * 1024);
            }
        } else {
#pragma unroll
            for (int u = 0; u < NKQ / NW; ++u) {
                const int blk = NW * u + w, row = blk * RPB + lane / (64 / RPB);
                const size_t off = size_t(min(c0 + row, L - 1)) * kstride + 8 * kq_piece(blk);
                dma16_nt(kb + off, lk + blk * 1024);
                dma16_nt(qb + off, lq + blk * 1024);
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0): the copies (and the gate inputs) have landed
        asm volatile("" ::: "memory");
        if (w == 0) chunk_gates(sm, gt, bt, n, lane);
        __syncthreads();


        // P1: Gram tiles, transposed so that a lane holds four consecutive j of one
        // t: wave w takes a row band of A (from K K^T) and one of P (from Q K^T),
        // all four tiles of each (the masks zero what lies above the diagonal),
        // written as one 16-byte store of A[t][j .. j + 3] and two 8-byte stores of
        // P's hi and lo parts per tile.  The j side and P's band take rows in the
        // tau order, which the key/query and matrix swizzles keep free of bank
        // conflicts; A's band keeps rows 16 w .. 16 w + 15, for which its padded
        // fp32 rows are conflict-free.
        {
            const int ta = 16 * w + lr, tp = tau(3 - w, lr);   // the lane's t in each band
            f32x4 aT[4], pT[4];
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) aT[jt] = pT[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb2 = 0; kb2 < KB; ++kb2) {
                const bf16x8 kt_b = lds16(sm.K + kq_off<DK>(ta, 4 * kb2 + lg));
                const bf16x8 qt_b = lds16(sm.Q + aKQ[kb2] + Tc(3 - w) * 2 * DK);
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) {
                    const bf16x8 kj = lds16(sm.K + aKQ[kb2] + Tc(jt) * 2 * DK);
                    aT[jt] = mma(kj, kt_b, aT[jt]);
                    pT[jt] = mma(kj, qt_b, pT[jt]);
                }
            }
            const float Gta = sm.G[ta], Gtp = sm.G[tp], bta = sm.bet[ta];
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                const int j0 = Tc(jt) + 8 * lg;   // rows 4 lg + r of tile jt: tau(jt, 4 lg + r)
                const float4 Gj = *reinterpret_cast<const float4 *>(&sm.G[j0]);
                float av[4], pv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = j0 + r;
                    av[r] = j < ta ? bta * __expf(Gta - (&Gj.x)[r]) * aT[jt][r] : 0.f;
                    pv[r] = j <= tp ? __expf(Gtp - (&Gj.x)[r]) * pT[jt][r] : 0.f;
                }
                *reinterpret_cast<float4 *>(&sm.A[ta][j0]) = make_float4(av[0], av[1], av[2], av[3]);
                typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                typedef float f32x2 __attribute__((ext_vector_type(2)));
                uint32_t hi[2], lo[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const uint32_t u = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{pv[2 * i], pv[2 * i + 1]}), bf16x2));
                    hi[i] = u;
                    const float h0 = __uint_as_float(u << 16), h1 = __uint_as_float(u & 0xffff0000u);
                    lo[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{pv[2 * i] - h0, pv[2 * i + 1] - h1}), bf16x2));
                }
                const int off = mat_off(0, tp, j0 >> 3) + 2 * (j0 & 7);
                *reinterpret_cast<uint2 *>(sm.PM + off) = make_uint2(hi[0], hi[1]);
                *reinterpret_cast<uint2 *>(sm.PM + off + C * C * 2) = make_uint2(lo[0], lo[1]);
            }
        }
        // Y = Q S^T for the wave's two row tiles (tau token order): Q's last use.
        f32x4 Y[2][4];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) Y[rt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < KB; ++p) {
            Split8 sB[2];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const float x[8] = {st[rt][2 * p][0], st[rt][2 * p][1], st[rt][2 * p][2], st[rt][2 * p][3],
                                    st[rt][2 * p + 1][0], st[rt][2 * p + 1][1], st[rt][2 * p + 1][2],
                                    st[rt][2 * p + 1][3]};
                sB[rt] = split8(x);
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const bf16x8 qa = lds16(sm.Q + aKQ[p] + Tc(tt) * 2 * DK);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    Y[rt][tt] = mma(qa, sB[rt].hi, Y[rt][tt]);
                    Y[rt][tt] = mma(qa, sB[rt].lo, Y[rt][tt]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();   // A and P complete; Q is dead
        // The chunk's values into Q's space (V), [t][DV] bf16 rows (block = 4
        // rows), landing while the inverse runs.
        if (n == C) {
            const uint8_t *vc = reinterpret_cast<const uint8_t *>(vbase + size_t(c0) * vstride);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int blk = NW * u + w;
                dma16s_nt(vc + size_t(4 * blk) * vstride_b, vo_v[u], lv + blk * 1024);
            }
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int blk = NW * u + w, row = 4 * blk + (ln >> 4);
                dma16_nt(vbase + size_t(min(c0 + row, L - 1)) * vstride + 8 * ((ln & 15) ^ vswz(row)),
                         lv + blk * 1024);
            }
        }

        // P2: Linv = (I + A)^{-1} in place (each block is read before it is overwritten).
        tri_inverse(sm.A, sm.A, sm.scr, w, ln, [] {});
        // P3: Linv split into hi/lo (zero in the strictly upper blocks), in place.
        Split8 lsp[C * C / 8 / 256];
#pragma unroll
        for (int u = 0; u < C * C / 8 / 256; ++u) {
            const int idx = tid + 256 * u, t = idx / (C / 8), j8 = (idx - t * (C / 8)) * 8;
            float a[8];
            *reinterpret_cast<float4 *>(a) = *reinterpret_cast<const float4 *>(&sm.A[t][j8]);
            *reinterpret_cast<float4 *>(a + 4) = *reinterpret_cast<const float4 *>(&sm.A[t][j8 + 4]);
            if ((j8 >> 4) > (t >> 4)) {
#pragma unroll
                for (int e = 0; e < 8; ++e) a[e] = 0.f;
            }
            lsp[u] = split8(a);
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < C * C / 8 / 256; ++u) {
            const int idx = tid + 256 * u, t = idx / (C / 8), j8 = (idx - t * (C / 8)) * 8;
            *reinterpret_cast<bf16x8 *>(sm.Li + mat_off(0, t, j8 >> 3)) = lsp[u].hi;
            *reinterpret_cast<bf16x8 *>(sm.Li + mat_off(1, t, j8 >> 3)) = lsp[u].lo;
        }
        __syncthreads();

        // P4: the wave's state-coupled products.  X = K S^T.
        f32x4 X[2][4];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) X[rt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < KB; ++p) {
            Split8 sB[2];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const float x[8] = {st[rt][2 * p][0], st[rt][2 * p][1], st[rt][2 * p][2], st[rt][2 * p][3],
                                    st[rt][2 * p + 1][0], st[rt][2 * p + 1][1], st[rt][2 * p + 1][2],
                                    st[rt][2 * p + 1][3]};
                sB[rt] = split8(x);
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const bf16x8 ka = lds16(sm.K + aKQ[p] + Tc(tt) * 2 * DK);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    X[rt][tt] = mma(ka, sB[rt].hi, X[rt][tt]);
                    X[rt][tt] = mma(ka, sB[rt].lo, X[rt][tt]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // The chunk's values have landed in Q's space (every wave's copies).
        __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0)
        __syncthreads();
        // Gates of the lane's tokens t0 .. t0 + 3, t0 = 32 p + 8 lg + 4 hh, read where used.
        auto gate4 = [&](const float *arr, int p, int hh) {
            return *reinterpret_cast<const float4 *>(arr + 32 * p + 8 * lg + 4 * hh);
        };
        // R = diag(beta) (V - diag(gamma) X), split as the B operand of D = Linv R.
        Split8 rB[2][2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            float4 ga[2], be[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                ga[hh] = gate4(sm.gam, p, hh);
                be[hh] = gate4(sm.bet, p, hh);
            }
            // v[t][irow[0]] and v[t][irow[1]] (adjacent) by one 4-byte read per token.
            float vv[2][2][4];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int vrow = 32 * p + 8 * lg + 4 * hh + r, vbyte = 2 * (32 * w + 2 * lr);
                    const uint32_t pair = *reinterpret_cast<const uint32_t *>(
                        sm.V + vrow * 2 * DV + ((((vbyte >> 4) ^ vswz(vrow)) << 4) | (vbyte & 15)));
                    vv[0][hh][r] = __uint_as_float(pair << 16);
                    vv[1][hh][r] = __uint_as_float(pair & 0xffff0000u);
                }
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                float x[8];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        x[4 * hh + r] = (&be[hh].x)[r] * (vv[rt][hh][r] - (&ga[hh].x)[r] * X[rt][2 * p + hh][r]);
                rB[rt][p] = split8(x);
            }
        }
        // D = Linv R (p <= tt / 2).
        f32x4 D[2][4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            D[0][tt] = D[1][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p <= tt / 2; ++p) {
                Split8 li;
                li.hi = lds16(sm.Li + aM[p] + Tc(tt) * 128);
                li.lo = lds16(sm.Li + aM[p] + Tc(tt) * 128 + C * C * 2);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) D[rt][tt] = mma3(li, rB[rt][p], D[rt][tt]);
            }
        }
        // O = diag(gamma) Y + P D, stored for tokens < n (D split as is).
        {
            Split8 dB[2][2];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    float x[8];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                        for (int r = 0; r < 4; ++r) x[4 * hh + r] = D[rt][2 * p + hh][r];
                    dB[rt][p] = split8(x);
                }
            float *orow = o + (row0 * H + h) * DV;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const float4 ga = gate4(sm.gam, tt >> 1, tt & 1);
                f32x4 Ot[2] = {Y[0][tt], Y[1][tt]};
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) Ot[rt][r] *= (&ga.x)[r];
#pragma unroll
                for (int p = 0; p <= tt / 2; ++p) {
                    Split8 pm;
                    pm.hi = lds16(sm.PM + aM[p] + Tc(tt) * 128);
                    pm.lo = lds16(sm.PM + aM[p] + Tc(tt) * 128 + C * C * 2);
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt) Ot[rt] = mma3(pm, dB[rt][p], Ot[rt]);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tr = 32 * (tt >> 1) + 8 * lg + 4 * (tt & 1) + r;
                    if (tr < n) {
                        typedef float f32x2 __attribute__((ext_vector_type(2)));
                        __builtin_nontemporal_store(f32x2{Ot[0][r], Ot[1][r]},
                                                    reinterpret_cast<f32x2 *>(orow + size_t(tr) * vstride + irow[0]));
                    }
                }
            }
        }
        // D scaled by e and split, for the state update.
        Split8 eB[2][2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            float4 ee[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) ee[hh] = gate4(sm.ee, p, hh);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                float y[8];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int r = 0; r < 4; ++r) y[4 * hh + r] = (&ee[hh].x)[r] * D[rt][2 * p + hh][r];
                eB[rt][p] = split8(y);
            }
        }
        const float glast = sm.gam[n - 1];
        // S <- gamma_last S + K^T diag(e) D.
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            const int h8 = (kt & 1) << 3;
            bf16x8 kta[2];
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const uint8_t *base = sm.K + aTR[kt >> 1] + 32 * p * 2 * DK + h8;
                kta[p] = cat4(read_tr(base), read_tr(base + 4 * 2 * DK));
            }
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                f32x4 U = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    U = mma(kta[p], eB[rt][p].hi, U);
                    U = mma(kta[p], eB[rt][p].lo, U);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) st[rt][kt][r] = glast * st[rt][kt][r] + U[r];
            }
        }
        __syncthreads();   // the next chunk's copies overwrite K, Q and the matrices
    }

    {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int lr = ln & 15, lg = ln >> 4;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            float *Srow = S + (size_t(bh) * DV + 32 * w + 2 * lr + rt) * DK;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
                *reinterpret_cast<float4 *>(Srow + 32 * (kt >> 1) + 8 * lg + 4 * (kt & 1)) =
                    make_float4(st[rt][kt][0], st[rt][kt][1], st[rt][kt][2], st[rt][kt][3]);
        }
    }
}

template <int DK, int DV>
hipError_t launch_dk_dv(float *S, const void *q, const void *k, const void *v, const float *g,
                        const float *beta, int L, const gdn_shape &s, float *o, void *ws,
                        size_t ws_bytes, hipStream_t st) {
    auto *qq = static_cast<const __hip_bfloat16 *>(q);
    auto *kk = static_cast<const __hip_bfloat16 *>(k);
    auto *vv = static_cast<const __hip_bfloat16 *>(v);
    const long heads = long(s.B) * s.H;
    const int nchunks = (L + C - 1) / C;
    if (heads < kFewHeads && ws != nullptr && ws_bytes >= size_t(heads) * nchunks * kPrepBytes) {
        uint8_t *wsb = static_cast<uint8_t *>(ws);
        const int nscan = int(heads) * (DV / 32);
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 0;
        // Prep workgroups beside the scan: the compute units it leaves idle, in
        // multiples of 8 so scan workgroup i stays on XCD i % 8.
        const int nside = (cus - nscan) / 8 * 8;
        // Chunk segments: the first is prepped alone, each later one while the
        // scan walks the one before.  A side prep on the idle compute units
        // keeps pace with the scan chunk for chunk, so the segments are equal.
        // Short prompts, or a scan that leaves too few units idle, use one
        // segment (prep, then scan).
        constexpr int kSeg = 4;
        int bnd[kSeg + 2], nseg = 1;
        bnd[0] = 0;
        bnd[1] = nchunks;
        if (nchunks >= 4 * kSeg && nside >= 8 && 2 * nside >= nscan) {
            nseg = kSeg;
            for (int j = 1; j <= kSeg; ++j) bnd[j] = nchunks * j / kSeg;
        }
        bnd[nseg + 1] = nchunks;
        const int units0 = int(heads) * bnd[1];
        hipLaunchKernelGGL((prefill_prep_kernel<DK>), dim3(unsigned(units0)), dim3(512), 0, st, qq, kk, g, beta, L,
                           s.H, int(heads), nchunks, 0, bnd[1], wsb);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        for (int j = 0; j < nseg; ++j) {
            const int pbeg = bnd[j + 1], pend = j + 1 < nseg ? bnd[j + 2] : pbeg;
            const int nprep = pend > pbeg ? std::min(nside, int(heads) * (pend - pbeg) + 7) / 8 * 8 : 0;
            hipLaunchKernelGGL((prefill_stage_kernel<DK, DV>), dim3(unsigned(nprep + nscan)), dim3(256), 0, st, S,
                               qq, kk, vv, g, beta, L, s.H, int(heads), nchunks, bnd[j], bnd[j + 1], pbeg, pend,
                               nprep, nscan, wsb, o);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    // One pass: one workgroup per head.
    if constexpr (DV == 128) {
        hipLaunchKernelGGL((prefill_pass_kernel<DK>), dim3(unsigned(heads)), dim3(256), 0, st, S, qq, kk, vv, g,
                           beta, L, s.H, o);
    } else {
        hipLaunchKernelGGL((prefill_kernel<DK, DV, DV / 16>), dim3(unsigned(heads)), dim3(4 * DV), 0, st,
                           S, qq, kk, vv, g, beta, L, s.H, o);
    }
    return hipGetLastError();
}

}  // namespace

size_t prefill_workspace_bytes(const gdn_shape &shp, int L) {
    const long heads = long(shp.B) * shp.H;
    if (heads >= kFewHeads || L <= 0) return 0;
    return size_t(heads) * size_t((L + C - 1) / C) * kPrepBytes;
}

hipError_t launch_prefill(float *S, const void *q, const void *k, const void *v, const float *g,
                          const float *beta, int L, gdn_in_dtype dt, const gdn_shape &shp, float *o,
                          void *ws, size_t ws_bytes, hipStream_t stream) {
    if (dt != GDN_IN_BF16) return hipErrorInvalidValue;
    if (shp.dk == 128 && shp.dv == 128)
        return launch_dk_dv<128, 128>(S, q, k, v, g, beta, L, shp, o, ws, ws_bytes, stream);
    if (shp.dk == 128 && shp.dv == 64)
        return launch_dk_dv<128, 64>(S, q, k, v, g, beta, L, shp, o, ws, ws_bytes, stream);
    if (shp.dk == 64 && shp.dv == 128)
        return launch_dk_dv<64, 128>(S, q, k, v, g, beta, L, shp, o, ws, ws_bytes, stream);
    return launch_dk_dv<64, 64>(S, q, k, v, g, beta, L, shp, o, ws, ws_bytes, stream);
}

}  // namespace gdn
