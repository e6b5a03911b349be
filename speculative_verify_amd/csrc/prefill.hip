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
// One workgroup owns RS = 16 * NWS value rows of one (instance, head) -- rows of S
// never interact, so slices of the value index are independent -- and walks the
// chunks in order with its state slice held in registers.  Wave w owns 16 value
// rows.  Per chunk, all waves first build the shared chunk quantities (staged
// keys and queries, gates, Gram matrices, Linv) in LDS, then each wave runs the
// state-coupled products for its rows.  MFMA results feed the next MFMA straight
// from registers: a 16x16 result tile holds rows 4*(lane/16)+r of column lane%16,
// which is the layout of a B operand whose contraction index runs over those rows.
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int C = GDN_PREFILL_CHUNK;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ inline f32x4 mma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

struct Split8 {
    bf16x8 hi, lo;
};

__device__ inline Split8 split8(const float (&x)[8]) {
    Split8 s;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const __bf16 h = static_cast<__bf16>(x[e]);
        s.hi[e] = h;
        s.lo[e] = static_cast<__bf16>(x[e] - static_cast<float>(h));
    }
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
    float Wb[3][16][20];    // block-inverse scratch
    float gam[C], ee[C], bet[C], G[C];
};

template <int DK, int DV, int NWS>
__global__ __launch_bounds__(64 * NWS) void prefill_kernel(
    float *__restrict__ S, const __hip_bfloat16 *__restrict__ q, const __hip_bfloat16 *__restrict__ k,
    const __hip_bfloat16 *__restrict__ v, const float *__restrict__ g, const float *__restrict__ beta,
    int L, int H, float *__restrict__ o) {
    constexpr int RS = 16 * NWS;       // value rows per workgroup
    constexpr int SLICES = DV / RS;
    constexpr int KT = DK / 16;        // 16-key tiles
    constexpr int KB = DK / 32;        // 32-key contraction blocks
    constexpr int NT = 64 * NWS;
    constexpr int NLD = C * DK / 8 / NT;  // 16-byte staging pieces per thread per tensor
    static_assert(SLICES * RS == DV && KB >= 1, "tiling");
    static_assert(NLD >= 1 && NLD * NT * 8 == C * DK, "staging tiling");

    __shared__ Smem<DK> sm;

    const int wg = blockIdx.x;
    const int bh = wg / SLICES, slice = wg - bh * SLICES;
    const int b = bh / H, h = bh - b * H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int irow = slice * RS + w * 16 + lr;  // value row of this lane's column

    for (int idx = tid; idx < C * (C + 4); idx += NT) {
        (&sm.Am[0][0])[idx] = 0.f;
        (&sm.Tm[0][0])[idx] = 0.f;
        (&sm.Pm[0][0])[idx] = 0.f;
    }

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

        // ---- stage the chunk's keys, queries and gates (rows >= n are zero) ----
        // Every load is issued before any store, so one memory latency covers them.
        {
            uint4 kv[NLD], qv[NLD];
#pragma unroll
            for (int u = 0; u < NLD; ++u) {
                const int idx = tid + u * NT;
                const int t = idx / (DK / 8), col = (idx - t * (DK / 8)) * 8;
                // Clamped rows keep every load valid and branch-free; rows past
                // the prompt are zeroed after the load.
                const size_t off = ((row0 + min(t, n - 1)) * H + h) * DK + col;
                kv[u] = *reinterpret_cast<const uint4 *>(k + off);
                qv[u] = *reinterpret_cast<const uint4 *>(q + off);
                if (t >= n) {
                    kv[u] = make_uint4(0u, 0u, 0u, 0u);
                    qv[u] = make_uint4(0u, 0u, 0u, 0u);
                }
            }
            const size_t gi = (row0 + min(lane, n - 1)) * H + h;
            float gt = g[gi], bt = beta[gi];
            if (lane >= n) {
                gt = 0.f;
                bt = 0.f;
            }
#pragma unroll
            for (int u = 0; u < NLD; ++u) {
                const int idx = tid + u * NT;
                const int t = idx / (DK / 8), col = (idx - t * (DK / 8)) * 8;
                *reinterpret_cast<uint4 *>(&sm.Ks[t][col]) = kv[u];
                *reinterpret_cast<uint4 *>(&sm.Qs[t][col]) = qv[u];
                const __bf16 *kh = reinterpret_cast<const __bf16 *>(&kv[u]);
#pragma unroll
                for (int e = 0; e < 8; ++e) sm.Kt[col + e][t] = kh[e];
            }
            if (w == 0) {
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
        }
        __syncthreads();

        // ---- Gram tiles: A from K K^T, P from Q K^T (lower tiles only) ----
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

        // ---- Linv = (I + A)^{-1}, by 16x16 blocks ----
        // Diagonal blocks by forward substitution: lane = (block lg, column lr).
        if (w == 0) {
            const int base = 16 * lg;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = r == lr ? 1.f : 0.f;
#pragma unroll
                for (int jj = 0; jj < r; ++jj) acc -= sm.Am[base + r][base + jj] * x[jj];
                x[r] = acc;
                asm volatile("" ::: "memory");  // keep each row's loads with its row (register pressure)
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.Tm[base + r][base + lr] = x[r];
        }
        __syncthreads();
        // Off-diagonal blocks, one block diagonal at a time:
        //   X_ij = -X_ii sum_{m=j}^{i-1} A_im X_mj   (i = j + d).
        for (int d = 1; d <= 3; ++d) {
            const int npairs = 4 - d;
            for (int idx = tid; idx < npairs * 256; idx += NT) {
                const int j = idx >> 8, r = (idx >> 4) & 15, cc = idx & 15;
                const int i = j + d;
                float acc = 0.f;
                for (int mb = j; mb < i; ++mb)
#pragma unroll
                    for (int m = 0; m < 16; ++m)
                        acc += sm.Am[16 * i + r][16 * mb + m] * sm.Tm[16 * mb + m][16 * j + cc];
                sm.Wb[j][r][cc] = acc;
            }
            __syncthreads();
            for (int idx = tid; idx < npairs * 256; idx += NT) {
                const int j = idx >> 8, r = (idx >> 4) & 15, cc = idx & 15;
                const int i = j + d;
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < 16; ++m) acc += sm.Tm[16 * i + r][16 * i + m] * sm.Wb[j][m][cc];
                sm.Tm[16 * i + r][16 * j + cc] = -acc;
            }
            __syncthreads();
        }

        // ---- state-coupled products for this wave's 16 value rows ----
        // The contraction over keys visits, for block p and lane group lg, keys
        // 32p + 4lg + {0..3} and 32p + 16 + 4lg + {0..3}: the keys this lane holds
        // in st[2p] and st[2p+1].
        float vv[4][4];  // v[t][irow] for t = 16 tt + 4 lg + r
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * tt + 4 * lg + r;
                const float x = load1(v + ((row0 + min(t, n - 1)) * H + h) * DV + irow);
                vv[tt][r] = t < n ? x : 0.f;
            }
        Split8 sB[KB];
#pragma unroll
        for (int p = 0; p < KB; ++p) {
            const float x[8] = {st[2 * p][0], st[2 * p][1], st[2 * p][2], st[2 * p][3],
                                st[2 * p + 1][0], st[2 * p + 1][1], st[2 * p + 1][2], st[2 * p + 1][3]};
            sB[p] = split8(x);
        }
        // R = diag(beta) (V - diag(gamma) K S^T), rows t = 16 tt + 4 lg + r.
        float R[4][4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            f32x4 X = {0.f, 0.f, 0.f, 0.f};
            const int t = 16 * tt + lr;
#pragma unroll
            for (int p = 0; p < KB; ++p) {
                const bf16x8 ka = cat4(*reinterpret_cast<const bf16x4 *>(&sm.Ks[t][32 * p + 4 * lg]),
                                       *reinterpret_cast<const bf16x4 *>(&sm.Ks[t][32 * p + 16 + 4 * lg]));
                X = mma(ka, sB[p].hi, X);
                X = mma(ka, sB[p].lo, X);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tr = 16 * tt + 4 * lg + r;
                R[tt][r] = sm.bet[tr] * (vv[tt][r] - sm.gam[tr] * X[r]);
            }
        }
        // D = Linv R (Linv is lower triangular: only blocks p <= tt / 2).
        Split8 rB[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const float x[8] = {R[2 * p][0], R[2 * p][1], R[2 * p][2], R[2 * p][3],
                                R[2 * p + 1][0], R[2 * p + 1][1], R[2 * p + 1][2], R[2 * p + 1][3]};
            rB[p] = split8(x);
        }
        f32x4 D[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            D[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int t = 16 * tt + lr;
#pragma unroll
            for (int p = 0; p <= tt / 2; ++p) {
                const float4 a0 = *reinterpret_cast<const float4 *>(&sm.Tm[t][32 * p + 4 * lg]);
                const float4 a1 = *reinterpret_cast<const float4 *>(&sm.Tm[t][32 * p + 16 + 4 * lg]);
                const float x[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                D[tt] = mma3(split8(x), rB[p], D[tt]);
            }
        }
        // O = diag(gamma) Q S^T + P D.
        Split8 dB[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const float x[8] = {D[2 * p][0], D[2 * p][1], D[2 * p][2], D[2 * p][3],
                                D[2 * p + 1][0], D[2 * p + 1][1], D[2 * p + 1][2], D[2 * p + 1][3]};
            dB[p] = split8(x);
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            f32x4 Y = {0.f, 0.f, 0.f, 0.f};
            const int t = 16 * tt + lr;
#pragma unroll
            for (int p = 0; p < KB; ++p) {
                const bf16x8 qa = cat4(*reinterpret_cast<const bf16x4 *>(&sm.Qs[t][32 * p + 4 * lg]),
                                       *reinterpret_cast<const bf16x4 *>(&sm.Qs[t][32 * p + 16 + 4 * lg]));
                Y = mma(qa, sB[p].hi, Y);
                Y = mma(qa, sB[p].lo, Y);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) Y[r] *= sm.gam[16 * tt + 4 * lg + r];
#pragma unroll
            for (int p = 0; p <= tt / 2; ++p) {
                const float4 a0 = *reinterpret_cast<const float4 *>(&sm.Pm[t][32 * p + 4 * lg]);
                const float4 a1 = *reinterpret_cast<const float4 *>(&sm.Pm[t][32 * p + 16 + 4 * lg]);
                const float x[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                Y = mma3(split8(x), dB[p], Y);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tr = 16 * tt + 4 * lg + r;
                if (tr < n) o[((row0 + tr) * H + h) * DV + irow] = Y[r];
            }
        }
        // S <- gamma_last S + K^T diag(e) D; the result tiles over keys match st[][].
        Split8 eB[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = sm.ee[32 * p + 4 * lg + e] * D[2 * p][e];
                x[4 + e] = sm.ee[32 * p + 16 + 4 * lg + e] * D[2 * p + 1][e];
            }
            eB[p] = split8(x);
        }
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
        }
        __syncthreads();  // the next chunk overwrites the shared buffers
    }

#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
        *reinterpret_cast<float4 *>(Srow + 16 * kt + 4 * lg) =
            make_float4(st[kt][0], st[kt][1], st[kt][2], st[kt][3]);
}

template <int DK, int DV, int NWS>
hipError_t launch_t(float *S, const void *q, const void *k, const void *v, const float *g,
                    const float *beta, int L, const gdn_shape &s, float *o, hipStream_t st) {
    constexpr int SLICES = DV / (16 * NWS);
    const dim3 grid(unsigned(s.B) * unsigned(s.H) * SLICES), block(64 * NWS);
    hipLaunchKernelGGL((prefill_kernel<DK, DV, NWS>), grid, block, 0, st, S,
                       static_cast<const __hip_bfloat16 *>(q), static_cast<const __hip_bfloat16 *>(k),
                       static_cast<const __hip_bfloat16 *>(v), g, beta, L, s.H, o);
    return hipGetLastError();
}

}  // namespace

// One workgroup per (instance, head): the chunk's shared quantities (Gram
// matrices, Linv, gates) are built once per head, and each wave owns 16 value rows.
hipError_t launch_prefill(float *S, const void *q, const void *k, const void *v, const float *g,
                          const float *beta, int L, gdn_in_dtype dt, const gdn_shape &shp, float *o,
                          hipStream_t stream) {
    if (dt != GDN_IN_BF16) return hipErrorInvalidValue;
    if (shp.dk == 128 && shp.dv == 128) return launch_t<128, 128, 8>(S, q, k, v, g, beta, L, shp, o, stream);
    if (shp.dk == 128 && shp.dv == 64) return launch_t<128, 64, 4>(S, q, k, v, g, beta, L, shp, o, stream);
    if (shp.dk == 64 && shp.dv == 128) return launch_t<64, 128, 8>(S, q, k, v, g, beta, L, shp, o, stream);
    return launch_t<64, 64, 4>(S, q, k, v, g, beta, L, shp, o, stream);
}

}  // namespace gdn
