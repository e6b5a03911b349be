// verify.hip -- the verify kernel: outputs of a T-row speculative block from the
// checkpoint state, without writing the state.
//
// One workgroup owns one (instance, head): its whole dv x dk fp32 state is read
// from HBM exactly once, into registers, and never written (the value-column
// partition of the lithos-metal README, "How it works", region table, "GDN
// mixer" row, with one wave per 16..32 value rows).
//
// Instead of stepping the state T times in registers (about 3T FMA per state
// element), the block is solved in its UT form with chunk = T.  With
// G_t = g_1 + ... + g_t, gamma_t = exp(G_t) and Gamma_tj = exp(G_t - G_j):
//
//   delta_t = beta_t (v_t - gamma_t S k_t) - sum_{j<t} beta_t Gamma_tj (k_t.k_j) delta_j
//   o_t     = gamma_t S q_t + sum_{j<=t} Gamma_tj (q_t.k_j) delta_j
//
// so the state enters only through the 2T projections [K;Q] S^T, one dense
// (2T x dk) x (dk x dv) contraction per head.  That contraction runs on fp32
// MFMA (v_mfma_f32_16x16x4_f32): products are exact fp32 products, so no split
// of the fp32 state is needed, and the VALU is left with O(T^2) work per value
// row.  The key Gram matrix [K;Q] K^T rides along in the same loop.
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

__device__ inline float comp(const float4 &v, int c) {
    return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
}

// X rows: 0..T-1 hold k_1..k_T, T..2T-1 hold q_1..q_T, the rest are zero.
// MT = number of 16-row MFMA tiles of X (1 for T <= 8, 2 for T <= 16).
template <int DK, int DV, typename TIn, int MT>
__global__ __launch_bounds__(kThreads) void verify_kernel(
    const float *__restrict__ S, const TIn *__restrict__ q, const TIn *__restrict__ k,
    const TIn *__restrict__ v, const float *__restrict__ g, const float *__restrict__ beta,
    int T, int B, int H, float *__restrict__ o, uint8_t *__restrict__ rec) {
    constexpr int RW = DV / kWaves;  // value rows per wave
    constexpr int NT = RW / 16;      // 16-row MFMA tiles per wave
    constexpr int KM = DK / 16;      // 16-key groups (4 keys per lane group)
    constexpr int XR = 16 * MT;      // rows of X
    constexpr int XS = DK + 4;       // LDS row stride of X, floats
    constexpr int PS = DV + 4;       // LDS row stride of P, floats
    constexpr int TM = 8 * MT;       // largest T for this instantiation
    constexpr int GM = KM / kWaves;  // key groups per wave for the Gram matrix
    static_assert(NT >= 1 && GM >= 1 && TM * TM <= kThreads, "shape");

    __shared__ __attribute__((aligned(16))) float X[XR * XS];
    __shared__ __attribute__((aligned(16))) float P[XR * PS];  // [K;Q] S^T, rows x, cols value row
    __shared__ float gpart[kWaves][XR * XR];                   // per-wave partial Gram
    __shared__ float coefM[TM * TM], coefN[TM * TM];
    __shared__ float Gpre[TM], gam[TM], bsh[TM];

    const int bh = blockIdx.x;
    const int b = bh / H, h = bh - b * H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    const int lr = lane & 15, lg = lane >> 4;
    const RecLayout RL = rec_layout(B, T, H, DK, DV, int(sizeof(TIn)));

    // 1. The head's state: rows w*RW + nt*16 + lr, keys 16m + 4lg .. +3.
    //    Issued first so the whole 64 KiB is in flight while inputs are staged.
    const float *Sh = S + size_t(bh) * DV * DK;
    float4 sreg[NT][KM];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int m = 0; m < KM; ++m)
            sreg[nt][m] = *reinterpret_cast<const float4 *>(
                Sh + size_t(w * RW + nt * 16 + lr) * DK + 16 * m + 4 * lg);

    // 2. This thread's value column v_t[tid] for the row phase.
    float vreg[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) vreg[t] = 0.f;
    if (tid < DV) {
#pragma unroll
        for (int t = 0; t < TM; ++t)
            if (t < T) vreg[t] = load1(v + (size_t(b * T + t) * H + h) * DV + tid);
    }

    // 3. Keys and queries -> X (fp32); keys also -> the record.
    TIn *kcopy = reinterpret_cast<TIn *>(rec + RL.kcopy);
    for (int c = tid; c < 2 * T * DK / 8; c += kThreads) {
        const int e = c * 8, r = e / DK, col = e - r * DK;
        const bool isk = r < T;
        const int t = isk ? r : r - T;
        const size_t src = (size_t(b * T + t) * H + h) * DK + col;
        In8<TIn> x;
        x.load((isk ? k : q) + src);
        if (isk) x.store_raw(kcopy + src);
        float4 lo = {x.get(0), x.get(1), x.get(2), x.get(3)};
        float4 hi = {x.get(4), x.get(5), x.get(6), x.get(7)};
        *reinterpret_cast<float4 *>(X + r * XS + col) = lo;
        *reinterpret_cast<float4 *>(X + r * XS + col + 4) = hi;
    }
    for (int idx = tid; idx < (XR - 2 * T) * DK; idx += kThreads) {
        const int r = 2 * T + idx / DK;
        X[r * XS + idx % DK] = 0.f;
    }
    if (tid < T) bsh[tid] = beta[size_t(b * T + tid) * H + h];
    if (tid == 0) {
        // Log-decay prefix sums, in one fixed order; the commit reuses these values.
        float gl[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t) gl[t] = t < T ? g[size_t(b * T + t) * H + h] : 0.f;
        float acc = 0.f;
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            acc += gl[t];
            Gpre[t] = acc;
        }
    }
    __syncthreads();

    // 4. [K;Q] S^T and the Gram matrix [K;Q] K^T on fp32 MFMA.  The contraction
    //    index (keys) is visited as 16m + 4lg + c for lane group lg, slot c; A and
    //    B use the same order, so each product pairs matching keys.
    f32x4 acc[MT][NT];
    f32x4 gacc[MT][MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < MT; ++j) gacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int m = 0; m < KM; ++m) {
        float4 a[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            a[mt] = *reinterpret_cast<const float4 *>(X + (mt * 16 + lr) * XS + 16 * m + 4 * lg);
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        comp(a[mt], c), comp(sreg[nt][m], c), acc[mt][nt], 0, 0, 0);
        if (m / GM == w) {
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

    // 5. Results -> LDS.  Lane (lr, lg) of a 16x16 tile holds rows 4lg..4lg+3 of
    //    column lr.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                P[(mt * 16 + 4 * lg + r) * PS + w * RW + nt * 16 + lr] = acc[mt][nt][r];
#pragma unroll
    for (int m1 = 0; m1 < MT; ++m1)
#pragma unroll
        for (int m2 = 0; m2 < MT; ++m2)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                gpart[w][(m1 * 16 + 4 * lg + r) * XR + m2 * 16 + lr] = gacc[m1][m2][r];
    __syncthreads();

    // 6. Block coefficients (shared by every value row of the head):
    //    coefM[t][j] = beta_t Gamma_tj k_t.k_j  (j < t),  coefN[t][j] = Gamma_tj q_t.k_j  (j <= t).
    if (tid < TM * TM) {
        const int t = tid / TM, j = tid - t * TM;
        float cm = 0.f, cn = 0.f;
        if (t < T && j <= t) {
            const float dec = expf(Gpre[t] - Gpre[j]);
            float kk = 0.f, qk = 0.f;
#pragma unroll
            for (int ww = 0; ww < kWaves; ++ww) {
                kk += gpart[ww][t * XR + j];
                qk += gpart[ww][(T + t) * XR + j];
            }
            if (j < t) cm = bsh[t] * dec * kk;
            cn = dec * qk;
        }
        coefM[tid] = cm;
        coefN[tid] = cn;
    }
    if (tid < T) {
        gam[tid] = expf(Gpre[tid]);
        reinterpret_cast<float *>(rec + RL.G)[size_t(b * T + tid) * H + h] = Gpre[tid];
    }
    __syncthreads();

    // 7. Value rows: forward substitution for delta, then the outputs.
    if (tid < DV) {
        const int i = tid;
        float *Drec = reinterpret_cast<float *>(rec + RL.delta);
        float d[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            if (t < T) {
                float dt = bsh[t] * (vreg[t] - gam[t] * P[t * PS + i]);
#pragma unroll
                for (int j = 0; j < t; ++j) dt -= coefM[t * TM + j] * d[j];
                d[t] = dt;
                float ot = gam[t] * P[(T + t) * PS + i];
#pragma unroll
                for (int j = 0; j <= t; ++j) ot += coefN[t * TM + j] * d[j];
                const size_t idx = (size_t(b * T + t) * H + h) * DV + i;
                o[idx] = ot;
                Drec[idx] = dt;
            }
        }
    }

    // 8. Mark the block pending for this instance; the header describes the record.
    if (tid == 0 && h == 0) {
        RecCtrl *ctrl = reinterpret_cast<RecCtrl *>(rec + RL.ctrl);
        ctrl[b].err = 0u;
        ctrl[b].done = 0u;
        ctrl[b].valid = kRecValid;
    }
    if (tid == 0 && bh == 0) {
        RecHeader *hd = reinterpret_cast<RecHeader *>(rec);
        hd->T = T;
        hd->B = B;
        hd->H = H;
        hd->dk = DK;
        hd->dv = DV;
        hd->in_dt = sizeof(TIn) == 2 ? GDN_IN_BF16 : GDN_IN_F32;
        hd->magic = kRecMagic;
    }
}

template <int DK, int DV, typename TIn>
hipError_t launch_t(const float *S, const void *q, const void *k, const void *v, const float *g,
                    const float *beta, int T, const gdn_shape &s, float *o, void *rec,
                    hipStream_t st) {
    const dim3 grid(unsigned(s.B) * unsigned(s.H)), block(kThreads);
    auto *qq = static_cast<const TIn *>(q);
    auto *kk = static_cast<const TIn *>(k);
    auto *vv = static_cast<const TIn *>(v);
    auto *rr = static_cast<uint8_t *>(rec);
    if (T <= 8)
        hipLaunchKernelGGL((verify_kernel<DK, DV, TIn, 1>), grid, block, 0, st, S, qq, kk, vv, g,
                           beta, T, s.B, s.H, o, rr);
    else
        hipLaunchKernelGGL((verify_kernel<DK, DV, TIn, 2>), grid, block, 0, st, S, qq, kk, vv, g,
                           beta, T, s.B, s.H, o, rr);
    return hipGetLastError();
}

template <typename TIn>
hipError_t launch_dt(const float *S, const void *q, const void *k, const void *v, const float *g,
                     const float *beta, int T, const gdn_shape &s, float *o, void *rec,
                     hipStream_t st) {
    if (s.dk == 128 && s.dv == 128) return launch_t<128, 128, TIn>(S, q, k, v, g, beta, T, s, o, rec, st);
    if (s.dk == 128 && s.dv == 64) return launch_t<128, 64, TIn>(S, q, k, v, g, beta, T, s, o, rec, st);
    if (s.dk == 64 && s.dv == 128) return launch_t<64, 128, TIn>(S, q, k, v, g, beta, T, s, o, rec, st);
    return launch_t<64, 64, TIn>(S, q, k, v, g, beta, T, s, o, rec, st);
}

}  // namespace

hipError_t launch_verify(const float *S, const void *q, const void *k, const void *v,
                         const float *g, const float *beta, int T, gdn_in_dtype dt,
                         const gdn_shape &shp, float *o, void *record, hipStream_t stream) {
    if (dt == GDN_IN_BF16)
        return launch_dt<__hip_bfloat16>(S, q, k, v, g, beta, T, shp, o, record, stream);
    return launch_dt<float>(S, q, k, v, g, beta, T, shp, o, record, stream);
}

}  // namespace gdn
