// verify.hip -- the verify kernel: outputs of a T-row speculative block from the
// checkpoint state, without writing the state.
//
// One single-wave workgroup owns 16 value rows of one (instance, head): its
// slice of the dv x dk fp32 state is read from HBM exactly once, into registers,
// and never written (the value-column partition of the lithos-metal README, "How
// it works", region table, "GDN mixer" row).  Rows of S never interact, so the
// slices need no communication; single-wave workgroups need no barriers, and
// thousands of them keep loads of some waves overlapped with MFMA work of others.
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

__device__ inline float comp(const float4 &v, int c) {
    return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Four consecutive input elements: the A operand of one fp32 MFMA k-step group.
template <typename TIn> struct X4;
template <> struct X4<float> {
    float4 v;
    __device__ inline void load(const float *p) { v = *reinterpret_cast<const float4 *>(p); }
    __device__ inline void zero() { v = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ inline void store(float *p) const { *reinterpret_cast<float4 *>(p) = v; }
    __device__ inline float f(int c) const { return comp(v, c); }
};
template <> struct X4<__hip_bfloat16> {
    uint2 v;
    __device__ inline void load(const __hip_bfloat16 *p) { v = *reinterpret_cast<const uint2 *>(p); }
    __device__ inline void zero() { v = make_uint2(0u, 0u); }
    __device__ inline void store(__hip_bfloat16 *p) const { *reinterpret_cast<uint2 *>(p) = v; }
    __device__ inline float f(int c) const {
        const uint32_t w = c < 2 ? v.x : v.y;
        return __uint_as_float((c & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};

__device__ inline bf16x8 cat_bf16(const uint2 &a, const uint2 &b) {
    const uint4 u = make_uint4(a.x, a.y, b.x, b.y);
    return __builtin_bit_cast(bf16x8, u);
}

// Workgroup id -> (head, 16-row slice).  Workgroups are dealt to the 8 XCDs in
// id order, so within each run of 8 * SL ids the XCD index picks the head and
// the rest picks the slice: all slices of a head run on one XCD and share its L2
// for the head's q, k and v rows.
template <int SL>
__device__ inline void map_workgroup(int id, int nheads, int &bh, int &sl) {
    constexpr int G8 = 8 * SL;
    const int full = nheads / 8;
    const int grp = id / G8;
    if (grp < full) {
        const int rem = id - grp * G8;
        bh = grp * 8 + (rem & 7);
        sl = rem >> 3;
    } else {
        const int r2 = id - full * G8;
        bh = full * 8 + r2 / SL;
        sl = r2 - (r2 / SL) * SL;
    }
}

// One wave owns 16 value rows of one (instance, head).
// X rows: 0..T-1 hold k_1..k_T, T..2T-1 hold q_1..q_T, the rest are zero.
// MT = number of 16-row MFMA tiles of X (1 for T <= 8, 2 for T <= 16).
template <int DK, int DV, typename TIn, int MT>
__global__ __launch_bounds__(64) void verify_kernel(
    const float *__restrict__ S, const TIn *__restrict__ q, const TIn *__restrict__ k,
    const TIn *__restrict__ v, const float *__restrict__ g, const float *__restrict__ beta,
    int T, int B, int H, float *__restrict__ o, uint8_t *__restrict__ rec) {
    constexpr int KM = DK / 16;      // 16-key groups (4 keys per lane group)
    constexpr int XR = 16 * MT;      // rows of X
    constexpr int TM = 8 * MT;       // largest T for this instantiation
    constexpr int SL = DV / 16;      // 16-row slices per head
    constexpr bool kBf16 = sizeof(TIn) == 2;

    __shared__ float Pw[XR][17];                     // [K;Q] S^T for this wave's rows
    __shared__ float coefM[TM][TM + 1], coefN[TM][TM + 1];
    __shared__ float Gs[TM], gam[TM], bs[TM];

    int bh, sl;
    map_workgroup<SL>(blockIdx.x, B * H, bh, sl);
    const int b = bh / H, h = bh - b * H;
    const int lane = threadIdx.x, lr = lane & 15, lg = lane >> 4;
    const int row0 = sl * 16;
    const RecLayout RL = rec_layout(B, T, H, DK, DV, int(sizeof(TIn)));

    // 1. The slice's state: row row0 + lr, keys 16m + 4lg .. +3.  Issued first so
    //    all of it is in flight together.
    const float *Srow = S + (size_t(bh) * DV + row0 + lr) * DK + 4 * lg;
    float4 sreg[KM];
#pragma unroll
    for (int m = 0; m < KM; ++m) sreg[m] = *reinterpret_cast<const float4 *>(Srow + 16 * m);

    // 2. X rows for the A operands, straight from global memory (the head's rows
    //    are shared by its slices through L2).  Every load below reads a valid
    //    address (indices are clamped) and is masked afterwards: branch-free loads
    //    issue back to back instead of each waiting for all earlier ones.
    X4<TIn> xa[MT][KM];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int x = 16 * mt + lr;
        const bool isk = x < T, live = x < 2 * T;
        const int t = isk ? x : min(x - T, T - 1);
        const TIn *src = (isk ? k : q) + (size_t(b * T + t) * H + h) * DK;
#pragma unroll
        for (int m = 0; m < KM; ++m) {
            xa[mt][m].load(src + 16 * m + 4 * lg);
            if (!live) xa[mt][m].zero();
        }
    }
    // 3. Value column of this lane's row for the row phase (lanes 0..15 use it).
    float vreg[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t)
        vreg[t] = load1(v + (size_t(b * T + min(t, T - 1)) * H + h) * DV + row0 + lr);
    // 4. Gates: log-decay prefix sums in one fixed order (the commit reuses them).
    {
        float gl[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const float gv = g[size_t(b * T + min(t, T - 1)) * H + h];
            gl[t] = t < T ? gv : 0.f;
        }
        const float bl = beta[size_t(b * T + min(lane, T - 1)) * H + h];
        float pre = 0.f, mine = 0.f;
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            pre += gl[t];
            if (t == lane) mine = pre;
        }
        if (lane < T) {
            Gs[lane] = mine;
            gam[lane] = expf(mine);
            bs[lane] = bl;
        }
    }

    // 5. [K;Q] S^T on fp32 MFMA; the contraction visits keys 16m + 4lg + c for lane
    //    group lg, slot c, in A and B alike.
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < KM; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[mt][m].f(c), comp(sreg[m], c),
                                                               acc[mt], 0, 0, 0);
    // Gram matrix X X^T.  bf16 rows multiply exactly on bf16 MFMA (keys 16(2p) +
    // 4lg + {0..3} and 16(2p+1) + 4lg + {0..3} in slots 0..7); fp32 rows use fp32
    // MFMA.
    f32x4 gacc[MT][MT];
#pragma unroll
    for (int m1 = 0; m1 < MT; ++m1)
#pragma unroll
        for (int m2 = 0; m2 < MT; ++m2) gacc[m1][m2] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (kBf16) {
#pragma unroll
        for (int p = 0; p < KM / 2; ++p)
#pragma unroll
            for (int m1 = 0; m1 < MT; ++m1)
#pragma unroll
                for (int m2 = 0; m2 < MT; ++m2)
                    gacc[m1][m2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        cat_bf16(xa[m1][2 * p].v, xa[m1][2 * p + 1].v),
                        cat_bf16(xa[m2][2 * p].v, xa[m2][2 * p + 1].v), gacc[m1][m2], 0, 0, 0);
    } else {
#pragma unroll
        for (int m = 0; m < KM; ++m)
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int m1 = 0; m1 < MT; ++m1)
#pragma unroll
                    for (int m2 = 0; m2 < MT; ++m2)
                        gacc[m1][m2] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                            xa[m1][m].f(c), xa[m2][m].f(c), gacc[m1][m2], 0, 0, 0);
    }

    // 6. Lane (lr, lg) of a 16x16 result tile holds rows 4lg..4lg+3 of column lr.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) Pw[16 * mt + 4 * lg + r][lr] = acc[mt][r];
    __syncthreads();
    //    Block coefficients: coefM[t][j] = beta_t Gamma_tj k_t.k_j (j < t),
    //    coefN[t][j] = Gamma_tj q_t.k_j (j <= t).
#pragma unroll
    for (int m1 = 0; m1 < MT; ++m1)
#pragma unroll
        for (int m2 = 0; m2 < MT; ++m2)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int x = 16 * m1 + 4 * lg + r, y = 16 * m2 + lr;
                const float val = gacc[m1][m2][r];
                if (x < T && y < x) coefM[x][y] = bs[x] * expf(Gs[x] - Gs[y]) * val;
                if (x >= T && x < 2 * T && y <= x - T)
                    coefN[x - T][y] = expf(Gs[x - T] - Gs[y]) * val;
            }
    __syncthreads();

    // 7. Value rows (lanes 0..15): forward substitution for delta, then outputs.
    if (lg == 0) {
        const int i = row0 + lr;
        float *Drec = reinterpret_cast<float *>(rec + RL.delta);
        float d[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            if (t < T) {
                float dt = bs[t] * (vreg[t] - gam[t] * Pw[t][lr]);
#pragma unroll
                for (int j = 0; j < t; ++j) dt -= coefM[t][j] * d[j];
                d[t] = dt;
                float ot = gam[t] * Pw[T + t][lr];
#pragma unroll
                for (int j = 0; j <= t; ++j) ot += coefN[t][j] * d[j];
                const size_t idx = (size_t(b * T + t) * H + h) * DV + i;
                o[idx] = ot;
                Drec[idx] = dt;
            }
        }
    }

    // 8. Record bookkeeping.  Slice 0 stores the head's gates and keys; the first
    //    slices set the pending-block flags of the commit workgroups.
    if (sl == 0) {
        if (lane < T) reinterpret_cast<float *>(rec + RL.G)[size_t(b * T + lane) * H + h] = Gs[lane];
        if (lr < T) {
            TIn *kc = reinterpret_cast<TIn *>(rec + RL.kcopy) + (size_t(b * T + lr) * H + h) * DK + 4 * lg;
#pragma unroll
            for (int m = 0; m < KM; ++m) xa[0][m].store(kc + 16 * m);
        }
    }
    if (lane == 0 && sl < DV / kCommitRows)
        reinterpret_cast<uint32_t *>(rec + RL.flags)[size_t(bh) * kCommitSlices + sl] = kRecValid;
    if (lane == 0 && sl == 0 && h == 0) reinterpret_cast<RecCtrl *>(rec + RL.ctrl)[b].err = 0u;
    if (lane == 0 && sl == 0 && bh == 0) {
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

template <int DK, int DV, typename TIn>
hipError_t launch_t(const float *S, const void *q, const void *k, const void *v, const float *g,
                    const float *beta, int T, const gdn_shape &s, float *o, void *rec,
                    hipStream_t st) {
    const dim3 grid(unsigned(s.B) * unsigned(s.H) * unsigned(DV / 16)), block(64);
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
