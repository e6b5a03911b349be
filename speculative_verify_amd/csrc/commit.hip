// commit.hip -- GPU-resident commit of a verified block's accepted prefix.
//
// The lithos-metal README ("How it works") keeps accepted tokens and the
// recurrent state's commit/rollback on the GPU; the devdoido audit (DSpark
// section) rewinds the recurrent state to the accepted tokens after every
// acceptance decision.  Here the accepted row count n is read from device memory
// and the state is rebuilt from the block's checkpoint (S itself, which the
// verify never wrote) and the record's delta rows:
//
//   S_n = exp(G_n) S + sum_{j<=n} exp(G_n - G_j) delta_j k_j^T
//
// n = 0 touches nothing, so a full rollback is bit-exact.  Each workgroup owns
// 32 value rows of one head; it reads them and writes them once (n + 1 FMA per
// element, far below the VALU ridge, so the kernel streams at HBM speed).  Each
// workgroup checks and clears its own pending-block flag, so workgroups never
// wait on or count each other.
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = kCommitRows;

template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void commit_kernel(float *__restrict__ S,
                                                          uint8_t *__restrict__ rec,
                                                          const int32_t *__restrict__ n_acc,
                                                          int32_t *__restrict__ pos, int B,
                                                          int H) {
    constexpr int SLICES = DV / kRows;
    constexpr int F4_ROW = DK / 4;                       // float4 per state row
    constexpr int NP = kRows * F4_ROW / kThreads;        // float4 per thread
    static_assert(NP >= 1 && kRows * F4_ROW == NP * kThreads, "tiling");
    static_assert(SLICES <= kCommitSlices, "one pending flag per commit workgroup");
    static_assert(GDN_T_MAX * kRows % kThreads == 0 && GDN_T_MAX * (DK / 8) <= kThreads, "staging");

    __shared__ __attribute__((aligned(16))) float cd[GDN_T_MAX][kRows];  // exp(G_n-G_j) delta_j
    __shared__ __attribute__((aligned(16))) float kk[GDN_T_MAX][DK];  // k_j

    const int wg = blockIdx.x;
    const int bh = wg / SLICES, slice = wg - bh * SLICES;
    const int b = bh / H, h = bh - b * H;
    const int tid = threadIdx.x;
    const bool leader = (h == 0 && slice == 0 && tid == 0);

    const RecHeader *hd = reinterpret_cast<const RecHeader *>(rec);
    RecCtrl *ctrl = reinterpret_cast<RecCtrl *>(rec + 256);

    // Record checks.  A record that no verify has written has no block to commit.
    if (hd->magic != kRecMagic) {
        if (leader) atomicOr(&ctrl[b].err, uint32_t(GDN_REC_NO_BLOCK));
        return;
    }
    const int T = hd->T, in_dt = hd->in_dt;
    if (hd->B != B || hd->H != H || hd->dk != DK || hd->dv != DV || T < 1 || T > GDN_T_MAX ||
        (in_dt != GDN_IN_F32 && in_dt != GDN_IN_BF16)) {
        if (leader && b < hd->B) atomicOr(&ctrl[b].err, uint32_t(GDN_REC_SHAPE));
        return;
    }
    const RecLayout RL = rec_layout(B, T, H, DK, DV, in_dt == GDN_IN_BF16 ? 2 : 4);
    uint32_t *flag = reinterpret_cast<uint32_t *>(rec + RL.flags) + size_t(bh) * kCommitSlices + slice;
    const int n = n_acc[b];
    // Every workgroup of an instance sees the same header and n, and its own flag,
    // which the same verify set for all of them: they all take the same branch.
    if (*flag != kRecValid) {
        if (leader) atomicOr(&ctrl[b].err, uint32_t(GDN_REC_NO_BLOCK));
        return;
    }
    if (n < 0 || n > T) {
        if (leader) atomicOr(&ctrl[b].err, uint32_t(GDN_REC_N_RANGE));
        return;
    }

    if (n > 0) {
        // Thread tid owns rows 4 (tid / F4_ROW) + p, p < NP, at columns 4 (tid % F4_ROW)..+3:
        // one 16-byte LDS read of k_j and one of the rows' coefficients per term.
        float4 *Sh = reinterpret_cast<float4 *>(S + size_t(bh) * DV * DK + size_t(slice) * kRows * DK);
        const int c4 = tid % F4_ROW, r0 = NP * (tid / F4_ROW);
        float4 s[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) s[p] = ld_stream(reinterpret_cast<const float *>(Sh + (r0 + p) * F4_ROW + c4));

        const float *G = reinterpret_cast<const float *>(rec + RL.G);
        const float *D = reinterpret_cast<const float *>(rec + RL.delta);
        const float Gn = G[(size_t(b) * T + (n - 1)) * H + h];
        // Stage the n replayed rows.  Loads read clamped, always-valid rows and
        // are masked at the store, so they issue back to back.
        constexpr int CDP = GDN_T_MAX * kRows / kThreads;  // cd entries per thread
#pragma unroll
        for (int u = 0; u < CDP; ++u) {
            const int idx = tid + u * kThreads, j = idx / kRows, r = idx - j * kRows;
            const size_t row = size_t(b) * T + min(j, n - 1);
            const float val = expf(Gn - G[row * H + h]) * D[(row * H + h) * DV + slice * kRows + r];
            if (j < n) cd[j][r] = val;
        }
        {
            constexpr int PIECES = DK / 8;  // 8-element pieces per key row
            const int j = tid / PIECES, col = (tid - j * PIECES) * 8;
            const size_t off = ((size_t(b) * T + min(j, n - 1)) * H + h) * DK + col;
            float x[8];
            if (in_dt == GDN_IN_BF16) {
                const uint4 raw = *reinterpret_cast<const uint4 *>(
                    reinterpret_cast<const uint16_t *>(rec + RL.kcopy) + off);
                const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[2 * e] = __uint_as_float(w4[e] << 16);
                    x[2 * e + 1] = __uint_as_float(w4[e] & 0xffff0000u);
                }
            } else {
                const float *K = reinterpret_cast<const float *>(rec + RL.kcopy) + off;
                const float4 a = *reinterpret_cast<const float4 *>(K);
                const float4 c = *reinterpret_cast<const float4 *>(K + 4);
                x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
                x[4] = c.x; x[5] = c.y; x[6] = c.z; x[7] = c.w;
            }
            if (j < n) {
                *reinterpret_cast<float4 *>(&kk[j][col]) = make_float4(x[0], x[1], x[2], x[3]);
                *reinterpret_cast<float4 *>(&kk[j][col + 4]) = make_float4(x[4], x[5], x[6], x[7]);
            }
        }
        __syncthreads();

        const float gam = expf(Gn);
        float4 a[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            a[p].x = gam * s[p].x;
            a[p].y = gam * s[p].y;
            a[p].z = gam * s[p].z;
            a[p].w = gam * s[p].w;
        }
        for (int j = 0; j < n; ++j) {
            const float4 kv = *reinterpret_cast<const float4 *>(&kk[j][4 * c4]);
            float cdj[NP];
            if constexpr (NP == 4) {
                const float4 c = *reinterpret_cast<const float4 *>(&cd[j][r0]);
                cdj[0] = c.x; cdj[1] = c.y; cdj[2] = c.z; cdj[3] = c.w;
            } else {
#pragma unroll
                for (int p = 0; p < NP; ++p) cdj[p] = cd[j][r0 + p];
            }
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                a[p].x += cdj[p] * kv.x;
                a[p].y += cdj[p] * kv.y;
                a[p].z += cdj[p] * kv.z;
                a[p].w += cdj[p] * kv.w;
            }
        }
#pragma unroll
        for (int p = 0; p < NP; ++p) st_stream(reinterpret_cast<float *>(Sh + (r0 + p) * F4_ROW + c4), a[p]);
    }

    // Retire this workgroup's share of the block (every wave has read the flag
    // above, before this barrier) and let one workgroup advance pos.
    __syncthreads();
    if (tid == 0) {
        *flag = 0u;
        if (pos && h == 0 && slice == 0) pos[b] += n;
    }
}

template <int DK, int DV>
hipError_t launch_t(float *S, void *rec, const int32_t *n, int32_t *pos, const gdn_shape &s,
                    hipStream_t st) {
    const dim3 grid(unsigned(s.B) * unsigned(s.H) * unsigned(DV / kRows)), block(kThreads);
    hipLaunchKernelGGL((commit_kernel<DK, DV>), grid, block, 0, st, S, static_cast<uint8_t *>(rec),
                       n, pos, s.B, s.H);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_commit(float *S, void *record, const int32_t *n_accepted, int32_t *pos,
                         const gdn_shape &shp, hipStream_t stream) {
    if (shp.dk == 128 && shp.dv == 128) return launch_t<128, 128>(S, record, n_accepted, pos, shp, stream);
    if (shp.dk == 128 && shp.dv == 64) return launch_t<128, 64>(S, record, n_accepted, pos, shp, stream);
    if (shp.dk == 64 && shp.dv == 128) return launch_t<64, 128>(S, record, n_accepted, pos, shp, stream);
    return launch_t<64, 64>(S, record, n_accepted, pos, shp, stream);
}

}  // namespace gdn
