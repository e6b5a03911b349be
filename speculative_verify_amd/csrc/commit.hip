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
// element, far below the VALU ridge, so the kernel streams at HBM speed).
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 32;

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

    __shared__ float cd[GDN_T_MAX][kRows];                            // exp(G_n-G_j) delta_j
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
    RecCtrl &c = ctrl[b];
    const int n = n_acc[b];
    if (c.valid != kRecValid) {
        if (leader) atomicOr(&c.err, uint32_t(GDN_REC_NO_BLOCK));
        return;
    }
    if (n < 0 || n > T) {
        if (leader) atomicOr(&c.err, uint32_t(GDN_REC_N_RANGE));
        return;
    }

    if (n > 0) {
        const RecLayout RL = rec_layout(B, T, H, DK, DV, in_dt == GDN_IN_BF16 ? 2 : 4);
        float4 *Sh = reinterpret_cast<float4 *>(S + size_t(bh) * DV * DK + size_t(slice) * kRows * DK);
        float4 s[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) s[p] = Sh[tid + kThreads * p];

        const float *G = reinterpret_cast<const float *>(rec + RL.G);
        const float *D = reinterpret_cast<const float *>(rec + RL.delta);
        const float Gn = G[(size_t(b) * T + (n - 1)) * H + h];
        for (int idx = tid; idx < n * kRows; idx += kThreads) {
            const int j = idx / kRows, r = idx - j * kRows;
            const size_t row = size_t(b) * T + j;
            cd[j][r] = expf(Gn - G[row * H + h]) * D[(row * H + h) * DV + slice * kRows + r];
        }
        if (in_dt == GDN_IN_BF16) {
            const uint16_t *K = reinterpret_cast<const uint16_t *>(rec + RL.kcopy);
            for (int idx = tid; idx < n * DK; idx += kThreads) {
                const int j = idx / DK, m = idx - j * DK;
                kk[j][m] = bf16_bits_to_f32(K[((size_t(b) * T + j) * H + h) * DK + m]);
            }
        } else {
            const float *K = reinterpret_cast<const float *>(rec + RL.kcopy);
            for (int idx = tid; idx < n * DK; idx += kThreads) {
                const int j = idx / DK, m = idx - j * DK;
                kk[j][m] = K[((size_t(b) * T + j) * H + h) * DK + m];
            }
        }
        __syncthreads();

        const float gam = expf(Gn);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int f = tid + kThreads * p;
            const int row = f / F4_ROW, c4 = f - row * F4_ROW;
            float4 a;
            a.x = gam * s[p].x;
            a.y = gam * s[p].y;
            a.z = gam * s[p].z;
            a.w = gam * s[p].w;
            for (int j = 0; j < n; ++j) {
                const float cdj = cd[j][row];
                const float4 kv = *reinterpret_cast<const float4 *>(&kk[j][4 * c4]);
                a.x += cdj * kv.x;
                a.y += cdj * kv.y;
                a.z += cdj * kv.z;
                a.w += cdj * kv.w;
            }
            Sh[f] = a;
        }
    }

    // The last workgroup of this instance retires the block and advances pos.
    // Every wave of every workgroup read c.valid above (its value decided a
    // branch, so the read has completed) before the barrier and the count below,
    // so no reader can see the block retired early.  The S stores need no
    // ordering against the count: nothing in this kernel reads them.
    __syncthreads();
    if (tid == 0) {
        const uint32_t old =
            __hip_atomic_fetch_add(&c.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old == uint32_t(H) * SLICES - 1u) {
            c.done = 0u;
            c.valid = 0u;
            if (pos) pos[b] += n;
        }
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
