// accept.hip -- acceptance of a verify block and rewind of the filter history,
// on the device.
//
// Acceptance is exact speculative sampling (the audited-numbers page, "How does
// DSpark speculative decoding create more than one token per read?").  Rows of
// the block are [anchor, d_1 .. d_{T-1}]; target row t's logits give the
// distribution of the token after row t, drafter row j the distribution d_{j+1}
// was drawn from.  Greedy keeps d_{j+1} while it equals target row j's argmax
// (lowest index among equals); sampled keeps it while u_j q(d) < p(d), with
// p = softmax(target / tau) and q = softmax(drafter / tau).  n = 1 + (kept
// drafts) rows are committed; the emitted token is the argmax of the first
// unmatched row (greedy), or a draw from max(0, p - q) at the first rejection /
// from p of the last row when every draft was kept (sampled).  A draw from
// weights w with uniform u is the smallest x with w_0 + .. + w_x > u sum(w).
//
// The work is a few passes over vocabulary rows, bound by memory traffic and
// launch latency.  Rows are cut into slices of kSlice entries, one workgroup
// each:
//   stats  (B x rows x slices): per slice, the argmax of the raw logits and, for
//          sampled mode, max and sum of exp of logits / tau;
//   decide (B): combine the slices of each row, walk the drafts in order,
//          write n and the emitted token (greedy);
//   mass   (B x slices, sampled): every workgroup makes the sampled decision
//          (the same in each), slice 0 writes n, then per slice the mass of
//          the weights the emitted token is drawn from;
//   pick   (B, sampled): find the slice, then the entry, where the cumulative
//          weight passes u times the total.
#include <climits>

#include <mutex>

#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kSlice = 4096;              // vocabulary entries per workgroup
constexpr int kThreads = 256;
constexpr int kPer = kSlice / kThreads;   // entries per thread

// Per-slice statistics of one row: max of x = logit / tau, sum of exp(x - max),
// the largest raw logit and its (lowest) index.
struct Part {
    float m, s, bv;
    int bi;
};

// What decide hands to mass and pick for one sequence.
struct Pick {
    int row;        // target (and drafter) row the token is drawn at
    int residual;   // 1: weights max(0, p - q); 0: weights p (bonus)
    float mt, st;   // target row: max and sum of exp
    float md, sd;   // drafter row (residual only)
    int amax;       // target row's argmax: the answer when the weights sum to 0
    int pad;
};

template <typename TIn>
__device__ inline float ld(const TIn *p, size_t i);
template <>
__device__ inline float ld<float>(const float *p, size_t i) {
    return p[i];
}
template <>
__device__ inline float ld<__hip_bfloat16>(const __hip_bfloat16 *p, size_t i) {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(p)[i]);
}

// (max, sum of exp) pairs: merge b into a.
__device__ inline void lse_merge(float &m, float &s, float m2, float s2) {
    if (m2 > m) {
        const float t = m;
        m = m2;
        m2 = t;
        const float u = s;
        s = s2;
        s2 = u;
    }
    if (m2 != -INFINITY) s += s2 * __expf(m2 - m);
}

// Argmax pairs: larger value, then lower index.
__device__ inline void amax_merge(float &v, int &i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) {
        v = v2;
        i = i2;
    }
}

template <typename TIn>
__device__ inline const TIn *row_ptr(const TIn *tgt, const TIn *drf, int b, int r, int T, int V) {
    return r < T ? tgt + (size_t(b) * T + r) * V : drf + (size_t(b) * (T - 1) + (r - T)) * V;
}

template <typename TIn, bool SAMPLED>
__global__ __launch_bounds__(kThreads) void accept_stats_kernel(const TIn *__restrict__ tgt,
                                                                const TIn *__restrict__ drf, int T, int V,
                                                                int ns, float inv_tau, Part *__restrict__ parts) {
    const int s = blockIdx.x, r = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const TIn *row = row_ptr(tgt, drf, b, r, T, V);
    const int lo = s * kSlice, hi = min(V, lo + kSlice);
    float x[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int i = lo + tid + k * kThreads;
        x[k] = i < hi ? ld(row, i) : -INFINITY;
    }
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int i = lo + tid + k * kThreads;
        if (i < hi && (x[k] > bv || bi == INT_MAX)) {   // k ascending: strict > keeps the lowest index
            bv = x[k];
            bi = i;
        }
    }
    float m = -INFINITY, sum = 0.f;
    if constexpr (SAMPLED) {
#pragma unroll
        for (int k = 0; k < kPer; ++k) m = fmaxf(m, x[k] * inv_tau);
        if (m != -INFINITY) {
#pragma unroll
            for (int k = 0; k < kPer; ++k) sum += __expf(x[k] * inv_tau - m);
        }
    }
    // Wave reduction, then across the four waves through LDS.
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        amax_merge(bv, bi, __shfl_xor(bv, off, 64), __shfl_xor(bi, off, 64));
        if constexpr (SAMPLED) lse_merge(m, sum, __shfl_xor(m, off, 64), __shfl_xor(sum, off, 64));
    }
    __shared__ Part wp[kThreads / 64];
    const int w = tid >> 6;
    if ((tid & 63) == 0) wp[w] = Part{m, sum, bv, bi};
    __syncthreads();
    if (tid == 0) {
        Part p = wp[0];
#pragma unroll
        for (int j = 1; j < kThreads / 64; ++j) {
            amax_merge(p.bv, p.bi, wp[j].bv, wp[j].bi);
            if constexpr (SAMPLED) lse_merge(p.m, p.s, wp[j].m, wp[j].s);
        }
        parts[(size_t(b) * gridDim.y + r) * ns + s] = p;
    }
}

constexpr int kPartChunk = 2048;   // (row, slice) statistics staged in LDS at a time

// The decision for sequence b, by one whole workgroup: combine the slices of
// every row (statistics staged in LDS, one row per wave), then walk the drafts.
// Returns m (kept drafts) to every thread; for sampled mode *pk_out gets the
// draw's description, and for greedy mode *greedy_next the emitted token.
template <typename TIn, bool SAMPLED>
__device__ __forceinline__ int decide_block(const TIn *__restrict__ tgt, const TIn *__restrict__ drf,
                                            const int32_t *__restrict__ drafts, const float *__restrict__ u_acc,
                                            int b, int T, int V, int ns, float inv_tau,
                                            const Part *__restrict__ parts, Pick *pk_out, int *greedy_next) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int rows = SAMPLED ? 2 * T - 1 : T;
    __shared__ Part stage[kPartChunk];
    __shared__ float M[2 * GDN_T_MAX], S[2 * GDN_T_MAX], BV[2 * GDN_T_MAX];
    __shared__ int AM[2 * GDN_T_MAX];
    if (tid < rows) {
        M[tid] = -INFINITY;
        S[tid] = 0.f;
        BV[tid] = -INFINITY;
        AM[tid] = INT_MAX;
    }
    // Every draft token, its uniform and (sampled) its two logits, fetched by one
    // lane each first (their loads overlap the staging below), so the walk reads only LDS.
    __shared__ int D[GDN_T_MAX];
    __shared__ float U[GDN_T_MAX], ZT[GDN_T_MAX], ZD[GDN_T_MAX];
    if (tid < T - 1) {
        const int d = drafts[size_t(b) * (T - 1) + tid];
        D[tid] = d;
        if constexpr (SAMPLED) {
            const bool ok = d >= 0 && d < V;
            U[tid] = u_acc[size_t(b) * (T - 1) + tid];
            ZT[tid] = ok ? ld(tgt, (size_t(b) * T + tid) * V + d) : 0.f;
            ZD[tid] = ok ? ld(drf, (size_t(b) * (T - 1) + tid) * V + d) : 0.f;
        }
    }
    const Part *pb = parts + size_t(b) * rows * ns;
    // Rows are walked in groups whose statistics fit the stage.
    const int rpc = max(1, kPartChunk / ns);            // whole rows per stage
    for (int r0 = 0; r0 < rows; r0 += rpc) {
        const int nr = min(rpc, rows - r0);
        for (int s0 = 0; s0 < ns; s0 += kPartChunk) {   // (a row longer than the stage: in pieces)
            const int sn = min(kPartChunk, ns - s0);
            const int cnt = nr == 1 ? sn : nr * ns;
            __syncthreads();
            for (int e = tid; e < cnt; e += kThreads) {
                const int rr = nr == 1 ? 0 : e / ns, jj = nr == 1 ? s0 + e : e - rr * ns;
                stage[e] = pb[size_t(r0 + rr) * ns + jj];
            }
            __syncthreads();
            for (int rr = w; rr < nr; rr += kThreads / 64) {
                float m = -INFINITY, sm = 0.f, bv = -INFINITY;
                int bi = INT_MAX;
                const int len = nr == 1 ? sn : ns;
                for (int j2 = lane; j2 < len; j2 += 64) {
                    const Part pp = stage[(nr == 1 ? 0 : rr * ns) + j2];
                    amax_merge(bv, bi, pp.bv, pp.bi);
                    if constexpr (SAMPLED) lse_merge(m, sm, pp.m, pp.s);
                }
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) {
                    amax_merge(bv, bi, __shfl_xor(bv, off, 64), __shfl_xor(bi, off, 64));
                    if constexpr (SAMPLED) lse_merge(m, sm, __shfl_xor(m, off, 64), __shfl_xor(sm, off, 64));
                }
                if (lane == 0) {
                    const int r = r0 + rr;
                    amax_merge(BV[r], AM[r], bv, bi);
                    if constexpr (SAMPLED) lse_merge(M[r], S[r], m, sm);
                }
            }
        }
    }
    __syncthreads();
    // The walk (cheap: at most T - 1 steps over LDS), by every thread alike.
    int m = 0;
    if constexpr (!SAMPLED) {
        while (m < T - 1 && D[m] == AM[m]) ++m;
        *greedy_next = AM[m];
    } else {
        while (m < T - 1) {
            const int d = D[m];
            if (d < 0 || d >= V) break;   // an out-of-range draft is rejected
            const float p = __expf(ZT[m] * inv_tau - M[m]) / S[m];
            const float q = __expf(ZD[m] * inv_tau - M[T + m]) / S[T + m];
            if (!(U[m] * q < p)) break;
            ++m;
        }
        Pick pk;
        pk.row = m;
        pk.residual = m < T - 1;
        pk.mt = M[m];
        pk.st = S[m];
        pk.md = pk.residual ? M[T + m] : 0.f;
        pk.sd = pk.residual ? S[T + m] : 1.f;
        pk.amax = AM[m];
        pk.pad = 0;
        *pk_out = pk;
    }
    __syncthreads();   // the staging buffers may be reused by the caller
    return m;
}

// Greedy decision: one workgroup per sequence.
template <typename TIn>
__global__ __launch_bounds__(kThreads) void accept_decide_kernel(const TIn *__restrict__ tgt,
                                                                 const int32_t *__restrict__ drafts, int T, int V,
                                                                 int ns, const Part *__restrict__ parts,
                                                                 int32_t *__restrict__ n_out,
                                                                 int32_t *__restrict__ next) {
    const int b = blockIdx.x;
    int nx = 0;
    const int m = decide_block<TIn, false>(tgt, nullptr, drafts, nullptr, b, T, V, ns, 1.f, parts, nullptr, &nx);
    if (threadIdx.x == 0) {
        next[b] = nx;
        n_out[b] = m + 1;
    }
}

// Weight of vocabulary entry i in the draw, p(i) or max(0, p(i) - q(i)) in
// fp32, then as an integer in units of 2^-52 (the weights sum to about 1, so a
// 64-bit total cannot overflow).  Every sum and prefix of the draw is then an
// exact integer sum: the same in any order, in any kernel.
constexpr double kFix = 4503599627370496.0;   // 2^52

template <typename TIn>
__device__ inline uint64_t draw_weight(const TIn *trow, const TIn *drow, const Pick &pk, float inv_tau, int i) {
    const float p = __expf(ld(trow, i) * inv_tau - pk.mt) / pk.st;
    float wt = p;
    if (pk.residual) {
        const float q = __expf(ld(drow, i) * inv_tau - pk.md) / pk.sd;
        wt = fmaxf(p - q, 0.f);
    }
    return static_cast<uint64_t>(double(wt) * kFix);
}

__device__ inline uint64_t shfl_xor_u64(uint64_t v, int off) {
    const uint32_t lo = __shfl_xor(uint32_t(v), off, 64), hi = __shfl_xor(uint32_t(v >> 32), off, 64);
    return (uint64_t(hi) << 32) | lo;
}
__device__ inline uint64_t shfl_up_u64(uint64_t v, int off) {
    const uint32_t lo = __shfl_up(uint32_t(v), off, 64), hi = __shfl_up(uint32_t(v >> 32), off, 64);
    return (uint64_t(hi) << 32) | lo;
}

// Exclusive prefix sum over the workgroup's threads (exact: integers).  Returns
// this thread's exclusive prefix; *total gets the sum of all.
__device__ inline uint64_t block_excl_scan(uint64_t v, uint64_t *total) {
    __shared__ uint64_t wsum[kThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    uint64_t incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint64_t y = shfl_up_u64(incl, off);
        if (lane >= off) incl += y;
    }
    __syncthreads();   // wsum free (an earlier scan may still read it)
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    uint64_t base = 0, all = 0;
#pragma unroll
    for (int j = 0; j < kThreads / 64; ++j) {
        if (j < w) base += wsum[j];
        all += wsum[j];
    }
    *total = all;
    return base + incl - v;
}

// Sampled decision and the draw's masses in one launch: every workgroup of a
// sequence makes the same decision from the same statistics (deterministic, so
// they agree), slice 0 publishes it, and each workgroup then weighs its slice
// of the row the token is drawn from.  One launch instead of a decision launch
// followed by a mass launch.
template <typename TIn>
__global__ __launch_bounds__(kThreads) void accept_mass_kernel(const TIn *__restrict__ tgt,
                                                               const TIn *__restrict__ drf,
                                                               const int32_t *__restrict__ drafts,
                                                               const float *__restrict__ u_acc, int T, int V, int ns,
                                                               float inv_tau, const Part *__restrict__ parts,
                                                               Pick *__restrict__ pick, int32_t *__restrict__ n_out,
                                                               uint64_t *__restrict__ mass) {
    const int s = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    Pick pk;
    const int m = decide_block<TIn, true>(tgt, drf, drafts, u_acc, b, T, V, ns, inv_tau, parts, &pk, nullptr);
    if (s == 0 && tid == 0) {
        pick[b] = pk;
        n_out[b] = m + 1;
    }
    const TIn *trow = tgt + (size_t(b) * T + pk.row) * V;
    const TIn *drow = pk.residual ? drf + (size_t(b) * (T - 1) + pk.row) * V : nullptr;
    const int lo = s * kSlice, hi = min(V, lo + kSlice);
    uint64_t acc = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int i = lo + tid + k * kThreads;
        if (i < hi) acc += draw_weight(trow, drow, pk, inv_tau, i);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += shfl_xor_u64(acc, off);
    __shared__ uint64_t ws[kThreads / 64];
    if ((tid & 63) == 0) ws[tid >> 6] = acc;
    __syncthreads();
    if (tid == 0) mass[size_t(b) * ns + s] = ws[0] + ws[1] + ws[2] + ws[3];
}

// The draw: target t = floor(u * total); the slice whose cumulative mass first
// passes t, then the entry within it.  All sums exact, so the slice's entries
// add up to its mass and the search always ends on an entry with weight.
template <typename TIn>
__global__ __launch_bounds__(kThreads) void accept_pick_kernel(const TIn *__restrict__ tgt,
                                                               const TIn *__restrict__ drf, int T, int V, int ns,
                                                               float inv_tau, const Pick *__restrict__ pick,
                                                               const uint64_t *__restrict__ mass,
                                                               const float *__restrict__ u_sample,
                                                               int32_t *__restrict__ next) {
    const int b = blockIdx.x, tid = threadIdx.x;
    const Pick pk = pick[b];
    const uint64_t *mb = mass + size_t(b) * ns;
    __shared__ int s_slice, s_found;
    __shared__ uint64_t s_rem;
    // Total mass (exact), then t.
    uint64_t part = 0;
    for (int j = tid; j < ns; j += kThreads) part += mb[j];
    uint64_t total;
    block_excl_scan(part, &total);
    if (total == 0) {   // every weight underflowed: the target row's argmax
        if (tid == 0) next[b] = pk.amax;
        return;
    }
    uint64_t t = static_cast<uint64_t>(double(u_sample[b]) * double(total));
    if (t >= total) t = total - 1;
    if (tid == 0) s_slice = INT_MAX;
    // The slice: chunks of kThreads slices, scanned in order.
    uint64_t carry = 0;
    for (int c0 = 0; c0 < ns; c0 += kThreads) {
        const int j = c0 + tid;
        const uint64_t mj = j < ns ? mb[j] : 0;
        uint64_t csum;
        const uint64_t ex = carry + block_excl_scan(mj, &csum);
        if (j < ns && ex <= t && t < ex + mj) {   // exactly one slice owns t
            s_slice = j;
            s_rem = t - ex;
        }
        carry += csum;
        __syncthreads();
        if (s_slice != INT_MAX) break;
    }
    const int sl = s_slice;
    const uint64_t rem = s_rem;
    // Within the slice: thread j owns entries lo + j kPer .. + kPer - 1, in order.
    const TIn *trow = tgt + (size_t(b) * T + pk.row) * V;
    const TIn *drow = pk.residual ? drf + (size_t(b) * (T - 1) + pk.row) * V : nullptr;
    const int lo = sl * kSlice + tid * kPer, hi = min(V, sl * kSlice + kSlice);
    uint64_t w[kPer], mine = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int i = lo + k;
        w[k] = i < hi ? draw_weight(trow, drow, pk, inv_tau, i) : 0;
        mine += w[k];
    }
    uint64_t stot;
    const uint64_t ex = block_excl_scan(mine, &stot);
    // (The entries were weighed again here; should any weight come out
    // differently from the mass kernel's, the target stays inside the slice.)
    const uint64_t rm = stot > 0 && rem >= stot ? stot - 1 : rem;
    if (tid == 0) s_found = INT_MAX;
    __syncthreads();
    if (ex <= rm && rm < ex + mine) {
        uint64_t r = ex;
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            r += w[k];
            if (r > rm) {
                s_found = lo + k;
                break;
            }
        }
    }
    __syncthreads();
    if (tid == 0) next[b] = s_found != INT_MAX ? s_found : pk.amax;
}

// Filter history rewind: thread per channel, the new window assembled in
// registers before it is written back.
template <typename E>
__global__ __launch_bounds__(256) void history_rewind_kernel(E *__restrict__ hist, const E *__restrict__ rows,
                                                             const int32_t *__restrict__ n, int W, int T, int C) {
    constexpr int kMaxW = GDN_HISTORY_MAX;
    const int c = blockIdx.x * 256 + threadIdx.x, b = blockIdx.y;
    if (c >= C) return;
    const int nn = n[b];
    if (nn < 0 || nn > T) return;   // out of range: the history is left as it was
    E v[kMaxW];
#pragma unroll
    for (int j = 0; j < kMaxW; ++j) {
        if (j < W) {
            const int k = j + nn;   // index in [history; rows 0 .. n-1]
            v[j] = k < W ? hist[(size_t(b) * W + k) * C + c] : rows[(size_t(b) * T + (k - W)) * C + c];
        }
    }
#pragma unroll
    for (int j = 0; j < kMaxW; ++j)
        if (j < W) hist[(size_t(b) * W + j) * C + c] = v[j];
}

struct AcceptWs {
    size_t parts, pick, mass, total;
};

AcceptWs accept_ws_layout(int B, int T, int V, bool sampled) {
    const int ns = (V + kSlice - 1) / kSlice, rows = sampled ? 2 * T - 1 : T;
    AcceptWs w;
    w.parts = 0;
    w.pick = w.parts + align256(size_t(B) * rows * ns * sizeof(Part));
    w.mass = w.pick + align256(size_t(B) * sizeof(Pick));
    w.total = w.mass + (sampled ? align256(size_t(B) * ns * sizeof(uint64_t)) : 0);
    return w;
}

template <typename TIn>
hipError_t accept_greedy_t(const TIn *tgt, const int32_t *drafts, int B, int T, int V, int32_t *n_out,
                           int32_t *next, uint8_t *ws, hipStream_t st) {
    const int ns = (V + kSlice - 1) / kSlice;
    const AcceptWs L = accept_ws_layout(B, T, V, false);
    Part *parts = reinterpret_cast<Part *>(ws + L.parts);
    hipLaunchKernelGGL((accept_stats_kernel<TIn, false>), dim3(ns, T, B), dim3(kThreads), 0, st, tgt,
                       static_cast<const TIn *>(nullptr), T, V, ns, 1.f, parts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((accept_decide_kernel<TIn>), dim3(B), dim3(kThreads), 0, st, tgt, drafts, T, V, ns, parts,
                       n_out, next);
    return hipGetLastError();
}

template <typename TIn>
hipError_t accept_sampled_t(const TIn *tgt, const TIn *drf, const int32_t *drafts, const float *u_acc,
                            const float *u_samp, float inv_tau, int B, int T, int V, int32_t *n_out,
                            int32_t *next, uint8_t *ws, hipStream_t st) {
    const int ns = (V + kSlice - 1) / kSlice;
    const AcceptWs L = accept_ws_layout(B, T, V, true);
    Part *parts = reinterpret_cast<Part *>(ws + L.parts);
    Pick *pick = reinterpret_cast<Pick *>(ws + L.pick);
    uint64_t *mass = reinterpret_cast<uint64_t *>(ws + L.mass);
    hipLaunchKernelGGL((accept_stats_kernel<TIn, true>), dim3(ns, 2 * T - 1, B), dim3(kThreads), 0, st, tgt, drf, T,
                       V, ns, inv_tau, parts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((accept_mass_kernel<TIn>), dim3(ns, B), dim3(kThreads), 0, st, tgt, drf, drafts, u_acc, T, V,
                       ns, inv_tau, parts, pick, n_out, mass);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((accept_pick_kernel<TIn>), dim3(B), dim3(kThreads), 0, st, tgt, drf, T, V, ns, inv_tau,
                       pick, mass, u_samp, next);
    return hipGetLastError();
}

}  // namespace

size_t accept_workspace_bytes(int B, int T, int V, bool sampled) {
    return accept_ws_layout(B, T, V, sampled).total;
}

hipError_t launch_accept_greedy(const void *tgt, gdn_in_dtype dt, const int32_t *drafts, int B, int T, int V,
                                int32_t *n_out, int32_t *next, void *ws, hipStream_t st) {
    uint8_t *w = static_cast<uint8_t *>(ws);
    if (dt == GDN_IN_BF16)
        return accept_greedy_t(static_cast<const __hip_bfloat16 *>(tgt), drafts, B, T, V, n_out, next, w, st);
    return accept_greedy_t(static_cast<const float *>(tgt), drafts, B, T, V, n_out, next, w, st);
}

hipError_t launch_accept_sampled(const void *tgt, const void *drf, gdn_in_dtype dt, const int32_t *drafts,
                                 const float *u_acc, const float *u_samp, float inv_tau, int B, int T, int V,
                                 int32_t *n_out, int32_t *next, void *ws, hipStream_t st) {
    uint8_t *w = static_cast<uint8_t *>(ws);
    if (dt == GDN_IN_BF16)
        return accept_sampled_t(static_cast<const __hip_bfloat16 *>(tgt), static_cast<const __hip_bfloat16 *>(drf),
                                drafts, u_acc, u_samp, inv_tau, B, T, V, n_out, next, w, st);
    return accept_sampled_t(static_cast<const float *>(tgt), static_cast<const float *>(drf), drafts, u_acc, u_samp,
                            inv_tau, B, T, V, n_out, next, w, st);
}

// Scratch of gdn_accept_sampled_noalloc: the workspace of one sampled call (per
// slice statistics, draw descriptors, slice masses), in device memory that the
// library owns for the life of the process, so that the call allocates nothing.
// Each device holds its own copy.  In host code `scratch` names a host-side
// stand-in, never the device array: its device address comes from
// hipGetSymbolAddress, resolved once per device (with that device current) and
// kept in scratch_ptr[].  Every call on a device shares that device's array;
// calls that overlap on one device race.
namespace {
static __device__ __align__(256) uint8_t scratch[kAcceptScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag scratch_once[kMaxDevices];
void *scratch_ptr[kMaxDevices];
hipError_t scratch_err[kMaxDevices];

// The device address of `scratch` on device `dev`, resolved on first use with
// `dev` current (the caller's current device is restored).
hipError_t scratch_on(int dev, void **out) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(scratch_once[dev], [dev] {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
        void *p = nullptr;
        if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur >= 0 && cur != dev) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        scratch_ptr[dev] = e == hipSuccess ? p : nullptr;
        scratch_err[dev] = e == hipSuccess && p == nullptr ? hipErrorInvalidSymbol : e;
    });
    *out = scratch_ptr[dev];
    return scratch_err[dev];
}
}  // namespace

hipError_t launch_accept_sampled_noalloc(const void *tgt, const void *drf, gdn_in_dtype dt, const int32_t *drafts,
                                         const float *u_acc, const float *u_samp, float inv_tau, int B, int T, int V,
                                         int32_t *n_out, int32_t *next, hipStream_t st) {
    if (accept_workspace_bytes(B, T, V, true) > kAcceptScratchBytes) return hipErrorInvalidValue;
    int dev = -1;
    hipError_t e = st != nullptr ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    void *ws = nullptr;
    if ((e = scratch_on(dev, &ws)) != hipSuccess) return e;
    return launch_accept_sampled(tgt, drf, dt, drafts, u_acc, u_samp, inv_tau, B, T, V, n_out, next, ws, st);
}

hipError_t launch_history_rewind(void *hist, const void *rows, const int32_t *n, int B, int W, int T, int C,
                                 gdn_in_dtype dt, hipStream_t st) {
    const dim3 grid((C + 255) / 256, B);
    if (dt == GDN_IN_BF16)
        hipLaunchKernelGGL((history_rewind_kernel<uint16_t>), grid, dim3(256), 0, st, static_cast<uint16_t *>(hist),
                           static_cast<const uint16_t *>(rows), n, W, T, C);
    else
        hipLaunchKernelGGL((history_rewind_kernel<uint32_t>), grid, dim3(256), 0, st, static_cast<uint32_t *>(hist),
                           static_cast<const uint32_t *>(rows), n, W, T, C);
    return hipGetLastError();
}

}  // namespace gdn
