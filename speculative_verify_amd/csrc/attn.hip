// attn.hip -- the verify pass's full-attention mixer: a T-row block of queries
// against a sequence's key/value cache, split over the context.
//
// The README page ("How it works", region table) gives the design: partition
// the K/V context, accumulate online-softmax statistics locally, merge the
// partial results before the output projection; the audited-numbers page ("How
// does lithos-metal fuse layer mixers on Metal?") keeps those running softmax
// totals in fp32 so the score table is never written.  Query row (t, h) attends
// to cache positions 0 .. ctx-1 and, causally, to the block's rows 0 .. t; query
// head h reads key/value head h / (Hq / Hkv).
//
// Split kernel: one workgroup per (instance, key/value head, 64 query rows,
// context split).  The split's keys stream through LDS in tiles of 64 (keys and
// values copied global -> LDS by global_load_lds, double-buffered); per tile
// each wave (16 query rows) forms S^T = K Q^T on bf16 MFMA (K from LDS as the A
// operand, Q^T held in registers as the B operand), updates its rows' running
// max and sum, and accumulates O^T += V^T P^T (V^T by LDS transpose reads, P^T
// straight from the score registers).  Score tile kt holds keys tau(kt, m) =
// 32 (kt/2) + 8 (m/4) + 4 (kt%2) + m%4, so a lane's scores of tiles 2p and
// 2p + 1 are keys 32p + 8 lg .. + 7: the slots of the B operand of the P V
// contraction over keys 32p .. 32p + 31.  The split writes (max, sum, O) per
// query row; the merge kernel combines the splits.  The split boundaries are
// computed on the device from the context length, so every split has work.
#include <algorithm>

#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kTile = 64;     // keys per tile
constexpr int kRows = 64;     // query rows per workgroup (4 waves x 16)

typedef short v4s __attribute__((ext_vector_type(4)));

__device__ inline f32x4 mma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline int tau(int tt, int m) { return 32 * (tt >> 1) + 8 * (m >> 2) + 4 * (tt & 1) + (m & 3); }
__device__ inline int swz16(int t) { return ((t & 3) << 2) | ((t >> 3) & 3); }
// Byte offset of 16-byte piece `piece` of row r (D-element bf16 rows, pieces
// XOR-swizzled in their low four bits).
template <int D>
__device__ inline int row_off(int r, int piece) {
    return r * (2 * D) + ((piece ^ swz16(r)) << 4);
}
// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// i % 4 of the 8 bytes addressed by lane 4 e + i / 4 (e = 0..3).
__device__ inline bf16x4 read_tr(const uint8_t *p) {
    const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)p);
    return __builtin_bit_cast(bf16x4, r);
}
__device__ inline bf16x8 cat4(const bf16x4 &a, const bf16x4 &b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ inline bf16x8 lds16(const uint8_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }

struct SplitRange {
    int begin, end;
};

// Keys [begin, end) of split s: the ctx + T positions cut into nspl runs of whole
// tiles, computed identically by every workgroup.
__device__ inline SplitRange split_range(int total, int nspl, int s) {
    const int tiles = (total + kTile - 1) / kTile;
    const int per = (tiles + nspl - 1) / nspl;
    const int b = min(total, s * per * kTile), e = min(total, (s + 1) * per * kTile);
    return {b, e};
}

template <int D>
__global__ __launch_bounds__(256) void attn_split_kernel(
    const __hip_bfloat16 *__restrict__ q, const __hip_bfloat16 *__restrict__ k_new,
    const __hip_bfloat16 *__restrict__ v_new, __hip_bfloat16 *__restrict__ k_cache,
    __hip_bfloat16 *__restrict__ v_cache, const int32_t *__restrict__ ctx_arr, int T, int Hq, int Hkv, int Lmax,
    int nspl, float scale_log2, float *__restrict__ part_acc, float *__restrict__ part_ml) {
    constexpr int ROWB = 2 * D;              // bytes per key row
    constexpr int TB = kTile * ROWB;         // bytes per K (or V) tile
    constexpr int NDMA = TB / 1024;          // 1 KiB copies per tile and tensor
    constexpr int KB = D / 32;               // 32-element contraction blocks of a row
    constexpr int DT = D / 16;               // 16-element output tiles
    struct alignas(16) Lds {
        uint8_t K[2][TB], V[2][TB];
    };
    __shared__ Lds sm;
    auto &Ks = sm.K;
    auto &Vs = sm.V;

    const int split = blockIdx.x, gy = blockIdx.y, b = blockIdx.z;
    const int G = Hq / Hkv, R = T * G, RG = (R + kRows - 1) / kRows;
    const int g = gy / RG, rg = gy - g * RG;
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ctx = ctx_arr[b];
    const bool bad = ctx < 0 || ctx > Lmax - T;
    const int total = ctx + T;
    const size_t pslot = ((size_t(b) * Hkv + g) * RG + rg) * nspl + split;
    const size_t kv_row = size_t(Hkv) * D;   // elements between positions

    // The block's rows join the cache at ctx .. ctx + T - 1 (one workgroup per
    // key/value head).  No workgroup of this launch reads those cache rows: the
    // block's keys and values are read from k_new / v_new.
    if (!bad && split == 0 && rg == 0) {
        for (int e = tid; e < T * (D / 8); e += 256) {
            const int t = e / (D / 8), c = (e - t * (D / 8)) * 8;
            const size_t src = (size_t(b) * T + t) * kv_row + size_t(g) * D + c;
            const size_t dst = (size_t(b) * Lmax + ctx + t) * kv_row + size_t(g) * D + c;
            *reinterpret_cast<uint4 *>(k_cache + dst) = *reinterpret_cast<const uint4 *>(k_new + src);
            *reinterpret_cast<uint4 *>(v_cache + dst) = *reinterpret_cast<const uint4 *>(v_new + src);
        }
    }
    const SplitRange sr = bad ? SplitRange{0, 0} : split_range(total, nspl, split);
    const int row = 16 * w + lr;              // this lane's query row in the workgroup
    if (sr.begin >= sr.end) {                 // an empty split: no keys
        if (lg == 0) {
            part_ml[(pslot * kRows + row) * 2] = -INFINITY;
            part_ml[(pslot * kRows + row) * 2 + 1] = 0.f;
        }
        return;
    }

    // Q^T as the B operand: query row i = rg*64 + row, token t = i / G, head
    // g*G + i % G; slots 32 kb + 8 lg .. + 7 of its d.
    const int qi = rg * kRows + row;
    const int qt = qi < R ? qi / G : T - 1;
    bf16x8 qf[KB];
    {
        const bool ok = qi < R;
        const __hip_bfloat16 *qrow = q + ((size_t(b) * T + qt) * Hq + g * G + (ok ? qi % G : 0)) * D;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const uint4 v = ok ? *reinterpret_cast<const uint4 *>(qrow + 32 * kb + 8 * lg) : make_uint4(0, 0, 0, 0);
            qf[kb] = __builtin_bit_cast(bf16x8, v);
        }
    }
    const int vis = qi < R ? ctx + qt : -1;  // last key position this row sees
    const bool rows_full = (rg + 1) * kRows <= R;   // every query row of the workgroup is real

    // Copies of tile k0 into stage st: wave w issues copies u = w, w + 4, ...;
    // copy u fills LDS bytes 1024 u + 16 lane, row r, slot sl = piece ^ swz16(r).
    // A tile of cached positions only (all but the split's last tile, as a rule)
    // is copied from a uniform base with per-lane byte offsets that are the same
    // for every tile and for keys and values; the other tiles take each row's
    // source (cache, block row or clamp) lane by lane.
    static_assert(NDMA % 4 == 0, "every wave issues the same number of copies");
    constexpr int NCW = NDMA / 4;
    uint32_t voff[NCW];
#pragma unroll
    for (int j = 0; j < NCW; ++j) {
        const int byte = 1024 * (w + 4 * j) + 16 * lane;
        const int r = byte / ROWB, sl = (byte - r * ROWB) >> 4;
        voff[j] = uint32_t((size_t(r) * kv_row + 8 * (sl ^ swz16(r))) * 2);
    }
    const bool fast_ok = size_t(kTile) * kv_row * 2 < (size_t(1) << 31);   // offsets fit 32 bits
    auto issue = [&](int k0, int st) {
        const uint32_t lk = lds_addr(Ks[st]), lv = lds_addr(Vs[st]);
        if (fast_ok && k0 + kTile <= ctx) {
            const size_t o = (size_t(b) * Lmax + k0) * kv_row + size_t(g) * D;
            const __hip_bfloat16 *kb = k_cache + o, *vb = v_cache + o;
#pragma unroll
            for (int j = 0; j < NCW; ++j) {
                dma16s_nt(kb, voff[j], lk + 1024 * (w + 4 * j));
                dma16s_nt(vb, voff[j], lv + 1024 * (w + 4 * j));
            }
            return;
        }
#pragma unroll
        for (int u = w; u < NDMA; u += 4) {
            const int byte = 1024 * u + 16 * lane;
            const int r = byte / ROWB, sl = (byte - r * ROWB) >> 4;
            const int piece = sl ^ swz16(r);
            const int p = min(k0 + r, total - 1);          // positions past the split end: any valid row
            const __hip_bfloat16 *ks, *vs;
            if (p < ctx) {
                const size_t o = (size_t(b) * Lmax + p) * kv_row + size_t(g) * D + 8 * piece;
                ks = k_cache + o;
                vs = v_cache + o;
            } else {
                const size_t o = (size_t(b) * T + (p - ctx)) * kv_row + size_t(g) * D + 8 * piece;
                ks = k_new + o;
                vs = v_new + o;
            }
            dma16_nt(ks, lk + 1024 * u);
            dma16_nt(vs, lv + 1024 * u);
        }
    };

    f32x4 acc[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    issue(sr.begin, 0);
    int st = 0;
    for (int k0 = sr.begin; k0 < sr.end; k0 += kTile, st ^= 1) {
        __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0): this tile's copies have landed
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (k0 + kTile < sr.end) issue(k0 + kTile, st ^ 1);
        asm volatile("" ::: "memory");
        const uint8_t *Kc = Ks[st], *Vc = Vs[st];

        // S^T tiles: keys tau(kt, 4 lg + r) of this lane's query row, log2 domain.
        // A tile of cached positions inside the split is visible to every query
        // row of the workgroup (each sees all of the cache): no mask.
        const bool unmasked = rows_full && k0 + kTile <= min(ctx, sr.end);
        float x[4][4];
        float mt = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const int r = tau(kt, lr);
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) s = mma(lds16(Kc + row_off<D>(r, 4 * kb + lg)), qf[kb], s);
            if (unmasked) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) x[kt][r4] = s[r4] * scale_log2;
            } else {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int p = k0 + 32 * (kt >> 1) + 8 * lg + 4 * (kt & 1) + r4;
                    x[kt][r4] = (p <= vis && p < sr.end) ? s[r4] * scale_log2 : -INFINITY;
                }
            }
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) mt = fmaxf(mt, x[kt][r4]);
        }
        mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float mn = fmaxf(m_run, mt);
        const float alpha = mn == -INFINITY ? 1.f : exp2f(m_run - mn);
        float ls = 0.f;
        bf16x8 pb[2];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const float pv = mn == -INFINITY ? 0.f : exp2f(x[kt][r4] - mn);
                ls += pv;
                pb[kt >> 1][4 * (kt & 1) + r4] = static_cast<__bf16>(pv);
            }
        ls += __shfl_xor(ls, 16, 64);
        ls += __shfl_xor(ls, 32, 64);
        l_run = l_run * alpha + ls;
        m_run = mn;
        // O^T += V^T P^T: tile dt's A operand is V^T at d = 32 (dt/2) + 8 (lr/4) +
        // 4 (dt%2) + lr%4 (row lr) and keys 32 pb + 8 lg + {0..7} (slots).
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            f32x4 a = acc[dt];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] *= alpha;
            const int piece = 4 * (dt >> 1) + (lr & 3), h8 = (dt & 1) << 3;
#pragma unroll
            for (int p2 = 0; p2 < 2; ++p2) {
                const int ta = 32 * p2 + 8 * lg + (lr >> 2);
                const bf16x8 va = cat4(read_tr(Vc + row_off<D>(ta, piece) + h8), read_tr(Vc + row_off<D>(ta + 4, piece) + h8));
                a = mma(va, pb[p2], a);
            }
            acc[dt] = a;
        }
    }

    // Partials: lane (lr, lg) holds O^T[d][row] for d = 32 P + 8 lg + {0..7}
    // (tiles 2P and 2P + 1).
    if (lg == 0) {
        part_ml[(pslot * kRows + row) * 2] = m_run;
        part_ml[(pslot * kRows + row) * 2 + 1] = l_run;
    }
    float *pa = part_acc + (pslot * kRows + row) * D;
#pragma unroll
    for (int P = 0; P < DT / 2; ++P) {
        const int d0 = 32 * P + 8 * lg;
        *reinterpret_cast<float4 *>(pa + d0) = make_float4(acc[2 * P][0], acc[2 * P][1], acc[2 * P][2], acc[2 * P][3]);
        *reinterpret_cast<float4 *>(pa + d0 + 4) =
            make_float4(acc[2 * P + 1][0], acc[2 * P + 1][1], acc[2 * P + 1][2], acc[2 * P + 1][3]);
    }
}

// Merge: thread (query row, 4 consecutive d) of one (instance, key/value head,
// 64 query rows) combines the splits: o = sum_s 2^(m_s - M) acc_s / sum_s
// 2^(m_s - M) l_s.  kMergeWg workgroups cover the 64 x D / 4 items of a row
// group.  An instance whose ctx is out of range gets NaN.
constexpr int kMergeChunk = 8;   // splits whose loads are issued together

template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float *__restrict__ part_acc,
                                                         const float *__restrict__ part_ml,
                                                         const int32_t *__restrict__ ctx_arr, int T, int Hq,
                                                         int Hkv, int Lmax, int nspl, float *__restrict__ o) {
    constexpr int RUNS = D / 4;                       // float4 runs of a row
    constexpr int WGS = kRows * RUNS / 256;           // workgroups per row group
    const int gy = blockIdx.x / WGS, part = blockIdx.x - gy * WGS, b = blockIdx.y;
    const int G = Hq / Hkv, R = T * G, RG = (R + kRows - 1) / kRows;
    const int g = gy / RG, rg = gy - g * RG;
    const int e = part * 256 + threadIdx.x;
    const int row = e / RUNS, d0 = (e - row * RUNS) * 4;
    const int qi = rg * kRows + row;
    if (qi >= R) return;
    const int t = qi / G, h = g * G + qi % G;
    float4 *dst = reinterpret_cast<float4 *>(o + ((size_t(b) * T + t) * Hq + h) * D + d0);
    const int ctx = ctx_arr[b];
    if (ctx < 0 || ctx > Lmax - T) {
        const float nan = __builtin_nanf("");
        *dst = make_float4(nan, nan, nan, nan);
        return;
    }
    const size_t base = ((size_t(b) * Hkv + g) * RG + rg) * nspl;
    const float *ml = part_ml + (base * kRows + row) * 2;   // split s at ml[s * 2 * kRows]
    const float *pa = part_acc + (base * kRows + row) * D + d0;
    float M = -INFINITY;
    for (int s = 0; s < nspl; ++s) M = fmaxf(M, ml[size_t(s) * 2 * kRows]);
    float L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < nspl; s0 += kMergeChunk) {
        float m[kMergeChunk], l[kMergeChunk];
        float4 a[kMergeChunk];
#pragma unroll
        for (int k = 0; k < kMergeChunk; ++k) {
            const int s = s0 + k;
            m[k] = s < nspl ? ml[size_t(s) * 2 * kRows] : -INFINITY;
            l[k] = s < nspl ? ml[size_t(s) * 2 * kRows + 1] : 0.f;
            a[k] = s < nspl ? *reinterpret_cast<const float4 *>(pa + size_t(s) * kRows * D)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int k = 0; k < kMergeChunk; ++k) {
            if (m[k] == -INFINITY) continue;
            const float f = exp2f(m[k] - M);
            L += f * l[k];
            acc.x += f * a[k].x;
            acc.y += f * a[k].y;
            acc.z += f * a[k].z;
            acc.w += f * a[k].w;
        }
    }
    const float inv = 1.f / L;
    *dst = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

int split_count(int B, int Hkv, int RG, int Lmax, int T) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    const long pairs = long(B) * Hkv * RG;
    const int tiles = (Lmax + kTile - 1) / kTile;
    long n = (cus + pairs - 1) / pairs;   // about one workgroup a compute unit
    n = std::max(1L, std::min<long>(n, tiles));
    return int(n);
}

template <int D>
hipError_t attn_t(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                  const int32_t *ctx, int T, float scale, const gdn_attn_shape &s, float *o, void *ws,
                  hipStream_t st) {
    const int G = s.Hq / s.Hkv, R = T * G, RG = (R + kRows - 1) / kRows;
    const int nspl = split_count(s.B, s.Hkv, RG, s.Lmax, T);
    const size_t nslot = size_t(s.B) * s.Hkv * RG * nspl * kRows;
    float *part_acc = static_cast<float *>(ws);
    float *part_ml = part_acc + nslot * D;
    const float scale_log2 = scale * 1.4426950408889634f;   // scores in the log2 domain: exp2
    hipLaunchKernelGGL((attn_split_kernel<D>), dim3(nspl, s.Hkv * RG, s.B), dim3(256), 0, st,
                       static_cast<const __hip_bfloat16 *>(q), static_cast<const __hip_bfloat16 *>(k_new),
                       static_cast<const __hip_bfloat16 *>(v_new), static_cast<__hip_bfloat16 *>(k_cache),
                       static_cast<__hip_bfloat16 *>(v_cache), ctx, T, s.Hq, s.Hkv, s.Lmax, nspl, scale_log2,
                       part_acc, part_ml);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_merge_kernel<D>), dim3(s.Hkv * RG * (kRows * D / 4 / 256), s.B), dim3(256), 0, st,
                       part_acc, part_ml, ctx, T, s.Hq, s.Hkv, s.Lmax, nspl, o);
    return hipGetLastError();
}

}  // namespace

size_t attn_workspace_bytes(const gdn_attn_shape &s, int T) {
    const int G = s.Hq / s.Hkv, R = T * G, RG = (R + kRows - 1) / kRows;
    const int nspl = split_count(s.B, s.Hkv, RG, s.Lmax, T);
    const size_t nslot = size_t(s.B) * s.Hkv * RG * nspl * kRows;
    return nslot * (size_t(s.d) + 2) * sizeof(float);
}

hipError_t launch_attn_verify(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                              const int32_t *ctx, int T, float scale, const gdn_attn_shape &s, float *o, void *ws,
                              hipStream_t st) {
    if (s.d == 256) return attn_t<256>(q, k_new, v_new, k_cache, v_cache, ctx, T, scale, s, o, ws, st);
    return attn_t<128>(q, k_new, v_new, k_cache, v_cache, ctx, T, scale, s, o, ws, st);
}

}  // namespace gdn
