// gdn_api.hip -- the C ABI of libgdn (declared in include/gdn.h): host-side
// argument checks, record and workspace sizing, and kernel dispatch.  Every check
// here runs before anything is launched, so a bad argument never reaches the GPU.
#include <limits.h>

#include <vector>

#include <cmath>

#include "gdn_internal.h"

using namespace gdn;

namespace {

bool aligned(const void *p, size_t a) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_shape(const gdn_shape *s) {
    if (!s) return GDN_EINVAL;
    if (s->B < 1 || s->H < 1) return GDN_EDIM;
    if ((s->dk != 64 && s->dk != 128) || (s->dv != 64 && s->dv != 128)) return GDN_EDIM;
    if (int64_t(s->B) * s->H > INT_MAX / 4) return GDN_EDIM;  // grid size and 32-bit row counters
    return GDN_OK;
}

bool valid_dtype(int dt) { return dt == GDN_IN_F32 || dt == GDN_IN_BF16; }

int hip_status(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_EHIP; }

constexpr int32_t kVocabMax = 1 << 26;

int check_accept_shape(const gdn_accept_shape *s) {
    if (s == nullptr) return GDN_EINVAL;
    if (s->B < 1 || s->B > 65535 || s->V < 1 || s->V > kVocabMax) return GDN_EDIM;
    if (s->T < 1 || s->T > GDN_T_MAX) return GDN_ERANGE;
    if (int64_t(s->B) * s->T * s->V > (int64_t(1) << 40)) return GDN_EDIM;
    return GDN_OK;
}

// The mixer's inputs and shape: d = 128, H a multiple of Hk, every pointer set
// and aligned.
int check_mixer(const gdn_mixer_inputs *in, const gdn_shape *shp, int32_t T) {
    int rc = check_shape(shp);
    if (rc != GDN_OK) return rc;
    if (in == nullptr) return GDN_EINVAL;
    if (shp->dk != 128 || shp->dv != 128 || in->Hk < 1 || shp->H % in->Hk != 0) return GDN_EDIM;
    if (T < 1 || T > GDN_T_MAX) return GDN_ERANGE;
    if (!aligned(in->x, 16) || !aligned(in->history, 16) || !aligned(in->conv_w, 16) || !aligned(in->a, 4) ||
        !aligned(in->b, 4) || !aligned(in->A_log, 4) || !aligned(in->dt_bias, 4) || !aligned(in->z, 2) ||
        !aligned(in->norm_w, 4))
        return GDN_EINVAL;
    return GDN_OK;
}

int check_attn_shape(const gdn_attn_shape *s, int32_t T) {
    if (s == nullptr) return GDN_EINVAL;
    if (s->B < 1 || s->B > 65535 || s->Hkv < 1 || s->Hq < s->Hkv || s->Hq % s->Hkv != 0) return GDN_EDIM;
    if (s->d != 128 && s->d != 256) return GDN_EDIM;
    if (T < 1 || T > GDN_T_MAX) return GDN_ERANGE;
    if (s->Lmax < T || int64_t(T) * (s->Hq / s->Hkv) > 256) return GDN_EDIM;
    if (int64_t(s->B) * s->Lmax * s->Hkv * s->d > (int64_t(1) << 40)) return GDN_EDIM;
    return GDN_OK;
}

}  // namespace

extern "C" {

size_t gdn_block_record_bytes(const gdn_shape *shp, int32_t T, gdn_in_dtype in_dt) {
    if (check_shape(shp) != GDN_OK || T < 1 || T > GDN_T_MAX || !valid_dtype(in_dt)) return 0;
    return rec_layout(shp->B, T, shp->H, shp->dk, shp->dv, esize_of(in_dt)).total;
}

int gdn_verify_block(const float *S, const void *q, const void *k, const void *v, const float *g,
                     const float *beta, int32_t T, gdn_in_dtype in_dt, const gdn_shape *shp,
                     float *o, void *record, size_t record_bytes, void *hip_stream) {
    int rc = check_shape(shp);
    if (rc != GDN_OK) return rc;
    if (!valid_dtype(in_dt)) return GDN_EINVAL;
    if (!aligned(S, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
        !aligned(o, 16) || !aligned(record, 16) || !aligned(g, 4) || !aligned(beta, 4))
        return GDN_EINVAL;
    if (T < 1 || T > GDN_T_MAX) return GDN_ERANGE;
    if (record_bytes < gdn_block_record_bytes(shp, T, in_dt)) return GDN_EWS;
    return hip_status(launch_verify(S, q, k, v, g, beta, T, in_dt, *shp, o, record,
                                    static_cast<hipStream_t>(hip_stream)));
}

int gdn_commit(float *S, void *record, const int32_t *n_accepted, int32_t *pos,
               const gdn_shape *shp, void *hip_stream) {
    int rc = check_shape(shp);
    if (rc != GDN_OK) return rc;
    if (!aligned(S, 16) || !aligned(record, 16) || !aligned(n_accepted, 4)) return GDN_EINVAL;
    if (pos != nullptr && !aligned(pos, 4)) return GDN_EINVAL;
    return hip_status(launch_commit(S, record, n_accepted, pos, *shp,
                                    static_cast<hipStream_t>(hip_stream)));
}

int gdn_commit_verify(float *S, void *record_prev, const int32_t *n_accepted, int32_t *pos, const void *q,
                      const void *k, const void *v, const float *g, const float *beta, int32_t T,
                      gdn_in_dtype in_dt, const gdn_shape *shp, float *o, void *record_next,
                      size_t record_next_bytes, void *hip_stream) {
    int rc = check_shape(shp);
    if (rc != GDN_OK) return rc;
    if (!valid_dtype(in_dt)) return GDN_EINVAL;
    if (!aligned(S, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(record_prev, 16) || !aligned(record_next, 16) || !aligned(g, 4) || !aligned(beta, 4) ||
        !aligned(n_accepted, 4))
        return GDN_EINVAL;
    if (pos != nullptr && !aligned(pos, 4)) return GDN_EINVAL;
    // The records must be distinct: record_prev may not start inside record_next
    // (its own length is only known on the device).
    const uintptr_t rp = reinterpret_cast<uintptr_t>(record_prev), rn = reinterpret_cast<uintptr_t>(record_next);
    if (rp >= rn && rp < rn + record_next_bytes) return GDN_EINVAL;
    if (rn > rp && rn - rp < 256) return GDN_EINVAL;  // overlaps record_prev's header at least
    if (T < 1 || T > GDN_T_MAX) return GDN_ERANGE;
    if (record_next_bytes < gdn_block_record_bytes(shp, T, in_dt)) return GDN_EWS;
    return hip_status(launch_commit_verify(S, record_prev, n_accepted, pos, q, k, v, g, beta, T, in_dt, *shp, o,
                                           record_next, static_cast<hipStream_t>(hip_stream)));
}

int gdn_record_status(const void *record, const gdn_shape *shp, int32_t *host_err_bits,
                      void *hip_stream) {
    int rc = check_shape(shp);
    if (rc != GDN_OK) return rc;
    if (!aligned(record, 16) || host_err_bits == nullptr) return GDN_EINVAL;
    std::vector<RecCtrl> ctrl(size_t(shp->B));
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    hipError_t e = hipMemcpyAsync(ctrl.data(), static_cast<const uint8_t *>(record) + 256,
                                  ctrl.size() * sizeof(RecCtrl), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return GDN_EHIP;
    for (int b = 0; b < shp->B; ++b) host_err_bits[b] = int32_t(ctrl[size_t(b)].err);
    return GDN_OK;
}

size_t gdn_prefill_workspace_bytes(const gdn_shape *shp, int32_t L, int32_t chunk) {
    if (check_shape(shp) != GDN_OK || L < 0 || chunk != GDN_PREFILL_CHUNK) return 0;
    return prefill_workspace_bytes(*shp, L);
}

int gdn_prefill_chunked(float *S, const void *q, const void *k, const void *v, const float *g,
                        const float *beta, int32_t L, int32_t chunk, gdn_in_dtype in_dt,
                        const gdn_shape *shp, float *o, void *ws, size_t ws_bytes,
                        void *hip_stream) {
    int rc = check_shape(shp);
    if (rc != GDN_OK) return rc;
    if (in_dt != GDN_IN_BF16) return GDN_EINVAL;  // the chunk kernels take bf16 q, k, v
    if (L < 0 || chunk != GDN_PREFILL_CHUNK) return GDN_ERANGE;
    if (L == 0) return GDN_OK;
    if (!aligned(S, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
        !aligned(o, 16) || !aligned(g, 4) || !aligned(beta, 4))
        return GDN_EINVAL;
    if (ws != nullptr && !aligned(ws, 16)) return GDN_EINVAL;
    if (int64_t(L) * shp->B * shp->H > int64_t(INT_MAX)) return GDN_EDIM;
    return hip_status(launch_prefill(S, q, k, v, g, beta, L, in_dt, *shp, o, ws, ws_bytes,
                                     static_cast<hipStream_t>(hip_stream)));
}

size_t gdn_accept_workspace_bytes(const gdn_accept_shape *shp, int32_t sampled) {
    if (check_accept_shape(shp) != GDN_OK) return 0;
    return accept_workspace_bytes(shp->B, shp->T, shp->V, sampled != 0);
}

int gdn_accept_greedy(const void *target_logits, gdn_in_dtype dt, const int32_t *draft_tokens,
                      const gdn_accept_shape *shp, int32_t *n_out, int32_t *next_token, void *ws,
                      size_t ws_bytes, void *hip_stream) {
    int rc = check_accept_shape(shp);
    if (rc != GDN_OK) return rc;
    if (!valid_dtype(dt)) return GDN_EINVAL;
    if (!aligned(target_logits, size_t(esize_of(dt))) || !aligned(n_out, 4) || !aligned(next_token, 4) ||
        !aligned(ws, 16))
        return GDN_EINVAL;
    if (shp->T > 1 && !aligned(draft_tokens, 4)) return GDN_EINVAL;
    if (ws_bytes < accept_workspace_bytes(shp->B, shp->T, shp->V, false)) return GDN_EWS;
    return hip_status(launch_accept_greedy(target_logits, dt, draft_tokens, shp->B, shp->T, shp->V, n_out,
                                           next_token, ws, static_cast<hipStream_t>(hip_stream)));
}

int gdn_accept_sampled(const void *target_logits, const void *draft_logits, gdn_in_dtype dt,
                       const int32_t *draft_tokens, const float *u_accept, const float *u_sample,
                       float temperature, const gdn_accept_shape *shp, int32_t *n_out, int32_t *next_token,
                       void *ws, size_t ws_bytes, void *hip_stream) {
    int rc = check_accept_shape(shp);
    if (rc != GDN_OK) return rc;
    if (!valid_dtype(dt)) return GDN_EINVAL;
    if (!(temperature > 0.f) || !std::isfinite(temperature)) return GDN_ERANGE;
    const size_t es = size_t(esize_of(dt));
    if (!aligned(target_logits, es) || !aligned(u_sample, 4) || !aligned(n_out, 4) || !aligned(next_token, 4) ||
        !aligned(ws, 16))
        return GDN_EINVAL;
    if (shp->T > 1 && (!aligned(draft_logits, es) || !aligned(draft_tokens, 4) || !aligned(u_accept, 4)))
        return GDN_EINVAL;
    if (ws_bytes < accept_workspace_bytes(shp->B, shp->T, shp->V, true)) return GDN_EWS;
    return hip_status(launch_accept_sampled(target_logits, draft_logits, dt, draft_tokens, u_accept, u_sample,
                                            1.f / temperature, shp->B, shp->T, shp->V, n_out, next_token, ws,
                                            static_cast<hipStream_t>(hip_stream)));
}

int gdn_accept_sampled_noalloc(const void *target_logits, const void *draft_logits, gdn_in_dtype dt,
                               const int32_t *draft_tokens, const float *u_accept, const float *u_sample,
                               float temperature, const gdn_accept_shape *shp, int32_t *n_out,
                               int32_t *next_token, void *hip_stream) {
    int rc = check_accept_shape(shp);
    if (rc != GDN_OK) return rc;
    if (!valid_dtype(dt)) return GDN_EINVAL;
    if (!(temperature > 0.f) || !std::isfinite(temperature)) return GDN_ERANGE;
    const size_t es = size_t(esize_of(dt));
    if (!aligned(target_logits, es) || !aligned(u_sample, 4) || !aligned(n_out, 4) || !aligned(next_token, 4))
        return GDN_EINVAL;
    if (shp->T > 1 && (!aligned(draft_logits, es) || !aligned(draft_tokens, 4) || !aligned(u_accept, 4)))
        return GDN_EINVAL;
    if (accept_workspace_bytes(shp->B, shp->T, shp->V, true) > kAcceptScratchBytes) return GDN_EWS;
    return hip_status(launch_accept_sampled_noalloc(target_logits, draft_logits, dt, draft_tokens, u_accept,
                                                    u_sample, 1.f / temperature, shp->B, shp->T, shp->V, n_out,
                                                    next_token, static_cast<hipStream_t>(hip_stream)));
}

size_t gdn_accept_noalloc_max_bytes(void) { return kAcceptScratchBytes; }

int gdn_history_rewind(void *history, const void *rows, const int32_t *n, int32_t B, int32_t W, int32_t T,
                       int32_t C, gdn_in_dtype dt, void *hip_stream) {
    if (!valid_dtype(dt)) return GDN_EINVAL;
    if (B < 1 || C < 1 || B > 65535) return GDN_EDIM;
    if (W < 1 || W > GDN_HISTORY_MAX || T < 1 || T > GDN_T_MAX) return GDN_ERANGE;
    const size_t es = size_t(esize_of(dt));
    if (!aligned(history, es) || !aligned(rows, es) || !aligned(n, 4)) return GDN_EINVAL;
    return hip_status(
        launch_history_rewind(history, rows, n, B, W, T, C, dt, static_cast<hipStream_t>(hip_stream)));
}

int gdn_mixer_verify(const float *S, const gdn_mixer_inputs *in, int32_t T, const gdn_shape *shp, float *y,
                     void *record, size_t record_bytes, void *hip_stream) {
    int rc = check_mixer(in, shp, T);
    if (rc != GDN_OK) return rc;
    if (!aligned(S, 16) || !aligned(y, 16) || !aligned(record, 16)) return GDN_EINVAL;
    if (record_bytes < gdn_block_record_bytes(shp, T, GDN_IN_BF16)) return GDN_EWS;
    return hip_status(launch_mixer_verify(S, *in, T, *shp, y, record, static_cast<hipStream_t>(hip_stream)));
}

int gdn_mixer_commit_verify(float *S, void *record_prev, const int32_t *n_accepted, int32_t *pos,
                            const gdn_mixer_inputs *in, int32_t T, const gdn_shape *shp, float *y,
                            void *record_next, size_t record_next_bytes, void *hip_stream) {
    int rc = check_mixer(in, shp, T);
    if (rc != GDN_OK) return rc;
    if (!aligned(S, 16) || !aligned(y, 16) || !aligned(record_prev, 16) || !aligned(record_next, 16) ||
        !aligned(n_accepted, 4))
        return GDN_EINVAL;
    if (pos != nullptr && !aligned(pos, 4)) return GDN_EINVAL;
    const uintptr_t rp = reinterpret_cast<uintptr_t>(record_prev), rn = reinterpret_cast<uintptr_t>(record_next);
    if (rp >= rn && rp < rn + record_next_bytes) return GDN_EINVAL;
    if (rn > rp && rn - rp < 256) return GDN_EINVAL;
    if (record_next_bytes < gdn_block_record_bytes(shp, T, GDN_IN_BF16)) return GDN_EWS;
    return hip_status(launch_mixer_commit_verify(S, record_prev, n_accepted, pos, *in, T, *shp, y, record_next,
                                                 static_cast<hipStream_t>(hip_stream)));
}

size_t gdn_attn_workspace_bytes(const gdn_attn_shape *shp, int32_t T) {
    if (check_attn_shape(shp, T) != GDN_OK) return 0;
    return attn_workspace_bytes(*shp, T);
}

int gdn_attn_verify(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                    const int32_t *ctx, int32_t T, float scale, const gdn_attn_shape *shp, float *o, void *ws,
                    size_t ws_bytes, void *hip_stream) {
    int rc = check_attn_shape(shp, T);
    if (rc != GDN_OK) return rc;
    if (!std::isfinite(scale)) return GDN_ERANGE;
    if (!aligned(q, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
        !aligned(v_cache, 16) || !aligned(ctx, 4) || !aligned(o, 16) || !aligned(ws, 16))
        return GDN_EINVAL;
    if (ws_bytes < attn_workspace_bytes(*shp, T)) return GDN_EWS;
    return hip_status(launch_attn_verify(q, k_new, v_new, k_cache, v_cache, ctx, T, scale, *shp, o, ws,
                                         static_cast<hipStream_t>(hip_stream)));
}

const char *gdn_strerror(int status) {
    switch (status) {
        case GDN_OK: return "ok";
        case GDN_EINVAL: return "invalid argument: null or misaligned pointer, or unknown dtype";
        case GDN_EDIM: return "invalid shape: B, H >= 1 and dk, dv in {64, 128} required";
        case GDN_ERANGE: return "out of range: T in [1, 16], L >= 0 and chunk == 64 required";
        case GDN_EWS: return "record or workspace buffer too small";
        case GDN_EHIP: return "HIP runtime error";
        default: return "unknown gdn status";
    }
}

}  // extern "C"
