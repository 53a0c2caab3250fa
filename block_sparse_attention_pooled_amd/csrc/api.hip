// C ABI entry points (include/stepdllm.h): validation, workspace carve-up,
// launch sequencing and the denoising-step driver.  Host code only.
//
// Schedule: "Step-dLLM: Adaptive Step-aware Sparse Attention for Efficient
// Diffusion LLM Inference", abstract (mask refreshed at anchor steps, reused
// within each interval); "SparseD: Sparse Attention for Diffusion Language
// Models", abstract (dense attention for the early steps, then one sparse
// pattern reused for every later step).
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/stepdllm.h"
#include "common.h"

using sd::Dims;
using sd::WsLayout;

namespace {

int check_dims(const stepdllm_dims *d, Dims *out) {
    if (!d) return STEPDLLM_EINVAL;
    if (d->n_q_heads <= 0 || d->n_kv_heads <= 0 || d->seq_len <= 0 || d->head_dim <= 0 ||
        d->block <= 0)
        return STEPDLLM_EINVAL;
    if (d->n_q_heads % d->n_kv_heads != 0) return STEPDLLM_EINVAL;
    if (d->n_q_heads > sd::kMaxHeads) return STEPDLLM_EUNSUPPORTED;
    if (d->seq_len % d->block != 0) return STEPDLLM_EINVAL;
    if (d->head_dim != 64 && d->head_dim != 128) return STEPDLLM_EUNSUPPORTED;
    if (d->block != 64 && d->block != 128) return STEPDLLM_EUNSUPPORTED;
    const int64_t nb = d->seq_len / d->block;
    if (nb > sd::kMaxBlocks) return STEPDLLM_EUNSUPPORTED;
    if ((int64_t)d->n_q_heads * nb * nb >= ((int64_t)1 << 31)) return STEPDLLM_EUNSUPPORTED;
    if ((int64_t)d->n_q_heads * d->seq_len * d->head_dim >= ((int64_t)1 << 40))
        return STEPDLLM_EUNSUPPORTED;
    if (out) {
        out->H = d->n_q_heads;
        out->Hkv = d->n_kv_heads;
        out->L = d->seq_len;
        out->d = d->head_dim;
        out->B = d->block;
        out->nb = (int)nb;
        out->G = d->n_q_heads / d->n_kv_heads;
    }
    return STEPDLLM_OK;
}

// Budget of kept entries out of n for sparsity s: ceil((1 - s) * n), with s
// read as the decimal number the caller wrote, i.e. the decimal with the
// fewest significant digits that converts back to the same double (the
// nearest of that length).  The ceiling is then exact: with s = m / 10^e,
// (1 - s) * n = n - m * n / 10^e, so K = n - floor(m * n / 10^e) in 128-bit
// integers (m < 10^17, n < 2^31).  s = 0 keeps all n, s = 1 keeps none.
int64_t exact_budget(int64_t n, double s) {
    if (!(s > 0.0)) return n;
    if (s >= 1.0) return 0;
    for (int p = 1; p <= 17; ++p) {
        char buf[48];
        snprintf(buf, sizeof buf, "%.*e", p - 1, s);   // d.ddd...e-XX, p digits
        if (strtod(buf, nullptr) != s) continue;
        unsigned long long digits = 0;
        const char *c = buf;
        for (; *c && *c != 'e'; ++c)
            if (*c >= '0' && *c <= '9') digits = digits * 10 + (unsigned long long)(*c - '0');
        const int e = (p - 1) - atoi(c + 1);   // s = digits / 10^e, e >= 1
        if (e > 36) return n;                  // s * n < 1
        unsigned __int128 pow10 = 1;
        for (int i = 0; i < e; ++i) pow10 *= 10;
        return n - (int64_t)(((unsigned __int128)digits * (unsigned __int128)n) / pow10);
    }
    return n;   // not reached: 17 significant digits always read back
}

int64_t keep_count(const Dims &D, double s) { return exact_budget(D.n_scores(), s); }

// Uniform per-head budget: k_h of each head's nb * nb scores.
int64_t keep_count_per_head(const Dims &D, double s) {
    return exact_budget((int64_t)D.nb * D.nb, s);
}

// Column-sparse variant: k_c of each head's L key columns.
int64_t keep_count_columns(const Dims &D, double s) { return exact_budget(D.L, s); }

bool sparsity_ok(double s) { return s >= 0.0 && s <= 1.0; }   // false for NaN

int hip_status(hipError_t e) { return e == hipSuccess ? STEPDLLM_OK : STEPDLLM_EHIP; }

// state_ready: the global select state was already prepared (by the score
// launch of build_mask).
int select_and_plan(const Dims &D, double sparsity, bool per_head, const float *p, char *ws,
                    const WsLayout &w, int32_t *row_ptr, int32_t *col_idx, bool state_ready,
                    hipStream_t s) {
    const int64_t k_h = per_head ? keep_count_per_head(D, sparsity) : 0;
    const int64_t K = per_head ? k_h * D.H : keep_count(D, sparsity);
    // The global budget's list launch also writes the plan's row records and
    // head counts.
    int st = hip_status(
        per_head ? sd::launch_select_per_head(D, k_h, p, ws, w, row_ptr, col_idx, s)
                 : sd::launch_select(D, K, p, ws, w, row_ptr, col_idx, state_ready, true, s));
    if (st) return st;
    return hip_status(sd::launch_plan(D, row_ptr, col_idx, K, ws, w, !per_head, s));
}

int build_mask(const stepdllm_dims *dims, double sparsity, bool per_head, const uint16_t *q,
               const uint16_t *k, void *ws, size_t ws_bytes, int32_t *row_ptr, int32_t *col_idx,
               float *scores_out, void *stream) {
    Dims D;
    int st = check_dims(dims, &D);
    if (st) return st;
    if (!sparsity_ok(sparsity) || !q || !k || !ws || !row_ptr || !col_idx) return STEPDLLM_EINVAL;
    WsLayout w = sd::ws_layout(D);
    if ((int64_t)ws_bytes < w.total) return STEPDLLM_EWORKSPACE;
    char *base = static_cast<char *>(ws);
    hipStream_t s = static_cast<hipStream_t>(stream);
    float *qb = reinterpret_cast<float *>(base + w.qb);
    float *kb = reinterpret_cast<float *>(base + w.kb);
    float *p = reinterpret_cast<float *>(base + w.p);
    // Global budget: the pool launch prepares the select state and the score
    // launch counts the first digit of the select.
    const int64_t sel_init_K = per_head ? -1 : keep_count(D, sparsity);
    if ((st = hip_status(sd::launch_pool(D, q, k, qb, kb, base, w, sel_init_K, s)))) return st;
    if ((st = hip_status(sd::launch_scores(D, qb, kb, p, scores_out, base, w, !per_head, s))))
        return st;
    return select_and_plan(D, sparsity, per_head, p, base, w, row_ptr, col_idx, !per_head, s);
}

int select_mask(const stepdllm_dims *dims, double sparsity, bool per_head, const float *scores,
                void *ws, size_t ws_bytes, int32_t *row_ptr, int32_t *col_idx, void *stream) {
    Dims D;
    int st = check_dims(dims, &D);
    if (st) return st;
    if (!sparsity_ok(sparsity) || !scores || !ws || !row_ptr || !col_idx) return STEPDLLM_EINVAL;
    WsLayout w = sd::ws_layout(D);
    if ((int64_t)ws_bytes < w.total) return STEPDLLM_EWORKSPACE;
    return select_and_plan(D, sparsity, per_head, scores, static_cast<char *>(ws), w, row_ptr,
                           col_idx, false, static_cast<hipStream_t>(stream));
}

int build_col_mask(const stepdllm_dims *dims, double sparsity, const uint16_t *q,
                   const uint16_t *k, void *ws, size_t ws_bytes, int32_t *cols,
                   float *scores_out, void *stream) {
    Dims D;
    int st = check_dims(dims, &D);
    if (st) return st;
    if (!sparsity_ok(sparsity) || !q || !k || !ws || !cols) return STEPDLLM_EINVAL;
    WsLayout w = sd::ws_layout(D);
    if ((int64_t)ws_bytes < w.total) return STEPDLLM_EWORKSPACE;
    char *base = static_cast<char *>(ws);
    hipStream_t s = static_cast<hipStream_t>(stream);
    float *qb = reinterpret_cast<float *>(base + w.qb);
    float *c = scores_out ? scores_out : reinterpret_cast<float *>(base + w.col_scores);
    if ((st = hip_status(sd::launch_pool_q(D, q, qb, s)))) return st;
    if ((st = hip_status(sd::launch_col_scores(D, qb, k, base, w, c, s)))) return st;
    return hip_status(
        sd::launch_col_select(D, keep_count_columns(D, sparsity), c, base, w, cols, s));
}

int col_attn(const stepdllm_dims *dims, const uint16_t *q, const uint16_t *k, const uint16_t *v,
             const int32_t *cols, int64_t k_c, uint16_t *o, void *stream) {
    Dims D;
    int st = check_dims(dims, &D);
    if (st) return st;
    if (!q || !k || !v || !o || (k_c > 0 && !cols)) return STEPDLLM_EINVAL;
    if (k_c < 0 || k_c > D.L) return STEPDLLM_EINVAL;
    return hip_status(sd::launch_col_attn(D, q, k, v, cols, k_c, o,
                                          static_cast<hipStream_t>(stream)));
}

}  // namespace

struct stepdllm_driver {
    Dims D;
    stepdllm_schedule sched;
    char *ws;
    size_t ws_bytes;
    int32_t *row_ptr, *col_idx;
    int64_t K;
    bool have_mask;
};

extern "C" {

int64_t stepdllm_keep_count(const stepdllm_dims *dims, double sparsity) {
    Dims D;
    int st = check_dims(dims, &D);
    if (st) return st;
    if (!sparsity_ok(sparsity)) return STEPDLLM_EINVAL;
    return keep_count(D, sparsity);
}

int64_t stepdllm_keep_count_per_head(const stepdllm_dims *dims, double sparsity) {
    Dims D;
    int st = check_dims(dims, &D);
    if (st) return st;
    if (!sparsity_ok(sparsity)) return STEPDLLM_EINVAL;
    return keep_count_per_head(D, sparsity) * D.H;
}

int64_t stepdllm_keep_count_columns(const stepdllm_dims *dims, double sparsity) {
    Dims D;
    int st = check_dims(dims, &D);
    if (st) return st;
    if (!sparsity_ok(sparsity)) return STEPDLLM_EINVAL;
    return keep_count_columns(D, sparsity);
}

int64_t stepdllm_workspace_bytes(const stepdllm_dims *dims) {
    Dims D;
    int st = check_dims(dims, &D);
    if (st) return st;
    return sd::ws_layout(D).total;
}

int stepdllm_workspace_layout(const stepdllm_dims *dims, stepdllm_ws_layout *out) {
    Dims D;
    int st = check_dims(dims, &D);
    if (st) return st;
    if (!out) return STEPDLLM_EINVAL;
    WsLayout w = sd::ws_layout(D);
    out->pooled_q = w.qb;
    out->pooled_k = w.kb;
    out->scores = w.p;
    out->select = w.sel;
    out->work = w.work;
    out->work_meta = w.work_meta;
    out->head_select = w.hsel;
    out->col_scores = w.col_scores;
    out->col_stats = w.col_stats;
    out->work_rec = w.work_rec;
    out->total = w.total;
    return STEPDLLM_OK;
}

int stepdllm_build_mask(const stepdllm_dims *dims, double sparsity, const uint16_t *q,
                        const uint16_t *k, void *ws, size_t ws_bytes, int32_t *row_ptr,
                        int32_t *col_idx, float *scores_out, void *stream) {
    return build_mask(dims, sparsity, false, q, k, ws, ws_bytes, row_ptr, col_idx, scores_out,
                      stream);
}

int stepdllm_build_mask_per_head(const stepdllm_dims *dims, double sparsity, const uint16_t *q,
                                 const uint16_t *k, void *ws, size_t ws_bytes, int32_t *row_ptr,
                                 int32_t *col_idx, float *scores_out, void *stream) {
    return build_mask(dims, sparsity, true, q, k, ws, ws_bytes, row_ptr, col_idx, scores_out,
                      stream);
}

int stepdllm_select_mask(const stepdllm_dims *dims, double sparsity, const float *scores,
                         void *ws, size_t ws_bytes, int32_t *row_ptr, int32_t *col_idx,
                         void *stream) {
    return select_mask(dims, sparsity, false, scores, ws, ws_bytes, row_ptr, col_idx, stream);
}

int stepdllm_select_mask_per_head(const stepdllm_dims *dims, double sparsity,
                                  const float *scores, void *ws, size_t ws_bytes,
                                  int32_t *row_ptr, int32_t *col_idx, void *stream) {
    return select_mask(dims, sparsity, true, scores, ws, ws_bytes, row_ptr, col_idx, stream);
}

int stepdllm_plan(const stepdllm_dims *dims, const int32_t *row_ptr, const int32_t *col_idx,
                  int64_t nnz, void *ws, size_t ws_bytes, void *stream) {
    Dims D;
    int st = check_dims(dims, &D);
    if (st) return st;
    if (!row_ptr || !col_idx || !ws) return STEPDLLM_EINVAL;
    if (nnz < 0 || nnz > D.n_scores()) return STEPDLLM_EINVAL;
    WsLayout w = sd::ws_layout(D);
    if ((int64_t)ws_bytes < w.total) return STEPDLLM_EWORKSPACE;
    return hip_status(sd::launch_plan(D, row_ptr, col_idx, nnz, static_cast<char *>(ws), w, false,
                                      static_cast<hipStream_t>(stream)));
}

int stepdllm_sparse_attn(const stepdllm_dims *dims, const uint16_t *q, const uint16_t *k,
                         const uint16_t *v, const int32_t *col_idx, int64_t nnz,
                         void *ws, size_t ws_bytes, uint16_t *o, void *stream) {
    Dims D;
    int st = check_dims(dims, &D);
    if (st) return st;
    if (!q || !k || !v || !col_idx || !ws || !o) return STEPDLLM_EINVAL;
    if (nnz < 0 || nnz > D.n_scores()) return STEPDLLM_EINVAL;
    WsLayout w = sd::ws_layout(D);
    if ((int64_t)ws_bytes < w.total) return STEPDLLM_EWORKSPACE;
    char *base = static_cast<char *>(ws);
    const int4 *recs = reinterpret_cast<const int4 *>(base + w.work_rec);
    int32_t *meta = reinterpret_cast<int32_t *>(base + w.work_meta);
    return hip_status(sd::launch_sparse_attn(D, q, k, v, col_idx, recs, meta, nnz, o,
                                             static_cast<hipStream_t>(stream)));
}

int stepdllm_sparse_attn_group(const stepdllm_dims *dims, const uint16_t *q, const uint16_t *k,
                               const uint16_t *v, const int32_t *row_ptr,
                               const int32_t *col_idx, int64_t nnz, uint16_t *o, void *stream) {
    Dims D;
    int st = check_dims(dims, &D);
    if (st) return st;
    if (!q || !k || !v || !row_ptr || !col_idx || !o) return STEPDLLM_EINVAL;
    if (nnz < 0 || nnz > D.n_scores()) return STEPDLLM_EINVAL;
    if (D.B != 64) return STEPDLLM_EUNSUPPORTED;
    return hip_status(sd::launch_group_attn(D, q, k, v, row_ptr, col_idx, nnz, o,
                                            static_cast<hipStream_t>(stream)));
}

int stepdllm_dense_attn(const stepdllm_dims *dims, const uint16_t *q, const uint16_t *k,
                        const uint16_t *v, uint16_t *o, void *stream) {
    Dims D;
    int st = check_dims(dims, &D);
    if (st) return st;
    if (!q || !k || !v || !o) return STEPDLLM_EINVAL;
    return hip_status(sd::launch_dense_attn(D, q, k, v, o, static_cast<hipStream_t>(stream)));
}

int stepdllm_build_col_mask(const stepdllm_dims *dims, double sparsity, const uint16_t *q,
                            const uint16_t *k, void *ws, size_t ws_bytes, int32_t *cols,
                            float *scores_out, void *stream) {
    return build_col_mask(dims, sparsity, q, k, ws, ws_bytes, cols, scores_out, stream);
}

int stepdllm_select_col_mask(const stepdllm_dims *dims, double sparsity, const float *scores,
                             void *ws, size_t ws_bytes, int32_t *cols, void *stream) {
    Dims D;
    int st = check_dims(dims, &D);
    if (st) return st;
    if (!sparsity_ok(sparsity) || !scores || !ws || !cols) return STEPDLLM_EINVAL;
    WsLayout w = sd::ws_layout(D);
    if ((int64_t)ws_bytes < w.total) return STEPDLLM_EWORKSPACE;
    return hip_status(sd::launch_col_select(D, keep_count_columns(D, sparsity), scores,
                                            static_cast<char *>(ws), w, cols,
                                            static_cast<hipStream_t>(stream)));
}

int stepdllm_col_attn(const stepdllm_dims *dims, const uint16_t *q, const uint16_t *k,
                      const uint16_t *v, const int32_t *cols, int64_t k_c, uint16_t *o,
                      void *stream) {
    return col_attn(dims, q, k, v, cols, k_c, o, stream);
}

int stepdllm_block_mass(const stepdllm_dims *dims, const uint16_t *q, const uint16_t *k,
                        float *mass, void *stream) {
    Dims D;
    int st = check_dims(dims, &D);
    if (st) return st;
    if (!q || !k || !mass) return STEPDLLM_EINVAL;
    return hip_status(sd::launch_block_mass(D, q, k, mass, static_cast<hipStream_t>(stream)));
}

int stepdllm_col_recall(const stepdllm_dims *dims, const uint16_t *q, const uint16_t *k,
                        const int32_t *cols, int64_t k_c, float *recall, void *stream) {
    Dims D;
    int st = check_dims(dims, &D);
    if (st) return st;
    if (!q || !k || !recall || (k_c > 0 && !cols)) return STEPDLLM_EINVAL;
    if (k_c < 0 || k_c > D.L) return STEPDLLM_EINVAL;
    return hip_status(sd::launch_col_recall(D, q, k, cols, k_c, recall,
                                            static_cast<hipStream_t>(stream)));
}

int stepdllm_mask_recall(const stepdllm_dims *dims, const float *mass, const int32_t *row_ptr,
                         const int32_t *col_idx, int64_t nnz, float *recall, void *stream) {
    Dims D;
    int st = check_dims(dims, &D);
    if (st) return st;
    if (!mass || !row_ptr || !col_idx || !recall) return STEPDLLM_EINVAL;
    if (nnz < 0 || nnz > D.n_scores()) return STEPDLLM_EINVAL;
    return hip_status(sd::launch_mask_recall(D, mass, row_ptr, col_idx, nnz, recall,
                                             static_cast<hipStream_t>(stream)));
}

int stepdllm_driver_create(stepdllm_driver **out, const stepdllm_dims *dims,
                           const stepdllm_schedule *schedule, void *ws, size_t ws_bytes,
                           int32_t *row_ptr, int32_t *col_idx) {
    if (!out) return STEPDLLM_EINVAL;
    *out = nullptr;
    Dims D;
    int st = check_dims(dims, &D);
    if (st) return st;
    if (!schedule || !ws || !col_idx) return STEPDLLM_EINVAL;
    if (!sparsity_ok(schedule->sparsity) || schedule->dense_steps < 0 ||
        schedule->refresh_every < 0 ||
        (schedule->per_head_budget != 0 && schedule->per_head_budget != 1) ||
        (schedule->column_sparse != 0 && schedule->column_sparse != 1) ||
        (schedule->column_sparse && schedule->per_head_budget))
        return STEPDLLM_EINVAL;
    if (!schedule->column_sparse && !row_ptr) return STEPDLLM_EINVAL;
    if ((int64_t)ws_bytes < sd::ws_layout(D).total) return STEPDLLM_EWORKSPACE;
    stepdllm_driver *drv = static_cast<stepdllm_driver *>(malloc(sizeof(stepdllm_driver)));
    if (!drv) return STEPDLLM_ENOMEM;
    drv->D = D;
    drv->sched = *schedule;
    drv->ws = static_cast<char *>(ws);
    drv->ws_bytes = ws_bytes;
    drv->row_ptr = row_ptr;
    drv->col_idx = col_idx;
    drv->K = schedule->column_sparse     ? keep_count_columns(D, schedule->sparsity)
             : schedule->per_head_budget ? keep_count_per_head(D, schedule->sparsity) * D.H
                                         : keep_count(D, schedule->sparsity);
    drv->have_mask = false;
    *out = drv;
    return STEPDLLM_OK;
}

int stepdllm_driver_step_kind(const stepdllm_driver *drv, int32_t step) {
    if (!drv || step < 0) return STEPDLLM_EINVAL;
    const int32_t dense = drv->sched.dense_steps, every = drv->sched.refresh_every;
    if (step < dense) return 0;
    const int32_t since = step - dense;
    if (since == 0 || (every > 0 && since % every == 0)) return 1;
    return 2;
}

int stepdllm_step(stepdllm_driver *drv, int32_t step, const uint16_t *q, const uint16_t *k,
                  const uint16_t *v, uint16_t *o, void *stream) {
    const int kind = stepdllm_driver_step_kind(drv, step);
    if (kind < 0) return kind;
    if (!q || !k || !v || !o) return STEPDLLM_EINVAL;
    stepdllm_dims dims = {drv->D.H, drv->D.Hkv, drv->D.L, drv->D.d, drv->D.B};
    if (kind == 0) return stepdllm_dense_attn(&dims, q, k, v, o, stream);
    if (kind == 1) {
        int st = drv->sched.column_sparse
                     ? build_col_mask(&dims, drv->sched.sparsity, q, k, drv->ws, drv->ws_bytes,
                                      drv->col_idx, nullptr, stream)
                     : build_mask(&dims, drv->sched.sparsity, drv->sched.per_head_budget != 0, q,
                                  k, drv->ws, drv->ws_bytes, drv->row_ptr, drv->col_idx, nullptr,
                                  stream);
        if (st) return st;
        drv->have_mask = true;
    } else if (!drv->have_mask) {
        return STEPDLLM_ESTATE;
    }
    if (drv->sched.column_sparse)
        return col_attn(&dims, q, k, v, drv->col_idx, drv->K, o, stream);
    return stepdllm_sparse_attn(&dims, q, k, v, drv->col_idx, drv->K, drv->ws, drv->ws_bytes, o,
                                stream);
}

int stepdllm_driver_destroy(stepdllm_driver *drv) {
    free(drv);
    return STEPDLLM_OK;
}

const char *stepdllm_status_string(int status) {
    switch (status) {
    case STEPDLLM_OK: return "ok";
    case STEPDLLM_EINVAL: return "invalid argument";
    case STEPDLLM_EUNSUPPORTED: return "unsupported shape (head_dim, block or block count)";
    case STEPDLLM_EWORKSPACE: return "workspace too small";
    case STEPDLLM_EHIP: return "HIP launch error";
    case STEPDLLM_ESTATE: return "no mask built yet (reuse step before any anchor)";
    case STEPDLLM_ENOMEM: return "host memory allocation failed";
    default: return "unknown status";
    }
}

}  // extern "C"
