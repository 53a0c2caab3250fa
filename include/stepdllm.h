/*
 * stepdllm.h -- C ABI of the MI355X (gfx950) pooled block-sparse attention
 * library for diffusion-LLM denoising.
 *
 * What it computes (sources cited by page title and place):
 *  - "Step-dLLM: Adaptive Step-aware Sparse Attention for Efficient Diffusion
 *    LLM Inference" (arXiv 2611.01320), abstract: a diffusion LLM recomputes
 *    full bidirectional attention at every denoising step; Step-dLLM refreshes
 *    a block-sparse mask at anchor steps, reuses it within each interval,
 *    allocates the kept blocks under one head-adaptive global budget, and runs
 *    a fused block-sparse attention kernel, measured against dense
 *    FlashAttention.
 *  - "SparseD: Sparse Attention for Diffusion Language Models"
 *    (arXiv 2509.24014), abstract: full attention in the early steps, then one
 *    sparse pattern computed once and reused for all later steps.
 *  - "Block Approximate Sparse Attention (BA-Att)" abstract: blocks are
 *    selected in a block-wise pre-downsampled (pooled) space.
 *  - "PulseCol" abstract: periodically refreshed column-sparse attention
 *    (individual key columns kept instead of blocks); the column-sparse
 *    entry points below.
 * The pages leave the block score open; this library scores a (query block,
 * key block) pair by the mean-pooled queries and keys, Qb . Kb^T / sqrt(d),
 * softmaxed over key blocks per (head, query block), and keeps the
 * K = ceil((1 - s) * H * nb^2) largest over all heads at once, ties going to
 * the lowest flat index (h * nb + i) * nb + j.
 *
 * Conventions for every entry point:
 *  - bf16 tensors are passed as uint16_t (raw bf16 bits).
 *  - Q and O are [H, L, d] row-major; K and V are [Hkv, L, d]; batch 1.
 *    Query head h reads key/value head h / (H / Hkv).
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *    library never allocates or frees device memory; the caller provides a
 *    workspace of stepdllm_workspace_bytes() bytes (256-byte aligned).
 *  - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *    enqueued asynchronously on it; no call synchronises the host.  Device
 *    faults surface at the caller's next synchronisation.
 *  - Arguments are validated on the host before anything is enqueued; on any
 *    error nothing is launched and a negative stepdllm_status is returned.
 *  - The library holds no global mutable state: calls on different streams
 *    with different workspaces may run concurrently.  Calls that share a
 *    workspace must be ordered by the caller (same stream, or events).
 *  - Supported shapes: head_dim in {64, 128}; block in {64, 128};
 *    seq_len % block == 0; n_q_heads % n_kv_heads == 0; nb = seq_len / block
 *    at most 1024; H at most 1024; H * nb * nb < 2^31.
 */
#ifndef STEPDLLM_H
#define STEPDLLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    STEPDLLM_OK = 0,
    STEPDLLM_EINVAL = -1,       /* bad argument: null pointer, bad size or ratio, sparsity not in [0,1] */
    STEPDLLM_EUNSUPPORTED = -2, /* valid shape the kernels do not implement (head_dim, block, nb) */
    STEPDLLM_EWORKSPACE = -3,   /* workspace smaller than stepdllm_workspace_bytes() */
    STEPDLLM_EHIP = -4,         /* the HIP runtime rejected a launch */
    STEPDLLM_ESTATE = -5,       /* driver: a reuse step came before any mask was built */
    STEPDLLM_ENOMEM = -6        /* driver: the host allocation of the driver object failed */
} stepdllm_status;

typedef struct {
    int32_t n_q_heads;  /* H   */
    int32_t n_kv_heads; /* Hkv */
    int32_t seq_len;    /* L   */
    int32_t head_dim;   /* d   */
    int32_t block;      /* B: tokens per block, for pooling and for the mask */
} stepdllm_dims;

/* Denoising schedule ([SparseD] dense warm-up, [Step-dLLM] anchors + reuse).
 * Step t < dense_steps runs dense attention.  Step dense_steps is an anchor;
 * after it, every refresh_every-th step is an anchor (refresh_every == 0:
 * the first mask is reused to the end).  An anchor builds the mask from its
 * own Q/K and then runs sparse attention with it. */
typedef struct {
    int32_t dense_steps;
    int32_t refresh_every;
    double sparsity;    /* s in [0, 1]: fraction of the H*nb*nb blocks dropped */
    int32_t per_head_budget;  /* 0: head-adaptive global budget (Step-dLLM);
                                 1: the uniform per-head budget it is compared
                                 with (see stepdllm_build_mask_per_head) */
    int32_t column_sparse;    /* 0: block mask; 1: column mask (PulseCol
                                 variant): anchors run stepdllm_build_col_mask,
                                 sparse steps stepdllm_col_attn; col_idx holds
                                 H * k_c entries, row_ptr is unused (may be
                                 NULL); per_head_budget must be 0 */
} stepdllm_schedule;

/* Byte offsets of the intermediates inside a workspace (read-only views for
 * inspection; contents are valid after the call that writes them). */
typedef struct {
    int64_t pooled_q;   /* fp32 [H, nb, d]: block means of Q                      */
    int64_t pooled_k;   /* fp32 [Hkv, nb, d]: block means of K                    */
    int64_t scores;     /* fp32 [H, nb, nb]: row-softmaxed pooled scores          */
    int64_t select;     /* uint32 [32]: [0] cut key, [1] count above the cut,
                           [2] ties kept at the cut, [3] K; the other words
                           are the select's working state                        */
    int64_t work;       /* int32 [8 * cap]: attention work order, cap =
                           min(H, ceil(H/8) + 2) * nb positions per die;
                           -1 = padding                                           */
    int64_t work_meta;  /* int32 [16]: [0] cap, [1] number of non-empty rows,
                           [2], [3] address (low, high word) of the col_idx
                           array the plan was made from, [4] its nnz, [5] H,
                           [6] nb; [7] the plan check word: set to 0 by every
                           plan, then each stepdllm_sparse_attn ORs in 1 if
                           its col_idx, nnz, H or nb differ from [2]-[6] (every
                           row then outputs zeros) and 2 if some row's first
                           two list entries in col_idx differ from the ones
                           its plan record holds (that row outputs zeros)     */
    int64_t head_select;/* uint32 [H, 8]: per-head select state under the uniform
                           budget: [h*8 + 0] cut key, [+1] count above the cut,
                           [+2] ties kept at the cut, [+3] k_h; the column mask
                           uses it with k_c                                       */
    int64_t col_scores; /* fp32 [H, L]: column masses of the last column mask
                           built without scores_out                               */
    int64_t col_stats;  /* fp32 [H, nb, 2]: per pooled query, max (log2 units)
                           and normaliser of its scores over all keys             */
    int64_t work_rec;   /* int32 [8 * cap, 4]: per work position, the record the
                           sparse launch reads: row (-1 = padding), list begin,
                           list end (both clamped into [0, nnz]), first two
                           block ids (bits 0-15 and 16-31, clamped into
                           [0, nb); 0 where the list is shorter)                 */
    int64_t total;      /* == stepdllm_workspace_bytes()                          */
} stepdllm_ws_layout;

/* Number of kept blocks under the head-adaptive global budget (Step-dLLM
 * abstract: one sparsity budget shared by all heads of the layer, so heads
 * compete for it): K = ceil((1 - s) * H * nb^2), counted over query heads.
 * s is read as the decimal number the caller wrote (the shortest decimal that
 * converts back to the same double, e.g. 0.3 for the double nearest 0.3), and
 * the ceiling is evaluated exactly on it, so K never depends on binary
 * representation error.  s in [0, 1]: s = 0 keeps every block, s = 1 none.
 * Host only.  Returns K >= 0, or a negative stepdllm_status. */
int64_t stepdllm_keep_count(const stepdllm_dims *dims, double sparsity);

/* Workspace size in bytes for these dims, or a negative stepdllm_status. */
int64_t stepdllm_workspace_bytes(const stepdllm_dims *dims);

/* Fill *out with the workspace layout for these dims. */
int stepdllm_workspace_layout(const stepdllm_dims *dims, stepdllm_ws_layout *out);

/* Anchor-step mask build (Step-dLLM abstract: mask refreshed at an anchor
 * step under a head-adaptive global budget):
 *   pool Q and K over blocks -> pooled scores + row softmax -> global top-K
 *   -> per-row kept-block lists -> attention work order.
 * q: [H, L, d] bf16, k: [Hkv, L, d] bf16.
 * row_ptr: int32 [H*nb + 1] (out), col_idx: int32 [K] (out), K from
 * stepdllm_keep_count: row r = h*nb + i keeps key blocks
 * col_idx[row_ptr[r] .. row_ptr[r+1]) in ascending order; a row may be empty.
 * scores_out (nullable): fp32 [H, nb, nb] copy of the softmaxed scores.
 * The work order is left in the workspace for stepdllm_sparse_attn. */
int stepdllm_build_mask(const stepdllm_dims *dims, double sparsity,
                        const uint16_t *q, const uint16_t *k,
                        void *ws, size_t ws_bytes,
                        int32_t *row_ptr, int32_t *col_idx, float *scores_out,
                        void *stream);

/* The selection half of the mask build on caller-given scores: global top-K
 * of scores [H, nb, nb] fp32 (finite; order is by value, ties by lowest flat
 * index), per-row lists and work order.  Same outputs as stepdllm_build_mask. */
int stepdllm_select_mask(const stepdllm_dims *dims, double sparsity,
                         const float *scores, void *ws, size_t ws_bytes,
                         int32_t *row_ptr, int32_t *col_idx, void *stream);

/* The uniform per-head budget, the baseline that the Step-dLLM abstract sets
 * its head-adaptive budget against: every head keeps the same number
 * k_h = ceil((1 - s) * nb^2) of its own nb^2 pooled scores (evaluated
 * exactly on the decimal s, as in stepdllm_keep_count), largest first, ties
 * by lowest index.
 * Host only.  Returns H * k_h (the length of col_idx), or a negative status. */
int64_t stepdllm_keep_count_per_head(const stepdllm_dims *dims, double sparsity);

/* stepdllm_build_mask with the uniform per-head budget: same arguments,
 * outputs and work order; col_idx holds H * k_h entries. */
int stepdllm_build_mask_per_head(const stepdllm_dims *dims, double sparsity,
                                 const uint16_t *q, const uint16_t *k,
                                 void *ws, size_t ws_bytes,
                                 int32_t *row_ptr, int32_t *col_idx,
                                 float *scores_out, void *stream);

/* stepdllm_select_mask with the uniform per-head budget. */
int stepdllm_select_mask_per_head(const stepdllm_dims *dims, double sparsity,
                                  const float *scores, void *ws, size_t ws_bytes,
                                  int32_t *row_ptr, int32_t *col_idx, void *stream);

/* Work order for a caller-built mask (row_ptr as above; col_idx holds nnz
 * list entries).  The pages give no work order (the Step-dLLM abstract only
 * names an IO-aware fused kernel); this is the library's own scheduling
 * reading, with no effect on any output.  The GPU's 8 dies (XCDs) each have
 * their own L2 and take workgroups round robin, so all rows of a head go to
 * one die.  A head weighs (B/32) * kept blocks + 4 * rows that
 * keep a block (its 32-key steps plus a fixed start-up and write-out per row);
 * heads are ranked by weight (descending, ties by id) and each goes to the
 * least-loaded die that holds fewer than min(H, ceil(H/8) + 2) heads (ties:
 * lowest die); a die's list is first the rows of its heads that keep a
 * block (heads in that order, each head's rows by list length descending,
 * ties by row id), then the rows that keep none (same head order, rows
 * ascending), at positions [x*cap, x*cap + cap) of the work order.  Workgroup
 * b of the sparse launch takes position b / 8 of die b % 8's list, so each die
 * starts its longest rows first, the hardware hands the next row to whichever
 * workgroup slot frees first, and the zero rows fill the slots that free up
 * at the end.  Beside the order, each position gets a record
 * (work_rec in the layout) of the row's list bounds and first two block ids,
 * so the plan describes this mask's contents, not only its row lengths: plan
 * again after any change to row_ptr or col_idx.  The plan also tags the
 * workspace with col_idx's address, nnz, H and nb and clears the check word
 * (work_meta in the layout), which stepdllm_sparse_attn uses to detect a
 * stale plan.  Memory safety on malformed masks: list positions outside
 * [0, nnz) are not read. */
int stepdllm_plan(const stepdllm_dims *dims, const int32_t *row_ptr,
                  const int32_t *col_idx, int64_t nnz,
                  void *ws, size_t ws_bytes, void *stream);

/* Block-sparse bidirectional attention (the fused kernel of the Step-dLLM
 * abstract): for each token t of query block i in head h,
 *   o_t = sum_u softmax_u(q_t . k_u / sqrt(d)) v_u
 * over the tokens u of the key blocks listed for row h*nb + i, from key head
 * h / (H/Hkv).  A row with no kept block outputs zeros.  The mask is the one
 * whose plan stepdllm_build_mask / select_mask / plan left in ws: the launch
 * takes each row's list bounds and first two block ids from the plan's
 * records and the rest of the list from col_idx, which must be the array the
 * plan was made from, unchanged since.
 * nnz is the length of col_idx (row_ptr[H*nb] for a well-formed mask, K for a
 * built one).  Stale plans are detected, not trusted: if col_idx, nnz or the
 * shape differ from the plan's tag, every row outputs zeros and bit 0 of the
 * check word (work_meta[7] in the workspace layout) is set; if a row's first
 * two list entries differ from its plan record (col_idx rewritten in place
 * after planning), that row outputs zeros and bit 1 is set.  The word is
 * cleared by every plan and read by the caller (device memory, after the
 * launch has completed); a rewrite that keeps every row's length and first
 * two entries is not detected.  Memory safety on malformed masks: list
 * positions at or past nnz are not read, and block ids outside [0, nb) are
 * clamped into range (the output of such a row is then unspecified).
 * ws is written (the check word) as well as read.
 * q [H,L,d], k/v [Hkv,L,d], o [H,L,d] bf16; bf16 MFMA with fp32 accumulation
 * and softmax; o rounded to nearest-even bf16. */
int stepdllm_sparse_attn(const stepdllm_dims *dims, const uint16_t *q,
                         const uint16_t *k, const uint16_t *v,
                         const int32_t *col_idx, int64_t nnz,
                         void *ws, size_t ws_bytes,
                         uint16_t *o, void *stream);

/* GQA variant of stepdllm_sparse_attn with group-shared K/V tiles: the heads
 * of a key head's group (h / (H/Hkv), the contiguous grouping of the
 * Step-dLLM layers' grouped-query attention) read the same K/V, so one
 * workgroup takes a pair of the group's query heads for one query block and
 * streams the union of their two kept-block lists through one K/V tile ring;
 * each head computes only on its own blocks, in the same order as
 * stepdllm_sparse_attn, so each head's output is identical to it.  A tile
 * kept by both heads is read once.  Needs no plan and no workspace: the lists
 * come straight from row_ptr [H*nb + 1] / col_idx [nnz] (list positions
 * outside [0, nnz) are not read, block ids outside [0, nb) are clamped).
 * Block size 64 only (EUNSUPPORTED otherwise).  A head with an empty list
 * outputs zeros. */
int stepdllm_sparse_attn_group(const stepdllm_dims *dims, const uint16_t *q,
                               const uint16_t *k, const uint16_t *v,
                               const int32_t *row_ptr, const int32_t *col_idx,
                               int64_t nnz, uint16_t *o, void *stream);

/* Dense bidirectional attention, every block kept: the same-GPU baseline that
 * stands for the dense FlashAttention of the Step-dLLM and SparseD abstracts. */
int stepdllm_dense_attn(const stepdllm_dims *dims, const uint16_t *q,
                        const uint16_t *k, const uint16_t *v, uint16_t *o,
                        void *stream);

/* Column-sparse variant ("PulseCol" abstract: column-sparse attention whose
 * pattern is found at an early step, reused, and refreshed at a few
 * intermediate steps).  The page leaves the column score open; the reading
 * here mirrors the block path's pooled scoring:
 *   c[h,u] = (1/nb) sum_i softmax_u(qb[h,i] . k_u / sqrt(d))
 * over all L key tokens u of key head h / (H/Hkv), qb[h,i] the mean of query
 * block i rounded to bf16; each head keeps the same number
 * k_c = ceil((1 - s) * L) of its columns (evaluated exactly on the decimal s,
 * as in stepdllm_keep_count), largest mass first, ties by lowest column, and
 * every query of the
 * head attends to exactly those key tokens.
 * Host only.  Returns k_c, or a negative status. */
int64_t stepdllm_keep_count_columns(const stepdllm_dims *dims, double sparsity);

/* Column mask of one step: q [H,L,d], k [Hkv,L,d] bf16 -> cols int32
 * [H, k_c] (out; head h's kept columns, ascending).  scores_out (nullable):
 * fp32 [H, L] receives c (otherwise c stays in the workspace).  Masses on
 * bf16 MFMA with fp32 accumulation, exact per-pooled-query max and normaliser
 * (two passes over the keys), deterministic.  Uses the workspace. */
int stepdllm_build_col_mask(const stepdllm_dims *dims, double sparsity,
                            const uint16_t *q, const uint16_t *k,
                            void *ws, size_t ws_bytes, int32_t *cols,
                            float *scores_out, void *stream);

/* The selection half on caller-given masses scores [H, L] fp32 (finite):
 * per head the k_c largest (ties by lowest column), ascending in cols. */
int stepdllm_select_col_mask(const stepdllm_dims *dims, double sparsity,
                             const float *scores, void *ws, size_t ws_bytes,
                             int32_t *cols, void *stream);

/* Column-sparse attention: every token t of head h attends to the key tokens
 * cols[h*k_c .. h*k_c + k_c) of key head h / (H/Hkv),
 *   o_t = sum_a softmax_a(q_t . k_{cols[a]} / sqrt(d)) v_{cols[a]},
 * k_c in [0, L] (0 gives zeros).  Entries are expected in [0, L); any other
 * entry reads zero K and V rows (no fault, output unspecified).  Same
 * arithmetic as stepdllm_sparse_attn; K/V rows are gathered per entry. */
int stepdllm_col_attn(const stepdllm_dims *dims, const uint16_t *q,
                      const uint16_t *k, const uint16_t *v,
                      const int32_t *cols, int64_t k_c, uint16_t *o,
                      void *stream);

/* Mask quality (a diagnostic, off the per-step path).  The BA-Att abstract
 * compares block selection in the pooled, pre-downsampled space with the
 * block map of the exact attention; Step-dLLM reuses one mask across a
 * refresh interval.  stepdllm_block_mass writes the true block attention mass
 *   mass[h,i,j] = (1/B) sum_{t in q-block i} sum_{u in k-block j}
 *                 softmax_u(q_t . k_u / sqrt(d))       (all L keys, key head
 *                                                       h / (H/Hkv))
 * fp32 [H, nb, nb] (caller-owned device memory; each row sums to 1 up to fp32
 * rounding).  q [H,L,d], k [Hkv,L,d] bf16.  Scores on bf16 MFMA with fp32
 * accumulation; exact per-query max and normaliser (two passes over the keys);
 * deterministic. */
int stepdllm_block_mass(const stepdllm_dims *dims, const uint16_t *q,
                        const uint16_t *k, float *mass, void *stream);

/* Recall of a block mask against a block mass map: recall[r] (fp32, [H*nb])
 * is the sum of mass[r, j] over the kept blocks j of row r (1 when the kept
 * blocks hold all of the row's attention, 0 for an empty row).  row_ptr /
 * col_idx as for stepdllm_sparse_attn; list positions at or past nnz are not
 * read and block ids outside [0, nb) add nothing. */
int stepdllm_mask_recall(const stepdllm_dims *dims, const float *mass,
                         const int32_t *row_ptr, const int32_t *col_idx,
                         int64_t nnz, float *recall, void *stream);

/* Recall of a column mask (the column-sparse variant's counterpart of
 * stepdllm_mask_recall): recall[r] (fp32, [H*nb]) for row r = h*nb + i is
 *   (1/B) sum_{t in q-block i} sum_{a < k_c} softmax_u(q_t . k_u / sqrt(d))
 *                                            at u = cols[h*k_c + a]
 * (all L keys of key head h / (H/Hkv) in the softmax): the share of the
 * row's exact attention on the kept columns.  Entries are expected distinct
 * and in [0, L); others are clamped into range.  Exact per-token max and
 * normaliser over all keys (bf16 MFMA, fp32), then the kept columns only;
 * deterministic. */
int stepdllm_col_recall(const stepdllm_dims *dims, const uint16_t *q,
                        const uint16_t *k, const int32_t *cols, int64_t k_c,
                        float *recall, void *stream);

/* Step driver: a small host object owned by the library; device buffers
 * (workspace, row_ptr [H*nb+1], col_idx [K]; column mode: col_idx [H*k_c]
 * and no row_ptr) stay owned by the caller and
 * must outlive the driver.  stepdllm_step runs what the schedule asks for at
 * step `step` (dense / anchor: build mask + sparse / reuse: sparse) and
 * returns STEPDLLM_ESTATE for a reuse step before any anchor.  A driver is
 * not thread-safe; use one driver per stream. */
typedef struct stepdllm_driver stepdllm_driver;

int stepdllm_driver_create(stepdllm_driver **out, const stepdllm_dims *dims,
                           const stepdllm_schedule *schedule, void *ws,
                           size_t ws_bytes, int32_t *row_ptr, int32_t *col_idx);
/* Kind of step `step`: 0 dense, 1 anchor, 2 reuse (negative on error). */
int stepdllm_driver_step_kind(const stepdllm_driver *drv, int32_t step);
int stepdllm_step(stepdllm_driver *drv, int32_t step, const uint16_t *q,
                  const uint16_t *k, const uint16_t *v, uint16_t *o,
                  void *stream);
int stepdllm_driver_destroy(stepdllm_driver *drv);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * denoising step as stepdllm_step with a driver made from (dims, schedule,
 * row_ptr, col_idx) -- dense / anchor (mask build into row_ptr, col_idx, then
 * sparse attention) / reuse (sparse attention on the stored mask) -- but with
 * no driver object and no workspace argument: the workspace is a static
 * device array inside the library of STEPDLLM_NOALLOC_SCRATCH_BYTES (80 MiB,
 * enough for every shape up to L = 65536, H = 32, 128-token blocks), one copy
 * per GPU, looked up on the first call on each device and held until the
 * process ends.  Shapes whose workspace (stepdllm_workspace_bytes) is larger
 * are rejected with STEPDLLM_EWORKSPACE.  The call allocates nothing: no
 * hipMalloc, hipFree or host allocation.  The stream must belong to the
 * current device.  Every call on one GPU shares that GPU's array, which keeps
 * the last call's contents: a reuse step runs on the plan the last anchor
 * call on this GPU left there (if that anchor was for another col_idx or
 * shape, the stale-plan check of stepdllm_sparse_attn makes the output
 * zeros); calls that overlap on one GPU (other streams, other threads) race
 * on the array and must be serialised by the caller.  The output of each
 * step is identical to stepdllm_step's.  Nothing in the array needs to start
 * at zero: every launch writes what it later reads. */
#define STEPDLLM_NOALLOC_SCRATCH_BYTES (80ll << 20)
int stepdllm_step_noalloc(const stepdllm_dims *dims, const stepdllm_schedule *schedule,
                          int32_t step, const uint16_t *q, const uint16_t *k,
                          const uint16_t *v, int32_t *row_ptr, int32_t *col_idx,
                          uint16_t *o, void *stream);

/* Static description of a status code. */
const char *stepdllm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* STEPDLLM_H */
