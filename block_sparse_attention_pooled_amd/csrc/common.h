// Internal helpers shared by the library's HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace sd {

constexpr int kWave = 64;            // CDNA wavefront width
constexpr int kMaxBlocks = 1024;     // largest nb = L / B supported
constexpr int kMaxHeads = 1024;      // largest number of query heads supported
constexpr int kDies = 8;             // XCDs: workgroup b of a launch runs on die b % 8
constexpr int kRadixBins = 2048;     // 11-bit digits (11 + 11 + 10 = 32 bits)
constexpr int kSelectWords = 32;     // select state words in the workspace
constexpr int kHeadSelWords = 8;     // per-head select state words (uniform budget)
constexpr int kCompactRows = 16;     // rows per workgroup of the list compaction

// Select state words.
enum SelectWord {
    SEL_CUT = 0,      // orderable key of the K-th largest score
    SEL_ABOVE = 1,    // number of scores strictly above the cut
    SEL_TIES = 2,     // ties at the cut to keep (lowest flat indices first)
    SEL_K = 3,        // K
    SEL_PREFIX = 4,   // running prefix during the radix passes
    SEL_REMAIN = 5,   // K minus the count already above the prefix bucket
    SEL_PASS = 8,     // 8..16: state entering digit pass 0..2 (prefix, count
                      // above the prefix, rank wanted inside it), 3 words each
};

// Words of the plan's metadata (work_meta in the workspace).
enum MetaWord {
    kMetaCap = 0,        // work-order positions per die
    kMetaNonEmpty = 1,   // rows that keep a block
    kMetaListLo = 2,     // tag: address of the col_idx array planned (low, high word),
    kMetaListHi = 3,     //      its length nnz, the head count H and block count nb
    kMetaNnz = 4,
    kMetaHeads = 5,
    kMetaNb = 6,
    kMetaCheck = 7,      // cleared by each plan; sparse launches OR in the bits below
};
constexpr int kCheckStalePlan = 1;     // launch on another col_idx, nnz or shape than planned
constexpr int kCheckListChanged = 2;   // a row's first list entries differ from its record

// Shapes after validation, with derived sizes.
struct Dims {
    int H, Hkv, L, d, B, nb, G;
    int64_t rows() const { return (int64_t)H * nb; }
    // Heads a die may take in the work order: ceil(H / kDies) plus two of
    // slack for balancing, at most H.
    int die_heads() const { return std::min(H, (H + kDies - 1) / kDies + 2); }
    // Work-order positions per die (rows of die_heads() heads).
    int64_t die_cap() const { return (int64_t)die_heads() * nb; }
    int64_t n_scores() const { return (int64_t)H * nb * nb; }
    // Key splits of the column-mass statistics pass (1024 keys each).
    int64_t col_splits() const { return ((int64_t)L + 1023) / 1024; }
};

// Workspace carve-up (byte offsets, 256-byte aligned).
struct WsLayout {
    int64_t qb, kb, p, hist, sel, gt, eq, tie_base, work, work_meta, hsel, col_scores, col_stats,
        col_part, col_q16, plan_head_base, work_rec, row_agg, row_rec, head_counts, total;
};

inline int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

inline WsLayout ws_layout(const Dims &D) {
    WsLayout w;
    int64_t off = 0;
    auto take = [&](int64_t bytes) { int64_t o = off; off = align256(off + bytes); return o; };
    w.qb = take((int64_t)D.H * D.nb * D.d * 4);
    w.kb = take((int64_t)D.Hkv * D.nb * D.d * 4);
    w.p = take(D.n_scores() * 4);
    w.hist = take(3 * kRadixBins * 4);
    w.sel = take(kSelectWords * 4);
    w.gt = take(D.rows() * 4);
    w.eq = take(D.rows() * 4);
    w.tie_base = take(D.rows() * 4);
    w.work = take(kDies * D.die_cap() * 4);
    w.work_meta = take(16 * 4);
    w.hsel = take((int64_t)D.H * kHeadSelWords * 4);
    w.col_scores = take((int64_t)D.H * D.L * 4);   // column masses (column-sparse variant)
    w.col_stats = take(D.rows() * 8);              // per pooled query: max, 1 / normaliser
    w.col_part = take(D.rows() * D.col_splits() * 8);   // per key split: max, normaliser
    w.col_q16 = take((int64_t)D.H * ((D.nb + 31) / 32) * 32 * D.d * 2);   // bf16 pooled Q
    w.plan_head_base = take((int64_t)D.H * 8);     // each head's first non-empty / empty position
    w.work_rec = take(kDies * D.die_cap() * 16);   // int4 record per work position
    // per compaction workgroup: above-cut and at-cut counts of its rows
    w.row_agg = take(2 * ((D.rows() + kCompactRows - 1) / kCompactRows) * 4);
    w.row_rec = take(D.rows() * 16);               // each row's plan record, from the list launch
    w.head_counts = take((int64_t)D.H * 8);        // each head's kept blocks, non-empty rows
    w.total = off;
    return w;
}

// Monotone map from fp32 to uint32: a < b (as floats, -0 < +0) iff key(a) < key(b).
__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Mask-building launches (mask_kernels.hip).
// With sel_init_K >= 0 the launch also prepares the global select state in ws
// for a budget of sel_init_K (zero histograms).
hipError_t launch_pool(const Dims &D, const uint16_t *q, const uint16_t *k, float *qb, float *kb,
                       char *ws, const WsLayout &w, int64_t sel_init_K, hipStream_t s);
// With first_digit set the launch also counts the scores into the first digit
// histogram of the global select (prepared by launch_pool); launch_select then
// runs with state_ready and starts at the second digit.
hipError_t launch_scores(const Dims &D, const float *qb, const float *kb, float *p, float *copy,
                         char *ws, const WsLayout &w, bool first_digit, hipStream_t s);
// With plan_inputs set, the list launch also writes what launch_plan with
// prepared set reads: each row's plan record (w.row_rec) and each head's kept
// blocks and non-empty rows (w.head_counts).
hipError_t launch_select(const Dims &D, int64_t K, const float *p, char *ws, const WsLayout &w,
                         int32_t *row_ptr, int32_t *col_idx, bool state_ready, bool plan_inputs,
                         hipStream_t s);
// Uniform per-head budget: head h keeps its k_h largest scores.
hipError_t launch_select_per_head(const Dims &D, int64_t k_h, const float *p, char *ws,
                                  const WsLayout &w, int32_t *row_ptr, int32_t *col_idx,
                                  hipStream_t s);
// Work order of the mask row_ptr / col_idx (nnz list entries): the row ids
// into w.work and one record per position into w.work_rec (row, list begin,
// list end, first two block ids in 16 bits each; row -1 for padding).
// prepared: the row records and head counts come from the list launch
// (launch_select with plan_inputs), not from row_ptr and col_idx.
hipError_t launch_plan(const Dims &D, const int32_t *row_ptr, const int32_t *col_idx,
                       int64_t nnz, char *ws, const WsLayout &w, bool prepared, hipStream_t s);

// Column-sparse variant.  Block means of Q only (mask_kernels.hip).
hipError_t launch_pool_q(const Dims &D, const uint16_t *q, float *qb, hipStream_t s);
// Per head, the k_c largest of the head's L column masses c, listed ascending
// in cols [H, k_c] (mask_kernels.hip).
hipError_t launch_col_select(const Dims &D, int64_t k_c, const float *c, char *ws,
                             const WsLayout &w, int32_t *cols, hipStream_t s);
// Column masses c [H, L] of the pooled queries qb (col_kernels.hip).
hipError_t launch_col_scores(const Dims &D, const float *qb, const uint16_t *k, char *ws,
                             const WsLayout &w, float *c, hipStream_t s);

// Mask quality launches (quality_kernels.hip).
hipError_t launch_block_mass(const Dims &D, const uint16_t *q, const uint16_t *k, float *mass,
                             hipStream_t s);
// Recall of a column mask per row: mean over the query block of the full
// softmax probability on cols[h*k_c .. +k_c).
hipError_t launch_col_recall(const Dims &D, const uint16_t *q, const uint16_t *k,
                             const int32_t *cols, int64_t k_c, float *recall, hipStream_t s);
hipError_t launch_mask_recall(const Dims &D, const float *mass, const int32_t *row_ptr,
                              const int32_t *col_idx, int64_t nnz, float *recall,
                              hipStream_t s);

// Attention launches (attn_kernels.hip).
// Rows, list bounds and first block ids from the work records of the plan.
// meta: the plan's metadata words; the launch checks the tag and ORs the
// check bits into meta[kMetaCheck].
hipError_t launch_sparse_attn(const Dims &D, const uint16_t *q, const uint16_t *k,
                              const uint16_t *v, const int32_t *col_idx, const int4 *recs,
                              int32_t *meta, int64_t n_idx, uint16_t *o, hipStream_t s);
hipError_t launch_dense_attn(const Dims &D, const uint16_t *q, const uint16_t *k,
                             const uint16_t *v, uint16_t *o, hipStream_t s);
// GQA variant: one workgroup per (KV group, pair of its query heads, query
// block) streams the union of the pair's lists through one K/V ring; each
// head's output equals launch_sparse_attn's.  Block size 64 only.
hipError_t launch_group_attn(const Dims &D, const uint16_t *q, const uint16_t *k,
                             const uint16_t *v, const int32_t *row_ptr, const int32_t *col_idx,
                             int64_t nnz, uint16_t *o, hipStream_t s);
// Every query of head h over the key tokens cols[h*k_c .. h*k_c + k_c).
hipError_t launch_col_attn(const Dims &D, const uint16_t *q, const uint16_t *k,
                           const uint16_t *v, const int32_t *cols, int64_t k_c, uint16_t *o,
                           hipStream_t s);

}  // namespace sd
