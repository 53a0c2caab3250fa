// Anchor-step mask construction on gfx950: block mean-pooling, pooled scores
// with a per-row softmax, the global top-K (radix select over all heads), the
// per-row kept-block lists, and the attention work order.
//
// Method: "Step-dLLM: Adaptive Step-aware Sparse Attention for Efficient
// Diffusion LLM Inference", abstract (block-sparse mask refreshed at anchor
// steps under one head-adaptive global budget); block scores in a pooled,
// pre-downsampled space as in the BA-Att abstract.  The pooled statistic is
// the block mean, the score is Qb.Kb^T/sqrt(d) softmaxed over key blocks, and
// the budget keeps the K largest scores of all heads together, ties to the
// lowest flat index.
//
// These kernels are HBM/latency bound (they run once per anchor and touch
// each byte of Q, K and the score matrix a few times); none is a contraction
// worth MFMA.  Every reduction whose order fixes a result bit is written in a
// fixed order, and atomics are used only for integer histogram counts, so the
// mask is deterministic.
#include "common.h"

namespace sd {

namespace {

__device__ __forceinline__ uint64_t lanemask_lt() {
    return (1ull << (threadIdx.x & 63)) - 1ull;
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Exclusive scan of one int64 per thread across a 1024-thread block.
__device__ int64_t block_exclusive_scan_1024(int64_t x, int64_t *total) {
    __shared__ int64_t wsum[16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int64_t inc = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int64_t y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int64_t before = 0, all = 0;
    for (int w = 0; w < 16; ++w) {
        if (w < wave) before += wsum[w];
        all += wsum[w];
    }
    __syncthreads();
    *total = all;
    return before + inc - x;
}

// ------------------------------------------------------------------- pool --
// One thread owns 4 consecutive columns of one (head, block) and adds the B
// rows in ascending token order in fp32, then scales by 1/B (a power of two,
// exact).  A wave covers 4 (d=64) or 2 (d=128) blocks with 128/256-byte
// contiguous segments per load, and a thread keeps a whole 64-row batch of
// loads in flight.
template <int D>
__global__ __launch_bounds__(256) void k_pool(const uint16_t *__restrict__ q,
                                              const uint16_t *__restrict__ k,
                                              float *__restrict__ qb, float *__restrict__ kb,
                                              int L, int B, int64_t nq_items, int64_t nk_items) {
    constexpr int CG = D / 4;   // 4-column groups per row
    int64_t it = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const uint16_t *src = q;
    float *dst = qb;
    if (it >= nq_items) {
        it -= nq_items;
        if (it >= nk_items) return;
        src = k;
        dst = kb;
    }
    const int cg = (int)(it % CG);
    const int64_t hb = it / CG;              // head * nb + block
    const int nb = L / B;
    const int64_t head = hb / nb;
    const int blk = (int)(hb % nb);
    const uint2 *p = reinterpret_cast<const uint2 *>(src + (head * L + (int64_t)blk * B) * D) + cg;
    float acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = 0.0f;
    // Batches of 64 rows: all of a batch's loads are in flight before the
    // first add; the adds still run in ascending token order.
    constexpr int kBatch = 64;   // B is 64 or 128
    for (int t0 = 0; t0 < B; t0 += kBatch) {
        uint2 u[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) u[j] = p[(int64_t)(t0 + j) * CG];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const uint32_t w[2] = {u[j].x, u[j].y};
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                acc[2 * c] = acc[2 * c] + bf16_bits_to_float(w[c] & 0xFFFFu);
                acc[2 * c + 1] = acc[2 * c + 1] + bf16_bits_to_float(w[c] >> 16);
            }
        }
    }
    const float inv_b = 1.0f / (float)B;
    *reinterpret_cast<float4 *>(dst + hb * D + cg * 4) =
        make_float4(acc[0] * inv_b, acc[1] * inv_b, acc[2] * inv_b, acc[3] * inv_b);
}

// Select state before the first digit pass: all three histograms zero, the
// rank wanted = K.
__device__ void select_init(uint32_t *__restrict__ hist, uint32_t *__restrict__ sel, int64_t K,
                            int tid, int nthreads) {
    for (int b = tid; b < 3 * kRadixBins; b += nthreads) hist[b] = 0;
    if (tid == 0) {
        sel[SEL_PREFIX] = 0;
        sel[SEL_ABOVE] = 0;
        sel[SEL_REMAIN] = (uint32_t)K;
        sel[SEL_K] = (uint32_t)K;
        sel[SEL_CUT] = 0xFFFFFFFFu;   // K == 0: nothing is above the cut ...
        sel[SEL_TIES] = 0;            // ... and no tie is kept
        sel[SEL_PASS + 0] = 0;        // state entering digit pass 0: prefix,
        sel[SEL_PASS + 1] = 0;        // count above it,
        sel[SEL_PASS + 2] = (uint32_t)K;   // rank wanted inside it
    }
}

// ---------------------------------------------------------- score + softmax --
// A workgroup of 512 threads owns 16 query-block rows of one head.  Key-block
// means stream through LDS 64 rows at a time (read once per 16 rows), each
// thread's loads in flight together.  Thread (r, jj) forms two dot products
// at once, row r against tile columns jj and jj + 32, each in ascending c with
// separately rounded multiply and add.  The scaled scores of the 16 rows wait
// in LDS (up to kMaxBlocks per row: 105 KB in all, within gfx950's 160 KB per
// workgroup); then each row is softmaxed by its 32 lanes and written once.
// With init_sel set, block 0 also prepares the select state of a global
// budget of init_K (the job of k_select_init).
constexpr int kScoreRows = 16;
constexpr int kScoreCols = 64;
constexpr int kScoreThreads = kScoreRows * 32;

template <int D>
__global__ __launch_bounds__(kScoreThreads) void k_scores(const float *__restrict__ qb,
                                                          const float *__restrict__ kb,
                                                          float *__restrict__ p,
                                                          float *__restrict__ copy, int nb, int G,
                                                          float sigma,
                                                          uint32_t *__restrict__ init_hist,
                                                          uint32_t *__restrict__ init_sel,
                                                          int64_t init_K) {
#pragma clang fp contract(off)
    __shared__ float sq[kScoreRows][D];
    __shared__ float sk[kScoreCols][D + 1];
    __shared__ float srow[kScoreRows][kMaxBlocks];
    const int tid = threadIdx.x;
    // The global select that follows reads a fresh state: block 0 sets it.
    if (init_sel && blockIdx.x == 0) select_init(init_hist, init_sel, init_K, tid, kScoreThreads);
    const int tiles = (nb + kScoreRows - 1) / kScoreRows;
    // Workgroups go round-robin to the 8 dies, each with its own L2: renumber
    // so that consecutive tiles (one head's rows, sharing its key means) run
    // on one die, and each die fetches a head's key means once.
    int bid = blockIdx.x;
    if (gridDim.x % 8 == 0) bid = (bid % 8) * (gridDim.x / 8) + bid / 8;
    const int h = bid / tiles;
    const int i0 = (bid % tiles) * kScoreRows;
    const int g = h / G;
    constexpr int Q4 = (kScoreRows * D / 4 + kScoreThreads - 1) / kScoreThreads;
    constexpr int K4 = kScoreCols * D / 4 / kScoreThreads;
    {
        float4 v[Q4];
#pragma unroll
        for (int t = 0; t < Q4; ++t) {
            const int x = tid + kScoreThreads * t, r = x / (D / 4), c4 = x % (D / 4);
            v[t] = (r < kScoreRows && i0 + r < nb)
                       ? reinterpret_cast<const float4 *>(qb + ((int64_t)h * nb + i0 + r) * D)[c4]
                       : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
#pragma unroll
        for (int t = 0; t < Q4; ++t) {
            const int x = tid + kScoreThreads * t, r = x / (D / 4), c4 = x % (D / 4);
            if (r < kScoreRows) *reinterpret_cast<float4 *>(&sq[r][4 * c4]) = v[t];
        }
    }
    const int r = tid / 32, jj = tid % 32;
    for (int j0 = 0; j0 < nb; j0 += kScoreCols) {
        float4 v[K4];
#pragma unroll
        for (int t = 0; t < K4; ++t) {
            const int x = tid + kScoreThreads * t, rr = x / (D / 4), c4 = x % (D / 4);
            v[t] = (j0 + rr < nb) ? reinterpret_cast<const float4 *>(
                                        kb + ((int64_t)g * nb + j0 + rr) * D)[c4]
                                  : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < K4; ++t) {
            const int x = tid + kScoreThreads * t, rr = x / (D / 4), c4 = x % (D / 4);
            sk[rr][4 * c4] = v[t].x;
            sk[rr][4 * c4 + 1] = v[t].y;
            sk[rr][4 * c4 + 2] = v[t].z;
            sk[rr][4 * c4 + 3] = v[t].w;
        }
        __syncthreads();
        float d0 = 0.0f, d1 = 0.0f;
        for (int c = 0; c < D; ++c) {
            const float a = sq[r][c];
            float p0 = a * sk[jj][c], p1 = a * sk[jj + 32][c];
            d0 = d0 + p0;
            d1 = d1 + p1;
        }
        const int j = j0 + jj;
        if (j < nb) srow[r][j] = d0 * sigma;
        if (j + 32 < nb) srow[r][j + 32] = d1 * sigma;
    }
    __syncthreads();
    if (i0 + r >= nb) return;
    float m = -INFINITY;
    for (int j = jj; j < nb; j += 32) m = fmaxf(m, srow[r][j]);
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 32));
    float sum = 0.0f;
    for (int j = jj; j < nb; j += 32) {
        float e = expf(srow[r][j] - m);
        srow[r][j] = e;
        sum = sum + e;
    }
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) sum = sum + __shfl_xor(sum, o, 32);
    const int64_t base = ((int64_t)h * nb + i0 + r) * nb;
    for (int j = jj; j < nb; j += 32) {
        float v = srow[r][j] / sum;
        p[base + j] = v;
        if (copy) copy[base + j] = v;
    }
}

// ------------------------------------------------------------ radix select --
// The K-th largest order key among all H*nb*nb scores, in three digit passes
// (bits 31..21, 20..10, 9..0).  The state words hold the running prefix and the
// rank still wanted inside the prefix bucket; at the end the cut key, the
// count strictly above it and the number of ties at the cut to keep.
__global__ __launch_bounds__(1024) void k_select_init(uint32_t *__restrict__ hist,
                                                      uint32_t *__restrict__ sel, int64_t K) {
    select_init(hist, sel, K, threadIdx.x, 1024);
}

__device__ __forceinline__ void digit_of_pass(int pass, int &shift, uint32_t &hi_mask,
                                              uint32_t &dmask) {
    shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    hi_mask = pass == 0 ? 0u : (pass == 1 ? 0xFFE00000u : 0xFFFFFC00u);
    dmask = pass == 2 ? 0x3FFu : 0x7FFu;
}

// One step of the select, by a 1024-thread block: given the state entering
// digit pass `pass` (prefix, count above it, rank wanted inside it) and that
// pass's histogram, take the bins in descending order (thread t owns ranks 2t
// and 2t + 1) and return, to every thread, the state after the pass.
struct RadixState {
    uint32_t prefix;
    uint32_t above;
    uint32_t remain;
};

__device__ RadixState radix_step(const uint32_t *__restrict__ hp, int pass, RadixState in) {
    __shared__ RadixState out;
    int shift;
    uint32_t hi_mask, dmask;
    digit_of_pass(pass, shift, hi_mask, dmask);
    const int nbins = (int)dmask + 1;
    const int64_t remain = in.remain;
    const int r0 = 2 * threadIdx.x, r1 = r0 + 1;
    const int b0 = nbins - 1 - r0, b1 = nbins - 1 - r1;
    const int64_t c0 = r0 < nbins ? hp[b0] : 0;
    const int64_t c1 = r1 < nbins ? hp[b1] : 0;
    int64_t total;
    const int64_t before = block_exclusive_scan_1024(c0 + c1, &total);
    int win_bin = -1;
    int64_t above = 0;
    if (r0 < nbins && before < remain && remain <= before + c0) {
        win_bin = b0;
        above = before;
    } else if (r1 < nbins && before + c0 < remain && remain <= before + c0 + c1) {
        win_bin = b1;
        above = before + c0;
    }
    if (win_bin >= 0) {
        out.prefix = in.prefix | ((uint32_t)win_bin << shift);
        out.above = in.above + (uint32_t)above;
        out.remain = (uint32_t)(remain - above);
    }
    __syncthreads();
    return out;
}

__device__ __forceinline__ RadixState load_state(const uint32_t *__restrict__ sel, int pass) {
    return RadixState{sel[SEL_PASS + 3 * pass], sel[SEL_PASS + 3 * pass + 1],
                      sel[SEL_PASS + 3 * pass + 2]};
}

// Digit pass `pass` over the scores whose key matches the prefix fixed so
// far.  For pass > 0 every workgroup first redoes the previous pass's step
// from its histogram (cheaper than a launch of its own) and workgroup 0
// records the state it enters with.  A workgroup histograms its share in LDS:
// the lanes of a wave that fall in one bin are counted with one atomic, for
// up to two bins per element slot (the pooled scores crowd into a few bins of
// the first digit), the rest one by one; its nonzero bins are then added to
// the pass's global histogram.
constexpr int kRadixThreads = 1024;

__global__ __launch_bounds__(kRadixThreads) void k_radix_pass(const float *__restrict__ p,
                                                              int64_t n,
                                                              uint32_t *__restrict__ sel,
                                                              uint32_t *__restrict__ hist,
                                                              int pass) {
    __shared__ uint32_t h[kRadixBins];
    const int tid = threadIdx.x, lane = tid & 63;
    for (int b = tid; b < kRadixBins; b += kRadixThreads) h[b] = 0;
    RadixState st = load_state(sel, 0);
    if (pass > 0) {
        st = radix_step(hist + (pass - 1) * kRadixBins, pass - 1, load_state(sel, pass - 1));
        if (blockIdx.x == 0 && tid == 0) {
            sel[SEL_PASS + 3 * pass] = st.prefix;
            sel[SEL_PASS + 3 * pass + 1] = st.above;
            sel[SEL_PASS + 3 * pass + 2] = st.remain;
        }
    }
    __syncthreads();
    int shift;
    uint32_t hi_mask, dmask;
    digit_of_pass(pass, shift, hi_mask, dmask);
    const uint32_t prefix = st.prefix;
    auto count = [&](float x, bool in_range) {
        const uint32_t key = order_key(x);
        const bool valid = in_range && (key & hi_mask) == prefix;
        const uint32_t bin = (key >> shift) & dmask;
        uint64_t todo = __ballot(valid);
        for (int round = 0; round < 2 && todo; ++round) {
            const int leader = __builtin_ctzll(todo);
            const uint32_t lb = __builtin_amdgcn_readlane(bin, leader);
            const uint64_t same = __ballot(valid && bin == lb) & todo;
            if (lane == leader) atomicAdd(&h[lb], (uint32_t)__popcll(same));
            todo &= ~same;
        }
        if ((todo >> lane) & 1) atomicAdd(&h[bin], 1u);
    };
    const int64_t stride = (int64_t)gridDim.x * kRadixThreads;
    const int64_t n4 = n >> 2;
    const float4 *p4 = reinterpret_cast<const float4 *>(p);
    for (int64_t base = (int64_t)blockIdx.x * kRadixThreads; base < n4; base += stride) {
        const int64_t x = base + tid;
        const bool in = x < n4;
        const float4 v = in ? p4[x] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        count(v.x, in);
        count(v.y, in);
        count(v.z, in);
        count(v.w, in);
    }
    for (int64_t base = (n4 << 2) + (int64_t)blockIdx.x * kRadixThreads; base < n; base += stride) {
        const int64_t x = base + tid;
        count(x < n ? p[x] : 0.0f, x < n);
    }
    __syncthreads();
    uint32_t *hp = hist + pass * kRadixBins;
    for (int b = tid; b < kRadixBins; b += kRadixThreads)
        if (h[b]) atomicAdd(&hp[b], h[b]);
}

// The last step, one block: the state after digit pass 2 fixes the cut (the
// K-th largest key), the count strictly above it and the ties to keep.
__global__ __launch_bounds__(kRadixThreads) void k_radix_final(const uint32_t *__restrict__ hist,
                                                               uint32_t *__restrict__ sel) {
    const RadixState st = radix_step(hist + 2 * kRadixBins, 2, load_state(sel, 2));
    if (threadIdx.x == 0) {
        sel[SEL_PREFIX] = st.prefix;
        sel[SEL_ABOVE] = st.above;
        sel[SEL_REMAIN] = st.remain;
        sel[SEL_CUT] = st.prefix;
        sel[SEL_TIES] = st.remain;
    }
}

// --------------------------------------------------------------- compaction --
// Per row (one wave; 16 rows per workgroup): how many scores are above the
// cut and how many equal it.  Rows come in groups of group_rows that share one
// select state (all rows for the global budget, one head's rows for the
// per-head one), kHeadSelWords apart.  With agg set, workgroup b also writes
// its rows' sums of both counts to agg[2b], agg[2b + 1].

__global__ __launch_bounds__(1024) void k_row_count(const float *__restrict__ p, int nb,
                                                    int64_t rows, int64_t group_rows,
                                                    const uint32_t *__restrict__ sel,
                                                    int32_t *__restrict__ gt,
                                                    int32_t *__restrict__ eq,
                                                    int32_t *__restrict__ agg) {
    __shared__ int32_t sg[kCompactRows], se[kCompactRows];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * kCompactRows + wave;
    int cg = 0, ce = 0;
    if (r < rows) {
        const uint32_t cut = sel[(r / group_rows) * kHeadSelWords + SEL_CUT];
        for (int j = lane; j < nb; j += 64) {
            uint32_t key = order_key(p[r * nb + j]);
            cg += key > cut;
            ce += key == cut;
        }
        cg = wave_sum(cg);
        ce = wave_sum(ce);
        if (lane == 0) {
            gt[r] = cg;
            eq[r] = ce;
        }
    }
    if (!agg) return;
    if (lane == 0) {
        sg[wave] = cg;
        se[wave] = ce;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t a = 0, b = 0;
        for (int w = 0; w < kCompactRows; ++w) {
            a += sg[w];
            b += se[w];
        }
        agg[2 * blockIdx.x] = a;
        agg[2 * blockIdx.x + 1] = b;
    }
}

// Global budget, one wave per row (16 rows per workgroup): row_ptr and the
// row's kept blocks in ascending order.  The cut ties are kept in flat order,
// so over any run of rows that starts at row 0 the ties kept are
// min(ties, ties met): the list start of workgroup b's first row is (above-cut
// count of the rows before) + min(ties, cut ties before), both from the
// per-workgroup sums of k_row_count.  Inside the workgroup the rows add up in
// LDS.  K bounds col_idx.
__global__ __launch_bounds__(1024) void k_row_emit(const float *__restrict__ p, int nb,
                                                   int64_t rows, int64_t K,
                                                   const uint32_t *__restrict__ sel,
                                                   const int32_t *__restrict__ gt,
                                                   const int32_t *__restrict__ eq,
                                                   const int32_t *__restrict__ agg,
                                                   int32_t *__restrict__ row_ptr,
                                                   int32_t *__restrict__ col_idx) {
    __shared__ int64_t row_eq[kCompactRows], row_kept[kCompactRows];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t r = (int64_t)blockIdx.x * kCompactRows + wave;
    int64_t g_loc = 0, e_loc = 0;
    for (int64_t b = tid; b < blockIdx.x; b += 1024) {
        g_loc += agg[2 * b];
        e_loc += agg[2 * b + 1];
    }
    int64_t g_before, e_before;
    block_exclusive_scan_1024(g_loc, &g_before);
    block_exclusive_scan_1024(e_loc, &e_before);
    const uint32_t cut = sel[SEL_CUT];
    const int64_t ties = sel[SEL_TIES];
    const int64_t my_gt = r < rows ? gt[r] : 0, my_eq = r < rows ? eq[r] : 0;
    if (lane == 0) row_eq[wave] = my_eq;
    __syncthreads();
    int64_t tie = e_before;
    for (int w = 0; w < wave; ++w) tie += row_eq[w];
    int64_t take = ties - tie;
    take = take < 0 ? 0 : (take > my_eq ? my_eq : take);
    if (lane == 0) row_kept[wave] = my_gt + take;
    __syncthreads();
    if (r >= rows) return;
    int64_t out = g_before + (ties < e_before ? ties : e_before);
    for (int w = 0; w < wave; ++w) out += row_kept[w];
    if (lane == 0) {
        row_ptr[r] = (int32_t)out;
        if (r == rows - 1) row_ptr[rows] = (int32_t)(out + my_gt + take);
    }
    const uint64_t lt = lanemask_lt();
    for (int j0 = 0; j0 < nb; j0 += 64) {
        const int j = j0 + lane;
        const bool valid = j < nb;
        const uint32_t key = valid ? order_key(p[r * nb + j]) : 0u;
        const bool is_eq = valid && key == cut;
        const uint64_t eqm = __ballot(is_eq);
        const int64_t my_tie = tie + __popcll(eqm & lt);
        const bool keep = valid && (key > cut || (is_eq && my_tie < ties));
        const uint64_t km = __ballot(keep);
        const int64_t slot = out + __popcll(km & lt);
        if (keep && slot < K) col_idx[slot] = j;   // K bounds the list; never exceeded
        out += __popcll(km);
        tie += __popcll(eqm);
    }
}

// Per row (one wave): write the kept key blocks in ascending order.  tie_base
// counts the cut ties before the row within its group; K bounds col_idx.
__global__ __launch_bounds__(256) void k_row_scatter(const float *__restrict__ p, int nb,
                                                     int64_t rows, int64_t group_rows, int64_t K,
                                                     const uint32_t *__restrict__ sel,
                                                     const int32_t *__restrict__ tie_base,
                                                     const int32_t *__restrict__ row_ptr,
                                                     int32_t *__restrict__ col_idx) {
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;
    const int lane = threadIdx.x & 63;
    const uint32_t *gs = sel + (r / group_rows) * kHeadSelWords;
    const uint32_t cut = gs[SEL_CUT];
    const int64_t ties = gs[SEL_TIES];
    int64_t tie = tie_base[r];
    int64_t out = row_ptr[r];
    const uint64_t lt = lanemask_lt();
    for (int j0 = 0; j0 < nb; j0 += 64) {
        const int j = j0 + lane;
        const bool valid = j < nb;
        const uint32_t key = valid ? order_key(p[r * nb + j]) : 0u;
        const bool is_eq = valid && key == cut;
        const uint64_t eqm = __ballot(is_eq);
        const int64_t my_tie = tie + __popcll(eqm & lt);
        const bool keep = valid && (key > cut || (is_eq && my_tie < ties));
        const uint64_t km = __ballot(keep);
        const int64_t slot = out + __popcll(km & lt);
        if (keep && slot < K) col_idx[slot] = j;   // K bounds the list; never exceeded
        out += __popcll(km);
        tie += __popcll(eqm);
    }
}

// ------------------------------------------------- uniform per-head budget --
// One workgroup per head: the k_h-th largest order key of the head's nb*nb
// scores by the same three digit passes, with the histogram in LDS.  State
// words at hsel[h * kHeadSelWords]: cut key, count above it, ties to keep, k_h.
__global__ __launch_bounds__(1024) void k_head_select(const float *__restrict__ p, int64_t per,
                                                      int64_t k_h,
                                                      uint32_t *__restrict__ hsel) {
    __shared__ uint32_t hist[kRadixBins];
    __shared__ uint32_t win[2];
    const int h = blockIdx.x, tid = threadIdx.x;
    const float *ph = p + (int64_t)h * per;
    uint32_t *out = hsel + (int64_t)h * kHeadSelWords;
    if (k_h <= 0) {   // nothing kept: no score is above the cut, no tie is kept
        if (tid == 0) {
            out[SEL_CUT] = 0xFFFFFFFFu;
            out[SEL_ABOVE] = 0;
            out[SEL_TIES] = 0;
            out[SEL_K] = 0;
        }
        return;
    }
    uint32_t prefix = 0;
    int64_t remain = k_h;   // rank wanted inside the prefix bucket, counted from the top
    for (int pass = 0; pass < 3; ++pass) {
        int shift;
        uint32_t hi_mask, dmask;
        digit_of_pass(pass, shift, hi_mask, dmask);
        for (int b = tid; b < kRadixBins; b += 1024) hist[b] = 0;
        __syncthreads();
        for (int64_t x = tid; x < per; x += 1024) {
            const uint32_t key = order_key(ph[x]);
            if ((key & hi_mask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
        }
        __syncthreads();
        // Bins in descending order; thread t owns ranks 2t and 2t+1.
        const int nbins = (int)dmask + 1;
        const int r0 = 2 * tid, r1 = r0 + 1;
        const int b0 = nbins - 1 - r0, b1 = nbins - 1 - r1;
        const int64_t c0 = r0 < nbins ? hist[b0] : 0;
        const int64_t c1 = r1 < nbins ? hist[b1] : 0;
        int64_t total;
        const int64_t before = block_exclusive_scan_1024(c0 + c1, &total);
        if (r0 < nbins && before < remain && remain <= before + c0) {
            win[0] = (uint32_t)b0;
            win[1] = (uint32_t)(remain - before);
        } else if (r1 < nbins && before + c0 < remain && remain <= before + c0 + c1) {
            win[0] = (uint32_t)b1;
            win[1] = (uint32_t)(remain - before - c0);
        }
        __syncthreads();
        prefix |= win[0] << shift;
        remain = win[1];
        __syncthreads();
    }
    if (tid == 0) {
        out[SEL_CUT] = prefix;
        out[SEL_ABOVE] = (uint32_t)(k_h - remain);
        out[SEL_TIES] = (uint32_t)remain;
        out[SEL_K] = (uint32_t)k_h;
    }
}

// One workgroup per head: cut ties before each row within the head (flat
// order) and the row's kept count, written over gt.
__global__ __launch_bounds__(1024) void k_head_ties(int32_t *__restrict__ gt,
                                                    const int32_t *__restrict__ eq, int nb,
                                                    const uint32_t *__restrict__ hsel,
                                                    int32_t *__restrict__ tie_base) {
    const int h = blockIdx.x, i = threadIdx.x;
    const int64_t r = (int64_t)h * nb + i;
    const int64_t ties = hsel[(int64_t)h * kHeadSelWords + SEL_TIES];
    const int e = i < nb ? eq[r] : 0;
    int64_t total;
    const int64_t before = block_exclusive_scan_1024(e, &total);
    if (i < nb) {
        int64_t take = ties - before;
        take = take < 0 ? 0 : (take > e ? e : take);
        tie_base[r] = (int32_t)before;
        gt[r] = (int32_t)(gt[r] + take);
    }
}

// One block: row_ptr as the exclusive prefix of the kept counts.
__global__ __launch_bounds__(1024) void k_kept_scan(const int32_t *__restrict__ kept,
                                                    int64_t rows,
                                                    int32_t *__restrict__ row_ptr) {
    const int64_t per = (rows + 1023) / 1024;
    const int64_t lo = min(rows, (int64_t)threadIdx.x * per);
    const int64_t hi = min(rows, lo + per);
    int64_t local = 0;
    for (int64_t r = lo; r < hi; ++r) local += kept[r];
    int64_t total;
    int64_t out = block_exclusive_scan_1024(local, &total);
    for (int64_t r = lo; r < hi; ++r) {
        row_ptr[r] = (int32_t)out;
        out += kept[r];
    }
    if (threadIdx.x == 0) row_ptr[rows] = (int32_t)total;
}

// ------------------------------------------------------------ column lists --
// Column-sparse variant ("PulseCol" abstract: column-sparse attention): head
// h keeps the k_c largest of its L column masses, the per-head select state
// (cut key, ties kept at the cut) coming from k_head_select.  One workgroup
// per head; thread t owns a contiguous run of columns.  Ties at the cut are
// kept in ascending column order, so the kept set is the top-k_c under
// (value descending, index ascending) and the list comes out ascending.
__global__ __launch_bounds__(1024) void k_col_compact(const float *__restrict__ c, int L,
                                                      const uint32_t *__restrict__ hsel,
                                                      int64_t k_c, int32_t *__restrict__ cols) {
    const int h = blockIdx.x, tid = threadIdx.x;
    const float *ch = c + (int64_t)h * L;
    const uint32_t cut = hsel[(int64_t)h * kHeadSelWords + SEL_CUT];
    const int64_t ties = hsel[(int64_t)h * kHeadSelWords + SEL_TIES];
    const int per = (L + 1023) / 1024;
    const int lo = min(L, tid * per), hi = min(L, lo + per);
    int64_t n_eq = 0;
    for (int u = lo; u < hi; ++u) n_eq += order_key(ch[u]) == cut;
    int64_t total;
    const int64_t eq_before = block_exclusive_scan_1024(n_eq, &total);
    int64_t n_keep = 0, e = eq_before;
    for (int u = lo; u < hi; ++u) {
        const uint32_t key = order_key(ch[u]);
        if (key > cut) {
            ++n_keep;
        } else if (key == cut) {
            n_keep += e < ties;
            ++e;
        }
    }
    int64_t out = block_exclusive_scan_1024(n_keep, &total);
    int32_t *dst = cols + (int64_t)h * k_c;
    e = eq_before;
    for (int u = lo; u < hi; ++u) {
        const uint32_t key = order_key(ch[u]);
        bool keep = key > cut;
        if (key == cut) keep = e++ < ties;
        if (keep && out < k_c) dst[out++] = u;
    }
}

// --------------------------------------------------------------------- plan --
// Work order for the attention launch.  The GPU has kDies dies (XCDs), each
// with its own L2, and workgroup b of a launch runs on die b % kDies.  All
// rows of a head go to one die so that the head's K/V stay in that die's L2:
//  * a head weighs (B/32) * kept + 4 * nonempty: the 32-key steps of its
//    kept blocks plus four steps per row that keeps a block, for the row's
//    fixed start-up and write-out;
//  * heads are ranked by weight (descending, ties by head id) and, in that
//    order, each goes to the die with the least weight so far among those
//    holding fewer than min(H, ceil(H / kDies) + 2) heads (ties: lowest die);
//  * die x's list, at work[x*cap ..], cap = (heads a die may hold) * nb, is
//    first the non-empty rows of its heads (heads in assignment order, each
//    head's rows by list length descending, ties by row id), then their empty
//    rows (same head order, rows ascending): empty rows only write zeros and
//    run in the launch's ramp-down; unused positions hold -1;
//  * beside it, work_rec holds one record per position for the attention
//    launch: row, list begin, list end (clamped into [0, nnz]) and the row's
//    first two block ids (16 bits each, clamped into [0, nb)), so that a
//    workgroup's first K/V loads need one load, not a chain of three; padding
//    records have row -1.
// Two launches.  k_plan_assign, one workgroup: the heads' weights straight
// from row_ptr, their ranks, the die assignment by one wave with one die per
// lane (the least-loaded open die found by a three-step 8-lane argmin), each
// head's first position among its die's non-empty rows and among its die's
// empty rows, the padding and the meta words.  k_plan_rows, one wave per
// head: the head's row records, its rows by list length descending, ties by
// row id, with a stable counting sort (length histogram, descending bucket
// starts, ranks among equal lengths from wave ballots), written straight to
// the head's positions.

// One step of the die argmin: take the (load, die) pair of the lane that
// dpp_ctrl names when it is smaller.
template <int CTRL>
__device__ __forceinline__ void argmin_step(int64_t &load, int &die) {
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)load, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(load >> 32), CTRL, 0xF, 0xF, false);
    const int64_t l2 = (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
    const int d2 = __builtin_amdgcn_update_dpp(0, die, CTRL, 0xF, 0xF, false);
    const bool take = l2 < load || (l2 == load && d2 < die);
    load = take ? l2 : load;
    die = take ? d2 : die;
}

constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void k_plan_assign(const int32_t *__restrict__ row_ptr,
                                                              const int32_t *list, int64_t nnz,
                                                              int H, int nb, int steps_per_block,
                                                              int32_t *__restrict__ head_base,
                                                              int32_t *__restrict__ work,
                                                              int4 *__restrict__ work_rec,
                                                              int32_t *__restrict__ meta) {
    static_assert(kDies == 8, "the die argmin covers 8 lanes");
    __shared__ int64_t weight[kMaxHeads];
    __shared__ int32_t ne[kMaxHeads], kept[kMaxHeads];
    __shared__ int32_t order[kMaxHeads];
    __shared__ int32_t die_of[kMaxHeads], slot_of[kMaxHeads];
    __shared__ int32_t die_list[kDies * kMaxHeads];   // die x's heads in slot order
    __shared__ int32_t die_heads[kDies];
    __shared__ int32_t nonempty;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cap_h = min(H, (H + kDies - 1) / kDies + 2);
    const int cap = cap_h * nb;   // below 2^31: 8 * cap <= 8 * H * nb
    for (int h = tid; h < H; h += kPlanThreads) ne[h] = kept[h] = 0;
    if (tid == 0) nonempty = 0;
    __syncthreads();
    // Per head: rows that keep a block and blocks kept.  Thread t reads the
    // bounds of rows 4u .. 4u + 3, u = t, t + 1024, ..., in one batch.
    const int rows = H * nb;
    for (int r = 4 * tid; r < rows; r += 4 * kPlanThreads) {
        int v[5];
#pragma unroll
        for (int k = 0; k < 5; ++k) v[k] = row_ptr[min(r + k, rows)];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int len = v[k + 1] - v[k];
            if (r + k < rows && len > 0) {
                atomicAdd(&ne[(r + k) / nb], 1);
                atomicAdd(&kept[(r + k) / nb], len);
            }
        }
    }
    __syncthreads();
    for (int h = tid; h < H; h += kPlanThreads) {
        weight[h] = (int64_t)steps_per_block * kept[h] + 4 * (int64_t)ne[h];
        atomicAdd(&nonempty, ne[h]);
    }
    __syncthreads();
    for (int h = tid; h < H; h += kPlanThreads) {
        int rank = 0;
        for (int o = 0; o < H; ++o)
            rank += (weight[o] > weight[h]) || (weight[o] == weight[h] && o < h);
        order[rank] = h;
    }
    __syncthreads();
    if (wave == 0) {
        // Lane x < 8 holds die x: its weight so far and its head count.
        int64_t my_load = 0;
        int my_count = 0;
        for (int a0 = 0; a0 < H; a0 += 64) {
            const int my_h = a0 + lane < H ? order[a0 + lane] : 0;
            const int64_t my_w = weight[my_h];
            const int n = min(64, H - a0);
            for (int a = 0; a < n; ++a) {
                const int h = __builtin_amdgcn_readlane(my_h, a);
                const int64_t wh = (int64_t)(
                    ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(my_w >> 32), a) << 32) |
                    (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)my_w, a));
                int64_t load = (lane < kDies && my_count < cap_h) ? my_load : INT64_MAX;
                int die = lane;
                argmin_step<0xB1>(load, die);    // quad_perm [1,0,3,2]
                argmin_step<0x4E>(load, die);    // quad_perm [2,3,0,1]
                argmin_step<0x141>(load, die);   // row_half_mirror: lane i <-> 7 - i
                const int best = __builtin_amdgcn_readlane(die, 0);
                if (lane == best) {
                    die_of[h] = best;
                    slot_of[h] = my_count;
                    die_list[best * cap_h + my_count] = h;
                    ++my_count;
                    my_load += wh;
                }
            }
        }
        if (lane < kDies) die_heads[lane] = my_count;
    }
    __syncthreads();
    // Each head's two bases: its die's non-empty rows come first (heads in
    // slot order), then the die's empty rows (same order).
    for (int h = tid; h < H; h += kPlanThreads) {
        const int x = die_of[h], sl = slot_of[h];
        int ne_before = 0, ne_die = 0, em_before = 0;
        for (int c = 0; c < die_heads[x]; ++c) {
            const int n_o = ne[die_list[x * cap_h + c]];
            ne_die += n_o;
            if (c < sl) {
                ne_before += n_o;
                em_before += nb - n_o;
            }
        }
        head_base[2 * h] = x * cap + ne_before;
        head_base[2 * h + 1] = x * cap + ne_die + em_before;
    }
    // Padding: the positions past each die's heads.
    for (int q = tid; q < kDies * cap; q += kPlanThreads) {
        const int x = q / cap;
        if (q - x * cap >= die_heads[x] * nb) {
            work[q] = -1;
            work_rec[q] = make_int4(-1, 0, 0, 0);
        }
    }
    if (tid == 0) {
        meta[kMetaCap] = (int32_t)cap;
        meta[kMetaNonEmpty] = nonempty;
        const uint64_t addr = reinterpret_cast<uint64_t>(list);
        meta[kMetaListLo] = (int32_t)(uint32_t)addr;
        meta[kMetaListHi] = (int32_t)(uint32_t)(addr >> 32);
        meta[kMetaNnz] = (int32_t)nnz;
        meta[kMetaHeads] = H;
        meta[kMetaNb] = nb;
        meta[kMetaCheck] = 0;
    }
}

__global__ __launch_bounds__(64) void k_plan_rows(const int32_t *__restrict__ row_ptr,
                                                  const int32_t *__restrict__ col_idx,
                                                  int64_t nnz, int nb,
                                                  const int32_t *__restrict__ head_base,
                                                  int32_t *__restrict__ work,
                                                  int4 *__restrict__ work_rec) {
    constexpr int kRowsPerLane = kMaxBlocks / 64;
    __shared__ int32_t nx[kMaxBlocks + 1];   // histogram, first staging row_ptr
    __shared__ int16_t ln[kMaxBlocks];
    __shared__ int4 rec[kMaxBlocks];
    const int lane = threadIdx.x, h = blockIdx.x;
    const uint64_t lt = lanemask_lt();
    const int64_t r0 = (int64_t)h * nb;
    const int64_t ne_base = head_base[2 * h], em_base = head_base[2 * h + 1];
    // Stage row_ptr[r0 .. r0 + nb] (loads issued together), then the lengths.
    // A wave's LDS requests complete in order.
    for (int c = 0; c <= nb; c += 512) {
        int v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = row_ptr[r0 + min(c + lane + 64 * j, nb)];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (c + lane + 64 * j <= nb) nx[c + lane + 64 * j] = v[j];
    }
    // Records: list bounds clamped into [0, nnz], the first two ids of the
    // list (all loads of a lane issued together).
    int lo[kRowsPerLane], hi[kRowsPerLane], id0[kRowsPerLane], id1[kRowsPerLane];
#pragma unroll
    for (int t = 0; t < kRowsPerLane; ++t) {
        const int i = lane + 64 * t;
        lo[t] = hi[t] = id0[t] = id1[t] = 0;
        if (i < nb) {
            lo[t] = max(nx[i], 0);
            hi[t] = (int)min((int64_t)nx[i + 1], nnz);
            if (hi[t] > lo[t]) {
                id0[t] = col_idx[lo[t]];
                if (hi[t] - lo[t] > 1) id1[t] = col_idx[lo[t] + 1];
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kRowsPerLane; ++t) {
        const int i = lane + 64 * t;
        if (i < nb) {
            const int a = min(max(id0[t], 0), nb - 1), b = min(max(id1[t], 0), nb - 1);
            rec[i] = make_int4((int)r0 + i, lo[t], hi[t], a | (b << 16));
        }
    }
    int my_ne = 0;
    for (int i = lane; i < nb; i += 64) {
        const int64_t len = (int64_t)nx[i + 1] - nx[i];
        ln[i] = (int16_t)min(max(len, (int64_t)0), (int64_t)nb);
        my_ne += len > 0;
    }
    const int ne_cnt = wave_sum(my_ne);   // the sorted order puts these first
    for (int l = lane; l <= nb; l += 64) nx[l] = 0;
    for (int i = lane; i < nb; i += 64) atomicAdd(&nx[ln[i]], 1);
    // Bucket starts, longest lists first: nx[l] = rows with length > l.
    int carry = 0;
    for (int c0 = nb; c0 >= 0; c0 -= 64) {
        const int l = c0 - lane;
        const int cnt = l >= 0 ? nx[l] : 0;
        int inc = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(inc, o);
            if (lane >= o) inc += y;
        }
        if (l >= 0) nx[l] = carry + inc - cnt;
        carry += __shfl(inc, 63);
    }
    for (int i0 = 0; i0 < nb; i0 += 64) {
        const int i = i0 + lane;
        const bool valid = i < nb;
        const int len = valid ? ln[i] : 0;
        uint64_t same = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < 11; ++bit) {
            const bool mine = (len >> bit) & 1;
            const uint64_t b = __ballot(valid && mine);
            same &= mine ? b : ~b;
        }
        const int rank = __popcll(same & lt);
        const int pos = valid ? nx[len] + rank : 0;
        if (valid && pos < nb) {
            const int64_t at = pos < ne_cnt ? ne_base + pos : em_base + (pos - ne_cnt);
            work[at] = (int32_t)(r0 + i);
            work_rec[at] = rec[i];
        }
        if (valid && rank == 0) nx[len] += __popcll(same);
    }
}

}  // namespace

// ------------------------------------------------------------------ launches --
hipError_t launch_pool(const Dims &D, const uint16_t *q, const uint16_t *k, float *qb, float *kb,
                       hipStream_t s) {
    const int64_t cg = D.d / 4;
    const int64_t nq = (int64_t)D.H * D.nb * cg, nk = (int64_t)D.Hkv * D.nb * cg;
    const int64_t grid = (nq + nk + 255) / 256;
    if (D.d == 128)
        hipLaunchKernelGGL(k_pool<128>, dim3((unsigned)grid), dim3(256), 0, s, q, k, qb, kb, D.L,
                           D.B, nq, nk);
    else
        hipLaunchKernelGGL(k_pool<64>, dim3((unsigned)grid), dim3(256), 0, s, q, k, qb, kb, D.L,
                           D.B, nq, nk);
    return hipGetLastError();
}

hipError_t launch_pool_q(const Dims &D, const uint16_t *q, float *qb, hipStream_t s) {
    const int64_t nq = (int64_t)D.H * D.nb * (D.d / 4);
    const int64_t grid = (nq + 255) / 256;
    if (D.d == 128)
        hipLaunchKernelGGL(k_pool<128>, dim3((unsigned)grid), dim3(256), 0, s, q, nullptr, qb,
                           nullptr, D.L, D.B, nq, (int64_t)0);
    else
        hipLaunchKernelGGL(k_pool<64>, dim3((unsigned)grid), dim3(256), 0, s, q, nullptr, qb,
                           nullptr, D.L, D.B, nq, (int64_t)0);
    return hipGetLastError();
}

hipError_t launch_col_select(const Dims &D, int64_t k_c, const float *c, char *ws,
                             const WsLayout &w, int32_t *cols, hipStream_t s) {
    uint32_t *hsel = reinterpret_cast<uint32_t *>(ws + w.hsel);
    hipLaunchKernelGGL(k_head_select, dim3(D.H), dim3(1024), 0, s, c, (int64_t)D.L, k_c, hsel);
    if (k_c > 0)
        hipLaunchKernelGGL(k_col_compact, dim3(D.H), dim3(1024), 0, s, c, D.L, hsel, k_c, cols);
    return hipGetLastError();
}

hipError_t launch_scores(const Dims &D, const float *qb, const float *kb, float *p, float *copy,
                         char *ws, const WsLayout &w, int64_t sel_init_K, hipStream_t s) {
    uint32_t *hist = sel_init_K >= 0 ? reinterpret_cast<uint32_t *>(ws + w.hist) : nullptr;
    uint32_t *sel = sel_init_K >= 0 ? reinterpret_cast<uint32_t *>(ws + w.sel) : nullptr;
    const int tiles = (D.nb + kScoreRows - 1) / kScoreRows;
    const float sigma = (float)(1.0 / sqrt((double)D.d));
    dim3 grid((unsigned)(D.H * tiles));
    if (D.d == 128)
        hipLaunchKernelGGL(k_scores<128>, grid, dim3(kScoreThreads), 0, s, qb, kb, p, copy, D.nb,
                           D.G, sigma, hist, sel, sel_init_K);
    else
        hipLaunchKernelGGL(k_scores<64>, grid, dim3(kScoreThreads), 0, s, qb, kb, p, copy, D.nb,
                           D.G, sigma, hist, sel, sel_init_K);
    return hipGetLastError();
}

hipError_t launch_select(const Dims &D, int64_t K, const float *p, char *ws, const WsLayout &w,
                         int32_t *row_ptr, int32_t *col_idx, bool state_ready, hipStream_t s) {
    uint32_t *hist = reinterpret_cast<uint32_t *>(ws + w.hist);
    uint32_t *sel = reinterpret_cast<uint32_t *>(ws + w.sel);
    int32_t *gt = reinterpret_cast<int32_t *>(ws + w.gt);
    int32_t *eq = reinterpret_cast<int32_t *>(ws + w.eq);
    const int64_t n = D.n_scores(), rows = D.rows();
    if (!state_ready) hipLaunchKernelGGL(k_select_init, dim3(1), dim3(1024), 0, s, hist, sel, K);
    if (K > 0) {
        int64_t g = (n / 4 + kRadixThreads - 1) / kRadixThreads;
        g = g < 1 ? 1 : (g > 256 ? 256 : g);
        for (int pass = 0; pass < 3; ++pass)
            hipLaunchKernelGGL(k_radix_pass, dim3((unsigned)g), dim3(kRadixThreads), 0, s, p, n,
                               sel, hist, pass);
        hipLaunchKernelGGL(k_radix_final, dim3(1), dim3(kRadixThreads), 0, s, hist, sel);
    }
    int32_t *agg = reinterpret_cast<int32_t *>(ws + w.row_agg);
    const unsigned row_grid = (unsigned)((rows + kCompactRows - 1) / kCompactRows);
    hipLaunchKernelGGL(k_row_count, dim3(row_grid), dim3(1024), 0, s, p, D.nb, rows, rows, sel, gt,
                       eq, agg);
    hipLaunchKernelGGL(k_row_emit, dim3(row_grid), dim3(1024), 0, s, p, D.nb, rows, K, sel, gt, eq,
                       agg, row_ptr, col_idx);
    return hipGetLastError();
}

hipError_t launch_select_per_head(const Dims &D, int64_t k_h, const float *p, char *ws,
                                  const WsLayout &w, int32_t *row_ptr, int32_t *col_idx,
                                  hipStream_t s) {
    uint32_t *hsel = reinterpret_cast<uint32_t *>(ws + w.hsel);
    int32_t *gt = reinterpret_cast<int32_t *>(ws + w.gt);
    int32_t *eq = reinterpret_cast<int32_t *>(ws + w.eq);
    int32_t *tie_base = reinterpret_cast<int32_t *>(ws + w.tie_base);
    const int64_t rows = D.rows();
    const unsigned row_grid = (unsigned)((rows + 3) / 4);
    hipLaunchKernelGGL(k_head_select, dim3(D.H), dim3(1024), 0, s, p, (int64_t)D.nb * D.nb, k_h,
                       hsel);
    hipLaunchKernelGGL(k_row_count, dim3((unsigned)((rows + kCompactRows - 1) / kCompactRows)),
                       dim3(1024), 0, s, p, D.nb, rows, (int64_t)D.nb, hsel, gt, eq, nullptr);
    hipLaunchKernelGGL(k_head_ties, dim3(D.H), dim3(1024), 0, s, gt, eq, D.nb, hsel, tie_base);
    hipLaunchKernelGGL(k_kept_scan, dim3(1), dim3(1024), 0, s, gt, rows, row_ptr);
    hipLaunchKernelGGL(k_row_scatter, dim3(row_grid), dim3(256), 0, s, p, D.nb, rows,
                       (int64_t)D.nb, k_h * D.H, hsel, tie_base, row_ptr, col_idx);
    return hipGetLastError();
}

hipError_t launch_plan(const Dims &D, const int32_t *row_ptr, const int32_t *col_idx,
                       int64_t nnz, char *ws, const WsLayout &w, hipStream_t s) {
    int32_t *work = reinterpret_cast<int32_t *>(ws + w.work);
    int4 *work_rec = reinterpret_cast<int4 *>(ws + w.work_rec);
    int32_t *meta = reinterpret_cast<int32_t *>(ws + w.work_meta);
    int32_t *head_base = reinterpret_cast<int32_t *>(ws + w.plan_head_base);
    hipLaunchKernelGGL(k_plan_assign, dim3(1), dim3(kPlanThreads), 0, s, row_ptr, col_idx, nnz,
                       D.H, D.nb, D.B / 32, head_base, work, work_rec, meta);
    hipLaunchKernelGGL(k_plan_rows, dim3(D.H), dim3(64), 0, s, row_ptr, col_idx, nnz, D.nb,
                       head_base, work, work_rec);
    return hipGetLastError();
}

}  // namespace sd
