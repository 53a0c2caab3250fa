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
// A workgroup pools kPoolPairs consecutive (head, block) pairs of Q (or K),
// which are one contiguous piece of the tensor: its 256 threads first copy
// the piece into LDS with 16-byte buffer->LDS loads (1 KiB per wave
// instruction, all of a wave's loads in flight), then thread t adds the B
// rows of two columns of one block in ascending token order in fp32 (the
// order of the definition) and scales by 1/B (a power of two, exact).
// With init_sel set, block 0 also prepares the global select state for a
// budget of init_K (zero histograms), which the score launch then fills.
__device__ void select_init(uint32_t *__restrict__ hist, uint32_t *__restrict__ sel, int64_t K,
                            int tid, int nthreads);

template <int D>
constexpr int pool_pairs() { return 256 / (D / 2); }   // (head, block) pairs per workgroup
// Cache policy of the pool's loads: non-temporal (each byte of Q and K is
// read once), 5.74 against 5.48 TB/s in the bench's kernel trace.
constexpr int kLoadStreaming = 2;

template <int D, int BLK>
__global__ __launch_bounds__(256) void k_pool(const uint16_t *__restrict__ q,
                                              const uint16_t *__restrict__ k,
                                              float *__restrict__ qb, float *__restrict__ kb,
                                              int64_t q_pairs, int64_t k_pairs,
                                              uint32_t *__restrict__ init_hist,
                                              uint32_t *__restrict__ init_sel, int64_t init_K) {
    constexpr int PAIRS = pool_pairs<D>();
    constexpr int PIECE = PAIRS * BLK * D * 2;   // bytes: 64 KiB (B = 64) or 128 KiB (B = 128)
    constexpr int LOADS = PIECE / 1024;          // 1 KiB wave loads per piece
    __shared__ __attribute__((aligned(16))) uint16_t piece[PIECE / 2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (init_sel && blockIdx.x == 0) select_init(init_hist, init_sel, init_K, tid, 256);
    // Group g of PAIRS consecutive (head, block) pairs; the last group of a
    // tensor may hold fewer (its loads past the tensor read zeros).
    const int64_t q_groups = (q_pairs + PAIRS - 1) / PAIRS;
    const int64_t k_groups = (k_pairs + PAIRS - 1) / PAIRS;
    int64_t g = blockIdx.x;
    const uint16_t *src = q;
    float *dst = qb;
    int64_t pairs = q_pairs;
    if (g >= q_groups) {
        g -= q_groups;
        if (g >= k_groups) return;
        src = k;
        dst = kb;
        pairs = k_pairs;
    }
    const int here = (int)min((int64_t)PAIRS, pairs - g * PAIRS);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(src + g * (PIECE / 2)), 0, here * (PIECE / PAIRS), 0x00020000);
#pragma unroll
    for (int t = wave; t < LOADS; t += 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (__attribute__((address_space(3))) void *)(piece + t * 512), 16, lane * 16,
            t * 1024, 0, kLoadStreaming);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int pr = tid / (D / 2), c = tid % (D / 2);   // pair, column pair
    const uint32_t *rows = reinterpret_cast<const uint32_t *>(piece) + pr * BLK * (D / 2) + c;
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll 16
    for (int t = 0; t < BLK; ++t) {
        const uint32_t w = rows[t * (D / 2)];
        a0 = a0 + bf16_bits_to_float(w & 0xFFFFu);
        a1 = a1 + bf16_bits_to_float(w >> 16);
    }
    const float inv_b = 1.0f / (float)BLK;
    if (pr < here)
        *reinterpret_cast<float2 *>(dst + (g * PAIRS + pr) * D + 2 * c) =
            make_float2(a0 * inv_b, a1 * inv_b);
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
// means stream through LDS 128 rows at a time (read once per 16 rows; the
// next 128 are loaded into registers while the current ones are used).  Wave
// w forms the products of rows 2w and 2w + 1, lane c of it those of columns c
// and c + 64 of the tile: each operand is one 16-byte LDS read per four
// elements (rows padded by four floats so that the lanes' reads hit distinct
// banks), and each dot product is summed in ascending element order with
// separately rounded multiply and add, then scaled.  Each wave softmaxes its
// own two rows (lane l takes columns l + 64 t, then a butterfly over the
// wave): rows of at most 128 blocks straight from registers, wider rows from
// LDS (up to kMaxBlocks per row), in the same order.  With hist0 set, the
// workgroup also counts its scores into the histogram of the first digit of
// the global select (bits 31..21 of the order keys; the pool launch zeroed
// it), so the select starts at its second digit.
constexpr int kScoreRows = 16;
constexpr int kScoreCols = 128;
constexpr int kScoreThreads = 512;

template <int D>
__global__ __launch_bounds__(kScoreThreads) void k_scores(const float *__restrict__ qb,
                                                          const float *__restrict__ kb,
                                                          float *__restrict__ p,
                                                          float *__restrict__ copy, int nb, int G,
                                                          float sigma,
                                                          uint32_t *__restrict__ hist0) {
#pragma clang fp contract(off)
    constexpr int SP = D + 4;   // padded LDS row (floats)
    static_assert(kScoreCols * SP >= kRadixBins, "the first-digit histogram reuses the key tile");
    __shared__ __attribute__((aligned(16))) float sq[kScoreRows * SP];
    __shared__ __attribute__((aligned(16))) float sk[kScoreCols * SP];
    __shared__ float srow[kScoreRows][kMaxBlocks];
    const int tid = threadIdx.x;
    const int tiles = (nb + kScoreRows - 1) / kScoreRows;
    // Workgroups go round-robin to the 8 dies, each with its own L2: renumber
    // so that consecutive tiles (one head's rows, sharing its key means) run
    // on one die, and each die fetches a head's key means once.
    int bid = blockIdx.x;
    if (gridDim.x % 8 == 0) bid = (bid % 8) * (gridDim.x / 8) + bid / 8;
    const int h = bid / tiles;
    const int i0 = (bid % tiles) * kScoreRows;
    const int g = h / G;
    constexpr int C4 = D / 4;   // float4 per row
    constexpr int Q4 = (kScoreRows * C4 + kScoreThreads - 1) / kScoreThreads;
    constexpr int K4 = kScoreCols * C4 / kScoreThreads;
#pragma unroll
    for (int t = 0; t < Q4; ++t) {
        const int x = tid + kScoreThreads * t, r = x / C4, c4 = x % C4;
        if (r < kScoreRows)
            *reinterpret_cast<float4 *>(&sq[r * SP + 4 * c4]) =
                i0 + r < nb
                    ? reinterpret_cast<const float4 *>(qb + ((int64_t)h * nb + i0 + r) * D)[c4]
                    : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    float4 kv[K4];
    auto load_keys = [&](int j0) {
#pragma unroll
        for (int t = 0; t < K4; ++t) {
            const int x = tid + kScoreThreads * t, rr = x / C4, c4 = x % C4;
            kv[t] = j0 + rr < nb ? reinterpret_cast<const float4 *>(
                                       kb + ((int64_t)g * nb + j0 + rr) * D)[c4]
                                 : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
    };
    load_keys(0);
    const int w2 = 2 * (tid >> 6), cl = tid & 63;
    const float *q0 = sq + w2 * SP, *q1 = q0 + SP;
    const float *k0 = sk + cl * SP, *k1 = sk + (cl + 64) * SP;
    float s00 = 0.0f, s01 = 0.0f, s10 = 0.0f, s11 = 0.0f;
    for (int j0 = 0; j0 < nb; j0 += kScoreCols) {
        __syncthreads();   // the previous tile's reads are done
#pragma unroll
        for (int t = 0; t < K4; ++t) {
            const int x = tid + kScoreThreads * t, rr = x / C4, c4 = x % C4;
            *reinterpret_cast<float4 *>(&sk[rr * SP + 4 * c4]) = kv[t];
        }
        __syncthreads();
        if (j0 + kScoreCols < nb) load_keys(j0 + kScoreCols);
        s00 = s01 = s10 = s11 = 0.0f;
#pragma unroll 8
        for (int c = 0; c < D; c += 4) {
            const float4 x0 = *reinterpret_cast<const float4 *>(q0 + c);
            const float4 x1 = *reinterpret_cast<const float4 *>(q1 + c);
            const float4 y0 = *reinterpret_cast<const float4 *>(k0 + c);
            const float4 y1 = *reinterpret_cast<const float4 *>(k1 + c);
            s00 = s00 + x0.x * y0.x; s01 = s01 + x0.x * y1.x;
            s10 = s10 + x1.x * y0.x; s11 = s11 + x1.x * y1.x;
            s00 = s00 + x0.y * y0.y; s01 = s01 + x0.y * y1.y;
            s10 = s10 + x1.y * y0.y; s11 = s11 + x1.y * y1.y;
            s00 = s00 + x0.z * y0.z; s01 = s01 + x0.z * y1.z;
            s10 = s10 + x1.z * y0.z; s11 = s11 + x1.z * y1.z;
            s00 = s00 + x0.w * y0.w; s01 = s01 + x0.w * y1.w;
            s10 = s10 + x1.w * y0.w; s11 = s11 + x1.w * y1.w;
        }
        s00 = s00 * sigma;
        s01 = s01 * sigma;
        s10 = s10 * sigma;
        s11 = s11 * sigma;
        if (nb > kScoreCols) {   // wider rows wait in LDS
            const int j = j0 + cl;
            if (j < nb) {
                srow[w2][j] = s00;
                srow[w2 + 1][j] = s10;
            }
            if (j + 64 < nb) {
                srow[w2][j + 64] = s01;
                srow[w2 + 1][j + 64] = s11;
            }
        }
    }
    uint32_t *hh = reinterpret_cast<uint32_t *>(sk);   // free once the products are done
    __syncthreads();
    if (hist0)
        for (int b = tid; b < kRadixBins; b += kScoreThreads) hh[b] = 0;
    // Softmax of rows w2 and w2 + 1 by the wave that formed them: lane l
    // takes columns l + 64 t (t ascending), then a 6-level butterfly over the
    // wave.  Rows of at most 128 blocks are still in registers (lane l holds
    // columns l and l + 64); wider rows are read back from LDS in the same
    // order, so both give the same sums.
    const int64_t base0 = ((int64_t)h * nb + i0 + w2) * nb;
    const bool ok0 = i0 + w2 < nb, ok1 = i0 + w2 + 1 < nb;
    auto wave_max = [](float x) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
        return x;
    };
    auto wave_fsum = [](float x) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) x = x + __shfl_xor(x, o);
        return x;
    };
    if (nb <= kScoreCols) {
        const bool v0 = cl < nb, v1 = cl + 64 < nb;
        const float m0 = wave_max(fmaxf(v0 ? s00 : -INFINITY, v1 ? s01 : -INFINITY));
        const float m1 = wave_max(fmaxf(v0 ? s10 : -INFINITY, v1 ? s11 : -INFINITY));
        const float e00 = v0 ? expf(s00 - m0) : 0.0f, e01 = v1 ? expf(s01 - m0) : 0.0f;
        const float e10 = v0 ? expf(s10 - m1) : 0.0f, e11 = v1 ? expf(s11 - m1) : 0.0f;
        const float z0 = wave_fsum(e00 + e01), z1 = wave_fsum(e10 + e11);
        const float p00 = e00 / z0, p01 = e01 / z0, p10 = e10 / z1, p11 = e11 / z1;
        if (ok0) {
            if (v0) p[base0 + cl] = p00;
            if (v1) p[base0 + cl + 64] = p01;
            if (copy && v0) copy[base0 + cl] = p00;
            if (copy && v1) copy[base0 + cl + 64] = p01;
        }
        if (ok1) {
            if (v0) p[base0 + nb + cl] = p10;
            if (v1) p[base0 + nb + cl + 64] = p11;
            if (copy && v0) copy[base0 + nb + cl] = p10;
            if (copy && v1) copy[base0 + nb + cl + 64] = p11;
        }
        if (!hist0) return;
        __syncthreads();   // the histogram is zeroed
        // First-digit histogram (bits 31..21 of the order keys).
        if (ok0 && v0) atomicAdd(&hh[order_key(p00) >> 21], 1u);
        if (ok0 && v1) atomicAdd(&hh[order_key(p01) >> 21], 1u);
        if (ok1 && v0) atomicAdd(&hh[order_key(p10) >> 21], 1u);
        if (ok1 && v1) atomicAdd(&hh[order_key(p11) >> 21], 1u);
    } else {
        float m0 = -INFINITY, m1 = -INFINITY;
        for (int j = cl; j < nb; j += 64) {
            m0 = fmaxf(m0, srow[w2][j]);
            m1 = fmaxf(m1, srow[w2 + 1][j]);
        }
        m0 = wave_max(m0);
        m1 = wave_max(m1);
        float z0 = 0.0f, z1 = 0.0f;
        for (int j = cl; j < nb; j += 64) {
            const float e0 = expf(srow[w2][j] - m0), e1 = expf(srow[w2 + 1][j] - m1);
            srow[w2][j] = e0;
            srow[w2 + 1][j] = e1;
            z0 = z0 + e0;
            z1 = z1 + e1;
        }
        z0 = wave_fsum(z0);
        z1 = wave_fsum(z1);
        if (hist0) __syncthreads();   // the histogram is zeroed
        for (int j = cl; j < nb; j += 64) {
            const float a0 = srow[w2][j] / z0, a1 = srow[w2 + 1][j] / z1;
            if (ok0) {
                p[base0 + j] = a0;
                if (copy) copy[base0 + j] = a0;
                if (hist0) atomicAdd(&hh[order_key(a0) >> 21], 1u);
            }
            if (ok1) {
                p[base0 + nb + j] = a1;
                if (copy) copy[base0 + nb + j] = a1;
                if (hist0) atomicAdd(&hh[order_key(a1) >> 21], 1u);
            }
        }
        if (!hist0) return;
    }
    __syncthreads();
    for (int b = tid; b < kRadixBins; b += kScoreThreads)
        if (hh[b]) atomicAdd(&hist0[b], hh[b]);
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
// the pass's global histogram.  The workgroup's first batch of scores does
// not depend on the prefix: its loads are issued before the digit step.
constexpr int kRadixThreads = 1024;

__global__ __launch_bounds__(kRadixThreads) void k_radix_pass(const float *__restrict__ p,
                                                              int64_t n,
                                                              uint32_t *__restrict__ sel,
                                                              uint32_t *__restrict__ hist,
                                                              int pass) {
    __shared__ uint32_t h[kRadixBins];
    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t stride = (int64_t)gridDim.x * kRadixThreads;
    const int64_t n4 = n >> 2;
    const float4 *p4 = reinterpret_cast<const float4 *>(p);
    const int64_t first = (int64_t)blockIdx.x * kRadixThreads;
    const bool in0 = first + tid < n4;
    const float4 v0 = in0 ? p4[first + tid] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
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
    if (first < n4) {
        count(v0.x, in0);
        count(v0.y, in0);
        count(v0.z, in0);
        count(v0.w, in0);
    }
    for (int64_t base = first + stride; base < n4; base += stride) {
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

// --------------------------------------------------------------- compaction --
// Per row (one wave; 16 rows per workgroup): how many scores are above the
// cut and how many equal it.  Rows come in groups of group_rows that share one
// select state (all rows for the global budget, one head's rows for the
// per-head one), kHeadSelWords apart.  With agg set, workgroup b also writes
// its rows' sums of both counts to agg[2b], agg[2b + 1].

// With zero_words set, workgroup 0 also clears n_zero words (the head counts
// that k_row_emit adds to).
// With final_hist set (global budget, K > 0), every workgroup first takes the
// select's last digit step from the histogram of the last pass (cheaper than a
// launch of its own); workgroup 0 records the cut, the count above it and the
// ties to keep in the state words.
__global__ __launch_bounds__(1024) void k_row_count(const float *__restrict__ p, int nb,
                                                    int64_t rows, int64_t group_rows,
                                                    uint32_t *__restrict__ sel,
                                                    const uint32_t *__restrict__ final_hist,
                                                    int32_t *__restrict__ gt,
                                                    int32_t *__restrict__ eq,
                                                    int32_t *__restrict__ agg,
                                                    int32_t *__restrict__ zero_words, int n_zero) {
    __shared__ int32_t sg[kCompactRows], se[kCompactRows];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * kCompactRows + wave;
    // The row's first 128 scores, loaded before the digit step they do not
    // depend on.
    const float *pr = p + r * nb;
    const float pre0 = r < rows && lane < nb ? pr[lane] : 0.0f;
    const float pre1 = r < rows && lane + 64 < nb ? pr[lane + 64] : 0.0f;
    if (zero_words && blockIdx.x == 0)
        for (int t = threadIdx.x; t < n_zero; t += 1024) zero_words[t] = 0;
    uint32_t final_cut = 0;
    if (final_hist) {
        const RadixState st = radix_step(final_hist, 2, load_state(sel, 2));
        final_cut = st.prefix;
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            sel[SEL_PREFIX] = st.prefix;
            sel[SEL_ABOVE] = st.above;
            sel[SEL_REMAIN] = st.remain;
            sel[SEL_CUT] = st.prefix;
            sel[SEL_TIES] = st.remain;
        }
    }
    int cg = 0, ce = 0;
    if (r < rows) {
        const uint32_t cut =
            final_hist ? final_cut : sel[(r / group_rows) * kHeadSelWords + SEL_CUT];
        for (int j = lane; j < nb; j += 64) {
            const uint32_t key = order_key(j < 64 ? pre0 : (j < 128 ? pre1 : pr[j]));
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
// LDS.  K bounds col_idx.  With rec_out set, each row's plan record goes to
// rec_out[row] (row, list begin, list end, first two kept ids in 16 bits each,
// as k_plan_rows forms it) and each head's kept blocks and non-empty rows are
// added to head_counts[h], head_counts[H + h] (cleared by k_row_count).
__global__ __launch_bounds__(1024) void k_row_emit(const float *__restrict__ p, int nb,
                                                   int64_t rows, int64_t K,
                                                   const uint32_t *__restrict__ sel,
                                                   const int32_t *__restrict__ gt,
                                                   const int32_t *__restrict__ eq,
                                                   const int32_t *__restrict__ agg,
                                                   int32_t *__restrict__ row_ptr,
                                                   int32_t *__restrict__ col_idx,
                                                   int4 *__restrict__ rec_out,
                                                   int32_t *__restrict__ head_counts, int H) {
    __shared__ int64_t row_eq[kCompactRows], row_kept[kCompactRows];
    __shared__ int32_t s_hk[kCompactRows], s_hn[kCompactRows];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t r = (int64_t)blockIdx.x * kCompactRows + wave;
    // Loads that do not depend on the scans below, issued first: the cut,
    // the row's counts and its first 128 scores.
    const uint32_t cut = sel[SEL_CUT];
    const int64_t ties = sel[SEL_TIES];
    const int64_t my_gt = r < rows ? gt[r] : 0, my_eq = r < rows ? eq[r] : 0;
    const float *pr = p + r * nb;
    const float pre0 = r < rows && lane < nb ? pr[lane] : 0.0f;
    const float pre1 = r < rows && lane + 64 < nb ? pr[lane + 64] : 0.0f;
    int64_t g_loc = 0, e_loc = 0;
    for (int64_t b = tid; b < blockIdx.x; b += 1024) {
        g_loc += agg[2 * b];
        e_loc += agg[2 * b + 1];
    }
    int64_t g_before, e_before;
    block_exclusive_scan_1024(g_loc, &g_before);
    block_exclusive_scan_1024(e_loc, &e_before);
    if (lane == 0) row_eq[wave] = my_eq;
    __syncthreads();
    int64_t tie = e_before;
    for (int w = 0; w < wave; ++w) tie += row_eq[w];
    int64_t take = ties - tie;
    take = take < 0 ? 0 : (take > my_eq ? my_eq : take);
    if (lane == 0) row_kept[wave] = my_gt + take;
    if (tid < kCompactRows) s_hk[tid] = s_hn[tid] = 0;
    __syncthreads();
    // The rows of this workgroup start at head h_first.
    const int64_t h_first = (int64_t)blockIdx.x * kCompactRows / nb;
    if (r < rows) {
        int64_t out = g_before + (ties < e_before ? ties : e_before);
        for (int w = 0; w < wave; ++w) out += row_kept[w];
        const int64_t start = out, kept = my_gt + take;
        if (lane == 0) {
            row_ptr[r] = (int32_t)out;
            if (r == rows - 1) row_ptr[rows] = (int32_t)(out + kept);
        }
        const uint64_t lt = lanemask_lt();
        int id0 = 0, id1 = 0, seen = 0;
        for (int j0 = 0; j0 < nb; j0 += 64) {
            const int j = j0 + lane;
            const bool valid = j < nb;
            const uint32_t key =
                valid ? order_key(j0 == 0 ? pre0 : (j0 == 64 ? pre1 : pr[j])) : 0u;
            const bool is_eq = valid && key == cut;
            const uint64_t eqm = __ballot(is_eq);
            const int64_t my_tie = tie + __popcll(eqm & lt);
            const bool keep = valid && (key > cut || (is_eq && my_tie < ties));
            const uint64_t km = __ballot(keep);
            const int64_t slot = out + __popcll(km & lt);
            if (keep && slot < K) col_idx[slot] = j;   // K bounds the list; never exceeded
            if (rec_out && seen < 2 && km) {   // the first two ids, for the record
                const uint64_t km1 = km & (km - 1);
                if (seen == 0) {
                    id0 = j0 + __builtin_ctzll(km);
                    if (km1) id1 = j0 + __builtin_ctzll(km1);
                } else {
                    id1 = j0 + __builtin_ctzll(km);
                }
                seen += km1 ? 2 : 1;
            }
            out += __popcll(km);
            tie += __popcll(eqm);
        }
        // The row's plan record, as k_plan_rows forms it from the lists, and
        // its share of its head's counts.
        if (rec_out && lane == 0) {
            const int lo = (int)max(start, (int64_t)0), hi = (int)min(start + kept, K);
            const int a = min(max(id0, 0), nb - 1), b = min(max(id1, 0), nb - 1);
            rec_out[r] = make_int4((int)r, lo, hi, a | (b << 16));
            const int hl = (int)(r / nb - h_first);
            atomicAdd(&s_hk[hl], (int32_t)kept);
            atomicAdd(&s_hn[hl], kept > 0 ? 1 : 0);
        }
    }
    if (!rec_out) return;
    __syncthreads();
    if (tid < kCompactRows && h_first + tid < H && (s_hk[tid] || s_hn[tid])) {
        atomicAdd(&head_counts[h_first + tid], s_hk[tid]);
        atomicAdd(&head_counts[H + h_first + tid], s_hn[tid]);
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
// The select of one head by its 1024-thread workgroup (ph: the head's per
// scores), its state words written to out; returns the cut and the ties to
// keep to every thread.
struct CutTies {
    uint32_t cut;
    int64_t ties;
};

__device__ CutTies head_select(const float *__restrict__ ph, int64_t per, int64_t k_h,
                               uint32_t *__restrict__ out) {
    __shared__ uint32_t hist[kRadixBins];
    __shared__ uint32_t win[2];
    const int tid = threadIdx.x;
    if (k_h <= 0) {   // nothing kept: no score is above the cut, no tie is kept
        if (tid == 0) {
            out[SEL_CUT] = 0xFFFFFFFFu;
            out[SEL_ABOVE] = 0;
            out[SEL_TIES] = 0;
            out[SEL_K] = 0;
        }
        return CutTies{0xFFFFFFFFu, 0};
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
    return CutTies{prefix, remain};
}

__global__ __launch_bounds__(1024) void k_head_select(const float *__restrict__ p, int64_t per,
                                                      int64_t k_h,
                                                      uint32_t *__restrict__ hsel) {
    const int h = blockIdx.x;
    head_select(p + (int64_t)h * per, per, k_h, hsel + (int64_t)h * kHeadSelWords);
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
// h keeps the k_c largest of its L column masses.  One workgroup per head
// takes the head's select (as k_head_select, state words to hsel) and then
// writes its list: thread t owns a contiguous run of columns.  Ties at the
// cut are kept in ascending column order, so the kept set is the top-k_c
// under (value descending, index ascending) and the list comes out
// ascending.
__global__ __launch_bounds__(1024) void k_col_select(const float *__restrict__ c, int L,
                                                     uint32_t *__restrict__ hsel, int64_t k_c,
                                                     int32_t *__restrict__ cols) {
    const int h = blockIdx.x, tid = threadIdx.x;
    const float *ch = c + (int64_t)h * L;
    const CutTies ct = head_select(ch, L, k_c, hsel + (int64_t)h * kHeadSelWords);
    if (k_c <= 0) return;   // an empty list
    const uint32_t cut = ct.cut;
    const int64_t ties = ct.ties;
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
// Prepared (lists from the mask build, which also counted each head's kept
// blocks and non-empty rows) and H <= kPlanHeadsMax: one launch,
// k_plan_heads, one workgroup per head.  Every workgroup redoes the die part
// from the heads' counts (the same values in every workgroup: a few hundred
// LDS operations for a few dozen heads), takes its own head's two base
// positions, writes its share of the padding (workgroup 0 the meta words),
// then places its head's rows.  Otherwise two launches.  k_plan_assign, one
// workgroup: the heads' weights (from the mask build's counts, or from one
// pass over row_ptr: rows summed per lane, then per wave and head, into LDS
// counters), their ranks, the die assignment by one wave (one lane per die,
// the least-loaded open die by a cross-lane minimum), each head's first
// position among its die's non-empty rows and among its die's empty rows, the
// padding and the meta words (including the tag of the list the plan
// describes).  k_plan_rows, one wave per head: the head's row records, its
// rows by list length descending, ties by row id, with a stable counting sort
// (length histogram, descending bucket starts, ranks among equal lengths from
// wave ballots), written straight to the head's positions.

constexpr int kPlanThreads = 1024;
constexpr int kPlanHeadsThreads = 256;
constexpr int kPlanHeadsMax = 256;

// The heads' ranks by weight (descending, ties by head id) by every thread of
// the block, then the die assignment by wave 0: die_of[h], slot_of[h],
// die_list[x * cap_h + slot] (die x's heads in slot order), die_heads[x].
// Ends with the block synchronised.
__device__ void assign_dies(int H, bool narrow, int cap_h, const int64_t *weight, int32_t *order,
                            int32_t *die_of, int32_t *slot_of, int32_t *die_list,
                            int32_t *die_heads) {
    static_assert(kDies == 8, "the die loop covers 8 dies");
    const int tid = threadIdx.x, lane = tid & 63, nthreads = blockDim.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    for (int h = tid; h < H; h += nthreads) {
        int rank = 0;
        for (int o = 0; o < H; ++o)
            rank += (weight[o] > weight[h]) || (weight[o] == weight[h] && o < h);
        order[rank] = h;
    }
    __syncthreads();
    if (wave == 0 && narrow) {
        // Heads by rank, each to the least-loaded die with room (ties: lowest
        // die).  Every load is below 2^28 (known from nnz on the host), so
        // lane x < 8 holds die x's key load * 8 + x (~0 once the die is
        // full) and the least key over lanes 0..7 (three DPP minima) names
        // the die.  Lane a keeps the die and slot of the a-th head of each 64.
        uint32_t dload = 0;
        int dcnt = 0;
        for (int a0 = 0; a0 < H; a0 += 64) {
            const int my_h = a0 + lane < H ? order[a0 + lane] : 0;
            const uint32_t my_w = (uint32_t)weight[my_h];
            int my_die = 0, my_slot = 0;
            const int n = min(64, H - a0);
            for (int a = 0; a < n; ++a) {
                const uint32_t wh = (uint32_t)__builtin_amdgcn_readlane((int)my_w, a);
                int key = lane < kDies && dcnt < cap_h ? (int)((dload << 3) | (uint32_t)lane) : -1;
                key = (int)min((uint32_t)key, (uint32_t)__builtin_amdgcn_update_dpp(
                                                  -1, key, 0xB1, 0xF, 0xF, false));   // lane ^ 1
                key = (int)min((uint32_t)key, (uint32_t)__builtin_amdgcn_update_dpp(
                                                  -1, key, 0x4E, 0xF, 0xF, false));   // lane ^ 2
                key = (int)min((uint32_t)key, (uint32_t)__builtin_amdgcn_update_dpp(
                                                  -1, key, 0x141, 0xF, 0xF, false));  // 7 - lane
                const int best = __builtin_amdgcn_readfirstlane(key) & 7;
                const int slot = __builtin_amdgcn_readlane(dcnt, best);
                dload += lane == best ? wh : 0u;
                dcnt += lane == best ? 1 : 0;
                my_die = lane == a ? best : my_die;
                my_slot = lane == a ? slot : my_slot;
            }
            if (lane < n) {
                die_of[my_h] = my_die;
                slot_of[my_h] = my_slot;
                die_list[my_die * cap_h + my_slot] = my_h;
            }
        }
        if (lane < kDies) die_heads[lane] = dcnt;
    } else if (wave == 0) {
        // The same greedy with 64-bit loads in scalar registers; lane a of
        // the wave keeps the die and slot of the a-th head of each 64.
        int64_t load[kDies];
        int cnt[kDies];
#pragma unroll
        for (int x = 0; x < kDies; ++x) {
            load[x] = 0;
            cnt[x] = 0;
        }
        for (int a0 = 0; a0 < H; a0 += 64) {
            const int my_h = a0 + lane < H ? order[a0 + lane] : 0;
            const int64_t my_w = weight[my_h];
            int my_die = 0, my_slot = 0;
            const int n = min(64, H - a0);
            for (int a = 0; a < n; ++a) {
                const int64_t wh = (int64_t)(
                    ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(my_w >> 32), a) << 32) |
                    (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)my_w, a));
                int best = 0;
                int64_t best_load = INT64_MAX;
#pragma unroll
                for (int x = 0; x < kDies; ++x) {
                    const bool take = cnt[x] < cap_h && load[x] < best_load;
                    best_load = take ? load[x] : best_load;
                    best = take ? x : best;
                }
                int slot = 0;
#pragma unroll
                for (int x = 0; x < kDies; ++x) {
                    load[x] += x == best ? wh : 0;
                    slot = x == best ? cnt[x] : slot;
                    cnt[x] += x == best ? 1 : 0;
                }
                my_die = lane == a ? best : my_die;
                my_slot = lane == a ? slot : my_slot;
            }
            if (lane < n) {
                die_of[my_h] = my_die;
                slot_of[my_h] = my_slot;
                die_list[my_die * cap_h + my_slot] = my_h;
            }
        }
        if (lane < kDies) {
            int c = 0;
#pragma unroll
            for (int x = 0; x < kDies; ++x) c = x == lane ? cnt[x] : c;
            die_heads[lane] = c;
        }
    }
    __syncthreads();
}

// Head h's first position among its die's non-empty rows (x) and among its
// die's empty rows (y): a die's non-empty rows come first (heads in slot
// order), then its empty rows (same order).
__device__ int2 head_bases(int h, int nb, int cap, int cap_h, const int32_t *ne,
                           const int32_t *die_of, const int32_t *slot_of,
                           const int32_t *die_list, const int32_t *die_heads) {
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
    return make_int2(x * cap + ne_before, x * cap + ne_die + em_before);
}

// Padding records (row -1) at the positions past each die's heads, for
// positions first, first + stride, ...
__device__ void plan_padding(int nb, int cap, const int32_t *die_heads, int64_t first,
                             int64_t stride, int32_t *__restrict__ work,
                             int4 *__restrict__ work_rec) {
    for (int64_t q = first; q < (int64_t)kDies * cap; q += stride) {
        const int x = (int)(q / cap);
        if (q - (int64_t)x * cap >= (int64_t)die_heads[x] * nb) {
            work[q] = -1;
            work_rec[q] = make_int4(-1, 0, 0, 0);
        }
    }
}

// The meta words: positions per die, non-empty rows, and the tag of the list
// the plan describes (address, length, heads, blocks per row), with the
// stale-list check word cleared.
__device__ void plan_meta(int H, int nb, int cap, const int32_t *ne, const int32_t *list,
                          int64_t nnz, int32_t *__restrict__ meta) {
    int nonempty = 0;
    for (int h = 0; h < H; ++h) nonempty += ne[h];
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

// One wave: a head's rows (records rec[i] and clamped list lengths ln[i] of
// rows r0 + i, i < nb, in LDS; ne_cnt of them non-empty) by list length
// descending, ties by row id, to positions ne_base + rank (non-empty rows)
// and em_base + rank - ne_cnt (empty rows).  nx is LDS for nb + 1 counters.
__device__ void place_head_rows(int nb, int64_t r0, int ne_cnt, int64_t ne_base, int64_t em_base,
                                int32_t *nx, const int16_t *ln, const int4 *rec,
                                int32_t *__restrict__ work, int4 *__restrict__ work_rec) {
    const int lane = threadIdx.x & 63;
    const uint64_t lt = lanemask_lt();
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

__global__ __launch_bounds__(kPlanThreads) void k_plan_assign(const int32_t *__restrict__ row_ptr,
                                                              const int32_t *list, int64_t nnz,
                                                              int H, int nb, int steps_per_block,
                                                              bool narrow,
                                                              const int32_t *head_counts,
                                                              int32_t *__restrict__ head_base,
                                                              int32_t *__restrict__ work,
                                                              int4 *__restrict__ work_rec,
                                                              int32_t *__restrict__ meta) {
    __shared__ int64_t weight[kMaxHeads];
    __shared__ int32_t ne[kMaxHeads];
    __shared__ int32_t order[kMaxHeads];
    __shared__ int32_t die_of[kMaxHeads], slot_of[kMaxHeads];
    __shared__ int32_t die_list[kDies * kMaxHeads];
    __shared__ int32_t die_heads[kDies];
    const int tid = threadIdx.x, lane = tid & 63;
    if (head_counts) {   // counted by the list launch
        for (int h = tid; h < H; h += kPlanThreads) {
            weight[h] = (int64_t)steps_per_block * head_counts[h] + 4 * (int64_t)head_counts[H + h];
            ne[h] = head_counts[H + h];
        }
    } else {
        // Per head: rows that keep a block and blocks kept.  Thread t reads
        // the bounds of rows 4u .. 4u + 3, u = t, t + 1024, ..., all in one
        // batch per round; a wave's rows that fall in one head add with one
        // LDS atomic.
        __shared__ int32_t kept[kMaxHeads];
        for (int h = tid; h < H; h += kPlanThreads) ne[h] = kept[h] = 0;
        __syncthreads();
        const int rows = H * nb;
        for (int r0 = 0; r0 < rows; r0 += 4 * kPlanThreads) {
            const int r = r0 + 4 * tid;
            int v[5];
#pragma unroll
            for (int k = 0; k < 5; ++k) v[k] = row_ptr[min(r + k, rows)];
            // Rows of the thread's first row's head are summed here; rows of
            // later heads (only where a head boundary falls inside the four)
            // add one by one below.
            const int h_lo = min(r, rows - 1) / nb;
            int ne_lo = 0, kept_lo = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int len = v[k + 1] - v[k];
                if (r + k < rows && len > 0) {
                    if ((r + k) / nb == h_lo) {
                        ++ne_lo;
                        kept_lo += len;
                    } else {
                        atomicAdd(&ne[(r + k) / nb], 1);
                        atomicAdd(&kept[(r + k) / nb], len);
                    }
                }
            }
            // Lanes of the wave with the same head add with one atomic.
            uint64_t todo = __ballot(r < rows);
            while (todo) {
                const int leader = __builtin_ctzll(todo);
                const int hl = __builtin_amdgcn_readlane(h_lo, leader);
                const uint64_t same = __ballot(r < rows && h_lo == hl) & todo;
                int a = (same >> lane) & 1 ? ne_lo : 0, b = (same >> lane) & 1 ? kept_lo : 0;
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) {
                    a += __shfl_xor(a, o);
                    b += __shfl_xor(b, o);
                }
                if (lane == leader) {
                    atomicAdd(&ne[hl], a);
                    atomicAdd(&kept[hl], b);
                }
                todo &= ~same;
            }
        }
        __syncthreads();
        for (int h = tid; h < H; h += kPlanThreads)
            weight[h] = (int64_t)steps_per_block * kept[h] + 4 * (int64_t)ne[h];
    }
    __syncthreads();
    const int cap_h = min(H, (H + kDies - 1) / kDies + 2);
    const int cap = cap_h * nb;   // below 2^31: 8 * cap <= 8 * H * nb
    assign_dies(H, narrow, cap_h, weight, order, die_of, slot_of, die_list, die_heads);
    for (int h = tid; h < H; h += kPlanThreads) {
        const int2 b = head_bases(h, nb, cap, cap_h, ne, die_of, slot_of, die_list, die_heads);
        head_base[2 * h] = b.x;
        head_base[2 * h + 1] = b.y;
    }
    plan_padding(nb, cap, die_heads, tid, kPlanThreads, work, work_rec);
    if (tid == 0) plan_meta(H, nb, cap, ne, list, nnz, meta);
}

__global__ __launch_bounds__(64) void k_plan_rows(const int32_t *__restrict__ row_ptr,
                                                  const int32_t *__restrict__ col_idx,
                                                  int64_t nnz, int nb,
                                                  const int32_t *__restrict__ head_base,
                                                  const int4 *__restrict__ rec_in,
                                                  int32_t *__restrict__ work,
                                                  int4 *__restrict__ work_rec) {
    constexpr int kRowsPerLane = kMaxBlocks / 64;
    __shared__ int32_t nx[kMaxBlocks + 1];   // histogram, first staging row_ptr
    __shared__ int16_t ln[kMaxBlocks];
    __shared__ int4 rec[kMaxBlocks];
    const int lane = threadIdx.x, h = blockIdx.x;
    const int64_t r0 = (int64_t)h * nb;
    int my_ne = 0;
    if (rec_in) {   // records formed by the list launch
        for (int i = lane; i < nb; i += 64) {
            const int4 rc = rec_in[r0 + i];
            rec[i] = rc;
            const int len = rc.z - rc.y;
            ln[i] = (int16_t)min(max(len, 0), nb);
            my_ne += len > 0;
        }
    } else {
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
        for (int i = lane; i < nb; i += 64) {
            const int64_t len = (int64_t)nx[i + 1] - nx[i];
            ln[i] = (int16_t)min(max(len, (int64_t)0), (int64_t)nb);
            my_ne += len > 0;
        }
    }
    place_head_rows(nb, r0, wave_sum(my_ne), head_base[2 * h], head_base[2 * h + 1], nx, ln, rec,
                    work, work_rec);
}

// The whole plan in one launch from the mask build's records and head counts
// (H <= kPlanHeadsMax): workgroup h stages head h's records, redoes the die
// part, writes its share of the padding (workgroup 0 also the meta words)
// and places head h's rows, exactly as k_plan_assign then k_plan_rows do.
__global__ __launch_bounds__(kPlanHeadsThreads) void k_plan_heads(
    const int32_t *list, int64_t nnz, int H, int nb, int steps_per_block, bool narrow,
    const int32_t *__restrict__ head_counts, const int4 *__restrict__ rec_in,
    int32_t *__restrict__ work, int4 *__restrict__ work_rec, int32_t *__restrict__ meta) {
    __shared__ int64_t weight[kPlanHeadsMax];
    __shared__ int32_t ne[kPlanHeadsMax];
    __shared__ int32_t order[kPlanHeadsMax];
    __shared__ int32_t die_of[kPlanHeadsMax], slot_of[kPlanHeadsMax];
    __shared__ int32_t die_list[kDies * kPlanHeadsMax];
    __shared__ int32_t die_heads[kDies];
    __shared__ int32_t nx[kMaxBlocks + 1];
    __shared__ int16_t ln[kMaxBlocks];
    __shared__ int4 rec[kMaxBlocks];
    const int tid = threadIdx.x, h = blockIdx.x;
    const int64_t r0 = (int64_t)h * nb;
    // The head's records and every head's counts, loads issued together.
    for (int i = tid; i < nb; i += kPlanHeadsThreads) {
        const int4 rc = rec_in[r0 + i];
        rec[i] = rc;
        ln[i] = (int16_t)min(max(rc.z - rc.y, 0), nb);
    }
    for (int x = tid; x < H; x += kPlanHeadsThreads) {
        weight[x] = (int64_t)steps_per_block * head_counts[x] + 4 * (int64_t)head_counts[H + x];
        ne[x] = head_counts[H + x];
    }
    __syncthreads();
    const int cap_h = min(H, (H + kDies - 1) / kDies + 2);
    const int cap = cap_h * nb;
    assign_dies(H, narrow, cap_h, weight, order, die_of, slot_of, die_list, die_heads);
    plan_padding(nb, cap, die_heads, (int64_t)h * kPlanHeadsThreads + tid,
                 (int64_t)gridDim.x * kPlanHeadsThreads, work, work_rec);
    if (h == 0 && tid == 0) plan_meta(H, nb, cap, ne, list, nnz, meta);
    if (tid >= 64) return;
    int my_ne = 0;
    for (int i = tid; i < nb; i += 64) my_ne += ln[i] > 0;
    const int2 b = head_bases(h, nb, cap, cap_h, ne, die_of, slot_of, die_list, die_heads);
    place_head_rows(nb, r0, wave_sum(my_ne), b.x, b.y, nx, ln, rec, work, work_rec);
}

}  // namespace

// ------------------------------------------------------------------ launches --
namespace {
// Every die load fits in 28 bits when the weight of the whole mask does (for
// a well-formed mask the list lengths add up to nnz; a malformed one only
// gets another valid assignment of heads to dies).
bool plan_narrow(const Dims &D, int64_t nnz) {
    return (int64_t)(D.B / 32) * nnz + 4 * D.rows() < ((int64_t)1 << 28);
}

template <int D>
void pool_launch(const Dims &Dm, const uint16_t *q, const uint16_t *k, float *qb, float *kb,
                 int64_t q_pairs, int64_t k_pairs, uint32_t *hist, uint32_t *sel, int64_t K,
                 hipStream_t s) {
    constexpr int PAIRS = pool_pairs<D>();
    const unsigned grid = (unsigned)((q_pairs + PAIRS - 1) / PAIRS + (k_pairs + PAIRS - 1) / PAIRS);
    if (Dm.B == 64)
        hipLaunchKernelGGL((k_pool<D, 64>), dim3(grid), dim3(256), 0, s, q, k, qb, kb, q_pairs,
                           k_pairs, hist, sel, K);
    else
        hipLaunchKernelGGL((k_pool<D, 128>), dim3(grid), dim3(256), 0, s, q, k, qb, kb, q_pairs,
                           k_pairs, hist, sel, K);
}
}  // namespace

hipError_t launch_pool(const Dims &D, const uint16_t *q, const uint16_t *k, float *qb, float *kb,
                       char *ws, const WsLayout &w, int64_t sel_init_K, hipStream_t s) {
    uint32_t *hist = sel_init_K >= 0 ? reinterpret_cast<uint32_t *>(ws + w.hist) : nullptr;
    uint32_t *sel = sel_init_K >= 0 ? reinterpret_cast<uint32_t *>(ws + w.sel) : nullptr;
    const int64_t kv_pairs = (int64_t)D.Hkv * D.nb;
    if (D.d == 128)
        pool_launch<128>(D, q, k, qb, kb, D.rows(), kv_pairs, hist, sel, sel_init_K, s);
    else
        pool_launch<64>(D, q, k, qb, kb, D.rows(), kv_pairs, hist, sel, sel_init_K, s);
    return hipGetLastError();
}

hipError_t launch_pool_q(const Dims &D, const uint16_t *q, float *qb, hipStream_t s) {
    if (D.d == 128)
        pool_launch<128>(D, q, nullptr, qb, nullptr, D.rows(), 0, nullptr, nullptr, 0, s);
    else
        pool_launch<64>(D, q, nullptr, qb, nullptr, D.rows(), 0, nullptr, nullptr, 0, s);
    return hipGetLastError();
}

hipError_t launch_col_select(const Dims &D, int64_t k_c, const float *c, char *ws,
                             const WsLayout &w, int32_t *cols, hipStream_t s) {
    uint32_t *hsel = reinterpret_cast<uint32_t *>(ws + w.hsel);
    hipLaunchKernelGGL(k_col_select, dim3(D.H), dim3(1024), 0, s, c, D.L, hsel, k_c, cols);
    return hipGetLastError();
}

hipError_t launch_scores(const Dims &D, const float *qb, const float *kb, float *p, float *copy,
                         char *ws, const WsLayout &w, bool first_digit, hipStream_t s) {
    uint32_t *hist0 = first_digit ? reinterpret_cast<uint32_t *>(ws + w.hist) : nullptr;
    const int tiles = (D.nb + kScoreRows - 1) / kScoreRows;
    const float sigma = (float)(1.0 / sqrt((double)D.d));
    dim3 grid((unsigned)(D.H * tiles));
    if (D.d == 128)
        hipLaunchKernelGGL(k_scores<128>, grid, dim3(kScoreThreads), 0, s, qb, kb, p, copy, D.nb,
                           D.G, sigma, hist0);
    else
        hipLaunchKernelGGL(k_scores<64>, grid, dim3(kScoreThreads), 0, s, qb, kb, p, copy, D.nb,
                           D.G, sigma, hist0);
    return hipGetLastError();
}

hipError_t launch_select(const Dims &D, int64_t K, const float *p, char *ws, const WsLayout &w,
                         int32_t *row_ptr, int32_t *col_idx, bool state_ready, bool plan_inputs,
                         hipStream_t s) {
    uint32_t *hist = reinterpret_cast<uint32_t *>(ws + w.hist);
    uint32_t *sel = reinterpret_cast<uint32_t *>(ws + w.sel);
    int32_t *gt = reinterpret_cast<int32_t *>(ws + w.gt);
    int32_t *eq = reinterpret_cast<int32_t *>(ws + w.eq);
    const int64_t n = D.n_scores(), rows = D.rows();
    // With state_ready the state is set and the first digit's histogram is
    // already counted (pool and score launches of the mask build).
    if (!state_ready) hipLaunchKernelGGL(k_select_init, dim3(1), dim3(1024), 0, s, hist, sel, K);
    if (K > 0) {
        int64_t g = (n / 4 + kRadixThreads - 1) / kRadixThreads;
        g = g < 1 ? 1 : (g > 256 ? 256 : g);
        for (int pass = state_ready ? 1 : 0; pass < 3; ++pass)
            hipLaunchKernelGGL(k_radix_pass, dim3((unsigned)g), dim3(kRadixThreads), 0, s, p, n,
                               sel, hist, pass);
    }
    // The last digit step (the cut) is taken by the count launch.
    int32_t *agg = reinterpret_cast<int32_t *>(ws + w.row_agg);
    const unsigned row_grid = (unsigned)((rows + kCompactRows - 1) / kCompactRows);
    int32_t *head_counts =
        plan_inputs ? reinterpret_cast<int32_t *>(ws + w.head_counts) : nullptr;
    hipLaunchKernelGGL(k_row_count, dim3(row_grid), dim3(1024), 0, s, p, D.nb, rows, rows, sel,
                       K > 0 ? hist + 2 * kRadixBins : nullptr, gt, eq, agg, head_counts,
                       2 * D.H);
    hipLaunchKernelGGL(k_row_emit, dim3(row_grid), dim3(1024), 0, s, p, D.nb, rows, K, sel, gt, eq,
                       agg, row_ptr, col_idx,
                       plan_inputs ? reinterpret_cast<int4 *>(ws + w.row_rec) : nullptr,
                       head_counts, D.H);
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
                       dim3(1024), 0, s, p, D.nb, rows, (int64_t)D.nb, hsel, nullptr, gt, eq,
                       nullptr, nullptr, 0);
    hipLaunchKernelGGL(k_head_ties, dim3(D.H), dim3(1024), 0, s, gt, eq, D.nb, hsel, tie_base);
    hipLaunchKernelGGL(k_kept_scan, dim3(1), dim3(1024), 0, s, gt, rows, row_ptr);
    hipLaunchKernelGGL(k_row_scatter, dim3(row_grid), dim3(256), 0, s, p, D.nb, rows,
                       (int64_t)D.nb, k_h * D.H, hsel, tie_base, row_ptr, col_idx);
    return hipGetLastError();
}

hipError_t launch_plan(const Dims &D, const int32_t *row_ptr, const int32_t *col_idx,
                       int64_t nnz, char *ws, const WsLayout &w, bool prepared, hipStream_t s) {
    int32_t *work = reinterpret_cast<int32_t *>(ws + w.work);
    int4 *work_rec = reinterpret_cast<int4 *>(ws + w.work_rec);
    int32_t *meta = reinterpret_cast<int32_t *>(ws + w.work_meta);
    int32_t *head_base = reinterpret_cast<int32_t *>(ws + w.plan_head_base);
    const int32_t *head_counts =
        prepared ? reinterpret_cast<const int32_t *>(ws + w.head_counts) : nullptr;
    const int4 *rec_in = prepared ? reinterpret_cast<const int4 *>(ws + w.row_rec) : nullptr;
    if (prepared && D.H <= kPlanHeadsMax) {
        hipLaunchKernelGGL(k_plan_heads, dim3(D.H), dim3(kPlanHeadsThreads), 0, s, col_idx, nnz,
                           D.H, D.nb, D.B / 32, plan_narrow(D, nnz), head_counts, rec_in, work,
                           work_rec, meta);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_plan_assign, dim3(1), dim3(kPlanThreads), 0, s, row_ptr, col_idx, nnz,
                       D.H, D.nb, D.B / 32, plan_narrow(D, nnz), head_counts, head_base, work,
                       work_rec, meta);
    hipLaunchKernelGGL(k_plan_rows, dim3(D.H), dim3(64), 0, s, row_ptr, col_idx, nnz, D.nb,
                       head_base, rec_in, work, work_rec);
    return hipGetLastError();
}

}  // namespace sd
