// Mask quality: the true block attention mass of the full softmax map, and
// the recall of a block mask against it.
//
// "Block Approximate Sparse Attention (BA-Att)" (abstract) compares block
// selection in the pooled, pre-downsampled space with the block map of the
// exact attention (post-downsampling); "Step-dLLM" (abstract) reuses one mask
// across a refresh interval.  Here:
//     A[h,i,j] = (1/B) * sum_{t in q-block i} sum_{u in k-block j} softmax_u(q_t . k_u / sqrt(d))
// over all L keys of key head h / (H/Hkv) (bidirectional), and the recall of
// a mask row is the sum of A[h,i,j] over its kept blocks j.  Each row of A
// sums to 1, so recall 1 means the kept blocks hold all of the row's
// attention.  A diagnostic, off the per-step path.
//
// Block mass kernel: one workgroup per (head, query block); one wave per 32
// query rows.  Scores are formed transposed (S^T = K . Q^T,
// v_mfma_f32_32x32x16_bf16, Q^T in registers, K fragments loaded straight
// into registers one chunk ahead), so each lane holds 16 of the 32 keys of one
// query column.  Pass 1 takes every query's exact max and normaliser over all
// keys (fp32, log2 units); pass 2 recomputes the scores and sums each 32-key
// chunk's probability over the wave's queries.  The waves' partial sums meet
// in LDS and are added in wave order, so the result is deterministic.
#include "common.h"

namespace sd {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMassChunk = 32;   // keys per score tile

template <int D, int BLK>
__global__ __launch_bounds__(BLK / 32 * 64) void k_block_mass(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, float *__restrict__ mass,
    int L, int nb, int G, int H, float scale_log2) {
    constexpr int WQ = BLK / 32;   // waves (32 query rows each)
    constexpr int KS = D / 16;
    __shared__ float part[WQ][kMaxBlocks];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, hh = lane >> 5;

    int row = blockIdx.x;
    if ((H & 7) == 0) {   // keep each head's rows on one XCD (round-robin dispatch)
        const int x = row & 7, kk = row >> 3;
        row = (x + 8 * (kk / nb)) * nb + kk % nb;
    }
    const int h = row / nb, blk = row % nb, g = h / G;
    const int64_t qbase = ((int64_t)h * L + (int64_t)blk * BLK + 32 * wave) * D;
    const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(k + (int64_t)g * L * D), 0, L * D * 2, 0x00020000);

    // Q^T fragments: lane holds query col, dims 16*s + 8*hh .. +8.
    bf16x8 qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
        qf[s] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4 *>(q + qbase + (int64_t)col * D + 16 * s + 8 * hh));
    // K fragments of chunk c: lane row = key col, dims 16*s + 8*hh.
    const uint32_t k_voff = (uint32_t)(col * D * 2 + 16 * hh);
    auto load_k = [&](int c, bf16x8 (&kf)[KS]) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
            kf[s] = __builtin_bit_cast(
                bf16x8, __builtin_amdgcn_raw_buffer_load_b128(k_rsrc, k_voff,
                                                              c * kMassChunk * D * 2 + 32 * s, 0));
    };
    auto scores = [&](const bf16x8 (&kf)[KS], f32x16 &sacc) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], sacc, 0, 0, 0);
    };

    const int n_chunks = L / kMassChunk;
    bf16x8 ka[KS], kb[KS];

    // Pass 1: per query column, running max m and sum l of 2^(s*scale - m)
    // over this lane's keys (the other 16 keys of each chunk are in lane ^ 32).
    float m = -INFINITY, l = 0.0f;
    auto pass1 = [&](const bf16x8 (&kf)[KS]) {
        f32x16 sacc;
        scores(kf, sacc);
        float cm = sacc[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) cm = fmaxf(cm, sacc[i]);
        const float m_new = fmaxf(m, cm * scale_log2);
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc += __builtin_amdgcn_exp2f(fmaf(sacc[i], scale_log2, -m_new));
        l = l * __builtin_amdgcn_exp2f(m - m_new) + acc;
        m = m_new;
    };
    load_k(0, ka);
    for (int c = 0; c < n_chunks; c += 2) {
        if (c + 1 < n_chunks) load_k(c + 1, kb);
        pass1(ka);
        if (c + 1 < n_chunks) {
            if (c + 2 < n_chunks) load_k(c + 2, ka);
            pass1(kb);
        }
    }
    {   // both lane halves of a column hold different keys
        const float m2 = __shfl_xor(m, 32), l2 = __shfl_xor(l, 32);
        const float mm = fmaxf(m, m2);
        l = l * __builtin_amdgcn_exp2f(m - mm) + l2 * __builtin_amdgcn_exp2f(m2 - mm);
        m = mm;
    }
    const float inv_l = 1.0f / l;

    // Pass 2: probability of each chunk, summed over this wave's 32 queries.
    auto pass2 = [&](const bf16x8 (&kf)[KS]) -> float {
        f32x16 sacc;
        scores(kf, sacc);
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc += __builtin_amdgcn_exp2f(fmaf(sacc[i], scale_log2, -m));
        float p = acc * inv_l;
        p += __shfl_xor(p, 32);
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) p += __shfl_xor(p, o);
        return p;   // the same in every lane
    };
    constexpr int CPB = BLK / kMassChunk;
    float blk_acc = 0.0f;
    auto add_chunk = [&](int c, float p) {
        blk_acc += p;
        if (c % CPB == CPB - 1) {
            if (lane == 0) part[wave][c / CPB] = blk_acc;
            blk_acc = 0.0f;
        }
    };
    load_k(0, ka);
    for (int c = 0; c < n_chunks; c += 2) {
        if (c + 1 < n_chunks) load_k(c + 1, kb);
        add_chunk(c, pass2(ka));
        if (c + 1 < n_chunks) {
            if (c + 2 < n_chunks) load_k(c + 2, ka);
            add_chunk(c + 1, pass2(kb));
        }
    }
    __syncthreads();
    float *arow = mass + (int64_t)row * nb;
    for (int j = tid; j < nb; j += WQ * 64) {
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < WQ; ++w) s += part[w][j];
        arow[j] = s * (1.0f / BLK);
    }
}

// Recall of a column mask (the column-sparse variant, "PulseCol" abstract):
// per row (head, query block), the mean over its query tokens of the full
// softmax probability on the head's kept key columns.  Same workgroup shape
// and pass 1 as k_block_mass (exact max and normaliser over all L keys); pass
// 2 walks only the kept columns, 32 list entries at a time, each lane
// gathering its key's K row, and entries past the list count nothing.
template <int D, int BLK>
__global__ __launch_bounds__(BLK / 32 * 64) void k_col_recall(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const int32_t *__restrict__ cols, int64_t k_c, float *__restrict__ recall, int L, int nb,
    int G, int H, float scale_log2) {
    constexpr int WQ = BLK / 32;
    constexpr int KS = D / 16;
    __shared__ float part[WQ];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, hh = lane >> 5;

    int row = blockIdx.x;
    if ((H & 7) == 0) {   // keep each head's rows on one XCD (round-robin dispatch)
        const int x = row & 7, kk = row >> 3;
        row = (x + 8 * (kk / nb)) * nb + kk % nb;
    }
    const int h = row / nb, blk = row % nb, g = h / G;
    const int64_t qbase = ((int64_t)h * L + (int64_t)blk * BLK + 32 * wave) * D;
    const uint16_t *kh = k + (int64_t)g * L * D;
    const __amdgpu_buffer_rsrc_t k_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)kh, 0, L * D * 2, 0x00020000);

    bf16x8 qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
        qf[s] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4 *>(q + qbase + (int64_t)col * D + 16 * s + 8 * hh));
    const uint32_t k_voff = (uint32_t)(col * D * 2 + 16 * hh);
    auto load_k = [&](int c, bf16x8 (&kf)[KS]) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
            kf[s] = __builtin_bit_cast(
                bf16x8, __builtin_amdgcn_raw_buffer_load_b128(k_rsrc, k_voff,
                                                              c * kMassChunk * D * 2 + 32 * s, 0));
    };
    auto scores = [&](const bf16x8 (&kf)[KS], f32x16 &sacc) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], sacc, 0, 0, 0);
    };

    // Pass 1: per query column, max m and sum l of 2^(s*scale - m) over all keys.
    const int n_chunks = L / kMassChunk;
    bf16x8 ka[KS], kb[KS];
    float m = -INFINITY, l = 0.0f;
    auto pass1 = [&](const bf16x8 (&kf)[KS]) {
        f32x16 sacc;
        scores(kf, sacc);
        float cm = sacc[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) cm = fmaxf(cm, sacc[i]);
        const float m_new = fmaxf(m, cm * scale_log2);
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc += __builtin_amdgcn_exp2f(fmaf(sacc[i], scale_log2, -m_new));
        l = l * __builtin_amdgcn_exp2f(m - m_new) + acc;
        m = m_new;
    };
    load_k(0, ka);
    for (int c = 0; c < n_chunks; c += 2) {
        if (c + 1 < n_chunks) load_k(c + 1, kb);
        pass1(ka);
        if (c + 1 < n_chunks) {
            if (c + 2 < n_chunks) load_k(c + 2, ka);
            pass1(kb);
        }
    }
    {
        const float m2 = __shfl_xor(m, 32), l2 = __shfl_xor(l, 32);
        const float mm = fmaxf(m, m2);
        l = l * __builtin_amdgcn_exp2f(m - mm) + l2 * __builtin_amdgcn_exp2f(m2 - mm);
        m = mm;
    }

    // Pass 2: the kept columns.  Lane row col of chunk c is list entry 32*c + col.
    const int32_t *ch = cols + (int64_t)h * k_c;
    const int n_cc = (int)((k_c + kMassChunk - 1) / kMassChunk);
    auto load_kc = [&](int c, bf16x8 (&kf)[KS]) {
        const int64_t a = (int64_t)c * kMassChunk + col;
        int tok = a < k_c ? ch[a] : 0;
        tok = min(max(tok, 0), L - 1);
#pragma unroll
        for (int s = 0; s < KS; ++s)
            kf[s] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const uint4 *>(kh + (int64_t)tok * D + 16 * s + 8 * hh));
    };
    float acc = 0.0f;
    auto pass2 = [&](int c, const bf16x8 (&kf)[KS]) {
        f32x16 sacc;
        scores(kf, sacc);
        // Accumulator i of this lane is key 8*(i/4) + 4*hh + i%4 of the chunk.
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if ((int64_t)c * kMassChunk + 8 * (i >> 2) + 4 * hh + (i & 3) < k_c)
                acc += __builtin_amdgcn_exp2f(fmaf(sacc[i], scale_log2, -m));
    };
    if (n_cc > 0) load_kc(0, ka);
    for (int c = 0; c < n_cc; c += 2) {
        if (c + 1 < n_cc) load_kc(c + 1, kb);
        pass2(c, ka);
        if (c + 1 < n_cc) {
            if (c + 2 < n_cc) load_kc(c + 2, ka);
            pass2(c + 1, kb);
        }
    }
    float p = acc / l;
    p += __shfl_xor(p, 32);
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) p += __shfl_xor(p, o);
    if (lane == 0) part[wave] = p;
    __syncthreads();
    if (tid == 0) {
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < WQ; ++w) s += part[w];
        recall[row] = s * (1.0f / BLK);
    }
}

template <int D, int BLK>
hipError_t launch_col_recall_t(const Dims &Dm, const uint16_t *q, const uint16_t *k,
                               const int32_t *cols, int64_t k_c, float *recall, hipStream_t s) {
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    hipLaunchKernelGGL((k_col_recall<D, BLK>), dim3((unsigned)Dm.rows()), dim3(BLK / 32 * 64), 0,
                       s, q, k, cols, k_c, recall, Dm.L, Dm.nb, Dm.G, Dm.H, scale_log2);
    return hipGetLastError();
}

// One wave per row: the mass on the row's kept blocks.  List positions at or
// past nnz are not read; block ids outside [0, nb) add nothing.
__global__ __launch_bounds__(256) void k_mask_recall(const float *__restrict__ mass, int64_t rows,
                                                     int nb, const int32_t *__restrict__ row_ptr,
                                                     const int32_t *__restrict__ col_idx,
                                                     int64_t nnz, float *__restrict__ recall) {
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;
    const int lane = threadIdx.x & 63;
    const int64_t e0 = max((int64_t)row_ptr[r], (int64_t)0);
    const int64_t e1 = min((int64_t)row_ptr[r + 1], nnz);
    float acc = 0.0f;
    for (int64_t e = e0 + lane; e < e1; e += 64) {
        const int j = col_idx[e];
        if (j >= 0 && j < nb) acc += mass[r * nb + j];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) recall[r] = acc;
}

template <int D, int BLK>
hipError_t launch_mass_t(const Dims &Dm, const uint16_t *q, const uint16_t *k, float *mass,
                         hipStream_t s) {
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    hipLaunchKernelGGL((k_block_mass<D, BLK>), dim3((unsigned)Dm.rows()), dim3(BLK / 32 * 64), 0,
                       s, q, k, mass, Dm.L, Dm.nb, Dm.G, Dm.H, scale_log2);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_block_mass(const Dims &D, const uint16_t *q, const uint16_t *k, float *mass,
                             hipStream_t s) {
    if (D.d == 128 && D.B == 64) return launch_mass_t<128, 64>(D, q, k, mass, s);
    if (D.d == 128 && D.B == 128) return launch_mass_t<128, 128>(D, q, k, mass, s);
    if (D.d == 64 && D.B == 64) return launch_mass_t<64, 64>(D, q, k, mass, s);
    return launch_mass_t<64, 128>(D, q, k, mass, s);
}

hipError_t launch_col_recall(const Dims &D, const uint16_t *q, const uint16_t *k,
                             const int32_t *cols, int64_t k_c, float *recall, hipStream_t s) {
    if (D.d == 128 && D.B == 64) return launch_col_recall_t<128, 64>(D, q, k, cols, k_c, recall, s);
    if (D.d == 128 && D.B == 128)
        return launch_col_recall_t<128, 128>(D, q, k, cols, k_c, recall, s);
    if (D.d == 64 && D.B == 64) return launch_col_recall_t<64, 64>(D, q, k, cols, k_c, recall, s);
    return launch_col_recall_t<64, 128>(D, q, k, cols, k_c, recall, s);
}

hipError_t launch_mask_recall(const Dims &D, const float *mass, const int32_t *row_ptr,
                              const int32_t *col_idx, int64_t nnz, float *recall,
                              hipStream_t s) {
    const int64_t rows = D.rows();
    hipLaunchKernelGGL(k_mask_recall, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, mass,
                       rows, D.nb, row_ptr, col_idx, nnz, recall);
    return hipGetLastError();
}

}  // namespace sd
