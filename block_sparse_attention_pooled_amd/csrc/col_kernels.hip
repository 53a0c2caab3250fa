// Column masses for the column-sparse variant.
//
// "PulseCol" (abstract) replaces block sparsity with column sparsity: a head
// keeps individual key columns, found at an early denoising step and
// refreshed at a few intermediate ones.  How columns are scored is not on the
// page; the reading here mirrors the block path's pooled scoring ("BA-Att",
// abstract: selection in a block-wise pre-downsampled space):
//     c[h,u] = (1/nb) * sum_i softmax_u(qb[h,i] . k_u / sqrt(d))
// over all L keys u of key head h / (H/Hkv), where qb[h,i] is the mean of
// query block i rounded to bf16 (the matrix-core input).  c estimates the
// share of head h's attention that lands on key u; each head's row sums to 1.
//
// Pass 1 (k_col_stats): one workgroup per (head, 32 pooled queries), eight
// waves splitting the keys; scores transposed (S^T = K . Qb^T, lane = pooled
// query) so each lane keeps its query's running max and normaliser in
// registers; the waves' states are merged in wave order.  Pass 2
// (k_col_mass): one wave per 32 keys, scores untransposed (S = Qb . K^T, lane
// = key), so each lane adds its key's probabilities over the 16 pooled queries
// it holds, walking all pooled queries of the head in order.  Both passes use
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation; every sum is in a fixed
// order, so the result is deterministic.
#include "common.h"

namespace sd {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kColChunk = 32;     // keys per score tile
constexpr int kStatWaves = 8;     // waves splitting the keys in pass 1
constexpr int kMassWaves = 4;     // 32-key chunks per workgroup in pass 2

// Pooled-query fragment: 8 consecutive fp32 dims rounded to bf16 (RNE); a
// query past the head's last block is zero.
__device__ __forceinline__ bf16x8 pooled_frag(const float *p, bool valid) {
    bf16x8 r;
    if (valid) {
        const float4 a = *reinterpret_cast<const float4 *>(p);
        const float4 b = *reinterpret_cast<const float4 *>(p + 4);
        r[0] = (__bf16)a.x;
        r[1] = (__bf16)a.y;
        r[2] = (__bf16)a.z;
        r[3] = (__bf16)a.w;
        r[4] = (__bf16)b.x;
        r[5] = (__bf16)b.y;
        r[6] = (__bf16)b.z;
        r[7] = (__bf16)b.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = (__bf16)0.0f;
    }
    return r;
}

template <int D>
__global__ __launch_bounds__(kStatWaves * 64) void k_col_stats(
    const float *__restrict__ qb, const uint16_t *__restrict__ k, float2 *__restrict__ stats,
    int L, int nb, int G, float scale_log2) {
    constexpr int KS = D / 16;
    __shared__ float2 part[kStatWaves][32];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, hh = lane >> 5;
    const int tiles = (nb + 31) / 32;
    const int h = blockIdx.x / tiles, tile = blockIdx.x % tiles, g = h / G;
    const int r = tile * 32 + col;
    const bool valid = r < nb;

    bf16x8 qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
        qf[s] = pooled_frag(qb + ((int64_t)h * nb + (valid ? r : 0)) * D + 16 * s + 8 * hh, valid);
    const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(k + (int64_t)g * L * D), 0, L * D * 2, 0x00020000);
    const uint32_t k_voff = (uint32_t)(col * D * 2 + 16 * hh);
    auto load_k = [&](int c, bf16x8 (&kf)[KS]) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
            kf[s] = __builtin_bit_cast(
                bf16x8, __builtin_amdgcn_raw_buffer_load_b128(k_rsrc, k_voff,
                                                              c * kColChunk * D * 2 + 32 * s, 0));
    };
    // Running max m and sum l of 2^(s*scale - m) over this lane's keys (the
    // other 16 keys of each chunk are in lane ^ 32), log2 units.
    float m = -INFINITY, l = 0.0f;
    auto pass1 = [&](const bf16x8 (&kf)[KS]) {
        f32x16 sacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], sacc, 0, 0, 0);
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
    // This wave's chunks: wave, wave + 8, ...
    const int n_chunks = L / kColChunk;
    bf16x8 ka[KS], kb[KS];
    int c = wave;
    if (c < n_chunks) load_k(c, ka);
    for (; c < n_chunks; c += 2 * kStatWaves) {
        const int c1 = c + kStatWaves;
        if (c1 < n_chunks) load_k(c1, kb);
        pass1(ka);
        if (c1 < n_chunks) {
            if (c1 + kStatWaves < n_chunks) load_k(c1 + kStatWaves, ka);
            pass1(kb);
        }
    }
    if (l > 0.0f) {   // both lane halves of a query hold different keys
        const float m2 = __shfl_xor(m, 32), l2 = __shfl_xor(l, 32);
        const float mm = fmaxf(m, m2);
        l = l * __builtin_amdgcn_exp2f(m - mm) + l2 * __builtin_amdgcn_exp2f(m2 - mm);
        m = mm;
    }
    if (lane < 32) part[wave][lane] = make_float2(m, l);
    __syncthreads();
    if (wave == 0 && lane < 32 && valid) {
        float M = -INFINITY, S = 0.0f;
#pragma unroll
        for (int w = 0; w < kStatWaves; ++w) {
            const float2 p = part[w][lane];
            if (p.y > 0.0f) {   // a wave with no chunk holds (-inf, 0)
                const float mm = fmaxf(M, p.x);
                S = S * __builtin_amdgcn_exp2f(M - mm) + p.y * __builtin_amdgcn_exp2f(p.x - mm);
                M = mm;
            }
        }
        stats[(int64_t)h * nb + r] = make_float2(M, S);
    }
}

template <int D>
__global__ __launch_bounds__(kMassWaves * 64) void k_col_mass(
    const float *__restrict__ qb, const uint16_t *__restrict__ k,
    const float2 *__restrict__ stats, float *__restrict__ c, int L, int nb, int G,
    float scale_log2) {
    constexpr int KS = D / 16;
    __shared__ float2 st[kMaxBlocks];   // per pooled query: max, 1 / normaliser
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, hh = lane >> 5;
    const int n_chunks = L / kColChunk;
    const int groups = (n_chunks + kMassWaves - 1) / kMassWaves;
    const int h = blockIdx.x / groups, grp = blockIdx.x % groups, g = h / G;
    for (int i = tid; i < nb; i += kMassWaves * 64) {
        const float2 s = stats[(int64_t)h * nb + i];
        st[i] = make_float2(s.x, 1.0f / s.y);
    }
    __syncthreads();
    const int chunk = grp * kMassWaves + wave;
    if (chunk >= n_chunks) return;
    const int key = chunk * kColChunk + col;

    // K^T fragments: lane column = key, dims 16*s + 8*hh.
    bf16x8 kf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
        kf[s] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4 *>(k + ((int64_t)g * L + key) * D + 16 * s +
                                                     8 * hh));
    float acc = 0.0f;
    const int tiles = (nb + 31) / 32;
    for (int t = 0; t < tiles; ++t) {
        const int r = t * 32 + col;
        const bool valid = r < nb;
        bf16x8 qf[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s)
            qf[s] = pooled_frag(qb + ((int64_t)h * nb + (valid ? r : 0)) * D + 16 * s + 8 * hh,
                                valid);
        f32x16 sacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[s], kf[s], sacc, 0, 0, 0);
        // Accumulator i of this lane is pooled query 8*(i/4) + 4*hh + i%4 of the tile.
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int q = t * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
            if (q < nb) {
                const float2 s = st[q];
                acc += __builtin_amdgcn_exp2f(fmaf(sacc[i], scale_log2, -s.x)) * s.y;
            }
        }
    }
    acc += __shfl_xor(acc, 32);
    if (lane < 32) c[(int64_t)h * L + key] = acc * (1.0f / (float)nb);
}

template <int D>
hipError_t launch_col_scores_t(const Dims &Dm, const float *qb, const uint16_t *k,
                               float2 *stats, float *c, hipStream_t s) {
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    const int tiles = (Dm.nb + 31) / 32;
    hipLaunchKernelGGL((k_col_stats<D>), dim3((unsigned)(Dm.H * tiles)), dim3(kStatWaves * 64), 0,
                       s, qb, k, stats, Dm.L, Dm.nb, Dm.G, scale_log2);
    const int n_chunks = Dm.L / kColChunk;
    const int groups = (n_chunks + kMassWaves - 1) / kMassWaves;
    hipLaunchKernelGGL((k_col_mass<D>), dim3((unsigned)(Dm.H * groups)), dim3(kMassWaves * 64), 0,
                       s, qb, k, stats, c, Dm.L, Dm.nb, Dm.G, scale_log2);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_col_scores(const Dims &D, const float *qb, const uint16_t *k, char *ws,
                             const WsLayout &w, float *c, hipStream_t s) {
    float2 *stats = reinterpret_cast<float2 *>(ws + w.col_stats);
    if (D.d == 128) return launch_col_scores_t<128>(D, qb, k, stats, c, s);
    return launch_col_scores_t<64>(D, qb, k, stats, c, s);
}

}  // namespace sd
