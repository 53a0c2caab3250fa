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
// Pass 1 (k_col_part): one workgroup per (head, four tiles of 32 pooled
// queries, 1024-key split); four waves per tile, each walking one quarter of
// the split's 32-key chunks in ascending order (16 waves per workgroup hide
// the chunk loads' latency).  The four waves of a quarter share each chunk
// through LDS (one coalesced buffer->LDS copy of its 32 rows), so a head's K
// is read once per four tiles.  Scores are transposed (S^T = K . Qb^T, lane =
// pooled query) so each lane keeps its query's running max and normaliser in
// registers; the quarters' states are merged in quarter order and written per
// split.  Split-0 workgroups also write their tiles' bf16 query fragments in
// MFMA lane order.  k_col_merge folds the splits in order.
// Pass 2 (k_col_mass): one wave per 32 keys, scores untransposed (S = Qb .
// K^T, lane = key), so each lane adds its key's probabilities over the 16
// pooled queries it holds, walking the head's query tiles in order with the
// next tile's fragments in flight; its K chunk reaches LDS through coalesced
// buffer->LDS loads.  Both passes use v_mfma_f32_32x32x16_bf16 with fp32
// accumulation; every sum is in a fixed order, so the result is
// deterministic.
#include "common.h"

namespace sd {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kColChunk = 32;       // keys per score tile
constexpr int kPartTiles = 4;       // tiles of 32 pooled queries per pass-1 workgroup
constexpr int kPartParts = 4;       // waves per tile, each over a quarter of the split
constexpr int kPartChunks = 32;     // 32-key chunks per split: 1024 keys
constexpr int kMassWaves = 4;       // 32-key chunks per pass-2 workgroup

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

// 16 bytes per lane from a buffer straight into LDS (64 lanes -> 1 KiB
// contiguous at `lds`).
__device__ __forceinline__ void col_load_lds16(__amdgpu_buffer_rsrc_t rsrc, uint16_t *lds,
                                               uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)lds,
                                             16, voff, soff, 0, 0);
}

// Merge (m2, l2) into (m, l): maxima in log2 units, l sums of 2^(s - m).
__device__ __forceinline__ void merge_state(float &m, float &l, float m2, float l2) {
    if (l2 > 0.0f) {   // an empty state is (-inf, 0)
        const float mm = fmaxf(m, m2);
        l = l * __builtin_amdgcn_exp2f(m - mm) + l2 * __builtin_amdgcn_exp2f(m2 - mm);
        m = mm;
    }
}

template <int D>
__global__ __launch_bounds__(kPartTiles * kPartParts * 64) void k_col_part(
    const float *__restrict__ qb, const uint16_t *__restrict__ k, float2 *__restrict__ part,
    uint4 *__restrict__ q16, int L, int nb, int G, int splits, float scale_log2) {
    constexpr int KS = D / 16;
    constexpr int NSEG = D / 8;                 // 16-byte segments per K row
    constexpr int RPL = 64 / NSEG;              // rows per 1 KiB load
    constexpr int LOADS = kColChunk / RPL;      // 1 KiB loads per chunk
    constexpr int WL = LOADS / kPartTiles;      // of which each wave of a quarter issues WL
    constexpr int CHUNK = kColChunk * D;        // bf16 elements of a chunk
    static_assert(LOADS % kPartTiles == 0, "a chunk's loads split evenly over a quarter's waves");
    __shared__ float2 wstate[kPartParts - 1][kPartTiles][32];   // quarters 1.. states
    // Two chunk stages per quarter: the next chunk lands while this one is used.
    __shared__ __attribute__((aligned(16))) uint16_t ring[kPartParts][2][CHUNK];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int slot = wave % kPartTiles, part_i = wave / kPartTiles;
    const int col = lane & 31, hh = lane >> 5;
    const int tiles = (nb + 31) / 32;
    const int groups = (tiles + kPartTiles - 1) / kPartTiles;
    const int split = blockIdx.x % splits;
    const int hg = blockIdx.x / splits;
    const int h = hg / groups, tile = (hg % groups) * kPartTiles + slot, g = h / G;
    // The head's last group can have fewer tiles: those waves still load
    // their share of each chunk but compute nothing.
    const bool active = tile < tiles;
    const int ht = h * tiles + (active ? tile : 0);
    const int r = tile * 32 + col;
    const bool valid = active && r < nb;

    // The tile's bf16 query fragments: quarter 0 forms them from the fp32
    // pooled means and shares them through LDS with the other quarters.
    __shared__ uint4 qshare[kPartTiles][KS][64];
    bf16x8 qf[KS];
    if (part_i == 0) {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qf[s] = pooled_frag(qb + ((int64_t)h * nb + (valid ? r : 0)) * D + 16 * s + 8 * hh,
                                valid);
            qshare[slot][s][lane] = __builtin_bit_cast(uint4, qf[s]);
        }
        if (split == 0 && active) {
            uint4 *dst = q16 + (int64_t)ht * KS * 64 + lane;
#pragma unroll
            for (int s = 0; s < KS; ++s) dst[s * 64] = __builtin_bit_cast(uint4, qf[s]);
        }
    }
    __syncthreads();
    if (part_i != 0) {
#pragma unroll
        for (int s = 0; s < KS; ++s) qf[s] = __builtin_bit_cast(bf16x8, qshare[slot][s][lane]);
    }
    // A chunk is 32 consecutive key rows, contiguous in memory: load t of the
    // chunk copies rows RPL*t .. +RPL (1 KiB) into the stage, segment x of row
    // w stored at x ^ (w % NSEG), so the fragment reads below hit distinct
    // banks.  Reads past the key head return zeros.
    const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(k + (int64_t)g * L * D), 0, L * D * 2, 0x00020000);
    const int r_in = lane / NSEG, sp = lane % NSEG;
    uint32_t voff[WL];
#pragma unroll
    for (int tt = 0; tt < WL; ++tt) {
        const int w = (slot * WL + tt) * RPL + r_in;
        voff[tt] = (uint32_t)(r_in * D * 2 + 16 * (sp ^ (w % NSEG)));
    }
    auto issue = [&](int c, uint16_t *dst) {
#pragma unroll
        for (int tt = 0; tt < WL; ++tt) {
            const int t = slot * WL + tt;
            col_load_lds16(k_rsrc, dst + t * 512, voff[tt],
                           (uint32_t)(c * kColChunk * D * 2 + t * RPL * D * 2));
        }
    };
    // K as the A operand: lane row = key col, dims 16*s + 8*hh.
    auto read = [&](const uint16_t *kt, bf16x8 (&kf)[KS]) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
            kf[s] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const uint4 *>(kt + col * D +
                                                        8 * ((2 * s + hh) ^ (col % NSEG))));
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
        for (int i = 0; i < 16; ++i)
            acc += __builtin_amdgcn_exp2f(fmaf(sacc[i], scale_log2, -m_new));
        l = l * __builtin_amdgcn_exp2f(m - m_new) + acc;
        m = m_new;
    };
    // This quarter's chunks in ascending order.  Every wave runs all steps (the
    // barriers are common); a step reads its chunk, then starts the next
    // chunk's loads into the other stage (read one step earlier), then forms
    // the scores.  s_waitcnt fields: vmcnt 3:0 and 15:14, expcnt 6:4, lgkmcnt
    // 11:8; 0x0070 waits for every load and LDS access.
    constexpr int kPartLen = kPartChunks / kPartParts;
    const int n_chunks = L / kColChunk;
    const int c0 = split * kPartChunks + part_i * kPartLen;
    const int c_lim = min(n_chunks, c0 + kPartLen);
    if (c0 < c_lim) issue(c0, ring[part_i][0]);
    for (int j = 0; j < kPartLen; ++j) {
        __builtin_amdgcn_s_waitcnt(0x0070);
        __syncthreads();
        const int cj = c0 + j;
        bf16x8 kf[KS];
        if (active && cj < c_lim) read(ring[part_i][j & 1], kf);
        if (cj + 1 < c_lim) issue(cj + 1, ring[part_i][(j + 1) & 1]);
        if (active && cj < c_lim) pass1(kf);
    }
    merge_state(m, l, __shfl_xor(m, 32), __shfl_xor(l, 32));
    if (part_i > 0 && lane < 32) wstate[part_i - 1][slot][lane] = make_float2(m, l);
    __syncthreads();
    if (part_i == 0 && lane < 32 && valid) {
#pragma unroll
        for (int q = 0; q < kPartParts - 1; ++q)
            merge_state(m, l, wstate[q][slot][lane].x, wstate[q][slot][lane].y);
        part[((int64_t)h * nb + r) * splits + split] = make_float2(m, l);
    }
}

// Per pooled query: fold the key splits in split order -> (max, 1 / normaliser).
__global__ __launch_bounds__(256) void k_col_merge(const float2 *__restrict__ part,
                                                   float2 *__restrict__ stats, int64_t rows,
                                                   int splits) {
    const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (x >= rows) return;
    float M = -INFINITY, S = 0.0f;
    for (int s = 0; s < splits; ++s) {
        const float2 p = part[x * splits + s];
        merge_state(M, S, p.x, p.y);
    }
    stats[x] = make_float2(M, 1.0f / S);
}

template <int D>
__global__ __launch_bounds__(kMassWaves * 64) void k_col_mass(
    const uint4 *__restrict__ q16, const uint16_t *__restrict__ k,
    const float2 *__restrict__ stats, float *__restrict__ c, int L, int nb, int G,
    float scale_log2) {
    constexpr int KS = D / 16;
    constexpr int NSEG = D / 8;                 // 16-byte segments per K row
    constexpr int RPL = 64 / NSEG;              // rows per 1 KiB load
    constexpr int LOADS = kColChunk / RPL;      // 1 KiB loads per chunk
    constexpr int CHUNK = kColChunk * D;        // bf16 elements of a chunk
    __shared__ float2 st[kMaxBlocks];   // per pooled query: max, 1 / normaliser
    __shared__ __attribute__((aligned(16))) uint16_t kl[kMassWaves][CHUNK];   // each wave's chunk
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, hh = lane >> 5;
    const int n_chunks = L / kColChunk;
    const int groups = (n_chunks + kMassWaves - 1) / kMassWaves;
    const int h = blockIdx.x / groups, grp = blockIdx.x % groups, g = h / G;
    const int chunk = grp * kMassWaves + wave;
    // This wave's chunk (32 contiguous key rows) into its own stage with
    // coalesced buffer->LDS loads, segment x of row w stored at x ^ (w %
    // NSEG); reads past the key head return zeros.
    const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(k + (int64_t)g * L * D), 0, L * D * 2, 0x00020000);
    const int r_in = lane / NSEG, sp = lane % NSEG;
    if (chunk < n_chunks) {
#pragma unroll
        for (int t = 0; t < LOADS; ++t)
            col_load_lds16(k_rsrc, kl[wave] + t * 512,
                           (uint32_t)(r_in * D * 2 + 16 * (sp ^ ((t * RPL + r_in) % NSEG))),
                           (uint32_t)(chunk * kColChunk * D * 2 + t * RPL * D * 2));
    }
    for (int i = tid; i < nb; i += kMassWaves * 64) st[i] = stats[(int64_t)h * nb + i];
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt 0, lgkmcnt 0: the chunk and the stats
    __syncthreads();
    if (chunk >= n_chunks) return;
    const int key = chunk * kColChunk + col;

    // K^T fragments: lane column = key, dims 16*s + 8*hh.
    bf16x8 kf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
        kf[s] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4 *>(kl[wave] + col * D +
                                                    8 * ((2 * s + hh) ^ (col % NSEG))));
    // Query fragments of tile t, as pass 1 left them (lane order).
    const int tiles = (nb + 31) / 32;
    const uint4 *qh = q16 + (int64_t)h * tiles * KS * 64 + lane;
    auto load_q = [&](int t, bf16x8 (&qf)[KS]) {
#pragma unroll
        for (int s = 0; s < KS; ++s) qf[s] = __builtin_bit_cast(bf16x8, qh[(t * KS + s) * 64]);
    };
    float acc = 0.0f;
    auto tile_mass = [&](int t, const bf16x8 (&qf)[KS]) {
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
                const float2 sq = st[q];
                acc += __builtin_amdgcn_exp2f(fmaf(sacc[i], scale_log2, -sq.x)) * sq.y;
            }
        }
    };
    bf16x8 qa[KS], qb2[KS];
    load_q(0, qa);
    for (int t = 0; t < tiles; t += 2) {
        if (t + 1 < tiles) load_q(t + 1, qb2);
        tile_mass(t, qa);
        if (t + 1 < tiles) {
            if (t + 2 < tiles) load_q(t + 2, qa);
            tile_mass(t + 1, qb2);
        }
    }
    acc += __shfl_xor(acc, 32);
    if (lane < 32) c[(int64_t)h * L + key] = acc * (1.0f / (float)nb);
}

template <int D>
hipError_t launch_col_scores_t(const Dims &Dm, const float *qb, const uint16_t *k, char *ws,
                               const WsLayout &w, float *c, hipStream_t s) {
    float2 *stats = reinterpret_cast<float2 *>(ws + w.col_stats);
    float2 *part = reinterpret_cast<float2 *>(ws + w.col_part);
    uint4 *q16 = reinterpret_cast<uint4 *>(ws + w.col_q16);
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    const int tiles = (Dm.nb + 31) / 32;
    const int splits = (int)Dm.col_splits();
    const int tile_groups = (tiles + kPartTiles - 1) / kPartTiles;
    hipLaunchKernelGGL((k_col_part<D>), dim3((unsigned)(Dm.H * tile_groups * splits)),
                       dim3(kPartTiles * kPartParts * 64), 0, s, qb, k, part, q16, Dm.L, Dm.nb,
                       Dm.G, splits, scale_log2);
    hipLaunchKernelGGL(k_col_merge, dim3((unsigned)((Dm.rows() + 255) / 256)), dim3(256), 0, s,
                       part, stats, Dm.rows(), splits);
    const int n_chunks = Dm.L / kColChunk;
    const int groups = (n_chunks + kMassWaves - 1) / kMassWaves;
    hipLaunchKernelGGL((k_col_mass<D>), dim3((unsigned)(Dm.H * groups)), dim3(kMassWaves * 64), 0,
                       s, q16, k, stats, c, Dm.L, Dm.nb, Dm.G, scale_log2);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_col_scores(const Dims &D, const float *qb, const uint16_t *k, char *ws,
                             const WsLayout &w, float *c, hipStream_t s) {
    if (D.d == 128) return launch_col_scores_t<128>(D, qb, k, ws, w, c, s);
    return launch_col_scores_t<64>(D, qb, k, ws, w, c, s);
}

}  // namespace sd
