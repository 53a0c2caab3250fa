// Block-sparse and dense bidirectional attention on gfx950 MFMA.
//
// Method: the fused block-sparse attention kernel of "Step-dLLM: Adaptive
// Step-aware Sparse Attention for Efficient Diffusion LLM Inference"
// (abstract), measured against dense attention ("dense FlashAttention").
// For every token t of query block i in head h:
//     o_t = sum_u softmax_u(q_t . k_u / sqrt(d)) v_u
// over the tokens u of the key blocks kept for row (h, i), from key head
// h / (H/Hkv); the dense kernel keeps every block.  Attention is
// bidirectional (no causal mask).
//
// Design (one workgroup per (head, query block) row):
//  * A wave owns 64 query rows and half of every 64-token key chunk pair:
//    waves (wq, wk) with wq the 64-row query slice and wk in {0, 1} taking
//    alternate 32-token key chunks.  Each wave keeps its own online-softmax
//    state; the two halves are merged once per row.
//  * Scores are computed transposed, S^T = K . Q^T, with
//    v_mfma_f32_32x32x16_bf16: the key chunk is the A operand (straight 16-byte
//    global loads of K rows), Q^T the B operand (held in registers for the whole
//    row).  In the accumulator layout every lane then holds one query column,
//    so the softmax rescale of O^T is a per-lane scalar and the fp32 scores
//    convert in place into the B operand of O^T += V^T . P^T (the key order
//    inside a 16-wide k step is permuted consistently on both operands).
//  * V^T is the A operand of the second product; V rows are transposed into a
//    per-wave LDS tile (4 keys x 1 column per 8-byte store) in that same
//    permuted key order, then read back with 16-byte LDS loads.
//  * fp32 accumulation and softmax (exp2 with log2(e)/sqrt(d) folded in), bf16
//    round-to-nearest-even output.
#include "common.h"

namespace sd {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChunk = 32;          // keys per wave step
constexpr int kVtStride = 40;       // bf16 per V^T row in LDS (32 keys + pad)

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t *p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(p));
}

__device__ __forceinline__ uint16_t bf16_rne(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

template <int D, int BLK, bool DENSE>
__global__ __launch_bounds__(128 * (BLK / 64)) void k_attn(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const int32_t *__restrict__ row_ptr,
    const int32_t *__restrict__ col_idx, const int32_t *__restrict__ work,
    uint16_t *__restrict__ o, int L, int nb, int G, int H, int n_idx, float scale_log2) {
    constexpr int WQ = BLK / 64;                // 64-row query slices per block
    constexpr int KS = D / 16;                  // k steps of the score product
    constexpr int MT = D / 32;                  // 32-row tiles of O^T
    constexpr int CHUNKS = BLK / kChunk;        // key chunks per key block
    constexpr int VT_ELEMS = D * kVtStride;     // per wave
    __shared__ __attribute__((aligned(16))) uint16_t vt_all[2 * WQ * VT_ELEMS];
    __shared__ float xchg[WQ][32][64];          // O^T exchange, one tile at a time
    __shared__ float ml[WQ][4][64];             // m, l exchange

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wq = wave >> 1, wk = wave & 1;
    const int col = lane & 31, hh = lane >> 5;

    // Row of this workgroup.
    int row;
    if (DENSE) {
        const int b = blockIdx.x;
        if ((H & 7) == 0) {   // keep each head's rows on one XCD (round-robin dispatch)
            const int x = b & 7, kk = b >> 3;
            row = (x + 8 * (kk / nb)) * nb + kk % nb;
        } else {
            row = b;
        }
    } else {
        row = work[blockIdx.x];
        if (row < 0 || row >= H * nb) return;   // malformed work order: nothing to do
    }
    const int h = row / nb, blk = row % nb, g = h / G;
    const int q0 = blk * BLK + 64 * wq;
    const int64_t qbase = ((int64_t)h * L + q0) * D;
    const int64_t kvbase = (int64_t)g * L * D;

    int e_begin = 0, e_end = nb;
    if (!DENSE) {
        e_begin = max(row_ptr[row], 0);
        e_end = min(row_ptr[row + 1], n_idx);
    }
    if (e_end <= e_begin) {     // no kept block: the row attends to nothing
        if (wk == 0) {
            uint4 z = make_uint4(0, 0, 0, 0);
            for (int x = lane; x < 64 * D / 8; x += 64)
                *reinterpret_cast<uint4 *>(o + qbase + (int64_t)x * 8) = z;
        }
        return;
    }

    // Q^T operand fragments: lane holds query col (32*nt + col), dims 16*s + 8*hh .. +8.
    bf16x8 qf[2][KS];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int s = 0; s < KS; ++s)
            qf[nt][s] = load_bf16x8(q + qbase + (int64_t)(32 * nt + col) * D + 16 * s + 8 * hh);

    f32x16 oacc[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[mt][nt][i] = 0.0f;
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.0f, 0.0f};

    uint16_t *vt = vt_all + wave * VT_ELEMS;

    for (int e = e_begin; e < e_end; ++e) {
        const int j = DENSE ? e : col_idx[e];
        if ((unsigned)j >= (unsigned)nb) continue;   // out-of-range block ids are skipped
#pragma unroll
        for (int c = wk; c < CHUNKS; c += 2) {
            const int kv0 = j * BLK + c * kChunk;
            // K chunk as the A operand: lane row = key (kv0 + col), dims 16*s + 8*hh.
            bf16x8 kf[KS];
#pragma unroll
            for (int s = 0; s < KS; ++s)
                kf[s] = load_bf16x8(k + kvbase + (int64_t)(kv0 + col) * D + 16 * s + 8 * hh);
            // V chunk rows (4 consecutive keys x 8 dims per unit), to be transposed.
            constexpr int UNITS = (8 * D / 8) / 64;    // units per lane
            uint4 vrow[UNITS][4];
#pragma unroll
            for (int x = 0; x < UNITS; ++x) {
                const int u = lane + 64 * x;
                const int b = u % (D / 8), a = u / (D / 8);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    vrow[x][r] = *reinterpret_cast<const uint4 *>(
                        v + kvbase + (int64_t)(kv0 + 4 * a + r) * D + 8 * b);
            }
            // S^T = K . Q^T (32 keys x 64 queries).
            f32x16 sacc[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[nt][i] = 0.0f;
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    sacc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[nt][s], sacc[nt],
                                                                       0, 0, 0);
            }
            // Transposed V tile into LDS: slot order within the chunk is
            // 16*ks + 8*hh + e  <->  key 16*ks + 8*(e/4) + 4*hh + e%4.
#pragma unroll
            for (int x = 0; x < UNITS; ++x) {
                const int u = lane + 64 * x;
                const int b = u % (D / 8), a = u / (D / 8);
                const int slot0 = 16 * (a >> 2) + 8 * (a & 1) + 4 * ((a & 3) >> 1);
                const uint32_t w[4][4] = {
                    {vrow[x][0].x, vrow[x][0].y, vrow[x][0].z, vrow[x][0].w},
                    {vrow[x][1].x, vrow[x][1].y, vrow[x][1].z, vrow[x][1].w},
                    {vrow[x][2].x, vrow[x][2].y, vrow[x][2].z, vrow[x][2].w},
                    {vrow[x][3].x, vrow[x][3].y, vrow[x][3].z, vrow[x][3].w}};
#pragma unroll
                for (int dd = 0; dd < 8; ++dd) {
                    const int sh = (dd & 1) * 16;
                    const uint32_t e0 = (w[0][dd >> 1] >> sh) & 0xFFFFu;
                    const uint32_t e1 = (w[1][dd >> 1] >> sh) & 0xFFFFu;
                    const uint32_t e2 = (w[2][dd >> 1] >> sh) & 0xFFFFu;
                    const uint32_t e3 = (w[3][dd >> 1] >> sh) & 0xFFFFu;
                    *reinterpret_cast<uint2 *>(vt + (8 * b + dd) * kVtStride + slot0) =
                        make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
                }
            }
            // Online softmax over this chunk, per query column.
            bf16x8 pf[2][2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                float mx = sacc[nt][0];
#pragma unroll
                for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[nt][i]);
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float m_new = fmaxf(m_run[nt], mx * scale_log2);
                const float alpha = exp2f(m_run[nt] - m_new);
                float psum = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float pv = exp2f(fmaf(sacc[nt][i], scale_log2, -m_new));
                    psum += pv;
                    pf[nt][i >> 3][i & 7] = (__bf16)pv;
                }
                l_run[nt] = l_run[nt] * alpha + psum;
                m_run[nt] = m_new;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[mt][nt][i] *= alpha;
            }
            __builtin_amdgcn_wave_barrier();
            // O^T += V^T . P^T.
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const bf16x8 vf = __builtin_bit_cast(
                        bf16x8, *reinterpret_cast<const uint4 *>(
                                    vt + (32 * mt + col) * kVtStride + 16 * ks + 8 * hh));
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
                        oacc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            vf, pf[nt][ks], oacc[mt][nt], 0, 0, 0);
                }
            __builtin_amdgcn_wave_barrier();
        }
    }

    // Column sums: the two lane halves hold different keys of the same column.
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) l_run[nt] += __shfl_xor(l_run[nt], 32);

    // Merge the two key halves (wk = 1 hands its state to wk = 0), then write.
    if (wk == 1) {
        ml[wq][0][lane] = m_run[0];
        ml[wq][1][lane] = m_run[1];
        ml[wq][2][lane] = l_run[0];
        ml[wq][3][lane] = l_run[1];
    }
    __syncthreads();
    float a_self[2], a_other[2], inv_l[2];
    if (wk == 0) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const float m1 = ml[wq][nt][lane], l1 = ml[wq][2 + nt][lane];
            const float mm = fmaxf(m_run[nt], m1);
            a_self[nt] = exp2f(m_run[nt] - mm);
            a_other[nt] = exp2f(m1 - mm);
            inv_l[nt] = 1.0f / (l_run[nt] * a_self[nt] + l1 * a_other[nt]);
        }
    }
    uint16_t *orow = o + qbase;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        __syncthreads();
        if (wk == 1) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int i = 0; i < 16; ++i) xchg[wq][16 * nt + i][lane] = oacc[mt][nt][i];
        }
        __syncthreads();
        if (wk == 0) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    uint32_t packed[2];
#pragma unroll
                    for (int r = 0; r < 4; r += 2) {
                        const int i = 4 * i4 + r;
                        const float x0 = (oacc[mt][nt][i] * a_self[nt] +
                                          xchg[wq][16 * nt + i][lane] * a_other[nt]) * inv_l[nt];
                        const float x1 = (oacc[mt][nt][i + 1] * a_self[nt] +
                                          xchg[wq][16 * nt + i + 1][lane] * a_other[nt]) * inv_l[nt];
                        packed[r >> 1] = (uint32_t)bf16_rne(x0) | ((uint32_t)bf16_rne(x1) << 16);
                    }
                    const int qr = 32 * nt + col;
                    const int dcol = 32 * mt + 8 * i4 + 4 * hh;
                    *reinterpret_cast<uint2 *>(orow + (int64_t)qr * D + dcol) =
                        make_uint2(packed[0], packed[1]);
                }
            }
        }
    }
}

template <int D, int BLK, bool DENSE>
hipError_t launch_attn_t(const Dims &Dm, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         const int32_t *row_ptr, const int32_t *col_idx, const int32_t *work,
                         int n_idx, uint16_t *o, hipStream_t s) {
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    hipLaunchKernelGGL((k_attn<D, BLK, DENSE>), dim3((unsigned)Dm.rows()), dim3(128 * (BLK / 64)),
                       0, s, q, k, v, row_ptr, col_idx, work, o, Dm.L, Dm.nb, Dm.G, Dm.H,
                       n_idx, scale_log2);
    return hipGetLastError();
}

template <bool DENSE>
hipError_t launch_attn(const Dims &D, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                       const int32_t *row_ptr, const int32_t *col_idx, const int32_t *work,
                       int n_idx, uint16_t *o, hipStream_t s) {
    if (D.d == 128 && D.B == 64)
        return launch_attn_t<128, 64, DENSE>(D, q, k, v, row_ptr, col_idx, work, n_idx, o, s);
    if (D.d == 128 && D.B == 128)
        return launch_attn_t<128, 128, DENSE>(D, q, k, v, row_ptr, col_idx, work, n_idx, o, s);
    if (D.d == 64 && D.B == 64)
        return launch_attn_t<64, 64, DENSE>(D, q, k, v, row_ptr, col_idx, work, n_idx, o, s);
    return launch_attn_t<64, 128, DENSE>(D, q, k, v, row_ptr, col_idx, work, n_idx, o, s);
}

}  // namespace

hipError_t launch_sparse_attn(const Dims &D, const uint16_t *q, const uint16_t *k,
                              const uint16_t *v, const int32_t *row_ptr, const int32_t *col_idx,
                              const int32_t *work, int64_t n_idx, uint16_t *o, hipStream_t s) {
    return launch_attn<false>(D, q, k, v, row_ptr, col_idx, work, (int)n_idx, o, s);
}

hipError_t launch_dense_attn(const Dims &D, const uint16_t *q, const uint16_t *k,
                             const uint16_t *v, uint16_t *o, hipStream_t s) {
    return launch_attn<true>(D, q, k, v, nullptr, nullptr, nullptr, 0, o, s);
}

}  // namespace sd
