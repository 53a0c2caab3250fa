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
//  * A wave owns QW = 32 query rows and walks every 32-key chunk of every
//    kept block with one online-softmax state, so no partial results are
//    merged; a workgroup is the BLK / 32 waves of one query block.  About 200
//    VGPRs per wave, so two waves share each SIMD and one wave's softmax
//    (VALU) overlaps the other's matrix work; with a 32 KiB ring per
//    workgroup, four 64-row workgroups fit on a CU.
//  * Scores are computed transposed, S^T = K . Q^T, with
//    v_mfma_f32_32x32x16_bf16: K is the A operand, Q^T the B operand (held in
//    registers for the whole row).  In the accumulator layout every lane holds
//    one query column, so the softmax rescale of O^T is a per-lane scalar and
//    the fp32 scores convert in place into the B operand of O^T += V^T . P^T.
//    Inside a 16-wide k step the key order is permuted, consistently for P^T
//    and V^T: slot 16*ks + 8*hh + e holds key 16*ks + 8*(e/4) + 4*hh + e%4.
//  * K and V chunks stream through a two-stage LDS ring shared by the waves
//    of the workgroup and filled by direct buffer->LDS loads
//    (buffer_load_dwordx4 ... lds), 16-byte segments XOR-swizzled per row so
//    that operand reads are free of bank conflicts.  A chunk's fragments are
//    read out of LDS (K with ds_read_b128, V^T with the gfx950 transposing
//    ds_read_b64_tr_b16) before the next chunk's loads are issued, so those
//    loads fly during the MFMA/softmax body; one barrier per chunk orders the
//    shared stages.
//  * fp32 accumulation and softmax (exp2 with log2(e)/sqrt(d) folded in); the
//    running max is raised only when a chunk exceeds it by more than 8 (log2
//    units), so the O^T rescale is rare.  bf16 round-to-nearest-even output.
#include "common.h"

namespace sd {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
#define SD_LDS __attribute__((address_space(3)))
#define SD_GLOBAL __attribute__((address_space(1)))

constexpr int kChunk = 32;          // keys per wave step
constexpr int kQW = 32;             // query rows per wave

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t *p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(p));
}

__device__ __forceinline__ uint16_t bf16_rne(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// 16 bytes per lane from a buffer straight into LDS (64 lanes -> 1 KiB
// contiguous at `lds`).
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, uint16_t *lds,
                                           uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (SD_LDS void *)lds, 16, voff, soff, 0, 0);
}

// Swizzles of the 16-byte segment index inside a row of a 32 x D tile.
// K is read one row per lane (32 rows at a fixed segment): XOR with the row.
// V is read by the transposing load, 4 consecutive rows x 4 segments per
// 16 lanes: XOR with a multiple of 4 that differs between those rows.
template <int D>
__device__ __forceinline__ int swz_k(int row) { return row & (D / 8 - 1); }
template <int D>
__device__ __forceinline__ int swz_v(int row) {
    return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

template <int D, int BLK, int QW, bool DENSE>
__global__ __launch_bounds__(BLK / QW * 64, QW == 32 ? 2 : 1) void k_attn(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const int32_t *__restrict__ row_ptr,
    const int32_t *__restrict__ col_idx, const int32_t *__restrict__ work,
    uint16_t *__restrict__ o, int L, int nb, int G, int H, int n_idx, float scale_log2) {
    constexpr int NT = QW / 32;                 // 32-query tiles per wave
    constexpr int WQ = BLK / QW;                // query slices (= waves) per block
    constexpr int KS = D / 16;                  // k steps of the score product
    constexpr int MT = D / 32;                  // 32-row tiles of O^T
    constexpr int CPB = BLK / kChunk;           // chunks per key block
    constexpr int TILE = kChunk * D;            // bf16 elements in a 32-key tile
    constexpr int STAGE = 2 * TILE;             // K tile + V tile
    constexpr int NSEG = D / 8;                 // 16-byte segments per row
    constexpr int ROWS_PER_LOAD = 64 / NSEG;    // rows covered by one wave load
    constexpr int LOADS = kChunk / ROWS_PER_LOAD;   // wave loads per tile
    // One two-stage ring, shared by the WQ waves of the workgroup.
    __shared__ __attribute__((aligned(16))) uint16_t ring[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int wq = wave;
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
        // Workgroup b runs on die b % kDies: take that die's list.
        const int64_t cap = (int64_t)((H + kDies - 1) / kDies) * nb;
        const int b = blockIdx.x;
        row = __builtin_amdgcn_readfirstlane(work[(b % kDies) * cap + b / kDies]);
        if (row < 0 || row >= H * nb) return;   // padding (or a malformed order): nothing to do
    }
    const int h = row / nb, blk = row % nb, g = h / G;
    const int q0 = blk * BLK + QW * wq;
    const int64_t qbase = ((int64_t)h * L + q0) * D;
    const int64_t kvbase = (int64_t)g * L * D;

    int e_begin = 0, e_end = nb;
    if (!DENSE) {
        e_begin = max(__builtin_amdgcn_readfirstlane(row_ptr[row]), 0);
        e_end = min(__builtin_amdgcn_readfirstlane(row_ptr[row + 1]), n_idx);
    }
    if (e_end <= e_begin) {     // no kept block: the row attends to nothing
        const uint4 z = make_uint4(0, 0, 0, 0);
        for (int x = lane; x < QW * D / 8; x += 64)
            *reinterpret_cast<uint4 *>(o + qbase + (int64_t)x * 8) = z;
        return;
    }

    // Q^T operand fragments: lane holds query col (32*nt + col), dims 16*s + 8*hh .. +8.
    bf16x8 qf[NT][KS];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int s = 0; s < KS; ++s)
            qf[nt][s] = load_bf16x8(q + qbase + (int64_t)(32 * nt + col) * D + 16 * s + 8 * hh);

    f32x16 oacc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[mt][nt][i] = 0.0f;
    float m_run[NT], l_run[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        m_run[nt] = -INFINITY;
        l_run[nt] = 0.0f;
    }

    // The row's chunks: every 32-key chunk of every kept block e, in order.
    const int n_total = (e_end - e_begin) * CPB;
    auto chunk_key0 = [&](int n) -> int {
        const int e = e_begin + n / CPB;
        int j = DENSE ? e : __builtin_amdgcn_readfirstlane(col_idx[e]);
        j = min(max(j, 0), nb - 1);   // malformed ids are clamped into range
        return j * BLK + (n % CPB) * kChunk;
    };
    uint16_t *my_ring = ring;

    // Direct global->LDS loads of chunk n's K and V rows into stage st.  Wave
    // load t writes 64 x 16 contiguous bytes: rows t*ROWS_PER_LOAD + lane/NSEG,
    // stored segment lane%NSEG, which holds source segment (stored ^ swizzle).
    // Buffer loads over this key head: the chunk and row-group offsets are
    // scalar, the per-lane swizzled offsets are fixed; reads past the head
    // return zeros.
    const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(k + kvbase), 0, L * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(v + kvbase), 0, L * D * 2, 0x00020000);
    const int r_in = lane / NSEG, sp = lane % NSEG;
    // The WQ waves of the workgroup split each tile's LOADS wave loads:
    // this wave issues loads t = tt*WQ + wq.  Per-lane offsets (row within the
    // load and swizzled segment) are fixed per tt; row groups and the chunk
    // are scalar offsets.
    constexpr int MY_LOADS = LOADS / WQ;
    uint32_t k_voff[MY_LOADS];
#pragma unroll
    for (int tt = 0; tt < MY_LOADS; ++tt) {
        const int r = (tt * WQ + wq) * ROWS_PER_LOAD + r_in;
        k_voff[tt] = (uint32_t)(r_in * D * 2 + 16 * (sp ^ swz_k<D>(r)));
    }
    const uint32_t v_voff = (uint32_t)(r_in * D * 2 + 16 * (sp ^ swz_v<D>(r_in)));
    auto issue = [&](int n, int st) {
        const uint32_t kv_off = (uint32_t)chunk_key0(n) * (D * 2);
        uint16_t *kt = my_ring + st * STAGE;
        uint16_t *vt = kt + TILE;
#pragma unroll
        for (int tt = 0; tt < MY_LOADS; ++tt) {
            const int t = tt * WQ + wq;
            const uint32_t soff = kv_off + t * ROWS_PER_LOAD * D * 2;
            load_lds16(k_rsrc, kt + t * 512, k_voff[tt], soff);
            load_lds16(v_rsrc, vt + t * 512, v_voff, soff);
        }
    };

    // Operand fragments of the chunk in stage st.
    auto read_frags = [&](int st, bf16x8 (&kf)[KS], bf16x8 (&vf)[MT][2]) {
        const uint16_t *kt = my_ring + st * STAGE;
        const uint16_t *vt = kt + TILE;
        // K as the A operand: lane row = key col, dims 16*s + 8*hh.
#pragma unroll
        for (int s = 0; s < KS; ++s)
            kf[s] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const uint4 *>(
                            kt + col * D + 8 * ((2 * s + hh) ^ swz_k<D>(col))));
        // V^T as the A operand: lane row = dim 32*mt + col, 8 keys in slot order.
        // Transposing load: lane i of a 16-lane group gets element i%4 of the
        // 8-byte pieces addressed by lanes 4k + i/4, k = 0..3.  Addressing lane
        // (group gq, index i) points at key row 16*ks + 8*r + 4*(gq/2) + i/4,
        // dims 32*mt + 16*(gq%2) + 4*(i%4) .. +4.
        const int gq = lane >> 4, i16 = lane & 15;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                i16x4 part[2];
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int vrow = 16 * ks + 8 * r + 4 * (gq >> 1) + (i16 >> 2);
                    const int dim0 = 32 * mt + 16 * (gq & 1) + 4 * (i16 & 3);
                    const int seg = dim0 >> 3;
                    const uint16_t *pp =
                        vt + vrow * D + 8 * (seg ^ swz_v<D>(vrow)) + (dim0 & 7);
                    part[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (SD_LDS i16x4 *)(pp));
                }
                vf[mt][ks] = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
            }
    };

    auto compute_chunk = [&](const bf16x8 (&kf)[KS], const bf16x8 (&vf)[MT][2]) {
        // S^T = K . Q^T (32 keys x 64 queries).
        f32x16 sacc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[nt][i] = 0.0f;
#pragma unroll
            for (int s = 0; s < KS; ++s)
                sacc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[nt][s], sacc[nt], 0,
                                                                   0, 0);
        }
        // Online softmax per query column, log2 units, lazily rescaled.
        float mx[NT];
        bool raise = false;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            float a0 = fmaxf(fmaxf(sacc[nt][0], sacc[nt][1]), sacc[nt][2]);
            float a1 = fmaxf(fmaxf(sacc[nt][3], sacc[nt][4]), sacc[nt][5]);
            float a2 = fmaxf(fmaxf(sacc[nt][6], sacc[nt][7]), sacc[nt][8]);
            float a3 = fmaxf(fmaxf(sacc[nt][9], sacc[nt][10]), sacc[nt][11]);
            float a4 = fmaxf(fmaxf(sacc[nt][12], sacc[nt][13]), sacc[nt][14]);
            float m = fmaxf(fmaxf(a0, a1), fmaxf(fmaxf(a2, a3), fmaxf(a4, sacc[nt][15])));
            m = fmaxf(m, __shfl_xor(m, 32));
            mx[nt] = m * scale_log2;
            raise = raise || (mx[nt] > m_run[nt] + 8.0f);
        }
        if (__any(raise)) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const float m_new = fmaxf(m_run[nt], mx[nt]);
                const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - m_new);
                l_run[nt] *= alpha;
                m_run[nt] = m_new;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[mt][nt][i] *= alpha;
            }
        }
        bf16x8 pf[NT][2];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const float neg_m = -m_run[nt];
            float psum = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[nt][i], scale_log2, neg_m));
                psum += pv;
                pf[nt][i >> 3][i & 7] = (__bf16)pv;
            }
            l_run[nt] += psum;
        }
        // O^T += V^T . P^T.
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    oacc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        vf[mt][ks], pf[nt][ks], oacc[mt][nt], 0, 0, 0);
    };

    issue(0, 0);
    for (int n = 0; n < n_total; ++n) {
        const int st = n & 1;
        bf16x8 kf[KS];
        bf16x8 vf[MT][2];
        // Chunk n's direct-to-LDS loads are the oldest vector-memory operations
        // in flight: wait for all of them before any LDS read of the stage (the
        // compiler does not order LDS reads after buffer->LDS loads by itself).
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        // With a shared ring, the other waves' loads of this chunk must have
        // landed too, and every wave must have finished reading the stage the
        // next loads overwrite (read in the previous step, before its wait).
        if (WQ > 1) __syncthreads();
        read_frags(st, kf, vf);
        if (WQ > 1) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (n + 1 < n_total) issue(n + 1, st ^ 1);
        compute_chunk(kf, vf);
    }

    // Column sums: the two lane halves hold different keys of the same column.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) l_run[nt] += __shfl_xor(l_run[nt], 32);

    // O = O^T / l, rounded to bf16: lane holds query col (32*nt + col) and 4
    // consecutive dims per group of 4 accumulators.
    uint16_t *orow = o + qbase;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const float inv_l = 1.0f / l_run[nt];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int i = 4 * i4;
                const uint32_t lo = (uint32_t)bf16_rne(oacc[mt][nt][i] * inv_l) |
                                    ((uint32_t)bf16_rne(oacc[mt][nt][i + 1] * inv_l) << 16);
                const uint32_t hi = (uint32_t)bf16_rne(oacc[mt][nt][i + 2] * inv_l) |
                                    ((uint32_t)bf16_rne(oacc[mt][nt][i + 3] * inv_l) << 16);
                const int qr = 32 * nt + col;
                const int dcol = 32 * mt + 8 * i4 + 4 * hh;
                *reinterpret_cast<uint2 *>(orow + (int64_t)qr * D + dcol) = make_uint2(lo, hi);
            }
    }
}

template <int D, int BLK, int QW, bool DENSE>
hipError_t launch_attn_t(const Dims &Dm, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         const int32_t *row_ptr, const int32_t *col_idx, const int32_t *work,
                         int n_idx, uint16_t *o, hipStream_t s) {
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    const unsigned grid = (unsigned)(DENSE ? Dm.rows() : kDies * Dm.die_cap());
    hipLaunchKernelGGL((k_attn<D, BLK, QW, DENSE>), dim3(grid), dim3(BLK / QW * 64),
                       0, s, q, k, v, row_ptr, col_idx, work, o, Dm.L, Dm.nb, Dm.G, Dm.H,
                       n_idx, scale_log2);
    return hipGetLastError();
}

template <bool DENSE>
hipError_t launch_attn(const Dims &D, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                       const int32_t *row_ptr, const int32_t *col_idx, const int32_t *work,
                       int n_idx, uint16_t *o, hipStream_t s) {
    if (D.d == 128 && D.B == 64)
        return launch_attn_t<128, 64, kQW, DENSE>(D, q, k, v, row_ptr, col_idx, work, n_idx, o, s);
    if (D.d == 128 && D.B == 128)
        return launch_attn_t<128, 128, kQW, DENSE>(D, q, k, v, row_ptr, col_idx, work, n_idx, o, s);
    if (D.d == 64 && D.B == 64)
        return launch_attn_t<64, 64, kQW, DENSE>(D, q, k, v, row_ptr, col_idx, work, n_idx, o, s);
    return launch_attn_t<64, 128, kQW, DENSE>(D, q, k, v, row_ptr, col_idx, work, n_idx, o, s);
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
