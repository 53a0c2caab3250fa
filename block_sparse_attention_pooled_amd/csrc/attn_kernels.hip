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
//    merged; a workgroup is the BLK / 32 waves of one query block.  Under 256
//    VGPRs per wave, so two waves share each SIMD; with 40 KiB of LDS per
//    workgroup, four 64-row workgroups fit on a CU.
//  * In sparse mode a workgroup starts from the plan's record for its work
//    position (row, list bounds, first two block ids), so its first K/V loads
//    leave one load after it starts; the rest of the list is read 64 ids at a
//    time into one register.
//  * Scores are computed transposed, S^T = K . Q^T, with
//    v_mfma_f32_32x32x16_bf16: K is the A operand, Q^T the B operand (held in
//    registers for the whole row).  In the accumulator layout every lane holds
//    one query column, so the softmax rescale of O^T is a per-lane scalar and
//    the fp32 scores convert in place into the B operand of O^T += V^T . P^T.
//    Inside a 16-wide k step the key order is permuted, consistently for P^T
//    and V^T: slot 16*ks + 8*hh + e holds key 16*ks + 8*(e/4) + 4*hh + e%4.
//  * K and V chunks stream through LDS rings (three K stages, two V stages)
//    shared by the waves of the workgroup and filled by direct buffer->LDS
//    loads (buffer_load_dwordx4 ... lds), 16-byte segments XOR-swizzled per
//    row so that operand reads are free of bank conflicts.  K fragments are
//    read with ds_read_b128, V^T fragments with the gfx950 transposing
//    ds_read_b64_tr_b16; one barrier per chunk orders the shared stages.
//  * Software pipeline: the scores of chunk n+1 are formed on the matrix
//    cores while the weights of chunk n are formed on the VALU, and the next
//    chunks' loads fly during the whole step.
//  * fp32 accumulation and softmax (exp2 with log2(e)/sqrt(d) folded in); the
//    running max is raised only when a chunk exceeds it by more than 8 (log2
//    units), so the O^T rescale is rare; the normaliser sums the bf16-rounded
//    weights that enter the product.  bf16 round-to-nearest-even output,
//    staged through the (then free) rings so that every store writes whole
//    rows: scattered 8-byte stores from the accumulator layout cost the
//    memory path far more than their bytes.
//
// Column mode: the column-sparse variant ("PulseCol", abstract: individual
// key columns kept instead of blocks).  Every query of head h attends to the
// k_c key tokens listed for the head; a chunk is 32 consecutive list entries
// and each lane's rows of a K/V tile are gathered by buffer->LDS loads whose
// per-lane offsets come from the list.  The list entries a step needs are
// loaded one step ahead; a short last chunk has its missing keys' scores set
// to -inf, so they get weight 0.
//
// Group mode (grouped-query attention, heads h / (H/Hkv) sharing a key head):
// a workgroup takes two query heads of one KV group for one query block and
// streams the union of their kept-block lists through one K/V ring, so a tile
// both keep is read once.  Each wave computes only the chunks its head keeps
// (reads, scores, weights and products are skipped otherwise; the barriers
// stay common), so each head's output is that of the sparse mode bit for bit.
#include "common.h"

namespace sd {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define SD_LDS __attribute__((address_space(3)))
#define SD_GLOBAL __attribute__((address_space(1)))

constexpr int kChunk = 32;          // keys per wave step
constexpr int kQW = 32;             // query rows per wave

// Which keys a row walks.
constexpr int kModeSparse = 0;      // the kept blocks of the row (CSR lists, work order)
constexpr int kModeDense = 1;       // every key block
constexpr int kModeCols = 2;        // the head's kept key columns (col_idx = [H, n_idx])
constexpr int kModeGroup = 3;       // two heads of one KV group over the union of their lists
constexpr int kGroupHeads = 2;      // query heads per workgroup in group mode

// Issue order of one full pipeline step (d = 128: 16 MFMAs, 24 LDS reads, 8
// buffer->LDS loads, about 60 VALU): while the score chain runs, each MFMA is
// followed by two fragment reads, five softmax VALU ops and one ring load;
// while the O product runs, by one read and three VALU ops.  Against the
// compiler's own order, 0.3-1.7% faster on 8K launches (64-token blocks) and
// 1.2-1.9% at 64K (128-token blocks), sparse and dense, same results.  (The
// column instance is slower with it: it stays with the compiler's order.)
__device__ __forceinline__ void step_issue_order() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // VALU
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // vector memory read
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
}

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t *p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(p));
}

// O is written once and read by a later kernel: non-temporal stores stream it
// out instead of leaving dirty lines in this die's L2 for the end-of-kernel
// write-back.
__device__ __forceinline__ void store_nt(uint16_t *p, uint4 v) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4 *>(p));
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

template <int D, int BLK, int QW, int MODE>
__global__ __launch_bounds__(BLK / QW * 64 * (MODE == kModeGroup ? kGroupHeads : 1),
                             QW == 32 ? 2 : 1) void k_attn(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const int32_t *__restrict__ row_ptr,
    const int32_t *__restrict__ col_idx, const int4 *__restrict__ recs,
    int32_t *__restrict__ meta, uint16_t *__restrict__ o, int L, int nb, int G, int H, int n_idx,
    int64_t cap, float scale_log2) {
    constexpr int NT = QW / 32;                 // 32-query tiles per wave
    constexpr int WQ = BLK / QW;                // query slices (waves) per query block
    constexpr bool GROUP = MODE == kModeGroup;
    constexpr int HS = GROUP ? kGroupHeads : 1; // query heads per workgroup
    constexpr int NW = WQ * HS;                 // waves per workgroup
    constexpr int KS = D / 16;                  // k steps of the score product
    constexpr int MT = D / 32;                  // 32-row tiles of O^T
    constexpr int CPB = BLK / kChunk;           // chunks per key block
    constexpr int TILE = kChunk * D;            // bf16 elements in a 32-key tile
    constexpr int NSEG = D / 8;                 // 16-byte segments per row
    constexpr int ROWS_PER_LOAD = 64 / NSEG;    // rows covered by one wave load
    constexpr int LOADS = kChunk / ROWS_PER_LOAD;   // wave loads per tile
    constexpr bool SPARSE = MODE == kModeSparse;
    constexpr bool COLS = MODE == kModeCols;
    // The fixed issue order is tuned for (and applied to) these instances.
    constexpr bool ORDERED = D == 128 && (SPARSE || MODE == kModeDense);
    // A three-stage K ring and a two-stage V ring, shared by the NW waves of
    // the workgroup.
    __shared__ __attribute__((aligned(16))) uint16_t rings[5 * TILE];
    // Group mode: the union of the heads' lists, one entry per key block:
    // block id | (bit s set when head slot s keeps it) << 16.
    __shared__ int32_t uni[GROUP ? kMaxBlocks : 1];
    __shared__ int32_t uflag[GROUP ? kMaxBlocks : 1];
    __shared__ int32_t uwave[GROUP ? NW : 1];
    uint16_t *const kring = rings;
    uint16_t *const vring = rings + 3 * TILE;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int wq = wave % WQ;                   // query slice of this wave
    const int hs = wave / WQ;                   // head slot (group mode)
    const int col = lane & 31, hh = lane >> 5;

    // Row of this workgroup and, in sparse mode, its list bounds and first
    // two block ids from the work record.
    int row;
    int rec_begin = 0, rec_end = 0, rec_ids = 0;
    bool head_ok = true;          // group mode: this wave's head slot holds a head
    int grp_row0 = 0;             // group mode: row of head slot 0
    if (GROUP) {
        // Workgroup b: KV group g, head pair p (heads g*G + 2p, + 1), query
        // block i; the pairs of a group sit on one XCD when they can.
        const int pairs = (G + kGroupHeads - 1) / kGroupHeads;
        const int units = H / G * pairs;
        const int b = blockIdx.x;
        int gp, i;
        if ((units & 7) == 0) {
            gp = (b & 7) + 8 * ((b >> 3) / nb);
            i = (b >> 3) % nb;
        } else {
            gp = b / nb;
            i = b % nb;
        }
        const int g_ = gp / pairs, slot0 = (gp % pairs) * kGroupHeads;
        head_ok = slot0 + hs < G;
        grp_row0 = (g_ * G + slot0) * nb + i;
        row = head_ok ? grp_row0 + hs * nb : grp_row0;
    } else if (!SPARSE) {
        const int b = blockIdx.x;
        if ((H & 7) == 0) {   // keep each head's rows on one XCD (round-robin dispatch)
            const int x = b & 7, kk = b >> 3;
            row = (x + 8 * (kk / nb)) * nb + kk % nb;
        } else {
            row = b;
        }
    } else {
        // Workgroup b runs on die b % kDies: take position b / kDies of that
        // die's list (cap positions per die).  One record holds everything
        // the first K/V loads need, so they leave one load after the start.
        const int b = blockIdx.x;
        const int4 rc = recs[(b % kDies) * cap + b / kDies];
        // The plan's tag: the list array and length it was made from, and
        // the shape.  A launch on another array, length or shape (a stale
        // plan) writes zeros and flags bit 0 of the check word.
        const int4 tag = *reinterpret_cast<const int4 *>(meta + kMetaListLo);
        const int tag_nb = meta[kMetaNb];
        row = __builtin_amdgcn_readfirstlane(rc.x);
        if (row < 0 || row >= H * nb) return;   // padding (or a malformed order): nothing to do
        rec_begin = __builtin_amdgcn_readfirstlane(rc.y);
        rec_end = __builtin_amdgcn_readfirstlane(rc.z);
        rec_ids = __builtin_amdgcn_readfirstlane(rc.w);
        const uint64_t list_addr = reinterpret_cast<uint64_t>(col_idx);
        if (tag.x != (int)(uint32_t)list_addr || tag.y != (int)(uint32_t)(list_addr >> 32) ||
            tag.z != n_idx || tag.w != H || tag_nb != nb) {
            if (tid == 0) atomicOr(meta + kMetaCheck, kCheckStalePlan);
            rec_end = rec_begin;   // no chunk: the row writes zeros
        }
    }
    const int h = row / nb, blk = row % nb, g = h / G;
    const int q0 = blk * BLK + QW * wq;
    const int64_t qbase = ((int64_t)h * L + q0) * D;
    const int64_t kvbase = (int64_t)g * L * D;

    int e_begin = 0, e_end = nb;
    if (SPARSE) {
        e_begin = max(rec_begin, 0);
        e_end = min(rec_end, n_idx);
    }
    int n_union = 0;
    if (GROUP) {
        // Union of the head slots' lists (positions past n_idx are not read,
        // ids clamped into [0, nb)), then compacted in ascending block order.
        for (int j = tid; j < nb; j += NW * 64) uflag[j] = 0;
        __syncthreads();
#pragma unroll
        for (int sl = 0; sl < HS; ++sl) {
            const int gr = grp_row0 + sl * nb;
            const bool ok = (grp_row0 / nb) % G + sl < G && gr < H * nb;
            const int lo = ok ? max(row_ptr[gr], 0) : 0;
            const int hi = ok ? min(row_ptr[gr + 1], n_idx) : 0;
            for (int e = lo + tid; e < hi; e += NW * 64)
                atomicOr(&uflag[min(max(col_idx[e], 0), nb - 1)], 1 << sl);
        }
        __syncthreads();
        const int per = (nb + NW * 64 - 1) / (NW * 64);
        const int j0 = min(tid * per, nb), j1 = min(j0 + per, nb);
        int cnt = 0;
        for (int j = j0; j < j1; ++j) cnt += uflag[j] != 0;
        int inc = cnt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(inc, off);
            if (lane >= off) inc += y;
        }
        if (lane == 63) uwave[wave] = inc;
        __syncthreads();
        int pos = inc - cnt;
        for (int w = 0; w < wave; ++w) pos += uwave[w];
        for (int w = 0; w < NW; ++w) n_union += uwave[w];
        for (int j = j0; j < j1; ++j)
            if (uflag[j]) uni[pos++] = j | (uflag[j] << 16);
        __syncthreads();
    }
    // The row's chunks: every 32-key chunk of every kept block e, in order
    // (column mode: 32 consecutive entries of the head's column list; group
    // mode: every chunk of the union, each wave computing only its head's).
    const int n_total = COLS  ? (n_idx + kChunk - 1) / kChunk
                        : GROUP ? n_union * CPB
                                : (e_end > e_begin ? (e_end - e_begin) * CPB : 0);
    if (n_total <= 0) {     // no kept key: the row attends to nothing
        const uint4 z = make_uint4(0, 0, 0, 0);
        if (head_ok)
            for (int x = lane; x < QW * D / 8; x += 64)
                store_nt(o + qbase + (int64_t)x * 8, z);
        return;
    }
    // Group mode: does this wave's head keep union entry e (chunks CPB*e ..)?
    auto member = [&](int n) -> bool {
        if (!GROUP) return true;
        const int ent = __builtin_amdgcn_readfirstlane(uni[n / CPB]);
        return head_ok && ((ent >> (16 + hs)) & 1);
    };

    // Q^T operand fragments: lane holds query col (32*nt + col), dims 16*s + 8*hh .. +8.
    bf16x8 qf[NT][KS];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int s = 0; s < KS; ++s)
            qf[nt][s] = load_bf16x8(q + qbase + (int64_t)(32 * nt + col) * D + 16 * s + 8 * hh);

    // The row's key-block ids, 64 at a time in one register: lane i holds the
    // id of kept block e_begin + 64*ids_grp + i.  Ids are then taken with
    // readlane, so the chunk loop issues no scalar loads (a wait on one would
    // also wait on every LDS read in flight).  Loaded after Q, so the first
    // wait on them also retires the Q loads before the loop.
    int ids = 0, ids_grp = 0;
    if (SPARSE) {
        const int e = e_begin + lane;
        ids = e < e_end ? col_idx[e] : 0;
    }

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

    auto chunk_key0 = [&](int n) -> int {
        const int e_rel = n / CPB;
        int j;
        if (GROUP) {
            j = __builtin_amdgcn_readfirstlane(uni[e_rel]) & 0xFFFF;
        } else if (!SPARSE) {
            j = e_begin + e_rel;
        } else if (e_rel < 2) {   // the record's ids: no wait on the list load
            j = (rec_ids >> (16 * e_rel)) & 0xFFFF;
        } else {
            const int grp = e_rel >> 6;
            if (grp != ids_grp) {
                const int e = e_begin + 64 * grp + lane;
                ids = e < e_end ? col_idx[e] : 0;
                ids_grp = grp;
            }
            j = __builtin_amdgcn_readlane(ids, e_rel & 63);
        }
        j = min(max(j, 0), nb - 1);   // malformed ids are clamped into range
        return j * BLK + (n % CPB) * kChunk;
    };

    // Direct global->LDS loads of chunk c's K (or V) rows into stage st.  Wave
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
    // The NW waves of the workgroup split each tile's LOADS wave loads:
    // this wave issues loads t = tt*NW + wave.
    static_assert(LOADS % NW == 0, "a tile's loads split evenly over the waves");
    constexpr int MY_LOADS = LOADS / NW;
    uint32_t k_voff[MY_LOADS];
#pragma unroll
    for (int tt = 0; tt < MY_LOADS; ++tt) {
        const int r = (tt * NW + wave) * ROWS_PER_LOAD + r_in;
        k_voff[tt] = (uint32_t)(r_in * D * 2 + 16 * (sp ^ swz_k<D>(r)));
    }
    const uint32_t v_voff = (uint32_t)(r_in * D * 2 + 16 * (sp ^ swz_v<D>(r_in)));
    auto issue_k = [&](int key0, uint16_t *dst) {
        const uint32_t off = (uint32_t)key0 * (D * 2);
#pragma unroll
        for (int tt = 0; tt < MY_LOADS; ++tt) {
            const int t = tt * NW + wave;
            load_lds16(k_rsrc, dst + t * 512, k_voff[tt], off + t * ROWS_PER_LOAD * D * 2);
        }
    };
    auto issue_v = [&](int key0, uint16_t *dst) {
        const uint32_t off = (uint32_t)key0 * (D * 2);
#pragma unroll
        for (int tt = 0; tt < MY_LOADS; ++tt) {
            const int t = tt * NW + wave;
            load_lds16(v_rsrc, dst + t * 512, v_voff, off + t * ROWS_PER_LOAD * D * 2);
        }
    };
    // Column mode: list entry 32*c + r is the token of row r of chunk c.  A
    // lane's row in its wave load tt is (tt*WQ + wq)*ROWS_PER_LOAD + r_in;
    // entries past the list read 0 (a valid token whose weight is masked).
    const __amdgpu_buffer_rsrc_t c_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(col_idx + (COLS ? (int64_t)h * n_idx : 0)), 0, COLS ? n_idx * 4 : 0,
        0x00020000);
    const uint32_t tok_voff = (uint32_t)((wave * ROWS_PER_LOAD + r_in) * 4);
    auto load_tok = [&](int c, int (&tok)[MY_LOADS]) {
#pragma unroll
        for (int tt = 0; tt < MY_LOADS; ++tt)
            tok[tt] = (int)__builtin_amdgcn_raw_buffer_load_b32(
                c_rsrc, tok_voff + tt * NW * ROWS_PER_LOAD * 4, c * kChunk * 4, 0);
    };
    // Gathered rows: the token's row in the key head, at the segment the
    // contiguous loads would use.  Tokens outside the head read zeros.
    auto issue_k_tok = [&](const int (&tok)[MY_LOADS], uint16_t *dst) {
#pragma unroll
        for (int tt = 0; tt < MY_LOADS; ++tt) {
            const int t = tt * NW + wave;
            load_lds16(k_rsrc, dst + t * 512,
                       (uint32_t)tok[tt] * (D * 2) + (k_voff[tt] - r_in * D * 2), 0);
        }
    };
    auto issue_v_tok = [&](const int (&tok)[MY_LOADS], uint16_t *dst) {
#pragma unroll
        for (int tt = 0; tt < MY_LOADS; ++tt) {
            const int t = tt * NW + wave;
            load_lds16(v_rsrc, dst + t * 512,
                       (uint32_t)tok[tt] * (D * 2) + (v_voff - r_in * D * 2), 0);
        }
    };
    // Valid keys of the last chunk (column mode); accumulator i of a lane is
    // key 8*(i/4) + 4*hh + i%4 of the chunk.
    const int tail = COLS ? n_idx - (n_total - 1) * kChunk : kChunk;
    auto mask_tail = [&](f32x16 (&sacc)[NT]) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (8 * (i >> 2) + 4 * hh + (i & 3) >= tail) sacc[nt][i] = -INFINITY;
    };

    // K as the A operand of the score product: lane row = key col, dims
    // 16*s + 8*hh.
    auto read_k = [&](const uint16_t *kt, bf16x8 (&kf)[KS]) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
            kf[s] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const uint4 *>(
                            kt + col * D + 8 * ((2 * s + hh) ^ swz_k<D>(col))));
    };
    // V^T as the A operand: lane row = dim 32*mt + col, 8 keys in slot order.
    // Transposing load: lane i of a 16-lane group gets element i%4 of the
    // 8-byte pieces addressed by lanes 4k + i/4, k = 0..3.  Addressing lane
    // (group gq, index i) points at key row 16*ks + 8*r + 4*(gq/2) + i/4,
    // dims 32*mt + 16*(gq%2) + 4*(i%4) .. +4.
    auto read_v = [&](const uint16_t *vt, bf16x8 (&vf)[MT][2]) {
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

    // S^T = K . Q^T (32 keys x QW queries).
    auto scores = [&](const bf16x8 (&kf)[KS], f32x16 (&sacc)[NT]) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[nt][i] = 0.0f;
#pragma unroll
            for (int s = 0; s < KS; ++s)
                sacc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[nt][s], sacc[nt], 0,
                                                                   0, 0);
        }
    };
    // Online softmax per query column, log2 units, lazily rescaled: each lane
    // checks its 16 keys of the column (the other 16 are in lane ^ 32) against
    // the running max; the max only moves here, from the max over all 32 keys,
    // so both halves of a column always hold the same value.
    // in_step: called at the end of a pipeline step (its straight-line code
    // ends at the rescale branch, where the step's issue order is set).
    auto update_max = [&](const f32x16 (&sacc)[NT], bool in_step) {
        float mx[NT];
        bool raise = false;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            float a0 = fmaxf(fmaxf(sacc[nt][0], sacc[nt][1]), sacc[nt][2]);
            float a1 = fmaxf(fmaxf(sacc[nt][3], sacc[nt][4]), sacc[nt][5]);
            float a2 = fmaxf(fmaxf(sacc[nt][6], sacc[nt][7]), sacc[nt][8]);
            float a3 = fmaxf(fmaxf(sacc[nt][9], sacc[nt][10]), sacc[nt][11]);
            float a4 = fmaxf(fmaxf(sacc[nt][12], sacc[nt][13]), sacc[nt][14]);
            const float m = fmaxf(fmaxf(a0, a1), fmaxf(fmaxf(a2, a3), fmaxf(a4, sacc[nt][15])));
            mx[nt] = m * scale_log2;
            raise = raise || (mx[nt] > m_run[nt] + 8.0f);
        }
        if (ORDERED && in_step) step_issue_order();
        if (__any(raise)) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const float m_new = fmaxf(m_run[nt], fmaxf(mx[nt], __shfl_xor(mx[nt], 32)));
                const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - m_new);
                l_run[nt] *= alpha;
                m_run[nt] = m_new;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[mt][nt][i] *= alpha;
            }
        }
    };
    // Weights of chunk (scores sacc) as the bf16 B operand; the normaliser
    // sums the weights as rounded for the product.
    auto weights = [&](const f32x16 (&sacc)[NT], bf16x8 (&pf)[NT][2]) {
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const float neg_m = -m_run[nt];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                pf[nt][i >> 3][i & 7] =
                    (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[nt][i], scale_log2, neg_m));
            float psum = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                psum = __builtin_amdgcn_fdot2_f32_bf16(
                    bf16x2{pf[nt][i >> 2][2 * (i & 3)], pf[nt][i >> 2][2 * (i & 3) + 1]}, one,
                    psum, false);
            l_run[nt] += psum;
        }
    };
    // O^T += V^T . P^T.
    auto pv = [&](const bf16x8 (&vf)[MT][2], const bf16x8 (&pf)[NT][2]) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    oacc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        vf[mt][ks], pf[nt][ks], oacc[mt][nt], 0, 0, 0);
    };

    // Ring waits.  Only direct-to-LDS loads are in flight at the vmcnt wait,
    // so vmcnt(0) means this wave's share of the stages has landed (the
    // compiler does not order LDS reads after buffer->LDS loads by itself);
    // lgkmcnt(0) means this wave has finished every read it issued.  After
    // both, the barrier makes every wave's share visible and frees the stages
    // read before it.
    auto sync = [&] {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (NW > 1) __syncthreads();
    };

    // Software pipeline over the row's chunks; K(c) sits in K stage c%3, V(c)
    // in V stage c%2.  Entering step n: the scores S(n) are formed and the
    // running max covers them, K(n+1) is in registers, and V(n) and K(n+2)
    // are being loaded.  Step n:
    //   sync; read V(n); S(n+1) = K(n+1) . Q^T on the matrix cores while the
    //   weights P(n) are formed on the VALU; read K(n+2) into registers once
    //   S(n+1) has consumed K(n+1); load V(n+1) (its stage was read in step
    //   n-1) and K(n+3) (stage of K(n), read in step n-2); O^T += V(n) . P(n)
    //   on the matrix cores while the max of S(n+1) is taken; rare rescale.
    // The loads and the LDS reads of a step touch different stages, so their
    // order inside the step is left to the compiler (see body below).  FULL
    // steps have every chunk up to n+3; the last steps are guarded.
    bf16x8 kf[KS];
    // Column mode: tokens of the next V load (chunk n+1) and K load (chunk
    // n+3), loaded during the previous step.
    int tok_v[MY_LOADS], tok_k[MY_LOADS];
    // One step's work on the rings.  The stages it loads (K(n+3), V(n+1)) and
    // the stages it reads (V(n), K(n+2)) are always different, and every load
    // of an earlier step has landed at the sync before it.  Passing the four
    // stages as restrict pointers tells the compiler so: it then neither makes
    // each LDS read wait for every buffer->LDS load in flight nor has to keep
    // the loads after the reads, and the step needs fewer registers (no
    // instance spills).
    // m0, m1, m2: this wave computes chunks n, n+1, n+2 (always, except for
    // the chunks of the union that its head does not keep in group mode).
    auto body = [&](int n, bool full, bool has1, bool has2, bool has3, bool m0, bool m1, bool m2,
                    int key1, int key3, uint16_t *__restrict__ kdst, uint16_t *__restrict__ vdst,
                    const uint16_t *__restrict__ ksrc, const uint16_t *__restrict__ vsrc,
                    f32x16 (&s_cur)[NT], f32x16 (&s_next)[NT]) {
        bf16x8 vf[MT][2];
        bf16x8 pf[NT][2];
        if (m0) read_v(vsrc, vf);
        if (has1 && m1) scores(kf, s_next);
        if (COLS && has1 && n + 1 == n_total - 1 && tail < kChunk) mask_tail(s_next);
        if (m0) weights(s_cur, pf);
        if (has2 && m2) read_k(ksrc, kf);
        if (COLS) {
            if (has1) issue_v_tok(tok_v, vdst);
            if (has3) issue_k_tok(tok_k, kdst);
            // A FULL step has chunks up to n+4 (the loop runs while n+4 <
            // n_total); a tail step never needs chunk n+4.
            if (full || n + 2 < n_total) load_tok(n + 2, tok_v);
            if (full) load_tok(n + 4, tok_k);
        } else {
            if (has1) issue_v(key1, vdst);
            if (has3) issue_k(key3, kdst);
        }
        if (m0) pv(vf, pf);
        if (has1 && m1) update_max(s_next, true);
    };
    auto step = [&](int n, bool full, f32x16 (&s_cur)[NT], f32x16 (&s_next)[NT]) {
        const bool has1 = full || n + 1 < n_total;
        const bool has2 = full || n + 2 < n_total;
        const bool has3 = full || n + 3 < n_total;
        sync();
        // Keys of the next loads first: a reload of the ids waits on vector
        // memory, which is idle right after the sync.
        const int key1 = (!COLS && has1) ? chunk_key0(n + 1) : 0;
        const int key3 = (!COLS && has3) ? chunk_key0(n + 3) : 0;
        const bool m0 = member(n), m1 = has1 && member(n + 1), m2 = has2 && member(n + 2);
        body(n, full, has1, has2, has3, m0, m1, m2, key1, key3, kring + (n % 3) * TILE,
             vring + ((n + 1) & 1) * TILE, kring + ((n + 2) % 3) * TILE, vring + (n & 1) * TILE,
             s_cur, s_next);
    };

    f32x16 sA[NT], sB[NT];
    // Prologue: K(0..2) and V(0) in flight; S(0) and its max; K(1) into
    // registers.
    if (COLS) {
        int t0[MY_LOADS], t2[MY_LOADS];
        load_tok(0, t0);
        load_tok(1, tok_v);
        load_tok(2, t2);
        load_tok(3, tok_k);
        issue_k_tok(t0, kring);
        issue_v_tok(t0, vring);
        if (n_total > 1) issue_k_tok(tok_v, kring + TILE);
        if (n_total > 2) issue_k_tok(t2, kring + 2 * TILE);
    } else {
        const int key0 = chunk_key0(0);
        issue_k(key0, kring);
        issue_v(key0, vring);
        if (n_total > 1) issue_k(chunk_key0(1), kring + TILE);
        if (n_total > 2) issue_k(chunk_key0(2), kring + 2 * TILE);
    }
    sync();
    // The row's first two list entries must still be the ones its record
    // holds (col_idx rewritten after planning): otherwise the row writes
    // zeros and flags bit 1 of the check word.  Lanes 0 and 1 of the first
    // id load hold them, landed at the sync above, so the check adds no load.
    bool list_changed = false;
    if (SPARSE) {
        const int c0 = min(max(__builtin_amdgcn_readlane(ids, 0), 0), nb - 1);
        const int c1 = e_end - e_begin > 1 ? min(max(__builtin_amdgcn_readlane(ids, 1), 0), nb - 1) : 0;
        list_changed = (c0 | (c1 << 16)) != rec_ids;
    }
    const bool p0 = member(0), p1 = n_total > 1 && member(1);
    if (p0) read_k(kring, kf);
    if (p0) scores(kf, sA);
    if (COLS && n_total == 1 && tail < kChunk) mask_tail(sA);
    if (p1) read_k(kring + TILE, kf);
    if (p0) update_max(sA, false);

    int n = 0;
    for (; n + 4 < n_total; n += 2) {
        step(n, true, sA, sB);
        step(n + 1, true, sB, sA);
    }
    // 1 to 4 chunks remain, starting at an even n.
    step(n, false, sA, sB);
    if (n + 1 < n_total) step(n + 1, false, sB, sA);
    if (n + 2 < n_total) step(n + 2, false, sA, sB);
    if (n + 3 < n_total) step(n + 3, false, sB, sA);

    // Column sums: the two lane halves hold different keys of the same column.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) l_run[nt] += __shfl_xor(l_run[nt], 32);

    if (list_changed && tid == 0) atomicOr(meta + kMetaCheck, kCheckListChanged);

    // O = O^T / l, rounded to bf16, staged through LDS so that every store
    // writes whole rows.  Lane holds query col (32*nt + col) and 4 consecutive
    // dims per group of 4 accumulators; the wave's 32 x D tile goes into the
    // rings (every wave has finished reading them after the sync), row-major
    // with 16-byte segment s of row r stored at s ^ (r % segments), then each
    // lane reads back 16 contiguous bytes and the wave stores 64 x 16 bytes
    // of consecutive rows per instruction.
    sync();
    constexpr int SEGS = D / 8;                 // 16-byte segments per row
    constexpr int RPI = 64 / SEGS;              // rows per store instruction
    static_assert(NW * QW * D <= 5 * TILE, "the staged tiles fit in the rings");
    uint16_t *ot = rings + wave * QW * D;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        // Group mode: a head that keeps no block of the union writes zeros.
        const float inv_l = (GROUP && !(l_run[nt] > 0.0f)) ? 0.0f : 1.0f / l_run[nt];
        const int r = 32 * nt + col;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int i = 4 * i4;
                // Four dims at once: two packed round-to-nearest-even converts.
                const bf16x4 v4 = {(__bf16)(oacc[mt][nt][i] * inv_l),
                                   (__bf16)(oacc[mt][nt][i + 1] * inv_l),
                                   (__bf16)(oacc[mt][nt][i + 2] * inv_l),
                                   (__bf16)(oacc[mt][nt][i + 3] * inv_l)};
                const int seg = 4 * mt + i4;    // dims 8*seg .. +8; this lane's half is 4*hh
                *reinterpret_cast<bf16x4 *>(ot + r * D + 8 * (seg ^ (r & (SEGS - 1))) + 4 * hh) =
                    v4;
            }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (!head_ok) return;
    uint16_t *orow = o + qbase;
#pragma unroll
    for (int t = 0; t < QW / RPI; ++t) {
        const int r = t * RPI + lane / SEGS, sg = lane % SEGS;
        uint4 val = *reinterpret_cast<const uint4 *>(ot + r * D + 8 * (sg ^ (r & (SEGS - 1))));
        if (list_changed) val = make_uint4(0, 0, 0, 0);
        store_nt(orow + (int64_t)r * D + 8 * sg, val);
    }
}

template <int D, int BLK, int QW, int MODE>
hipError_t launch_attn_t(const Dims &Dm, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         const int32_t *row_ptr, const int32_t *col_idx, const int4 *recs,
                         int32_t *meta, int n_idx, uint16_t *o, hipStream_t s) {
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    const int64_t cap = Dm.die_cap();
    const int64_t group_units =
        (int64_t)(Dm.H / Dm.G) * ((Dm.G + kGroupHeads - 1) / kGroupHeads) * Dm.nb;
    const unsigned grid = (unsigned)(MODE == kModeSparse  ? kDies * cap
                                     : MODE == kModeGroup ? group_units
                                                          : Dm.rows());
    const unsigned threads = BLK / QW * 64 * (MODE == kModeGroup ? kGroupHeads : 1);
    hipLaunchKernelGGL((k_attn<D, BLK, QW, MODE>), dim3(grid), dim3(threads), 0, s, q, k, v,
                       row_ptr, col_idx, recs, meta, o, Dm.L, Dm.nb, Dm.G, Dm.H, n_idx, cap,
                       scale_log2);
    return hipGetLastError();
}

template <int MODE>
hipError_t launch_attn(const Dims &D, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                       const int32_t *col_idx, const int4 *recs, int32_t *meta, int n_idx,
                       uint16_t *o, hipStream_t s) {
    if (D.d == 128 && D.B == 64)
        return launch_attn_t<128, 64, kQW, MODE>(D, q, k, v, nullptr, col_idx, recs, meta, n_idx,
                                                 o, s);
    if (D.d == 128 && D.B == 128)
        return launch_attn_t<128, 128, kQW, MODE>(D, q, k, v, nullptr, col_idx, recs, meta, n_idx,
                                                  o, s);
    if (D.d == 64 && D.B == 64)
        return launch_attn_t<64, 64, kQW, MODE>(D, q, k, v, nullptr, col_idx, recs, meta, n_idx,
                                                o, s);
    return launch_attn_t<64, 128, kQW, MODE>(D, q, k, v, nullptr, col_idx, recs, meta, n_idx, o,
                                             s);
}

}  // namespace

hipError_t launch_sparse_attn(const Dims &D, const uint16_t *q, const uint16_t *k,
                              const uint16_t *v, const int32_t *col_idx, const int4 *recs,
                              int32_t *meta, int64_t n_idx, uint16_t *o, hipStream_t s) {
    return launch_attn<kModeSparse>(D, q, k, v, col_idx, recs, meta, (int)n_idx, o, s);
}

hipError_t launch_dense_attn(const Dims &D, const uint16_t *q, const uint16_t *k,
                             const uint16_t *v, uint16_t *o, hipStream_t s) {
    // Dense rows have no block lists, so 128 queries can share every K/V tile
    // (half the tile loads per flop).  Each wave still holds the same 32
    // queries and walks the same 32-key chunks in the same order, so the
    // output is the same as with 64-query workgroups, bit for bit.
    if (D.B == 64 && D.L % 128 == 0) {
        Dims D2 = D;
        D2.B = 128;
        D2.nb = D.L / 128;
        return launch_attn<kModeDense>(D2, q, k, v, nullptr, nullptr, nullptr, 0, o, s);
    }
    return launch_attn<kModeDense>(D, q, k, v, nullptr, nullptr, nullptr, 0, o, s);
}

hipError_t launch_col_attn(const Dims &D, const uint16_t *q, const uint16_t *k,
                           const uint16_t *v, const int32_t *cols, int64_t k_c, uint16_t *o,
                           hipStream_t s) {
    // Every query block of a head attends to the head's same key columns, so
    // 128 queries share each gathered K/V tile, as in dense mode (same output
    // bit for bit).
    if (D.B == 64 && D.L % 128 == 0) {
        Dims D2 = D;
        D2.B = 128;
        D2.nb = D.L / 128;
        return launch_attn<kModeCols>(D2, q, k, v, cols, nullptr, nullptr, (int)k_c, o, s);
    }
    return launch_attn<kModeCols>(D, q, k, v, cols, nullptr, nullptr, (int)k_c, o, s);
}

hipError_t launch_group_attn(const Dims &D, const uint16_t *q, const uint16_t *k,
                             const uint16_t *v, const int32_t *row_ptr, const int32_t *col_idx,
                             int64_t nnz, uint16_t *o, hipStream_t s) {
    if (D.B != 64) return hipErrorInvalidValue;   // the entry point rejects it first
    if (D.d == 128)
        return launch_attn_t<128, 64, kQW, kModeGroup>(D, q, k, v, row_ptr, col_idx, nullptr,
                                                       nullptr, (int)nnz, o, s);
    return launch_attn_t<64, 64, kQW, kModeGroup>(D, q, k, v, row_ptr, col_idx, nullptr,
                                                  nullptr, (int)nnz, o, s);
}

}  // namespace sd
