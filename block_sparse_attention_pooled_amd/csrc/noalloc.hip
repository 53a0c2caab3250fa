// stepdllm_step_noalloc: the denoising step of stepdllm_step for callers that
// cannot allocate device memory (code under HIP graph capture, serving loops
// or harnesses that forbid hipMalloc).  The workspace every mask build and
// sparse launch needs (pooled means, scores, select state, work order and
// plan records) is a static device array of this file instead of a
// caller-owned buffer.  Host code only, apart from the array.
#include <mutex>

#include "../../include/stepdllm.h"
#include "common.h"

// The workspace of stepdllm_step_noalloc: one copy per GPU the library runs
// on, held until the process ends.  In host code the name is only a handle
// for hipGetSymbolAddress (the address of the current device's copy), never a
// device address: kernels are given that looked-up address.
static __device__ __align__(256) char scratch[STEPDLLM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int64_t kScratchBytes = STEPDLLM_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

std::mutex g_mu;
void *g_addr[kMaxDevices];   // device address of `scratch` on each device, once looked up

// The current device's copy of the array (looked up once per device, with
// that device current).
int scratch_address(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return STEPDLLM_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return STEPDLLM_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_addr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return STEPDLLM_EHIP;
        g_addr[dev] = p;
    }
    *out = g_addr[dev];
    return STEPDLLM_OK;
}

}  // namespace

extern "C" int stepdllm_step_noalloc(const stepdllm_dims *dims,
                                     const stepdllm_schedule *schedule, int32_t step,
                                     const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                     int32_t *row_ptr, int32_t *col_idx, uint16_t *o,
                                     void *stream) {
    const int64_t need = stepdllm_workspace_bytes(dims);
    if (need < 0) return (int)need;
    if (!schedule || step < 0 || !q || !k || !v || !o || !col_idx) return STEPDLLM_EINVAL;
    if (schedule->dense_steps < 0 || schedule->refresh_every < 0 ||
        !(schedule->sparsity >= 0.0 && schedule->sparsity <= 1.0) ||
        (schedule->per_head_budget != 0 && schedule->per_head_budget != 1) ||
        (schedule->column_sparse != 0 && schedule->column_sparse != 1) ||
        (schedule->column_sparse && schedule->per_head_budget) ||
        (!schedule->column_sparse && !row_ptr))
        return STEPDLLM_EINVAL;
    if (need > kScratchBytes) return STEPDLLM_EWORKSPACE;
    void *ws = nullptr;
    int st = scratch_address(&ws);
    if (st) return st;
    // The step kind of the schedule (as stepdllm_driver_step_kind).
    const int32_t since = step - schedule->dense_steps;
    if (since < 0) return stepdllm_dense_attn(dims, q, k, v, o, stream);
    const bool anchor =
        since == 0 || (schedule->refresh_every > 0 && since % schedule->refresh_every == 0);
    const double s = schedule->sparsity;
    const size_t ws_bytes = (size_t)kScratchBytes;
    if (schedule->column_sparse) {
        const int64_t k_c = stepdllm_keep_count_columns(dims, s);
        if (k_c < 0) return (int)k_c;
        if (anchor &&
            (st = stepdllm_build_col_mask(dims, s, q, k, ws, ws_bytes, col_idx, nullptr, stream)))
            return st;
        return stepdllm_col_attn(dims, q, k, v, col_idx, k_c, o, stream);
    }
    const int64_t K = schedule->per_head_budget ? stepdllm_keep_count_per_head(dims, s)
                                                : stepdllm_keep_count(dims, s);
    if (K < 0) return (int)K;
    if (anchor) {
        st = schedule->per_head_budget
                 ? stepdllm_build_mask_per_head(dims, s, q, k, ws, ws_bytes, row_ptr, col_idx,
                                                nullptr, stream)
                 : stepdllm_build_mask(dims, s, q, k, ws, ws_bytes, row_ptr, col_idx, nullptr,
                                       stream);
        if (st) return st;
    }
    return stepdllm_sparse_attn(dims, q, k, v, col_idx, K, ws, ws_bytes, o, stream);
}
