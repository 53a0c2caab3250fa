// Data-path rates of the chip at the attention kernel's occupancy: a
// measurement aid for the attention kernel's roofline, not part of the
// library.
//
// Four workgroups of two waves per CU, 40 KiB of LDS each, as the d = 128,
// 64-token-block attention kernel runs.  Per wave and loop iteration:
//   fill   8 buffer->LDS loads of 1 KiB (one 32-key step's share of a K and a
//          V tile), one iteration of loads kept in flight, from a 1 MiB
//          source that stays in L2
//   b128   8 ds_read_b128 (a step's K fragments, 8 KiB per wave)
//   tr     16 ds_read_b64_tr_b16 (a step's V fragments, 8 KiB per wave)
//   step   a step's reads and loads plus its 16 MFMAs (8 chained score
//          products on the K fragments, 8 value products on the V
//          fragments), without the softmax
//   mfma   the 16 MFMAs alone, on register operands
// Each workgroup reads the shader clock counter (s_memtime) and the constant
// 100 MHz counter (s_memrealtime) around its loop, which gives the clock the
// chip held; cycles per iteration are the launch's wall time per iteration at
// that clock.  Then a streaming read of 128 MiB with non-temporal 16-byte
// loads (512 workgroups of 256 threads), rotating over 8 buffers so that no
// pass is served by the 256 MB last-level cache: median of 40 passes.
//
// Prints one JSON line.  Every LDS address stays below 40 KiB, every buffer
// offset inside its buffer.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <vector>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define PR_LDS __attribute__((address_space(3)))

constexpr int kLdsBytes = 40960;
constexpr int kFillBase = 24576;          // fill region: 16 x 1 KiB at the top of LDS
constexpr int kSrcBytes = 1 << 20;
constexpr int kModes = 5;
enum { kFill = 0, kB128 = 1, kTr = 2, kStep = 3, kMfma = 4 };
const char *const kNames[kModes] = {"fill", "b128", "tr", "step", "mfma"};

template <int MODE>
__global__ __launch_bounds__(128) void k_path(const uint16_t *__restrict__ src,
                                              float *__restrict__ sink,
                                              uint64_t *__restrict__ times, int iters) {
    constexpr bool FILL = MODE == kFill || MODE == kStep;
    constexpr bool B128 = MODE == kB128 || MODE == kStep;
    constexpr bool TR = MODE == kTr || MODE == kStep;
    constexpr bool MF = MODE == kStep || MODE == kMfma;
    __shared__ __attribute__((aligned(16))) uint16_t lds[kLdsBytes / 2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    for (int i = tid; i < kLdsBytes / 2; i += 128) lds[i] = (uint16_t)(0x3c00 + ((i * 37) & 0xff));
    __syncthreads();
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)src, 0, kSrcBytes, 0x00020000);
    const char *base = reinterpret_cast<const char *>(lds);
    uint32_t x = 0;
    f32x16 sacc, oacc[4];
    for (int i = 0; i < 16; ++i) {
        sacc[i] = 0.0f;
        for (int m = 0; m < 4; ++m) oacc[m][i] = 0.0f;
    }
    const bf16x8 qf =
        __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(base + lane * 16));
    const bf16x8 pf =
        __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(base + 1024 + lane * 16));
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        asm volatile("" ::: "memory");   // the reads below are issued every iteration
        const int half = (it & 1) * 8192;   // reads stay in [0, 16 KiB)
        bf16x8 kf[8], vf[8];
        if (B128) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint4 v =
                    *reinterpret_cast<const uint4 *>(base + half + j * 1024 + lane * 16);
                kf[j] = __builtin_bit_cast(bf16x8, v);
                if (!MF) x ^= v.x ^ v.y ^ v.z ^ v.w;
            }
        }
        if (TR) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                i16x4 p[2];
#pragma unroll
                for (int r = 0; r < 2; ++r)
                    p[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (PR_LDS i16x4 *)(base + half + (2 * j + r) * 512 + lane * 8));
                vf[j] = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(p[0], p[1], 0, 1, 2, 3, 4, 5, 6, 7));
                if (!MF) x ^= __builtin_bit_cast(uint2, p[0]).x ^ __builtin_bit_cast(uint2, p[1]).x;
            }
        }
        if (FILL) {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int blk = (blockIdx.x * 16 + it * 8 + wave * 8 + t) & 1023;   // < 1 MiB
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsrc, (PR_LDS void *)(base + kFillBase + (wave * 8 + t) * 1024), 16,
                    (uint32_t)(lane * 16), (uint32_t)(blk * 1024), 0, 0);
            }
        }
        if (MF) {
            if (MODE == kMfma) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    kf[j] = qf;
                    vf[j] = pf;
                }
            }
            f32x16 s = sacc;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[j], qf, s, 0, 0, 0);
            sacc = s;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    oacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[4 * ks + m], pf,
                                                                      oacc[m], 0, 0, 0);
        }
        if (MODE == kFill) {
            asm volatile("s_waitcnt vmcnt(8)" ::: "memory");   // one iteration in flight
            __syncthreads();
        }
        if (MODE == kStep) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the step's loads landed
            __syncthreads();
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    float s = (float)x;
    for (int i = 0; i < 16; ++i) s += sacc[i] + oacc[0][i] + oacc[1][i] + oacc[2][i] + oacc[3][i];
    sink[blockIdx.x * 128 + tid] = s;
    if (tid == 0) {
        times[2 * blockIdx.x] = t1 - t0;
        times[2 * blockIdx.x + 1] = r1 - r0;
    }
}

__global__ __launch_bounds__(256) void k_stream(const u32x4 *__restrict__ p, size_t n16,
                                                uint32_t *__restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t x = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(p + i);
        const u32x4 b = __builtin_nontemporal_load(p + i + stride);
        const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
        const u32x4 e = a ^ b ^ c ^ d;
        x ^= e.x ^ e.y ^ e.z ^ e.w;
    }
    for (; i < n16; i += stride) {
        const u32x4 a = __builtin_nontemporal_load(p + i);
        x ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    sink[(size_t)blockIdx.x * 256 + threadIdx.x] = x;
}

bool ok(hipError_t e, const char *what) {
    if (e != hipSuccess) {
        std::fprintf(stderr, "path_rates: %s: %s\n", what, hipGetErrorString(e));
        return false;
    }
    return true;
}

struct Rate {
    double ns_per_iter, ghz, cycles_per_iter;
};

template <int MODE>
bool run_mode(int wgs, const uint16_t *src, float *sink, uint64_t *t, int iters, Rate &out) {
    hipEvent_t e0, e1;
    if (!ok(hipEventCreate(&e0), "hipEventCreate") || !ok(hipEventCreate(&e1), "hipEventCreate"))
        return false;
    hipLaunchKernelGGL(k_path<MODE>, dim3(wgs), dim3(128), 0, 0, src, sink, t, iters / 8);
    if (!ok(hipGetLastError(), "launch") || !ok(hipDeviceSynchronize(), "warm-up")) return false;
    if (!ok(hipEventRecord(e0, 0), "hipEventRecord")) return false;
    hipLaunchKernelGGL(k_path<MODE>, dim3(wgs), dim3(128), 0, 0, src, sink, t, iters);
    if (!ok(hipGetLastError(), "launch") || !ok(hipEventRecord(e1, 0), "hipEventRecord") ||
        !ok(hipEventSynchronize(e1), "run"))
        return false;
    float ms = 0.0f;
    if (!ok(hipEventElapsedTime(&ms, e0, e1), "hipEventElapsedTime")) return false;
    std::vector<uint64_t> h(2 * (size_t)wgs);
    if (!ok(hipMemcpy(h.data(), t, h.size() * 8, hipMemcpyDeviceToHost), "hipMemcpy")) return false;
    double cyc = 0.0, us = 0.0;
    for (int w = 0; w < wgs; ++w) {
        cyc += (double)h[2 * w];
        us += (double)h[2 * w + 1] / 100.0;   // 100 MHz counter
    }
    out.ghz = cyc / us / 1e3;
    out.ns_per_iter = ms * 1e6 / iters;
    out.cycles_per_iter = out.ns_per_iter * out.ghz;
    return ok(hipEventDestroy(e0), "hipEventDestroy") && ok(hipEventDestroy(e1), "hipEventDestroy");
}

bool stream_rate(int grid, double &gbs_median, double &gbs_best) {
    const size_t bytes = (size_t)128 << 20, n16 = bytes / 16;
    std::vector<u32x4 *> bufs(8, nullptr);
    uint32_t *sink = nullptr;
    bool good = ok(hipMalloc(&sink, (size_t)grid * 256 * 4), "hipMalloc");
    for (auto &b : bufs)
        good = good && ok(hipMalloc(&b, bytes), "hipMalloc") &&
               ok(hipMemset(b, 1, bytes), "hipMemset");
    hipEvent_t e0, e1;
    good = good && ok(hipEventCreate(&e0), "hipEventCreate") &&
           ok(hipEventCreate(&e1), "hipEventCreate");
    std::vector<float> ts;
    for (int r = 0; good && r < 48; ++r) {
        good = ok(hipEventRecord(e0, 0), "hipEventRecord");
        hipLaunchKernelGGL(k_stream, dim3(grid), dim3(256), 0, 0, bufs[r % 8], n16, sink);
        good = good && ok(hipGetLastError(), "launch") &&
               ok(hipEventRecord(e1, 0), "hipEventRecord") && ok(hipEventSynchronize(e1), "stream");
        float ms = 0.0f;
        good = good && ok(hipEventElapsedTime(&ms, e0, e1), "hipEventElapsedTime");
        if (r >= 8) ts.push_back(ms);   // the first pass over each buffer is a warm-up
    }
    if (good) {
        std::sort(ts.begin(), ts.end());
        gbs_median = bytes / (double)ts[ts.size() / 2] / 1e6;
        gbs_best = bytes / (double)ts[0] / 1e6;
        good = ok(hipEventDestroy(e0), "hipEventDestroy") &&
               ok(hipEventDestroy(e1), "hipEventDestroy");
    }
    for (auto b : bufs)
        if (b) good = ok(hipFree(b), "hipFree") && good;
    if (sink) good = ok(hipFree(sink), "hipFree") && good;
    return good;
}

}  // namespace

int main() {
    hipDeviceProp_t prop;
    int dev = 0;
    if (!ok(hipGetDevice(&dev), "hipGetDevice") ||
        !ok(hipGetDeviceProperties(&prop, dev), "hipGetDeviceProperties"))
        return 1;
    const int cus = prop.multiProcessorCount, wgs = cus * 4;   // all resident at once
    uint16_t *src = nullptr;
    float *sink = nullptr;
    uint64_t *t = nullptr;
    if (!ok(hipMalloc(&src, kSrcBytes), "hipMalloc") ||
        !ok(hipMemset(src, 0x3c, kSrcBytes), "hipMemset") ||
        !ok(hipMalloc(&sink, sizeof(float) * 128 * wgs), "hipMalloc") ||
        !ok(hipMalloc(&t, sizeof(uint64_t) * 2 * wgs), "hipMalloc"))
        return 1;
    const int iters = 8192;
    Rate r[kModes];
    if (!run_mode<kFill>(wgs, src, sink, t, iters, r[kFill]) ||
        !run_mode<kB128>(wgs, src, sink, t, iters, r[kB128]) ||
        !run_mode<kTr>(wgs, src, sink, t, iters, r[kTr]) ||
        !run_mode<kStep>(wgs, src, sink, t, iters, r[kStep]) ||
        !run_mode<kMfma>(wgs, src, sink, t, iters, r[kMfma]))
        return 1;
    double med = 0.0, best = 0.0;
    if (!stream_rate(512, med, best)) return 1;
    // Bytes per CU and iteration: 8 waves x 8 KiB filled or read.
    const double fill_b = 8.0 * 8192, read_b = 8.0 * 8192;
    std::printf("{\"cus\": %d, \"waves_per_cu\": 8, \"iters\": %d", cus, iters);
    for (int m = 0; m < kModes; ++m) {
        std::printf(", \"%s\": {\"ns_per_iter\": %.1f, \"ghz\": %.3f, \"cycles_per_iter\": %.0f",
                    kNames[m],
                    r[m].ns_per_iter, r[m].ghz, r[m].cycles_per_iter);
        if (m == kFill)
            std::printf(", \"bytes_per_clk_per_cu\": %.1f", fill_b / r[m].cycles_per_iter);
        if (m == kB128 || m == kTr)
            std::printf(", \"bytes_per_clk_per_cu\": %.1f", read_b / r[m].cycles_per_iter);
        std::printf("}");
    }
    std::printf(", \"stream_read_128mib\": {\"gbs_median\": %.0f, \"gbs_best\": %.0f, "
                "\"frac_of_8tbs\": %.3f}}\n",
                med, best, med / 8000.0);
    return ok(hipFree(src), "hipFree") && ok(hipFree(sink), "hipFree") &&
                   ok(hipFree(t), "hipFree")
               ? 0
               : 1;
}
