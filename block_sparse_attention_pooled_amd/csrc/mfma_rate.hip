// Sustained bf16 MFMA rate of this GPU: a measurement aid for the attention
// kernels' roofline, not part of the library.
//
// One wave per SIMD on every CU runs 8 independent v_mfma_f32_32x32x16_bf16
// accumulation chains (no memory traffic, no VALU work in the loop) on
// operands drawn either from N(0, 1) (rounded to bf16) or all zero.  Each wave
// reads the shader clock counter (s_memtime) and the constant 100 MHz counter
// (s_memrealtime) around the loop, so the run reports the MFMA rate and the
// shader clock the chip actually held under that load.  On MI355X the clock,
// and with it the rate, depends on the operand values: the power drawn by the
// matrix cores does.
//
// Prints one JSON line: {"random": {...}, "zero": {...}} with TFLOP/s, GHz
// and cycles per MFMA for each operand kind.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChains = 8;
constexpr int kOperands = 4;
constexpr int kSrcVectors = 1 << 16;   // uint4 operand vectors in the source buffer

__global__ __launch_bounds__(64) void k_mfma_rate(const uint4 *__restrict__ src,
                                                  float *__restrict__ sink,
                                                  uint64_t *__restrict__ times, int iters) {
    const int gid = blockIdx.x * 64 + threadIdx.x;
    bf16x8 a[kOperands], b[kOperands];
#pragma unroll
    for (int i = 0; i < kOperands; ++i) {
        a[i] = __builtin_bit_cast(bf16x8, src[(gid * 2 * kOperands + i) % kSrcVectors]);
        b[i] = __builtin_bit_cast(bf16x8, src[(gid * 2 * kOperands + kOperands + i) % kSrcVectors]);
    }
    f32x16 acc[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][i] = 0.0f;
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; it += kOperands) {
#pragma unroll
        for (int u = 0; u < kOperands; ++u)
#pragma unroll
            for (int j = 0; j < kChains; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    a[j % kOperands], b[(j + u) % kOperands], acc[j], 0, 0, 0);
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kChains; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += acc[j][i];
    sink[gid] = s;   // keeps the chains live
    if (threadIdx.x == 0) {
        times[2 * blockIdx.x] = t1 - t0;
        times[2 * blockIdx.x + 1] = r1 - r0;
    }
}

bool ok(hipError_t e, const char *what) {
    if (e != hipSuccess) {
        std::fprintf(stderr, "mfma_rate: %s: %s\n", what, hipGetErrorString(e));
        return false;
    }
    return true;
}

}  // namespace

int main() {
    int dev = 0;
    hipDeviceProp_t prop;
    if (!ok(hipGetDevice(&dev), "hipGetDevice") ||
        !ok(hipGetDeviceProperties(&prop, dev), "hipGetDeviceProperties"))
        return 1;
    const int waves = prop.multiProcessorCount * 4;   // one wave per SIMD
    const int iters = 20000;                           // a multiple of kOperands
    uint4 *d_src = nullptr;
    float *d_sink = nullptr;
    uint64_t *d_t = nullptr;
    if (!ok(hipMalloc(&d_src, sizeof(uint4) * kSrcVectors), "hipMalloc") ||
        !ok(hipMalloc(&d_sink, sizeof(float) * waves * 64), "hipMalloc") ||
        !ok(hipMalloc(&d_t, sizeof(uint64_t) * 2 * waves), "hipMalloc"))
        return 1;
    std::vector<uint16_t> h((size_t)kSrcVectors * 8);
    std::mt19937 g(7);
    std::normal_distribution<float> nd(0.0f, 1.0f);
    std::printf("{");
    for (int kind = 0; kind < 2; ++kind) {
        for (auto &x : h) {
            const float f = kind == 0 ? nd(g) : 0.0f;
            uint32_t u;
            std::memcpy(&u, &f, 4);
            x = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);   // bf16, nearest even
        }
        if (!ok(hipMemcpy(d_src, h.data(), h.size() * 2, hipMemcpyHostToDevice), "hipMemcpy"))
            return 1;
        hipEvent_t e0, e1;
        if (!ok(hipEventCreate(&e0), "hipEventCreate") || !ok(hipEventCreate(&e1), "hipEventCreate"))
            return 1;
        hipLaunchKernelGGL(k_mfma_rate, dim3(waves), dim3(64), 0, 0, d_src, d_sink, d_t, iters / 4);
        if (!ok(hipDeviceSynchronize(), "warm-up")) return 1;
        hipEventRecord(e0, 0);
        hipLaunchKernelGGL(k_mfma_rate, dim3(waves), dim3(64), 0, 0, d_src, d_sink, d_t, iters);
        hipEventRecord(e1, 0);
        if (!ok(hipEventSynchronize(e1), "run")) return 1;
        float ms = 0.0f;
        hipEventElapsedTime(&ms, e0, e1);
        std::vector<uint64_t> t(2 * (size_t)waves);
        if (!ok(hipMemcpy(t.data(), d_t, t.size() * 8, hipMemcpyDeviceToHost), "hipMemcpy"))
            return 1;
        double cyc = 0.0, real_us = 0.0;
        for (int w = 0; w < waves; ++w) {
            cyc += (double)t[2 * w];
            real_us += (double)t[2 * w + 1] / 100.0;   // 100 MHz counter
        }
        cyc /= waves;
        real_us /= waves;
        const double mfmas = (double)kChains * iters;
        const double flops = 2.0 * 32 * 32 * 16 * mfmas * waves;
        std::printf("%s\"%s\": {\"tflops\": %.1f, \"ghz\": %.3f, \"cycles_per_mfma\": %.2f, "
                    "\"ms\": %.3f, \"waves\": %d}",
                    kind ? ", " : "", kind == 0 ? "random" : "zero", flops / ms / 1e9,
                    cyc / real_us / 1e3, cyc / mfmas, ms, waves);
        hipEventDestroy(e0);
        hipEventDestroy(e1);
    }
    std::printf("}\n");
    hipFree(d_src);
    hipFree(d_sink);
    hipFree(d_t);
    return 0;
}
