// Measurement helper: the throughput a loop of one dense MFMA instruction reaches on this
// device, with nothing else in the loop (no loads, no operand forming), for benchmarks to
// report beside the chip's published peak.  Each wavefront keeps 16 independent accumulator
// chains of v_mfma_f32_16x16x32_{f16,bf16}, each updated in place (the instruction is written
// out, so the compiler neither folds chains nor moves accumulators between registers); two
// wavefronts per SIMD, every compute unit busy.
#include <algorithm>

#include "sata_device.h"
#include "sata_internal.h"

namespace sata {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));

constexpr int kChains = 16;
constexpr int kLoopThreads = 256;

template <bool BF16>
__global__ __launch_bounds__(kLoopThreads) void mfma_loop_kernel(int iters, float *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    f32x4 acc[kChains];
#pragma unroll
    for (int i = 0; i < kChains; ++i) acc[i] = f32x4{(float)i, 0.f, 0.f, 0.f};
    if constexpr (BF16) {
        b8 a, b;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[e] = (__bf16)(1e-3f * (lane + e));
            b[e] = (__bf16)(1e-3f * (lane - e));
        }
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < kChains; ++i)
                __asm__ volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[i]) : "v"(a), "v"(b));
        }
    } else {
        h8 a, b;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[e] = (_Float16)(1e-3f * (lane + e));
            b[e] = (_Float16)(1e-3f * (lane - e));
        }
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < kChains; ++i)
                __asm__ volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc[i]) : "v"(a), "v"(b));
        }
    }
    // the last results are complete before they are read
    __asm__ volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kChains; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
    out[blockIdx.x * kLoopThreads + threadIdx.x] = s;
}

}  // namespace

hipError_t measure_mfma_loop(bool bf16, double *tflops) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int grid = std::max(cus, 1) * 2;   // 8 wavefronts per compute unit: two per SIMD
    const int iters = 4096;
    float *out = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if ((e = hipMalloc(&out, (size_t)grid * kLoopThreads * sizeof(float))) != hipSuccess) return e;
    auto launch = [&]() {
        if (bf16) hipLaunchKernelGGL(mfma_loop_kernel<true>, dim3(grid), dim3(kLoopThreads), 0, 0, iters, out);
        else hipLaunchKernelGGL(mfma_loop_kernel<false>, dim3(grid), dim3(kLoopThreads), 0, 0, iters, out);
        return hipGetLastError();
    };
    float ms = 0.f;
    if ((e = hipEventCreate(&e0)) == hipSuccess && (e = hipEventCreate(&e1)) == hipSuccess &&
        (e = launch()) == hipSuccess && (e = hipDeviceSynchronize()) == hipSuccess &&   // warm-up
        (e = hipEventRecord(e0, 0)) == hipSuccess && (e = launch()) == hipSuccess &&
        (e = hipEventRecord(e1, 0)) == hipSuccess && (e = hipEventSynchronize(e1)) == hipSuccess)
        e = hipEventElapsedTime(&ms, e0, e1);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    (void)hipFree(out);
    if (e != hipSuccess) return e;
    const double flops = (double)grid * (kLoopThreads / 64) * iters * kChains * (2.0 * 16 * 16 * 32);
    *tflops = flops / ((double)ms * 1e-3) / 1e12;
    return hipSuccess;
}

}  // namespace sata
