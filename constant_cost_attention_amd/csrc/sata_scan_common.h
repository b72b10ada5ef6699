// Device helpers shared by the prefill scans (sata_prefill.hip, sata_scan16.hip):
// decoding of the quad words of the prefill's feature view, the truncated
// exponential weight of the intra-chunk term, and the persistent scans' bounded
// wait for a predecessor work item.
//
//   [hotdry] blog.hotdry.top, "Symmetry-aware Taylor approximation attention:
//            engineering a constant per-token cost" (2026-02-05).
#pragma once

#include "sata_device.h"
#include "sata_internal.h"

namespace sata {

__device__ __forceinline__ int qd_i1(uint32_t w) { return (int)(w & 0xffu); }
__device__ __forceinline__ int qd_i2(uint32_t w) { return (int)((w >> 8) & 0xffu); }
__device__ __forceinline__ int qd_i0(uint32_t w) { return (int)((w >> 16) & 0xffu); }
__device__ __forceinline__ int qd_b(uint32_t w) { return (int)((w >> 24) & 0xfu); }
__device__ __forceinline__ uint32_t qd_mask(uint32_t w) { return w >> 28; }
// alpha! of the quad's prefix (i0, i1, i2) (sorted; absent indices are >= D),
// and its reciprocal, the prefix's share of the multinomial readout weight.
// Without order-4 features (TRIPLE false) i0 is always absent.
template <int D, bool TRIPLE> __device__ __forceinline__ float qd_pfact(uint32_t w) {
    const int i1 = qd_i1(w), i2 = qd_i2(w);
    const bool e12 = i1 == i2 && i1 < D;
    if constexpr (!TRIPLE) return e12 ? 2.f : 1.f;
    const int i0 = qd_i0(w);
    const bool e01 = i0 == i1 && i0 < D;
    return e01 ? (e12 ? 6.f : 2.f) : (e12 ? 2.f : 1.f);
}
template <int D, bool TRIPLE> __device__ __forceinline__ float qd_pweight(uint32_t w) {
    const int i1 = qd_i1(w), i2 = qd_i2(w);
    const bool e12 = i1 == i2 && i1 < D;
    if constexpr (!TRIPLE) return e12 ? 0.5f : 1.f;
    const int i0 = qd_i0(w);
    const bool e01 = i0 == i1 && i0 < D;
    return e01 ? (e12 ? 1.f / 6.f : 0.5f) : (e12 ? 0.5f : 1.f);
}

// w(x) = sum_{p<P} x^p/p! (Horner, P <= 5)
__device__ __forceinline__ float taylor_w(float x, float c0, float c1, float c2, float c3, float c4, int P) {
    float w = P >= 5 ? c4 : 0.f;
    if (P >= 4) w = w * x + c3;
    if (P >= 3) w = w * x + c2;
    if (P >= 2) w = w * x + c1;
    return w * x + c0;
}

struct TaylorArgs {
    float scale, c0, c1, c2, c3, c4;
    int P;
    int raw;          // write the numerator y[:d_V] unnormalised
};

// A persistent scan's wait for the state its predecessor item leaves: poll the item's progress
// flag (agent-scope acquire) until it reaches `need`, at most spin_limit times.  A wait that
// runs out sets kErrScanWait in the state's error word (pinned host memory, system scope; NULL
// for internal states whose caller checks otherwise) and returns, so the kernel still ends;
// the call's output and state are then invalid and the host reports it.
__device__ __forceinline__ void wait_predecessor(uint32_t *flag, uint32_t need, int spin_limit, uint32_t *err) {
    for (int spin = 0; spin < spin_limit; ++spin) {
        if (__hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) >= need) return;
        __builtin_amdgcn_s_sleep(2);
    }
    if (__hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) >= need) return;
    if (err) __hip_atomic_fetch_or(err, kErrScanWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

}  // namespace sata
