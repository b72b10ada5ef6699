// Standalone feature expansion (tests and inspection).
//
// Writes, for every input row x and every feature f = (i_1..i_p) of order p,
// the key-side monomial prod_r x[i_r] or the query-side value
// prod_r x[i_r] / (alpha_f! d_K^(p/2)), with the same tuple table and the same
// device monomial the decode and prefill kernels use [hotdry, "Core insight
// of symmetric tensor decomposition"; "Engineering realisation of the
// constant compute cost": keys are mapped to the minimal-basis features
// through M_p].  The row is staged in LDS with the constant-1 and constant-0
// slots after its d_K entries.
//
// Grid: (ceil(m_pad / 256), rows); 256 lanes, one feature per lane.
//
//   [hotdry] blog.hotdry.top, "Symmetry-aware Taylor approximation attention:
//            engineering a constant per-token cost" (2026-02-05).
#include <algorithm>

#include "sata_device.h"
#include "sata_internal.h"

namespace sata {

template <typename TIn>
__global__ __launch_bounds__(256) void expand_kernel(const uint32_t *__restrict__ tup,
                                                     const float *__restrict__ coef, int dk,
                                                     int64_t m_pad, const TIn *__restrict__ x,
                                                     float *__restrict__ out, int side) {
    __shared__ float sx[136];   // d_K <= 128 values, then the constant-1 and constant-0 slots
    const int64_t row = blockIdx.y;
    const int tid = threadIdx.x;
    if (tid < dk) sx[tid] = to_f32(x[row * dk + tid]);
    if (tid == 0) { sx[dk] = 1.f; sx[dk + 1] = 0.f; }
    __syncthreads();
    const int64_t f = (int64_t)blockIdx.x * 256 + tid;
    if (f >= m_pad) return;
    const float mono = monomial(tup[f], sx, 1);
    out[row * m_pad + f] = side ? coef[f] * mono : mono;
}

// Zero fill (used instead of hipMemsetAsync so that a caller may capture the
// clear in a HIP graph): count4 16-byte units from p (16-byte aligned), then the
// last count % 4 floats one at a time.
__global__ __launch_bounds__(256) void zero_kernel(float4 *__restrict__ p, int64_t count4, float *__restrict__ tail,
                                                   int ntail) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count4; i += stride)
        p[i] = float4{0.f, 0.f, 0.f, 0.f};
    if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0.f;
}

hipError_t launch_zero(float *p, int64_t count, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    const int64_t count4 = count / 4;
    const int ntail = (int)(count - 4 * count4);
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((count4 + 255) / 256, 8192));
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<float4 *>(p), count4, p + 4 * count4, ntail);
    return hipGetLastError();
}

hipError_t launch_expand(const sata_index *idx, const void *x, void *out, int64_t rows, int side,
                         sata_dtype in_dt, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    const dim3 grid((unsigned)((idx->m_pad + 255) / 256), (unsigned)rows);
    if (in_dt == SATA_F32)
        hipLaunchKernelGGL(expand_kernel<float>, grid, dim3(256), 0, stream, idx->d_tup, idx->d_coef,
                           idx->dk, idx->m_pad, static_cast<const float *>(x), static_cast<float *>(out), side);
    else
        hipLaunchKernelGGL(expand_kernel<bf16_t>, grid, dim3(256), 0, stream, idx->d_tup, idx->d_coef,
                           idx->dk, idx->m_pad, static_cast<const bf16_t *>(x), static_cast<float *>(out), side);
    return hipGetLastError();
}

}  // namespace sata
