// Fused SATA decode step for gfx950.
//
// One new token per head.  For every feature f of every order the kernel reads
// the state column S[:, f] once, adds the key monomial times [v, 1], writes it
// back and, in the same pass, accumulates the query-weighted readout
// [hotdry, "Engineering realisation of the constant compute cost": per token,
// map k through M_p, accumulate into the fixed state, weight and sum the
// orders' contributions].  All orders run in the same grid [hotdry, "Hardware
// optimisation paths and current limits": the orders have no data dependence].
//
// Work is HBM-bound: 2 * sizeof(state element) * m * (d_V + 1) bytes per
// head-token of state traffic against 4 * m * (d_V + 1) FLOPs.  Layout of the
// state: [bh][d_V+1][m_pad] fp32 or bf16, so a wavefront's 64 lanes touch
// 64 * FPT consecutive features of one row: fully coalesced 16-byte accesses.
// A bf16 state is widened to fp32 in registers, updated and read out there, and
// rounded (to nearest even) only when stored: half the bytes of the fp32 state
// [hotdry, "Hardware optimisation paths and current limits": half-precision
// storage halves the bandwidth].
//
// Grid: (ceil(m_pad / (256 * FPT)), B*H) workgroups of 256 lanes; lane owns FPT
// consecutive features (4 fp32 or 8 bf16), i.e. one 16-byte word of every state
// row.  Each workgroup leaves d_V+1 partial sums; a second, tiny kernel adds the
// partials of a head in a fixed order and normalises, so results are
// deterministic.
//
//   [hotdry] blog.hotdry.top, "Symmetry-aware Taylor approximation attention:
//            engineering a constant per-token cost" (2026-02-05).
#include "sata_device.h"
#include "sata_internal.h"

namespace sata {

constexpr int kDecThreads = 256;
template <typename TS> constexpr int dec_fpt() { return 16 / (int)sizeof(TS); }   // features per lane

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // one 16-byte word of a state row

// A state word as fp32 values, and back.
__device__ __forceinline__ void widen(const u32x4 u, float (&x)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = __uint_as_float(u[j]);
}
__device__ __forceinline__ void widen(const u32x4 u, float (&x)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[2 * j] = __uint_as_float(u[j] << 16);
        x[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
    }
}
__device__ __forceinline__ u32x4 narrow(const float (&x)[4]) {
    return u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
}
__device__ __forceinline__ u32x4 narrow(const float (&x)[8]) {
    return u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
}

// Wave-level reduce-scatter of DV (power of two) per-lane values followed by a
// plain reduction across the remaining lane groups: afterwards lane l holds the
// wavefront sum of column (l % DV).
template <int DV>
__device__ __forceinline__ float wave_reduce_scatter(float (&a)[DV]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int half = DV / 2; half >= 1; half /= 2) {
        const bool upper = (lane & half) != 0;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            const float send = upper ? a[i] : a[i + half];
            const float keep = upper ? a[i + half] : a[i];
            a[i] = keep + __shfl_xor(send, half, 64);
        }
    }
    float r = a[0];
#pragma unroll
    for (int off = DV; off < 64; off *= 2) r += __shfl_xor(r, off, 64);
    return r;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off /= 2) x += __shfl_xor(x, off, 64);
    return x;
}

// The lane's column loads are issued in two batches of ~(d_V+1)/2 rows, the
// second batch before any store of the first, so each lane keeps up to d_V+1
// 16-byte loads in flight; one wavefront per SIMD then saturates the HBM
// read-modify-write stream (the state is far larger than every cache).
template <int DV, typename TIn, typename TS>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_kernel(const uint32_t *__restrict__ tup, const float *__restrict__ coef, TS *__restrict__ state,
                   int64_t m_pad, int dk, const TIn *__restrict__ q, const TIn *__restrict__ k,
                   const TIn *__restrict__ v, float *__restrict__ partial) {
    constexpr int NC = DV + 1;
    constexpr int R = (NC + 1) / 2;          // rows per load batch
    constexpr int FPT = dec_fpt<TS>();
    __shared__ float sq[72], sk[72], sv[NC];
    __shared__ float red[kDecThreads / 64][NC];
    const int bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t f0 = ((int64_t)blockIdx.x * kDecThreads + tid) * FPT;
    const bool valid = f0 < m_pad;   // m_pad is a multiple of 64, so all FPT features are in range
    TS *Sb = state + (int64_t)bh * NC * m_pad + f0;
    auto row = [&](int r) { return reinterpret_cast<u32x4 *>(Sb + (int64_t)r * m_pad); };

    // first batch of state rows goes out before anything else
    u32x4 s0[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (valid) s0[r] = __builtin_nontemporal_load(row(r));
    uint4 t4[FPT / 4];
    float4 c4[FPT / 4];
#pragma unroll
    for (int h = 0; h < FPT / 4; ++h) {
        t4[h] = uint4{0u, 0u, 0u, 0u};
        c4[h] = float4{0.f, 0.f, 0.f, 0.f};
        if (valid) {
            t4[h] = *reinterpret_cast<const uint4 *>(tup + f0 + 4 * h);
            c4[h] = *reinterpret_cast<const float4 *>(coef + f0 + 4 * h);
        }
    }
    if (tid < dk) {
        sq[tid] = to_f32(q[(int64_t)bh * dk + tid]);
        sk[tid] = to_f32(k[(int64_t)bh * dk + tid]);
    }
    if (tid == 0) {
        sq[dk] = 1.f; sk[dk] = 1.f; sq[dk + 1] = 0.f; sk[dk + 1] = 0.f;
        sv[DV] = 1.f;
    }
    if (tid < DV) sv[tid] = to_f32(v[(int64_t)bh * DV + tid]);
    __syncthreads();

    float phk[FPT], psq[FPT];
#pragma unroll
    for (int h = 0; h < FPT / 4; ++h) {
        const uint32_t tt[4] = {t4[h].x, t4[h].y, t4[h].z, t4[h].w};
        const float cc[4] = {c4[h].x, c4[h].y, c4[h].z, c4[h].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            phk[4 * h + j] = monomial(tt[j], sk, 1);
            psq[4 * h + j] = cc[j] * monomial(tt[j], sq, 1);
        }
    }

    // second batch in flight while the first is updated, stored and read out
    u32x4 s1[NC - R];
#pragma unroll
    for (int r = 0; r < NC - R; ++r)
        if (valid) s1[r] = __builtin_nontemporal_load(row(R + r));
    float acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        float x[FPT];
        widen(c < R ? s0[c] : s1[c - R], x);
        const float vc = sv[c];
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < FPT; ++j) {
            x[j] += phk[j] * vc;
            a += psq[j] * x[j];
        }
        if (valid) __builtin_nontemporal_store(narrow(x), row(c));
        acc[c] = valid ? a : 0.f;
    }

    // workgroup reduction of the d_V + 1 readout sums
    float vals[DV];
#pragma unroll
    for (int c = 0; c < DV; ++c) vals[c] = acc[c];
    const float col = wave_reduce_scatter<DV>(vals);
    const float den = wave_sum(acc[DV]);
    const int lane = tid & 63, wave = tid >> 6;
    if (lane < DV) red[wave][lane] = col;
    if (lane == 0) red[wave][DV] = den;
    __syncthreads();
    if (tid < NC) {
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kDecThreads / 64; ++w) sum += red[w][tid];
        partial[((int64_t)bh * gridDim.x + blockIdx.x) * NC + tid] = sum;
    }
}

// Adds a head's partial sums in block order and divides by the normaliser.
template <int DV, typename TOut>
__global__ __launch_bounds__(128) void decode_finish_kernel(const float *__restrict__ partial, int nblk,
                                                            TOut *__restrict__ out) {
    constexpr int NC = DV + 1;
    __shared__ float y[NC];
    const int bh = blockIdx.x, tid = threadIdx.x;
    if (tid < NC) {
        float s = 0.f;
        for (int b = 0; b < nblk; ++b) s += partial[((int64_t)bh * nblk + b) * NC + tid];
        y[tid] = s;
    }
    __syncthreads();
    if (tid < DV) out[(int64_t)bh * DV + tid] = from_f32<TOut>(y[tid] / y[DV]);
}

static int64_t decode_blocks(const sata_index *idx, int fpt) {
    const int64_t per = (int64_t)kDecThreads * fpt;
    return (idx->m_pad + per - 1) / per;
}

int64_t decode_workspace_bytes(const sata_index *idx, int64_t bh) {
    return bh * decode_blocks(idx, 4) * (idx->dv + 1) * (int64_t)sizeof(float);   // the larger (fp32) grid
}

template <int DV, typename TIn, typename TOut, typename TS>
static hipError_t launch_decode_t(const sata_index *idx, const sata_state *st, const void *q,
                                  const void *k, const void *v, void *out, hipStream_t stream) {
    const int64_t bh = (int64_t)st->batch * st->heads;
    const int nblk = (int)decode_blocks(idx, dec_fpt<TS>());
    float *partial = static_cast<float *>(st->d_work);
    {
        ProfScope ps(kProfDecode, stream);
        hipLaunchKernelGGL((decode_kernel<DV, TIn, TS>), dim3(nblk, (unsigned)bh), dim3(kDecThreads), 0, stream,
                           idx->d_tup, idx->d_coef, static_cast<TS *>(st->d_state), idx->m_pad, idx->dk,
                           static_cast<const TIn *>(q), static_cast<const TIn *>(k),
                           static_cast<const TIn *>(v), partial);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    {
        ProfScope ps(kProfDecodeFinish, stream);
        hipLaunchKernelGGL((decode_finish_kernel<DV, TOut>), dim3((unsigned)bh), dim3(128), 0, stream,
                           partial, nblk, static_cast<TOut *>(out));
    }
    return hipGetLastError();
}

template <int DV, typename TS>
static hipError_t launch_decode_ts(const sata_index *idx, const sata_state *st, const void *q,
                                   const void *k, const void *v, void *out, sata_dtype in_dt,
                                   sata_dtype out_dt, hipStream_t s) {
    if (in_dt == SATA_F32 && out_dt == SATA_F32) return launch_decode_t<DV, float, float, TS>(idx, st, q, k, v, out, s);
    if (in_dt == SATA_F32 && out_dt == SATA_BF16) return launch_decode_t<DV, float, bf16_t, TS>(idx, st, q, k, v, out, s);
    if (in_dt == SATA_BF16 && out_dt == SATA_F32) return launch_decode_t<DV, bf16_t, float, TS>(idx, st, q, k, v, out, s);
    return launch_decode_t<DV, bf16_t, bf16_t, TS>(idx, st, q, k, v, out, s);
}

template <int DV>
static hipError_t launch_decode_dv(const sata_index *idx, const sata_state *st, const void *q,
                                   const void *k, const void *v, void *out, sata_dtype in_dt,
                                   sata_dtype out_dt, hipStream_t s) {
    if (st->dtype == SATA_BF16) return launch_decode_ts<DV, bf16_t>(idx, st, q, k, v, out, in_dt, out_dt, s);
    return launch_decode_ts<DV, float>(idx, st, q, k, v, out, in_dt, out_dt, s);
}

// Element-wise state conversion between fp32 and bf16 (round to nearest even).
template <typename TSrc, typename TDst>
__global__ __launch_bounds__(256) void convert_kernel(const TSrc *__restrict__ src, TDst *__restrict__ dst, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        dst[i] = from_f32<TDst>(to_f32(src[i]));
}

hipError_t launch_state_convert(const sata_state *src, sata_state *dst, hipStream_t stream) {
    const int64_t n = (int64_t)src->batch * src->heads * (src->idx->dv + 1) * src->idx->m_pad;
    const unsigned grid = (unsigned)std::min<int64_t>((n + 255) / 256, 1 << 16);
    if (src->dtype == SATA_F32 && dst->dtype == SATA_BF16)
        hipLaunchKernelGGL((convert_kernel<float, bf16_t>), dim3(grid), dim3(256), 0, stream,
                           static_cast<const float *>(src->d_state), static_cast<bf16_t *>(dst->d_state), n);
    else if (src->dtype == SATA_BF16 && dst->dtype == SATA_F32)
        hipLaunchKernelGGL((convert_kernel<bf16_t, float>), dim3(grid), dim3(256), 0, stream,
                           static_cast<const bf16_t *>(src->d_state), static_cast<float *>(dst->d_state), n);
    else
        return hipMemcpyAsync(dst->d_state, src->d_state, (size_t)src->state_bytes, hipMemcpyDeviceToDevice, stream);
    return hipGetLastError();
}

hipError_t launch_decode(const sata_index *idx, const sata_state *st, const void *q, const void *k,
                         const void *v, void *out, sata_dtype in_dt, sata_dtype out_dt,
                         hipStream_t stream) {
    switch (idx->dv) {
        case 8: return launch_decode_dv<8>(idx, st, q, k, v, out, in_dt, out_dt, stream);
        case 16: return launch_decode_dv<16>(idx, st, q, k, v, out, in_dt, out_dt, stream);
        case 32: return launch_decode_dv<32>(idx, st, q, k, v, out, in_dt, out_dt, stream);
        case 64: return launch_decode_dv<64>(idx, st, q, k, v, out, in_dt, out_dt, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sata
