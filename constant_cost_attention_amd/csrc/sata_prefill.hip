// Chunked SATA prefill for gfx950.
//
// The sequence is cut into chunks of C tokens.  For a chunk c of a head
//   Y_c  = psi(Q_c) . S^(c-1)                      (inter-chunk readout)
//        + (w(Q_c K_c^T / sqrt d) o causal) [V_c | 1]   (intra-chunk, direct)
//   S^(c) = S^(c-1) + phi(K_c)^T [V_c | 1]           (chunk state, scanned)
//   o    = Y_c[:, :d_V] / Y_c[:, d_V]
// where phi is the plain key monomial of every feature and psi the query
// monomial times 1/(alpha! d^(p/2)) [hotdry, "Core insight of symmetric tensor
// decomposition" and "Engineering realisation of the constant compute cost":
// fixed state S_p = sum phi_p(k) (x) [v, 1], orders weighted and summed, the
// "+1" column normalises].  The two contractions per chunk are dense GEMMs
// with one dimension d_V + 1; they run on MFMA (bf16 operands for bf16
// inputs, fp32 operands for fp32 inputs) with fp32 accumulation.
//
// Kernel 1 (scan): grid (slices, B*H).  A workgroup owns a slice of FS
// features of one head and keeps that slice of the fp32 state in MFMA
// accumulator registers for the whole walk over the chunks of a segment, so
// the state never leaves the chip between chunks; every order is scanned in
// the same grid [hotdry, "Hardware optimisation paths and current limits":
// the orders are independent and can run in parallel].  Per chunk it forms
// psi(Q_c) and phi(K_c) for its slice in registers from LDS copies of the
// chunk (the index tables of the slice are staged in LDS too), reads out its
// share of Y_c and updates its state slice.  The four wavefronts' readouts are
// added in LDS and one (C x (d_V+1)) partial per workgroup and chunk is
// written out.
// Kernel 2 (combine): grid (chunks, B*H).  Adds the slices' partials in a
// fixed order, adds the direct intra-chunk Taylor term and normalises.
//
//   [hotdry] blog.hotdry.top, "Symmetry-aware Taylor approximation attention:
//            engineering a constant per-token cost" (2026-02-05).
#include <algorithm>

#include "sata_device.h"
#include "sata_internal.h"

namespace sata {

constexpr int kNW = 4;                 // wavefronts per workgroup
constexpr int kThreads = 64 * kNW;
constexpr int64_t kWorkCap = (int64_t)4 << 30;   // partial-sum workspace cap (bytes)

template <int D, int DV, int C, int FW, typename TIn>
struct ScanCfg {
    static constexpr bool BF = sizeof(TIn) == 2;
    static constexpr int FS = kNW * FW;          // features per workgroup
    static constexpr int NC = DV + 1;            // value columns + normaliser
    static constexpr int NT = (NC + 15) / 16;    // 16-column MFMA tiles
    static constexpr int NCP = NT * 16;
    static constexpr int MT = FW / 16;           // 16-feature tiles per wavefront
    static constexpr int TT = C / 16;            // 16-token tiles per chunk
    static constexpr int KS = C + 4;             // Kt row stride (floats)
    static constexpr int QS = D + 4;             // Qs row stride (floats)
    static constexpr int VS = BF ? C + 8 : C + 4;   // Vt row stride (elements)
    static constexpr int YS = NCP + 1;           // Yred row stride (floats)
    // LDS carve-up (bytes)
    static constexpr int OFF_K = 0;
    static constexpr int OFF_Q = OFF_K + (D + 2) * KS * 4;
    static constexpr int OFF_V = OFF_Q + C * QS * 4;
    static constexpr int OFF_Y = OFF_V + NCP * VS * (BF ? 2 : 4);
    static constexpr int OFF_T = OFF_Y + C * YS * 4;
    static constexpr int OFF_C = OFF_T + FS * 4;
    static constexpr int LDS = OFF_C + FS * 4;
    static_assert(FW % 32 == 0, "features per wave must be a multiple of 32");
    static_assert(C % 32 == 0, "chunk must be a multiple of 32");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <int D, int DV, int C, int FW, typename TIn>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_scan_kernel(const uint32_t *__restrict__ tup, const float *__restrict__ coef,
                         float *__restrict__ state, int64_t m_pad,
                         const TIn *__restrict__ q, const TIn *__restrict__ k,
                         const TIn *__restrict__ v, int64_t n, int64_t tok0, int nchunk,
                         float *__restrict__ partial) {
    using Cfg = ScanCfg<D, DV, C, FW, TIn>;
    constexpr int NC = Cfg::NC, NT = Cfg::NT, NCP = Cfg::NCP, MT = Cfg::MT, TT = Cfg::TT;
    constexpr int KS = Cfg::KS, QS = Cfg::QS, VS = Cfg::VS, YS = Cfg::YS, FS = Cfg::FS;
    extern __shared__ __align__(16) unsigned char lds[];
    float *Kt = reinterpret_cast<float *>(lds + Cfg::OFF_K);     // [D+2][KS]  dim-major
    float *Qs = reinterpret_cast<float *>(lds + Cfg::OFF_Q);     // [C][QS]    token-major
    float *Yr = reinterpret_cast<float *>(lds + Cfg::OFF_Y);     // [C][YS]
    uint32_t *Ts = reinterpret_cast<uint32_t *>(lds + Cfg::OFF_T);   // [FS]
    float *Cs = reinterpret_cast<float *>(lds + Cfg::OFF_C);         // [FS]

    const int slice = blockIdx.x, nslices = gridDim.x;
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int64_t fslice = (int64_t)slice * FS;
    const int fw0 = wave * FW;                    // wave's first feature within the slice

    for (int i = tid; i < FS; i += kThreads) {
        Ts[i] = tup[fslice + i];
        Cs[i] = coef[fslice + i];
    }

    // state slice -> accumulators: S[j][nt][r] = state[c = 16 nt + li][f = 16 j + 4 g + r]
    float *Sh = state + bh * NC * m_pad;
    f32x4 S[MT][NT];
#pragma unroll
    for (int j = 0; j < MT; ++j)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int c = 16 * nt + li;
                const int64_t f = fslice + fw0 + 16 * j + 4 * g + r;
                S[j][nt][r] = (c < NC && f < m_pad) ? Sh[(int64_t)c * m_pad + f] : 0.f;
            }
    __syncthreads();
    uint32_t myT[MT];                              // update-side tuples of this lane's feature rows
#pragma unroll
    for (int j = 0; j < MT; ++j) myT[j] = Ts[fw0 + 16 * j + li];

    const TIn *qh = q + bh * n * D;
    const TIn *kh = k + bh * n * D;
    const TIn *vh = v + bh * n * DV;

    for (int cc = 0; cc < nchunk; ++cc) {
        const int64_t t0 = tok0 + (int64_t)cc * C;
        __syncthreads();
        // ---- stage the chunk: K dim-major, Q token-major (fp32), V col-major (operand dtype)
        for (int i = tid; i < C * D; i += kThreads) {
            const int t = i / D, d = i - t * D;
            const bool ok = t0 + t < n;
            const int64_t src = (t0 + t) * D + d;
            Kt[d * KS + t] = ok ? to_f32(kh[src]) : 0.f;
            Qs[t * QS + d] = ok ? to_f32(qh[src]) : 0.f;
        }
        for (int t = tid; t < C; t += kThreads) {
            Kt[D * KS + t] = 1.f; Kt[(D + 1) * KS + t] = 0.f;
            Qs[t * QS + D] = 1.f; Qs[t * QS + D + 1] = 0.f;
        }
        for (int i = tid; i < C * NCP; i += kThreads) {
            const int t = i / NCP, c = i - t * NCP;
            const bool ok = t0 + t < n;
            float val = 0.f;
            if (ok) val = c < DV ? to_f32(vh[(t0 + t) * DV + c]) : (c == DV ? 1.f : 0.f);
            if constexpr (Cfg::BF) reinterpret_cast<bf16_t *>(lds + Cfg::OFF_V)[c * VS + t] = from_f32<bf16_t>(val);
            else reinterpret_cast<float *>(lds + Cfg::OFF_V)[c * VS + t] = val;
        }
        __syncthreads();

        // ---- inter-chunk readout: Y = psi(Q_c)[:, slice] . S[slice, :]
        f32x4 Y[TT][NT];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) Y[tt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

        if constexpr (Cfg::BF) {
            // K step kk covers feature tiles 2kk and 2kk+1: operand slot 8g+jj maps to
            // row 4g+jj of tile 2kk (jj<4) or row 4g+jj-4 of tile 2kk+1 (jj>=4), which are
            // exactly this lane's own accumulator registers.
#pragma unroll
            for (int kk = 0; kk < MT / 2; ++kk) {
                bf16x8 B[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    float b[8];
#pragma unroll
                    for (int r = 0; r < 4; ++r) { b[r] = S[2 * kk][nt][r]; b[4 + r] = S[2 * kk + 1][nt][r]; }
                    B[nt] = pack_bf16x8(b);
                }
                uint32_t ft[8];
                float fc[8];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int lf = fw0 + 32 * kk + (jj < 4 ? 4 * g + jj : 16 + 4 * g + jj - 4);
                    ft[jj] = Ts[lf];
                    fc[jj] = Cs[lf];
                }
#pragma unroll
                for (int tt = 0; tt < TT; ++tt) {
                    const float *qrow = Qs + (16 * tt + li) * QS;
                    float a[8];
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) a[jj] = fc[jj] * monomial(ft[jj], qrow, 1);
                    const bf16x8 A = pack_bf16x8(a);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) Y[tt][nt] = mfma_bf16(A, B[nt], Y[tt][nt]);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < MT; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int lf = fw0 + 16 * j + 4 * g + r;
                    const uint32_t ft = Ts[lf];
                    const float fc = Cs[lf];
#pragma unroll
                    for (int tt = 0; tt < TT; ++tt) {
                        const float a = fc * monomial(ft, Qs + (16 * tt + li) * QS, 1);
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) Y[tt][nt] = mfma_f32(a, S[j][nt][r], Y[tt][nt]);
                    }
                }
        }

        // ---- chunk state: S[slice, :] += phi(K_c)[:, slice]^T [V_c | 1]
        if constexpr (Cfg::BF) {
            const bf16_t *Vt = reinterpret_cast<const bf16_t *>(lds + Cfg::OFF_V);
#pragma unroll
            for (int ks = 0; ks < C / 32; ++ks) {
                const int tb = 32 * ks + 8 * g;
                bf16x8 B[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    B[nt] = *reinterpret_cast<const bf16x8 *>(Vt + (16 * nt + li) * VS + tb);
#pragma unroll
                for (int j = 0; j < MT; ++j) {
                    const uint32_t t = myT[j];
                    const float *k1 = Kt + tup_i1(t) * KS + tb;
                    const float *k2 = Kt + tup_i2(t) * KS + tb;
                    const float *k3 = Kt + tup_i3(t) * KS + tb;
                    float a[8];
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) a[jj] = k1[jj] * k2[jj] * k3[jj];
                    const bf16x8 A = pack_bf16x8(a);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) S[j][nt] = mfma_bf16(A, B[nt], S[j][nt]);
                }
            }
        } else {
            const float *Vt = reinterpret_cast<const float *>(lds + Cfg::OFF_V);
#pragma unroll 4
            for (int ks = 0; ks < C / 4; ++ks) {
                const int tb = 4 * ks + g;
                float B[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) B[nt] = Vt[(16 * nt + li) * VS + tb];
#pragma unroll
                for (int j = 0; j < MT; ++j) {
                    const float a = monomial(myT[j], Kt + tb, KS);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) S[j][nt] = mfma_f32(a, B[nt], S[j][nt]);
                }
            }
        }

        // ---- add the four wavefronts' readouts in a fixed order, write the partial
#pragma unroll
        for (int wv = 0; wv < kNW; ++wv) {
            if (wave == wv) {
#pragma unroll
                for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            float *dst = Yr + (16 * tt + 4 * g + r) * YS + 16 * nt + li;
                            *dst = (wv == 0 ? 0.f : *dst) + Y[tt][nt][r];
                        }
            }
            __syncthreads();
        }
        float *pdst = partial + (((bh * nchunk + cc) * nslices) + slice) * (int64_t)C * NC;
        for (int i = tid; i < C * NC; i += kThreads) {
            const int t = i / NC, c = i - t * NC;
            pdst[i] = Yr[t * YS + c];
        }
    }

    // accumulators -> state slice
#pragma unroll
    for (int j = 0; j < MT; ++j)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int c = 16 * nt + li;
                const int64_t f = fslice + fw0 + 16 * j + 4 * g + r;
                if (c < NC && f < m_pad) Sh[(int64_t)c * m_pad + f] = S[j][nt][r];
            }
}

// Kernel 2: direct intra-chunk Taylor term + sum of the slices' partials +
// normalisation.  LDS: phase 1 holds Q and K (fp32) and the weight matrix;
// phase 2 reuses the Q/K area for [V | 1] and the output sums.
template <int D, int DV, int C, typename TIn, typename TOut>
__global__ __launch_bounds__(256) void prefill_combine_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
    TOut *__restrict__ out, int64_t n, int64_t tok0, int nchunk, int nslices,
    const float *__restrict__ partial, float scale, float c0, float c1, float c2, float c3, int P) {
    constexpr int NC = DV + 1;
    constexpr int QKS = D + 1;
    constexpr int WS = C + 1;
    extern __shared__ __align__(16) unsigned char lds[];
    float *Qs = reinterpret_cast<float *>(lds);          // [C][QKS]
    float *Ks = Qs + C * QKS;                            // [C][QKS]
    float *Wm = Ks + C * QKS;                            // [C][WS]
    float *Vs = Qs;                                      // phase 2: [C][NC]
    float *Ys = Qs + C * NC;                             // phase 2: [C][NC]
    const int cc = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t t0 = tok0 + (int64_t)cc * C;
    const int nvalid = (int)std::min<int64_t>(C, n - t0);

    for (int i = tid; i < C * D; i += 256) {
        const int t = i / D, d = i - t * D;
        const bool ok = t < nvalid;
        const int64_t src = (bh * n + t0 + t) * D + d;
        Qs[t * QKS + d] = ok ? to_f32(q[src]) : 0.f;
        Ks[t * QKS + d] = ok ? to_f32(k[src]) : 0.f;
    }
    __syncthreads();
    for (int i = tid; i < C * C; i += 256) {
        const int r = i / C, j = i - r * C;
        float w = 0.f;
        if (j <= r && r < nvalid) {
            float x = 0.f;
#pragma unroll 8
            for (int d = 0; d < D; ++d) x += Qs[r * QKS + d] * Ks[j * QKS + d];
            x *= scale;
            // w(x) = sum_{p<P} x^p/p! by Horner, P <= 4
            w = (P >= 4) ? c3 : 0.f;
            if (P >= 3) w = w * x + c2;
            if (P >= 2) w = w * x + c1;
            w = w * x + c0;
        }
        Wm[r * WS + j] = w;
    }
    __syncthreads();
    for (int i = tid; i < C * NC; i += 256) {
        const int t = i / NC, c = i - t * NC;
        float val = 0.f;
        if (t < nvalid) val = c < DV ? to_f32(v[(bh * n + t0 + t) * DV + c]) : 1.f;
        Vs[i] = val;
    }
    __syncthreads();
    const float *pbase = partial + ((bh * nchunk + cc) * nslices) * (int64_t)C * NC;
    for (int i = tid; i < C * NC; i += 256) {
        const int t = i / NC, c = i - t * NC;
        float y = 0.f;
        for (int s = 0; s < nslices; ++s) y += pbase[(int64_t)s * C * NC + i];
        float yi = 0.f;
        for (int j = 0; j <= t; ++j) yi += Wm[t * WS + j] * Vs[j * NC + c];
        Ys[i] = y + yi;
    }
    __syncthreads();
    for (int i = tid; i < C * DV; i += 256) {
        const int t = i / DV, c = i - t * DV;
        if (t < nvalid) out[(bh * n + t0 + t) * DV + c] = from_f32<TOut>(Ys[t * NC + c] / Ys[t * NC + DV]);
    }
}

// ---------------------------------------------------------------- host side

static int pick_fw(int dk, int64_t bh, int64_t m) {
    // Features per wave: 128 when that still gives at least ~2 workgroups per
    // CU-slot worth of slices across the heads, else 64 (many small heads).
    const int64_t slices128 = (m + 4 * 128 - 1) / (4 * 128);
    if (dk <= 16 || bh * slices128 < 256) return 64;
    return 128;
}

PrefillPlan plan_prefill(const sata_index *idx, int64_t bh, int64_t n, int chunk, sata_dtype in_dt) {
    PrefillPlan p;
    (void)in_dt;
    p.chunk = chunk ? chunk : (idx->dk == 64 ? 128 : 64);
    if (p.chunk != 64 && p.chunk != 128) return p;
    p.fw = pick_fw(idx->dk, bh, idx->m);
    p.fs = kNW * p.fw;
    p.slices = (int)((idx->m + p.fs - 1) / p.fs);
    const int64_t nchunks = (n + p.chunk - 1) / p.chunk;
    const int64_t per_chunk = bh * p.slices * (int64_t)p.chunk * (idx->dv + 1) * 4;
    p.seg_chunks = std::max<int64_t>(1, std::min<int64_t>(nchunks, kWorkCap / per_chunk));
    p.work_bytes = p.seg_chunks * per_chunk;
    p.ok = true;
    return p;
}

template <int D, int C, int FW, typename TIn, typename TOut>
static hipError_t run_prefill(const sata_index *idx, const sata_state *st, const PrefillPlan &plan,
                              const void *q, const void *k, const void *v, void *out, int64_t n,
                              hipStream_t stream) {
    using Cfg = ScanCfg<D, D, C, FW, TIn>;
    const int64_t bh = (int64_t)st->batch * st->heads;
    auto scan = prefill_scan_kernel<D, D, C, FW, TIn>;
    auto comb = prefill_combine_kernel<D, D, C, TIn, TOut>;
    constexpr int comb_lds = (2 * C * (D + 1) + C * (C + 1)) * 4;
    static_assert(2 * C * (D + 2) * 4 <= 2 * C * (D + 1) * 4 + C * (C + 1) * 4, "phase-2 fits");
    static_assert(comb_lds <= 160 * 1024, "combine LDS budget");
    hipError_t e = hipFuncSetAttribute((const void *)scan, hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void *)comb, hipFuncAttributeMaxDynamicSharedMemorySize, comb_lds);
    if (e != hipSuccess) return e;
    const int64_t nchunks = (n + C - 1) / C;
    float *partial = static_cast<float *>(st->d_work);
    for (int64_t c0 = 0; c0 < nchunks; c0 += plan.seg_chunks) {
        const int nseg = (int)std::min<int64_t>(plan.seg_chunks, nchunks - c0);
        const int64_t tok0 = c0 * C;
        {
            ProfScope ps(kProfScan, stream);
            hipLaunchKernelGGL(scan, dim3(plan.slices, (unsigned)bh), dim3(kThreads), Cfg::LDS, stream,
                               idx->d_tup, idx->d_coef, st->d_state, idx->m_pad,
                               static_cast<const TIn *>(q), static_cast<const TIn *>(k),
                               static_cast<const TIn *>(v), n, tok0, nseg, partial);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        {
            ProfScope ps(kProfCombine, stream);
            hipLaunchKernelGGL(comb, dim3(nseg, (unsigned)bh), dim3(256), comb_lds, stream,
                               static_cast<const TIn *>(q), static_cast<const TIn *>(k),
                               static_cast<const TIn *>(v), static_cast<TOut *>(out), n, tok0, nseg,
                               plan.slices, partial, 1.0f / sqrtf((float)D), idx->taylor[0],
                               idx->taylor[1], idx->taylor[2], idx->taylor[3], idx->P);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int D, int C, int FW>
static hipError_t run_dt(const sata_index *idx, const sata_state *st, const PrefillPlan &plan,
                         const void *q, const void *k, const void *v, void *out, int64_t n,
                         sata_dtype in_dt, sata_dtype out_dt, hipStream_t s) {
    if (in_dt == SATA_F32) {
        if (out_dt == SATA_F32) return run_prefill<D, C, FW, float, float>(idx, st, plan, q, k, v, out, n, s);
        return run_prefill<D, C, FW, float, bf16_t>(idx, st, plan, q, k, v, out, n, s);
    }
    if (out_dt == SATA_F32) return run_prefill<D, C, FW, bf16_t, float>(idx, st, plan, q, k, v, out, n, s);
    return run_prefill<D, C, FW, bf16_t, bf16_t>(idx, st, plan, q, k, v, out, n, s);
}

template <int D>
static hipError_t run_d(const sata_index *idx, const sata_state *st, const PrefillPlan &plan,
                        const void *q, const void *k, const void *v, void *out, int64_t n,
                        sata_dtype in_dt, sata_dtype out_dt, hipStream_t s) {
    if (plan.chunk == 64) {
        if (plan.fw == 64) return run_dt<D, 64, 64>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, s);
        return run_dt<D, 64, 128>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, s);
    }
    if (plan.fw == 64) return run_dt<D, 128, 64>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, s);
    return run_dt<D, 128, 128>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, s);
}

hipError_t launch_prefill(const sata_index *idx, const sata_state *st, const PrefillPlan &plan,
                          const void *q, const void *k, const void *v, void *out, int64_t n,
                          sata_dtype in_dt, sata_dtype out_dt, hipStream_t stream) {
    switch (idx->dk) {
        case 8: return run_d<8>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, stream);
        case 16: return run_d<16>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, stream);
        case 32: return run_d<32>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, stream);
        case 64: return run_d<64>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sata
