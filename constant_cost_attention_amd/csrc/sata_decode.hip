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
#include <type_traits>

#include "sata_device.h"
#include "sata_internal.h"

namespace sata {

constexpr int kDecThreads = 256;
// LDS staging length of a token's q or k: the d_K values, the constant-1 and
// constant-0 slots, padding (d_K <= 64 goes with d_V <= 64, d_K = 128 with
// d_V = 128).
template <int DV> constexpr int tok_stage() { return DV > 64 ? 136 : 72; }
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Features per lane of the plain step and the read kernel: one 16-byte word of
// every state row (4 fp32 or 8 bf16).
template <typename TS> constexpr int dec_fpt() { return 16 / (int)sizeof(TS); }

// A lane's word of one state row, and its conversion to FPT fp32 values and
// back (bf16 rounds to nearest even).
template <typename TS, int FPT> struct Word;
template <> struct Word<float, 4> {
    typedef u32x4 T;
    static __device__ __forceinline__ void widen(const T u, float (&x)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = __uint_as_float(u[j]);
    }
    static __device__ __forceinline__ T narrow(const float (&x)[4]) {
        return T{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
    }
};
template <int N> struct WordBf16 {
    typedef uint32_t T __attribute__((ext_vector_type(N / 2)));
    static __device__ __forceinline__ void widen(const T u, float (&x)[N]) {
#pragma unroll
        for (int j = 0; j < N / 2; ++j) {
            x[2 * j] = __uint_as_float(u[j] << 16);
            x[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ T narrow(const float (&x)[N]) {
        T r;
#pragma unroll
        for (int j = 0; j < N / 2; ++j) r[j] = pack_bf16x2(x[2 * j], x[2 * j + 1]);
        return r;
    }
};
template <> struct Word<bf16_t, 8> : WordBf16<8> {};
template <> struct Word<bf16_t, 4> : WordBf16<4> {};
template <int N> struct WordF16 {
    typedef uint32_t T __attribute__((ext_vector_type(N / 2)));
    typedef _Float16 H2 __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ void widen(const T u, float (&x)[N]) {
#pragma unroll
        for (int j = 0; j < N / 2; ++j) {
            // (the element goes through a scalar first: a bit cast applied to the indexed
            // vector element directly compiles to a read of element 0 for every j)
            const uint32_t e = u[j];
            const H2 h = __builtin_bit_cast(H2, e);
            x[2 * j] = (float)h[0];
            x[2 * j + 1] = (float)h[1];
        }
    }
    static __device__ __forceinline__ T narrow(const float (&x)[N]) {   // nearest even
        T r;
#pragma unroll
        for (int j = 0; j < N / 2; ++j) r[j] = __builtin_bit_cast(uint32_t, H2{(_Float16)x[2 * j], (_Float16)x[2 * j + 1]});
        return r;
    }
};
template <> struct Word<f16_t, 8> : WordF16<8> {};
template <> struct Word<f16_t, 4> : WordF16<4> {};

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

// Per-lane feature weights of the lane's FPT features: the query side
// (coefficient times monomial) or the key side (plain monomial).
template <int FPT>
__device__ __forceinline__ void lane_tables(bool valid, const uint32_t *tup, const float *coef, int64_t f0,
                                            uint32_t (&tt)[FPT], float (&cc)[FPT]) {
    static_assert(FPT % 4 == 0, "tables are read 16 bytes (4 features) at a time");
#pragma unroll
    for (int h = 0; h < FPT / 4; ++h) {
        uint4 t4 = uint4{0u, 0u, 0u, 0u};
        float4 c4 = float4{0.f, 0.f, 0.f, 0.f};
        if (valid) {
            t4 = *reinterpret_cast<const uint4 *>(tup + f0 + 4 * h);
            c4 = *reinterpret_cast<const float4 *>(coef + f0 + 4 * h);
        }
        tt[4 * h] = t4.x; tt[4 * h + 1] = t4.y; tt[4 * h + 2] = t4.z; tt[4 * h + 3] = t4.w;
        cc[4 * h] = c4.x; cc[4 * h + 1] = c4.y; cc[4 * h + 2] = c4.z; cc[4 * h + 3] = c4.w;
    }
}

// Workgroup reduction of the d_V + 1 per-lane readout sums into one partial
// row per workgroup.
template <int DV>
__device__ __forceinline__ void store_partial(float (&acc)[DV + 1], float (&red)[kDecThreads / 64][DV + 1],
                                              float *partial, int bh) {
    constexpr int NC = DV + 1;
    const int tid = threadIdx.x;
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

// The plain decode step: update the state by the step's token, read out the
// updated state.
//
// The lane's row loads are issued in two batches, the second before any
// store of the first, so each lane keeps up to d_V+1 16-byte loads in flight;
// one wavefront per SIMD then saturates the HBM read-modify-write stream (the
// state is far larger than every cache).
template <int DV, typename TIn, typename TS>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_kernel(const uint32_t *__restrict__ tup, const float *__restrict__ coef, TS *__restrict__ state,
                   int64_t m_pad, int dk, const TIn *__restrict__ q, const TIn *__restrict__ k,
                   const TIn *__restrict__ v, float *__restrict__ partial, int64_t fbase) {
    constexpr int NC = DV + 1;
    constexpr int FPT = dec_fpt<TS>();
    constexpr int R = (NC + 1) / 2;                    // rows of the first load batch
    typedef Word<TS, FPT> Wd;
    __shared__ float sq[tok_stage<DV>()], sk[tok_stage<DV>()], sv[NC];
    __shared__ float red[kDecThreads / 64][NC];
    const int bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t f0 = fbase + ((int64_t)blockIdx.x * kDecThreads + tid) * FPT;
    const bool valid = f0 < m_pad;   // m_pad and fbase are multiples of 64
    TS *Sb = state + (int64_t)bh * NC * m_pad + f0;
    auto row = [&](int r) { return reinterpret_cast<typename Wd::T *>(Sb + (int64_t)r * m_pad); };

    // first batch of state rows goes out before anything else
    typename Wd::T s[NC];
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (valid) s[r] = __builtin_nontemporal_load(row(r));
    uint32_t tt[FPT];
    float cc[FPT];
    lane_tables<FPT>(valid, tup, coef, f0, tt, cc);
    // the token into LDS; only entries up to d_K + 1 are read (index d_K is the
    // constant 1, d_K + 1 the padding 0)
    if (tid <= dk + 1) {
        sq[tid] = tid < dk ? to_f32(q[(int64_t)bh * dk + tid]) : (tid == dk ? 1.f : 0.f);
        sk[tid] = tid < dk ? to_f32(k[(int64_t)bh * dk + tid]) : (tid == dk ? 1.f : 0.f);
    }
    if (tid < NC) sv[tid] = tid < DV ? to_f32(v[(int64_t)bh * DV + tid]) : 1.f;
    __syncthreads();

    float phk[FPT], psq[FPT];
#pragma unroll
    for (int j = 0; j < FPT; ++j) {
        phk[j] = monomial(tt[j], sk, 1);
        psq[j] = cc[j] * monomial(tt[j], sq, 1);
    }

    // second batch in flight while the first is updated, stored and read out
#pragma unroll
    for (int r = R; r < NC; ++r)
        if (valid) s[r] = __builtin_nontemporal_load(row(r));
    float acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        float x[FPT];
        Wd::widen(s[c], x);
        const float vc = sv[c];
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < FPT; ++j) {
            x[j] += phk[j] * vc;
            a += psq[j] * x[j];
        }
        if (valid) __builtin_nontemporal_store(Wd::narrow(x), row(c));
        acc[c] = valid ? a : 0.f;
    }
    store_partial<DV>(acc, red, partial, bh);
}

// Small-batch variant of the plain step (UPDATE) and of the read kernel: the
// d_V + 1 rows of a feature tile are split over workgroups, rows_per_group()
// each (at most 16).  With few heads the whole-tile kernels leave a grid of a
// few hundred long workgroups, at one per compute unit, in which each
// workgroup's two load batches wait on each other and the last round runs
// on part of the chip.  Here every workgroup issues all its rows at once
// (one round trip), holds a fraction of the registers (several workgroups
// per compute unit) and the grid is d_V + 1 / rows_per_group() times
// finer.  A lane past the last feature re-reads the last word (in bounds,
// weight 0) and stores nothing.  The key-side monomials and tables are
// recomputed per group (cheap, and the tables stay in L2).  Each workgroup
// writes the partial sums of its own rows of its tile's partial row.
template <int DV> constexpr int rows_per_group() {
    constexpr int NC = DV + 1;
    constexpr int groups = (NC + 15) / 16;
    return (NC + groups - 1) / groups;
}
template <int DV, typename TIn, typename TS, bool UPDATE>
__global__ __launch_bounds__(kDecThreads)
void decode_rows_kernel(const uint32_t *__restrict__ tup, const float *__restrict__ coef, TS *__restrict__ state,
                        int64_t m_pad, int dk, const TIn *__restrict__ q, const TIn *__restrict__ k,
                        const TIn *__restrict__ v, float *__restrict__ partial, int64_t fbase) {
    constexpr int NC = DV + 1;
    constexpr int NR = rows_per_group<DV>();
    constexpr int FPT = dec_fpt<TS>();
    typedef Word<TS, FPT> Wd;
    __shared__ float sq[tok_stage<DV>()], sk[tok_stage<DV>()], sv[NR];
    __shared__ float red[kDecThreads / 64][16];
    const int bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int r0 = blockIdx.z * NR;
    const int nr = min(NR, NC - r0);                 // rows of this group (uniform)
    const int64_t f0 = fbase + ((int64_t)blockIdx.x * kDecThreads + tid) * FPT;
    const bool valid = f0 < m_pad;                   // m_pad and fbase are multiples of 64
    TS *Sb = state + ((int64_t)bh * NC + r0) * m_pad + min<int64_t>(f0, m_pad - FPT);
    auto row = [&](int r) { return reinterpret_cast<typename Wd::T *>(Sb + (int64_t)r * m_pad); };

    typename Wd::T s[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r)
        if (r < nr) s[r] = __builtin_nontemporal_load(row(r));
    uint32_t tt[FPT];
    float cc[FPT];
    lane_tables<FPT>(true, tup, coef, min<int64_t>(f0, m_pad - FPT), tt, cc);
    if (tid <= dk + 1) {
        sq[tid] = tid < dk ? to_f32(q[(int64_t)bh * dk + tid]) : (tid == dk ? 1.f : 0.f);
        if (UPDATE) sk[tid] = tid < dk ? to_f32(k[(int64_t)bh * dk + tid]) : (tid == dk ? 1.f : 0.f);
    }
    if (UPDATE && tid < nr) sv[tid] = r0 + tid < DV ? to_f32(v[(int64_t)bh * DV + r0 + tid]) : 1.f;
    __syncthreads();

    float phk[FPT], psq[FPT];
#pragma unroll
    for (int j = 0; j < FPT; ++j) {
        if (UPDATE) phk[j] = monomial(tt[j], sk, 1);
        psq[j] = valid ? cc[j] * monomial(tt[j], sq, 1) : 0.f;
    }
    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        if (r < nr) {
            float x[FPT];
            Wd::widen(s[r], x);
            float a = 0.f;
#pragma unroll
            for (int j = 0; j < FPT; ++j) {
                if (UPDATE) x[j] += phk[j] * sv[r];
                a += psq[j] * x[j];
            }
            if (UPDATE && valid) __builtin_nontemporal_store(Wd::narrow(x), row(r));
            acc[r] = a;
        }
    }
    const float col = wave_reduce_scatter<16>(acc);
    const int lane = tid & 63, wave = tid >> 6;
    if (lane < 16) red[wave][lane] = col;
    __syncthreads();
    if (tid < nr) {
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kDecThreads / 64; ++w) sum += red[w][tid];
        partial[((int64_t)bh * gridDim.x + blockIdx.x) * NC + r0 + tid] = sum;
    }
}

// Fold of a decode window on the matrix cores: the state update by the
// window's tokens is the rank-T product S[c][f] += sum_t [v_t, 1][c] phi(k_t)[f],
// a dense contraction over the tokens.  On v_mfma_f32_16x16x4f32 (A: features x
// 4 tokens, B: 4 tokens x 16 columns) a lane's accumulator holds 4
// consecutive features of one state row, i.e. one state word: the word is
// loaded into the accumulator, ceil(T/4) MFMAs add the tokens, and it is
// read out (if q is given) and stored back.  fp32 throughout (bf16 words are
// widened and rounded to nearest even when stored), so the result matches
// T plain steps up to rounding.  A wavefront owns 64 features (4 groups of
// 16) of every row, in 5 column tiles of 16 (rows past d_V are masked); the
// tokens are the npend deferred ones followed by the step's own if k is
// given, staged in LDS with padding slots whose [v, 1] row is zero.  Four
// wavefronts per SIMD (123 registers, 40 KB of LDS per workgroup) keep enough
// state words in flight: a load covers 64 bytes of 16 rows, so HBM is served
// best by many wavefronts at once.
// NF: index slots the monomials multiply (3 up to P = 4, 4 for P = 5).
constexpr int kFoldThreads = 256;
// BLOCK (the block prefill): before the update, the block's nq queries (fp32 rows of qs,
// [bh][kMaxDecodeWindow][d_K]) are read out against the state as loaded, on
// v_mfma_f32_16x16x4f32: a lane's state value S[16 ct + l16][fw + 16 g + 4 lg + r] is the B
// element for K index lg and column l16 of step (g, r), and the query-side monomial of that
// feature for query l16 of the tile the A element, used by every column tile.  One partial
// row per (workgroup, query): bpartial [bh][workgroups][kMaxDecodeWindow][d_V+1].
template <int DV, typename TIn, typename TS, int NF, bool BLOCK = false>
__global__ __launch_bounds__(kFoldThreads) __attribute__((amdgpu_waves_per_eu(DV > 64 ? 2 : 4, DV > 64 ? 2 : 4)))
void decode_fold_kernel(const uint32_t *__restrict__ tup, const float *__restrict__ coef, TS *__restrict__ state,
                        int64_t m_pad, int dk, const TIn *__restrict__ q, const TIn *__restrict__ k,
                        const TIn *__restrict__ v, const float *__restrict__ pend_k, const float *__restrict__ pend_v,
                        int npend, float *__restrict__ partial, const float *__restrict__ qs, int nq,
                        float *__restrict__ bpartial, int64_t fbase) {
    constexpr int NC = DV + 1;
    constexpr int CT = (NC + 15) / 16;               // column tiles
    constexpr int T = kMaxDecodeWindow;
    typedef Word<TS, 4> Wd;
    constexpr int KST = tok_stage<DV>();
    __shared__ float sq[KST], sk[T][KST];
    __shared__ float sv[T][CT * 16];                 // [token][column], zero past d_V and for padding slots
    __shared__ float red[kFoldThreads / 64][CT * 16];
    const int bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const bool readout = q != nullptr;
    const int ntok = npend + (k != nullptr ? 1 : 0);
    const int kt = (ntok + 3) / 4;                   // token groups of 4
    const int64_t fw = fbase + ((int64_t)blockIdx.x * (kFoldThreads / 64) + wave) * 64;   // the wavefront's first feature
    const bool active = fw < m_pad;
    // the lane's state word of feature group g (features fw + 16 g + 4 lg .. + 3) lies inside
    // the rows (m_pad and fbase are multiples of 64, so a wavefront's words are all inside or
    // all past the end; the check per word keeps that from being an assumption)
    auto wok = [&](int g) { return fw + 16 * g + 4 * lg < m_pad; };
    const uint32_t padt = (uint32_t)(dk + 1) * 0x01010101u;   // a tuple of monomial 0
    TS *Sb = state + (int64_t)bh * NC * m_pad;

    // the wavefront's state words: feature group g, column tile ct -> row ct*16 + l16,
    // features fw + 16 g + 4 lg .. + 3
    f32x4 acc[4][CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        const int c = ct * 16 + l16;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            acc[g][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (wok(g) && c < NC) {
                float x[4];
                Wd::widen(*reinterpret_cast<const typename Wd::T *>(Sb + (int64_t)c * m_pad + fw + 16 * g + 4 * lg), x);
                acc[g][ct] = f32x4{x[0], x[1], x[2], x[3]};
            }
        }
    }
    if constexpr (BLOCK) {
        // the block's queries in the key area, their readout sums in the value area
        // ([waves][16 queries][columns] fills the [tokens][columns] area exactly)
        static_assert(kFoldThreads / 64 * 16 == T, "readout sums fit the value area");
        float(*redb)[16][CT * 16] = reinterpret_cast<float(*)[16][CT * 16]>(&sv[0][0]);
        for (int i = tid; i < T * KST; i += kFoldThreads) {
            const int t = i / KST, c = i % KST;
            float x = 0.f;
            if (t < nq) x = c < dk ? qs[((int64_t)bh * kMaxDecodeWindow + t) * dk + c] : (c == dk ? 1.f : 0.f);
            sk[t][c] = x;
        }
        __syncthreads();
        for (int qt = 0; qt < (nq + 15) / 16; ++qt) {
            const float *qrow = sk[16 * qt + l16];
            f32x4 Y[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) Y[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint32_t tt[4];
                float cc[4];
                lane_tables<4>(wok(g), tup, coef, wok(g) ? fw + 16 * g + 4 * lg : 0, tt, cc);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float a = cc[r] * monomial_n<NF>(tt[r], qrow, 1);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) Y[ct] = mfma_f32(a, acc[g][ct][r], Y[ct]);
                }
            }
            // Y[ct][rr]: query 16 qt + 4 lg + rr, column 16 ct + l16
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) redb[wave][4 * lg + rr][16 * ct + l16] = Y[ct][rr];
            __syncthreads();
            for (int i = tid; i < 16 * NC; i += kFoldThreads) {
                const int qi = i / NC, c = i % NC, t = 16 * qt + qi;
                if (t < nq) {
                    float sum = 0.f;
#pragma unroll
                    for (int w = 0; w < kFoldThreads / 64; ++w) sum += redb[w][qi][c];
                    bpartial[(((int64_t)bh * gridDim.x + blockIdx.x) * kMaxDecodeWindow + t) * NC + c] = sum;
                }
            }
            __syncthreads();
        }
    }
    for (int i = tid; i < T * KST; i += kFoldThreads) {
        const int t = i / KST, c = i % KST;
        float x = 0.f;
        if (t < ntok && c < dk)
            x = t < npend ? pend_k[((int64_t)bh * kMaxDecodeWindow + t) * dk + c] : to_f32(k[(int64_t)bh * dk + c]);
        else if (c == dk)
            x = 1.f;
        sk[t][c] = x;
    }
    for (int i = tid; i < T * CT * 16; i += kFoldThreads) {
        const int t = i / (CT * 16), c = i % (CT * 16);
        float x = 0.f;
        if (t < ntok) {
            if (c == DV) x = 1.f;
            else if (c < DV) x = t < npend ? pend_v[((int64_t)bh * kMaxDecodeWindow + t) * DV + c]
                                           : to_f32(v[(int64_t)bh * DV + c]);
        }
        sv[t][c] = x;
    }
    if (readout && tid < KST) sq[tid] = tid < dk ? to_f32(q[(int64_t)bh * dk + tid]) : (tid == dk ? 1.f : 0.f);
    __syncthreads();

    if (active) {
        // A operand: lane holds feature fw + 16 g + l16 of token 4 kk + lg
        uint32_t ta[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) ta[g] = fw + 16 * g + l16 < m_pad ? tup[fw + 16 * g + l16] : padt;
        for (int kk = 0; kk < kt; ++kk) {
            float a[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) a[g] = monomial_n<NF>(ta[g], sk[4 * kk + lg], 1);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const float b = sv[4 * kk + lg][ct * 16 + l16];
#pragma unroll
                for (int g = 0; g < 4; ++g) acc[g][ct] = mfma_f32(a[g], b, acc[g][ct]);
            }
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int c = ct * 16 + l16;
            if (c < NC) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float x[4] = {acc[g][ct][0], acc[g][ct][1], acc[g][ct][2], acc[g][ct][3]};
                    if (wok(g))
                        *reinterpret_cast<typename Wd::T *>(Sb + (int64_t)c * m_pad + fw + 16 * g + 4 * lg) = Wd::narrow(x);
                }
            }
        }
    }
    if (!readout) return;
    // readout of the updated words: lane's column ct*16 + l16, summed over its
    // 16 features, then over the 4 lane groups, the wavefronts and (in the
    // finish kernel) the workgroups
    float psq[4][4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t f = fw + 16 * g + 4 * lg + r;
            psq[g][r] = wok(g) ? coef[f] * monomial_n<NF>(tup[f], sq, 1) : 0.f;
        }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        float y = 0.f;
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r) y += psq[g][r] * acc[g][ct][r];
        y += __shfl_xor(y, 16, 64);
        y += __shfl_xor(y, 32, 64);
        if (lg == 0) red[wave][ct * 16 + l16] = y;
    }
    __syncthreads();
    if (tid < NC) {
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kFoldThreads / 64; ++w) sum += red[w][tid];
        partial[((int64_t)bh * gridDim.x + blockIdx.x) * NC + tid] = sum;
    }
}

// fp16 states keep the features of orders 0 and 1 (f < m_low of every row, a multiple of 64)
// in fp32 (sata_state::d_low); the main kernels start at feature m_low and leave them out.
// This kernel, one workgroup per head on the same stream after the step's main kernel, adds
// the tokens to fold in -- the npend deferred ones (pend_k / pend_v), then the step's own
// (k, v) when given -- reads out with q when given, and adds the readout to the head's first
// partial row (written by the main kernel) for the finish kernel.  Thread t takes the word
// w = t % W (features 8w .. 8w+7, W = m_low / 8) of the rows t / W + j G (G = 256 / W): the
// word's monomials are formed once per token for all its rows.  Tokens are staged in LDS 16
// at a time; the readout goes through LDS so each row is summed over its words in order.
constexpr int kLowThreads = 256;
constexpr int kLowStage = 16;
template <int DV, typename TIn, int NF>
__global__ __launch_bounds__(kLowThreads) void decode_low_kernel(
    const uint32_t *__restrict__ tup, const float *__restrict__ coef, float *__restrict__ low, int64_t m_low, int dk,
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v, const float *__restrict__ pend_k,
    const float *__restrict__ pend_v, int npend, float *__restrict__ partial, int nblk) {
    constexpr int NC = DV + 1;
    constexpr int KST = tok_stage<DV>();
    // rows per thread: W <= 16 words (d_K <= 64, m_low <= 128, G >= 16) or 24 (d_K = 128,
    // m_low = 192, G = 10)
    constexpr int RPT = DV > 64 ? 13 : 5;
    constexpr int WMAX = DV > 64 ? 24 : 16;
    __shared__ float sk[kLowStage][KST], sv[kLowStage][NC], sq[KST];
    __shared__ float red[NC * WMAX];
    const int bh = blockIdx.x, tid = threadIdx.x;
    const int W = (int)(m_low / 8), G = kLowThreads / W;
    const int w = tid % W, g0 = tid / W;
    const bool act = g0 < G;
    float *L = low + (int64_t)bh * NC * m_low + 8 * w;
    uint32_t tt[8];
    float cc[8];
    lane_tables<8>(act, tup, coef, 8 * w, tt, cc);
    float x[RPT][8];
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int c = g0 + j * G;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[j][e] = 0.f;
        if (act && c < NC) {
            const float4 a = *reinterpret_cast<const float4 *>(L + (int64_t)c * m_low);
            const float4 b = *reinterpret_cast<const float4 *>(L + (int64_t)c * m_low + 4);
            x[j][0] = a.x; x[j][1] = a.y; x[j][2] = a.z; x[j][3] = a.w;
            x[j][4] = b.x; x[j][5] = b.y; x[j][6] = b.z; x[j][7] = b.w;
        }
    }
    const int ntok = npend + (k != nullptr ? 1 : 0);
    for (int t0 = 0; t0 < ntok; t0 += kLowStage) {
        __syncthreads();   // the previous group has been used
        for (int i = tid; i < kLowStage * KST; i += kLowThreads) {
            const int t = i / KST, c = i % KST, tok = t0 + t;
            float val = 0.f;
            if (tok < ntok && c < dk)
                val = tok < npend ? pend_k[((int64_t)bh * kMaxDecodeWindow + tok) * dk + c] : to_f32(k[(int64_t)bh * dk + c]);
            else if (tok < ntok && c == dk)
                val = 1.f;
            sk[t][c] = val;
        }
        for (int i = tid; i < kLowStage * NC; i += kLowThreads) {
            const int t = i / NC, c = i % NC, tok = t0 + t;
            float val = 0.f;
            if (tok < ntok)
                val = c == DV ? 1.f
                              : (tok < npend ? pend_v[((int64_t)bh * kMaxDecodeWindow + tok) * DV + c]
                                             : to_f32(v[(int64_t)bh * DV + c]));
            sv[t][c] = val;
        }
        __syncthreads();
        const int nt = min(kLowStage, ntok - t0);
        for (int t = 0; t < nt; ++t) {
            float phk[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) phk[e] = monomial_n<NF>(tt[e], sk[t], 1);
#pragma unroll
            for (int j = 0; j < RPT; ++j) {
                const int c = g0 + j * G;
                if (act && c < NC) {
                    const float vc = sv[t][c];
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[j][e] += phk[e] * vc;
                }
            }
        }
    }
    if (ntok > 0) {
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const int c = g0 + j * G;
            if (act && c < NC) {
                *reinterpret_cast<float4 *>(L + (int64_t)c * m_low) = float4{x[j][0], x[j][1], x[j][2], x[j][3]};
                *reinterpret_cast<float4 *>(L + (int64_t)c * m_low + 4) = float4{x[j][4], x[j][5], x[j][6], x[j][7]};
            }
        }
    }
    if (q == nullptr) return;
    if (tid < KST) sq[tid] = tid < dk ? to_f32(q[(int64_t)bh * dk + tid]) : (tid == dk ? 1.f : 0.f);
    __syncthreads();
    float psq[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) psq[e] = cc[e] * monomial_n<NF>(tt[e], sq, 1);
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int c = g0 + j * G;
        if (act && c < NC) {
            float a = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) a += psq[e] * x[j][e];
            red[c * W + w] = a;
        }
    }
    __syncthreads();
    if (tid < NC) {
        float sum = 0.f;
        for (int ww = 0; ww < W; ++ww) sum += red[tid * W + ww];
        partial[(int64_t)bh * nblk * NC + tid] += sum;
    }
}

// Readout of the state as it stands, without an update: the non-folding steps
// of a deferred decode.  A pure read stream, so a workgroup walks tpw
// consecutive feature tiles (256 * FPT features each) of its head and keeps
// the next half-tile's rows in flight while it reads out the current half;
// the readout sums accumulate across the tiles and are reduced once.  tpw is
// at most kReadTiles, fewer when the batch is small (read_tiles_per_block).
constexpr int kReadTiles = 8;
template <int DV, typename TIn, typename TS>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_read_kernel(const uint32_t *__restrict__ tup, const float *__restrict__ coef,
                        const TS *__restrict__ state, int64_t m_pad, int dk, const TIn *__restrict__ q,
                        float *__restrict__ partial, int tpw, int64_t fbase) {
    constexpr int NC = DV + 1;
    constexpr int RA = (NC + 1) / 2;   // rows of the first half-tile
    constexpr int FPT = dec_fpt<TS>();
    constexpr int TILE = kDecThreads * FPT;
    typedef Word<TS, FPT> Wd;
    typedef typename Wd::T WT;
    __shared__ float sq[tok_stage<DV>()];
    __shared__ float red[kDecThreads / 64][NC];
    const int bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t tiles = (m_pad + TILE - 1) / TILE;
    const int64_t first = (int64_t)blockIdx.x * tpw;
    const int tn = (int)min<int64_t>(tpw, tiles - first);
    const TS *Sb = state + (int64_t)bh * NC * m_pad;
    // A lane past the last feature re-reads the last word (in bounds, weight 0),
    // so every load is unconditional.
    auto fidx = [&](int i) { return fbase + (first + i) * TILE + (int64_t)tid * FPT; };
    auto fclamp = [&](int i) { return min<int64_t>(fidx(i), m_pad - FPT); };
    auto row = [&](int64_t f, int r) { return reinterpret_cast<const WT *>(Sb + (int64_t)r * m_pad + f); };
    auto tables = [&](int i, uint32_t (&tt)[FPT], float (&cc)[FPT]) {
        lane_tables<FPT>(true, tup, coef, fclamp(i), tt, cc);
    };

    uint32_t tt[FPT];
    float cc[FPT];
    tables(0, tt, cc);
    bool valid = fidx(0) < m_pad;
    WT sa[RA], sb[NC - RA];
    {
        const int64_t f = fclamp(0);
#pragma unroll
        for (int r = 0; r < RA; ++r) sa[r] = __builtin_nontemporal_load(row(f, r));
#pragma unroll
        for (int r = RA; r < NC; ++r) sb[r - RA] = __builtin_nontemporal_load(row(f, r));
    }
    if (tid < tok_stage<DV>()) sq[tid] = tid < dk ? to_f32(q[(int64_t)bh * dk + tid]) : (tid == dk ? 1.f : 0.f);
    __syncthreads();

    float acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = 0.f;
    // One tile's readout, half by half.  With `next`, the following tile's
    // tables and first half are issued once the first half is consumed, its
    // second half once the second half is; the phases stay in program order.
    auto tile = [&](auto next, int64_t fn, int inext) {
        float psq[FPT];
#pragma unroll
        for (int j = 0; j < FPT; ++j) psq[j] = valid ? cc[j] * monomial(tt[j], sq, 1) : 0.f;
#pragma unroll
        for (int c = 0; c < RA; ++c) {
            float x[FPT];
            Wd::widen(sa[c], x);
#pragma unroll
            for (int j = 0; j < FPT; ++j) acc[c] += psq[j] * x[j];
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (decltype(next)::value) {
            tables(inext, tt, cc);
            valid = fidx(inext) < m_pad;
#pragma unroll
            for (int r = 0; r < RA; ++r) sa[r] = __builtin_nontemporal_load(row(fn, r));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = RA; c < NC; ++c) {
            float x[FPT];
            Wd::widen(sb[c - RA], x);
#pragma unroll
            for (int j = 0; j < FPT; ++j) acc[c] += psq[j] * x[j];
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (decltype(next)::value) {
#pragma unroll
            for (int r = RA; r < NC; ++r) sb[r - RA] = __builtin_nontemporal_load(row(fn, r));
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    for (int i = 0; i + 1 < tn; ++i) tile(std::true_type{}, fclamp(i + 1), i + 1);
    tile(std::false_type{}, 0, 0);
    store_partial<DV>(acc, red, partial, bh);
}

// Adds a head's partial sums in a fixed order (four interleaved groups of
// workgroups, then the groups in turn), then (deferred steps) the direct
// Taylor-weighted terms of the npend pending tokens and of the step's own
// token, w(q.k_t / sqrt(d_K)) [v_t, 1] with w(x) = sum_{p<P} x^p / p!, the
// same sum the state's orders give for one token [hotdry, "Core insight of
// symmetric tensor decomposition"]; divides by the normaliser; and (deferred
// steps) appends the step's token to the pending buffers at slot npend.
constexpr int kFinishThreads = 320;
template <int DV, typename TIn, typename TOut>
__global__ __launch_bounds__(kFinishThreads) void decode_finish_kernel(
    const float *__restrict__ partial, int nblk, TOut *__restrict__ out, int direct, int dk, int P,
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v, float *__restrict__ pend_k,
    float *__restrict__ pend_v, int npend) {
    constexpr int NC = DV + 1;
    constexpr int G = 4 * NC <= kFinishThreads ? 4 : 2;   // partial-sum groups per column
    static_assert(G * NC <= kFinishThreads, "one thread per (group, column)");
    static_assert(kFinishThreads % 16 == 0, "16 threads per token");
    __shared__ float part[G][NC];
    __shared__ float y[NC];
    __shared__ float wt[kMaxDecodeWindow];
    const int bh = blockIdx.x, tid = threadIdx.x;
    const int ntok = direct ? npend + 1 : 0;
    // column c, group g: the partial rows b = g, g + G, ... (several loads in flight)
    if (tid < G * NC) {
        const int c = tid % NC, g = tid / NC;
        const float *pr = partial + (int64_t)bh * nblk * NC + c;
        float s = 0.f;
#pragma unroll 4
        for (int b = g; b < nblk; b += G) s += pr[(int64_t)b * NC];
        part[g][c] = s;
    }
    // token t (a deferred slot, or the step's own): 16 threads share q.k_t
    for (int t0 = 0; t0 < ntok; t0 += kFinishThreads / 16) {
        const int t = t0 + (tid >> 4), i = tid & 15;
        float d = 0.f;
        if (t < ntok) {
            for (int r = i; r < dk; r += 16) {
                const float kv = t < npend ? pend_k[((int64_t)bh * kMaxDecodeWindow + t) * dk + r]
                                           : to_f32(k[(int64_t)bh * dk + r]);
                d += to_f32(q[(int64_t)bh * dk + r]) * kv;
            }
        }
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) d += __shfl_xor(d, off, 16);
        if (t < ntok && i == 0) {
            const float x = d * rsqrtf((float)dk);
            float w = 0.f, term = 1.f;
            for (int p = 0; p < P; ++p) {
                w += term;
                term = term * x / (float)(p + 1);
            }
            wt[t] = w;
        }
    }
    __syncthreads();
    if (tid < NC) {
        float s = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) s += part[g][tid];
        for (int t = 0; t < ntok; ++t) {
            const float vt = tid == DV ? 1.f
                             : (t < npend ? pend_v[((int64_t)bh * kMaxDecodeWindow + t) * DV + tid]
                                          : to_f32(v[(int64_t)bh * DV + tid]));
            s += wt[t] * vt;
        }
        y[tid] = s;
    }
    __syncthreads();
    if (tid < DV) out[(int64_t)bh * DV + tid] = from_f32<TOut>(y[tid] / y[DV]);
    if (direct) {
        if (tid < dk) pend_k[((int64_t)bh * kMaxDecodeWindow + npend) * dk + tid] = to_f32(k[(int64_t)bh * dk + tid]);
        if (tid < DV) pend_v[((int64_t)bh * kMaxDecodeWindow + npend) * DV + tid] = to_f32(v[(int64_t)bh * DV + tid]);
    }
}

static int64_t decode_blocks(const sata_index *idx, int fpt) {
    const int64_t per = (int64_t)kDecThreads * fpt;
    return (idx->m_pad + per - 1) / per;
}
// Tiles per workgroup of the read kernel: kReadTiles while the grid still has
// about four workgroups per compute unit (256 of them), fewer for small
// batches, down to one tile per workgroup.
static int read_tiles_per_block(int64_t bh, int64_t tiles) {
    return (int)std::max<int64_t>(1, std::min<int64_t>(kReadTiles, bh * tiles / 1024));
}
// Whether the plain step and the read kernel split each tile's rows over
// workgroups: when the whole-tile grid would hold fewer than 32 workgroups per
// compute unit (256 of them).  Measured at d = 64: the split grid is ahead up
// to 6144 tile workgroups (by 30% at 8 heads of fp32 state, 1 to 3% at 128
// heads, 2.6% for 256 heads of bf16 state), the whole-tile kernels at 12032
// (256 heads of fp32 state, by 2 to 4%).
static bool split_rows(int64_t bh, int64_t tiles) { return bh * tiles < 32 * 256; }
static int64_t fold_blocks(const sata_index *idx) {
    const int64_t per = kFoldThreads / 64 * 64;   // 64 features per wavefront
    return (idx->m_pad + per - 1) / per;
}

int64_t decode_workspace_bytes(const sata_index *idx, int64_t bh) {
    // one partial row per workgroup; the fold has the most workgroups
    const int64_t blocks = std::max(fold_blocks(idx), decode_blocks(idx, 4));
    return bh * blocks * (idx->dv + 1) * (int64_t)sizeof(float);
}

template <int DV, typename TIn, typename TOut, typename TS>
static hipError_t launch_decode_t(const sata_index *idx, const sata_state *st, const void *q, const void *k,
                                  const void *v, void *out, DecodeMode mode, hipStream_t stream) {
    const int64_t bh = (int64_t)st->batch * st->heads;
    const bool fold = mode == kDecodeFold || mode == kDecodeFlush;
    // workgroups per head: the plain step one tile of 256 lanes x FPT features,
    // the read kernel tpw such tiles, the fold 64 features per wavefront
    const int64_t tiles = decode_blocks(idx, dec_fpt<TS>());
    const int tpw = read_tiles_per_block(bh, tiles);
    constexpr int NR = rows_per_group<DV>();
    // d_V = 128 always splits: a whole tile's 129 rows do not fit one lane's registers
    const int groups = DV > 64 || split_rows(bh, tiles) ? (DV + 1 + NR - 1) / NR : 1;
    const dim3 grid((unsigned)(fold ? fold_blocks(idx) : mode == kDecodeRead && groups == 1 ? (tiles + tpw - 1) / tpw : tiles),
                    (unsigned)bh, (unsigned)(fold ? 1 : groups));
    const int nblk = (int)grid.x;
    float *partial = static_cast<float *>(st->d_work);
    TS *S = static_cast<TS *>(st->d_state);
    const int64_t fbase = st->m_low;   // fp16 states: the lowest orders are the low kernel's
    const TIn *qi = static_cast<const TIn *>(q), *ki = static_cast<const TIn *>(k), *vi = static_cast<const TIn *>(v);
    switch (mode) {
        case kDecodePlain: {
            ProfScope ps(kProfDecode, stream);
            if (groups > 1)
                hipLaunchKernelGGL((decode_rows_kernel<DV, TIn, TS, true>), grid, dim3(kDecThreads), 0, stream,
                                   idx->d_tup, idx->d_coef, S, idx->m_pad, idx->dk, qi, ki, vi, partial, fbase);
            else if constexpr (DV <= 64)
                hipLaunchKernelGGL((decode_kernel<DV, TIn, TS>), grid, dim3(kDecThreads), 0, stream, idx->d_tup,
                                   idx->d_coef, S, idx->m_pad, idx->dk, qi, ki, vi, partial, fbase);
            break;
        }
        case kDecodeRead: {
            ProfScope ps(kProfDecodeRead, stream);
            if (groups > 1)
                hipLaunchKernelGGL((decode_rows_kernel<DV, TIn, TS, false>), grid, dim3(kDecThreads), 0, stream,
                                   idx->d_tup, idx->d_coef, S, idx->m_pad, idx->dk, qi, nullptr, nullptr, partial,
                                   fbase);
            else if constexpr (DV <= 64)
                hipLaunchKernelGGL((decode_read_kernel<DV, TIn, TS>), grid, dim3(kDecThreads), 0, stream, idx->d_tup,
                                   idx->d_coef, S, idx->m_pad, idx->dk, qi, partial, tpw, fbase);
            break;
        }
        case kDecodeFold:
        case kDecodeFlush: {
            ProfScope ps(kProfDecodeFold, stream);
            const bool step = mode == kDecodeFold;
            auto fold = idx->P >= 5 ? decode_fold_kernel<DV, TIn, TS, 4> : decode_fold_kernel<DV, TIn, TS, 3>;
            hipLaunchKernelGGL(fold, grid, dim3(kFoldThreads), 0, stream, idx->d_tup, idx->d_coef, S, idx->m_pad,
                               idx->dk, step ? qi : nullptr, step ? ki : nullptr, step ? vi : nullptr, st->d_pend_k,
                               st->d_pend_v, st->npend, partial, nullptr, 0, nullptr, fbase);
            break;
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (st->m_low > 0) {
        // the fp32 words of the lowest orders: the same update (a read step adds nothing, a
        // fold the deferred tokens and the step's own) and readout, into workgroup 0's row
        ProfScope ps(kProfDecodeLow, stream);
        const bool upd = mode != kDecodeRead, fold_in = mode == kDecodeFold || mode == kDecodeFlush;
        const bool own = mode == kDecodePlain || mode == kDecodeFold;
        auto lowk = idx->P >= 5 ? decode_low_kernel<DV, TIn, 4> : decode_low_kernel<DV, TIn, 3>;
        hipLaunchKernelGGL(lowk, dim3((unsigned)bh), dim3(kLowThreads), 0, stream, idx->d_tup, idx->d_coef, st->d_low,
                           st->m_low, idx->dk, mode == kDecodeFlush ? nullptr : qi, upd && own ? ki : nullptr,
                           upd && own ? vi : nullptr, st->d_pend_k, st->d_pend_v, fold_in ? st->npend : 0, partial,
                           nblk);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (mode == kDecodeFlush) return hipSuccess;
    {
        ProfScope ps(kProfDecodeFinish, stream);
        const int direct = mode == kDecodeRead ? 1 : 0;
        hipLaunchKernelGGL((decode_finish_kernel<DV, TIn, TOut>), dim3((unsigned)bh), dim3(kFinishThreads), 0, stream, partial,
                           nblk, static_cast<TOut *>(out), direct, idx->dk, idx->P, qi, ki, vi, st->d_pend_k,
                           st->d_pend_v, st->npend);
    }
    return hipGetLastError();
}

template <int DV, typename TS>
static hipError_t launch_decode_ts(const sata_index *idx, const sata_state *st, const void *q,
                                   const void *k, const void *v, void *out, sata_dtype in_dt,
                                   sata_dtype out_dt, DecodeMode mode, hipStream_t s) {
    if (in_dt == SATA_F32 && out_dt == SATA_F32)
        return launch_decode_t<DV, float, float, TS>(idx, st, q, k, v, out, mode, s);
    if (in_dt == SATA_F32 && out_dt == SATA_BF16)
        return launch_decode_t<DV, float, bf16_t, TS>(idx, st, q, k, v, out, mode, s);
    if (in_dt == SATA_BF16 && out_dt == SATA_F32)
        return launch_decode_t<DV, bf16_t, float, TS>(idx, st, q, k, v, out, mode, s);
    return launch_decode_t<DV, bf16_t, bf16_t, TS>(idx, st, q, k, v, out, mode, s);
}

template <int DV>
static hipError_t launch_decode_dv(const sata_index *idx, const sata_state *st, const void *q,
                                   const void *k, const void *v, void *out, sata_dtype in_dt,
                                   sata_dtype out_dt, DecodeMode mode, hipStream_t s) {
    if (st->dtype == SATA_BF16) return launch_decode_ts<DV, bf16_t>(idx, st, q, k, v, out, in_dt, out_dt, mode, s);
    if (st->dtype == SATA_F16) return launch_decode_ts<DV, f16_t>(idx, st, q, k, v, out, in_dt, out_dt, mode, s);
    return launch_decode_ts<DV, float>(idx, st, q, k, v, out, in_dt, out_dt, mode, s);
}

// Element-wise state conversion between element types (to bf16 or fp16: round to nearest
// even).  Element i is feature i % m_pad of row i / m_pad; in an fp16 state the features
// below m_low are the fp32 values of its low array, and their fp16 slots are written as zero.
template <typename TS> constexpr bool has_low() { return std::is_same<TS, f16_t>::value; }
template <typename TSrc, typename TDst>
__global__ __launch_bounds__(256) void convert_kernel(const TSrc *__restrict__ src, const float *__restrict__ src_low,
                                                      int64_t src_m_low, TDst *__restrict__ dst,
                                                      float *__restrict__ dst_low, int64_t dst_m_low, int64_t m_pad,
                                                      int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t r = i / m_pad, f = i - r * m_pad;
        const float x = has_low<TSrc>() && f < src_m_low ? src_low[r * src_m_low + f] : to_f32(src[i]);
        if (has_low<TDst>() && f < dst_m_low) {
            dst_low[r * dst_m_low + f] = x;
            dst[i] = from_f32<TDst>(0.f);
        } else {
            dst[i] = from_f32<TDst>(x);
        }
    }
}

hipError_t launch_state_convert(const sata_state *src, sata_state *dst, hipStream_t stream) {
    if (src->dtype == dst->dtype)
        return hipMemcpyAsync(dst->d_state, src->d_state, (size_t)src->state_bytes, hipMemcpyDeviceToDevice, stream);
    const int64_t m_pad = src->idx->m_pad;
    const int64_t n = (int64_t)src->batch * src->heads * (src->idx->dv + 1) * m_pad;
    const unsigned grid = (unsigned)std::min<int64_t>((n + 255) / 256, 1 << 16);
    auto go = [&](auto s_t, auto d_t) {
        using TSrc = decltype(s_t);
        using TDst = decltype(d_t);
        hipLaunchKernelGGL((convert_kernel<TSrc, TDst>), dim3(grid), dim3(256), 0, stream,
                           static_cast<const TSrc *>(src->d_state), src->d_low, src->m_low,
                           static_cast<TDst *>(dst->d_state), dst->d_low, dst->m_low, m_pad, n);
        return hipGetLastError();
    };
    auto to = [&](auto s_t) {
        if (dst->dtype == SATA_BF16) return go(s_t, bf16_t{});
        if (dst->dtype == SATA_F16) return go(s_t, f16_t{});
        return go(s_t, float{});
    };
    if (src->dtype == SATA_BF16) return to(bf16_t{});
    if (src->dtype == SATA_F16) return to(f16_t{});
    return to(float{});
}

hipError_t launch_decode(const sata_index *idx, const sata_state *st, const void *q, const void *k,
                         const void *v, void *out, sata_dtype in_dt, sata_dtype out_dt, DecodeMode mode,
                         hipStream_t stream) {
    switch (idx->dv) {
        case 8: return launch_decode_dv<8>(idx, st, q, k, v, out, in_dt, out_dt, mode, stream);
        case 16: return launch_decode_dv<16>(idx, st, q, k, v, out, in_dt, out_dt, mode, stream);
        case 32: return launch_decode_dv<32>(idx, st, q, k, v, out, in_dt, out_dt, mode, stream);
        case 64: return launch_decode_dv<64>(idx, st, q, k, v, out, in_dt, out_dt, mode, stream);
        case 128: return launch_decode_dv<128>(idx, st, q, k, v, out, in_dt, out_dt, mode, stream);
        default: return hipErrorInvalidValue;
    }
}

// ---- Prefill in blocks through the state in HBM (shapes the scan kernels do not take) ----
// A sequence runs in blocks of up to kMaxDecodeWindow tokens.  The block's queries are read
// out against the state as it stands before the block, each query adds the direct
// Taylor-weighted terms w(q.k_j / sqrt(d_K)) [v_j, 1] of the block's tokens up to itself --
// what those tokens contribute through the state's orders [hotdry, "Core insight of
// symmetric tensor decomposition"] -- and the fold then adds the block's tokens to the
// state.  The readout runs inside the fold on the state words as loaded, so per block the
// state crosses HBM twice (one read, one write) and the path is bound by HBM; it serves
// d_K = 128 for fp32 inputs and five orders.

// fp32 copies of a block's rows: q into qs, k and v into the pending-token buffers, each laid
// out [bh][kMaxDecodeWindow][d] as the fold reads them.  Grid (T, B*H).
template <typename TIn>
__global__ __launch_bounds__(128) void block_stage_kernel(const TIn *__restrict__ q, const TIn *__restrict__ k,
                                                          const TIn *__restrict__ v, int64_t n, int64_t t0, int dk,
                                                          int dv, float *__restrict__ qs, float *__restrict__ pk,
                                                          float *__restrict__ pv) {
    const int64_t bh = blockIdx.y;
    const int t = blockIdx.x;
    const int64_t src = bh * n + t0 + t, dst = bh * kMaxDecodeWindow + t;
    for (int c = threadIdx.x; c < dk; c += 128) {
        qs[dst * dk + c] = to_f32(q[src * dk + c]);
        pk[dst * dk + c] = to_f32(k[src * dk + c]);
    }
    for (int c = threadIdx.x; c < dv; c += 128) pv[dst * dv + c] = to_f32(v[src * dv + c]);
}

// Query t of the block: its partial rows (one per readout workgroup, some 1400 per head at
// d_K = 128) added in a fixed order by G interleaved groups of threads per column, plus the
// direct terms of the block's tokens j <= t, normalised.  Grid (T, B*H).
constexpr int kBlockFinishThreads = 1024;
template <int DV, typename TOut>
__global__ __launch_bounds__(kBlockFinishThreads) void block_finish_kernel(
    const float *__restrict__ partial, int nblk, const float *__restrict__ qs, const float *__restrict__ pk,
    const float *__restrict__ pv, int dk, int P, int64_t n, int64_t t0, TOut *__restrict__ out) {
    constexpr int NC = DV + 1;
    constexpr int G = kBlockFinishThreads / NC;
    __shared__ float part[G][NC];
    __shared__ float y[NC];
    __shared__ float wt[kMaxDecodeWindow];
    const int t = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
    const int ntok = t + 1;
    if (tid < G * NC) {
        const int c = tid % NC, g = tid / NC;
        float s = 0.f;
#pragma unroll 4
        for (int b = g; b < nblk; b += G) s += partial[(((int64_t)bh * nblk + b) * kMaxDecodeWindow + t) * NC + c];
        part[g][c] = s;
    }
    const float *qt = qs + ((int64_t)bh * kMaxDecodeWindow + t) * dk;
    for (int j0 = 0; j0 < ntok; j0 += kBlockFinishThreads / 16) {
        const int j = j0 + (tid >> 4), i = tid & 15;
        float d = 0.f;
        if (j < ntok)
            for (int r = i; r < dk; r += 16) d += qt[r] * pk[((int64_t)bh * kMaxDecodeWindow + j) * dk + r];
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) d += __shfl_xor(d, off, 16);
        if (j < ntok && i == 0) {
            const float xs = d * rsqrtf((float)dk);
            float w = 0.f, term = 1.f;
            for (int p = 0; p < P; ++p) {
                w += term;
                term = term * xs / (float)(p + 1);
            }
            wt[j] = w;
        }
    }
    __syncthreads();
    if (tid < NC) {
        float s = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) s += part[g][tid];
        for (int j = 0; j < ntok; ++j)
            s += wt[j] * (tid == DV ? 1.f : pv[((int64_t)bh * kMaxDecodeWindow + j) * DV + tid]);
        y[tid] = s;
    }
    __syncthreads();
    if (tid < DV) out[((int64_t)bh * n + t0 + t) * DV + tid] = from_f32<TOut>(y[tid] / y[DV]);
}

int64_t block_prefill_workspace_bytes(const sata_index *idx, int64_t bh) {
    const int64_t tiles = fold_blocks(idx);
    return bh * tiles * kMaxDecodeWindow * (idx->dv + 1) * (int64_t)sizeof(float) +
           bh * kMaxDecodeWindow * idx->dk * (int64_t)sizeof(float);
}

template <int DV, typename TIn, typename TOut>
static hipError_t block_prefill_t(const sata_index *idx, sata_state *st, const void *q, const void *k, const void *v,
                                  void *out, int64_t n, hipStream_t stream) {
    const int64_t bh = (int64_t)st->batch * st->heads;
    const int64_t tiles = fold_blocks(idx);
    float *partial = static_cast<float *>(st->d_work);
    float *qs = partial + bh * tiles * kMaxDecodeWindow * (DV + 1);
    const TIn *qi = static_cast<const TIn *>(q), *ki = static_cast<const TIn *>(k), *vi = static_cast<const TIn *>(v);
    for (int64_t t0 = 0; t0 < n; t0 += kMaxDecodeWindow) {
        const int T = (int)std::min<int64_t>(kMaxDecodeWindow, n - t0);
        hipLaunchKernelGGL((block_stage_kernel<TIn>), dim3((unsigned)T, (unsigned)bh), dim3(128), 0, stream, qi, ki,
                           vi, n, t0, idx->dk, DV, qs, st->d_pend_k, st->d_pend_v);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        {
            // the block's readout against the state before it, and the block's tokens added
            ProfScope ps(kProfDecodeFold, stream);
            auto fold = idx->P >= 5 ? decode_fold_kernel<DV, float, float, 4, true>
                                    : decode_fold_kernel<DV, float, float, 3, true>;
            hipLaunchKernelGGL(fold, dim3((unsigned)tiles, (unsigned)bh), dim3(kFoldThreads), 0, stream, idx->d_tup,
                               idx->d_coef, static_cast<float *>(st->d_state), idx->m_pad, idx->dk, nullptr, nullptr,
                               nullptr, st->d_pend_k, st->d_pend_v, T, nullptr, qs, T, partial, (int64_t)0);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        {
            ProfScope ps(kProfCombine, stream);
            hipLaunchKernelGGL((block_finish_kernel<DV, TOut>), dim3((unsigned)T, (unsigned)bh), dim3(kBlockFinishThreads),
                               0, stream, partial, (int)tiles, qs, st->d_pend_k, st->d_pend_v, idx->dk, idx->P, n, t0,
                               static_cast<TOut *>(out));
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_block_prefill(const sata_index *idx, sata_state *st, const void *q, const void *k, const void *v,
                                void *out, int64_t n, sata_dtype in_dt, sata_dtype out_dt, hipStream_t stream) {
    if (idx->dv != 128 || st->dtype != SATA_F32) return hipErrorInvalidValue;
    if (in_dt == SATA_F32 && out_dt == SATA_F32)
        return block_prefill_t<128, float, float>(idx, st, q, k, v, out, n, stream);
    if (in_dt == SATA_F32 && out_dt == SATA_BF16)
        return block_prefill_t<128, float, bf16_t>(idx, st, q, k, v, out, n, stream);
    if (in_dt == SATA_BF16 && out_dt == SATA_F32)
        return block_prefill_t<128, bf16_t, float>(idx, st, q, k, v, out, n, stream);
    return block_prefill_t<128, bf16_t, bf16_t>(idx, st, q, k, v, out, n, stream);
}

}  // namespace sata
