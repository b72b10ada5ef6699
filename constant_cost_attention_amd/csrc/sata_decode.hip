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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Features per lane: one 16-byte word of every state row (4 fp32 or 8 bf16),
// except for a bf16 fold of W > 1 tokens, whose lanes take 8-byte words (4
// bf16) so that 4 features x W key monomials fit the register file.
template <typename TS, int W> constexpr int dec_fpt() {
    return (W > 1 && sizeof(TS) == 2) ? 4 : 16 / (int)sizeof(TS);
}

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

// State update by up to W tokens, then (if q is given) readout of the updated
// state.  The tokens are the npend pending ones of the head (fp32 rows of the
// pending buffers), followed by the step's own k, v if k is given.  W = 1 is
// the plain decode step; larger W folds a window of deferred tokens in one
// pass.
//
// The lane's row loads are issued in NB batches, each batch before any store
// of the previous one, so each lane keeps up to two batches of 16-byte loads
// in flight (all d_V+1 rows for the plain step); one wavefront per SIMD then
// saturates the HBM read-modify-write stream (the state is far larger than
// every cache).  A bf16 fold holds 8 features x W key monomials per lane, so
// it streams in four batches to stay within the register file.
template <int DV, typename TIn, typename TS, int W>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_kernel(const uint32_t *__restrict__ tup, const float *__restrict__ coef, TS *__restrict__ state,
                   int64_t m_pad, int dk, const TIn *__restrict__ q, const TIn *__restrict__ k,
                   const TIn *__restrict__ v, const float *__restrict__ pend_k, const float *__restrict__ pend_v,
                   int npend, float *__restrict__ partial) {
    constexpr int NC = DV + 1;
    constexpr int FPT = dec_fpt<TS, W>();
    constexpr int NB = 2;                              // load batches
    constexpr int RB = (NC + NB - 1) / NB;             // rows per batch
    typedef Word<TS, FPT> Wd;
    __shared__ float sq[72], sk[W][72];
    __shared__ __align__(16) float sv[NC][W];      // token-minor: one row's W values are contiguous
    __shared__ float red[kDecThreads / 64][NC];
    const int bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t f0 = ((int64_t)blockIdx.x * kDecThreads + tid) * FPT;
    const bool valid = f0 < m_pad;   // m_pad is a multiple of 64, so all FPT features are in range
    const bool readout = W == 1 || q != nullptr;   // a plain step always reads out
    TS *Sb = state + (int64_t)bh * NC * m_pad + f0;
    auto row = [&](int r) { return reinterpret_cast<typename Wd::T *>(Sb + (int64_t)r * m_pad); };

    // first batch of state rows goes out before anything else
    typename Wd::T s[NC];
#pragma unroll
    for (int r = 0; r < RB; ++r)
        if (valid) s[r] = __builtin_nontemporal_load(row(r));
    uint32_t tt[FPT];
    float cc[FPT];
    lane_tables<FPT>(valid, tup, coef, f0, tt, cc);

    // tokens into LDS: slot t < npend from the pending buffers, slot npend the
    // step's own token, the rest zero (they add nothing).  Only entries up to
    // d_K + 1 are read (index d_K is the constant 1, d_K + 1 the padding 0).
    if constexpr (W == 1) {
        if (tid <= dk + 1) {
            sq[tid] = tid < dk ? to_f32(q[(int64_t)bh * dk + tid]) : (tid == dk ? 1.f : 0.f);
            sk[0][tid] = tid < dk ? to_f32(k[(int64_t)bh * dk + tid]) : (tid == dk ? 1.f : 0.f);
        }
        if (tid < NC) sv[tid][0] = tid < DV ? to_f32(v[(int64_t)bh * DV + tid]) : 1.f;
    } else {
    const int ntok = npend + (k != nullptr ? 1 : 0);
    for (int i = tid; i < W * 72; i += kDecThreads) {
        const int t = i / 72, c = i % 72;
        float x = 0.f;
        if (t < ntok) {
            if (c < dk)
                x = t < npend ? pend_k[((int64_t)bh * kMaxDecodeWindow + t) * dk + c] : to_f32(k[(int64_t)bh * dk + c]);
            else if (c == dk) x = 1.f;
        }
        sk[t][c] = x;
    }
    for (int i = tid; i < W * NC; i += kDecThreads) {
        const int t = i / NC, c = i % NC;
        float x = 0.f;
        if (t < ntok) {
            if (c == DV) x = 1.f;
            else x = t < npend ? pend_v[((int64_t)bh * kMaxDecodeWindow + t) * DV + c] : to_f32(v[(int64_t)bh * DV + c]);
        }
        sv[c][t] = x;
    }
    if (readout && tid < 72) sq[tid] = tid < dk ? to_f32(q[(int64_t)bh * dk + tid]) : (tid == dk ? 1.f : 0.f);
    }
    __syncthreads();

    float phk[W][FPT], psq[FPT];
#pragma unroll
    for (int j = 0; j < FPT; ++j) {
#pragma unroll
        for (int t = 0; t < W; ++t) phk[t][j] = monomial(tt[j], sk[t], 1);
        psq[j] = readout ? cc[j] * monomial(tt[j], sq, 1) : 0.f;
    }

    float acc[NC];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        // next batch in flight while this one is updated, stored and read out
#pragma unroll
        for (int r = (b + 1) * RB; r < (b + 2) * RB && r < NC; ++r)
            if (valid) s[r] = __builtin_nontemporal_load(row(r));
#pragma unroll
        for (int c = b * RB; c < (b + 1) * RB && c < NC; ++c) {
            float x[FPT];
            Wd::widen(s[c], x);
            float vc[W];
#pragma unroll
            for (int t = 0; t < W; ++t) vc[t] = sv[c][t];
            float a = 0.f;
#pragma unroll
            for (int j = 0; j < FPT; ++j) {
#pragma unroll
                for (int t = 0; t < W; ++t) x[j] += phk[t][j] * vc[t];
                a += psq[j] * x[j];
            }
            if (valid) __builtin_nontemporal_store(Wd::narrow(x), row(c));
            acc[c] = valid ? a : 0.f;
        }
    }
    if (readout) store_partial<DV>(acc, red, partial, bh);
}

// Readout of the state as it stands, without an update: the non-folding steps
// of a deferred decode.  A pure read stream, so a workgroup walks TPW
// consecutive feature tiles (256 * FPT features each) of its head and keeps
// the next half-tile's rows in flight while it reads out the current half;
// the readout sums accumulate across the tiles and are reduced once.
constexpr int kReadTiles = 8;
template <int DV, typename TIn, typename TS>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_read_kernel(const uint32_t *__restrict__ tup, const float *__restrict__ coef,
                        const TS *__restrict__ state, int64_t m_pad, int dk, const TIn *__restrict__ q,
                        float *__restrict__ partial) {
    constexpr int NC = DV + 1;
    constexpr int RA = (NC + 1) / 2;   // rows of the first half-tile
    constexpr int FPT = dec_fpt<TS, 1>();
    constexpr int TILE = kDecThreads * FPT;
    typedef Word<TS, FPT> Wd;
    typedef typename Wd::T WT;
    __shared__ float sq[72];
    __shared__ float red[kDecThreads / 64][NC];
    const int bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t tiles = (m_pad + TILE - 1) / TILE;
    const int64_t first = (int64_t)blockIdx.x * kReadTiles;
    const int tn = (int)min<int64_t>(kReadTiles, tiles - first);
    const TS *Sb = state + (int64_t)bh * NC * m_pad;
    // A lane past the last feature re-reads the last word (in bounds, weight 0),
    // so every load is unconditional.
    auto fidx = [&](int i) { return (first + i) * TILE + (int64_t)tid * FPT; };
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
    if (tid < 72) sq[tid] = tid < dk ? to_f32(q[(int64_t)bh * dk + tid]) : (tid == dk ? 1.f : 0.f);
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
    constexpr int G = 4;                        // partial-sum groups per column
    static_assert(G * NC <= kFinishThreads, "one thread per (group, column)");
    static_assert(kMaxDecodeWindow * 16 <= kFinishThreads, "16 threads per token");
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
    {
        const int t = tid >> 4, i = tid & 15;
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

int64_t decode_workspace_bytes(const sata_index *idx, int64_t bh) {
    return bh * decode_blocks(idx, 4) * (idx->dv + 1) * (int64_t)sizeof(float);   // the larger (fp32) grid
}

template <int DV, typename TIn, typename TOut, typename TS>
static hipError_t launch_decode_t(const sata_index *idx, const sata_state *st, const void *q, const void *k,
                                  const void *v, void *out, DecodeMode mode, hipStream_t stream) {
    const int64_t bh = (int64_t)st->batch * st->heads;
    const bool fold = mode == kDecodeFold || mode == kDecodeFlush;
    const int fpt = fold ? dec_fpt<TS, kMaxDecodeWindow>() : dec_fpt<TS, 1>();
    const int64_t tiles = decode_blocks(idx, fpt);
    const dim3 grid((unsigned)(mode == kDecodeRead ? (tiles + kReadTiles - 1) / kReadTiles : tiles), (unsigned)bh);
    const int nblk = (int)grid.x;
    float *partial = static_cast<float *>(st->d_work);
    TS *S = static_cast<TS *>(st->d_state);
    const TIn *qi = static_cast<const TIn *>(q), *ki = static_cast<const TIn *>(k), *vi = static_cast<const TIn *>(v);
    switch (mode) {
        case kDecodePlain: {
            ProfScope ps(kProfDecode, stream);
            hipLaunchKernelGGL((decode_kernel<DV, TIn, TS, 1>), grid, dim3(kDecThreads), 0, stream, idx->d_tup,
                               idx->d_coef, S, idx->m_pad, idx->dk, qi, ki, vi, nullptr, nullptr, 0, partial);
            break;
        }
        case kDecodeRead: {
            ProfScope ps(kProfDecodeRead, stream);
            hipLaunchKernelGGL((decode_read_kernel<DV, TIn, TS>), grid, dim3(kDecThreads), 0, stream, idx->d_tup,
                               idx->d_coef, S, idx->m_pad, idx->dk, qi, partial);
            break;
        }
        case kDecodeFold:
        case kDecodeFlush: {
            ProfScope ps(kProfDecodeFold, stream);
            const bool step = mode == kDecodeFold;
            hipLaunchKernelGGL((decode_kernel<DV, TIn, TS, kMaxDecodeWindow>), grid, dim3(kDecThreads), 0, stream,
                               idx->d_tup, idx->d_coef, S, idx->m_pad, idx->dk, step ? qi : nullptr,
                               step ? ki : nullptr, step ? vi : nullptr, st->d_pend_k, st->d_pend_v, st->npend,
                               partial);
            break;
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || mode == kDecodeFlush) return e;
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
    return launch_decode_ts<DV, float>(idx, st, q, k, v, out, in_dt, out_dt, mode, s);
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
                         const void *v, void *out, sata_dtype in_dt, sata_dtype out_dt, DecodeMode mode,
                         hipStream_t stream) {
    switch (idx->dv) {
        case 8: return launch_decode_dv<8>(idx, st, q, k, v, out, in_dt, out_dt, mode, stream);
        case 16: return launch_decode_dv<16>(idx, st, q, k, v, out, in_dt, out_dt, mode, stream);
        case 32: return launch_decode_dv<32>(idx, st, q, k, v, out, in_dt, out_dt, mode, stream);
        case 64: return launch_decode_dv<64>(idx, st, q, k, v, out, in_dt, out_dt, mode, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sata
