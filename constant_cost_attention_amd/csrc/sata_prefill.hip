// Chunked SATA prefill for gfx950.
//
// The sequence is cut into chunks of C tokens.  For a chunk c of a head
//   Y_c   = psi(Q_c) . S^(c-1)                          (inter-chunk readout)
//         + (w(Q_c K_c^T / sqrt d) o causal) [V_c | 1]  (intra-chunk, direct)
//   S^(c) = S^(c-1) + phi(K_c)^T [V_c | 1]              (chunk state, scanned)
//   o     = Y_c[:, :d_V] / Y_c[:, d_V]
// with phi the plain key monomial of every feature and psi the query monomial
// times 1/(alpha! d^(p/2)) [hotdry, "Core insight of symmetric tensor
// decomposition"; "Engineering realisation of the constant compute cost":
// fixed state S_p = sum phi_p(k) (x) [v, 1], orders weighted and summed, the
// "+1" column normalises].  All contractions are dense GEMMs on MFMA (bf16
// operands for bf16 inputs, fp32 operands for fp32 inputs) with fp32
// accumulation.
//
// Kernel 1 (scan), grid (slices, B*H), 4 wavefronts.  A workgroup owns a
// slice of the head's features, viewed as "quads" (a pair prefix i1 <= i2 and
// an aligned block of four last indices, see sata_internal.h), and keeps that
// slice of the fp32 state in MFMA accumulators for its whole walk over the
// chunks: the state does not leave the chip between chunks, and every order is
// scanned in the same grid [hotdry, "Hardware optimisation paths and current
// limits": the orders are independent; the hierarchical index structure].
// Per chunk it stages Q, K (fp32) and [V | 1] (operand dtype) in LDS, forms
// the query and key features of its slice in registers (one pair product per
// quad, one aligned 16-byte load per four features), reads out its share of
// Y_c, adds the direct intra-chunk term for the query tiles it owns, updates
// its state slice, adds the four wavefronts' readouts in LDS and writes one
// partial per chunk.
//   MFMA tiles: 16x16x32 bf16 or 16x16x4 fp32.  A 16-feature tile holds four
//   quads (rows 4s + r = quad s, slot r).  The accumulator rows a lane owns
//   (rows 4g..4g+3) are exactly the K-slots the next MFMA wants from it, so
//   the state feeds the readout as an operand without data movement.
// Kernel 2 (reduce), grid (chunks, B*H): adds the slices' partials in a fixed
// order and normalises by the "+1" column.  Results are deterministic.
//
//   [hotdry] blog.hotdry.top, "Symmetry-aware Taylor approximation attention:
//            engineering a constant per-token cost" (2026-02-05).
#include <algorithm>

#include "sata_device.h"
#include "sata_internal.h"

namespace sata {

constexpr int kNW = 4;                           // wavefronts per workgroup
constexpr int kThreads = 64 * kNW;
constexpr int64_t kWorkCap = (int64_t)4 << 30;   // partial-sum workspace cap (bytes)

template <int D, int DV, int C, int MT, typename TIn>
struct ScanCfg {
    static constexpr bool BF = sizeof(TIn) == 2;
    static constexpr int NQW = 4 * MT;           // quads per wavefront (four streams of MT)
    static constexpr int NQ = kNW * NQW;         // quads per workgroup (slice)
    static constexpr int NC = DV + 1;            // value columns + normaliser
    static constexpr int NT = (NC + 15) / 16;    // 16-column MFMA tiles
    static constexpr int NCP = NT * 16;
    static constexpr int TT = C / 16;            // 16-token tiles per chunk
    static constexpr int TH = (BF ? 64 : 32) < C ? (BF ? 64 : 32) : C;   // tokens per readout pass
    static constexpr int TTH = TH / 16;          // token tiles per pass
    static constexpr int NH = C / TH;            // passes per chunk
    static constexpr int KR = D + 4;             // K rows: d_K dims, then 1, 0, 0, 0
    static constexpr int KS = C + 4;             // Kt row stride (floats)
    static constexpr int QS = D + 4;             // Qs row stride (floats): dims, then 1, 0, 0, 0
    static constexpr int VS = BF ? C + 8 : C + 4;   // Vt row stride (elements)
    static constexpr int ES = BF ? 2 : 4;
    static constexpr int OFF_K = 0;
    static constexpr int OFF_Q = OFF_K + KR * KS * 4;
    static constexpr int OFF_V = OFF_Q + TH * QS * 4;
    static constexpr int OFF_Y = (OFF_V + NC * VS * ES + 15) / 16 * 16;
    static constexpr int YB = TTH * NT * 64;     // f32x4 per wavefront readout buffer
    static constexpr int OFF_W = OFF_Y + kNW * YB * 16;
    static constexpr int OFF_QC = OFF_W + NQ * 4;
    static constexpr int LDS = OFF_QC + NQ * 16;
    static_assert(MT % 2 == 0, "tiles per wave must be even");
    static_assert(C % 32 == 0, "chunk must be a multiple of 32");
    static_assert(D % 8 == 0, "d_K must be a multiple of 8");
    static_assert(TTH <= kNW, "one token tile per wavefront in the reduce-scatter");
    static_assert(OFF_V % 16 == 0 && OFF_QC % 16 == 0, "alignment");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ int qd_i1(uint32_t w) { return (int)(w & 0xffu); }
__device__ __forceinline__ int qd_i2(uint32_t w) { return (int)((w >> 8) & 0xffu); }
__device__ __forceinline__ int qd_b(uint32_t w) { return (int)((w >> 16) & 0xffu); }
__device__ __forceinline__ uint32_t qd_mask(uint32_t w) { return w >> 24; }
__device__ __forceinline__ uint32_t qd_pair(uint32_t w) { return w & 0xffffu; }

// w(x) = sum_{p<P} x^p/p! (Horner, P <= 4)
__device__ __forceinline__ float taylor_w(float x, float c0, float c1, float c2, float c3, int P) {
    float w = P >= 4 ? c3 : 0.f;
    if (P >= 3) w = w * x + c2;
    if (P >= 2) w = w * x + c1;
    return w * x + c0;
}

struct TaylorArgs {
    float scale, c0, c1, c2, c3;
    int P;
};

// Direct intra-chunk term for query tile qt of chunk (t0, nvalid): Z (rows =
// queries 4g + r, column li of each 16-column tile) receives
// sum_{key <= query} w(q.k/sqrt d) [v, 1][key].  S^T = K Q^T is formed on MFMA
// with q and k read straight from global memory; its accumulator rows are the
// K-slots of the W [V|1] product, so W never leaves the registers.  [V | 1]
// comes from LDS (operand dtype, dim-major, row stride VS).
template <int D, int NT, int VS, typename TIn>
__device__ __forceinline__ void intra_tile(f32x4 (&Z)[NT], int qt, int g, int li, const TIn *qh, const TIn *kh,
                                           int64_t t0, int nvalid, const unsigned char *vt,
                                           const TaylorArgs &ta) {
    const int query = 16 * qt + li;
    if constexpr (sizeof(TIn) == 2) {
        constexpr int DS = D < 32 ? 1 : D / 32;            // 32-dim K steps (zero-padded below 32)
        const bf16_t *Vt = reinterpret_cast<const bf16_t *>(vt);
        auto load8 = [&](const TIn *base, int tok, int d0) -> bf16x8 {
            uint4 u = {0u, 0u, 0u, 0u};
            if (tok < nvalid && d0 < D) u = *reinterpret_cast<const uint4 *>(base + (t0 + tok) * D + d0);
            return __builtin_bit_cast(bf16x8, u);
        };
        bf16x8 Bq[DS];
#pragma unroll
        for (int s = 0; s < DS; ++s) Bq[s] = load8(qh, query, 32 * s + 8 * g);
        const int nks = qt / 2 + 1;                          // 32-key steps up to the diagonal
        for (int ks = 0; ks < nks; ++ks) {
            f32x4 sA = {0.f, 0.f, 0.f, 0.f}, sB = {0.f, 0.f, 0.f, 0.f};
            const int kA = 32 * ks + li, kB = kA + 16;        // this lane's key rows (A operand)
#pragma unroll
            for (int s = 0; s < DS; ++s) {
                sA = mfma_bf16(load8(kh, kA, 32 * s + 8 * g), Bq[s], sA);
                sB = mfma_bf16(load8(kh, kB, 32 * s + 8 * g), Bq[s], sB);
            }
            // S^T rows are keys 32ks + 4g + r (and +16), column is the query -> W[query][key]
            float w8[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int keyA = 32 * ks + 4 * g + r, keyB = keyA + 16;
                w8[r] = keyA <= query ? taylor_w(sA[r] * ta.scale, ta.c0, ta.c1, ta.c2, ta.c3, ta.P) : 0.f;
                w8[4 + r] = keyB <= query ? taylor_w(sB[r] * ta.scale, ta.c0, ta.c1, ta.c2, ta.c3, ta.P) : 0.f;
            }
            const bf16x8 A = pack_bf16x8(w8);
            // [V | 1] operand in the same key order: keys 32ks + 4g + 0..3 and +16
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const bf16_t *vr = Vt + (16 * nt + li) * VS + 32 * ks + 4 * g;
                const uint2 lo = *reinterpret_cast<const uint2 *>(vr);
                const uint2 hi = *reinterpret_cast<const uint2 *>(vr + 16);
                const uint4 u = {lo.x, lo.y, hi.x, hi.y};
                Z[nt] = mfma_bf16(A, __builtin_bit_cast(bf16x8, u), Z[nt]);
            }
        }
    } else {
        const float *Vt = reinterpret_cast<const float *>(vt);
        const bool qok = query < nvalid;
        for (int kt = 0; kt <= qt; ++kt) {
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
            const int key = 16 * kt + li;
            const bool kok = key < nvalid;
#pragma unroll
            for (int d4 = 0; d4 < D / 4; ++d4) {
                const int dd = 4 * d4 + g;
                const float a = kok ? to_f32(kh[(t0 + key) * D + dd]) : 0.f;
                const float b = qok ? to_f32(qh[(t0 + query) * D + dd]) : 0.f;
                s = mfma_f32(a, b, s);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int kr = 16 * kt + 4 * g + r;
                const float w = kr <= query ? taylor_w(s[r] * ta.scale, ta.c0, ta.c1, ta.c2, ta.c3, ta.P) : 0.f;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) Z[nt] = mfma_f32(w, Vt[(16 * nt + li) * VS + kr], Z[nt]);
            }
        }
    }
}

// Stage [V | 1] of a chunk into LDS, dim-major (row c, token t), operand dtype;
// invalid tokens get zeros (also in the ones column), so they add nothing.
// Writes rows 0..ROWS-1 (row DV is the ones column, rows above it zero).
template <int DV, int C, int ROWS, int VS, typename TIn>
__device__ __forceinline__ void stage_v(unsigned char *vt, const TIn *vh, int64_t t0, int nvalid, int tid,
                                        int nthreads) {
    for (int i = tid; i < C * ((ROWS + 7) / 8); i += nthreads) {
        const int t = i % C, c8 = (i / C) * 8;     // consecutive lanes: consecutive tokens
        float val[8];
        if (t < nvalid && c8 < DV) {
            const int64_t src = (t0 + t) * DV + c8;
            if constexpr (sizeof(TIn) == 2) {
                const uint4 u = *reinterpret_cast<const uint4 *>(vh + src);
                const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    val[2 * j] = __uint_as_float(uw[j] << 16);
                    val[2 * j + 1] = __uint_as_float(uw[j] & 0xffff0000u);
                }
            } else {
                const float4 a = *reinterpret_cast<const float4 *>(vh + src);
                const float4 b = *reinterpret_cast<const float4 *>(vh + src + 4);
                val[0] = a.x; val[1] = a.y; val[2] = a.z; val[3] = a.w;
                val[4] = b.x; val[5] = b.y; val[6] = b.z; val[7] = b.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) val[j] = (t < nvalid && c8 + j == DV) ? 1.f : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (c8 + j >= ROWS) break;
            if constexpr (sizeof(TIn) == 2) reinterpret_cast<bf16_t *>(vt)[(c8 + j) * VS + t] = from_f32<bf16_t>(val[j]);
            else reinterpret_cast<float *>(vt)[(c8 + j) * VS + t] = val[j];
        }
    }
}

template <int D, int DV, int C, int MT, typename TIn>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_scan_kernel(const uint32_t *__restrict__ qw0, const int32_t *__restrict__ qcidx,
                         const float4 *__restrict__ qcoef, float *__restrict__ state, int64_t m_pad,
                         const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
                         int64_t n, int64_t tok0, int nchunk, float *__restrict__ partial, float qscale) {
    using Cfg = ScanCfg<D, DV, C, MT, TIn>;
    constexpr int NC = Cfg::NC, NT = Cfg::NT, TT = Cfg::TT, TH = Cfg::TH, TTH = Cfg::TTH;
    constexpr int KS = Cfg::KS, QS = Cfg::QS, VS = Cfg::VS, NQ = Cfg::NQ, NQW = Cfg::NQW, YB = Cfg::YB;
    extern __shared__ __align__(16) unsigned char lds[];
    float *Kt = reinterpret_cast<float *>(lds + Cfg::OFF_K);      // [KR][KS]  dim-major, whole chunk
    float *Qs = reinterpret_cast<float *>(lds + Cfg::OFF_Q);      // [TH][QS]  one readout pass, dims scaled
    f32x4 *Yb = reinterpret_cast<f32x4 *>(lds + Cfg::OFF_Y);      // [kNW][TTH][NT][64] accumulator layout
    uint32_t *W0 = reinterpret_cast<uint32_t *>(lds + Cfg::OFF_W);   // [NQ]
    float4 *QC = reinterpret_cast<float4 *>(lds + Cfg::OFF_QC);      // [NQ]

    const int slice = blockIdx.x, nslices = gridDim.x;
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int64_t qs0 = (int64_t)slice * NQ;          // first quad of the slice
    const int wq0 = wave * NQW;                       // first quad of this wave within the slice
    // Four streams of MT consecutive quads per wave: tile j holds quad wq0 + s*MT + j in rows 4s..4s+3.
    // This lane's accumulator rows (4g + r) are stream g; its update rows (li) are stream li/4, slot li%4.

    for (int i = tid; i < NQ; i += kThreads) {
        W0[i] = qw0[qs0 + i];
        QC[i] = qcoef[qs0 + i];
    }

    float *Sh = state + bh * NC * m_pad;
    f32x4 S[MT][NT];
#pragma unroll
    for (int j = 0; j < MT; ++j) {
        const int64_t qd = qs0 + wq0 + g * MT + j;
        const uint32_t w = qw0[qd];
        const int32_t c0 = qcidx[qd];
        const uint32_t mask = qd_mask(w);
        const int z0 = mask ? __builtin_ctz(mask) : 0;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int c = 16 * nt + li;
                const bool ok = ((mask >> r) & 1u) && c < NC;
                S[j][nt][r] = ok ? Sh[(int64_t)c * m_pad + c0 + (r - z0)] : 0.f;
            }
    }
    __syncthreads();

    uint32_t myW[MT];                                  // update rows: stream li/4
#pragma unroll
    for (int j = 0; j < MT; ++j) myW[j] = W0[wq0 + (li >> 2) * MT + j];
    uint32_t shared_pair = 0;                          // readout K step kk: quads 2kk, 2kk+1 of stream g
#pragma unroll
    for (int kk = 0; kk < MT / 2; ++kk) {
        const int qa = wq0 + g * MT + 2 * kk;
        if (__all(qd_pair(W0[qa]) == qd_pair(W0[qa + 1]))) shared_pair |= 1u << kk;
    }

    const TIn *qh = q + bh * n * D;
    const TIn *kh = k + bh * n * D;
    const TIn *vh = v + bh * n * DV;

    auto stage_q = [&](int64_t tq0, int nq_valid) {
        for (int i = tid; i < TH * (D / 8); i += kThreads) {
            const int t = i % TH, d8 = (i / TH) * 8;
            float qv[8];
            if (t < nq_valid) {
                const int64_t src = (tq0 + t) * D + d8;
                if constexpr (Cfg::BF) {
                    const uint4 qu = *reinterpret_cast<const uint4 *>(qh + src);
                    const uint32_t qw[4] = {qu.x, qu.y, qu.z, qu.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        qv[2 * j] = __uint_as_float(qw[j] << 16);
                        qv[2 * j + 1] = __uint_as_float(qw[j] & 0xffff0000u);
                    }
                } else {
                    const float4 q0 = *reinterpret_cast<const float4 *>(qh + src);
                    const float4 q1 = *reinterpret_cast<const float4 *>(qh + src + 4);
                    qv[0] = q0.x; qv[1] = q0.y; qv[2] = q0.z; qv[3] = q0.w;
                    qv[4] = q1.x; qv[5] = q1.y; qv[6] = q1.z; qv[7] = q1.w;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) qv[j] = 0.f;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) qv[j] *= qscale;
            *reinterpret_cast<float4 *>(Qs + t * QS + d8) = float4{qv[0], qv[1], qv[2], qv[3]};
            *reinterpret_cast<float4 *>(Qs + t * QS + d8 + 4) = float4{qv[4], qv[5], qv[6], qv[7]};
        }
        for (int t = tid; t < TH; t += kThreads)
            *reinterpret_cast<float4 *>(Qs + t * QS + D) = float4{1.f, 0.f, 0.f, 0.f};
    };

    for (int cc = 0; cc < nchunk; ++cc) {
        const int64_t t0 = tok0 + (int64_t)cc * C;
        const int nvalid = n - t0 < C ? (int)(n - t0) : C;
        __syncthreads();          // previous chunk: update done with Kt/Vt, reduce-scatter done with Yb
        // ---- stage K (dim-major fp32), [V | 1] (operand dtype) for the chunk, Q for pass 0
        for (int i = tid; i < C * (D / 8); i += kThreads) {
            const int t = i % C, d8 = (i / C) * 8;     // consecutive lanes: consecutive tokens
            float kv[8];
            if (t < nvalid) {
                const int64_t src = (t0 + t) * D + d8;
                if constexpr (Cfg::BF) {
                    const uint4 ku = *reinterpret_cast<const uint4 *>(kh + src);
                    const uint32_t kw[4] = {ku.x, ku.y, ku.z, ku.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        kv[2 * j] = __uint_as_float(kw[j] << 16);
                        kv[2 * j + 1] = __uint_as_float(kw[j] & 0xffff0000u);
                    }
                } else {
                    const float4 k0 = *reinterpret_cast<const float4 *>(kh + src);
                    const float4 k1 = *reinterpret_cast<const float4 *>(kh + src + 4);
                    kv[0] = k0.x; kv[1] = k0.y; kv[2] = k0.z; kv[3] = k0.w;
                    kv[4] = k1.x; kv[5] = k1.y; kv[6] = k1.z; kv[7] = k1.w;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) kv[j] = 0.f;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) Kt[(d8 + j) * KS + t] = kv[j];
        }
        for (int t = tid; t < C; t += kThreads) {
            Kt[D * KS + t] = 1.f;
            Kt[(D + 1) * KS + t] = 0.f; Kt[(D + 2) * KS + t] = 0.f; Kt[(D + 3) * KS + t] = 0.f;
        }
        stage_v<DV, C, NC, VS, TIn>(lds + Cfg::OFF_V, vh, t0, nvalid, tid, kThreads);
        stage_q(t0, nvalid);
        __syncthreads();

        // ---- inter-chunk readout, Y = psi(Q_c)[:, slice] . S^(c-1)[slice, :], in passes of TH
        //      tokens; each wave's partial goes to its own LDS buffer, then wave w adds the four
        //      buffers' token tile w and writes it out (one barrier, no serial chain)
#pragma unroll
        for (int hf = 0; hf < Cfg::NH; ++hf) {
            if (hf > 0) {
                const int64_t tq0 = t0 + hf * TH;
                stage_q(tq0, n - tq0 < TH ? (int)(n - tq0) : TH);
                __syncthreads();
            }
            f32x4 Y[TTH][NT];
#pragma unroll
            for (int tt = 0; tt < TTH; ++tt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) Y[tt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

            if constexpr (Cfg::BF) {
                // psi = coef_z * (q_i1 q_i2) * q_(4b+z); q carries 1/sqrt(d), coef_z = 1/alpha!
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
                    const int qa = wq0 + g * MT + 2 * kk, qb = qa + 1;
                    const uint32_t wa = W0[qa], wb = W0[qb];
                    const float4 ca = QC[qa], cb = QC[qb];
                    const bool sp = (shared_pair >> kk) & 1u;
                    const int a1 = qd_i1(wa), a2 = qd_i2(wa), ab = 4 * qd_b(wa);
                    const int b1 = qd_i1(wb), b2 = qd_i2(wb), bb = 4 * qd_b(wb);
                    const float *row = Qs + li * QS;
                    float pa1 = row[a1], pa2 = row[a2], pb1 = 0.f, pb2 = 0.f;
                    if (!sp) { pb1 = row[b1]; pb2 = row[b2]; }
                    float4 xa = *reinterpret_cast<const float4 *>(row + ab);
                    float4 xb = *reinterpret_cast<const float4 *>(row + bb);
#pragma unroll
                    for (int tt = 0; tt < TTH; ++tt) {
                        float npa1 = 0.f, npa2 = 0.f, npb1 = 0.f, npb2 = 0.f;
                        float4 nxa = {0.f, 0.f, 0.f, 0.f}, nxb = {0.f, 0.f, 0.f, 0.f};
                        if (tt + 1 < TTH) {          // next tile's loads go out before this tile's math
                            const float *nrow = Qs + (16 * (tt + 1) + li) * QS;
                            npa1 = nrow[a1]; npa2 = nrow[a2];
                            if (!sp) { npb1 = nrow[b1]; npb2 = nrow[b2]; }
                            nxa = *reinterpret_cast<const float4 *>(nrow + ab);
                            nxb = *reinterpret_cast<const float4 *>(nrow + bb);
                        }
                        const float pa = pa1 * pa2;
                        const float pb = sp ? pa : pb1 * pb2;
                        float a[8] = {ca.x * xa.x, ca.y * xa.y, ca.z * xa.z, ca.w * xa.w,
                                      cb.x * xb.x, cb.y * xb.y, cb.z * xb.z, cb.w * xb.w};
#pragma unroll
                        for (int j = 0; j < 4; ++j) { a[j] *= pa; a[4 + j] *= pb; }
                        const bf16x8 A = pack_bf16x8(a);
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) Y[tt][nt] = mfma_bf16(A, B[nt], Y[tt][nt]);
                        pa1 = npa1; pa2 = npa2; pb1 = npb1; pb2 = npb2; xa = nxa; xb = nxb;
                    }
                }
            } else {
                // K step (j, r): lane group g holds slot r of quad wq0 + g*MT + j
#pragma unroll
                for (int j = 0; j < MT; ++j) {
                    const int qd = wq0 + g * MT + j;
                    const uint32_t w = W0[qd];
                    const float4 cq = QC[qd];
                    const float cr[4] = {cq.x, cq.y, cq.z, cq.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
#pragma unroll
                        for (int tt = 0; tt < TTH; ++tt) {
                            const float *row = Qs + (16 * tt + li) * QS;
                            const float a = cr[r] * row[qd_i1(w)] * row[qd_i2(w)] * row[4 * qd_b(w) + r];
#pragma unroll
                            for (int nt = 0; nt < NT; ++nt) Y[tt][nt] = mfma_f32(a, S[j][nt][r], Y[tt][nt]);
                        }
                    }
                }
            }

            f32x4 *mine = Yb + wave * YB;
#pragma unroll
            for (int tt = 0; tt < TTH; ++tt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) mine[(tt * NT + nt) * 64 + lane] = Y[tt][nt];
            __syncthreads();
            if (wave < TTH) {
                // partial layout per (bh, chunk, slice): [tt][c][16 tokens]; lane writes rows 4g..4g+3
                float *pdst = partial + ((bh * nchunk + cc) * nslices + slice) * (int64_t)(TT * NC * 16);
                const int tt = wave;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const int c = 16 * nt + li;
                    if (c < NC) {
                        f32x4 y = Yb[(tt * NT + nt) * 64 + lane];
#pragma unroll
                        for (int w = 1; w < kNW; ++w) y += Yb[w * YB + (tt * NT + nt) * 64 + lane];
                        *reinterpret_cast<f32x4 *>(pdst + ((int64_t)(hf * TTH + tt) * NC + c) * 16 + 4 * g) = y;
                    }
                }
            }
            if (hf + 1 < Cfg::NH) __syncthreads();   // Yb and Qs are rewritten by the next pass
        }

        // ---- chunk state: S[slice, :] += phi(K_c)[:, slice]^T [V_c | 1]
        if constexpr (Cfg::BF) {
            const bf16_t *Vt = reinterpret_cast<const bf16_t *>(lds + Cfg::OFF_V);
#pragma unroll 1
            for (int ks = 0; ks < C / 32; ++ks) {
                const int tb = 32 * ks + 8 * g;
                bf16x8 B[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    uint4 u = {0u, 0u, 0u, 0u};
                    if (16 * nt + li < NC) u = *reinterpret_cast<const uint4 *>(Vt + (16 * nt + li) * VS + tb);
                    B[nt] = __builtin_bit_cast(bf16x8, u);
                }
                float p2[8];
#pragma unroll
                for (int j = 0; j < MT; ++j) {
                    const uint32_t w = myW[j];
                    if (j == 0 || qd_pair(w) != qd_pair(myW[j > 0 ? j - 1 : 0])) {   // per lane: new pair
                        const float4 *k1 = reinterpret_cast<const float4 *>(Kt + qd_i1(w) * KS + tb);
                        const float4 *k2 = reinterpret_cast<const float4 *>(Kt + qd_i2(w) * KS + tb);
                        const float4 a0 = k1[0], a1 = k1[1], b0 = k2[0], b1 = k2[1];
                        p2[0] = a0.x * b0.x; p2[1] = a0.y * b0.y; p2[2] = a0.z * b0.z; p2[3] = a0.w * b0.w;
                        p2[4] = a1.x * b1.x; p2[5] = a1.y * b1.y; p2[6] = a1.z * b1.z; p2[7] = a1.w * b1.w;
                    }
                    const float4 *k3 = reinterpret_cast<const float4 *>(Kt + (4 * qd_b(w) + (li & 3)) * KS + tb);
                    const float4 c0 = k3[0], c1 = k3[1];
                    float a[8] = {p2[0] * c0.x, p2[1] * c0.y, p2[2] * c0.z, p2[3] * c0.w,
                                  p2[4] * c1.x, p2[5] * c1.y, p2[6] * c1.z, p2[7] * c1.w};
                    const bf16x8 A = pack_bf16x8(a);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) S[j][nt] = mfma_bf16(A, B[nt], S[j][nt]);
                }
            }
        } else {
            const float *Vt = reinterpret_cast<const float *>(lds + Cfg::OFF_V);
#pragma unroll 1
            for (int ks = 0; ks < C / 4; ++ks) {
                const int tb = 4 * ks + g;
                float B[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) B[nt] = 16 * nt + li < NC ? Vt[(16 * nt + li) * VS + tb] : 0.f;
#pragma unroll
                for (int j = 0; j < MT; ++j) {
                    const uint32_t w = myW[j];
                    const float a = Kt[qd_i1(w) * KS + tb] * Kt[qd_i2(w) * KS + tb] *
                                    Kt[(4 * qd_b(w) + (li & 3)) * KS + tb];
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) S[j][nt] = mfma_f32(a, B[nt], S[j][nt]);
                }
            }
        }
    }

    // accumulators -> state slice
#pragma unroll
    for (int j = 0; j < MT; ++j) {
        const int64_t qd = qs0 + wq0 + g * MT + j;
        const uint32_t w = qw0[qd];
        const int32_t c0 = qcidx[qd];
        const uint32_t mask = qd_mask(w);
        const int z0 = mask ? __builtin_ctz(mask) : 0;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int c = 16 * nt + li;
                if (((mask >> r) & 1u) && c < NC) Sh[(int64_t)c * m_pad + c0 + (r - z0)] = S[j][nt][r];
            }
    }
}

// Kernel 2: y = (direct intra-chunk term) + sum over slices of the partials
// (fixed order), o = y[:d_V] / y[d_V].  Partial layout per (bh, chunk, slice):
// [C/16][d_V+1][16 tokens] fp32.  Every thread first adds the slices' partials
// with 16-byte loads; then wave w < C/32 adds the intra-chunk term of query
// tiles w and C/16-1-w (tile qt needs qt+1 key tiles, so each wave does
// C/16+1 tiles' worth).
template <int D, int DV, int C, typename TIn, typename TOut>
__global__ __launch_bounds__(256) void prefill_reduce_kernel(const float *__restrict__ partial, int nslices,
                                                             int nchunk, int64_t n, int64_t tok0,
                                                             const TIn *__restrict__ q, const TIn *__restrict__ k,
                                                             const TIn *__restrict__ v, TOut *__restrict__ out,
                                                             TaylorArgs ta) {
    constexpr int NC = DV + 1, TT = C / 16, NT = (NC + 15) / 16, NCP = 16 * NT;
    constexpr int VS = sizeof(TIn) == 2 ? C + 8 : C + 4;
    constexpr int NV = TT * NC * 4;                 // float4 per partial
    constexpr int PER = (NV + 255) / 256;
    constexpr int VBYTES = NCP * VS * (int)sizeof(TIn);
    __shared__ __align__(16) unsigned char vt[VBYTES];
    __shared__ __align__(16) float ys[TT * NC * 16];
    const int cc = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int64_t t0 = tok0 + (int64_t)cc * C;
    const int nvalid = n - t0 < C ? (int)(n - t0) : C;
    const TIn *qh = q + bh * n * D;
    const TIn *kh = k + bh * n * D;
    const TIn *vh = v + bh * n * DV;

    // partial sums first: their loads are the long pole, issue them before the MFMA work
    const float4 *base = reinterpret_cast<const float4 *>(partial) + (bh * nchunk + cc) * (int64_t)nslices * NV;
    float4 acc[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] = float4{0.f, 0.f, 0.f, 0.f};
    int s = 0;
    for (; s + 1 < nslices; s += 2) {
        const float4 *p0 = base + (int64_t)s * NV, *p1 = p0 + NV;
        float4 a[PER], b[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int i = tid + 256 * j;
            a[j] = i < NV ? p0[i] : float4{0.f, 0.f, 0.f, 0.f};
            b[j] = i < NV ? p1[i] : float4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            acc[j].x += a[j].x; acc[j].y += a[j].y; acc[j].z += a[j].z; acc[j].w += a[j].w;
            acc[j].x += b[j].x; acc[j].y += b[j].y; acc[j].z += b[j].z; acc[j].w += b[j].w;
        }
    }
    if (s < nslices) {
        const float4 *p0 = base + (int64_t)s * NV;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int i = tid + 256 * j;
            if (i < NV) {
                const float4 a = p0[i];
                acc[j].x += a.x; acc[j].y += a.y; acc[j].z += a.z; acc[j].w += a.w;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int i = tid + 256 * j;
        if (i < NV) reinterpret_cast<float4 *>(ys)[i] = acc[j];
    }

    stage_v<DV, C, NCP, VS, TIn>(vt, vh, t0, nvalid, tid, 256);
    __syncthreads();
    static_assert(TT % 2 == 0 && TT / 2 <= 4, "query tiles pair up over the four wavefronts");
    if (wave < TT / 2) {
        const int qt = wave;
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int qq = pass == 0 ? qt : TT - 1 - qt;    // tiles w and TT-1-w: w+1 + TT-w key tiles
            f32x4 Z[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) Z[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            intra_tile<D, NT, VS, TIn>(Z, qq, g, li, qh, kh, t0, nvalid, vt, ta);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int c = 16 * nt + li;
                if (c < NC) {
                    float4 *p = reinterpret_cast<float4 *>(ys + (qq * NC + c) * 16 + 4 * g);
                    const float4 o = *p;
                    *p = float4{o.x + Z[nt][0], o.y + Z[nt][1], o.z + Z[nt][2], o.w + Z[nt][3]};
                }
            }
        }
    }
    __syncthreads();
    for (int i = tid; i < C * DV; i += 256) {
        const int t = i / DV, c = i - t * DV;
        if (t < nvalid) {
            const int tt = t >> 4, t16 = t & 15;
            const float y = ys[(tt * NC + c) * 16 + t16];
            const float den = ys[(tt * NC + DV) * 16 + t16];
            out[(bh * n + t0 + t) * DV + c] = from_f32<TOut>(y / den);
        }
    }
}

// ---------------------------------------------------------------- host side

// Tiles per wavefront (16 features each, four quads): as many as the register
// budget allows for the d_V + 1 columns, fewer when the head has few features.
static int pick_mt(const sata_index *idx, int64_t bh) {
    for (int mt : {8, 4}) {
        const int64_t per = (int64_t)kNW * 4 * mt;
        if (bh * ((idx->nq + per - 1) / per) >= 256) return mt;
    }
    return 2;
}

PrefillPlan plan_prefill(const sata_index *idx, int64_t bh, int64_t n, int chunk, sata_dtype in_dt) {
    PrefillPlan p;
    (void)in_dt;
    p.chunk = chunk ? chunk : (idx->dk == 64 ? 128 : 64);
    if (p.chunk != 64 && p.chunk != 128) return p;
    const int mt = pick_mt(idx, bh);
    p.fw = 16 * mt;
    p.fs = kNW * p.fw;
    const int64_t nq_slice = (int64_t)kNW * 4 * mt;
    p.slices = (int)((idx->nq + nq_slice - 1) / nq_slice);
    const int64_t nchunks = (n + p.chunk - 1) / p.chunk;
    const int64_t per_chunk = bh * p.slices * (int64_t)p.chunk * (idx->dv + 1) * 4;
    p.seg_chunks = std::max<int64_t>(1, std::min<int64_t>(nchunks, kWorkCap / per_chunk));
    p.work_bytes = p.seg_chunks * per_chunk;
    p.ok = (int64_t)p.slices * nq_slice <= idx->nq_tab;
    return p;
}

template <int D, int C, int MT, typename TIn, typename TOut>
static hipError_t run_prefill(const sata_index *idx, const sata_state *st, const PrefillPlan &plan,
                              const void *q, const void *k, const void *v, void *out, int64_t n,
                              hipStream_t stream) {
    using Cfg = ScanCfg<D, D, C, MT, TIn>;
    const int64_t bh = (int64_t)st->batch * st->heads;
    auto scan = prefill_scan_kernel<D, D, C, MT, TIn>;
    auto red = prefill_reduce_kernel<D, D, C, TIn, TOut>;
    hipError_t e = hipFuncSetAttribute((const void *)scan, hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS);
    if (e != hipSuccess) return e;
    TaylorArgs ta;
    ta.scale = 1.0f / sqrtf((float)D);
    ta.c0 = idx->taylor[0]; ta.c1 = idx->taylor[1]; ta.c2 = idx->taylor[2]; ta.c3 = idx->taylor[3];
    ta.P = idx->P;
    const int64_t nchunks = (n + C - 1) / C;
    float *partial = static_cast<float *>(st->d_work);
    for (int64_t c0 = 0; c0 < nchunks; c0 += plan.seg_chunks) {
        const int nseg = (int)std::min<int64_t>(plan.seg_chunks, nchunks - c0);
        const int64_t tok0 = c0 * C;
        {
            ProfScope ps(kProfScan, stream);
            hipLaunchKernelGGL(scan, dim3(plan.slices, (unsigned)bh), dim3(kThreads), Cfg::LDS, stream,
                               idx->d_qw0, idx->d_qcidx, reinterpret_cast<const float4 *>(idx->d_qcoef),
                               st->d_state, idx->m_pad, static_cast<const TIn *>(q),
                               static_cast<const TIn *>(k), static_cast<const TIn *>(v), n, tok0, nseg,
                               partial, ta.scale);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        {
            ProfScope ps(kProfCombine, stream);
            hipLaunchKernelGGL(red, dim3(nseg, (unsigned)bh), dim3(256), 0, stream, partial, plan.slices, nseg,
                               n, tok0, static_cast<const TIn *>(q), static_cast<const TIn *>(k),
                               static_cast<const TIn *>(v), static_cast<TOut *>(out), ta);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int D, int C, int MT>
static hipError_t run_dt(const sata_index *idx, const sata_state *st, const PrefillPlan &plan,
                         const void *q, const void *k, const void *v, void *out, int64_t n,
                         sata_dtype in_dt, sata_dtype out_dt, hipStream_t s) {
    if (in_dt == SATA_F32) {
        if (out_dt == SATA_F32) return run_prefill<D, C, MT, float, float>(idx, st, plan, q, k, v, out, n, s);
        return run_prefill<D, C, MT, float, bf16_t>(idx, st, plan, q, k, v, out, n, s);
    }
    if (out_dt == SATA_F32) return run_prefill<D, C, MT, bf16_t, float>(idx, st, plan, q, k, v, out, n, s);
    return run_prefill<D, C, MT, bf16_t, bf16_t>(idx, st, plan, q, k, v, out, n, s);
}

template <int D>
static hipError_t run_d(const sata_index *idx, const sata_state *st, const PrefillPlan &plan,
                        const void *q, const void *k, const void *v, void *out, int64_t n,
                        sata_dtype in_dt, sata_dtype out_dt, hipStream_t s) {
    const int mt = plan.fw / 16;
    if (plan.chunk == 64) {
        if (mt == 2) return run_dt<D, 64, 2>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, s);
        if (mt == 4) return run_dt<D, 64, 4>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, s);
        return run_dt<D, 64, 8>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, s);
    }
    if (mt == 2) return run_dt<D, 128, 2>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, s);
    if (mt == 4) return run_dt<D, 128, 4>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, s);
    return run_dt<D, 128, 8>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, s);
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
