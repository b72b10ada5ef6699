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
    static constexpr int NQW = 4 * MT;           // quads per wavefront
    static constexpr int NQ = kNW * NQW;         // quads per workgroup (slice)
    static constexpr int NC = DV + 1;            // value columns + normaliser
    static constexpr int NT = (NC + 15) / 16;    // 16-column MFMA tiles
    static constexpr int NCP = NT * 16;
    static constexpr int TT = C / 16;            // 16-token tiles per chunk
    static constexpr int TH = C < 64 ? C : 64;   // tokens per readout pass (register budget)
    static constexpr int TTH = TH / 16;          // token tiles per pass
    static constexpr int NH = C / TH;            // passes per chunk
    static constexpr int KR = D + 4;             // K rows: d_K dims, then 1, 0, 0, 0
    static constexpr int KS = C + 4;             // Kt row stride (floats)
    static constexpr int QS = D + 4;             // Qs row stride (floats): dims, then 1, 0, 0, 0
    static constexpr int VS = BF ? C + 8 : C + 4;   // Vt row stride (elements)
    static constexpr int ES = BF ? 2 : 4;
    static constexpr int OFF_K = 0;
    static constexpr int OFF_Q = OFF_K + KR * KS * 4;
    static constexpr int OFF_V = OFF_Q + C * QS * 4;
    static constexpr int OFF_Y = OFF_V + NCP * VS * ES;
    static constexpr int OFF_W = OFF_Y + TT * NT * 64 * 16;      // one reduction buffer per pass
    static constexpr int OFF_QC = OFF_W + NQ * 4;
    static constexpr int LDS = OFF_QC + NQ * 16;
    static_assert(MT % 2 == 0, "tiles per wave must be even");
    static_assert(C % 32 == 0, "chunk must be a multiple of 32");
    static_assert(D % 8 == 0, "d_K must be a multiple of 8");
    static_assert(OFF_V % 16 == 0 && OFF_Y % 16 == 0 && OFF_QC % 16 == 0, "alignment");
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

// Direct intra-chunk term for query tile qt of the chunk, key blocks handled by
// this wavefront (every kNW-th K step), added into Z (rows = queries 4g + r,
// column li of each 16-column tile).  Keys after a query get weight 0.
template <class Cfg>
__device__ __forceinline__ void intra_tile(f32x4 (&Z)[Cfg::NT], int qt, int wave, int g, int li,
                                           const float *Kt, const float *Qs, const unsigned char *lds,
                                           const TaylorArgs &ta) {
    constexpr int D = Cfg::D_, KS = Cfg::KS, QS = Cfg::QS, VS = Cfg::VS, NT = Cfg::NT;
    const int query = 16 * qt + li;
    if constexpr (Cfg::BF) {
        // Q^T operand for this query tile: lane (query li, dims 8g..8g+7 of each 32-dim step)
        bf16x8 Bq[D / 32 > 0 ? D / 32 : 1];
        const float *qrow = Qs + query * QS;
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
            float t[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) t[j] = qrow[32 * s + 8 * g + j];
            Bq[s] = pack_bf16x8(t);
        }
        const bf16_t *Vt = reinterpret_cast<const bf16_t *>(lds + Cfg::OFF_V);
        const int nks = qt / 2 + 1;                              // 32-key steps up to the diagonal
        for (int ks = wave; ks < nks; ks += kNW) {
            f32x4 sA = {0.f, 0.f, 0.f, 0.f}, sB = {0.f, 0.f, 0.f, 0.f};
            const int kA = 32 * ks + li, kB = kA + 16;           // this lane's key rows (A operand)
#pragma unroll
            for (int s = 0; s < D / 32; ++s) {
                float ta8[8], tb8[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    ta8[j] = Kt[(32 * s + 8 * g + j) * KS + kA];
                    tb8[j] = Kt[(32 * s + 8 * g + j) * KS + kB];
                }
                sA = mfma_bf16(pack_bf16x8(ta8), Bq[s], sA);
                sB = mfma_bf16(pack_bf16x8(tb8), Bq[s], sB);
            }
            if constexpr (D % 32) {
                // d_K = 8 or 16: one 32-wide K step with zero padding
                float ta8[8], tb8[8], tq[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int dd = 8 * g + j;
                    const bool in = dd < D;
                    ta8[j] = in ? Kt[dd * KS + kA] : 0.f;
                    tb8[j] = in ? Kt[dd * KS + kB] : 0.f;
                    tq[j] = in ? qrow[dd] : 0.f;
                }
                const bf16x8 bq = pack_bf16x8(tq);
                sA = mfma_bf16(pack_bf16x8(ta8), bq, sA);
                sB = mfma_bf16(pack_bf16x8(tb8), bq, sB);
            }
            // S^T rows are keys 4g + r (+16), column is query li -> weights W[query][key]
            float w8[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int keyA = 32 * ks + 4 * g + r, keyB = keyA + 16;
                w8[r] = keyA <= query ? taylor_w(sA[r] * ta.scale, ta.c0, ta.c1, ta.c2, ta.c3, ta.P) : 0.f;
                w8[4 + r] = keyB <= query ? taylor_w(sB[r] * ta.scale, ta.c0, ta.c1, ta.c2, ta.c3, ta.P) : 0.f;
            }
            const bf16x8 A = pack_bf16x8(w8);
            // [V | 1] operand with the same key order: keys 32ks + 4g + 0..3 and +16
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const bf16_t *vr = Vt + (16 * nt + li) * VS + 32 * ks + 4 * g;
                const uint2 lo = *reinterpret_cast<const uint2 *>(vr);
                const uint2 hi = *reinterpret_cast<const uint2 *>(vr + 16);
                uint4 u = {lo.x, lo.y, hi.x, hi.y};
                Z[nt] = mfma_bf16(A, __builtin_bit_cast(bf16x8, u), Z[nt]);
            }
        }
    } else {
        const float *Vt = reinterpret_cast<const float *>(lds + Cfg::OFF_V);
        const int nkt = qt + 1;                                  // 16-key tiles up to the diagonal
        for (int kt = wave; kt < nkt; kt += kNW) {
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
            const int key = 16 * kt + li;
#pragma unroll
            for (int d4 = 0; d4 < D / 4; ++d4) {
                const int dd = 4 * d4 + g;
                s = mfma_f32(Kt[dd * KS + key], Qs[query * QS + dd], s);
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

template <int D, int DV, int C, int MT, typename TIn>
struct ScanCfgD : ScanCfg<D, DV, C, MT, TIn> {
    static constexpr int D_ = D;
};

template <int D, int DV, int C, int MT, typename TIn>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_scan_kernel(const uint32_t *__restrict__ qw0, const int32_t *__restrict__ qcidx,
                         const float4 *__restrict__ qcoef, float *__restrict__ state, int64_t m_pad,
                         const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
                         int64_t n, int64_t tok0, int nchunk, float *__restrict__ partial, TaylorArgs ta) {
    using Cfg = ScanCfgD<D, DV, C, MT, TIn>;
    constexpr int NC = Cfg::NC, NT = Cfg::NT, NCP = Cfg::NCP, TT = Cfg::TT, KR = Cfg::KR;
    constexpr int KS = Cfg::KS, QS = Cfg::QS, VS = Cfg::VS, NQ = Cfg::NQ, NQW = Cfg::NQW;
    extern __shared__ __align__(16) unsigned char lds[];
    float *Kt = reinterpret_cast<float *>(lds + Cfg::OFF_K);      // [KR][KS]  dim-major
    float *Qs = reinterpret_cast<float *>(lds + Cfg::OFF_Q);      // [C][QS]   token-major
    f32x4 *Yr = reinterpret_cast<f32x4 *>(lds + Cfg::OFF_Y);      // [TT][NT][64] accumulator layout
    uint32_t *W0 = reinterpret_cast<uint32_t *>(lds + Cfg::OFF_W);   // [NQ]
    float4 *QC = reinterpret_cast<float4 *>(lds + Cfg::OFF_QC);      // [NQ]

    const int slice = blockIdx.x, nslices = gridDim.x;
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int64_t qs0 = (int64_t)slice * NQ;          // first quad of the slice
    const int wq0 = wave * NQW;                       // first quad of this wave within the slice

    for (int i = tid; i < NQ; i += kThreads) {
        W0[i] = qw0[qs0 + i];
        QC[i] = qcoef[qs0 + i];
    }

    // state slice -> accumulators.  Tile j of this wave = quads wq0 + 4j + s (rows 4s + r);
    // this lane owns rows 4g + r, i.e. quad wq0 + 4j + g, slot r, column 16 nt + li.
    float *Sh = state + bh * NC * m_pad;
    f32x4 S[MT][NT];
#pragma unroll
    for (int j = 0; j < MT; ++j) {
        const int64_t qd = qs0 + wq0 + 4 * j + g;
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

    // update-side quad of this lane's A-operand row li in tile j: quad wq0 + 4j + li/4, slot li%4
    uint32_t myW[MT];
#pragma unroll
    for (int j = 0; j < MT; ++j) myW[j] = W0[wq0 + 4 * j + (li >> 2)];
    // tile j reuses tile j-1's pair products when every row keeps its pair (wave-uniform)
    uint32_t same_prev = 0;
#pragma unroll
    for (int j = 1; j < MT; ++j)
        if (__all(qd_pair(myW[j]) == qd_pair(myW[j - 1]))) same_prev |= 1u << j;

    const TIn *qh = q + bh * n * D;
    const TIn *kh = k + bh * n * D;
    const TIn *vh = v + bh * n * DV;
    const int ntiles_owned = (TT + nslices - 1 - slice) / nslices;   // query tiles qt = slice + i*nslices

    for (int cc = 0; cc < nchunk; ++cc) {
        const int64_t t0 = tok0 + (int64_t)cc * C;
        const int nvalid = n - t0 < C ? (int)(n - t0) : C;
        __syncthreads();
        // ---- stage the chunk (invalid tokens: zeros, so they add nothing)
        for (int i = tid; i < C * (D / 8); i += kThreads) {
            const int t = i % C, d8 = (i / C) * 8;     // consecutive lanes: consecutive tokens
            float kv[8], qv[8];
            if (t < nvalid) {
                const int64_t src = (t0 + t) * D + d8;
                if constexpr (Cfg::BF) {
                    const uint4 ku = *reinterpret_cast<const uint4 *>(kh + src);
                    const uint4 qu = *reinterpret_cast<const uint4 *>(qh + src);
                    const uint32_t kw[4] = {ku.x, ku.y, ku.z, ku.w}, qw[4] = {qu.x, qu.y, qu.z, qu.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        kv[2 * j] = __uint_as_float(kw[j] << 16); kv[2 * j + 1] = __uint_as_float(kw[j] & 0xffff0000u);
                        qv[2 * j] = __uint_as_float(qw[j] << 16); qv[2 * j + 1] = __uint_as_float(qw[j] & 0xffff0000u);
                    }
                } else {
                    const float4 k0 = *reinterpret_cast<const float4 *>(kh + src);
                    const float4 k1 = *reinterpret_cast<const float4 *>(kh + src + 4);
                    const float4 q0 = *reinterpret_cast<const float4 *>(qh + src);
                    const float4 q1 = *reinterpret_cast<const float4 *>(qh + src + 4);
                    kv[0] = k0.x; kv[1] = k0.y; kv[2] = k0.z; kv[3] = k0.w;
                    kv[4] = k1.x; kv[5] = k1.y; kv[6] = k1.z; kv[7] = k1.w;
                    qv[0] = q0.x; qv[1] = q0.y; qv[2] = q0.z; qv[3] = q0.w;
                    qv[4] = q1.x; qv[5] = q1.y; qv[6] = q1.z; qv[7] = q1.w;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) { kv[j] = 0.f; qv[j] = 0.f; }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) Kt[(d8 + j) * KS + t] = kv[j];
            *reinterpret_cast<float4 *>(Qs + t * QS + d8) = float4{qv[0], qv[1], qv[2], qv[3]};
            *reinterpret_cast<float4 *>(Qs + t * QS + d8 + 4) = float4{qv[4], qv[5], qv[6], qv[7]};
        }
        for (int t = tid; t < C; t += kThreads) {
            Kt[D * KS + t] = 1.f;
            Kt[(D + 1) * KS + t] = 0.f; Kt[(D + 2) * KS + t] = 0.f; Kt[(D + 3) * KS + t] = 0.f;
            *reinterpret_cast<float4 *>(Qs + t * QS + D) = float4{1.f, 0.f, 0.f, 0.f};
        }
        for (int i = tid; i < C * (NCP / 8); i += kThreads) {
            const int t = i % C, c8 = (i / C) * 8;     // consecutive lanes: consecutive tokens
            float val[8];
            if (t < nvalid && c8 < DV) {
                const int64_t src = (t0 + t) * DV + c8;
                if constexpr (Cfg::BF) {
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
                if constexpr (Cfg::BF) reinterpret_cast<bf16_t *>(lds + Cfg::OFF_V)[(c8 + j) * VS + t] = from_f32<bf16_t>(val[j]);
                else reinterpret_cast<float *>(lds + Cfg::OFF_V)[(c8 + j) * VS + t] = val[j];
            }
        }
        __syncthreads();

        // ---- inter-chunk readout, Y = psi(Q_c)[:, slice] . S^(c-1)[slice, :], plus the direct
        //      intra-chunk term of the query tiles this slice owns, in passes of TH tokens;
        //      each pass's four wavefront partials are added in a fixed order in LDS
#pragma unroll
        for (int hf = 0; hf < Cfg::NH; ++hf) {
            constexpr int TTH = Cfg::TTH;
            f32x4 Y[TTH][NT];
#pragma unroll
            for (int tt = 0; tt < TTH; ++tt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) Y[tt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

            if constexpr (Cfg::BF) {
                // K step kk: tiles 2kk, 2kk+1; lane group g holds quads wq0+8kk+g and wq0+8kk+4+g
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
                    const int qa = wq0 + 8 * kk + g, qb = qa + 4;
                    const uint32_t wa = W0[qa], wb = W0[qb];
                    const float4 ca = QC[qa], cb = QC[qb];
                    const bool shared_pair = __all(qd_pair(wa) == qd_pair(wb));
#pragma unroll
                    for (int tt = 0; tt < TTH; ++tt) {
                        const float *row = Qs + (16 * (hf * TTH + tt) + li) * QS;
                        const float pa = row[qd_i1(wa)] * row[qd_i2(wa)];
                        const float pb = shared_pair ? pa : row[qd_i1(wb)] * row[qd_i2(wb)];
                        const float4 xa = *reinterpret_cast<const float4 *>(row + 4 * qd_b(wa));
                        const float4 xb = *reinterpret_cast<const float4 *>(row + 4 * qd_b(wb));
                        float a[8] = {ca.x * xa.x, ca.y * xa.y, ca.z * xa.z, ca.w * xa.w,
                                      cb.x * xb.x, cb.y * xb.y, cb.z * xb.z, cb.w * xb.w};
#pragma unroll
                        for (int j = 0; j < 4; ++j) { a[j] *= pa; a[4 + j] *= pb; }
                        const bf16x8 A = pack_bf16x8(a);
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) Y[tt][nt] = mfma_bf16(A, B[nt], Y[tt][nt]);
                    }
                }
            } else {
                // K step (j, r): lane group g holds slot r of quad wq0 + 4j + g
#pragma unroll
                for (int j = 0; j < MT; ++j) {
                    const int qd = wq0 + 4 * j + g;
                    const uint32_t w = W0[qd];
                    const float4 cq = QC[qd];
                    const float cr[4] = {cq.x, cq.y, cq.z, cq.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
#pragma unroll
                        for (int tt = 0; tt < TTH; ++tt) {
                            const float *row = Qs + (16 * (hf * TTH + tt) + li) * QS;
                            const float a = cr[r] * row[qd_i1(w)] * row[qd_i2(w)] * row[4 * qd_b(w) + r];
#pragma unroll
                            for (int nt = 0; nt < NT; ++nt) Y[tt][nt] = mfma_f32(a, S[j][nt][r], Y[tt][nt]);
                        }
                    }
                }
            }

            for (int oi = 0; oi < ntiles_owned; ++oi) {
                const int qt = slice + oi * nslices;
                if (qt / TTH != hf) continue;
                f32x4 Z[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) Z[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
                intra_tile<Cfg>(Z, qt, wave, g, li, Kt, Qs, lds, ta);
#pragma unroll
                for (int tt = 0; tt < TTH; ++tt)
                    if (hf * TTH + tt == qt) {
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) Y[tt][nt] += Z[nt];
                    }
            }

            f32x4 *Yh = Yr + hf * TTH * NT * 64;
#pragma unroll
            for (int wv = 0; wv < kNW - 1; ++wv) {
                if (wave == wv) {
#pragma unroll
                    for (int tt = 0; tt < TTH; ++tt)
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) {
                            f32x4 *p = Yh + (tt * NT + nt) * 64 + lane;
                            *p = wv == 0 ? Y[tt][nt] : *p + Y[tt][nt];
                        }
                }
                __syncthreads();
            }
            if (wave == kNW - 1) {
                // partial layout per (bh, chunk, slice): [tt][c][16 tokens]; lane writes rows 4g..4g+3
                float *pdst = partial + ((bh * nchunk + cc) * nslices + slice) * (int64_t)(TT * NC * 16);
#pragma unroll
                for (int tt = 0; tt < TTH; ++tt)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        const int c = 16 * nt + li;
                        if (c < NC) {
                            const f32x4 y = Yh[(tt * NT + nt) * 64 + lane] + Y[tt][nt];
                            *reinterpret_cast<f32x4 *>(pdst + ((int64_t)(hf * TTH + tt) * NC + c) * 16 + 4 * g) = y;
                        }
                    }
            }
        }

        // ---- chunk state: S[slice, :] += phi(K_c)[:, slice]^T [V_c | 1]
        if constexpr (Cfg::BF) {
            const bf16_t *Vt = reinterpret_cast<const bf16_t *>(lds + Cfg::OFF_V);
#pragma unroll 1
            for (int ks = 0; ks < C / 32; ++ks) {
                const int tb = 32 * ks + 8 * g;
                bf16x8 B[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    B[nt] = *reinterpret_cast<const bf16x8 *>(Vt + (16 * nt + li) * VS + tb);
                float p2[8];
#pragma unroll
                for (int j = 0; j < MT; ++j) {
                    const uint32_t w = myW[j];
                    if (j == 0 || !((same_prev >> j) & 1u)) {
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
                for (int nt = 0; nt < NT; ++nt) B[nt] = Vt[(16 * nt + li) * VS + tb];
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
        const int64_t qd = qs0 + wq0 + 4 * j + g;
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

// Kernel 2: y = sum over slices of the partials (fixed order), o = y[:d_V] / y[d_V].
// Partial layout per (bh, chunk, slice): [C/16][d_V+1][16 tokens] fp32.
template <int DV, int C, typename TOut>
__global__ __launch_bounds__(256) void prefill_reduce_kernel(const float *__restrict__ partial, int nslices,
                                                             int nchunk, int64_t n, int64_t tok0,
                                                             TOut *__restrict__ out) {
    constexpr int NC = DV + 1, TT = C / 16;
    constexpr int NV = TT * NC * 4;                 // float4 per partial
    constexpr int PER = (NV + 255) / 256;
    __shared__ float ys[TT * NC * 16];
    const int cc = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x;
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
    __syncthreads();
    const int64_t t0 = tok0 + (int64_t)cc * C;
    const int nvalid = n - t0 < C ? (int)(n - t0) : C;
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
    auto red = prefill_reduce_kernel<D, C, TOut>;
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
                               partial, ta);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        {
            ProfScope ps(kProfCombine, stream);
            hipLaunchKernelGGL(red, dim3(nseg, (unsigned)bh), dim3(256), 0, stream, partial, plan.slices, nseg,
                               n, tok0, static_cast<TOut *>(out));
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
