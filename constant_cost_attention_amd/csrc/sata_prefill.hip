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
#include <type_traits>

#ifndef UPDATE_KS_OUTER
#define UPDATE_KS_OUTER 0
#endif

#include "sata_device.h"
#include "sata_internal.h"
#include "sata_scan_common.h"

namespace sata {

constexpr int kNW = 4;                           // wavefronts per workgroup (default)

template <int D, int DV, int C, int MT, int NW, typename TIn>
struct ScanCfg {
    static constexpr bool BF = sizeof(TIn) == 2;
    static constexpr int THREADS = 64 * NW;       // NW wavefronts (4 or 8)
    // Persistent scheduling (see the kernel); one workgroup per item when false.
    static constexpr bool PERSIST = true;
    static constexpr int NP = NW * MT;            // positions (4 quads, 16 features) per slice
    static constexpr int NC = DV + 1;             // value columns + normaliser
    static constexpr int NT = (NC + 15) / 16;     // 16-column MFMA tiles
    static constexpr int TT = C / 16;             // 16-token tiles per chunk
    // Readout work split: TG groups of two token tiles each, and KH = NW / TG halves of the
    // slice's positions; wavefronts w and w + TG read out the same tiles from different halves.
    static constexpr int TPW = 2;                 // readout token tiles per wavefront
    static constexpr int TG = TT / TPW;
    static constexpr int KH = NW / TG;
    static constexpr int NPH = NP / KH;           // readout positions per K half
    static constexpr int KR = D + 4;              // K rows: d_K dims, then 1, 0, 0, 0
    static constexpr int KS = C + 4;              // Kt row stride (floats)
    static constexpr int QS = D + 4;              // Qs row stride (floats): dims, then 1, 0, 0, 0
    static constexpr int ES = BF ? 2 : 4;
    static constexpr int VS = BF ? C + 8 : C + 4; // Vt row stride (elements)
    // Readout operand copy of the slice's state.  bf16: [NP/2 K steps][NT][64 lanes] x 8 bf16;
    // fp32: [4 NP K steps][NT][64 lanes] x 1 float.  Shares its LDS with Kt + Vt (update phase).
    static constexpr int BCB = BF ? NP / 2 * NT * 64 * 16 : NP * 4 * NT * 64 * 4;
    static constexpr int KVB = KR * KS * 4 + (NC * VS * ES + 15) / 16 * 16;
    // Second K half's readout, handed to the first: bf16 (the partials' width) behind Kt + Vt in
    // the shared region; fp32 in a region of its own.
    static constexpr int YEB = (KH - 1) * TG * TPW * NT * 64 * (BF ? 8 : 16);
    static constexpr int XB0 = BF ? KVB + YEB : KVB;
    static constexpr int XB = (BCB > XB0 ? BCB : XB0);
    static constexpr int OFF_VT = KR * KS * 4;
    static constexpr int OFF_Q = (XB + 15) / 16 * 16;    // Qs [C][QS] fp32, scaled by 1/sqrt(d)
    static constexpr int OFF_W = OFF_Q + C * QS * 4;     // quad words [NP][4]
    static constexpr int OFF_QC = OFF_W + NP * 4 * 4;    // quad weights [NP][4] float4
    static constexpr int OFF_F = OFF_QC + NP * 4 * 16;   // position flags [NP]
    static constexpr int OFF_E = BF ? KVB : (OFF_F + NP * 4 + 15) / 16 * 16;   // second K half's readout
    static constexpr int OFF_R = BF ? (OFF_F + NP * 4 + 15) / 16 * 16 : OFF_E + YEB;
    // bf16 inputs: the next chunk's k and v arrive by direct global -> LDS loads into a raw
    // buffer of 1 KB blocks; block s holds 64 consecutive tokens x one 16-byte unit of dims.
    static constexpr bool DMA = BF;
    static constexpr int DB = D / (16 / ES);             // 16-byte units per token
    static constexpr int NSB = C / 64 * DB;              // blocks per tensor
    // The raw buffer is a __shared__ array of its own (RAWB bytes): the compiler can then tell
    // its asynchronous fills from every other LDS access and does not make those wait for them.
    // LDS is the dynamic part (launch argument).
    static constexpr int RAWB = DMA ? 2 * NSB * 1024 : 16;
    static constexpr int LDS = OFF_R;
    // Prefetch of one chunk's q, k or v: 16-byte units per thread.
    static constexpr int EPU = 16 / ES;                  // elements per unit
    static constexpr int UNITS = C * D / EPU;
    static constexpr int UPT = (UNITS + THREADS - 1) / THREADS;
    static_assert(DV == D, "d_V = d_K");
    static_assert(D % EPU == 0, "a unit holds whole dims of one token");
    static_assert(C % 64 == 0 && TG * KH == NW && KH <= 2, "readout split: 64 or 128 tokens per chunk");
    static_assert(!BF || NPH % 2 == 0, "bf16 K steps pair two positions");
    static_assert(NW == 4 || NW == 8, "4 or 8 wavefronts");
    static_assert(OFF_E % 16 == 0 && OFF_R % 16 == 0, "alignment");
    static_assert(OFF_Q % 16 == 0 && OFF_QC % 16 == 0, "alignment");
    static_assert(LDS + RAWB <= 160 * 1024, "LDS budget");
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
                w8[r] = keyA <= query ? taylor_w(sA[r] * ta.scale, ta.c0, ta.c1, ta.c2, ta.c3, ta.c4, ta.P) : 0.f;
                w8[4 + r] = keyB <= query ? taylor_w(sB[r] * ta.scale, ta.c0, ta.c1, ta.c2, ta.c3, ta.c4, ta.P) : 0.f;
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
                const float w = kr <= query ? taylor_w(s[r] * ta.scale, ta.c0, ta.c1, ta.c2, ta.c3, ta.c4, ta.P) : 0.f;
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

// One 16-byte unit of the chunk's q, k or v per (thread, u): token and first dim.
// Consecutive lanes take consecutive tokens, so the transposed (dim-major) LDS
// writes of k and v fall in consecutive banks.
template <int C, int EPU>
__device__ __forceinline__ void unit_coords(int i, int &t, int &d0) {
    t = i % C;
    d0 = (i / C) * EPU;
}

// Unpack one 16-byte unit into fp32.
template <typename TIn>
__device__ __forceinline__ void unpack_unit(const uint4 u, float (&x)[16 / sizeof(TIn)]) {
    if constexpr (sizeof(TIn) == 2) {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = __uint_as_float(w[j] << 16);
            x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        }
    } else {
        x[0] = __uint_as_float(u.x); x[1] = __uint_as_float(u.y);
        x[2] = __uint_as_float(u.z); x[3] = __uint_as_float(u.w);
    }
}

// Readout partials are kept in the input dtype's width: fp32 for fp32 inputs,
// bf16 for bf16 inputs (the operands of the readout are bf16 there already;
// the partials are summed in fp32).
template <typename TIn> struct PartialOf { using type = float; };
template <> struct PartialOf<bf16_t> { using type = bf16_t; };

__device__ __forceinline__ void store4(float *p, f32x4 y) { *reinterpret_cast<f32x4 *>(p) = y; }
__device__ __forceinline__ void store4(bf16_t *p, f32x4 y) {
    *reinterpret_cast<uint2 *>(p) = uint2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
}
__device__ __forceinline__ float4 load4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ float4 load4(const bf16_t *p) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    return float4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                  __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
}

// One 16-byte global -> LDS load per lane: lane i's bytes land at LDS offset lds + 16 i (lds is
// uniform).  Issued from asm so that the compiler does not hold every later LDS read until the
// load has landed (it cannot tell these writes from the update's reads); the consumer waits on
// vmcnt itself before a barrier.  The asm sets M0, which nothing else in these kernels uses.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory");
}
__device__ __forceinline__ uint32_t lds_offset(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

template <int D, int DV, int C, int MT, int NW, typename TIn, bool TRIPLE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void prefill_scan_kernel(const uint32_t *__restrict__ qw0, const int32_t *__restrict__ qcidx,
                         const float4 *__restrict__ qcoef, const uint32_t *__restrict__ qflags,
                         float *__restrict__ state, int64_t m_pad,
                         const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
                         int64_t n, int64_t tok0, int nchunk, typename PartialOf<TIn>::type *__restrict__ partial,
                         float qscale,
                         int nslices, int64_t nbh, int nsub, int sub_chunks, uint32_t *__restrict__ sync,
                         int item_base, int spin_limit, uint32_t *err) {
    using Cfg = ScanCfg<D, DV, C, MT, NW, TIn>;
    constexpr int NC = Cfg::NC, NT = Cfg::NT, TT = Cfg::TT, TPW = Cfg::TPW, NP = Cfg::NP, NPH = Cfg::NPH;
    constexpr int kThreads = Cfg::THREADS;
    constexpr int KS = Cfg::KS, QS = Cfg::QS, VS = Cfg::VS, EPU = Cfg::EPU, UNITS = Cfg::UNITS,
                  UPT = Cfg::UPT;
    extern __shared__ __align__(16) unsigned char lds[];
    float *Kt = reinterpret_cast<float *>(lds);                      // [KR][KS] dim-major (update)
    unsigned char *Vt = lds + Cfg::OFF_VT;                           // [NC][VS] operand dtype (update)
    unsigned char *Bc = lds;                                         // state copy (readout)
    float *Qs = reinterpret_cast<float *>(lds + Cfg::OFF_Q);         // [C][QS]
    uint32_t *W0 = reinterpret_cast<uint32_t *>(lds + Cfg::OFF_W);   // [NP][4]
    float4 *QC = reinterpret_cast<float4 *>(lds + Cfg::OFF_QC);      // [NP][4]
    uint32_t *QF = reinterpret_cast<uint32_t *>(lds + Cfg::OFF_F);   // [NP]
    unsigned char *YE = lds + Cfg::OFF_E;                            // [TG][TPW][NT][64] x 4 values
    __shared__ __align__(16) uint4 raw_lds[Cfg::RAWB / 16];
    uint4 *Raw = raw_lds;                                            // [2][NSB][64] (bf16 inputs)

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches below
    const int g = lane >> 4, li = lane & 15;
    const int p0 = wave * MT;                         // this wave's first position within the slice
    __shared__ int64_t s_item;

    // Work items are (sub-segment u, head bh, slice), u-major.  With a grid of one workgroup per
    // item (nsub = 1) the item is the block index.  Otherwise persistent workgroups take items
    // from a counter; item (u, bh, slice) continues the state left by (u - 1, bh, slice), which
    // was taken earlier by a running workgroup, and its flag (the number of finished
    // sub-segments, released at agent scope) is awaited with a bounded spin.
    const int64_t per_sub = nbh * nslices;
    const int64_t nitems = per_sub * nsub;
    // Thread 0 takes the next item in the same block that releases the finished one (see the
    // warp-specialised scan below for why there is only one such block per pass).
    if constexpr (Cfg::PERSIST) {
        if (tid == 0) s_item = (int64_t)atomicAdd(&sync[0], 1u) + item_base;
        __syncthreads();
    }
    for (int64_t pass = 0;; ++pass) {
    int64_t item;
    if constexpr (Cfg::PERSIST) {
        item = s_item;
        __syncthreads();   // every thread has read the item before thread 0 replaces it
    } else {
        item = pass == 0 ? (int64_t)blockIdx.x : nitems;
    }
    // uniform: every item-derived index and address stays scalar
    item = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(item >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)item));
    if (item >= nitems) break;
    const int u = (int)(item / per_sub);
    const int64_t rem = item % per_sub;
    const int64_t bh = rem / nslices;
    const int slice = (int)(rem % nslices);
    const int cbeg = u * sub_chunks;
    const int cend = cbeg + sub_chunks < nchunk ? cbeg + sub_chunks : nchunk;
    if (Cfg::PERSIST && u > 0) {
        if (tid == 0) wait_predecessor(sync + 1 + rem, (uint32_t)u, spin_limit, err);
        __syncthreads();   // thread 0's acquire invalidated the caches every wave reads through
    }
    const int64_t ps0 = (int64_t)slice * NP;          // first position of the slice
    // Tile j of this wave is position p0 + j (16 features: 4 streams x 4 slots).  Feature rows of
    // a tile: bf16 operands put stream li % 4, slot li / 4 on row li, so that the four lanes of a
    // DPP quad share a slot (one key load feeds all four); fp32 operands put stream li / 4, slot
    // li % 4 there.  The lane's accumulator rows 4g + r are then (stream r, slot g) for bf16 and
    // (stream g, slot r) for fp32.
    auto acc_stream = [&](int r) { return Cfg::BF ? r : g; };
    auto acc_slot = [&](int r) { return Cfg::BF ? g : r; };

    for (int i = tid; i < NP * 4; i += kThreads) {
        W0[i] = qw0[ps0 * 4 + i];
        QC[i] = qcoef[ps0 * 4 + i];
    }
    for (int i = tid; i < NP; i += kThreads) QF[i] = qflags[ps0 + i];

    float *Sh = state + bh * NC * m_pad;
    f32x4 S[MT][NT];
#pragma unroll
    for (int j = 0; j < MT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t qd = (ps0 + p0 + j) * 4 + acc_stream(r);
            const uint32_t w = qw0[qd];
            const int32_t c0 = qcidx[qd];
            const uint32_t mask = qd_mask(w);
            const int z0 = mask ? __builtin_ctz(mask) : 0, z = acc_slot(r);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int c = 16 * nt + li;
                const bool ok = ((mask >> z) & 1u) && c < NC;
                S[j][nt][r] = ok ? Sh[(int64_t)c * m_pad + c0 + (z - z0)] : 0.f;
            }
        }
    __syncthreads();

    // update-side view of this wave's positions: the lane's row li is (stream us, slot uz)
    const int us = Cfg::BF ? (li & 3) : (li >> 2), uz = Cfg::BF ? (li >> 2) : (li & 3);
    uint32_t uw[MT];
    uint32_t newgrp = 0;                               // bit j: position p0 + j starts a pair group
#pragma unroll
    for (int j = 0; j < MT; ++j) {
        uw[j] = W0[(p0 + j) * 4 + us];
        if (QF[p0 + j] & 2u) newgrp |= 1u << j;
    }
    newgrp = (uint32_t)__builtin_amdgcn_readfirstlane((int)newgrp);
    // slice-wide position masks (bit pos): group starts and mixed-weight positions
    static_assert(NP <= 64, "position masks are 64-bit");
    const uint64_t gmask = __ballot(lane < NP && (QF[lane < NP ? lane : 0] & 2u));
    const uint64_t nmask = __ballot(lane < NP && (QF[lane < NP ? lane : 0] & 1u));

    const TIn *qh = q + bh * n * D;
    const TIn *kh = k + bh * n * D;
    const TIn *vh = v + bh * n * DV;
    auto chunk_t0 = [&](int cc) { return tok0 + (int64_t)cc * C; };
    auto chunk_nv = [&](int cc) {
        const int64_t r = n - chunk_t0(cc);
        return r < C ? (int)r : C;
    };

    // ---- chunk staging: global -> registers (issued a phase ahead), registers -> LDS
    auto gload = [&](uint4 (&r)[UPT], const TIn *src, int cc) {
        const int64_t t0 = chunk_t0(cc);
        const int nv = chunk_nv(cc);
#pragma unroll
        for (int u = 0; u < UPT; ++u) {
            const int i = tid + u * kThreads;
            int t, d0;
            unit_coords<C, EPU>(i, t, d0);
            r[u] = uint4{0u, 0u, 0u, 0u};
            if (i < UNITS && t < nv) r[u] = *reinterpret_cast<const uint4 *>(src + (t0 + t) * D + d0);
        }
    };
    auto write_q = [&](const uint4 (&r)[UPT]) {     // Qs <- q / sqrt(d), row-major; invalid tokens are 0
#pragma unroll
        for (int u = 0; u < UPT; ++u) {
            const int i = tid + u * kThreads;
            if (i >= UNITS) break;
            int t, d0;
            unit_coords<C, EPU>(i, t, d0);
            float x[EPU];
            unpack_unit<TIn>(r[u], x);
#pragma unroll
            for (int e = 0; e < EPU; e += 4)
                *reinterpret_cast<float4 *>(Qs + t * QS + d0 + e) =
                    float4{x[e] * qscale, x[e + 1] * qscale, x[e + 2] * qscale, x[e + 3] * qscale};
        }
        for (int t = tid; t < C; t += kThreads) *reinterpret_cast<float4 *>(Qs + t * QS + D) = float4{1.f, 0.f, 0.f, 0.f};
    };
    auto write_kv = [&](const uint4 (&rk)[UPT], const uint4 (&rv)[UPT], int nv) {   // Kt, Vt dim-major
#pragma unroll
        for (int u = 0; u < UPT; ++u) {
            const int i = tid + u * kThreads;
            if (i >= UNITS) break;
            int t, d0;
            unit_coords<C, EPU>(i, t, d0);
            float x[EPU];
            unpack_unit<TIn>(rk[u], x);
#pragma unroll
            for (int e = 0; e < EPU; ++e) Kt[(d0 + e) * KS + t] = x[e];
            if constexpr (Cfg::BF) {
                const uint32_t w[4] = {rv[u].x, rv[u].y, rv[u].z, rv[u].w};
                uint16_t *V16 = reinterpret_cast<uint16_t *>(Vt);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    V16[(d0 + 2 * e) * VS + t] = (uint16_t)(w[e] & 0xffffu);
                    V16[(d0 + 2 * e + 1) * VS + t] = (uint16_t)(w[e] >> 16);
                }
            } else {
                unpack_unit<TIn>(rv[u], x);
#pragma unroll
                for (int e = 0; e < EPU; ++e) reinterpret_cast<float *>(Vt)[(d0 + e) * VS + t] = x[e];
            }
        }
        for (int t = tid; t < C; t += kThreads) {
            Kt[D * KS + t] = 1.f;
            Kt[(D + 1) * KS + t] = 0.f; Kt[(D + 2) * KS + t] = 0.f; Kt[(D + 3) * KS + t] = 0.f;
            if constexpr (Cfg::BF) reinterpret_cast<bf16_t *>(Vt)[DV * VS + t] = from_f32<bf16_t>(t < nv ? 1.f : 0.f);
            else reinterpret_cast<float *>(Vt)[DV * VS + t] = t < nv ? 1.f : 0.f;
        }
    };
    // bf16: issue the chunk's k and v as direct global -> LDS loads (no registers held); lanes
    // of block s take 64 consecutive tokens, so the later transposing read is conflict-free.
    auto dma_kv = [&](int cc) {
        if constexpr (Cfg::DMA) {
            constexpr int DB = Cfg::DB, NSB = Cfg::NSB;
            const int64_t t0 = chunk_t0(cc);
            const int nv = chunk_nv(cc);
            for (int sb = wave; sb < NSB; sb += NW) {
                const int t = (sb / DB) * 64 + lane;
                const int d0 = (sb % DB) * EPU;
                if (t < nv) {
                    dma16(kh + (t0 + t) * D + d0, lds_offset(Raw + sb * 64));
                    dma16(vh + (t0 + t) * D + d0, lds_offset(Raw + (NSB + sb) * 64));
                }
            }
        }
    };
    auto write_kv_raw = [&](int nv) {               // raw blocks -> Kt (fp32), Vt (bf16), dim-major
        if constexpr (Cfg::DMA) {
            constexpr int DB = Cfg::DB, NSB = Cfg::NSB;
            uint16_t *V16 = reinterpret_cast<uint16_t *>(Vt);
            for (int i = tid; i < NSB * 64; i += kThreads) {
                const int sb = i / 64, t = (sb / DB) * 64 + (i % 64), d0 = (sb % DB) * EPU;
                const bool ok = t < nv;
                const uint4 uk = ok ? Raw[i] : uint4{0u, 0u, 0u, 0u};
                const uint4 uv = ok ? Raw[NSB * 64 + i] : uint4{0u, 0u, 0u, 0u};
                float x[EPU];
                unpack_unit<TIn>(uk, x);
#pragma unroll
                for (int e = 0; e < EPU; ++e) Kt[(d0 + e) * KS + t] = x[e];
                const uint32_t w[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    V16[(d0 + 2 * e) * VS + t] = (uint16_t)(w[e] & 0xffffu);
                    V16[(d0 + 2 * e + 1) * VS + t] = (uint16_t)(w[e] >> 16);
                }
            }
            for (int t = tid; t < C; t += kThreads) {
                Kt[D * KS + t] = 1.f;
                Kt[(D + 1) * KS + t] = 0.f; Kt[(D + 2) * KS + t] = 0.f; Kt[(D + 3) * KS + t] = 0.f;
                reinterpret_cast<bf16_t *>(Vt)[DV * VS + t] = from_f32<bf16_t>(t < nv ? 1.f : 0.f);
            }
        }
    };
    // state accumulators -> readout operand copy in LDS (this wave's positions).  The copy
    // carries the slot weight relative to the pair weight: 1 except at a group's first position
    // (diagonal and invalid slots), so the readout forms every position alike.
    auto slot_ratio = [&](int p, float (&r4)[4]) {   // for the lane's accumulator rows r
        const float *qcf = reinterpret_cast<const float *>(QC);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int st = acc_stream(r);
            const uint32_t w = W0[p * 4 + st];
            const float rinv = qd_pfact<D, TRIPLE>(w);
            r4[r] = qcf[(p * 4 + st) * 4 + acc_slot(r)] * rinv;
        }
    };
    auto write_bcopy = [&]() {
        // plain copies of every position, then the wave's mixed-weight positions (uniform
        // branches) written again, rescaled; LDS keeps a wave's order, so the second write wins
        const uint32_t mixed = (uint32_t)((nmask >> p0) & ((1ull << MT) - 1));
        if constexpr (Cfg::BF) {
            // position p, streams 2 h2 and 2 h2 + 1 of slot g: K step p / 2, reader lane group
            // 2 (p % 2) + h2, elements 2 g and 2 g + 1
            uint32_t *B4 = reinterpret_cast<uint32_t *>(Bc);
            auto entry = [&](int p, int nt, int h2) {   // index into B4
                const int kk = p >> 1, gr = 2 * (p & 1) + h2;
                return ((kk * NT + nt) * 64 + gr * 16 + li) * 4 + g;
            };
#pragma unroll
            for (int j = 0; j < MT; ++j)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    B4[entry(p0 + j, nt, 0)] = pack_bf16x2(S[j][nt][0], S[j][nt][1]);
                    B4[entry(p0 + j, nt, 1)] = pack_bf16x2(S[j][nt][2], S[j][nt][3]);
                }
#pragma unroll
            for (int j = 0; j < MT; ++j) {
                if ((mixed >> j) & 1u) {
                    float r4[4];
                    slot_ratio(p0 + j, r4);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        B4[entry(p0 + j, nt, 0)] = pack_bf16x2(S[j][nt][0] * r4[0], S[j][nt][1] * r4[1]);
                        B4[entry(p0 + j, nt, 1)] = pack_bf16x2(S[j][nt][2] * r4[2], S[j][nt][3] * r4[3]);
                    }
                }
            }
        } else {
            float *Bf = reinterpret_cast<float *>(Bc);
#pragma unroll
            for (int j = 0; j < MT; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) Bf[(((p0 + j) * 4 + r) * NT + nt) * 64 + lane] = S[j][nt][r];
            for (uint32_t mm = mixed; mm; mm &= mm - 1) {
                const int p = p0 + __builtin_ctz(mm);
                float r4[4];
                slot_ratio(p, r4);
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) Bf[((p * 4 + r) * NT + nt) * 64 + lane] *= r4[r];
            }
        }
    };

    uint4 rk[Cfg::DMA ? 1 : UPT], rv[Cfg::DMA ? 1 : UPT], rq[UPT];
    if (cbeg < cend) {
        if constexpr (Cfg::DMA) {
            dma_kv(cbeg);
        } else {
            gload(rk, kh, cbeg);
            gload(rv, vh, cbeg);
        }
        gload(rq, qh, cbeg);
        write_q(rq);
        if (cbeg + 1 < cend) gload(rq, qh, cbeg + 1);
    }
    write_bcopy();
    __syncthreads();

    constexpr int TG = Cfg::TG;
    const int tt0 = (wave % TG) * TPW;                // this wave's readout token tiles
    const int half = wave / TG;                       // and K half: positions [half * NPH, (half + 1) * NPH)
    const int pbeg = half * NPH;
    for (int cc = cbeg; cc < cend; ++cc) {
        // ---- inter-chunk readout Y = psi(Q_c)[:, slice] . S^(c-1)[slice, :] for this wave's tiles,
        //      over its half of the slice's positions (state operand from LDS)
        f32x4 Y[TPW][NT];
        {
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) Y[tt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const float *qrow[TPW];
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) qrow[tt] = Qs + (16 * (tt0 + tt) + li) * QS;
            if constexpr (Cfg::BF) {
                // K step kk covers positions 2 kk and 2 kk + 1.  Lane group g takes position
                // 2 kk + g / 2, streams 2 (g % 2) + sl (sl = 0, 1) and slots z = 0..3 as elements
                // 2 z + sl: one 16-byte q load per token tile and two pair products.  Within a pair group the block advances by
                // one per position; the pair products and block are re-read from the quad table only
                // where a group starts (a uniform test: the lanes' positions see a start in the
                // three positions ending at 2 kk + 1).
                static_assert((NPH / 2) % 2 == 0, "an even number of K steps per wavefront");
                const bf16x8 *Bv = reinterpret_cast<const bf16x8 *>(Bc);
                const int hh = g >> 1, sp = 2 * (g & 1);
                const int kbeg = pbeg / 2, kend = (pbeg + NPH) / 2;
                float pc[TPW][2];
                int xo = 0;
                auto regroup = [&](int kk) {
                    const uint2 w2 = *reinterpret_cast<const uint2 *>(W0 + (2 * kk + hh) * 4 + sp);
                    const int i1a = qd_i1(w2.x), i2a = qd_i2(w2.x), i1b = qd_i1(w2.y), i2b = qd_i2(w2.y);
                    const float ca = qd_pweight<D, TRIPLE>(w2.x);
                    const float cb = qd_pweight<D, TRIPLE>(w2.y);
#pragma unroll
                    for (int tt = 0; tt < TPW; ++tt) {
                        pc[tt][0] = ca * qrow[tt][i1a] * qrow[tt][i2a];
                        pc[tt][1] = cb * qrow[tt][i1b] * qrow[tt][i2b];
                    }
                    if constexpr (TRIPLE) {
                        const int i0a = qd_i0(w2.x), i0b = qd_i0(w2.y);
#pragma unroll
                        for (int tt = 0; tt < TPW; ++tt) {
                            pc[tt][0] *= qrow[tt][i0a];
                            pc[tt][1] *= qrow[tt][i0b];
                        }
                    }
                    xo = 4 * qd_b(w2.x);
                };
                auto advance = [&](int kk) {         // the lanes' positions move from 2 kk - 2 + hh
                    if (((gmask >> (2 * kk - 1)) & 7u) != 0) {
                        __asm__ volatile("" ::: "memory");
                        regroup(kk);
                    } else {
                        xo += 8;
                    }
                };
                auto load_b = [&](bf16x8 (&B)[NT], int kk) {
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) B[nt] = Bv[(kk * NT + nt) * 64 + lane];
                };
                auto form = [&](bf16x8 (&A)[TPW]) {
#pragma unroll
                    for (int tt = 0; tt < TPW; ++tt) {
                        const float4 x = *reinterpret_cast<const float4 *>(qrow[tt] + xo);
                        const float a[8] = {pc[tt][0] * x.x, pc[tt][1] * x.x, pc[tt][0] * x.y, pc[tt][1] * x.y,
                                            pc[tt][0] * x.z, pc[tt][1] * x.z, pc[tt][0] * x.w, pc[tt][1] * x.w};
                        A[tt] = pack_bf16x8(a);
                    }
                };
                auto mma = [&](const bf16x8 (&A)[TPW], const bf16x8 (&B)[NT]) {
#pragma unroll
                    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) Y[tt][nt] = mfma_bf16(A[tt], B[nt], Y[tt][nt]);
                };
                if constexpr (NW == 8) {
                    // two wavefronts per SIMD hide each other's latency: one operand set; the first
                    // step starts the accumulators from zero
                    regroup(kbeg);
                    {
                        bf16x8 A[TPW], B[NT];
                        load_b(B, kbeg);
                        form(A);
#pragma unroll
                        for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
                            for (int nt = 0; nt < NT; ++nt) Y[tt][nt] = mfma_bf16(A[tt], B[nt], f32x4{0.f, 0.f, 0.f, 0.f});
                    }
#pragma unroll 1
                    for (int kk = kbeg + 1; kk < kend; ++kk) {
                        advance(kk);
                        bf16x8 A[TPW], B[NT];
                        load_b(B, kk);
                        form(A);
                        mma(A, B);
                    }
                } else {
                // two operand sets in turn: step kk's products run while step kk + 1's are formed
                bf16x8 A0[TPW], B0[NT], A1[TPW], B1[NT];
                regroup(kbeg);
                load_b(B0, kbeg);
                form(A0);
#pragma unroll 1
                for (int kk = kbeg; kk + 2 < kend; kk += 2) {
                    advance(kk + 1);
                    load_b(B1, kk + 1);
                    form(A1);
                    mma(A0, B0);
                    advance(kk + 2);
                    load_b(B0, kk + 2);
                    form(A0);
                    mma(A1, B1);
                }
                advance(kend - 1);
                load_b(B1, kend - 1);
                form(A1);
                mma(A0, B0);
                mma(A1, B1);
                }
            } else {
                float pcur[TPW];                      // pair weight * q_i1 * q_i2 of stream g
                int xo = 0;                           // 4 b: the position's block of q
                const float *Bf = reinterpret_cast<const float *>(Bc);
#pragma unroll 1
                for (int pos = pbeg; pos < pbeg + NPH; ++pos) {
                    if (((gmask >> pos) & 1u) || pos == pbeg) {
                        const uint32_t w = W0[pos * 4 + g];
                        const int i1 = qd_i1(w), i2 = qd_i2(w);
                        const float cp = qd_pweight<D, TRIPLE>(w);
#pragma unroll
                        for (int tt = 0; tt < TPW; ++tt) pcur[tt] = cp * qrow[tt][i1] * qrow[tt][i2];
                        if constexpr (TRIPLE) {
                            const int i0 = qd_i0(w);
#pragma unroll
                            for (int tt = 0; tt < TPW; ++tt) pcur[tt] *= qrow[tt][i0];
                        }
                        xo = 4 * qd_b(w);
                    } else {
                        xo += 4;
                    }
                    float a[TPW][4];
#pragma unroll
                    for (int tt = 0; tt < TPW; ++tt) {
                        const float4 x = *reinterpret_cast<const float4 *>(qrow[tt] + xo);
                        a[tt][0] = pcur[tt] * x.x; a[tt][1] = pcur[tt] * x.y;
                        a[tt][2] = pcur[tt] * x.z; a[tt][3] = pcur[tt] * x.w;
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float B[NT];
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) B[nt] = Bf[((pos * 4 + r) * NT + nt) * 64 + lane];
#pragma unroll
                        for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
                            for (int nt = 0; nt < NT; ++nt) Y[tt][nt] = mfma_f32(a[tt][r], B[nt], Y[tt][nt]);
                    }
                }
            }
        }
        if constexpr (Cfg::DMA) __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this chunk's k, v in LDS
        __syncthreads();                              // state copy and Qs no longer read
        // second K half: hand the readout to the first (bf16 inputs: in bf16, behind Kt + Vt)
        auto ye_index = [&](int tt, int nt) { return (((wave % TG) * TPW + tt) * NT + nt) * 64 + lane; };
        if (Cfg::KH > 1 && half > 0) {
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    if constexpr (Cfg::BF)
                        reinterpret_cast<uint2 *>(YE)[ye_index(tt, nt)] =
                            uint2{pack_bf16x2(Y[tt][nt][0], Y[tt][nt][1]), pack_bf16x2(Y[tt][nt][2], Y[tt][nt][3])};
                    else
                        reinterpret_cast<f32x4 *>(YE)[ye_index(tt, nt)] = Y[tt][nt];
                }
        }
        if constexpr (Cfg::DMA) write_kv_raw(chunk_nv(cc));
        else write_kv(rk, rv, chunk_nv(cc));
        if (cc + 1 < cend) write_q(rq);
        __syncthreads();                              // exchange written
        if (half == 0) {
            // partial layout per (bh, chunk, slice): [TT][NC][16 tokens]; lane writes rows 4g..4g+3
            // one lane address per chunk; the tiles are constant offsets from it
            auto *pdst = partial + ((bh * nchunk + cc) * nslices + slice) * (int64_t)(TT * NC * 16) +
                         (int64_t)tt0 * NC * 16 + (li * 16 + 4 * g);
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    f32x4 y = Y[tt][nt];
                    if constexpr (Cfg::KH > 1) {
                        if constexpr (Cfg::BF) {
                            const uint2 h = reinterpret_cast<const uint2 *>(YE)[ye_index(tt, nt)];
                            y[0] += __uint_as_float(h.x << 16); y[1] += __uint_as_float(h.x & 0xffff0000u);
                            y[2] += __uint_as_float(h.y << 16); y[3] += __uint_as_float(h.y & 0xffff0000u);
                        } else {
                            y += reinterpret_cast<const f32x4 *>(YE)[ye_index(tt, nt)];
                        }
                    }
                    const int c = 16 * nt + li;
                    if (c < NC) store4(pdst + (tt * NC + 16 * nt) * 16, y);
                }
        }
        if (cc + 1 < cend) {                          // next chunk's k, v: in flight during the update
            if constexpr (Cfg::DMA) {
                dma_kv(cc + 1);
            } else {
                gload(rk, kh, cc + 1);
                gload(rv, vh, cc + 1);
            }
        }

        // ---- chunk state: S[slice, :] += phi(K_c)[:, slice]^T [V_c | 1]
        if constexpr (Cfg::BF && (NW == 8 || UPDATE_KS_OUTER)) {
            // The chunk's 32-token K steps outer, positions inner (smaller register footprint): one
            // [V | 1] operand set at a time, the next K step's loaded during this one; the pair
            // products are re-formed at each K step's first position and at group starts.  Key
            // values of the last index come by DPP quad broadcast, as below.
            constexpr int NKS = C / 32;
            const bf16_t *V16 = reinterpret_cast<const bf16_t *>(Vt);
            auto load_v = [&](bf16x8 (&B)[NT], int ks) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    uint4 u = {0u, 0u, 0u, 0u};
                    if (16 * nt + li < NC) u = *reinterpret_cast<const uint4 *>(V16 + (16 * nt + li) * VS + 32 * ks + 8 * g);
                    B[nt] = __builtin_bit_cast(bf16x8, u);
                }
            };
            auto load_k3 = [&](int j, int ks) {
                return *reinterpret_cast<const float2 *>(Kt + (4 * qd_b(uw[j]) + uz) * KS + 32 * ks + 8 * g + 2 * us);
            };
            auto step = [&](const bf16x8 (&B)[NT], int ks) {
                const int tb = 32 * ks + 8 * g;
                float p2[8];
                float2 kc = load_k3(0, ks);
#pragma unroll
                for (int j = 0; j < MT; ++j) {
                    const uint32_t w = uw[j];
                    if (j == 0 || ((newgrp >> j) & 1u)) {
                        __asm__ volatile("" ::: "memory");   // keep the reload behind its (uniform) branch
                        const float4 *k1 = reinterpret_cast<const float4 *>(Kt + qd_i1(w) * KS + tb);
                        const float4 *k2 = reinterpret_cast<const float4 *>(Kt + qd_i2(w) * KS + tb);
                        const float4 a0 = k1[0], a1 = k1[1], b0 = k2[0], b1 = k2[1];
                        p2[0] = a0.x * b0.x; p2[1] = a0.y * b0.y; p2[2] = a0.z * b0.z; p2[3] = a0.w * b0.w;
                        p2[4] = a1.x * b1.x; p2[5] = a1.y * b1.y; p2[6] = a1.z * b1.z; p2[7] = a1.w * b1.w;
                        if constexpr (TRIPLE) {
                            const float4 *k0 = reinterpret_cast<const float4 *>(Kt + qd_i0(w) * KS + tb);
                            const float4 c0 = k0[0], c1 = k0[1];
                            p2[0] *= c0.x; p2[1] *= c0.y; p2[2] *= c0.z; p2[3] *= c0.w;
                            p2[4] *= c1.x; p2[5] *= c1.y; p2[6] *= c1.z; p2[7] *= c1.w;
                        }
                    }
                    float2 kn = kc;
                    if (j + 1 < MT) kn = load_k3(j + 1, ks);
                    const float x = kc.x, y = kc.y;
                    float a[8] = {p2[0] * quad_bcast<0>(x), p2[1] * quad_bcast<0>(y),
                                  p2[2] * quad_bcast<1>(x), p2[3] * quad_bcast<1>(y),
                                  p2[4] * quad_bcast<2>(x), p2[5] * quad_bcast<2>(y),
                                  p2[6] * quad_bcast<3>(x), p2[7] * quad_bcast<3>(y)};
                    const bf16x8 A = pack_bf16x8(a);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) S[j][nt] = mfma_bf16(A, B[nt], S[j][nt]);
                    kc = kn;
                }
            };
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                bf16x8 B[NT];
                load_v(B, ks);
                step(B, ks);
            }
        } else if constexpr (Cfg::BF) {
            // Positions outer, the chunk's 32-token K steps inner: the [V | 1] operand tiles of the
            // whole chunk stay in registers, and the pair products (per K step) are formed only where
            // a pair group starts (the same positions for all four streams).  The last-index key
            // values of a K step: each lane of a DPP quad (one slot, four streams) loads two of the
            // eight tokens, and the products take all eight by quad broadcast.  The next position's
            // key values are loaded while this position's products run.
            constexpr int NKS = C / 32;
            const bf16_t *V16 = reinterpret_cast<const bf16_t *>(Vt);
            bf16x8 B[NKS][NT];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    uint4 u = {0u, 0u, 0u, 0u};
                    if (16 * nt + li < NC) u = *reinterpret_cast<const uint4 *>(V16 + (16 * nt + li) * VS + 32 * ks + 8 * g);
                    B[ks][nt] = __builtin_bit_cast(bf16x8, u);
                }
            auto load_k3 = [&](float2 (&kd)[NKS], int j) {
                const float *k3 = Kt + (4 * qd_b(uw[j]) + uz) * KS + 8 * g + 2 * us;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) kd[ks] = *reinterpret_cast<const float2 *>(k3 + 32 * ks);
            };
            float p2[NKS][8];
            float2 kc[NKS];
            load_k3(kc, 0);
#pragma unroll
            for (int j = 0; j < MT; ++j) {
                const uint32_t w = uw[j];
                if (j == 0 || ((newgrp >> j) & 1u)) {
                    __asm__ volatile("" ::: "memory");   // keep the reload behind its (uniform) branch
                    const float *k1 = Kt + qd_i1(w) * KS + 8 * g;
                    const float *k2 = Kt + qd_i2(w) * KS + 8 * g;
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        const float4 a0 = *reinterpret_cast<const float4 *>(k1 + 32 * ks);
                        const float4 a1 = *reinterpret_cast<const float4 *>(k1 + 32 * ks + 4);
                        const float4 b0 = *reinterpret_cast<const float4 *>(k2 + 32 * ks);
                        const float4 b1 = *reinterpret_cast<const float4 *>(k2 + 32 * ks + 4);
                        p2[ks][0] = a0.x * b0.x; p2[ks][1] = a0.y * b0.y; p2[ks][2] = a0.z * b0.z; p2[ks][3] = a0.w * b0.w;
                        p2[ks][4] = a1.x * b1.x; p2[ks][5] = a1.y * b1.y; p2[ks][6] = a1.z * b1.z; p2[ks][7] = a1.w * b1.w;
                    }
                    if constexpr (TRIPLE) {
                        const float *k0 = Kt + qd_i0(w) * KS + 8 * g;
#pragma unroll
                        for (int ks = 0; ks < NKS; ++ks) {
                            const float4 c0 = *reinterpret_cast<const float4 *>(k0 + 32 * ks);
                            const float4 c1 = *reinterpret_cast<const float4 *>(k0 + 32 * ks + 4);
                            p2[ks][0] *= c0.x; p2[ks][1] *= c0.y; p2[ks][2] *= c0.z; p2[ks][3] *= c0.w;
                            p2[ks][4] *= c1.x; p2[ks][5] *= c1.y; p2[ks][6] *= c1.z; p2[ks][7] *= c1.w;
                        }
                    }
                }
                float2 kn[NKS];
                if (j + 1 < MT) load_k3(kn, j + 1);
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const float x = kc[ks].x, y = kc[ks].y;
                    float a[8] = {p2[ks][0] * quad_bcast<0>(x), p2[ks][1] * quad_bcast<0>(y),
                                  p2[ks][2] * quad_bcast<1>(x), p2[ks][3] * quad_bcast<1>(y),
                                  p2[ks][4] * quad_bcast<2>(x), p2[ks][5] * quad_bcast<2>(y),
                                  p2[ks][6] * quad_bcast<3>(x), p2[ks][7] * quad_bcast<3>(y)};
                    const bf16x8 A = pack_bf16x8(a);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) S[j][nt] = mfma_bf16(A, B[ks][nt], S[j][nt]);
                }
                if (j + 1 < MT) {
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) kc[ks] = kn[ks];
                }
            }
        } else {
            const float *Vf = reinterpret_cast<const float *>(Vt);
#pragma unroll 1
            for (int ks = 0; ks < C / 4; ++ks) {
                const int tb = 4 * ks + g;
                float B[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) B[nt] = 16 * nt + li < NC ? Vf[(16 * nt + li) * VS + tb] : 0.f;
#pragma unroll
                for (int j = 0; j < MT; ++j) {
                    const uint32_t w = uw[j];
                    float a = Kt[qd_i1(w) * KS + tb] * Kt[qd_i2(w) * KS + tb] * Kt[(4 * qd_b(w) + uz) * KS + tb];
                    if constexpr (TRIPLE) a *= Kt[qd_i0(w) * KS + tb];
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) S[j][nt] = mfma_f32(a, B[nt], S[j][nt]);
                }
            }
        }
        __syncthreads();                              // Kt, Vt no longer read
        write_bcopy();
        if (cc + 2 < cend) gload(rq, qh, cc + 2);     // the chunk after next's q: in flight during the readout
        __syncthreads();
    }

    // accumulators -> state slice
#pragma unroll
    for (int j = 0; j < MT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t qd = (ps0 + p0 + j) * 4 + acc_stream(r);
            const uint32_t w = qw0[qd];
            const int32_t c0 = qcidx[qd];
            const uint32_t mask = qd_mask(w);
            const int z0 = mask ? __builtin_ctz(mask) : 0, z = acc_slot(r);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int c = 16 * nt + li;
                if (((mask >> z) & 1u) && c < NC) Sh[(int64_t)c * m_pad + c0 + (z - z0)] = S[j][nt][r];
            }
        }
    if constexpr (Cfg::PERSIST) {
        // every wave's state stores reach L2 before the barrier; thread 0's agent-scope release
        // then writes L2 back before the flag
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
        __syncthreads();
        if (tid == 0) {
            __hip_atomic_store(&sync[1 + rem], (uint32_t)(u + 1), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            s_item = (int64_t)atomicAdd(&sync[0], 1u) + item_base;
        }
        __syncthreads();
    }
    }
}

// ---------------------------------------------------------------------------------------------
// Warp-specialised scan (bf16 inputs).  Eight wavefronts, two per SIMD: four "update"
// wavefronts keep the slice's state in their registers (MT positions each) and form the chunk
// state contraction; four "readout" wavefronts read the chunk out against the state copy in LDS
// (TPW token tiles each, every position of the slice) and stage the next chunk through their
// registers.  Readout and update of a chunk touch disjoint data (the state copy holds
// S^(c-1), the registers turn into S^(c)), so the two run at the same time on every SIMD; the
// second phase of a chunk writes the new state copy (update wavefronts) and the readout
// partials plus the next chunk's q, k and v (readout wavefronts).  Two barriers per chunk.
template <int D, int DV, int C, int MT>
struct WsCfg {
    static constexpr int NR = 4, NU = 4, NW = NR + NU, THREADS = 64 * NW;
    static constexpr int NP = NU * MT;            // positions per slice
    static constexpr int NS = NP / 2;             // readout K steps
    static constexpr int NC = DV + 1, NT = (NC + 15) / 16;
    static constexpr int TT = C / 16, TPW = TT / NR;
    static constexpr int KR = D + 4, KS = C + 4, QS = D + 4, VS = C + 8;
    // State copy: the NT - 1 full column tiles [NS][NT-1][64 lanes] x 16 B, then the last tile.
    // When the last tile holds only the normaliser column, just its lanes 16 g are kept:
    // [NS][4] x 16 B; otherwise [NS][64] x 16 B.
    static constexpr int LC = NC - 16 * (NT - 1);          // real columns of the last tile
    static constexpr int LASTW = LC == 1 ? 4 : 64;
    static constexpr int FULLB = NS * (NT - 1) * 64 * 16;
    static constexpr int BCB = FULLB + NS * LASTW * 16;
    static constexpr int OFF_K = (BCB + 15) / 16 * 16;     // Kt fp32 [KR][KS], dim-major
    static constexpr int OFF_V = OFF_K + KR * KS * 4;      // Vt bf16 [NC][VS], dim-major
    static constexpr int OFF_Q = OFF_V + (NC * VS * 2 + 15) / 16 * 16;   // Qs fp32 [C][QS]
    static constexpr int OFF_W = OFF_Q + C * QS * 4;       // quad words [NP][4]
    static constexpr int OFF_QC = OFF_W + NP * 16;         // quad weights [NP][4] float4
    static constexpr int OFF_F = OFF_QC + NP * 64;         // position flags [NP]
    static constexpr int LDS = OFF_F + NP * 4;
    static constexpr int EPU = 8;                          // bf16 values per 16-byte unit
    static constexpr int UNITS = C * D / EPU;              // units per tensor and chunk
    static constexpr int UPT = (UNITS + 64 * NR - 1) / (64 * NR);
    static_assert(DV == D, "d_V = d_K");
    static_assert(C % 64 == 0 && TT % NR == 0, "64 or 128 tokens per chunk");
    static_assert(NS % 2 == 0, "an even number of readout K steps");
    static_assert(NP <= 64 && (NP & (NP - 1)) == 0, "position masks are 64-bit");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <int D, int DV, int C, int MT, bool TRIPLE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_scan_ws_kernel(const uint32_t *__restrict__ qw0, const int32_t *__restrict__ qcidx,
                            const float4 *__restrict__ qcoef, const uint32_t *__restrict__ qflags,
                            float *__restrict__ state, int64_t m_pad,
                            const bf16_t *__restrict__ q, const bf16_t *__restrict__ k, const bf16_t *__restrict__ v,
                            int64_t n, int64_t tok0, int nchunk, bf16_t *__restrict__ partial, float qscale,
                            int nslices, int64_t nbh, int nsub, int sub_chunks, uint32_t *__restrict__ sync,
                            int item_base, int spin_limit, uint32_t *err) {
    using Cfg = WsCfg<D, DV, C, MT>;
    constexpr int NC = Cfg::NC, NT = Cfg::NT, TT = Cfg::TT, TPW = Cfg::TPW, NP = Cfg::NP, NS = Cfg::NS;
    constexpr int KS = Cfg::KS, QS = Cfg::QS, VS = Cfg::VS, EPU = Cfg::EPU, UNITS = Cfg::UNITS, UPT = Cfg::UPT;
    constexpr int LASTW = Cfg::LASTW;
    extern __shared__ __align__(16) unsigned char lds[];
    unsigned char *Bc = lds;
    float *Kt = reinterpret_cast<float *>(lds + Cfg::OFF_K);
    uint16_t *Vt = reinterpret_cast<uint16_t *>(lds + Cfg::OFF_V);
    float *Qs = reinterpret_cast<float *>(lds + Cfg::OFF_Q);
    uint32_t *W0 = reinterpret_cast<uint32_t *>(lds + Cfg::OFF_W);
    float4 *QC = reinterpret_cast<float4 *>(lds + Cfg::OFF_QC);
    uint32_t *QF = reinterpret_cast<uint32_t *>(lds + Cfg::OFF_F);
    __shared__ int64_t s_item;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool reader = wave < Cfg::NR;
    const int g = lane >> 4, li = lane & 15;
    const int64_t per_sub = nbh * nslices;
    const int64_t nitems = per_sub * nsub;

    // One thread-0 block per pass, at its end, both releases the finished item and takes the
    // next.  With a second thread-0 block at the top of the loop the compiler may thread one
    // branch into the other; the loop it then builds runs its barriers without thread 0, and
    // the other threads re-read an item that never changes.
    if (tid == 0) s_item = (int64_t)atomicAdd(&sync[0], 1u) + item_base;
    __syncthreads();
    for (;;) {
        int64_t item = s_item;
        __syncthreads();   // every thread has read the item before thread 0 replaces it
        item = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(item >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((int)item));
        if (item >= nitems) break;
        const int u = (int)(item / per_sub);
        const int64_t rem = item % per_sub;
        const int64_t bh = rem / nslices;
        const int slice = (int)(rem % nslices);
        const int cbeg = u * sub_chunks;
        const int cend = cbeg + sub_chunks < nchunk ? cbeg + sub_chunks : nchunk;
        if (u > 0) {   // the state of (u - 1, bh, slice) must have landed
            if (tid == 0) wait_predecessor(sync + 1 + rem, (uint32_t)u, spin_limit, err);
            __syncthreads();
        }
        const int64_t ps0 = (int64_t)slice * NP;
        for (int i = tid; i < NP * 4; i += Cfg::THREADS) {
            W0[i] = qw0[ps0 * 4 + i];
            QC[i] = qcoef[ps0 * 4 + i];
        }
        for (int i = tid; i < NP; i += Cfg::THREADS) QF[i] = qflags[ps0 + i];
        __syncthreads();
        const uint64_t gmask = __ballot(lane < NP && (QF[lane < NP ? lane : 0] & 2u));
        const uint64_t nmask = __ballot(lane < NP && (QF[lane < NP ? lane : 0] & 1u));
        const bf16_t *qh = q + bh * n * D;
        const bf16_t *kh = k + bh * n * D;
        const bf16_t *vh = v + bh * n * DV;
        auto chunk_t0 = [&](int cc) { return tok0 + (int64_t)cc * C; };
        auto chunk_nv = [&](int cc) {
            const int64_t r = n - chunk_t0(cc);
            return r < C ? (int)r : C;
        };

        if (reader) {
            // ------------------------------------------------ readout wavefronts
            const int rtid = tid;                       // 0 .. 255
            uint4 rq[UPT], rk[UPT], rv[UPT];
            // thread rtid's units: token rtid % C, dims (rtid / C) EPU + uu DU (a thread's units
            // share the token, as 64 NR is a multiple of C)
            static_assert((64 * Cfg::NR) % C == 0, "units of a thread share their token");
            constexpr int DU = (64 * Cfg::NR / C) * EPU;
            auto gload = [&](uint4 (&r)[UPT], const bf16_t *src, int cc) {
                const int64_t t0 = chunk_t0(cc);
                const int nv = chunk_nv(cc);
                const int t = rtid % C, db = (rtid / C) * EPU;
                const bf16_t *gs = src + (t0 + t) * D + db;
#pragma unroll
                for (int uu = 0; uu < UPT; ++uu) {
                    r[uu] = uint4{0u, 0u, 0u, 0u};
                    if (db + uu * DU < D && t < nv) r[uu] = *reinterpret_cast<const uint4 *>(gs + uu * DU);
                }
            };
            auto stage = [&](int cc) {                  // registers -> Qs, Kt, Vt for chunk cc
                const int nv = chunk_nv(cc);
                int t = rtid % C, db = (rtid / C) * EPU;
                __asm__ volatile("" : "+v"(t), "+v"(db));   // one lane base per call, constant offsets
                float *qd = Qs + t * QS + db;
                float *kd = Kt + db * KS + t;
                uint16_t *vd = Vt + db * VS + t;
#pragma unroll
                for (int uu = 0; uu < UPT; ++uu) {
                    if (db + uu * DU >= D) break;
                    float x[EPU];
                    unpack_unit<bf16_t>(rq[uu], x);
#pragma unroll
                    for (int e = 0; e < EPU; e += 4)
                        *reinterpret_cast<float4 *>(qd + uu * DU + e) =
                            float4{x[e] * qscale, x[e + 1] * qscale, x[e + 2] * qscale, x[e + 3] * qscale};
                    unpack_unit<bf16_t>(rk[uu], x);
#pragma unroll
                    for (int e = 0; e < EPU; ++e) kd[(uu * DU + e) * KS] = x[e];
                    const uint32_t w[4] = {rv[uu].x, rv[uu].y, rv[uu].z, rv[uu].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        vd[(uu * DU + 2 * e) * VS] = (uint16_t)(w[e] & 0xffffu);
                        vd[(uu * DU + 2 * e + 1) * VS] = (uint16_t)(w[e] >> 16);
                    }
                }
                for (int tt = rtid; tt < C; tt += 64 * Cfg::NR) {
                    *reinterpret_cast<float4 *>(Qs + tt * QS + D) = float4{1.f, 0.f, 0.f, 0.f};
                    Kt[D * KS + tt] = 1.f;
                    Kt[(D + 1) * KS + tt] = 0.f; Kt[(D + 2) * KS + tt] = 0.f; Kt[(D + 3) * KS + tt] = 0.f;
                    Vt[DV * VS + tt] = tt < nv ? (uint16_t)0x3f80u : (uint16_t)0u;   // bf16 1 (valid token), 0
                }
            };
            auto fetch = [&](int cc) {
                gload(rq, qh, cc);
                gload(rk, kh, cc);
                gload(rv, vh, cc);
            };
            if (cbeg < cend) {
                fetch(cbeg);
                stage(cbeg);
                if (cbeg + 1 < cend) fetch(cbeg + 1);
            }
            __syncthreads();   // A: first chunk staged, first state copy written

            // readout geometry: tiles tt0 .. tt0 + TPW - 1; lane group g takes position 2 kk + g / 2,
            // streams 2 (g % 2) + sl, slots z as elements 2 z + sl
            const int tt0 = wave * TPW;
            const int hh = g >> 1, sp = 2 * (g & 1);
            const float *qrow[TPW];
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) qrow[tt] = Qs + (16 * (tt0 + tt) + li) * QS;
            const bf16x8 *Bv = reinterpret_cast<const bf16x8 *>(Bc);
            const bf16x8 *Bl = reinterpret_cast<const bf16x8 *>(Bc + Cfg::FULLB);
            for (int cc = cbeg; cc < cend; ++cc) {
                f32x4 Y[TPW][NT];
                if constexpr (TPW == 1) {
                    // A K step's prefix factors (prefix weight times the prefix product of the lane's
                    // two streams at position 2 kk + hh) and q block offset, gathered two steps
                    // before its products: the quad-word read and the q reads that depend on it then
                    // overlap the products of the steps in between instead of stalling at each group
                    // start.  (The loop is unrolled, so each step's entries live for three steps.)
                    float pf[NS][TPW][2];
                    int xs[NS];
                    auto gather = [&](int kk) {
                        const uint2 w2 = *reinterpret_cast<const uint2 *>(W0 + (2 * kk + hh) * 4 + sp);
                        const int i1a = qd_i1(w2.x), i2a = qd_i2(w2.x), i1b = qd_i1(w2.y), i2b = qd_i2(w2.y);
                        const float ca = qd_pweight<D, TRIPLE>(w2.x);
                        const float cb = qd_pweight<D, TRIPLE>(w2.y);
    #pragma unroll
                        for (int tt = 0; tt < TPW; ++tt) {
                            pf[kk][tt][0] = ca * qrow[tt][i1a] * qrow[tt][i2a];
                            pf[kk][tt][1] = cb * qrow[tt][i1b] * qrow[tt][i2b];
                        }
                        if constexpr (TRIPLE) {
                            const int i0a = qd_i0(w2.x), i0b = qd_i0(w2.y);
    #pragma unroll
                            for (int tt = 0; tt < TPW; ++tt) {
                                pf[kk][tt][0] *= qrow[tt][i0a];
                                pf[kk][tt][1] *= qrow[tt][i0b];
                            }
                        }
                        xs[kk] = 4 * qd_b(w2.x);
                    };
                    auto load_b = [&](bf16x8 (&B)[NT], int kk) {
    #pragma unroll
                        for (int nt = 0; nt + 1 < NT; ++nt) B[nt] = Bv[(kk * (NT - 1) + nt) * 64 + lane];
                        if constexpr (LASTW == 4) {
                            uint4 z = {0u, 0u, 0u, 0u};
                            B[NT - 1] = __builtin_bit_cast(bf16x8, z);
                            if (li == 0) B[NT - 1] = Bl[kk * 4 + g];
                        } else {
                            B[NT - 1] = Bl[kk * 64 + lane];
                        }
                    };
                    auto form = [&](bf16x8 (&A)[TPW], int kk) {
    #pragma unroll
                        for (int tt = 0; tt < TPW; ++tt) {
                            const float4 x = *reinterpret_cast<const float4 *>(qrow[tt] + xs[kk]);
                            const float p0 = pf[kk][tt][0], p1 = pf[kk][tt][1];
                            const float a[8] = {p0 * x.x, p1 * x.x, p0 * x.y, p1 * x.y,
                                                p0 * x.z, p1 * x.z, p0 * x.w, p1 * x.w};
                            A[tt] = pack_bf16x8(a);
                        }
                    };
                    // two operand sets in turn: step kk's products run while step kk + 1's are formed
                    bf16x8 A[2][TPW], B[2][NT];
                    gather(0);
                    gather(1);
                    load_b(B[0], 0);
                    form(A[0], 0);
    #pragma unroll
                    for (int kk = 0; kk < NS; ++kk) {
                        if (kk + 2 < NS) gather(kk + 2);
                        if (kk + 1 < NS) {
                            load_b(B[(kk + 1) & 1], kk + 1);
                            form(A[(kk + 1) & 1], kk + 1);
                        }
    #pragma unroll
                        for (int tt = 0; tt < TPW; ++tt)
    #pragma unroll
                            for (int nt = 0; nt < NT; ++nt)
                                Y[tt][nt] = mfma_bf16(A[kk & 1][tt], B[kk & 1][nt],
                                                      kk == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : Y[tt][nt]);
                    }
                } else {
                    // Two token tiles per wavefront: the pair products are re-formed only where a
                    // pair group starts (measured faster here than gathering every step ahead).
                    float pc[TPW][2];
                    int xo = 0;
                    auto regroup = [&](int kk) {
                        const uint2 w2 = *reinterpret_cast<const uint2 *>(W0 + (2 * kk + hh) * 4 + sp);
                        const int i1a = qd_i1(w2.x), i2a = qd_i2(w2.x), i1b = qd_i1(w2.y), i2b = qd_i2(w2.y);
                        const float ca = qd_pweight<D, TRIPLE>(w2.x);
                        const float cb = qd_pweight<D, TRIPLE>(w2.y);
    #pragma unroll
                        for (int tt = 0; tt < TPW; ++tt) {
                            pc[tt][0] = ca * qrow[tt][i1a] * qrow[tt][i2a];
                            pc[tt][1] = cb * qrow[tt][i1b] * qrow[tt][i2b];
                        }
                        if constexpr (TRIPLE) {
                            const int i0a = qd_i0(w2.x), i0b = qd_i0(w2.y);
    #pragma unroll
                            for (int tt = 0; tt < TPW; ++tt) {
                                pc[tt][0] *= qrow[tt][i0a];
                                pc[tt][1] *= qrow[tt][i0b];
                            }
                        }
                        xo = 4 * qd_b(w2.x);
                    };
                    auto advance = [&](int kk) {
                        if (((gmask >> (2 * kk - 1)) & 7u) != 0) {
                            __asm__ volatile("" ::: "memory");
                            regroup(kk);
                        } else {
                            xo += 8;
                        }
                    };
                    auto load_b = [&](bf16x8 (&B)[NT], int kk) {
    #pragma unroll
                        for (int nt = 0; nt + 1 < NT; ++nt) B[nt] = Bv[(kk * (NT - 1) + nt) * 64 + lane];
                        if constexpr (LASTW == 4) {
                            uint4 z = {0u, 0u, 0u, 0u};
                            B[NT - 1] = __builtin_bit_cast(bf16x8, z);
                            if (li == 0) B[NT - 1] = Bl[kk * 4 + g];
                        } else {
                            B[NT - 1] = Bl[kk * 64 + lane];
                        }
                    };
                    auto form = [&](bf16x8 (&A)[TPW]) {
    #pragma unroll
                        for (int tt = 0; tt < TPW; ++tt) {
                            const float4 x = *reinterpret_cast<const float4 *>(qrow[tt] + xo);
                            const float a[8] = {pc[tt][0] * x.x, pc[tt][1] * x.x, pc[tt][0] * x.y, pc[tt][1] * x.y,
                                                pc[tt][0] * x.z, pc[tt][1] * x.z, pc[tt][0] * x.w, pc[tt][1] * x.w};
                            A[tt] = pack_bf16x8(a);
                        }
                    };
                    auto mma = [&](const bf16x8 (&A)[TPW], const bf16x8 (&B)[NT]) {
    #pragma unroll
                        for (int tt = 0; tt < TPW; ++tt)
    #pragma unroll
                            for (int nt = 0; nt < NT; ++nt) Y[tt][nt] = mfma_bf16(A[tt], B[nt], Y[tt][nt]);
                    };
                    // two operand sets in turn: step kk's products run while step kk + 1's are formed
                    bf16x8 A0[TPW], B0[NT], A1[TPW], B1[NT];
                    regroup(0);
                    load_b(B0, 0);
                    form(A0);
                    advance(1);
                    load_b(B1, 1);
                    form(A1);
    #pragma unroll
                    for (int tt = 0; tt < TPW; ++tt)
    #pragma unroll
                        for (int nt = 0; nt < NT; ++nt) Y[tt][nt] = mfma_bf16(A0[tt], B0[nt], f32x4{0.f, 0.f, 0.f, 0.f});
    #pragma unroll 1
                    for (int kk = 1; kk + 2 < NS; kk += 2) {
                        advance(kk + 1);
                        load_b(B0, kk + 1);
                        form(A0);
                        mma(A1, B1);
                        advance(kk + 2);
                        load_b(B1, kk + 2);
                        form(A1);
                        mma(A0, B0);
                    }
                    mma(A1, B1);
                }
                __syncthreads();   // B: readout and update of chunk cc done

                // partials of chunk cc: [TT][NC][16 tokens] per (bh, chunk, slice)
                bf16_t *pdst = partial + ((bh * nchunk + cc) * nslices + slice) * (int64_t)(TT * NC * 16) +
                               (int64_t)tt0 * NC * 16 + (li * 16 + 4 * g);
#pragma unroll
                for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        if (16 * nt + li < NC) store4(pdst + (tt * NC + 16 * nt) * 16, Y[tt][nt]);
                if (cc + 1 < cend) {
                    stage(cc + 1);
                    if (cc + 2 < cend) fetch(cc + 2);
                }
                __syncthreads();   // A: next chunk staged, new state copy written
            }
        } else {
            // ------------------------------------------------ update wavefronts
            const int uw_ = wave - Cfg::NR;
            const int p0 = uw_ * MT;
            // tile rows: stream li % 4, slot li / 4 (a DPP quad shares its slot); accumulator rows
            // 4 g + r: stream r, slot g
            const int us = li & 3, uz = li >> 2;
            float *Sh = state + bh * NC * m_pad;
            f32x4 S[MT][NT];
#pragma unroll
            for (int j = 0; j < MT; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t qd = (ps0 + p0 + j) * 4 + r;
                    const uint32_t w = qw0[qd];
                    const int32_t c0 = qcidx[qd];
                    const uint32_t mask = qd_mask(w);
                    const int z0 = mask ? __builtin_ctz(mask) : 0;
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        const int c = 16 * nt + li;
                        const bool ok = ((mask >> g) & 1u) && c < NC;
                        S[j][nt][r] = ok ? Sh[(int64_t)c * m_pad + c0 + (g - z0)] : 0.f;
                    }
                }
            uint32_t uw[MT];
            uint32_t newgrp = 0;
#pragma unroll
            for (int j = 0; j < MT; ++j) {
                uw[j] = W0[(p0 + j) * 4 + us];
                if (QF[p0 + j] & 2u) newgrp |= 1u << j;
            }
            newgrp = (uint32_t)__builtin_amdgcn_readfirstlane((int)newgrp);
            const uint32_t mixed = (uint32_t)((nmask >> p0) & ((1ull << MT) - 1));

            auto slot_ratio = [&](int p, float (&r4)[4]) {
                const float *qcf = reinterpret_cast<const float *>(QC);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t w = W0[p * 4 + r];
                    const float rinv = qd_pfact<D, TRIPLE>(w);
                    r4[r] = qcf[(p * 4 + r) * 4 + g] * rinv;
                }
            };
            // state accumulators -> state copy (slot weight over pair weight at mixed positions).
            // Position p0 + j, streams 2 h2 and 2 h2 + 1 of slot g: K step p0 / 2 + j / 2, reader
            // lane group 2 (j % 2) + h2 (p0 is even), word g of the 16-byte entry.  One lane base
            // per call (kept opaque so that the compiler does not hold an address per entry through
            // the chunk loop); every entry is a constant offset from it.
            static_assert(MT % 2 == 0, "positions of an update wavefront pair up in K steps");
            auto write_bcopy = [&]() {
                int lb = (p0 / 2) * (NT - 1) * 256 + li * 4 + g;
                int lbl = LASTW == 4 ? (p0 / 2) * 16 + g : (p0 / 2) * 256 + li * 4 + g;
                __asm__ volatile("" : "+v"(lb), "+v"(lbl));
                uint32_t *B4 = reinterpret_cast<uint32_t *>(Bc) + lb;
                uint32_t *BL4 = reinterpret_cast<uint32_t *>(Bc + Cfg::FULLB) + lbl;
                auto put = [&](int j, int nt, int h2, uint32_t val) {
                    const int kj = j >> 1, gr = 2 * (j & 1) + h2;
                    if (nt + 1 < NT) {
                        B4[(kj * (NT - 1) + nt) * 256 + gr * 64] = val;
                    } else if constexpr (LASTW == 4) {
                        if (li == 0) BL4[kj * 16 + gr * 4] = val;
                    } else {
                        BL4[kj * 256 + gr * 64] = val;
                    }
                };
#pragma unroll
                for (int j = 0; j < MT; ++j)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        put(j, nt, 0, pack_bf16x2(S[j][nt][0], S[j][nt][1]));
                        put(j, nt, 1, pack_bf16x2(S[j][nt][2], S[j][nt][3]));
                    }
#pragma unroll
                for (int j = 0; j < MT; ++j) {
                    if ((mixed >> j) & 1u) {
                        float r4[4];
                        slot_ratio(p0 + j, r4);
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) {
                            put(j, nt, 0, pack_bf16x2(S[j][nt][0] * r4[0], S[j][nt][1] * r4[1]));
                            put(j, nt, 1, pack_bf16x2(S[j][nt][2] * r4[2], S[j][nt][3] * r4[3]));
                        }
                    }
                }
            };
            write_bcopy();
            __syncthreads();   // A

            constexpr int NKS = C / 32;
            const bf16_t *V16 = reinterpret_cast<const bf16_t *>(Vt);
            auto load_v = [&](bf16x8 (&B)[NT], int ks) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    uint4 z = {0u, 0u, 0u, 0u};
                    if (16 * nt + li < NC) z = *reinterpret_cast<const uint4 *>(V16 + (16 * nt + li) * VS + 32 * ks + 8 * g);
                    B[nt] = __builtin_bit_cast(bf16x8, z);
                }
            };
            auto load_k3 = [&](int j, int ks) {
                return *reinterpret_cast<const float2 *>(Kt + (4 * qd_b(uw[j]) + uz) * KS + 32 * ks + 8 * g + 2 * us);
            };
            for (int cc = cbeg; cc < cend; ++cc) {
                // S[slice, :] += phi(K_c)[:, slice]^T [V_c | 1], the chunk's K steps outer
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    bf16x8 B[NT];
                    load_v(B, ks);
                    const int tb = 32 * ks + 8 * g;
                    float p2[8];
                    float2 kc = load_k3(0, ks);
#pragma unroll
                    for (int j = 0; j < MT; ++j) {
                        const uint32_t w = uw[j];
                        if (j == 0 || ((newgrp >> j) & 1u)) {
                            __asm__ volatile("" ::: "memory");   // keep the reload behind its (uniform) branch
                            const float4 *k1 = reinterpret_cast<const float4 *>(Kt + qd_i1(w) * KS + tb);
                            const float4 *k2 = reinterpret_cast<const float4 *>(Kt + qd_i2(w) * KS + tb);
                            const float4 a0 = k1[0], a1 = k1[1], b0 = k2[0], b1 = k2[1];
                            p2[0] = a0.x * b0.x; p2[1] = a0.y * b0.y; p2[2] = a0.z * b0.z; p2[3] = a0.w * b0.w;
                            p2[4] = a1.x * b1.x; p2[5] = a1.y * b1.y; p2[6] = a1.z * b1.z; p2[7] = a1.w * b1.w;
                            if constexpr (TRIPLE) {
                                const float4 *k0 = reinterpret_cast<const float4 *>(Kt + qd_i0(w) * KS + tb);
                                const float4 c0 = k0[0], c1 = k0[1];
                                p2[0] *= c0.x; p2[1] *= c0.y; p2[2] *= c0.z; p2[3] *= c0.w;
                                p2[4] *= c1.x; p2[5] *= c1.y; p2[6] *= c1.z; p2[7] *= c1.w;
                            }
                        }
                        float2 kn = kc;
                        if (j + 1 < MT) kn = load_k3(j + 1, ks);
                        const float x = kc.x, y = kc.y;
                        float a[8] = {p2[0] * quad_bcast<0>(x), p2[1] * quad_bcast<0>(y),
                                      p2[2] * quad_bcast<1>(x), p2[3] * quad_bcast<1>(y),
                                      p2[4] * quad_bcast<2>(x), p2[5] * quad_bcast<2>(y),
                                      p2[6] * quad_bcast<3>(x), p2[7] * quad_bcast<3>(y)};
                        const bf16x8 A = pack_bf16x8(a);
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) S[j][nt] = mfma_bf16(A, B[nt], S[j][nt]);
                        kc = kn;
                    }
                }
                __syncthreads();   // B
                write_bcopy();
                __syncthreads();   // A
            }
            // accumulators -> state slice (the memory clobber makes the compiler recompute the
            // addresses instead of holding the load's ones through the chunk loop)
            __asm__ volatile("" ::: "memory");
#pragma unroll
            for (int j = 0; j < MT; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t qd = (ps0 + p0 + j) * 4 + r;
                    const uint32_t w = qw0[qd];
                    const int32_t c0 = qcidx[qd];
                    const uint32_t mask = qd_mask(w);
                    const int z0 = mask ? __builtin_ctz(mask) : 0;
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        const int c = 16 * nt + li;
                        if (((mask >> g) & 1u) && c < NC) Sh[(int64_t)c * m_pad + c0 + (g - z0)] = S[j][nt][r];
                    }
                }
        }
        // every wave's state stores reach L2 before the barrier; thread 0's agent-scope release
        // then writes L2 back before the flag
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
        __syncthreads();
        if (tid == 0) {
            __hip_atomic_store(&sync[1 + rem], (uint32_t)(u + 1), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            s_item = (int64_t)atomicAdd(&sync[0], 1u) + item_base;
        }
        __syncthreads();
    }
}

// Order 0, the constant feature, is kept out of the scan: its state entries
// S[c][0] are the running sums of [v, 1][c] over all tokens seen [hotdry,
// "Engineering realisation of the constant compute cost": the "+1" column and
// the constant Taylor term], so a chunk's inter-chunk readout from order 0 is
// the sum of [v, 1] over every earlier token (weight 1/0! d^0 = 1).  First the
// per-chunk sums (block (chunk, head); groups of d_V + 1 threads split the
// tokens, then add in a fixed order), then per head the exclusive prefix over
// the chunks starting from S[:, 0], which also leaves S[:, 0] covering the call.
template <int DV, typename TIn>
__global__ __launch_bounds__(256) void order0_sums_kernel(const TIn *__restrict__ v, int64_t n, int C,
                                                          float *__restrict__ sums) {
    constexpr int NC = DV + 1, G = 256 / NC;
    __shared__ float part[G][NC];
    const int64_t cc = blockIdx.x, bh = blockIdx.y, nchunks = gridDim.x;
    const int64_t t0 = cc * C;
    const int nv = (int)min<int64_t>(C, n - t0);
    const int tid = threadIdx.x, g = tid / NC, c = tid % NC;
    if (g < G) {
        float s = 0.f;
        if (c < DV) {
            for (int t = g; t < nv; t += G) s += to_f32(v[(bh * n + t0 + t) * DV + c]);
        } else if (g == 0) {
            s = (float)nv;
        }
        part[g][c] = s;
    }
    __syncthreads();
    if (tid < NC) {
        float s = 0.f;
        for (int gg = 0; gg < G; ++gg) s += part[gg][tid];
        sums[(bh * nchunks + cc) * NC + tid] = s;
    }
}

template <int DV>
__global__ __launch_bounds__(256) void order0_prefix_kernel(const float *__restrict__ sums, float *__restrict__ prefix,
                                                            int64_t nchunks, float *__restrict__ state, int64_t m_pad) {
    constexpr int NC = DV + 1;
    const int64_t bh = blockIdx.x;
    const int c = threadIdx.x;
    if (c >= NC) return;
    float *s0 = state + (bh * NC + c) * m_pad;     // feature 0 of row c
    float run = *s0;
    const float *in = sums + bh * nchunks * NC + c;
    float *out = prefix + bh * nchunks * NC + c;
#pragma unroll 16
    for (int64_t cc = 0; cc < nchunks; ++cc) {
        const float x = in[cc * NC];
        out[cc * NC] = run;
        run += x;
    }
    *s0 = run;
}

// Kernel 2: y = (direct intra-chunk term) + sum over slices of the partials
// (fixed order) + the chunk's order-0 prefix, o = y[:d_V] / y[d_V] (or y[:d_V]
// itself when ta.raw; the normaliser y[d_V] also goes to den_out when that is
// given).  Partial layout per (bh, chunk, slice):
// [C/16][d_V+1][16 tokens] fp32.  Every thread first adds the slices' partials
// with 16-byte loads; then wave w < C/32 adds the intra-chunk term of query
// tiles w and C/16-1-w (tile qt needs qt+1 key tiles, so each wave does
// C/16+1 tiles' worth).
template <int D, int DV, int C, typename TIn, typename TOut>
__global__ __launch_bounds__(256) void prefill_reduce_kernel(const typename PartialOf<TIn>::type *__restrict__ partial,
                                                             int nslices,
                                                             int nchunk, int64_t n, int64_t tok0,
                                                             const TIn *__restrict__ q, const TIn *__restrict__ k,
                                                             const TIn *__restrict__ v, TOut *__restrict__ out,
                                                             TaylorArgs ta, float *__restrict__ den_out,
                                                             const float *__restrict__ o0pre) {
    constexpr int NC = DV + 1, TT = C / 16, NT = (NC + 15) / 16, NCP = 16 * NT;
    constexpr int VS = sizeof(TIn) == 2 ? C + 8 : C + 4;
    constexpr int NV = TT * NC * 4;                 // float4 per partial
    constexpr int PER = (NV + 255) / 256;
    constexpr int VBYTES = NCP * VS * (int)sizeof(TIn);
    __shared__ __align__(16) unsigned char vt[VBYTES];
    __shared__ __align__(16) float ys[TT * NC * 16];
    const int cc = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches below
    const int g = lane >> 4, li = lane & 15;
    const int64_t t0 = tok0 + (int64_t)cc * C;
    const int nvalid = n - t0 < C ? (int)(n - t0) : C;
    const TIn *qh = q + bh * n * D;
    const TIn *kh = k + bh * n * D;
    const TIn *vh = v + bh * n * DV;

    // partial sums first: their loads are the long pole, issue them before the MFMA work.
    // 16-byte loads (8 bf16 or 4 fp32 values), four slices in flight per thread.
    using PT = typename PartialOf<TIn>::type;
    constexpr int VEC = 16 / (int)sizeof(PT);       // values per load
    constexpr int NVV = NV * 4 / VEC;               // loads per slice
    constexpr int PERV = (NVV + 255) / 256;
    constexpr int SU = 4;                           // slices per round
    const PT *base = partial + (bh * nchunk + cc) * (int64_t)nslices * NV * 4;
    float acc[PERV][VEC];
#pragma unroll
    for (int j = 0; j < PERV; ++j)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[j][e] = 0.f;
    auto add_vec = [&](float (&a)[VEC], const uint4 &u) {
        if constexpr (VEC == 8) {
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a[2 * e] += __uint_as_float(w[e] << 16);
                a[2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
            }
        } else {
            a[0] += __uint_as_float(u.x); a[1] += __uint_as_float(u.y);
            a[2] += __uint_as_float(u.z); a[3] += __uint_as_float(u.w);
        }
    };
    int s = 0;
    for (; s + SU <= nslices; s += SU) {
        uint4 u[SU][PERV];
#pragma unroll
        for (int r = 0; r < SU; ++r)
#pragma unroll
            for (int j = 0; j < PERV; ++j) {
                const int i = tid + 256 * j;
                u[r][j] = i < NVV ? *reinterpret_cast<const uint4 *>(base + ((int64_t)(s + r) * NVV + i) * VEC)
                                  : uint4{0u, 0u, 0u, 0u};
            }
#pragma unroll
        for (int r = 0; r < SU; ++r)
#pragma unroll
            for (int j = 0; j < PERV; ++j) add_vec(acc[j], u[r][j]);
    }
    for (; s < nslices; ++s) {
#pragma unroll
        for (int j = 0; j < PERV; ++j) {
            const int i = tid + 256 * j;
            if (i < NVV) add_vec(acc[j], *reinterpret_cast<const uint4 *>(base + ((int64_t)s * NVV + i) * VEC));
        }
    }
#pragma unroll
    for (int j = 0; j < PERV; ++j) {
        const int i = tid + 256 * j;
        if (i < NVV) {
#pragma unroll
            for (int e = 0; e < VEC; e += 4)
                reinterpret_cast<float4 *>(ys)[i * (VEC / 4) + e / 4] = float4{acc[j][e], acc[j][e + 1], acc[j][e + 2], acc[j][e + 3]};
        }
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
    const float *pre = o0pre + (bh * ((n + C - 1) / C) + t0 / C) * NC;   // this chunk's order-0 prefix
    for (int i = tid; i < C * DV; i += 256) {
        const int t = i / DV, c = i - t * DV;
        if (t < nvalid) {
            const int tt = t >> 4, t16 = t & 15;
            const float y = ys[(tt * NC + c) * 16 + t16] + pre[c];
            const float den = ys[(tt * NC + DV) * 16 + t16] + pre[DV];
            out[(bh * n + t0 + t) * DV + c] = from_f32<TOut>(ta.raw ? y : y / den);
            if (den_out && c == 0) den_out[bh * n + t0 + t] = den;
        }
    }
}

// ---------------------------------------------------------------- host side

// Wavefronts per workgroup and positions per wavefront (16 features each); a
// slice holds NW * MT positions.  Four wavefronts with as many positions as the
// register budget allows for the d_V + 1 columns, fewer when the grid would not
// fill the chip.  The fp32 path keeps a 4-byte state copy in LDS, so it stops
// at 4.  (The kernel also supports eight wavefronts of fewer positions each.)
struct ScanShape {
    int nw, mt;
    bool ws;   // warp-specialised kernel: 4 update wavefronts of mt positions, 4 readout wavefronts
};
static ScanShape pick_shape(const sata_index *idx, int64_t bh, int chunk, sata_dtype in_dt) {
    const int64_t npos = idx->nq / 4;
    // bf16 inputs.  d_K = 64 in 128-token chunks: eight wavefronts that each read out and update
    // (four or two positions each); the warp-specialised kernel holds too few positions per
    // wavefront there.  Otherwise the warp-specialised kernel, 32 positions per slice when that
    // still gives every CU a slice, else 16.
    if (in_dt == SATA_BF16) {
        const bool many = bh * ((npos + 31) / 32) >= 256;
        if (idx->dk == 64 && chunk == 128) return {8, many ? 4 : 2, false};
        return {8, many ? 8 : 4, true};
    }
    for (int mt : {8, 4}) {
        if (mt == 8 && in_dt == SATA_F32) continue;
        const int64_t per = (int64_t)kNW * mt;
        if (bh * ((npos + per - 1) / per) >= 256) return {kNW, mt, false};
    }
    return {kNW, 2, false};
}

bool scan16_covers(const sata_index *idx, sata_dtype in_dt) {
    return in_dt == SATA_BF16 && idx->np16 > 0 && idx->dk == idx->dv &&
           (idx->dk == 16 || idx->dk == 32 || idx->dk == 64 || idx->dk == 128);
}

PrefillPlan plan_prefill(const sata_index *idx, int64_t bh, int64_t n, int chunk, sata_dtype in_dt, int64_t work_cap,
                         bool fp16_operands) {
    PrefillPlan p;
    const bool s16 = fp16_operands && scan16_covers(idx, in_dt);
    // default chunk: 128 tokens for the fp16-operand scan (measured faster than 64 at every
    // head size it takes up to 64, by 18-26%), for d_K = 64, and for fp32 inputs at d_K = 16
    // (1 x 8 x 4096: 0.437 ms per call against 0.482); 64 for the other scans
    p.chunk = chunk ? chunk : (s16 || idx->dk == 64 || (idx->dk == 16 && in_dt == SATA_F32) ? 128 : 64);
    // the fp16-operand scan at d_K = 16 by default takes 256-token chunks: its chunk steps are
    // short, so twice the work per step amortises the per-step staging and barriers (1 x 64 x
    // 131072: 3.35 ms per call against 3.52-3.64 at 128; scan 1.97 ms against 2.45-2.56)
    if (!chunk && s16 && idx->dk == 16) p.chunk = 256;
    if (p.chunk != 64 && p.chunk != 128 && !(p.chunk == 256 && s16 && idx->dk == 16)) return p;
    if (idx->dk == 128) {
        if (!s16) return p;   // no chunked plan: the block prefill covers it
        p.chunk = 64;         // the operand image of a 128-token chunk does not fit beside the state copy
    }
    const int64_t nchunks = (n + p.chunk - 1) / p.chunk;
    if (s16) {
        // fp16-operand scan: fp16 partials and one operand image per chunk of a segment
        p.s16 = true;
        p.mt = scan16_choose_mt(idx->dk, idx->np16, bh, idx->cus);
        const int np = 4 * p.mt;
        p.fs = 64 * np;
        p.fw = p.fs / 4;
        p.slices = (int)((idx->np16 + np - 1) / np);
        const int64_t part_chunk = bh * p.slices * (int64_t)p.chunk * (idx->dv + 1) * 2;
        const int64_t img_chunk = bh * scan16_image_bytes(idx->dk, p.chunk);
        p.sync_words = (kScanQueues + bh * p.slices + 3) / 4 * 4;   // queue counters, then the flags
        const int64_t o0_bytes = 2 * bh * std::max<int64_t>(nchunks, 1) * (idx->dv + 1) * (int64_t)sizeof(float);
        const int64_t fixed = 1024 + p.sync_words * 4 + o0_bytes;
        const int64_t room = std::max<int64_t>(work_cap - fixed, 0);
        p.seg_chunks = std::max<int64_t>(1, std::min<int64_t>(nchunks, room / (part_chunk + img_chunk)));
        p.sync_off = (p.seg_chunks * part_chunk + 255) / 256 * 256;
        p.o0_off = (p.sync_off + p.sync_words * 4 + 255) / 256 * 256;
        p.img_off = (p.o0_off + o0_bytes + 255) / 256 * 256;
        p.work_bytes = p.img_off + p.seg_chunks * img_chunk;
        p.ok = (int64_t)p.slices * np <= idx->np16 + kPos16Pad;
        return p;
    }
    const ScanShape sh = pick_shape(idx, bh, p.chunk, in_dt);
    p.ws = sh.ws;
    p.fw = 16 * sh.mt;
    const int64_t np_slice = (int64_t)(sh.ws ? 4 : sh.nw) * sh.mt;
    p.fs = (int)(16 * np_slice);
    const int64_t npos = idx->nq / 4;
    p.slices = (int)((npos + np_slice - 1) / np_slice);
    const int64_t pbytes = in_dt == SATA_BF16 ? 2 : 4;   // readout partials in the input's width
    const int64_t per_chunk = bh * p.slices * (int64_t)p.chunk * (idx->dv + 1) * pbytes;
    // after the partial sums: the scan's work counter and one progress flag per (head, slice),
    // then the order-0 chunk sums and their prefixes for the whole call (not segmented)
    p.sync_words = (1 + bh * p.slices + 3) / 4 * 4;
    const int64_t fixed = 512 + p.sync_words * 4 + 2 * bh * std::max<int64_t>(nchunks, 1) * (idx->dv + 1) * (int64_t)sizeof(float);
    const int64_t room = std::max<int64_t>(work_cap - fixed, 0);
    p.seg_chunks = per_chunk ? std::max<int64_t>(1, std::min<int64_t>(nchunks, room / per_chunk)) : nchunks;
    p.sync_off = (p.seg_chunks * per_chunk + 255) / 256 * 256;
    p.o0_off = (p.sync_off + p.sync_words * 4 + 255) / 256 * 256;
    p.work_bytes = p.o0_off + 2 * bh * std::max<int64_t>(nchunks, 1) * (idx->dv + 1) * (int64_t)sizeof(float);
    p.ok = (int64_t)p.slices * np_slice * 4 <= idx->nq_tab;
    return p;
}

// The scan kernel and its launch shape: the general kernel, or the warp-specialised one.
// TRIPLE: features of order 4 (P = 5), whose quads carry a three-index prefix.
template <int D, int C, int MT, int NW, typename TIn, bool WS, bool TRIPLE>
struct ScanSel {
    using Cfg = ScanCfg<D, D, C, MT, NW, TIn>;
    static constexpr int THREADS = Cfg::THREADS, LDS = Cfg::LDS;
    static constexpr bool PERSIST = Cfg::PERSIST;
    static constexpr auto kernel = prefill_scan_kernel<D, D, C, MT, NW, TIn, TRIPLE>;
};
template <int D, int C, int MT, int NW, bool TRIPLE>
struct ScanSel<D, C, MT, NW, bf16_t, true, TRIPLE> {
    using Cfg = WsCfg<D, D, C, MT>;
    static constexpr int THREADS = Cfg::THREADS, LDS = Cfg::LDS;
    static constexpr bool PERSIST = true;
    static constexpr auto kernel = prefill_scan_ws_kernel<D, D, C, MT, TRIPLE>;
};

template <int D, int C, int MT, int NW, typename TIn, typename TOut, bool WS, bool TRIPLE>
static hipError_t run_prefill(const sata_index *idx, const sata_state *st, const PrefillPlan &plan,
                              const void *q, const void *k, const void *v, void *out, int64_t n,
                              hipStream_t stream) {
    using Cfg = ScanSel<D, C, MT, NW, TIn, WS, TRIPLE>;
    const int64_t bh = (int64_t)st->batch * st->heads;
    auto scan = Cfg::kernel;
    auto red = prefill_reduce_kernel<D, D, C, TIn, TOut>;
    hipError_t e = hipFuncSetAttribute((const void *)scan, hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS);
    if (e != hipSuccess) return e;
    TaylorArgs ta;
    ta.scale = 1.0f / sqrtf((float)D);
    ta.c0 = idx->taylor[0]; ta.c1 = idx->taylor[1]; ta.c2 = idx->taylor[2]; ta.c3 = idx->taylor[3];
    ta.c4 = idx->taylor[4];
    ta.P = idx->P;
    ta.raw = plan.raw ? 1 : 0;
    const int64_t nchunks = (n + C - 1) / C;
    auto *partial = static_cast<typename PartialOf<TIn>::type *>(st->d_work);
    uint32_t *sync = reinterpret_cast<uint32_t *>(static_cast<char *>(st->d_work) + plan.sync_off);
    // Persistent grid: as many workgroups as fit on the device at once.
    int cus = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, st->device);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, scan, Cfg::THREADS, Cfg::LDS);
    if (e != hipSuccess) return e;
    const int64_t resident = (int64_t)std::max(cus, 1) * std::max(per_cu, 1);
    const int64_t items0 = bh * plan.slices;
    const ScanDebug dbg = scan_debug();
    // order 0: chunk sums of [v, 1], their prefixes from the state's entries, and those entries' update
    float *o0sums = reinterpret_cast<float *>(static_cast<char *>(st->d_work) + plan.o0_off);
    float *o0pre = o0sums + bh * nchunks * (D + 1);
    hipLaunchKernelGGL((order0_sums_kernel<D, TIn>), dim3((unsigned)nchunks, (unsigned)bh), dim3(256), 0, stream,
                       static_cast<const TIn *>(v), n, C, o0sums);
    hipLaunchKernelGGL((order0_prefix_kernel<D>), dim3((unsigned)bh), dim3((D + 1 + 63) / 64 * 64), 0, stream, o0sums,
                       o0pre, nchunks, static_cast<float *>(st->d_state), idx->m_pad);   // a thread per column
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    for (int64_t c0 = 0; c0 < nchunks; c0 += plan.seg_chunks) {
        const int nseg = (int)std::min<int64_t>(plan.seg_chunks, nchunks - c0);
        const int64_t tok0 = c0 * C;
        // Split the segment into sub-segments of at least 16 chunks until there are about a dozen
        // items per resident workgroup, so every CU gets the same share of the work (a grid of
        // at most one workgroup per CU gains nothing from splitting).
        int nsub = !Cfg::PERSIST || items0 <= cus ? 1
                 : (int)std::min<int64_t>((12 * resident + items0 - 1) / items0, std::max(1, nseg / 16));
        const int sub_chunks = (nseg + nsub - 1) / nsub;
        nsub = (nseg + sub_chunks - 1) / sub_chunks;
        const int64_t grid = Cfg::PERSIST ? std::min<int64_t>(items0 * nsub, resident) : items0;
        if (Cfg::PERSIST && items0 > 0) {
            e = launch_zero(reinterpret_cast<float *>(sync), plan.sync_words, stream);
            if (e != hipSuccess) return e;
        }
        if (items0 > 0) {   // P = 1: order 0 alone, no scan
            ProfScope ps(kProfScan, stream);
            hipLaunchKernelGGL(scan, dim3((unsigned)grid), dim3(Cfg::THREADS), Cfg::LDS, stream,
                               idx->d_qw0, idx->d_qcidx, reinterpret_cast<const float4 *>(idx->d_qcoef),
                               idx->d_qflags, static_cast<float *>(st->d_state), idx->m_pad, static_cast<const TIn *>(q),
                               static_cast<const TIn *>(k), static_cast<const TIn *>(v), n, tok0, nseg,
                               partial, ta.scale, plan.slices, bh, nsub, sub_chunks, sync, dbg.item_base,
                               dbg.spin_limit, st->d_err);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        {
            ProfScope ps(kProfCombine, stream);
            hipLaunchKernelGGL(red, dim3(nseg, (unsigned)bh), dim3(256), 0, stream, partial, plan.slices, nseg,
                               n, tok0, static_cast<const TIn *>(q), static_cast<const TIn *>(k),
                               static_cast<const TIn *>(v), static_cast<TOut *>(out), ta, plan.den_out, o0pre);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int D, int C, int MT, int NW, bool TRIPLE>
static hipError_t run_dt(const sata_index *idx, const sata_state *st, const PrefillPlan &plan,
                         const void *q, const void *k, const void *v, void *out, int64_t n,
                         sata_dtype in_dt, sata_dtype out_dt, hipStream_t s) {
    if constexpr (MT > 4 || NW > 4) {
        if (in_dt == SATA_F32) return hipErrorInvalidValue;   // pick_shape never plans this
    } else if (in_dt == SATA_F32) {
        if (out_dt == SATA_F32) return run_prefill<D, C, MT, NW, float, float, false, TRIPLE>(idx, st, plan, q, k, v, out, n, s);
        return run_prefill<D, C, MT, NW, float, bf16_t, false, TRIPLE>(idx, st, plan, q, k, v, out, n, s);
    }
    if (out_dt == SATA_F32) return run_prefill<D, C, MT, NW, bf16_t, float, false, TRIPLE>(idx, st, plan, q, k, v, out, n, s);
    return run_prefill<D, C, MT, NW, bf16_t, bf16_t, false, TRIPLE>(idx, st, plan, q, k, v, out, n, s);
}

template <int D, bool TRIPLE>
static hipError_t run_d(const sata_index *idx, const sata_state *st, const PrefillPlan &plan,
                        const void *q, const void *k, const void *v, void *out, int64_t n,
                        sata_dtype in_dt, sata_dtype out_dt, hipStream_t s) {
    const int mt = plan.fw / 16, nw = plan.fs / plan.fw;
    if (plan.ws) {
        if (in_dt != SATA_BF16) return hipErrorInvalidValue;   // never planned
        auto go = [&](auto cw, auto mw) -> hipError_t {
            constexpr int CC = decltype(cw)::value, MM = decltype(mw)::value;
            if (out_dt == SATA_F32) return run_prefill<D, CC, MM, 8, bf16_t, float, true, TRIPLE>(idx, st, plan, q, k, v, out, n, s);
            return run_prefill<D, CC, MM, 8, bf16_t, bf16_t, true, TRIPLE>(idx, st, plan, q, k, v, out, n, s);
        };
        using I64 = std::integral_constant<int, 64>;
        using I128 = std::integral_constant<int, 128>;
        using M4 = std::integral_constant<int, 4>;
        using M8 = std::integral_constant<int, 8>;
        if (plan.chunk == 64) return mt == 8 ? go(I64{}, M8{}) : go(I64{}, M4{});
        return mt == 8 ? go(I128{}, M8{}) : go(I128{}, M4{});
    }
    if (nw == 8) {
        if (plan.chunk != 128 || in_dt != SATA_BF16) return hipErrorInvalidValue;   // never planned
        if (mt == 2) return run_dt<D, 128, 2, 8, TRIPLE>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, s);
        return run_dt<D, 128, 4, 8, TRIPLE>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, s);
    }
    if (plan.chunk == 64) {
        if (mt == 2) return run_dt<D, 64, 2, 4, TRIPLE>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, s);
        if (mt == 4) return run_dt<D, 64, 4, 4, TRIPLE>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, s);
        return run_dt<D, 64, 8, 4, TRIPLE>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, s);
    }
    if (mt == 2) return run_dt<D, 128, 2, 4, TRIPLE>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, s);
    if (mt == 4) return run_dt<D, 128, 4, 4, TRIPLE>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, s);
    return run_dt<D, 128, 8, 4, TRIPLE>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, s);
}

// fp16-operand scan: the order-0 chunk sums and prefixes of the whole call, then per segment the
// operand images, the scan and the reduce (sata_scan16.hip).
template <int D>
static hipError_t run_prefill16(const sata_index *idx, const sata_state *st, const PrefillPlan &plan, const void *q,
                                const void *k, const void *v, void *out, int64_t n, sata_dtype out_dt,
                                hipStream_t stream) {
    const int C = plan.chunk;
    const int64_t bh = (int64_t)st->batch * st->heads;
    const int64_t nchunks = (n + C - 1) / C;
    TaylorArgs ta;
    ta.scale = 1.0f / sqrtf((float)D);
    ta.c0 = idx->taylor[0]; ta.c1 = idx->taylor[1]; ta.c2 = idx->taylor[2]; ta.c3 = idx->taylor[3];
    ta.c4 = idx->taylor[4];
    ta.P = idx->P;
    ta.raw = plan.raw ? 1 : 0;
    float *o0sums = reinterpret_cast<float *>(static_cast<char *>(st->d_work) + plan.o0_off);
    float *o0pre = o0sums + bh * nchunks * (D + 1);
    if (plan.v_f16)
        hipLaunchKernelGGL((order0_sums_kernel<D, f16_t>), dim3((unsigned)nchunks, (unsigned)bh), dim3(256), 0, stream,
                           static_cast<const f16_t *>(v), n, C, o0sums);
    else
        hipLaunchKernelGGL((order0_sums_kernel<D, bf16_t>), dim3((unsigned)nchunks, (unsigned)bh), dim3(256), 0, stream,
                           static_cast<const bf16_t *>(v), n, C, o0sums);
    hipLaunchKernelGGL((order0_prefix_kernel<D>), dim3((unsigned)bh), dim3((D + 1 + 63) / 64 * 64), 0, stream, o0sums,
                       o0pre, nchunks, static_cast<float *>(st->d_state), idx->m_pad);   // a thread per column
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    for (int64_t c0 = 0; c0 < nchunks; c0 += plan.seg_chunks) {
        const int nseg = (int)std::min<int64_t>(plan.seg_chunks, nchunks - c0);
        e = launch_scan16_segment(idx, st, plan, q, k, v, out, n, c0 * C, nseg, o0pre, ta, out_dt, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_prefill(const sata_index *idx, const sata_state *st, const PrefillPlan &plan,
                          const void *q, const void *k, const void *v, void *out, int64_t n,
                          sata_dtype in_dt, sata_dtype out_dt, hipStream_t stream) {
    // shared q and k, binary16 values: the fp16-operand scan only
    if (plan.qk_div < 1 || ((plan.qk_div != 1 || plan.v_f16) && !plan.s16)) return hipErrorInvalidValue;
    if (plan.s16) {
        if (in_dt != SATA_BF16) return hipErrorInvalidValue;   // never planned
        switch (idx->dk) {
            case 16: return run_prefill16<16>(idx, st, plan, q, k, v, out, n, out_dt, stream);
            case 32: return run_prefill16<32>(idx, st, plan, q, k, v, out, n, out_dt, stream);
            case 64: return run_prefill16<64>(idx, st, plan, q, k, v, out, n, out_dt, stream);
            case 128: return run_prefill16<128>(idx, st, plan, q, k, v, out, n, out_dt, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (idx->dk) {
        case 8: return idx->P >= 5 ? run_d<8, true>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, stream)
                                   : run_d<8, false>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, stream);
        case 16: return idx->P >= 5 ? run_d<16, true>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, stream)
                                    : run_d<16, false>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, stream);
        case 32: return idx->P >= 5 ? run_d<32, true>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, stream)
                                    : run_d<32, false>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, stream);
        case 64: return idx->P >= 5 ? run_d<64, true>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, stream)
                                    : run_d<64, false>(idx, st, plan, q, k, v, out, n, in_dt, out_dt, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sata
