// Chunked SATA prefill on fp16 MFMA operands for gfx950 (bf16 inputs, P <= 4,
// d_K = d_V in {16, 32, 64}).
//
// Same decomposition as the general scan (sata_prefill.hip): per chunk c of C
// tokens, Y_c = psi(Q_c) . S^(c-1) (inter-chunk readout), plus the direct
// intra-chunk Taylor term, and S^(c) = S^(c-1) + phi(K_c)^T [V_c | 1]
// [hotdry, "Engineering realisation of the constant compute cost"].  What
// differs is how the two contractions are fed to the matrix cores:
//
//  * Operands are fp16 (v_mfma_f32_16x16x32_f16, fp32 accumulation).  A
//    feature operand element is a product of fp16 values formed with packed
//    multiplies (two per instruction, no conversion), and the bf16 inputs
//    convert to fp16 exactly once they are scaled by powers of two:
//      k^ = k / 4,   q^ = 4 q / sqrt(d_K)
//    so an order-p key feature is phi/4^p and a query feature psi*4^p, which
//    keeps both inside fp16's normal range for inputs of the workloads' scale
//    (|k_i| <= d_K^(1/4)) while the products psi^.phi^ = psi.phi are unchanged.
//    The scan's accumulators hold S^ = S / 4^p (fp32); the state in HBM keeps
//    the plain layout (scaled back when stored).
//  * Features come in positions of 16 quads: 16 prefixes (pairs i1 <= i2,
//    absent indices first) that share an aligned block of four last indices
//    4b + z [hotdry, "Core insight of symmetric tensor decomposition": the
//    sorted-tuple basis; "Hardware optimisation paths and current limits":
//    the hierarchical structure].  An update tile is 16 prefixes x one slot z,
//    so the 16 lanes of a row group read the same key row (an LDS broadcast).
//  * A prepass writes each chunk's operands (k^ and [v | 1] dimension-major,
//    q^ token-major, fp16) as one image that the scan copies into LDS.
//  * Eight wavefronts, two per SIMD: four "update" wavefronts each keep MT
//    positions of the slice's state in accumulators; four "readout"
//    wavefronts each read out a quarter of the chunk's tokens against every
//    feature of the slice from an fp16 copy of the state in LDS, and store
//    fp16 partials scaled by a power of two that follows the number of tokens
//    seen (so they keep fp16's range), one per (chunk, slice); a reduce kernel
//    adds the slices.
//  * The copy is rewritten every R chunks only (R per head size): chunk c is
//    read out against S^(g-1), g = c - c mod R, and the reduce kernel adds the
//    keys of chunks g .. c as direct Taylor terms, exactly as it adds the
//    intra-chunk term.  Both sums are the same quantity split at another
//    token, so the result only differs in rounding.
//
//   [hotdry] blog.hotdry.top, "Symmetry-aware Taylor approximation attention:
//            engineering a constant per-token cost" (2026-02-05).
#include <algorithm>
#include <type_traits>

#include "sata_device.h"
#include "sata_internal.h"
#include "sata_scan_common.h"

namespace sata {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Block index of a quad word of the 16-stream view: its third byte (the view has no three-index
// prefixes), so head sizes up to 128 fit.
__device__ __forceinline__ int qd16_b(uint32_t w) { return (int)((w >> 16) & 0xffu); }

constexpr float kKeyScale = 0.25f;   // k^ = k / 4
constexpr float kQueryScale = 4.0f;  // q^ = 4 q / sqrt(d_K)

// One chunk's operand image (fp16), as the scan holds it in LDS:
//   Kt [D + 2][KS]: k^ by dimension (tokens contiguous), then a row of ones (absent
//                   prefix indices) and a row of zeros (padding prefixes);
//   Vt [D + 2][KS]: v by dimension, then the "+1" row (1 for valid tokens) and zeros;
//   Q  [C][QS]:     q^ by token, then 1 and 0 (absent and padding indices) and padding.
// Rows are padded (KS = C + 8, QS = D + 4 halves) so that 16 lanes reading 16
// different rows at one column do not meet in an LDS bank.  Invalid tokens of a
// ragged last chunk are zero everywhere (also in the "+1" row).
template <int D, int C> struct Img16 {
    static constexpr int KS = C + 8;
    static constexpr int QS = D + 4;
    static constexpr int KT_OFF = 0;
    static constexpr int V_OFF = (D + 2) * KS * 2;
    static constexpr int Q_OFF = V_OFF + (D + 2) * KS * 2;
    static constexpr int BYTES = Q_OFF + C * QS * 2;
    static_assert(BYTES % 16 == 0 && (KS * 2) % 16 == 0, "16-byte units");
};

// The eight values of a 16-byte unit of v as fp16: bf16 words widen exactly and round to fp16
// (exact inside its normal range); binary16 words are taken as they are.
__device__ __forceinline__ void v_unit_f16(const uint4 &u, const bf16_t *, f16 (&out)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        out[2 * e] = (f16)__uint_as_float(w[e] << 16);
        out[2 * e + 1] = (f16)__uint_as_float(w[e] & 0xffff0000u);
    }
}
__device__ __forceinline__ void v_unit_f16(const uint4 &u, const f16 *, f16 (&out)[8]) {
    const f16x8 h = __builtin_bit_cast(f16x8, u);
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = h[e];
}

// Prepass: grid (chunks of the segment, B*H), 256 threads.  Reads the chunk's
// q, k (bf16) and v (bf16, or binary16 for internal callers) once and writes its image; k and v
// are transposed through LDS.
template <int D, int C, typename TV>
__global__ __launch_bounds__(256) void scan16_prepass_kernel(const bf16_t *__restrict__ q, const bf16_t *__restrict__ k,
                                                             const TV *__restrict__ v, int64_t n, int64_t tok0,
                                                             int nchunk, float qscale, int qk_div,
                                                             unsigned char *__restrict__ img) {
    using I = Img16<D, C>;
    constexpr int TS = C + 8;                         // LDS transpose row stride (halves)
    __shared__ __align__(16) f16 tk[D * TS];
    __shared__ __align__(16) f16 tv[D * TS];
    const int cc = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t t0 = tok0 + (int64_t)cc * C;
    const int nv = n - t0 < C ? (int)(n - t0) : C;
    unsigned char *dst = img + ((int64_t)bh * nchunk + cc) * I::BYTES;
    f16 *Kt = reinterpret_cast<f16 *>(dst + I::KT_OFF);
    f16 *Vt = reinterpret_cast<f16 *>(dst + I::V_OFF);
    f16 *Q = reinterpret_cast<f16 *>(dst + I::Q_OFF);
    const int64_t bqk = bh / qk_div;                  // the head whose q and k this head reads
    const bf16_t *qh = q + (bqk * n + t0) * D, *kh = k + (bqk * n + t0) * D;
    const TV *vh = v + (bh * n + t0) * D;
    // 16-byte units of 8 dims: unit i = token i / (D/8), dims 8 (i % (D/8)) ...
    constexpr int UPT = D / 8;
    for (int i = tid; i < C * UPT; i += 256) {
        const int t = i / UPT, d0 = (i % UPT) * 8;
        uint4 uq = {0u, 0u, 0u, 0u}, uk = uq, uv = uq;
        if (t < nv) {
            uq = *reinterpret_cast<const uint4 *>(qh + (int64_t)t * D + d0);
            uk = *reinterpret_cast<const uint4 *>(kh + (int64_t)t * D + d0);
            uv = *reinterpret_cast<const uint4 *>(vh + (int64_t)t * D + d0);
        }
        const uint32_t wq[4] = {uq.x, uq.y, uq.z, uq.w}, wk[4] = {uk.x, uk.y, uk.z, uk.w};
        f16 hv[8];
        v_unit_f16(uv, vh, hv);
        f16x2 hq[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float q0 = __uint_as_float(wq[e] << 16) * qscale, q1 = __uint_as_float(wq[e] & 0xffff0000u) * qscale;
            hq[e] = f16x2{(f16)q0, (f16)q1};
            tk[(d0 + 2 * e) * TS + t] = (f16)(__uint_as_float(wk[e] << 16) * kKeyScale);
            tk[(d0 + 2 * e + 1) * TS + t] = (f16)(__uint_as_float(wk[e] & 0xffff0000u) * kKeyScale);
            tv[(d0 + 2 * e) * TS + t] = hv[2 * e];
            tv[(d0 + 2 * e + 1) * TS + t] = hv[2 * e + 1];
        }
        // Q rows are I::QS halves (not a multiple of 8): two 8-byte stores
        uint2 *qd = reinterpret_cast<uint2 *>(Q + t * I::QS + d0);
        qd[0] = uint2{__builtin_bit_cast(uint32_t, hq[0]), __builtin_bit_cast(uint32_t, hq[1])};
        qd[1] = uint2{__builtin_bit_cast(uint32_t, hq[2]), __builtin_bit_cast(uint32_t, hq[3])};
    }
    for (int t = tid; t < C; t += 256) {
        // dims D, D+1 (constants 1 and 0), D+2, D+3 (padding)
        const f16x2 one_zero = {(f16)1.f, (f16)0.f}, zz = {(f16)0.f, (f16)0.f};
        *reinterpret_cast<uint2 *>(Q + t * I::QS + D) =
            uint2{__builtin_bit_cast(uint32_t, one_zero), __builtin_bit_cast(uint32_t, zz)};
    }
    __syncthreads();
    // Kt and Vt rows: 16-byte units of 8 tokens; row D of Kt is 1, row D of Vt is 1 for
    // valid tokens; rows D + 1 and the padding columns are 0
    constexpr int RU = I::KS / 8;                     // units per row
    for (int i = tid; i < (D + 2) * RU; i += 256) {
        const int r = i / RU, t8 = (i % RU) * 8;
        f16 ok[8], ov[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int t = t8 + e;
            const bool in = t < C;
            if (r < D) {
                ok[e] = in ? tk[r * TS + t] : (f16)0.f;
                ov[e] = in ? tv[r * TS + t] : (f16)0.f;
            } else if (r == D) {
                ok[e] = in ? (f16)1.f : (f16)0.f;
                ov[e] = t < nv ? (f16)1.f : (f16)0.f;
            } else {
                ok[e] = (f16)0.f;
                ov[e] = (f16)0.f;
            }
        }
        *reinterpret_cast<f16x8 *>(Kt + r * I::KS + t8) = f16x8{ok[0], ok[1], ok[2], ok[3], ok[4], ok[5], ok[6], ok[7]};
        *reinterpret_cast<f16x8 *>(Vt + r * I::KS + t8) = f16x8{ov[0], ov[1], ov[2], ov[3], ov[4], ov[5], ov[6], ov[7]};
    }
}

template <int D, int C, int MT>
struct S16Cfg {
    static constexpr int NU = 4, NR = 4, THREADS = 512;   // update and readout wavefronts
    static constexpr int NC = D + 1, NT = (NC + 15) / 16, NTF = NT - 1;   // NTF full tiles + the normaliser tile
    static constexpr int NP = NU * MT;                  // positions (16 quads, 64 features) per slice
    static constexpr int NKS = 2 * NP;                  // readout K steps per slice: two slots of a position
    static constexpr int TT = C / 16, TPW = TT / NR;    // token tiles per chunk, per readout wavefront
    static constexpr int UKS = C / 32;                  // update K steps per chunk
    using I = Img16<D, C>;
    static constexpr int OFF_CP = 0;                                     // copy [NKS][NTF][64] x 16 B
    static constexpr int OFF_CL = OFF_CP + NKS * NTF * 64 * 16;          // normaliser tile [NKS][4] x 16 B, zero entry
    static constexpr int OFF_IMG = OFF_CL + (NKS * 4 + 1) * 16;
    static constexpr int OFF_W0 = OFF_IMG + I::BYTES;                    // quad words [NP][16]
    static constexpr int OFF_QC = OFF_W0 + NP * 16 * 4;                  // quad weights [NP][16] x 4
    static constexpr int OFF_FL = OFF_QC + NP * 16 * 16;                 // position flags [NP]
    static constexpr int LDS = OFF_FL + NP * 4;
    static constexpr int UNITS = I::BYTES / 16;
    static constexpr int UPT = (UNITS + 64 * NR - 1) / (64 * NR);       // image units per readout thread
    static_assert(NC == 16 * NTF + 1, "the last column tile holds the normaliser alone");
    static_assert(C % 64 == 0 && TT % NR == 0 && NKS % 2 == 0 && NKS >= 4, "64, 128 or 256 tokens per chunk");
    static_assert(NP <= 32, "position flags fit a 32-bit mask");
    static_assert(LDS + 128 <= 160 * 1024, "LDS budget (the kernel adds its item record, 112 bytes)");
};

// Order of a quad's prefix (present indices among i1, i2): the feature's order is one more.
template <int D> __device__ __forceinline__ int prefix_order(uint32_t w) {
    return (qd_i1(w) < D ? 1 : 0) + (qd_i2(w) < D ? 1 : 0);
}
// 4^-(order of the feature): the scale between the state and the scan's accumulators.
template <int D> __device__ __forceinline__ float acc_scale(uint32_t w) {
    const int p = prefix_order<D>(w) + 1;
    return p == 1 ? 0.25f : (p == 2 ? 0.0625f : 0.015625f);
}

// Power of two 2^-e with (tokens seen through the chunk) <= 2^e: the fp16 partials of a
// chunk hold y * 2^-e, whose magnitude then follows the inputs' rather than the token count.
__device__ __forceinline__ float partial_scale(float tokens_before, int C) {
    const int e = __builtin_amdgcn_frexp_expf(tokens_before + (float)C);
    return __builtin_amdgcn_ldexpf(1.0f, -e);
}

// Arguments of one scan work item: the run of chunks [cbeg, cend) of head bh, for the slice of
// positions starting at ps0.  gstart / mixedm: bit p set where position ps0 + p starts a
// prefix group / has slots of different weights.
// The record's pointers carry the global address space: read back from LDS they would otherwise
// be generic, and generic (FLAT) accesses also count against the LDS wait counter, so every LDS
// wait would wait for the image prefetch and the partial stores in flight as well.
#define S16_GLOBAL __attribute__((address_space(1)))
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// Word 3 of a raw buffer descriptor on this architecture: 32-bit data format, no swizzle, no
// index stride (loads of whole dwords; the range check uses the descriptor's byte count).
constexpr int kRawBufferWord3 = 0x00020000;

// LDS pointers of the role functions.  Outside a kernel, the dynamic LDS block is found through a
// per-kernel table in global memory; under register pressure the compiler reloads that base
// inside loops, and each reload waits for every global access in flight.  So each role reads
// the base once into a scalar register (opaque to the compiler, so it cannot be re-derived from
// the table) and forms typed LDS pointers (address space 3) from it.
#define S16_LDS __attribute__((address_space(3)))
__device__ __forceinline__ uint32_t s16_lds_base() {
    extern __shared__ __align__(16) unsigned char lds[];
    uint32_t b = (uint32_t)(uintptr_t)(S16_LDS unsigned char *)lds;
    __asm__ volatile("" : "+s"(b));   // opaque: kept in a scalar register, never re-derived
    return b;
}
template <typename T> __device__ __forceinline__ S16_LDS T *s16_lds(uint32_t base, int off) {
    return (S16_LDS T *)(uintptr_t)(base + (uint32_t)off);
}
struct S16Item {
    const S16_GLOBAL int32_t *pcidx;
    S16_GLOBAL float *state;
    int64_t m_pad;
    const S16_GLOBAL unsigned char *img;   // this head's chunk images of the segment
    S16_GLOBAL f16 *partial;
    const S16_GLOBAL float *o0pre;         // this head's order-0 prefixes of the call's chunks
    int64_t chunk0;               // first chunk of the segment within the call
    int64_t pbase;                // partial offset of (head, chunk 0, slice): ((bh nchunk) nslices + slice) ...
    int64_t pstride;              // partial stride per chunk
    int64_t bh, ps0;
    int cbeg, cend;
    int refresh;                  // chunks per refresh of the readout's state copy (cbeg is a multiple)
    uint32_t gstart, mixedm;
};

// Uniform copies of a work item's fields (read from the item record in LDS into scalar registers).
__device__ __forceinline__ int64_t rfl64(int64_t x) {
    return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)((uint64_t)x >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)x));
}
template <typename T> __device__ __forceinline__ T *rflp(T *p) { return reinterpret_cast<T *>(rfl64((int64_t)p)); }
__device__ __forceinline__ S16Item item_from_lds(const S16Item *s) {
    S16Item it;
    it.pcidx = rflp(s->pcidx);
    it.state = rflp(s->state);
    it.m_pad = rfl64(s->m_pad);
    it.img = rflp(s->img);
    it.partial = rflp(s->partial);
    it.o0pre = rflp(s->o0pre);
    it.chunk0 = rfl64(s->chunk0);
    it.pbase = rfl64(s->pbase);
    it.pstride = rfl64(s->pstride);
    it.bh = rfl64(s->bh);
    it.ps0 = rfl64(s->ps0);
    it.cbeg = __builtin_amdgcn_readfirstlane(s->cbeg);
    it.cend = __builtin_amdgcn_readfirstlane(s->cend);
    it.refresh = __builtin_amdgcn_readfirstlane(s->refresh);
    it.gstart = (uint32_t)__builtin_amdgcn_readfirstlane((int)s->gstart);
    it.mixedm = (uint32_t)__builtin_amdgcn_readfirstlane((int)s->mixedm);
    return it;
}

// The two roles of a work item, each compiled on its own (not inlined into the kernel), so that
// the register allocator sizes each role's live values separately instead of holding the union
// of both across the kernel.  Each role derives its wavefront index (uniform, a scalar register,
// so loop bounds and branches on it stay scalar) and its lane itself.

// Readout wavefront rw: token tiles TPW rw .. of the chunk, against every feature of the slice.
// Per chunk: Y = psi(Q_c)[tiles] . S^(c-1)[slice, :] from the fp16 state copy, with the K step's
// B operand loaded one step ahead (two register buffers), then the tiles stored as fp16
// partials.  Also stages each next chunk's image through its registers.
template <int D, int C, int MT>
__device__ __attribute__((noinline)) void scan16_readout(const S16Item *sit) {
    const S16Item it = item_from_lds(sit);
    const int rw = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int lane = __lane_id();
    using Cfg = S16Cfg<D, C, MT>;
    using I = typename Cfg::I;
    constexpr int NR = Cfg::NR, NC = Cfg::NC, NT = Cfg::NT, NTF = Cfg::NTF, NKS = Cfg::NKS;
    constexpr int TPW = Cfg::TPW, UPT = Cfg::UPT, QS = I::QS;
    const uint32_t lb = s16_lds_base();
    const S16_LDS u32x4 *CP = s16_lds<const u32x4>(lb, Cfg::OFF_CP);
    const S16_LDS u32x4 *CL = s16_lds<const u32x4>(lb, Cfg::OFF_CL);
    const S16_LDS f16 *Qs = s16_lds<const f16>(lb, Cfg::OFF_IMG + I::Q_OFF);
    const S16_LDS uint32_t *W0 = s16_lds<const uint32_t>(lb, Cfg::OFF_W0);
    const int g = lane >> 4, li = lane & 15;
    const int tbase = rw * TPW;               // first token tile of this wave
    const int rtid = rw * 64 + lane;          // 0 .. 64 NR - 1
    uint4 pre[UPT];
    auto fetch = [&](int cc) {
        // buffer loads: the chunk's image in a descriptor (uniform), one 32-bit offset per lane
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(it.img + (int64_t)cc * I::BYTES), 0, I::BYTES, kRawBufferWord3);
        const int v0 = rtid * 16;
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            // every lane loads (in the last pass the lanes past the image repeat its final unit,
            // which stage() skips): a fixed number of loads in flight lets later waits count
            // past them instead of draining all
            if ((i + 1) * 64 * NR <= Cfg::UNITS) {
                pre[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, v0, i * 64 * NR * 16, 0));
            } else {
                const int un = rtid + i * 64 * NR;
                const int off = (un < Cfg::UNITS ? un : Cfg::UNITS - 1) * 16;
                pre[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
            }
        }
    };
    auto stage = [&]() {
        S16_LDS u32x4 *dst = s16_lds<u32x4>(lb, Cfg::OFF_IMG);
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const int un = rtid + i * 64 * NR;
            if (un < Cfg::UNITS) dst[un] = __builtin_bit_cast(u32x4, pre[i]);
        }
    };
    // loads are issued every chunk (chunk indices clamped to the item's last), so each iteration
    // has the same loads in flight and the waits for them count exactly
    const int clast_chunk = it.cend - 1;
    fetch(it.cbeg);
    stage();
    fetch(it.cbeg + 1 < it.cend ? it.cbeg + 1 : clast_chunk);
    __syncthreads();   // Y: image of the first chunk and the first copy written

    f32x4 Y[TPW][NT];
    const S16_LDS f16 *qrow[TPW];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) qrow[tt] = Qs + (16 * (tbase + tt) + li) * QS;
    const S16_LDS u32x4 *clast = li == 0 ? CL + g : CL + Cfg::NKS * 4;   // normaliser lanes, else the zero entry
    const int clast_step = li == 0 ? 4 : 0;
    // Token count before each chunk (the normaliser entry of its order-0 prefix), loaded one
    // chunk ahead through the vector memory path (a lane-opaque offset keeps it off the scalar
    // cache, whose wait would also stall every LDS wait in between).
    int opq = 0;
    __asm__ volatile("" : "+v"(opq));
    auto count_before = [&](int cc) { return it.o0pre[(it.chunk0 + cc) * NC + D + opq]; };
    float cnt_next = count_before(it.cbeg);
    // partials: [chunk][TT][NC][16 tokens] fp16 per (head, slice)
    // (tile indices stay compile-time constants: a runtime index into Y would put it in scratch)
    auto store_partials = [&](int cc, float cnt) {
        const float sc = partial_scale(cnt, C);
        S16_GLOBAL f16 *pd = it.partial + it.pbase + cc * it.pstride + (int64_t)tbase * NC * 16 + (li * 16 + 4 * g);
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                if (nt < NTF || li == 0) {
                    const f16x2 a = {(f16)(Y[tt][nt][0] * sc), (f16)(Y[tt][nt][1] * sc)};
                    const f16x2 b = {(f16)(Y[tt][nt][2] * sc), (f16)(Y[tt][nt][3] * sc)};
                    *reinterpret_cast<S16_GLOBAL u32x2 *>(pd + (tt * NC + 16 * nt) * 16) =
                        u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
                }
            }
    };
    // prefix factors of the lane's four streams (4g .. 4g+3) for its token in each tile
    f16x2 pc[TPW][2];
    auto regroup = [&](int p) {
        const S16_LDS uint32_t *wp = W0 + p * 16 + 4 * g;
        uint32_t w[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = wp[r];
        f16x2 cw[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
            cw[h] = f16x2{(f16)qd_pweight<D, false>(w[2 * h]), (f16)qd_pweight<D, false>(w[2 * h + 1])};
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const f16x2 x1 = {qrow[tt][qd_i1(w[2 * h])], qrow[tt][qd_i1(w[2 * h + 1])]};
                const f16x2 x2 = {qrow[tt][qd_i2(w[2 * h])], qrow[tt][qd_i2(w[2 * h + 1])]};
                pc[tt][h] = x1 * x2 * cw[h];
            }
        }
    };
    // B operand of K step kk: the NTF tiles of the state copy and the normaliser entry
    auto loadB = [&](int kk, f16x8 (&B)[NT]) {
#pragma unroll
        for (int nt = 0; nt < NTF; ++nt) B[nt] = __builtin_bit_cast(f16x8, CP[(kk * NTF + nt) * 64 + lane]);
        B[NTF] = __builtin_bit_cast(f16x8, clast[kk * clast_step]);
    };
    // first last index (4 x block) of each position of the slice, read once per item into scalar
    // registers (an LDS read per K step would wait for the B prefetch in flight as well)
    int xb[Cfg::NP];
#pragma unroll
    for (int p = 0; p < Cfg::NP; ++p) xb[p] = __builtin_amdgcn_readfirstlane(4 * qd16_b(W0[p * 16]));
    // A operand of K step kk for each token tile (LDS reads of the query image, and the prefix
    // factors regrouped where a position starts)
    auto formA = [&](int kk, f16x8 (&A)[TPW], auto first) {
        const int p = kk >> 1, h = kk & 1;
        if (first || (h == 0 && ((it.gstart >> p) & 1u))) {
            __asm__ volatile("" ::: "memory");
            regroup(p);
        }
        const int xo = xb[p] + 2 * h;
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const f16x2 x = *reinterpret_cast<const S16_LDS f16x2 *>(qrow[tt] + xo);
            const f16x2 xl = {x[0], x[0]}, xh = {x[1], x[1]};
            const f16x2 a0 = pc[tt][0] * xl, a1 = pc[tt][1] * xl, a2 = pc[tt][0] * xh, a3 = pc[tt][1] * xh;
            A[tt] = f16x8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
        }
    };
    // the MFMAs of one K step: the first of a chunk starts the accumulators from zero (the
    // MFMA's constant operand), every other adds to them
    auto mma = [&](const f16x8 (&A)[TPW], const f16x8 (&B)[NT], auto first) {
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                Y[tt][nt] = mfma_f16(A[tt], B[nt], first ? f32x4{0.f, 0.f, 0.f, 0.f} : Y[tt][nt]);
    };
    for (int cc = it.cbeg; cc < it.cend; ++cc) {
        const float cnt_cur = cnt_next;
        cnt_next = count_before(cc + 1 < it.cend ? cc + 1 : clast_chunk);
        // ---- phase A: readout of chunk cc against S^(c-1).  Even K steps take their B operand
        // from Ba, odd ones from Bb; the next step's is read after the current step's A operand
        // (LDS reads complete in order, so waiting for A does not wait for the prefetch).
        f16x8 Ba[NT], Bb[NT], A[TPW];
        loadB(0, Ba);
        formA(0, A, std::true_type{});
        loadB(1, Bb);
        mma(A, Ba, std::true_type{});
#pragma unroll
        for (int kk = 1; kk + 2 < NKS; kk += 2) {
            formA(kk, A, std::false_type{});
            loadB(kk + 1, Ba);
            mma(A, Bb, std::false_type{});
            formA(kk + 1, A, std::false_type{});
            loadB(kk + 2, Bb);
            mma(A, Ba, std::false_type{});
        }
        formA(NKS - 1, A, std::false_type{});
        mma(A, Bb, std::false_type{});
        store_partials(cc, cnt_cur);
        __syncthreads();   // X: copy and image free
        // ---- phase B: stage the next chunk
        if (cc + 1 < it.cend) stage();
        fetch(cc + 2 < it.cend ? cc + 2 : clast_chunk);
        __syncthreads();   // Y: next image and copy written
    }
}

// Update wavefront uw: positions p0 = MT uw .. of the slice, their state in accumulators
// (S^ = S / 4^p).  Per chunk: S += phi(K_c)^T [V_c | 1] on fp16 MFMA, then the fp16 copy of the
// new state for the readout wavefronts.
template <int D, int C, int MT>
__device__ __attribute__((noinline)) void scan16_update(const S16Item *sit) {
    const S16Item it = item_from_lds(sit);
    const int uw = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) - S16Cfg<D, C, MT>::NR;
    const int lane = __lane_id();
    using Cfg = S16Cfg<D, C, MT>;
    using I = typename Cfg::I;
    constexpr int NC = Cfg::NC, NT = Cfg::NT, NTF = Cfg::NTF, UKS = Cfg::UKS, KS = I::KS;
    const uint32_t lb = s16_lds_base();
    S16_LDS u32x4 *CP = s16_lds<u32x4>(lb, Cfg::OFF_CP);
    S16_LDS u32x4 *CL = s16_lds<u32x4>(lb, Cfg::OFF_CL);
    const S16_LDS f16 *Kt = s16_lds<const f16>(lb, Cfg::OFF_IMG + I::KT_OFF);
    const S16_LDS f16 *Vt = s16_lds<const f16>(lb, Cfg::OFF_IMG + I::V_OFF);
    const S16_LDS uint32_t *W0 = s16_lds<const uint32_t>(lb, Cfg::OFF_W0);
    const S16_LDS f32x4 *QC = s16_lds<const f32x4>(lb, Cfg::OFF_QC);
    const int g = lane >> 4, li = lane & 15;
    const int p0 = uw * MT;
    S16_GLOBAL float *Sh = it.state + it.bh * NC * it.m_pad;
    f32x4 S[MT][4][NT];
    uint32_t wr[MT];                          // quad word of the lane's prefix (row li) per position
    int blk[MT];
    uint32_t newgrp = 0;
#pragma unroll
    for (int j = 0; j < MT; ++j) {
        wr[j] = W0[(p0 + j) * 16 + li];
        blk[j] = __builtin_amdgcn_readfirstlane(qd16_b(W0[(p0 + j) * 16]));
        if ((it.gstart >> (p0 + j)) & 1u) newgrp |= 1u << j;
    }
    // State element (row c, feature f) of the lane's prefix 4g + r at position p0 + j, slot z:
    // c = 16 nt + li, f = cidx + z - z0.  Column tiles are a uniform stride apart, so a quad's
    // NT x 4 elements share one lane offset; loads and stores go one quad at a time.
    const int64_t tstride = (int64_t)16 * it.m_pad;
    auto quad_at = [&](int j, int r, int &off, uint32_t &vmask, float &sc) {
        const uint32_t w = W0[(p0 + j) * 16 + 4 * g + r];
        const int32_t c0 = it.pcidx[(it.ps0 + p0 + j) * 16 + 4 * g + r];
        const uint32_t mask = qd_mask(w);
        const int z0 = mask ? __builtin_ctz(mask) : 0;
        off = mask ? li * (int)it.m_pad + c0 - z0 : 0;
        vmask = mask;
        sc = acc_scale<D>(w);
    };
    // state -> accumulators: lane (li, g) holds rows 4g + r (prefix 4g + r) of column 16 nt + li
#pragma unroll
    for (int j = 0; j < MT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int off;
            uint32_t vm;
            float sc;
            quad_at(j, r, off, vm, sc);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                // rows past the normaliser (columns 16 nt + li > d_V) and padding quads read the
                // head's first element instead, and the value is dropped: every address stays
                // inside this head's state
                const bool cok = 16 * nt + li < NC;
                const S16_GLOBAL float *rp = Sh + (cok ? nt * tstride + off : 0);
#pragma unroll
                for (int z = 0; z < 4; ++z) {
                    const bool ok = ((vm >> z) & 1u) && cok;
                    const float x = rp[ok ? z : 0];
                    S[j][z][nt][r] = ok ? x * sc : 0.f;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    // accumulators -> fp16 copy: K step 2 (p0 + j) + h holds slots 2h, 2h + 1 of position p0 + j;
    // the lane's 16 bytes are rows 4g .. 4g+3 of both slots, column li.  Slots of a group's first
    // position carry their weight relative to the prefix weight (0 for invalid slots).
    auto copy_position = [&](int j, auto scaled) {
        float rt[4][4];                       // [r][z]
        if constexpr (scaled) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t w = W0[(p0 + j) * 16 + 4 * g + r];
                const f32x4 cf = QC[(p0 + j) * 16 + 4 * g + r];
                const float pf = qd_pfact<D, false>(w);
#pragma unroll
                for (int z = 0; z < 4; ++z) rt[r][z] = cf[z] * pf;
            }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                f32x4 s0 = S[j][2 * h][nt], s1 = S[j][2 * h + 1][nt];
                if constexpr (scaled) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        s0[r] *= rt[r][2 * h];
                        s1[r] *= rt[r][2 * h + 1];
                    }
                }
                const f16x2 e0 = {(f16)s0[0], (f16)s0[1]}, e1 = {(f16)s0[2], (f16)s0[3]};
                const f16x2 e2 = {(f16)s1[0], (f16)s1[1]}, e3 = {(f16)s1[2], (f16)s1[3]};
                const u32x4 val = {__builtin_bit_cast(uint32_t, e0), __builtin_bit_cast(uint32_t, e1),
                                   __builtin_bit_cast(uint32_t, e2), __builtin_bit_cast(uint32_t, e3)};
                const int kk = 2 * (p0 + j) + h;
                if (nt < NTF) CP[(kk * NTF + nt) * 64 + lane] = val;
                else if (li == 0) CL[kk * 4 + g] = val;
            }
    };
    // (the branch is per position and uniform: one straight run of conversions and stores each way)
    auto write_copy = [&]() {
#pragma unroll
        for (int j = 0; j < MT; ++j) {
            if ((it.mixedm >> (p0 + j)) & 1u) copy_position(j, std::true_type{});
            else copy_position(j, std::false_type{});
        }
    };
    write_copy();
    __syncthreads();   // Y: image of the first chunk and the first copy written

    const int vlast = li == 0 ? D : D + 1;    // the "+1" row for column D, zeros for the rest
    int until_refresh = it.refresh;           // chunks left before the copy is rewritten
    // B operand of K step ks (32 tokens): the [V | 1] rows of the image
    auto loadB = [&](int ks, f16x8 (&B)[NT]) {
        const int tb = 32 * ks + 8 * g;
#pragma unroll
        for (int nt = 0; nt < NTF; ++nt) B[nt] = *reinterpret_cast<const S16_LDS f16x8 *>(Vt + (16 * nt + li) * KS + tb);
        B[NTF] = *reinterpret_cast<const S16_LDS f16x8 *>(Vt + vlast * KS + tb);
    };
    // one K step on operand B; the next step's B is read into Bn once this step's prefix reads
    // are out (LDS reads complete in order, so the waits for this step's keys do not wait for it)
    auto kstep = [&](int ks, const f16x8 (&B)[NT], f16x8 (&Bn)[NT]) {
        const int tb = 32 * ks + 8 * g;
        f16x8 p2;
#pragma unroll
        for (int j = 0; j < MT; ++j) {
            if (j == 0 || ((newgrp >> j) & 1u)) {
                __asm__ volatile("" ::: "memory");
                const f16x8 a = *reinterpret_cast<const S16_LDS f16x8 *>(Kt + qd_i1(wr[j]) * KS + tb);
                const f16x8 b = *reinterpret_cast<const S16_LDS f16x8 *>(Kt + qd_i2(wr[j]) * KS + tb);
                p2 = a * b;
            }
            f16x8 k3[4];
#pragma unroll
            for (int z = 0; z < 4; ++z) k3[z] = *reinterpret_cast<const S16_LDS f16x8 *>(Kt + (4 * blk[j] + z) * KS + tb);
            if (j == MT - 1 && ks + 1 < UKS) loadB(ks + 1, Bn);
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                const f16x8 A = p2 * k3[z];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) S[j][z][nt] = mfma_f16(A, B[nt], S[j][z][nt]);
            }
        }
    };
    static_assert(UKS % 2 == 0, "K steps pair up over the two B buffers");
    for (int cc = it.cbeg; cc < it.cend; ++cc) {
        // ---- phase A: S[slice, :] += phi(K_c)[:, slice]^T [V_c | 1], the K steps unrolled (their
        // B buffers alternate; a rolled loop would carry them and copy the accumulators)
        f16x8 Ba[NT], Bb[NT];
        loadB(0, Ba);
#pragma unroll
        for (int ks = 0; ks < UKS; ks += 2) {
            kstep(ks, Ba, Bb);
            kstep(ks + 1, Bb, Ba);
        }
        __syncthreads();   // X
        // the copy the readout reads is S^(c-1) only after chunks whose index within the segment is a
        // multiple of it.refresh; the readout of the chunks in between uses that older state, and the
        // reduce kernel adds their keys since then as direct terms
        if (--until_refresh == 0) {
            until_refresh = it.refresh;
            if (cc + 1 < it.cend) write_copy();
        }
        __syncthreads();   // Y
    }
    // accumulators -> state slice (plain layout)
#pragma unroll
    for (int j = 0; j < MT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int off;
            uint32_t vm;
            float sc;
            quad_at(j, r, off, vm, sc);
            sc = 1.0f / sc;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                S16_GLOBAL float *rp = Sh + nt * tstride + off;
                if (16 * nt + li < NC) {
#pragma unroll
                    for (int z = 0; z < 4; ++z)
                        if ((vm >> z) & 1u) rp[z] = S[j][z][nt][r] * sc;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
}

// Persistent scan: a grid of one workgroup per resident slot takes (sub-segment u, head, slice)
// items from one of kScanQueues counters, u-major; an item continues the state its predecessor
// (u - 1, head, slice) left, after an agent-scope acquire of that slice's progress flag (bounded
// wait), and releases its own flag once every wavefront's state stores are out.  The predecessor
// sits in the same queue, earlier, so a running workgroup has taken it.  Wavefronts 0..3 read out,
// 4..7 update (one of each per SIMD).
template <int D, int C, int MT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void scan16_kernel(const uint32_t *__restrict__ pw0, const int32_t *__restrict__ pcidx,
                   const float4 *__restrict__ pcoef, const uint32_t *__restrict__ pflags,
                   float *__restrict__ state, int64_t m_pad, const unsigned char *__restrict__ img, int nchunk,
                   f16 *__restrict__ partial, const float *__restrict__ o0pre, int64_t call_chunks, int64_t chunk0,
                   int nslices, int64_t nbh, int nsub, int sub_chunks, int refresh, uint32_t *__restrict__ sync,
                   int item_base, int spin_limit, uint32_t *err) {
    using Cfg = S16Cfg<D, C, MT>;
    using I = typename Cfg::I;
    constexpr int NP = Cfg::NP;
    extern __shared__ __align__(16) unsigned char lds[];
    uint4 *CL = reinterpret_cast<uint4 *>(lds + Cfg::OFF_CL);
    uint32_t *W0 = reinterpret_cast<uint32_t *>(lds + Cfg::OFF_W0);
    float4 *QC = reinterpret_cast<float4 *>(lds + Cfg::OFF_QC);
    uint32_t *FL = reinterpret_cast<uint32_t *>(lds + Cfg::OFF_FL);
    __shared__ int64_t s_item;
    __shared__ S16Item s_it;                  // the current item's record, read by both roles
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t per_sub = nbh * nslices;
    // Queue q of ngroups serves the (head, slice) pairs [lo, hi) (contiguous, head-major), for
    // every sub-segment, u-major; the workgroups with blockIdx.x % ngroups == q take from it.
    // Workgroups are dispatched to the chip's XCDs in turn, so with ngroups = kScanQueues a
    // queue's workgroups share one XCD and its L2, and the slices of a head walk the same
    // chunk images at the same time.
    const int ngroups = (int)gridDim.x < kScanQueues ? (int)gridDim.x : kScanQueues;
    const int grp = (int)blockIdx.x % ngroups;
    const int64_t lo = per_sub * grp / ngroups, hi = per_sub * (grp + 1) / ngroups;
    const int64_t cnt = hi - lo;
    const int64_t nitems = cnt * nsub;
    uint32_t *counter = sync + grp;
    uint32_t *flags = sync + kScanQueues;   // one per (head, slice): sub-segments finished
    // One thread-0 block per pass, at its end, both releases the finished item and takes
    // the next; a second thread-0 block at the top of the loop would let the compiler
    // thread one branch into the other and leave a loop whose barriers the other
    // threads pass without thread 0, re-reading an item that never changes.
    if (tid == 0) s_item = (int64_t)atomicAdd(counter, 1u) + item_base;
    __syncthreads();
    for (;;) {
        int64_t item = s_item;
        __syncthreads();   // every thread has read the item before thread 0 replaces it
        item = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(item >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((int)item));
        if (item >= nitems) break;
        const int u = (int)(item / cnt);
        const int64_t rem = lo + item % cnt;
        S16Item it;
        it.bh = rem / nslices;
        const int slice = (int)(rem % nslices);
        it.cbeg = u * sub_chunks;
        it.cend = it.cbeg + sub_chunks < nchunk ? it.cbeg + sub_chunks : nchunk;
        it.refresh = refresh;
        if (u > 0) {
            if (tid == 0) wait_predecessor(flags + rem, (uint32_t)u, spin_limit, err);
            __syncthreads();   // thread 0's acquire invalidated the caches every wave reads through
        }
        it.ps0 = (int64_t)slice * NP;
        for (int i = tid; i < NP * 16; i += Cfg::THREADS) {
            W0[i] = pw0[it.ps0 * 16 + i];
            QC[i] = pcoef[it.ps0 * 16 + i];
        }
        for (int i = tid; i < NP; i += Cfg::THREADS) FL[i] = pflags[it.ps0 + i];
        if (tid < 16) CL[Cfg::NKS * 4] = uint4{0u, 0u, 0u, 0u};   // the zero entry
        __syncthreads();
        const int l0 = tid & 63;
        it.gstart = (uint32_t)__ballot(l0 < NP && (FL[l0 < NP ? l0 : 0] & 2u));
        it.mixedm = (uint32_t)__ballot(l0 < NP && (FL[l0 < NP ? l0 : 0] & 1u));
        it.pcidx = (const S16_GLOBAL int32_t *)pcidx;
        it.state = (S16_GLOBAL float *)state;
        it.m_pad = m_pad;
        it.img = (const S16_GLOBAL unsigned char *)(img + it.bh * nchunk * (int64_t)I::BYTES);
        it.partial = (S16_GLOBAL f16 *)partial;
        it.pstride = (int64_t)nslices * (Cfg::TT * Cfg::NC * 16);
        it.pbase = (it.bh * nchunk * nslices + slice) * (int64_t)(Cfg::TT * Cfg::NC * 16);
        it.o0pre = (const S16_GLOBAL float *)(o0pre + it.bh * call_chunks * Cfg::NC);
        it.chunk0 = chunk0;
        if (tid == 0) s_it = it;
        __syncthreads();
        if (wave < Cfg::NR) scan16_readout<D, C, MT>(&s_it);
        else scan16_update<D, C, MT>(&s_it);
        // every wave's stores reach L2 before the barrier; thread 0's agent-scope release then
        // writes L2 back before the flag
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
        __syncthreads();
        if (tid == 0) {
            __hip_atomic_store(&flags[rem], (uint32_t)(u + 1), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            s_item = (int64_t)atomicAdd(counter, 1u) + item_base;
        }
        __syncthreads();
    }
}

// Direct Taylor terms of query tile qt of the chunk starting at token tq0 (fp16 operands)
// against the keys of one chunk starting at token tk0: Z (rows = queries 4g + r, column li of
// each 16-column tile) receives sum_key w(q.k/sqrt d) [v, 1][key], over the keys up to the query
// when the key chunk is the query's own (causal), over all C keys of an earlier chunk (full).
// S^T = K Q^T is formed on bf16 MFMA from q and k as given (exact products, fp32 sums); W = w(S^T)
// is packed to fp16 (w lies in [1/3, e] for |x| <= 1) and multiplies [V | 1] of the key chunk
// (its image rows, fp16, dimension-major, in LDS) on fp16 MFMA.  The accumulator rows of S^T are
// the K slots of the W [V | 1] product, so W never leaves the registers.  With KL the key chunk's
// rows come from LDS (kl: [C][D], zero past the valid keys) instead of global memory.
template <int D, int NT, int KS, int C, bool full, bool KL>
__device__ __forceinline__ void intra_tile16(f32x4 (&Z)[NT], int qt, int g, int li, const bf16_t *qh, const bf16_t *kh,
                                             int64_t tq0, int nvalid, int64_t tk0, const f16 *Vt,
                                             const bf16_t *kl, const TaylorArgs &ta) {
    const int query = 16 * qt + li;
    constexpr int DS = D < 32 ? 1 : D / 32;
    // rows at or past `lim` of the chunk read as zeros (a ragged last chunk)
    auto load8 = [&](const bf16_t *base, int64_t t0, int tok, int lim, int d0) -> bf16x8 {
        uint4 u = {0u, 0u, 0u, 0u};
        if (tok < lim && d0 < D) u = *reinterpret_cast<const uint4 *>(base + (t0 + tok) * D + d0);
        return __builtin_bit_cast(bf16x8, u);
    };
    bf16x8 Bq[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) Bq[s] = load8(qh, tq0, query, nvalid, 32 * s + 8 * g);
    const int klim = full ? C : nvalid;           // an earlier chunk is whole
    auto kstep = [&](int ks) {
        f32x4 sA = {0.f, 0.f, 0.f, 0.f}, sB = {0.f, 0.f, 0.f, 0.f};
        const int kA = 32 * ks + li, kB = kA + 16;
#pragma unroll
        for (int s = 0; s < DS; ++s) {
            if constexpr (KL) {
                const int d0 = 32 * s + 8 * g;
                const uint4 z = {0u, 0u, 0u, 0u};
                const uint4 ua = d0 < D ? *reinterpret_cast<const uint4 *>(kl + kA * D + d0) : z;
                const uint4 ub = d0 < D ? *reinterpret_cast<const uint4 *>(kl + kB * D + d0) : z;
                sA = mfma_bf16(__builtin_bit_cast(bf16x8, ua), Bq[s], sA);
                sB = mfma_bf16(__builtin_bit_cast(bf16x8, ub), Bq[s], sB);
            } else {
                sA = mfma_bf16(load8(kh, tk0, kA, klim, 32 * s + 8 * g), Bq[s], sA);
                sB = mfma_bf16(load8(kh, tk0, kB, klim, 32 * s + 8 * g), Bq[s], sB);
            }
        }
        f16 w8[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int keyA = 32 * ks + 4 * g + r, keyB = keyA + 16;
            w8[r] = (f16)(full || keyA <= query ? taylor_w(sA[r] * ta.scale, ta.c0, ta.c1, ta.c2, ta.c3, ta.c4, ta.P) : 0.f);
            w8[4 + r] = (f16)(full || keyB <= query ? taylor_w(sB[r] * ta.scale, ta.c0, ta.c1, ta.c2, ta.c3, ta.c4, ta.P) : 0.f);
        }
        const f16x8 A = {w8[0], w8[1], w8[2], w8[3], w8[4], w8[5], w8[6], w8[7]};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int row = 16 * nt + li <= D ? 16 * nt + li : D + 1;   // columns past the "+1" read zeros
            const f16 *vr = Vt + row * KS + 32 * ks + 4 * g;
            const uint2 lo = *reinterpret_cast<const uint2 *>(vr);
            const uint2 hi = *reinterpret_cast<const uint2 *>(vr + 16);
            Z[nt] = mfma_f16(A, __builtin_bit_cast(f16x8, uint4{lo.x, lo.y, hi.x, hi.y}), Z[nt]);
        }
    };
    // (rolled loops: an unrolled whole key chunk holds all its key loads at once, and the registers
    // that takes halve the kernel's occupancy)
    const int nks = full ? C / 32 : qt / 2 + 1;
#pragma unroll 1
    for (int ks = 0; ks < nks; ++ks) kstep(ks);
}

// Chunk c of the segment was read out against S^(g-1), g = c - c % refresh (the scan rewrites the
// readout's state copy every refresh chunks), so
// y = (direct Taylor terms of the keys of chunks g .. c, causal in c) + 2^e (sum over slices of the
// fp16 partials, fixed order) + the order-0 prefix before chunk g; o = y[:d_V] / y[d_V] (or
// y[:d_V] when ta.raw; y[d_V] also goes to den_out when given).  Grid (chunks of the segment,
// B*H), 256 threads.
template <int D, int C, typename TOut>
__global__ __launch_bounds__(256) void scan16_reduce_kernel(const f16 *__restrict__ partial, int nslices, int nchunk,
                                                            int64_t n, int64_t tok0, const bf16_t *__restrict__ q,
                                                            const bf16_t *__restrict__ k,
                                                            const unsigned char *__restrict__ img, TOut *__restrict__ out,
                                                            TaylorArgs ta, float *__restrict__ den_out,
                                                            const float *__restrict__ o0pre, int64_t call_chunks,
                                                            int qk_div, int refresh) {
    using I = Img16<D, C>;
    constexpr int NC = D + 1, TT = C / 16, NT = (NC + 15) / 16;
    constexpr int NV8 = TT * NC * 2;                // 16-byte loads (8 halves) per partial
    constexpr int PER = (NV8 + 255) / 256;
    constexpr int SU = 4;                           // slices per round
    __shared__ __align__(16) f16 vt[(D + 2) * I::KS];
    __shared__ __align__(16) float ys[TT * NC * 16];
    // at d_K <= 32 each key chunk of the window is staged in LDS beside its [V | 1] rows (the causal
    // term's key steps then wait on LDS rather than on global loads); at d_K = 64 and 128 the extra
    // LDS would cost the occupancy that the partial sums need
    constexpr bool KL = D <= 32;
    __shared__ __align__(16) bf16_t kls[KL ? C * D : 8];
    const int cc = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, li = lane & 15;
    const int64_t t0 = tok0 + (int64_t)cc * C;
    const int nvalid = n - t0 < C ? (int)(n - t0) : C;
    const int gc = cc - cc % refresh;                                // first chunk of the direct window
    const float *pre = o0pre + (bh * call_chunks + t0 / C) * NC;   // this chunk's order-0 prefix
    const float *pre_g = pre - (int64_t)(cc - gc) * NC;             // ... and the window's
    const float unscale = 1.0f / partial_scale(pre[D], C);

    const f16 *base = partial + (bh * nchunk + cc) * (int64_t)nslices * (TT * NC * 16);
    float acc[PER][8];
#pragma unroll
    for (int j = 0; j < PER; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
    auto add8 = [&](float (&a)[8], const uint4 &u) {
        const f16x8 h = __builtin_bit_cast(f16x8, u);
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] += (float)h[e];
    };
    int s = 0;
    for (; s + SU <= nslices; s += SU) {
        uint4 uu[SU][PER];
#pragma unroll
        for (int r = 0; r < SU; ++r)
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                const int i = tid + 256 * j;
                uu[r][j] = i < NV8 ? *reinterpret_cast<const uint4 *>(base + ((int64_t)(s + r) * NV8 + i) * 8)
                                   : uint4{0u, 0u, 0u, 0u};
            }
#pragma unroll
        for (int r = 0; r < SU; ++r)
#pragma unroll
            for (int j = 0; j < PER; ++j) add8(acc[j], uu[r][j]);
    }
    for (; s < nslices; ++s) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int i = tid + 256 * j;
            if (i < NV8) add8(acc[j], *reinterpret_cast<const uint4 *>(base + ((int64_t)s * NV8 + i) * 8));
        }
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int i = tid + 256 * j;
        if (i < NV8) {
            float4 *d = reinterpret_cast<float4 *>(ys) + 2 * i;
            d[0] = float4{acc[j][0] * unscale, acc[j][1] * unscale, acc[j][2] * unscale, acc[j][3] * unscale};
            d[1] = float4{acc[j][4] * unscale, acc[j][5] * unscale, acc[j][6] * unscale, acc[j][7] * unscale};
        }
    }
    // direct terms, one key chunk of the window at a time: its [V | 1] rows from its image, then
    // every query tile against its keys (tiles t and TT - 1 - t together, balanced over the causal
    // triangle; pairs dealt to the four wavefronts in turn)
    static_assert(TT % 2 == 0 && (TT / 2 <= 4 || TT % 8 == 0), "query tile pairs deal evenly to the wavefronts");
    const bf16_t *qh = q + (bh / qk_div) * n * D, *kh = k + (bh / qk_div) * n * D;
    for (int j = gc; j <= cc; ++j) {
        if (j > gc) __syncthreads();   // the previous key chunk's rows are no longer read
        {
            const uint4 *src = reinterpret_cast<const uint4 *>(img + (bh * nchunk + j) * (int64_t)I::BYTES + I::V_OFF);
            uint4 *dst = reinterpret_cast<uint4 *>(vt);
            for (int i = tid; i < (D + 2) * I::KS / 8; i += 256) dst[i] = src[i];
        }
        if constexpr (KL) {
            const int klim = j < cc ? C : nvalid;   // keys past the last valid token read as zeros
            const uint4 *src = reinterpret_cast<const uint4 *>(kh + (tok0 + (int64_t)j * C) * D);
            uint4 *dst = reinterpret_cast<uint4 *>(kls);
            for (int i = tid; i < C * D / 8; i += 256)
                dst[i] = i / (D / 8) < klim ? src[i] : uint4{0u, 0u, 0u, 0u};
        }
        __syncthreads();
#pragma unroll
        for (int pr = 0; pr < (TT / 2 + 3) / 4; ++pr) {
            const int pair = 4 * pr + wave;   // tiles pair and TT - 1 - pair
            if (pair >= TT / 2) continue;
#pragma unroll
            for (int pass = 0; pass < 2; ++pass) {
                const int qq = pass == 0 ? pair : TT - 1 - pair;
                const int64_t tk0 = tok0 + (int64_t)j * C;
                f32x4 Z[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) Z[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (j < cc) intra_tile16<D, NT, I::KS, C, true, KL>(Z, qq, g, li, qh, kh, t0, nvalid, tk0, vt, kls, ta);
                else intra_tile16<D, NT, I::KS, C, false, KL>(Z, qq, g, li, qh, kh, t0, nvalid, tk0, vt, kls, ta);
                // (each wavefront adds to its own query tiles' rows only)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const int c = 16 * nt + li;
                    if (c < NC) {
                        float4 *pp = reinterpret_cast<float4 *>(ys + (qq * NC + c) * 16 + 4 * g);
                        const float4 o = *pp;
                        *pp = float4{o.x + Z[nt][0], o.y + Z[nt][1], o.z + Z[nt][2], o.w + Z[nt][3]};
                    }
                }
            }
        }
    }
    __syncthreads();
    for (int i = tid; i < C * D; i += 256) {
        const int t = i / D, c = i - t * D;
        if (t < nvalid) {
            const int tt = t >> 4, t16 = t & 15;
            const float y = ys[(tt * NC + c) * 16 + t16] + pre_g[c];
            const float den = ys[(tt * NC + D) * 16 + t16] + pre_g[D];
            out[(bh * n + t0 + t) * D + c] = from_f32<TOut>(ta.raw ? y : y / den);
            if (den_out && c == 0) den_out[bh * n + t0 + t] = den;
        }
    }
}

// ---------------------------------------------------------------- host side

// Positions per update wavefront: as many as its accumulators (MT x 4 slots x column tiles x 4
// registers) allow next to the operands within 256 registers, or one when that many leaves
// fewer (head, slice) work items than compute units (few heads of a small head size: a head's
// chunks run one after another, so only more slices spread it over the chip).
constexpr int scan16_mt_max(int dk) { return dk == 128 ? 1 : dk == 64 ? 2 : dk == 32 ? 3 : 5; }

int scan16_choose_mt(int dk, int64_t np16, int64_t bh, int cus) {
    const int big = scan16_mt_max(dk);
    const int forced = scan_debug().positions;   // a measurement's choice
    if (forced == 1 || forced == big) return forced;
    const int64_t slices = (np16 + 4 * big - 1) / (4 * big);
    return bh * slices >= cus ? big : 1;
}

// Chunks per rewrite of the readout's state copy: the chunks in between are read out against the
// older copy, and the reduce kernel takes their keys as direct terms instead.
int scan16_refresh(int dk, int slices) {
    const int forced = scan_debug().refresh;   // a measurement's choice
    if (forced > 0) return forced;
    // The scan saves a copy phase per slice and chunk, the reduce kernel pays the wider direct
    // window once per head and chunk: with few slices per head (d_K = 16 prefills, the backward's
    // (P - 1)-order passes) the window costs more than it saves.  Otherwise the measured
    // whole-call optimum per head size.
    if (slices < 8) return 1;
    return dk == 64 ? 4 : 8;
}

int64_t scan16_image_bytes(int dk, int chunk) {
    auto b = [&](auto d, auto c) { return (int64_t)Img16<decltype(d)::value, decltype(c)::value>::BYTES; };
    using I16 = std::integral_constant<int, 16>;
    using I32 = std::integral_constant<int, 32>;
    using I64 = std::integral_constant<int, 64>;
    using C64 = std::integral_constant<int, 64>;
    using C128 = std::integral_constant<int, 128>;
    if (dk == 16) return chunk == 64 ? b(I16{}, C64{}) : chunk == 256 ? b(I16{}, std::integral_constant<int, 256>{})
                                                                      : b(I16{}, C128{});
    if (dk == 32) return chunk == 64 ? b(I32{}, C64{}) : b(I32{}, C128{});
    if (dk == 128) return b(std::integral_constant<int, 128>{}, C64{});   // 64-token chunks only
    return chunk == 64 ? b(I64{}, C64{}) : b(I64{}, C128{});
}

template <int D, int C, int MT, typename TOut>
static hipError_t run_scan16(const sata_index *idx, const sata_state *st, const PrefillPlan &plan, const void *q,
                             const void *k, const void *v, void *out, int64_t n, int64_t tok0, int nseg,
                             const float *o0pre, const TaylorArgs &ta, hipStream_t stream) {
    using Cfg = S16Cfg<D, C, MT>;
    const int64_t bh = (int64_t)st->batch * st->heads;
    auto scan = scan16_kernel<D, C, MT>;
    hipError_t e = hipFuncSetAttribute((const void *)scan, hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS);
    if (e != hipSuccess) return e;
    char *work = static_cast<char *>(st->d_work);
    f16 *partial = reinterpret_cast<f16 *>(work);
    uint32_t *sync = reinterpret_cast<uint32_t *>(work + plan.sync_off);
    unsigned char *img = reinterpret_cast<unsigned char *>(work + plan.img_off);
    const int64_t call_chunks = (n + C - 1) / C;
    const int64_t chunk0 = tok0 / C;
    if (plan.v_f16)
        hipLaunchKernelGGL((scan16_prepass_kernel<D, C, f16>), dim3((unsigned)nseg, (unsigned)bh), dim3(256), 0, stream,
                           static_cast<const bf16_t *>(q), static_cast<const bf16_t *>(k), static_cast<const f16 *>(v),
                           n, tok0, nseg, ta.scale * kQueryScale, plan.qk_div, img);
    else
        hipLaunchKernelGGL((scan16_prepass_kernel<D, C, bf16_t>), dim3((unsigned)nseg, (unsigned)bh), dim3(256), 0,
                           stream, static_cast<const bf16_t *>(q), static_cast<const bf16_t *>(k),
                           static_cast<const bf16_t *>(v), n, tok0, nseg, ta.scale * kQueryScale, plan.qk_div, img);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    int cus = 0, per_cu = 0;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, st->device)) != hipSuccess) return e;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, scan, Cfg::THREADS, Cfg::LDS)) != hipSuccess) return e;
    const int64_t resident = (int64_t)std::max(cus, 1) * std::max(per_cu, 1);
    const int64_t items0 = bh * plan.slices;
    const int refresh = scan16_refresh(D, plan.slices);
    // sub-segments of at least 64 chunks until there are about a dozen items per resident workgroup;
    // each a whole number of copy refresh intervals.  (Measured: each item loads and stores its
    // state slice and waits for its predecessor; 4 sub-segments per slice beat 8 at d_K = 32 by 6%
    // and more than 4 lose at d_K = 64.)
    int nsub = items0 <= cus ? 1 : (int)std::min<int64_t>((12 * resident + items0 - 1) / items0, std::max(1, nseg / 64));
    const int sub_chunks = ((nseg + nsub - 1) / nsub + refresh - 1) / refresh * refresh;
    nsub = (nseg + sub_chunks - 1) / sub_chunks;
    const int64_t grid = std::min<int64_t>(items0 * nsub, resident);
    if ((e = launch_zero(reinterpret_cast<float *>(sync), plan.sync_words, stream)) != hipSuccess) return e;
    const ScanDebug dbg = scan_debug();
    {
        ProfScope ps(kProfScan, stream);
        hipLaunchKernelGGL(scan, dim3((unsigned)grid), dim3(Cfg::THREADS), Cfg::LDS, stream, idx->d_p16_w0,
                           idx->d_p16_cidx, reinterpret_cast<const float4 *>(idx->d_p16_coef), idx->d_p16_flags,
                           static_cast<float *>(st->d_state), idx->m_pad, img, nseg, partial, o0pre, call_chunks, chunk0,
                           plan.slices, bh, nsub, sub_chunks, refresh, sync, dbg.item_base, dbg.spin_limit,
                           st->d_err);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {
        ProfScope ps(kProfCombine, stream);
        hipLaunchKernelGGL((scan16_reduce_kernel<D, C, TOut>), dim3((unsigned)nseg, (unsigned)bh), dim3(256), 0, stream,
                           partial, plan.slices, nseg, n, tok0, static_cast<const bf16_t *>(q),
                           static_cast<const bf16_t *>(k), img, static_cast<TOut *>(out), ta, plan.den_out, o0pre,
                           call_chunks, plan.qk_div, refresh);
    }
    return hipGetLastError();
}

hipError_t launch_scan16_segment(const sata_index *idx, const sata_state *st, const PrefillPlan &plan, const void *q,
                                 const void *k, const void *v, void *out, int64_t n, int64_t tok0, int nseg,
                                 const float *o0pre, const TaylorArgs &ta, sata_dtype out_dt, hipStream_t stream) {
    auto go = [&](auto dw, auto cw) -> hipError_t {
        constexpr int DD = decltype(dw)::value, CC = decltype(cw)::value, MX = scan16_mt_max(DD);
        if (plan.mt == MX) {
            if (out_dt == SATA_F32)
                return run_scan16<DD, CC, MX, float>(idx, st, plan, q, k, v, out, n, tok0, nseg, o0pre, ta, stream);
            return run_scan16<DD, CC, MX, bf16_t>(idx, st, plan, q, k, v, out, n, tok0, nseg, o0pre, ta, stream);
        }
        if (plan.mt != 1) return hipErrorInvalidValue;   // never planned
        if (out_dt == SATA_F32)
            return run_scan16<DD, CC, 1, float>(idx, st, plan, q, k, v, out, n, tok0, nseg, o0pre, ta, stream);
        return run_scan16<DD, CC, 1, bf16_t>(idx, st, plan, q, k, v, out, n, tok0, nseg, o0pre, ta, stream);
    };
    using C64 = std::integral_constant<int, 64>;
    using C128 = std::integral_constant<int, 128>;
    switch (idx->dk) {
        case 16:
            if (plan.chunk == 256) return go(std::integral_constant<int, 16>{}, std::integral_constant<int, 256>{});
            return plan.chunk == 64 ? go(std::integral_constant<int, 16>{}, C64{}) : go(std::integral_constant<int, 16>{}, C128{});
        case 32: return plan.chunk == 64 ? go(std::integral_constant<int, 32>{}, C64{}) : go(std::integral_constant<int, 32>{}, C128{});
        case 64: return plan.chunk == 64 ? go(std::integral_constant<int, 64>{}, C64{}) : go(std::integral_constant<int, 64>{}, C128{});
        case 128: return plan.chunk == 64 ? go(std::integral_constant<int, 128>{}, C64{}) : hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sata
