// Internal declarations shared by the host side of libsata and its kernels.
//
// Feature numbering and the packed tuple table
//   Features run order by order, p = 0..P-1; within an order they are the
//   sorted index tuples i_1 <= ... <= i_p over [0, d_K) in lexicographic order
//   (last index fastest) [hotdry, "Core insight of symmetric tensor
//   decomposition"; "Hardware optimisation paths and current limits" for the
//   nested i_1 <= ... <= i_p structure].  Each feature is packed in one 32-bit
//   word: bytes 0..2 are the tuple's indices, byte 3 its order.  Unused index
//   slots (orders below 3) hold d_K, which the kernels map to the constant 1;
//   padding features (f >= m) hold d_K + 1 in every slot, mapped to 0, so their
//   monomial vanishes.  Orders up to 3 (P <= 4) fit.
//
//   [hotdry] blog.hotdry.top, "Symmetry-aware Taylor approximation attention:
//            engineering a constant per-token cost" (2026-02-05).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <utility>
#include <vector>

#include "../../include/sata.h"

// Largest decode window: deferred tokens held per head before a fold.
constexpr int kMaxDecodeWindow = 64;

struct sata_index {
    int dk = 0, dv = 0, P = 0;
    int64_t m = 0;       // C(d_K+P-1, P-1)
    int64_t m_pad = 0;   // state row stride (multiple of 64)
    int64_t m_tab = 0;   // table length (multiple of kTablePad, covers every kernel's tail)
    int device = 0;
    int cus = 256;       // compute units of the device (work-item counts are planned against it)
    uint32_t *d_tup = nullptr;   // [m_tab] packed tuples: i1 | i2 << 8 | i3 << 16 | i4 << 24
    float *d_coef = nullptr;     // [m_tab] query-side readout weight 1/(alpha! d_K^(p/2)); 0 for padding
    float taylor[8] = {0};       // 1/p!, p < P (intra-chunk direct weights)
    // Prefill-side "pair-quad" view of the same features (see build_quads):
    // quads come in positions of four (one per stream), position-major.
    int64_t nq = 0;              // quads (4 per position)
    int64_t nq_tab = 0;          // quad table length (padded)
    uint32_t *d_qw0 = nullptr;   // [nq_tab] i1 | i2 << 8 | i0 << 16 | b << 24 | mask << 28
    int32_t *d_qcidx = nullptr;  // [nq_tab] state index of the first valid slot (-1: none)
    float *d_qcoef = nullptr;    // [nq_tab][4] query-side weights per slot (0: invalid)
    uint32_t *d_qflags = nullptr;   // [nq_tab / 4] per position: bit 0 mixed weights, bit 1 new pair group
    // The same features in positions of 16 quads (16 streams sharing a block), for the
    // fp16-operand scan: np16 positions, each [16] quad words, state indices and [16][4]
    // weights, plus a flag word; kPos16Pad padding positions follow.  Built for P <= 4 and
    // 16 <= d_K <= 128 (np16 = 0 otherwise).
    int64_t np16 = 0;
    uint32_t *d_p16_w0 = nullptr;
    int32_t *d_p16_cidx = nullptr;
    float *d_p16_coef = nullptr;
    uint32_t *d_p16_flags = nullptr;
    // The index of the same head sizes with P - 1 orders (the backward's dk and dq passes),
    // built by the first backward call that needs it and freed with this index.
    mutable sata_index *lower = nullptr;
    mutable std::mutex lower_mu;
    // Device temporaries of the backward calls on this index (pointer, bytes), kept between calls
    // and freed with the index: request i of a call reuses buffer i when it is large enough, and a
    // larger request replaces it.  bw_mu serialises the backward calls on the index.
    mutable std::vector<std::pair<void *, size_t>> bw_pool;
    mutable std::mutex bw_mu;
};

struct sata_state {
    const sata_index *idx = nullptr;
    int batch = 0, heads = 0;
    int device = 0;
    sata_dtype dtype = SATA_F32; // element type of the state
    void *d_state = nullptr;     // [B*H][d_V+1][m_pad] of dtype
    int64_t state_bytes = 0;
    // SATA_F16 states: features f < m_low (the lowest orders, a multiple of 64) are held in
    // fp32 at d_low [B*H][d_V+1][m_low], right after the fp16 array (whose slots for them
    // stay zero); 0 and NULL for the other types
    int64_t m_low = 0;
    float *d_low = nullptr;
    void *d_work = nullptr;      // prefill / decode partial sums (grown on demand)
    int64_t work_bytes = 0;
    int window = 1;              // decode steps per state update (1: every step)
    int npend = 0;               // deferred tokens not yet in d_state (host-side count, < window)
    float *d_pend_k = nullptr;   // [B*H][kMaxDecodeWindow][d_K] deferred keys (fp32)
    float *d_pend_v = nullptr;   // [B*H][kMaxDecodeWindow][d_V] deferred values (fp32)
    // Error word of the asynchronous work on this state, in pinned host memory that the
    // device writes (d_err is its device address): bit 0 = a prefill scan item gave up
    // waiting for its predecessor's state (the output and state of that call are invalid).
    // Checked, and cleared, by the next call on the state and by sata_state_check.
    uint32_t *h_err = nullptr;
    uint32_t *d_err = nullptr;
};

namespace sata {

constexpr int kTablePad = 2048;          // tables cover every slice up to this granularity
constexpr int kQuadPad = 1024;           // quad tables cover every prefill slice up to this granularity
constexpr int kPos16Pad = 64;            // padding positions after the 16-stream table (> any slice)
constexpr int kScanQueues = 8;           // work queues of the fp16-operand scan (one per XCD)

// Prefill feature view.  The features of orders 1..P-1 are grouped into
// "quads": a prefix (i0, i1, i2), sorted, any of which may be absent (absent
// ones come first), and an aligned block of four last indices 4b + z,
// z = 0..3; slot z is a feature when the tuple (prefix, 4b+z) is sorted, else
// padding.  Quads come in positions of four whose prefixes sweep the same
// blocks side by side (see build_quads), so the block b is common to a
// position.  Absent indices point at the constant-1 slot (d_K), padding quads
// at the constant-0 slot (d_K+1).  Order 0 has no quad.  b < 16 and the slot
// mask share the top byte of the quad word, so d_K <= 64.
struct QuadRec {
    uint32_t w0;
    int32_t cidx;
    float coef[4];
};
constexpr int kMaxOrder = 4;             // P <= 5: four index slots per feature tuple

// ---- launchers (defined in the .hip files) --------------------------------

// Decode: one token per head.  Returns hipSuccess or the launch error.
// Decode launches: a plain step (update by the step's token, read out), a
// deferred step's readout of the state as it stands (direct terms for the
// pending tokens and the step's own), a fold (update by the pending tokens and
// the step's own, read out), or a flush (update by the pending tokens only).
enum DecodeMode { kDecodePlain, kDecodeRead, kDecodeFold, kDecodeFlush };
hipError_t launch_decode(const sata_index *idx, const sata_state *st, const void *q, const void *k,
                         const void *v, void *out, sata_dtype in_dt, sata_dtype out_dt, DecodeMode mode,
                         hipStream_t stream);
int64_t decode_workspace_bytes(const sata_index *idx, int64_t bh);
// Prefill in blocks of up to kMaxDecodeWindow tokens through the state in HBM (d_K = d_V = 128,
// fp32 state): needs the pending-token buffers and block_prefill_workspace_bytes of workspace;
// the state must have no deferred tokens.
int64_t block_prefill_workspace_bytes(const sata_index *idx, int64_t bh);
hipError_t launch_block_prefill(const sata_index *idx, sata_state *st, const void *q, const void *k, const void *v,
                                void *out, int64_t n, sata_dtype in_dt, sata_dtype out_dt, hipStream_t stream);
hipError_t launch_state_convert(const sata_state *src, sata_state *dst, hipStream_t stream);

// Prefill plan: how the sequence is split into chunks, feature slices and
// segments, and how large the partial-sum workspace must be.
struct PrefillPlan {
    int chunk = 0;          // tokens per chunk
    int fw = 0;             // features per wave
    int fs = 0;             // features per workgroup slice
    bool ws = false;        // warp-specialised scan (fw = features per update wavefront)
    int slices = 0;         // workgroups per head
    int64_t seg_chunks = 0; // chunks per segment (bounded by the workspace cap)
    int64_t sync_off = 0;   // byte offset of the scan's counter and progress flags in the workspace
    int64_t sync_words = 0; // their count (a multiple of 4)
    int64_t o0_off = 0;     // byte offset of the order-0 chunk sums and prefixes (2 x [B*H][chunks][d_V+1] fp32)
    int64_t work_bytes = 0; // workspace needed
    bool s16 = false;       // fp16-operand scan (16-stream positions; sata_scan16.hip)
    int64_t img_off = 0;    // (s16) byte offset of the chunks' operand images in the workspace
    int mt = 0;             // (s16) positions per update wavefront
    bool ok = false;
    // output options for internal callers (the backward pass): write the
    // unnormalised numerator y[:d_V] instead of y[:d_V] / y[d_V], and/or the
    // normaliser y[d_V] of every token to den_out [B*H][n] (fp32)
    bool raw = false;
    float *den_out = nullptr;
    // (s16 only) heads share q and k in groups of qk_div: head h reads q and k of head
    // h / qk_div (the backward's pseudo-heads of one head differ only in v)
    int qk_div = 1;
    // (s16 only) v is binary16 rather than bf16: the backward's values (three more significand
    // bits; they are scaled into fp16's normal range)
    bool v_f16 = false;
};
// Largest prefill workspace planned by default (bytes; the device has 288 GB of HBM).  Longer
// calls run in segments of whole chunks; when the allocation fails, sata_prefill plans again
// under half the cap, down to one chunk per segment.
constexpr int64_t kWorkCap = (int64_t)16 << 30;
// fp16_operands: bf16 inputs may take the fp16-operand scan (exact for inputs inside fp16's
// normal range once scaled; the backward scales its gradient-weighted values into that range
// first).
PrefillPlan plan_prefill(const sata_index *idx, int64_t bh, int64_t n, int chunk, sata_dtype in_dt,
                         int64_t work_cap = kWorkCap, bool fp16_operands = true);
// Backward pass of a causal prefill from a zero state (sata_backward.hip);
// lower is the index with P - 1 orders (NULL when P == 1).  Synchronises the
// stream before returning (it frees its temporaries).
hipError_t launch_backward(const sata_index *idx, const sata_index *lower, int64_t bh, const void *q, const void *k,
                           const void *v, const void *dout, void *dq, void *dk, void *dv, int64_t n, int chunk,
                           sata_dtype in_dt, sata_dtype out_dt, int64_t mem_budget, hipStream_t s);
// The step the calling thread's last backward call was in (for error messages).
const char *backward_last_step();
// fp16-operand scan (sata_scan16.hip): whether it covers a prefill (bf16 inputs, P <= 4,
// d_K = d_V in {16, 32, 64, 128}), positions per slice and the operand image of one chunk
bool scan16_covers(const sata_index *idx, sata_dtype in_dt);
int scan16_choose_mt(int dk, int64_t np16, int64_t bh, int cus);
int64_t scan16_image_bytes(int dk, int chunk);
struct TaylorArgs;
// One segment of an fp16-operand prefill: operand images, scan, reduce (the order-0 prefixes
// o0pre of the whole call come first).
hipError_t launch_scan16_segment(const sata_index *idx, const sata_state *st, const PrefillPlan &plan, const void *q,
                                 const void *k, const void *v, void *out, int64_t n, int64_t tok0, int nseg,
                                 const float *o0pre, const TaylorArgs &ta, sata_dtype out_dt, hipStream_t stream);
hipError_t launch_prefill(const sata_index *idx, const sata_state *st, const PrefillPlan &plan,
                          const void *q, const void *k, const void *v, void *out, int64_t n,
                          sata_dtype in_dt, sata_dtype out_dt, hipStream_t stream);

// Kernel timing instrumentation (see sata_profile_enable).  A ProfScope
// records an event before and after the launches in its lifetime when
// profiling is on, and does nothing otherwise.
enum ProfKernel {
    kProfScan = 0, kProfCombine = 1, kProfDecode = 2, kProfDecodeFinish = 3, kProfDecodeRead = 4, kProfDecodeFold = 5,
    kProfDecodeLow = 6, kProfCount = 7
};
struct ProfScope {
    ProfScope(int kernel, hipStream_t stream);
    ~ProfScope();
    int kernel;
    hipStream_t stream;
    hipEvent_t start = nullptr;
};

hipError_t launch_zero(float *p, int64_t count, hipStream_t stream);
// Frees the backward calls' temporaries kept with an index (sata_backward.hip).
void free_backward_pool(const sata_index *idx);
// Dense TFLOP/s of a plain 16x16x32 MFMA loop on the current device (sata_measure.hip).
hipError_t measure_mfma_loop(bool bf16, double *tflops);

// Error bits a kernel may set in a state's error word.
constexpr uint32_t kErrScanWait = 1u;
// Bounded wait of the persistent scans for a predecessor's state: polls before giving up.
constexpr int kScanSpinLimit = 1 << 24;
// Fault injection for tests of the scans' error path (sata_debug_scan_faults): the persistent
// scans start taking work items at item_base instead of 0 (so the items before it never run
// and their successors' waits time out), and give up after spin_limit polls.
struct ScanDebug {
    int positions = 0;   // forced positions per update wavefront of the fp16-operand scan (0: the rule)
    int refresh = 0;     // forced chunks per state-copy refresh of the fp16-operand scan (0: the rule)
    int item_base = 0;
    int spin_limit = kScanSpinLimit;
};
ScanDebug scan_debug();
hipError_t launch_expand(const sata_index *idx, const void *x, void *out, int64_t rows, int side,
                         sata_dtype in_dt, hipStream_t stream);

}  // namespace sata
