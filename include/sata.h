/*
 * sata.h -- C ABI of the MI355X (gfx950) SATA attention library, libsata.so.
 *
 * SATA (symmetry-aware Taylor approximation) attention is causal attention
 * whose weight is the exp kernel truncated after P Taylor orders,
 *     x_ij = q_i . k_j / sqrt(d_K),   w(x) = sum_{p<P} x^p / p!,
 *     o_i  = sum_{j<=i} w(x_ij) v_j / sum_{j<=i} w(x_ij),
 * computed without an n x n matrix: keys and queries are mapped onto the
 * minimal basis of the symmetric tensors of order p (sorted index tuples
 * i_1 <= ... <= i_p, the tables M_p), and a fixed-size state
 *     S_p = sum_s phi_p(k_s) (x) [v_s, 1]
 * of (d_V + 1) * C(d_K+P-1, P-1) values per head is accumulated and read out.
 *
 * Citations (page title and section):
 *   [hotdry] blog.hotdry.top, "Symmetry-aware Taylor approximation attention:
 *            engineering a constant per-token cost" (2026-02-05):
 *            "Core insight of symmetric tensor decomposition" -- the minimal
 *            basis C(d_K+p-1, p) and the fixed, precomputed index tables M_p;
 *            "Engineering realisation of the constant compute cost" -- the
 *            state size, the per-token steps (map k through M_p, accumulate,
 *            weight and sum the orders' contributions) and the FLOP count;
 *            "Hardware optimisation paths and current limits" -- the
 *            hierarchical i_1 <= ... <= i_p structure, orders run in parallel.
 *   [mokono] www.mokono.cn attention-variants survey, standard attention:
 *            the (batch, heads, seq_len, dim) tensor layout.
 *
 * Conventions for every entry point
 *   - Status codes: every call returns sata_status; no C++ exception crosses
 *     this boundary.  Argument checks happen before any work is enqueued and
 *     have no side effects (SATA_ERR_INVALID).  sata_last_error() returns a
 *     thread-local message describing the last failure on this thread.
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the legacy
 *     default stream).  Calls that take a stream only enqueue work; kernel
 *     faults surface at the caller's next synchronisation.  A state must not
 *     be used from two streams at once.
 *   - Memory: q, k, v, out are device pointers owned by the caller, contiguous
 *     row-major, 16-byte aligned; `out` must not overlap q, k or v.  The
 *     library owns index and state memory (hipMalloc) and frees it in the
 *     *_free calls.
 *   - Supported shapes: d_K, d_V in {8, 16, 32, 64}, or d_K = d_V = 128;
 *     1 <= P <= 5.  Prefill needs d_K == d_V; at d_K = 128 it runs the
 *     chunked scan for bf16 inputs with P <= 4, and otherwise (fp32 inputs,
 *     P = 5) blocks of 64 tokens through the state in HBM, which is much
 *     slower; the backward takes d_K = 128 for bf16 inputs with 3 <= P <= 4
 *     and refuses it otherwise.  Other values return
 *     SATA_ERR_UNSUPPORTED.  The state grows as
 *     C(d_K+P-1, P-1) (d_V+1) fp32 values per head: at d_K = 64, 12.5 MB for
 *     P = 4 and 212 MB for P = 5; at d_K = 128 and P = 4, 189 MB.
 */
#ifndef SATA_H
#define SATA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SATA_OK = 0,
    SATA_ERR_INVALID = 1,      /* bad argument: null pointer, size, alignment, aliasing */
    SATA_ERR_UNSUPPORTED = 2,  /* valid but not built: (d_K, d_V, P, dtype, chunk) */
    SATA_ERR_OOM = 3,          /* device allocation failed */
    SATA_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} sata_status;

typedef enum {
    SATA_F32 = 0,              /* IEEE float32 */
    SATA_BF16 = 1,             /* bfloat16 (upper half of a float32) */
    SATA_F16 = 2               /* IEEE binary16: a decode state's element type only */
} sata_dtype;

/* Immutable, device-resident M_p tables and coefficients for one (d_K, d_V, P). */
typedef struct sata_index sata_index;
/* Fixed-size recurrent state of B x H heads plus its reusable workspace. */
typedef struct sata_state sata_state;

/* Build the index tables M_p for orders p = 0..P-1 [hotdry, "Core insight of
 * symmetric tensor decomposition": the sorted-tuple basis is fixed and can be
 * precomputed].  Features are numbered order by order (p = 0, 1, ..., P-1),
 * and within an order in lexicographic order of the sorted tuple (last index
 * fastest), so each order-(p-1) parent owns a contiguous run of children
 * [hotdry, "Hardware optimisation paths and current limits"].  Synchronous:
 * enumerates on the host, uploads to the current device.
 * d_k, d_v: head dims; P: number of Taylor orders (constant term included).
 * *out receives the handle on success and is untouched on failure. */
sata_status sata_build_index(int d_k, int d_v, int P, sata_index **out);

/* Free an index (NULL is a no-op).  The caller must ensure no enqueued work
 * still uses it (synchronise first). */
void sata_index_free(sata_index *idx);

/* m = C(d_K+P-1, P-1), the features per head over all orders
 * [hotdry, "Engineering realisation of the constant compute cost"]; -1 if idx
 * is NULL. */
int64_t sata_index_features(const sata_index *idx);

/* Shape of an index: any out-pointer may be NULL.  m_pad is the padded
 * feature stride of the state layout (a multiple of 64, >= m). */
sata_status sata_index_info(const sata_index *idx, int *d_k, int *d_v, int *P,
                            int64_t *m, int64_t *m_pad);

/* Allocate the zeroed state of batch x heads heads for `idx`, enqueueing the
 * clear on `stream`.  Layout (fp32): [batch][heads][d_V + 1][m_pad], feature
 * axis contiguous; row c < d_V holds sum_s prod_r k_s[i_r] * v_s[c], row d_V
 * holds sum_s prod_r k_s[i_r] (the "+1" column of [hotdry, "Engineering
 * realisation of the constant compute cost"]), features f >= m are zero.
 * The key side carries the plain monomial; the multinomial weight
 * p!/alpha!, the 1/p! of the Taylor term and d_K^(-p/2) are applied on the
 * query side at readout.  The state keeps a pointer to idx: free the state
 * before the index. */
sata_status sata_state_alloc(const sata_index *idx, int batch, int heads, void *stream,
                             sata_state **out);

/* As sata_state_alloc, with the state's element type chosen: SATA_F32 (what
 * sata_state_alloc gives), SATA_F16 or SATA_BF16.
 *
 * SATA_F16 [hotdry, "Hardware optimisation paths and current limits": Float16
 * storage is enough at P = 4 and halves the state's bandwidth]: the same layout
 * in binary16, except that the features of orders 0 and 1 -- the first
 * m_low = min(round_up(1 + d_K, 64), m_pad) features of each row, whose sums
 * grow with every token (the token count, the sums of k) and would stop
 * growing in 16 bits -- live in an fp32 array [batch][heads][d_V + 1][m_low]
 * that follows the binary16 one in the allocation (whose slots for them stay
 * zero).  Each decode step widens the stored values to fp32, adds the token's
 * term, reads out from the fp32 sums and stores them rounded to the nearest
 * binary16 (ties to even); the state holds 2 (d_V+1)(m_pad + 2 m_low) bytes
 * per head, 50.3% of the fp32 state at d_K = 64, P = 4.  At P = 4 the outputs
 * stay within 2e-2 of the exact Taylor attention for at least 1024 decode
 * steps after a conversion (measured: 6e-4 at d_K = 64, 2.2e-3 at d_K = 16).
 * Values must stay inside binary16's range (|S| < 65504 for the orders >= 2,
 * i.e. sums of monomials of k of degree >= 2 times v; unit-scale inputs stay
 * far below it).
 *
 * SATA_BF16: same layout, half the bytes.  A bf16
 * state serves sata_decode_step only: each step widens the stored values to
 * fp32, adds the new token's term, reads out from the fp32 sums and stores them
 * rounded to the nearest bf16 (ties to even), so the step streams half the
 * bytes of the fp32 state [hotdry, "Hardware optimisation paths and current
 * limits": half-precision storage halves the bandwidth of the state] at the
 * price of one bf16 rounding per element per step.  Those roundings
 * accumulate: with P = 4 and d_K >= 16 the outputs of up to 16 decode steps
 * after a conversion stay within 2e-2 (the bar of the bf16 paths) of the
 * exact Taylor attention, and the error keeps growing with the number of
 * steps (about 3e-2 after 64); fewer orders or smaller heads drift faster.
 * Use it for short decodes after a long prefill; the fp32 state is exact to
 * fp32 rounding at any length.  sata_prefill on a bf16 or fp16 state returns
 * SATA_ERR_UNSUPPORTED: prefill into an fp32 state and convert.  An unknown
 * state_dt returns SATA_ERR_INVALID. */
sata_status sata_state_alloc_dtype(const sata_index *idx, int batch, int heads, sata_dtype state_dt,
                                   void *stream, sata_state **out);

/* Copy src's content into dst, converting the element type (to bf16 or fp16
 * rounds to nearest even, except an fp16 state's fp32 orders; to fp32 is
 * exact; equal types copy).  Both must
 * belong to the same index and have the same batch and heads; src != dst
 * (else SATA_ERR_INVALID, nothing enqueued).  src's deferred decode tokens
 * (sata_state_set_decode_window) are folded into src first; dst's are
 * discarded.  Enqueued on `stream`; dst's workspace and window are
 * untouched. */
sata_status sata_state_convert(sata_state *src, sata_state *dst, void *stream);

/* Decode window: the number W of decode steps per update of the state buffer
 * (1 <= W <= 64, else SATA_ERR_INVALID; default 1).  With W > 1,
 * sata_decode_step defers the update: W - 1 steps in a row only read the
 * state out, adding each deferred token's (and the step's own) term from its
 * direct Taylor weight w(q.k_t / sqrt(d_K)) [v_t, 1] -- the single-token sum
 * that the state's orders hold for it [hotdry, "Core insight of symmetric
 * tensor decomposition"] -- and keep k and v of the step in a small per-head
 * buffer; every W-th step adds all of them to the state in one
 * read-modify-write pass (a rank-W product on the matrix cores, fp32) and
 * reads out from the result.  The outputs are the
 * same as with W = 1 up to rounding, and each step still costs a bounded
 * amount of work whatever the context length [hotdry, "Engineering
 * realisation of the constant compute cost"], while W - 1 of every W steps
 * stream the state once instead of twice.  Deferred tokens are folded in
 * before the window changes, before a prefill, before a conversion, and by
 * sata_state_flush; sata_state_reset discards them.  The first call with
 * W > 1 allocates the token buffers (hipMalloc, 64 slots per head). */
sata_status sata_state_set_decode_window(sata_state *st, int window, void *stream);

/* Fold the deferred decode tokens into the state buffer (no-op if none), so
 * that the buffer holds every token seen.  Enqueued on `stream`. */
sata_status sata_state_flush(sata_state *st, void *stream);

/* Synchronise `stream`, then report what asynchronous work on the state has
 * recorded in its error word since the last report: SATA_ERR_HIP (with the
 * detail in sata_last_error) if a prefill's scan gave up waiting for a work
 * item's predecessor, which leaves that prefill's output and the state
 * invalid; SATA_OK otherwise.  The word is cleared once reported.  Every
 * sata_prefill, sata_decode_step and sata_state_flush on the state reports
 * the word the same way (without synchronising) before enqueueing work. */
sata_status sata_state_check(sata_state *st, void *stream);

/* Zero the state (start a new sequence); enqueued on `stream`. */
sata_status sata_state_reset(sata_state *st, void *stream);

/* Free a state and its workspace (NULL is a no-op).  Synchronise first. */
void sata_state_free(sata_state *st);

/* Device pointer and byte size of the state buffer (for checkpointing or
 * inspection; the layout is given at sata_state_alloc, elements of the type
 * given at allocation).  Deferred decode tokens are not in it until
 * sata_state_flush. */
sata_status sata_state_data(const sata_state *st, void **dev_ptr, int64_t *bytes);

/* Causal prefill of n tokens for every head of the state, continuing from the
 * state's content (a zeroed state starts a fresh sequence); on return (in
 * stream order) the state covers every token seen.
 * q, k: [batch][heads][n][d_K]; v, out: [batch][heads][n][d_V]; in_dt is the
 * dtype of q, k, v; out_dt that of out.  Token i attends to every earlier
 * token and to itself.  The sequence is processed in chunks of `chunk` tokens
 * (0 = default: 256 for bf16 inputs with P <= 4 and d_K = d_V = 16; 128
 * for bf16 inputs with P <= 4 and d_K = d_V in {32, 64}, for d_K = 64, and
 * for fp32 inputs at d_K = 16; 64 otherwise; supported arguments: 0, 64,
 * 128; at d_K = 128 the chunk is always 64 tokens):
 * within a chunk the Taylor weights are formed directly, across chunks the
 * orders' states are scanned and read out [hotdry, "Engineering realisation
 * of the constant compute cost"]; results do not depend on the chunk length
 * beyond rounding.  (The fp16-operand scan below reads a chunk out against
 * the state of up to 7 chunks earlier and forms the weights of the keys in
 * between directly as well: the same terms, split at another token.)  For bf16 inputs with d_K = d_V in {16, 32, 64, 128} and
 * P <= 4 the scan's matrix operands are fp16: k / 4, 4 q / sqrt(d_K) and v
 * convert to fp16 exactly when their magnitudes lie in fp16's normal range
 * (6.1e-5 to 65504, or zero); smaller ones keep less precision and larger
 * ones overflow.  Rows of q and k of norm up to d_K^(1/4) and v of unit
 * scale lie well inside; give inputs far outside that scale as fp32.
 * n = 0 is a no-op.  May grow the state's workspace
 * (hipMalloc) on the first call at a given size: the partial readouts of up
 * to 16 GB are planned at once (longer calls run in segments of whole chunks);
 * if that allocation fails, the call plans again under half the workspace,
 * down to one chunk per segment, before it returns SATA_ERR_OOM.  A device-side
 * failure of the scan's work scheduling (a work item that gives up waiting for
 * its predecessor's state) cannot be seen when the call returns: it is
 * recorded in the state and reported as SATA_ERR_HIP by the next call on the
 * state or by sata_state_check, and that earlier call's output and state are
 * invalid. */
sata_status sata_prefill(const sata_index *idx, sata_state *st, const void *q, const void *k,
                         const void *v, void *out, int64_t n, int chunk, sata_dtype in_dt,
                         sata_dtype out_dt, void *stream);

/* Byte size of sata_prefill_noalloc's scratch array (128 MiB), which every
 * device the library runs on holds until the process ends. */
#define SATA_NOALLOC_SCRATCH_BYTES ((int64_t)128 << 20)

/* sata_prefill for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, and harnesses that forbid allocation.
 * Same arguments, results and error reporting as sata_prefill (outputs equal
 * sata_prefill's up to rounding; with the same segment plan, bit for bit), but
 * the call performs no hipMalloc, hipFree or other allocation: its workspace
 * is a file-scope device array of SATA_NOALLOC_SCRATCH_BYTES, looked up once
 * per device on the first call there, and the prefill runs in segments of
 * whole chunks sized to fit it (timing events of sata_profile_enable are not
 * recorded for it).  The caller still provides q, k, v, out and the state
 * (allocated beforehand).  Every call on a device shares that device's
 * array: calls that overlap in time on one device (other streams or host
 * threads) race and give wrong results; order them.  Returns
 * SATA_ERR_UNSUPPORTED where sata_prefill would take the block path (d_K =
 * 128 with fp32 inputs or P = 5) and when even single-chunk segments need
 * more workspace than the array holds (about 1.6 MB per head at d_K = 64,
 * P = 4, and 24 MB per head at d_K = 128), with the size needed in
 * sata_last_error. */
sata_status sata_prefill_noalloc(const sata_index *idx, sata_state *st, const void *q, const void *k,
                                 const void *v, void *out, int64_t n, int chunk, sata_dtype in_dt,
                                 sata_dtype out_dt, void *stream);

/* Gradients of a causal prefill of n tokens that starts from a zero state
 * (a fresh sequence): given dout = dL/dout for out = the prefill's output on
 * q, k, v, write dq, dk, dv = dL/dq, dL/dk, dL/dv.  Shapes and dtypes as for
 * sata_prefill: q, k, v, dout [batch][heads][n][d_K] of in_dt; dq, dk, dv of
 * grad_dt; d_K == d_V.  With g_i = [dout_i, -dout_i.out_i] / z_i (z_i the
 * normaliser) and w' the series with P - 1 orders, every gradient is a
 * causal or (on reversed time) anti-causal Taylor attention read out without
 * normalisation, so the pass runs on the prefill's fixed-state kernels with
 * a constant cost per token [hotdry, "Engineering realisation of the constant
 * compute cost"]: a forward pass for out and z, a pass of P orders for dv, and
 * passes of P - 1 orders over d_V + 1 pseudo-heads per head for dk and dq
 * (none when P == 1: dq = dk = 0).  With bf16 inputs every pass whose head
 * size and order the fp16-operand prefill scan covers runs on it; the
 * gradient-weighted values (g_i, and g_i[c] q_i) enter scaled by the power of
 * two that brings the largest |g| into [2^8, 2^9), and the results are scaled
 * back.  d_K = 128 needs bf16 inputs and 3 <= P <= 4 (SATA_ERR_UNSUPPORTED
 * otherwise).  The (P - 1)-order index is built on the first call and kept
 * with idx (freed by sata_index_free).  Its device temporaries (tens of GB
 * at d_K = 64, n = 65536) are allocated by the first call and kept with idx
 * for later calls, grown when a call needs more, and freed by
 * sata_index_free; backward calls on one index are serialised.  Synchronises
 * `stream` before returning.  Gradients must
 * not overlap the inputs or each other; n = 0 is a no-op. */
sata_status sata_prefill_backward(const sata_index *idx, int batch, int heads, const void *q, const void *k,
                                  const void *v, const void *dout, void *dq, void *dk, void *dv, int64_t n,
                                  int chunk, sata_dtype in_dt, sata_dtype grad_dt, void *stream);

/* Measurement helper for benchmarks (not part of the attention path): runs a
 * loop of v_mfma_f32_16x16x32 instructions (bf16 operands when bf16 != 0,
 * else fp16; fp32 accumulation; 16 independent accumulator chains per
 * wavefront and nothing else in the loop) on every compute unit of the
 * current device, two wavefronts per SIMD, and writes the dense TFLOP/s it
 * reaches to *tflops: the ceiling a kernel made of such instructions can
 * reach on this device, beside the published peak.  Synchronous; allocates
 * and frees a small output buffer and two events. */
sata_status sata_measure_mfma_loop(int bf16, double *tflops);

/* One decode step for every head: with q, k: [batch][heads][d_K] and
 * v: [batch][heads][d_V] of the new token, add phi(k) (x) [v, 1] to every
 * order's state, then read out and normalise into out: [batch][heads][d_V]
 * [hotdry, "Engineering realisation of the constant compute cost": the cost
 * per token is fixed by d_K, d_V and P].  Each head's state is streamed once
 * (read and written), coalesced along the feature axis.  With a decode window
 * above 1 the update is deferred (sata_state_set_decode_window). */
sata_status sata_decode_step(const sata_index *idx, sata_state *st, const void *q, const void *k,
                             const void *v, void *out, sata_dtype in_dt, sata_dtype out_dt,
                             void *stream);

/* Feature expansion on its own (tests and inspection): for rows x: [rows][d_K]
 * write out: [rows][m_pad] fp32 with, per feature f = (i_1..i_p) of order p,
 *   side 0 (key):   prod_r x[i_r]
 *   side 1 (query): prod_r x[i_r] / (alpha_f! * d_K^(p/2))
 * where alpha_f! is the product of the factorials of the index multiplicities,
 * so that sum_f key(k)_f * query(q)_f * p! over the features of order p equals
 * (q.k / sqrt(d_K))^p [hotdry, "Core insight of symmetric tensor
 * decomposition"].  Features f >= m are zero. */
sata_status sata_expand_features(const sata_index *idx, const void *x, void *out, int64_t rows,
                                 int side, sata_dtype in_dt, void *stream);

/* Host-only description of the feature tables sata_build_index uploads for
 * (d_k, P), without touching a GPU (tests and inspection).  Writes up to cap
 * entries: tuples[f] = the packed tuple word of feature f (bytes 0..2 the
 * indices i_1..i_p, unused slots = d_k; byte 3 the order p) and coef[f] =
 * 1/(alpha_f! d_k^(p/2)) rounded to fp32, in the feature order described at
 * sata_build_index.  Either array may be NULL.  Returns m, or -1 for
 * arguments sata_build_index would reject. */
int64_t sata_describe_features(int d_k, int P, uint32_t *tuples, float *coef, int64_t cap);

/* Host-only description of the prefill's grouped view of the same features
 * (tests and inspection): features are grouped into "quads", a sorted prefix
 * (i_1, i_2) (absent indices = d_k) and an aligned block of four last indices
 * i_3 = 4b + z.  w0[q] = i_1 | i_2 << 8 | b << 16 | mask << 24, where bit z of
 * mask marks slot z as a feature (else padding); cidx[q] is the feature index
 * of the first valid slot (-1 if none), and coef4[4q + z] the slot's
 * multinomial factor 1/alpha! (0 for padding); the slot's full readout weight
 * is that factor times d_k^(-p/2), which the prefill applies by scaling q.  The order-0 quad has b = d_k/4 and mask 1.  The
 * valid slots of consecutive quads are consecutive features.  Returns the
 * number of quads, or -1 for arguments sata_build_index would reject. */
int64_t sata_describe_quads(int d_k, int P, uint32_t *w0, int32_t *cidx, float *coef4, int64_t cap);

/* Host-only, for tests: the same features in the fp16-operand scan's view
 * (P <= 4, 16 <= d_K <= 128): positions of 16 quads sharing a block b, with
 * w0 = i1 | i2 << 8 | b << 16 | slot mask << 28 (absent indices are d_K,
 * padding quads d_K + 1), cidx and coef4 as above (16 per position), and per
 * position flags: bit 0 = some quad has invalid slots or slots of different
 * weights, bit 1 = the position starts a group (the 16 prefixes change; the
 * following positions of the group take blocks b + 1, b + 2, ...).  For P <= 3
 * a group takes 16 consecutive prefixes of the whole list, so some of its
 * quads have no valid slot in its lower blocks.  Writes up to cap positions
 * (16 cap quads, 64 cap weights; any pointer may be NULL) and returns the
 * number of positions (0 outside that range), or -1 for arguments
 * sata_build_index would reject. */
int64_t sata_describe_quads16(int d_k, int P, uint32_t *w0, int32_t *cidx, float *coef4, uint32_t *flags,
                              int64_t cap);

/* Host-only: the chunked prefill's plan for batch_heads heads of n tokens of
 * (d_k = d_v, P) with in_dt inputs under a workspace cap of work_cap bytes
 * (sata_prefill starts at 16 GB): returns the workspace bytes and writes the
 * chunks per segment and the feature slices per head (either pointer may be
 * NULL); -1 for arguments the chunked prefill does not take (d_k = 128 has a
 * plan only for bf16 inputs with P <= 4; the rest runs in blocks).  For tests
 * and capacity planning. */
int64_t sata_describe_prefill_plan(int d_k, int P, int64_t batch_heads, int64_t n, int chunk, int in_dt,
                                   int64_t work_cap, int64_t *seg_chunks, int64_t *slices);

/* Fault injection for tests of the prefill scan's error path (process-wide,
 * affects every later prefill until reset with (0, 0)): the persistent scan
 * starts taking work items at item_base instead of 0, so the first item_base
 * items never run, and gives up a wait for a predecessor after spin_limit
 * polls (0 = the default, 2^24).  An item whose predecessor never ran then
 * times out, records the failure in the state's error word and carries on,
 * so every kernel still ends; the call's output is invalid.  Without
 * sub-segments (a grid of at most one work item per compute unit) no item
 * waits and skipped items go unreported.  Negative arguments return
 * SATA_ERR_INVALID.  Not for production use. */
sata_status sata_debug_scan_faults(int item_base, int spin_limit);

/* Tile choice for measurement (process-wide, affects every later plan until
 * reset with 0): the fp16-operand prefill scan holds mt positions (64 features
 * each) of the state per update wavefront instead of the library's rule.
 * mt must be 0 (the rule), 1, or the largest the head size holds (5, 3, 2, 1
 * at d_K = 16, 32, 64, 128), else SATA_ERR_INVALID; a value the head size
 * does not hold leaves the rule in force for that size.  The chunk length is
 * sata_prefill's argument.  Not for production use. */
sata_status sata_debug_prefill_positions(int mt);

/* Copy refresh interval for measurement (process-wide, affects every later
 * call until reset with 0): the fp16-operand prefill scan rewrites the fp16
 * copy of the state that its readout reads every `chunks` chunks instead of
 * at the library's rule.  Chunks in between are read out against the last
 * copy, and the keys since that copy enter as direct Taylor terms (the
 * weights of the intra-chunk term), so the result is the same up to
 * rounding.  chunks must be 0 (the rule) or 1 .. 16, else SATA_ERR_INVALID.
 * Not for production use. */
sata_status sata_debug_prefill_refresh(int chunks);

/* Kernel timing instrumentation.  While enabled, every launch of the
 * library's kernels is bracketed by a HIP event pair recorded on the stream
 * the kernel is launched on.  sata_profile_enable(1) clears earlier records;
 * (0) stops recording and keeps them.  sata_profile_query waits for the
 * recorded events of one kernel and returns the summed duration (ms) and the
 * launch count.  Kernel ids: 0 prefill scan, 1 prefill combine, 2 decode
 * stream, 3 decode finish, 4 decode read (deferred steps), 5 decode fold,
 * 6 decode of an fp16 state's fp32 orders (names from
 * sata_profile_kernel_name, NULL for an unknown id).  Host-thread safe; not
 * meant to be left on in production. */
sata_status sata_profile_enable(int on);
sata_status sata_profile_query(int kernel, double *total_ms, int64_t *launches);
const char *sata_profile_kernel_name(int kernel);

/* Static description of a status code. */
const char *sata_status_string(sata_status s);

/* Thread-local detail of the last failure on the calling thread ("" if none). */
const char *sata_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SATA_H */
