// Host side of libsata: index construction, state management, argument
// validation and the extern "C" entry points declared in include/sata.h.
//
//   [hotdry] blog.hotdry.top, "Symmetry-aware Taylor approximation attention:
//            engineering a constant per-token cost" (2026-02-05).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <atomic>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "sata_internal.h"

namespace {

thread_local std::string g_last_error;
// Set while sata_prefill_noalloc runs on this thread: its launches record no timing events
// (which would create hipEvents).
thread_local bool t_prof_off = false;

sata_status fail(sata_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

sata_status fail_hip(hipError_t e, const char *what) {
    return fail(SATA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool supported_dim(int d) { return d == 8 || d == 16 || d == 32 || d == 64 || d == 128; }
// The prefill's quad words hold the block index in four bits (d_K / 4 <= 16).
constexpr int kMaxPrefillDim = 64;
// The 16-stream view (at most four orders) holds it in a byte: the fp16-operand scan's range.
constexpr int kMaxScan16Dim = 128;

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

int64_t dtype_bytes(sata_dtype t) { return t == SATA_BF16 || t == SATA_F16 ? 2 : 4; }

bool valid_dtype(int t) { return t == SATA_F32 || t == SATA_BF16; }              // inputs and outputs
bool valid_state_dtype(int t) { return t == SATA_F32 || t == SATA_BF16 || t == SATA_F16; }

// An fp16 state keeps the features of orders 0 and 1 (the constant and the d_K linear ones,
// which grow with every token) in fp32: the first 1 + d_K features, rounded up to 64 (all of
// them when P = 1), so that the fp16 words the decode kernels start from are 128-byte aligned.
int64_t f16_low_features(const sata_index *idx) { return std::min<int64_t>(round_up(1 + idx->dk, 64), idx->m_pad); }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void *a, int64_t na, const void *b, int64_t nb) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

// Sorted index tuples i_1 <= ... <= i_p over [0, d) in lexicographic order,
// last index fastest [hotdry, "Core insight of symmetric tensor
// decomposition": the minimal basis of the symmetric tensor of order p].
void enumerate_order(int d, int p, std::vector<std::vector<int>> &out) {
    std::vector<int> idx(p, 0);
    if (p == 0) { out.push_back(idx); return; }
    for (;;) {
        out.push_back(idx);
        int r = p - 1;
        while (r >= 0 && idx[r] == d - 1) --r;
        if (r < 0) break;
        ++idx[r];
        for (int s = r + 1; s < p; ++s) idx[s] = idx[r];
    }
}

// Product of the factorials of the run lengths of a sorted tuple (alpha!).
double alpha_factorial(const std::vector<int> &t) {
    double prod = 1.0;
    size_t i = 0;
    while (i < t.size()) {
        size_t j = i;
        while (j < t.size() && t[j] == t[i]) ++j;
        for (size_t a = 2; a <= j - i; ++a) prod *= (double)a;
        i = j;
    }
    return prod;
}

struct DeviceGuard {
    int prev = -1;
    bool ok = true;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) { ok = false; return; }
        if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

sata_status ensure_work(sata_state *st, int64_t bytes) {
    if (bytes <= st->work_bytes) return SATA_OK;
    if (st->d_work) {
        hipError_t e = hipFree(st->d_work);
        st->d_work = nullptr;
        st->work_bytes = 0;
        if (e != hipSuccess) return fail_hip(e, "hipFree(workspace)");
    }
    hipError_t e = hipMalloc(&st->d_work, (size_t)bytes);
    if (e != hipSuccess) {
        st->d_work = nullptr;
        (void)hipGetLastError();
        return fail(SATA_ERR_OOM, "workspace allocation of %lld bytes failed: %s", (long long)bytes,
                    hipGetErrorString(e));
    }
    st->work_bytes = bytes;
    return SATA_OK;
}

// Folds a state's deferred decode tokens into its buffer (no-op without any).
sata_status flush_pending(sata_state *st, hipStream_t stream) {
    if (st->npend == 0) return SATA_OK;
    hipError_t e = sata::launch_decode(st->idx, st, nullptr, nullptr, nullptr, nullptr, SATA_F32, SATA_F32,
                                       sata::kDecodeFlush, stream);
    if (e != hipSuccess) return fail_hip(e, "fold of deferred decode tokens");
    st->npend = 0;
    return SATA_OK;
}

// Allocates a state's pending-token buffers (kMaxDecodeWindow slots per head) on first use.
sata_status ensure_pending(sata_state *st) {
    if (st->d_pend_k) return SATA_OK;
    const int64_t slots = (int64_t)st->batch * st->heads * kMaxDecodeWindow;
    float *pk = nullptr, *pv = nullptr;
    hipError_t e = hipMalloc(&pk, (size_t)(slots * st->idx->dk * sizeof(float)));
    if (e == hipSuccess) e = hipMalloc(&pv, (size_t)(slots * st->idx->dv * sizeof(float)));
    if (e != hipSuccess) {
        (void)hipGetLastError();
        if (pk) (void)hipFree(pk);
        return fail(SATA_ERR_OOM, "pending-token buffers of %lld slots", (long long)slots);
    }
    st->d_pend_k = pk;
    st->d_pend_v = pv;
    return SATA_OK;
}

sata_status check_index_state(const sata_index *idx, const sata_state *st) {
    if (!idx) return fail(SATA_ERR_INVALID, "index is NULL");
    if (!st) return fail(SATA_ERR_INVALID, "state is NULL");
    if (st->idx != idx) return fail(SATA_ERR_INVALID, "state was allocated for a different index");
    return SATA_OK;
}

// Reports (and clears) what the device has written to the state's error word so far.  The
// word lives in pinned, device-mapped host memory, so reading it needs no synchronisation;
// work still in flight may set it later.
sata_status take_state_error(sata_state *st) {
    if (!st->h_err) return SATA_OK;
    const uint32_t bits = __atomic_exchange_n(st->h_err, 0u, __ATOMIC_ACQ_REL);
    if (bits & sata::kErrScanWait)
        return fail(SATA_ERR_HIP,
                    "an earlier prefill on this state is invalid: a scan work item gave up waiting for the "
                    "state of its predecessor (output and state of that call are wrong; reset the state)");
    if (bits) return fail(SATA_ERR_HIP, "an earlier call on this state reported device error bits 0x%x", bits);
    return SATA_OK;
}

std::atomic<int> g_debug_item_base{0};
std::atomic<int> g_debug_spin_limit{sata::kScanSpinLimit};
std::atomic<int> g_debug_positions{0};
std::atomic<int> g_debug_refresh{0};

}  // namespace

namespace sata {
hipError_t launch_zero(float *p, int64_t count, hipStream_t stream);
ScanDebug scan_debug() {
    ScanDebug d;
    d.item_base = g_debug_item_base.load(std::memory_order_relaxed);
    d.spin_limit = g_debug_spin_limit.load(std::memory_order_relaxed);
    d.positions = g_debug_positions.load(std::memory_order_relaxed);
    d.refresh = g_debug_refresh.load(std::memory_order_relaxed);
    return d;
}
}

namespace {

// Argument and state checks shared by sata_prefill and sata_prefill_noalloc (the second also
// reports, and clears, an error the device recorded on the state since the last call).  Sets
// *nothing for n == 0.
sata_status check_prefill_args(const sata_index *idx, sata_state *st, const void *q, const void *k, const void *v,
                               void *out, int64_t n, int chunk, sata_dtype in_dt, sata_dtype out_dt, bool *nothing) {
    sata_status s = check_index_state(idx, st);
    if (s != SATA_OK) return s;
    if (n < 0) return fail(SATA_ERR_INVALID, "n must be >= 0 (got %lld)", (long long)n);
    if (!valid_dtype(in_dt) || !valid_dtype(out_dt)) return fail(SATA_ERR_INVALID, "unknown dtype");
    if (chunk != 0 && chunk != 64 && chunk != 128)
        return fail(SATA_ERR_UNSUPPORTED, "chunk must be 0 (default), 64 or 128 (got %d)", chunk);
    if (idx->dk != idx->dv) return fail(SATA_ERR_UNSUPPORTED, "prefill needs d_k == d_v");
    if (st->dtype != SATA_F32)
        return fail(SATA_ERR_UNSUPPORTED, "prefill needs an fp32 state (convert a bf16 or fp16 state with sata_state_convert)");
    s = take_state_error(st);
    if (s != SATA_OK) return s;
    *nothing = n == 0;
    if (*nothing) return SATA_OK;
    if (!q || !k || !v || !out) return fail(SATA_ERR_INVALID, "q, k, v and out must be non-NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(SATA_ERR_INVALID, "q, k, v and out must be 16-byte aligned");
    const int64_t bh = (int64_t)st->batch * st->heads;
    const int64_t in_b = dtype_bytes(in_dt), out_b = dtype_bytes(out_dt);
    const int64_t nq = bh * n * idx->dk * in_b, nv = bh * n * idx->dv * in_b, no = bh * n * idx->dv * out_b;
    if (overlaps(out, no, q, nq) || overlaps(out, no, k, nq) || overlaps(out, no, v, nv))
        return fail(SATA_ERR_INVALID, "out overlaps q, k or v");
    return SATA_OK;
}

// ---- allocation-free prefill workspace
// sata_prefill_noalloc keeps its workspace (split-K partials, work-queue counters and progress
// flags, order-0 sums, chunk images) in this file-scope device array: every device the library
// runs on holds its own copy until the process ends.  In host code the name is a host-side
// stand-in, not a device address; the device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that pointer is used.
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kScratchDevices] = {};

}  // namespace

static __device__ __align__(256) unsigned char scratch[SATA_NOALLOC_SCRATCH_BYTES];

namespace {

// The current device's (dev's) address of the scratch array.
sata_status scratch_address(int dev, void **ptr) {
    if (dev < 0 || dev >= kScratchDevices)
        return fail(SATA_ERR_UNSUPPORTED, "device %d is beyond the %d devices the allocation-free prefill tracks", dev,
                    kScratchDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return fail_hip(e, "address of the allocation-free prefill's scratch array");
        if (!p) return fail(SATA_ERR_HIP, "the allocation-free prefill's scratch array has no device address");
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return SATA_OK;
}

struct ProfOff {
    ProfOff() { t_prof_off = true; }
    ~ProfOff() { t_prof_off = false; }
};

}  // namespace

extern "C" {

const char *sata_status_string(sata_status s) {
    switch (s) {
        case SATA_OK: return "ok";
        case SATA_ERR_INVALID: return "invalid argument";
        case SATA_ERR_UNSUPPORTED: return "unsupported configuration";
        case SATA_ERR_OOM: return "device out of memory";
        case SATA_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char *sata_last_error(void) { return g_last_error.c_str(); }

// Feature tables for (d_k, P): packed tuples and query-side readout weights
// 1/(alpha! d_k^(p/2)) (the multinomial p!/alpha! of the symmetric basis times
// the 1/p! of the Taylor term and the d_k^(-p/2) of the logit scale)
// [hotdry, "Core insight of symmetric tensor decomposition"].
static void build_tables(int d_k, int P, std::vector<uint32_t> &tup, std::vector<float> &coef) {
    const double sqd = std::sqrt((double)d_k);
    for (int p = 0; p < P; ++p) {
        std::vector<std::vector<int>> tuples;
        enumerate_order(d_k, p, tuples);
        const double dp = std::pow(sqd, (double)p);
        for (const auto &t : tuples) {
            uint32_t w = 0;
            for (int r = 0; r < sata::kMaxOrder; ++r) {
                const uint32_t slot = r < p ? (uint32_t)t[r] : (uint32_t)d_k;   // d_k -> constant 1
                w |= slot << (8 * r);
            }
            tup.push_back(w);
            coef.push_back((float)(1.0 / (alpha_factorial(t) * dp)));
        }
    }
}

// Quads for the prefill, in the order the scan kernel walks them.  A quad is a
// prefix (i0, i1, i2) of up to three sorted indices (absent ones first) and an
// aligned block of four last indices 4b + z; slot z is a feature when
// (prefix, 4b+z) is sorted.  Quads come in "positions" of `streams` quads (4
// for the general scan, 16 for the fp16-operand scan), one per stream, whose
// prefixes have the same block range: every prefix whose last
// index i2 lies in [4a, 4a+4) (order 4: i0 <= i1 <= i2; order 3: i1 <= i2;
// order 2: i2 alone; for a = 0 also the order-1 prefix with all absent)
// sweeps the blocks b = a .. d/4-1, and `streams` such prefixes sweep them side
// by side.  So within a position the block b is common, and only the first
// block of a group (the one holding 4b+z = i2) has slots below i2 (invalid)
// or a diagonal slot whose multiplicity differs from the rest.  Each valid
// slot carries the multinomial part 1/alpha! of its feature's readout weight
// 1/(alpha! d^(p/2)) [hotdry, "Core insight of symmetric tensor
// decomposition"]; the prefill applies d^(-p/2) by scaling q by 1/sqrt(d_K).
// The prefix product is shared by the four slots of a quad and by all blocks
// of its group [hotdry, "Hardware optimisation paths and current limits": the
// hierarchical index structure].  Order 0 (the constant feature) has no quad:
// its state entries are running sums of [v, 1], which the prefill keeps
// outside the scan.  Unused streams are padding quads (prefix product 0).
// flags[pos]: bit 0 = some quad of the position has slots with different
// weights (or invalid slots), bit 1 = the position starts a new group of
// prefixes.  Word w0: i1 | i2 << 8 | i0 << 16 | b << 24 | slot mask << 28; with
// block_byte (views without three-index prefixes, P <= 4) b takes the i0 byte
// instead: i1 | i2 << 8 | b << 16 | slot mask << 28, for d up to 1020.
// pool: a group takes `streams` consecutive prefixes of the whole list instead
// of those of one block a, and sweeps the blocks from that of its first prefix;
// a prefix whose i2 lies above a block has no valid slot there.  With P = 3
// there are only four prefixes per block a (five for a = 0), so a group of 16
// per block would be three quarters padding.
static void build_quads(int d, int P, std::vector<sata::QuadRec> &out, std::vector<uint32_t> &flags,
                        size_t streams = 4, bool block_byte = false, bool pool = false) {
    std::map<std::vector<int>, int32_t> index;   // sorted tuple -> feature index
    {
        int32_t f = 0;
        for (int p = 0; p < P; ++p) {
            std::vector<std::vector<int>> tuples;
            enumerate_order(d, p, tuples);
            for (const auto &t : tuples) index[t] = f++;
        }
    }
    const int none = d, pad = d + 1;
    struct Prefix { int i0, i1, i2; };
    auto make = [&](const Prefix &x, int b, uint32_t &nonuni) {
        sata::QuadRec q{};
        q.w0 = block_byte ? (uint32_t)pad | ((uint32_t)pad << 8) | ((uint32_t)b << 16)
                          : (uint32_t)pad | ((uint32_t)pad << 8) | ((uint32_t)none << 16) | ((uint32_t)b << 24);
        q.cidx = -1;
        if (x.i2 == pad) return q;
        std::vector<int> prefix;
        for (int i : {x.i0, x.i1, x.i2})
            if (i != none) prefix.push_back(i);
        uint32_t mask = 0;
        int first = -1;
        for (int z = 0; z < 4; ++z) {
            std::vector<int> t = prefix;
            const int last = 4 * b + z;
            const bool ok = t.empty() || last >= t.back();
            t.push_back(last);
            q.coef[z] = 0.f;
            if (!ok) continue;
            mask |= 1u << z;
            if (first < 0) {
                first = z;
                q.cidx = index.at(t);
            }
            q.coef[z] = (float)(1.0 / alpha_factorial(t));
        }
        q.w0 = block_byte ? (uint32_t)x.i1 | ((uint32_t)x.i2 << 8) | ((uint32_t)b << 16) | (mask << 28)
                          : (uint32_t)x.i1 | ((uint32_t)x.i2 << 8) | ((uint32_t)x.i0 << 16) | ((uint32_t)b << 24) | (mask << 28);
        if (mask != 0xfu || q.coef[0] != q.coef[1] || q.coef[0] != q.coef[2] || q.coef[0] != q.coef[3]) nonuni = 1;
        return q;
    };
    // the prefixes whose last index lies in block a
    auto block_prefixes = [&](int a) {
        std::vector<Prefix> prefixes;
        if (P >= 2 && a == 0) prefixes.push_back({none, none, none});
        for (int i2 = 4 * a; i2 < 4 * a + 4; ++i2) {
            if (P >= 5)
                for (int i1 = 0; i1 <= i2; ++i1)
                    for (int i0 = 0; i0 <= i1; ++i0) prefixes.push_back({i0, i1, i2});
            if (P >= 4)
                for (int i1 = 0; i1 <= i2; ++i1) prefixes.push_back({none, i1, i2});
            if (P >= 3) prefixes.push_back({none, none, i2});
        }
        return prefixes;
    };
    // groups of up to `streams` prefixes, each sweeping the blocks a0 .. d/4-1
    auto emit = [&](const std::vector<Prefix> &prefixes, size_t g, int a0) {
        for (int b = a0; b < d / 4; ++b) {
            uint32_t nonuni = 0;
            for (size_t s = 0; s < streams; ++s) {
                const bool have = g + s < prefixes.size();
                out.push_back(make(have ? prefixes[g + s] : Prefix{none, pad, pad}, b, nonuni));
            }
            flags.push_back(nonuni | (b == a0 ? 2u : 0u));
        }
    };
    if (pool) {
        std::vector<Prefix> all;
        std::vector<int> blk;   // block of each prefix's last index (0 for the empty prefix)
        for (int a = 0; a < d / 4; ++a)
            for (const Prefix &x : block_prefixes(a)) {
                all.push_back(x);
                blk.push_back(a);
            }
        for (size_t g = 0; g < all.size(); g += streams) emit(all, g, blk[g]);
        return;
    }
    for (int a = 0; a < d / 4; ++a) {
        const std::vector<Prefix> prefixes = block_prefixes(a);
        for (size_t g = 0; g < prefixes.size(); g += streams) emit(prefixes, g, a);
    }
}

// The 16-stream view of the fp16-operand scan (P <= 4): blocks in the i0 byte, and groups
// pooled across blocks when there are no two-index prefixes (P <= 3).
static void build_quads16(int d, int P, std::vector<sata::QuadRec> &out, std::vector<uint32_t> &flags) {
    build_quads(d, P, out, flags, 16, true, P <= 3);
}

static sata_status check_dims(int d_k, int d_v, int P) {
    if (d_k <= 0 || d_v <= 0) return fail(SATA_ERR_INVALID, "head dims must be positive (d_k=%d, d_v=%d)", d_k, d_v);
    if (P < 1) return fail(SATA_ERR_INVALID, "P must be >= 1 (got %d)", P);
    if (!supported_dim(d_k) || !supported_dim(d_v))
        return fail(SATA_ERR_UNSUPPORTED, "head dims must be 8, 16, 32, 64 or 128 (d_k=%d, d_v=%d)", d_k, d_v);
    if ((d_k == 128) != (d_v == 128))
        return fail(SATA_ERR_UNSUPPORTED, "d_k = 128 goes with d_v = 128 only (d_k=%d, d_v=%d)", d_k, d_v);
    if (P > sata::kMaxOrder + 1) return fail(SATA_ERR_UNSUPPORTED, "P <= %d supported (got %d)", sata::kMaxOrder + 1, P);
    return SATA_OK;
}

int64_t sata_describe_features(int d_k, int P, uint32_t *tuples, float *coef, int64_t cap) {
    g_last_error.clear();
    if (check_dims(d_k, d_k, P) != SATA_OK) return -1;
    std::vector<uint32_t> tup;
    std::vector<float> cf;
    build_tables(d_k, P, tup, cf);
    const int64_t m = (int64_t)tup.size();
    for (int64_t f = 0; f < m && f < cap; ++f) {
        if (tuples) tuples[f] = tup[(size_t)f];
        if (coef) coef[f] = cf[(size_t)f];
    }
    return m;
}

int64_t sata_describe_quads(int d_k, int P, uint32_t *w0, int32_t *cidx, float *coef4, int64_t cap) {
    g_last_error.clear();
    if (check_dims(d_k, d_k, P) != SATA_OK) return -1;
    std::vector<sata::QuadRec> quads;
    std::vector<uint32_t> flags;
    if (d_k <= kMaxPrefillDim) build_quads(d_k, P, quads, flags);   // no prefill (and no quads) above
    const int64_t nq = (int64_t)quads.size();
    for (int64_t i = 0; i < nq && i < cap; ++i) {
        if (w0) w0[i] = quads[(size_t)i].w0;
        if (cidx) cidx[i] = quads[(size_t)i].cidx;
        if (coef4)
            for (int z = 0; z < 4; ++z) coef4[4 * i + z] = quads[(size_t)i].coef[z];
    }
    return nq;
}

int64_t sata_describe_quads16(int d_k, int P, uint32_t *w0, int32_t *cidx, float *coef4, uint32_t *flags,
                              int64_t cap) {
    g_last_error.clear();
    if (check_dims(d_k, d_k, P) != SATA_OK) return -1;
    std::vector<sata::QuadRec> quads;
    std::vector<uint32_t> fl;
    if (P <= 4 && d_k >= 16 && d_k <= kMaxScan16Dim) build_quads16(d_k, P, quads, fl);
    const int64_t np = (int64_t)fl.size();
    for (int64_t p = 0; p < np && p < cap; ++p) {
        if (flags) flags[p] = fl[(size_t)p];
        for (int64_t i = 16 * p; i < 16 * p + 16; ++i) {
            if (w0) w0[i] = quads[(size_t)i].w0;
            if (cidx) cidx[i] = quads[(size_t)i].cidx;
            if (coef4)
                for (int z = 0; z < 4; ++z) coef4[4 * i + z] = quads[(size_t)i].coef[z];
        }
    }
    return np;
}

sata_status sata_build_index(int d_k, int d_v, int P, sata_index **out) {
    g_last_error.clear();
    if (!out) return fail(SATA_ERR_INVALID, "out is NULL");
    sata_status s = check_dims(d_k, d_v, P);
    if (s != SATA_OK) return s;

    std::vector<uint32_t> tup;
    std::vector<float> coef;
    build_tables(d_k, P, tup, coef);
    sata_index *idx = new (std::nothrow) sata_index();
    if (!idx) return fail(SATA_ERR_OOM, "host allocation failed");
    idx->dk = d_k;
    idx->dv = d_v;
    idx->P = P;
    idx->m = (int64_t)tup.size();
    idx->m_pad = round_up(idx->m, 64);
    idx->m_tab = round_up(idx->m, sata::kTablePad);
    double fact = 1.0;
    for (int p = 0; p < P; ++p) {
        if (p) fact *= p;
        idx->taylor[p] = (float)(1.0 / fact);
    }
    const uint32_t pad = (uint32_t)(d_k + 1) * 0x01010101u;   // slots -> constant 0
    tup.resize((size_t)idx->m_tab, pad);
    coef.resize((size_t)idx->m_tab, 0.f);
    std::vector<sata::QuadRec> quads;
    std::vector<uint32_t> qflags;
    if (d_k <= kMaxPrefillDim) build_quads(d_k, P, quads, qflags);   // prefill only
    idx->nq = (int64_t)quads.size();
    idx->nq_tab = round_up(std::max<int64_t>(idx->nq, 1), sata::kQuadPad);   // never empty (P = 1 has no quads)
    {
        sata::QuadRec padq{};
        padq.w0 = (uint32_t)(d_k + 1) | ((uint32_t)(d_k + 1) << 8) | ((uint32_t)d_k << 16);   // prefix product 0
        padq.cidx = -1;
        quads.resize((size_t)idx->nq_tab, padq);
        qflags.resize((size_t)(idx->nq_tab / 4), 2u);
    }
    // 16-stream positions for the fp16-operand scan (P <= 4, 16 <= d_K <= 128; block index
    // in a byte), padded with positions of padding quads (prefix product 0, block 0, flagged as
    // group starts) so that every slice of up to kPos16Pad positions lies inside the table
    std::vector<sata::QuadRec> quads16;
    std::vector<uint32_t> flags16;
    if (P <= 4 && d_k >= 16 && d_k <= kMaxScan16Dim) {
        build_quads16(d_k, P, quads16, flags16);
        idx->np16 = (int64_t)flags16.size();
        sata::QuadRec padq{};
        padq.w0 = (uint32_t)(d_k + 1) | ((uint32_t)(d_k + 1) << 8);
        padq.cidx = -1;
        quads16.resize((size_t)(idx->np16 + sata::kPos16Pad) * 16, padq);
        flags16.resize((size_t)(idx->np16 + sata::kPos16Pad), 2u);
    }
    std::vector<uint32_t> qw0(quads.size());
    std::vector<int32_t> qcidx(quads.size());
    std::vector<float> qcoef(quads.size() * 4);
    for (size_t i = 0; i < quads.size(); ++i) {
        qw0[i] = quads[i].w0;
        qcidx[i] = quads[i].cidx;
        for (int z = 0; z < 4; ++z) qcoef[i * 4 + z] = quads[i].coef[z];
    }
    if (hipGetDevice(&idx->device) != hipSuccess) {
        delete idx;
        (void)hipGetLastError();
        return fail(SATA_ERR_HIP, "no HIP device available");
    }
    {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, idx->device) == hipSuccess && cus > 0)
            idx->cus = cus;
        else
            (void)hipGetLastError();
    }
    auto release = [&]() {
        for (void *p : {(void *)idx->d_p16_w0, (void *)idx->d_p16_cidx, (void *)idx->d_p16_coef, (void *)idx->d_p16_flags})
            if (p) (void)hipFree(p);
        if (idx->d_tup) (void)hipFree(idx->d_tup);
        if (idx->d_coef) (void)hipFree(idx->d_coef);
        if (idx->d_qw0) (void)hipFree(idx->d_qw0);
        if (idx->d_qcidx) (void)hipFree(idx->d_qcidx);
        if (idx->d_qcoef) (void)hipFree(idx->d_qcoef);
        if (idx->d_qflags) (void)hipFree(idx->d_qflags);
        delete idx;
    };
    hipError_t e = hipMalloc(&idx->d_tup, tup.size() * sizeof(uint32_t));
    if (e == hipSuccess) e = hipMalloc(&idx->d_coef, coef.size() * sizeof(float));
    if (e == hipSuccess) e = hipMalloc(&idx->d_qw0, qw0.size() * sizeof(uint32_t));
    if (e == hipSuccess) e = hipMalloc(&idx->d_qcidx, qcidx.size() * sizeof(int32_t));
    if (e == hipSuccess) e = hipMalloc(&idx->d_qcoef, qcoef.size() * sizeof(float));
    if (e == hipSuccess) e = hipMalloc(&idx->d_qflags, qflags.size() * sizeof(uint32_t));
    std::vector<uint32_t> p16w0(quads16.size());
    std::vector<int32_t> p16cidx(quads16.size());
    std::vector<float> p16coef(quads16.size() * 4);
    for (size_t i = 0; i < quads16.size(); ++i) {
        p16w0[i] = quads16[i].w0;
        p16cidx[i] = quads16[i].cidx;
        for (int z = 0; z < 4; ++z) p16coef[i * 4 + z] = quads16[i].coef[z];
    }
    if (!quads16.empty()) {
        if (e == hipSuccess) e = hipMalloc(&idx->d_p16_w0, p16w0.size() * sizeof(uint32_t));
        if (e == hipSuccess) e = hipMalloc(&idx->d_p16_cidx, p16cidx.size() * sizeof(int32_t));
        if (e == hipSuccess) e = hipMalloc(&idx->d_p16_coef, p16coef.size() * sizeof(float));
        if (e == hipSuccess) e = hipMalloc(&idx->d_p16_flags, flags16.size() * sizeof(uint32_t));
    }
    if (e != hipSuccess) {
        (void)hipGetLastError();
        release();
        return fail(SATA_ERR_OOM, "index allocation failed");
    }
    e = hipMemcpy(idx->d_tup, tup.data(), tup.size() * sizeof(uint32_t), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(idx->d_coef, coef.data(), coef.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(idx->d_qw0, qw0.data(), qw0.size() * sizeof(uint32_t), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(idx->d_qcidx, qcidx.data(), qcidx.size() * sizeof(int32_t), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(idx->d_qcoef, qcoef.data(), qcoef.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e == hipSuccess)
        e = hipMemcpy(idx->d_qflags, qflags.data(), qflags.size() * sizeof(uint32_t), hipMemcpyHostToDevice);
    if (!quads16.empty()) {
        if (e == hipSuccess)
            e = hipMemcpy(idx->d_p16_w0, p16w0.data(), p16w0.size() * sizeof(uint32_t), hipMemcpyHostToDevice);
        if (e == hipSuccess)
            e = hipMemcpy(idx->d_p16_cidx, p16cidx.data(), p16cidx.size() * sizeof(int32_t), hipMemcpyHostToDevice);
        if (e == hipSuccess)
            e = hipMemcpy(idx->d_p16_coef, p16coef.data(), p16coef.size() * sizeof(float), hipMemcpyHostToDevice);
        if (e == hipSuccess)
            e = hipMemcpy(idx->d_p16_flags, flags16.data(), flags16.size() * sizeof(uint32_t), hipMemcpyHostToDevice);
    }
    if (e != hipSuccess) {
        release();
        return fail_hip(e, "index upload");
    }
    *out = idx;
    return SATA_OK;
}

void sata_index_free(sata_index *idx) {
    if (!idx) return;
    DeviceGuard g(idx->device);
    if (idx->d_tup) (void)hipFree(idx->d_tup);
    if (idx->d_coef) (void)hipFree(idx->d_coef);
    if (idx->d_qw0) (void)hipFree(idx->d_qw0);
    if (idx->d_qcidx) (void)hipFree(idx->d_qcidx);
    if (idx->d_qcoef) (void)hipFree(idx->d_qcoef);
    if (idx->d_qflags) (void)hipFree(idx->d_qflags);
    for (void *p : {(void *)idx->d_p16_w0, (void *)idx->d_p16_cidx, (void *)idx->d_p16_coef, (void *)idx->d_p16_flags})
        if (p) (void)hipFree(p);
    if (idx->lower) sata_index_free(idx->lower);
    sata::free_backward_pool(idx);
    delete idx;
}

int64_t sata_index_features(const sata_index *idx) { return idx ? idx->m : -1; }

sata_status sata_index_info(const sata_index *idx, int *d_k, int *d_v, int *P, int64_t *m, int64_t *m_pad) {
    if (!idx) return fail(SATA_ERR_INVALID, "index is NULL");
    if (d_k) *d_k = idx->dk;
    if (d_v) *d_v = idx->dv;
    if (P) *P = idx->P;
    if (m) *m = idx->m;
    if (m_pad) *m_pad = idx->m_pad;
    return SATA_OK;
}

sata_status sata_state_alloc_dtype(const sata_index *idx, int batch, int heads, sata_dtype state_dt, void *stream,
                                   sata_state **out) {
    g_last_error.clear();
    if (!idx) return fail(SATA_ERR_INVALID, "index is NULL");
    if (!out) return fail(SATA_ERR_INVALID, "out is NULL");
    if (batch < 1 || heads < 1) return fail(SATA_ERR_INVALID, "batch and heads must be >= 1 (%d, %d)", batch, heads);
    if (!valid_state_dtype(state_dt)) return fail(SATA_ERR_INVALID, "unknown state dtype");
    const int64_t bh = (int64_t)batch * heads;
    if (bh > 65535) return fail(SATA_ERR_UNSUPPORTED, "batch*heads <= 65535 supported (got %lld)", (long long)bh);
    DeviceGuard g(idx->device);
    if (!g.ok) return fail(SATA_ERR_HIP, "cannot select the index's device");
    sata_state *st = new (std::nothrow) sata_state();
    if (!st) return fail(SATA_ERR_OOM, "host allocation failed");
    st->idx = idx;
    st->batch = batch;
    st->heads = heads;
    st->device = idx->device;
    st->dtype = state_dt;
    // m_pad is a multiple of 64, so the main array's byte size is a multiple of 128 for any
    // element type; an fp16 state's fp32 words of the lowest orders follow it
    const int64_t main_bytes = bh * (idx->dv + 1) * idx->m_pad * dtype_bytes(state_dt);
    st->m_low = state_dt == SATA_F16 ? f16_low_features(idx) : 0;
    st->state_bytes = main_bytes + bh * (idx->dv + 1) * st->m_low * (int64_t)sizeof(float);
    hipError_t e = hipMalloc(&st->d_state, (size_t)st->state_bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        const long long nbytes = (long long)st->state_bytes;
        delete st;
        return fail(SATA_ERR_OOM, "state allocation of %lld bytes failed", nbytes);
    }
    if (st->m_low) st->d_low = reinterpret_cast<float *>(static_cast<char *>(st->d_state) + main_bytes);
    e = hipHostMalloc(reinterpret_cast<void **>(&st->h_err), sizeof(uint32_t),
                      hipHostMallocMapped | hipHostMallocCoherent);
    if (e == hipSuccess) {
        *st->h_err = 0u;
        e = hipHostGetDevicePointer(reinterpret_cast<void **>(&st->d_err), st->h_err, 0);
    }
    if (e != hipSuccess) {
        (void)hipGetLastError();
        if (st->h_err) (void)hipHostFree(st->h_err);
        (void)hipFree(st->d_state);
        delete st;
        return fail(SATA_ERR_OOM, "pinned error word allocation failed");
    }
    e = sata::launch_zero(static_cast<float *>(st->d_state), st->state_bytes / 4, (hipStream_t)stream);
    if (e != hipSuccess) {
        (void)hipHostFree(st->h_err);
        (void)hipFree(st->d_state);
        delete st;
        return fail_hip(e, "state clear");
    }
    *out = st;
    return SATA_OK;
}

sata_status sata_state_alloc(const sata_index *idx, int batch, int heads, void *stream, sata_state **out) {
    return sata_state_alloc_dtype(idx, batch, heads, SATA_F32, stream, out);
}

sata_status sata_state_convert(sata_state *src, sata_state *dst, void *stream) {
    g_last_error.clear();
    if (!src || !dst) return fail(SATA_ERR_INVALID, "src and dst must be non-NULL");
    if (src == dst) return fail(SATA_ERR_INVALID, "src and dst must be different states");
    if (src->idx != dst->idx) return fail(SATA_ERR_INVALID, "src and dst were allocated for different indexes");
    if (src->batch != dst->batch || src->heads != dst->heads)
        return fail(SATA_ERR_INVALID, "src and dst differ in batch or heads");
    DeviceGuard g(dst->device);
    if (!g.ok) return fail(SATA_ERR_HIP, "cannot select the state's device");
    sata_status s = flush_pending(src, (hipStream_t)stream);
    if (s != SATA_OK) return s;
    hipError_t e = sata::launch_state_convert(src, dst, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "state conversion");
    dst->npend = 0;
    return SATA_OK;
}

sata_status sata_state_reset(sata_state *st, void *stream) {
    g_last_error.clear();
    if (!st) return fail(SATA_ERR_INVALID, "state is NULL");
    DeviceGuard g(st->device);
    hipError_t e = sata::launch_zero(static_cast<float *>(st->d_state), st->state_bytes / 4, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "state clear");
    st->npend = 0;
    return SATA_OK;
}

void sata_state_free(sata_state *st) {
    if (!st) return;
    DeviceGuard g(st->device);
    if (st->d_state) (void)hipFree(st->d_state);
    if (st->d_work) (void)hipFree(st->d_work);
    if (st->d_pend_k) (void)hipFree(st->d_pend_k);
    if (st->d_pend_v) (void)hipFree(st->d_pend_v);
    if (st->h_err) (void)hipHostFree(st->h_err);
    delete st;
}

sata_status sata_state_data(const sata_state *st, void **dev_ptr, int64_t *bytes) {
    if (!st) return fail(SATA_ERR_INVALID, "state is NULL");
    if (dev_ptr) *dev_ptr = st->d_state;
    if (bytes) *bytes = st->state_bytes;
    return SATA_OK;
}

sata_status sata_prefill(const sata_index *idx, sata_state *st, const void *q, const void *k, const void *v,
                         void *out, int64_t n, int chunk, sata_dtype in_dt, sata_dtype out_dt, void *stream) {
    g_last_error.clear();
    bool nothing = false;
    sata_status s = check_prefill_args(idx, st, q, k, v, out, n, chunk, in_dt, out_dt, &nothing);
    if (s != SATA_OK || nothing) return s;
    const int64_t bh = (int64_t)st->batch * st->heads;
    if (idx->dk > kMaxPrefillDim && !sata::scan16_covers(idx, in_dt)) {
        // d_K = 128 outside the fp16-operand scan (fp32 inputs, five orders): blocks of up to
        // kMaxDecodeWindow tokens through the state in HBM (the chunk length does not apply)
        DeviceGuard g(st->device);
        if (!g.ok) return fail(SATA_ERR_HIP, "cannot select the state's device");
        s = ensure_pending(st);
        if (s != SATA_OK) return s;
        s = ensure_work(st, std::max(sata::block_prefill_workspace_bytes(idx, bh), sata::decode_workspace_bytes(idx, bh)));
        if (s != SATA_OK) return s;
        s = flush_pending(st, (hipStream_t)stream);
        if (s != SATA_OK) return s;
        hipError_t e = sata::launch_block_prefill(idx, st, q, k, v, out, n, in_dt, out_dt, (hipStream_t)stream);
        if (e != hipSuccess) return fail_hip(e, "block prefill launch");
        return SATA_OK;
    }
    DeviceGuard g(st->device);
    if (!g.ok) return fail(SATA_ERR_HIP, "cannot select the state's device");
    // Plan under the default workspace cap; if that workspace cannot be allocated, plan again
    // under half the previous workspace (fewer chunks per segment), down to one chunk.
    sata::PrefillPlan plan;
    for (int64_t cap = sata::kWorkCap;;) {
        plan = sata::plan_prefill(idx, bh, n, chunk, in_dt, cap);
        if (!plan.ok) return fail(SATA_ERR_UNSUPPORTED, "no prefill plan for this configuration");
        s = ensure_work(st, plan.work_bytes);
        if (s == SATA_OK) break;
        if (s != SATA_ERR_OOM || plan.seg_chunks <= 1) return s;
        cap = plan.work_bytes / 2;
    }
    s = flush_pending(st, (hipStream_t)stream);
    if (s != SATA_OK) return s;
    hipError_t e = sata::launch_prefill(idx, st, plan, q, k, v, out, n, in_dt, out_dt, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "prefill launch");
    return SATA_OK;
}

sata_status sata_prefill_noalloc(const sata_index *idx, sata_state *st, const void *q, const void *k, const void *v,
                                 void *out, int64_t n, int chunk, sata_dtype in_dt, sata_dtype out_dt, void *stream) {
    g_last_error.clear();
    bool nothing = false;
    sata_status s = check_prefill_args(idx, st, q, k, v, out, n, chunk, in_dt, out_dt, &nothing);
    if (s != SATA_OK || nothing) return s;
    if (idx->dk > kMaxPrefillDim && !sata::scan16_covers(idx, in_dt))
        return fail(SATA_ERR_UNSUPPORTED,
                    "the allocation-free prefill covers d_k <= %d, and d_k = 128 for bf16 inputs with P <= 4 "
                    "(got d_k=%d, P=%d)", kMaxPrefillDim, idx->dk, idx->P);
    const int64_t bh = (int64_t)st->batch * st->heads;
    ProfOff quiet;   // no timing events for any launch of this call
    DeviceGuard g(st->device);
    if (!g.ok) return fail(SATA_ERR_HIP, "cannot select the state's device");
    void *scr = nullptr;
    s = scratch_address(st->device, &scr);
    if (s != SATA_OK) return s;
    // segments sized to the scratch array; a call whose single-chunk segments still need more
    // (many heads) is refused
    const sata::PrefillPlan plan = sata::plan_prefill(idx, bh, n, chunk, in_dt, SATA_NOALLOC_SCRATCH_BYTES);
    if (!plan.ok) return fail(SATA_ERR_UNSUPPORTED, "no prefill plan for this configuration");
    if (plan.work_bytes > SATA_NOALLOC_SCRATCH_BYTES)
        return fail(SATA_ERR_UNSUPPORTED,
                    "this prefill needs a workspace of %lld bytes; the allocation-free scratch holds %lld "
                    "(use sata_prefill, or fewer heads per call)",
                    (long long)plan.work_bytes, (long long)SATA_NOALLOC_SCRATCH_BYTES);
    // deferred decode tokens fold into the state first; their buffers (and the decode
    // workspace) exist whenever there are any, so this allocates nothing either
    s = flush_pending(st, (hipStream_t)stream);
    if (s != SATA_OK) return s;
    sata_state view = *st;   // the same state, with the scratch array as its workspace
    view.d_work = scr;
    view.work_bytes = SATA_NOALLOC_SCRATCH_BYTES;
    hipError_t e = sata::launch_prefill(idx, &view, plan, q, k, v, out, n, in_dt, out_dt, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "allocation-free prefill launch");
    return SATA_OK;
}

sata_status sata_measure_mfma_loop(int bf16, double *tflops) {
    g_last_error.clear();
    if (!tflops) return fail(SATA_ERR_INVALID, "tflops is NULL");
    const hipError_t e = sata::measure_mfma_loop(bf16 != 0, tflops);
    if (e != hipSuccess) return fail_hip(e, "MFMA loop measurement");
    return SATA_OK;
}

sata_status sata_prefill_backward(const sata_index *idx, int batch, int heads, const void *q, const void *k,
                                  const void *v, const void *dout, void *dq, void *dk, void *dv, int64_t n, int chunk,
                                  sata_dtype in_dt, sata_dtype grad_dt, void *stream) {
    g_last_error.clear();
    if (!idx) return fail(SATA_ERR_INVALID, "index is NULL");
    if (batch < 1 || heads < 1) return fail(SATA_ERR_INVALID, "batch and heads must be >= 1 (%d, %d)", batch, heads);
    if (n < 0) return fail(SATA_ERR_INVALID, "n must be >= 0 (got %lld)", (long long)n);
    if (!valid_dtype(in_dt) || !valid_dtype(grad_dt)) return fail(SATA_ERR_INVALID, "unknown dtype");
    if (chunk != 0 && chunk != 64 && chunk != 128)
        return fail(SATA_ERR_UNSUPPORTED, "chunk must be 0 (default), 64 or 128 (got %d)", chunk);
    if (idx->dk != idx->dv) return fail(SATA_ERR_UNSUPPORTED, "the backward pass needs d_k == d_v");
    // above 64 every pass must run on the fp16-operand scan: bf16 inputs, and P - 1 orders that
    // still have features beyond order 0
    if (idx->dk > kMaxPrefillDim && !(sata::scan16_covers(idx, in_dt) && idx->P >= 3))
        return fail(SATA_ERR_UNSUPPORTED,
                    "the backward pass supports d_k <= %d, or d_k = %d with bf16 inputs and 3 <= P <= 4 "
                    "(got d_k=%d, P=%d)", kMaxPrefillDim, kMaxScan16Dim, idx->dk, idx->P);
    const int64_t bh = (int64_t)batch * heads;
    if (bh > 65535) return fail(SATA_ERR_UNSUPPORTED, "batch*heads <= 65535 supported (got %lld)", (long long)bh);
    if (n == 0) return SATA_OK;
    const void *ins[4] = {q, k, v, dout};
    void *outs[3] = {dq, dk, dv};
    for (const void *p : ins)
        if (!p || !aligned16(p)) return fail(SATA_ERR_INVALID, "q, k, v and dout must be non-NULL and 16-byte aligned");
    for (void *p : outs)
        if (!p || !aligned16(p)) return fail(SATA_ERR_INVALID, "dq, dk and dv must be non-NULL and 16-byte aligned");
    const int64_t nin = bh * n * idx->dk * dtype_bytes(in_dt), nout = bh * n * idx->dk * dtype_bytes(grad_dt);
    for (int a = 0; a < 3; ++a) {
        for (const void *i : ins)
            if (overlaps(outs[a], nout, i, nin)) return fail(SATA_ERR_INVALID, "gradients overlap the inputs");
        for (int b = a + 1; b < 3; ++b)
            if (overlaps(outs[a], nout, outs[b], nout)) return fail(SATA_ERR_INVALID, "gradients overlap each other");
    }
    DeviceGuard g(idx->device);
    if (!g.ok) return fail(SATA_ERR_HIP, "cannot select the index's device");
    const sata_index *lower = nullptr;
    if (idx->P >= 2) {
        std::lock_guard<std::mutex> lock(idx->lower_mu);
        if (!idx->lower) {
            sata_index *built = nullptr;
            sata_status s = sata_build_index(idx->dk, idx->dv, idx->P - 1, &built);
            if (s != SATA_OK) return s;
            idx->lower = built;
        }
        lower = idx->lower;
    }
    const int64_t kBudget = (int64_t)8 << 30;   // bytes of per-column temporaries per pass
    std::lock_guard<std::mutex> pool_lock(idx->bw_mu);   // the index's pool of temporaries
    hipError_t e = sata::launch_backward(idx, lower, bh, q, k, v, dout, dq, dk, dv, n, chunk, in_dt, grad_dt, kBudget,
                                         (hipStream_t)stream);
    if (e == hipErrorMemoryAllocation || e == hipErrorOutOfMemory) {
        (void)hipGetLastError();
        return fail(SATA_ERR_OOM, "backward temporaries could not be allocated");
    }
    if (e == hipErrorLaunchTimeOut)
        return fail(SATA_ERR_HIP, "backward: a prefill scan work item gave up waiting for the state of its "
                                  "predecessor (the gradients are invalid)");
    if (e != hipSuccess) {
        const std::string what = std::string("backward (") + sata::backward_last_step() + ")";
        return fail_hip(e, what.c_str());
    }
    return SATA_OK;
}

sata_status sata_decode_step(const sata_index *idx, sata_state *st, const void *q, const void *k, const void *v,
                             void *out, sata_dtype in_dt, sata_dtype out_dt, void *stream) {
    g_last_error.clear();
    sata_status s = check_index_state(idx, st);
    if (s != SATA_OK) return s;
    if (!valid_dtype(in_dt) || !valid_dtype(out_dt)) return fail(SATA_ERR_INVALID, "unknown dtype");
    if (!q || !k || !v || !out) return fail(SATA_ERR_INVALID, "q, k, v and out must be non-NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(SATA_ERR_INVALID, "q, k, v and out must be 16-byte aligned");
    s = take_state_error(st);
    if (s != SATA_OK) return s;
    const int64_t bh = (int64_t)st->batch * st->heads;
    const int64_t in_b = dtype_bytes(in_dt), out_b = dtype_bytes(out_dt);
    const int64_t nq = bh * idx->dk * in_b, nv = bh * idx->dv * in_b, no = bh * idx->dv * out_b;
    if (overlaps(out, no, q, nq) || overlaps(out, no, k, nq) || overlaps(out, no, v, nv))
        return fail(SATA_ERR_INVALID, "out overlaps q, k or v");
    DeviceGuard g(st->device);
    if (!g.ok) return fail(SATA_ERR_HIP, "cannot select the state's device");
    s = ensure_work(st, sata::decode_workspace_bytes(idx, bh));
    if (s != SATA_OK) return s;
    const sata::DecodeMode mode = st->window <= 1              ? sata::kDecodePlain
                                  : st->npend + 1 < st->window ? sata::kDecodeRead
                                                               : sata::kDecodeFold;
    hipError_t e = sata::launch_decode(idx, st, q, k, v, out, in_dt, out_dt, mode, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "decode launch");
    if (mode == sata::kDecodeRead) ++st->npend;
    if (mode == sata::kDecodeFold) st->npend = 0;
    return SATA_OK;
}

sata_status sata_state_set_decode_window(sata_state *st, int window, void *stream) {
    g_last_error.clear();
    if (!st) return fail(SATA_ERR_INVALID, "state is NULL");
    if (window < 1 || window > kMaxDecodeWindow)
        return fail(SATA_ERR_INVALID, "window must be in [1, %d] (got %d)", kMaxDecodeWindow, window);
    DeviceGuard g(st->device);
    if (!g.ok) return fail(SATA_ERR_HIP, "cannot select the state's device");
    if (window > 1) {
        sata_status sp = ensure_pending(st);
        if (sp != SATA_OK) return sp;
    }
    sata_status s = flush_pending(st, (hipStream_t)stream);
    if (s != SATA_OK) return s;
    st->window = window;
    return SATA_OK;
}

sata_status sata_state_flush(sata_state *st, void *stream) {
    g_last_error.clear();
    if (!st) return fail(SATA_ERR_INVALID, "state is NULL");
    DeviceGuard g(st->device);
    if (!g.ok) return fail(SATA_ERR_HIP, "cannot select the state's device");
    sata_status s = take_state_error(st);
    if (s != SATA_OK) return s;
    return flush_pending(st, (hipStream_t)stream);
}

sata_status sata_state_check(sata_state *st, void *stream) {
    g_last_error.clear();
    if (!st) return fail(SATA_ERR_INVALID, "state is NULL");
    DeviceGuard g(st->device);
    if (!g.ok) return fail(SATA_ERR_HIP, "cannot select the state's device");
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "stream synchronisation");
    return take_state_error(st);
}

sata_status sata_debug_scan_faults(int item_base, int spin_limit) {
    g_last_error.clear();
    if (item_base < 0) return fail(SATA_ERR_INVALID, "item_base must be >= 0 (got %d)", item_base);
    if (spin_limit < 0) return fail(SATA_ERR_INVALID, "spin_limit must be >= 0 (got %d)", spin_limit);
    g_debug_item_base.store(item_base, std::memory_order_relaxed);
    g_debug_spin_limit.store(spin_limit ? spin_limit : sata::kScanSpinLimit, std::memory_order_relaxed);
    return SATA_OK;
}

sata_status sata_debug_prefill_positions(int mt) {
    g_last_error.clear();
    if (mt != 0 && mt != 1 && mt != 2 && mt != 3 && mt != 5)
        return fail(SATA_ERR_INVALID, "positions per update wavefront must be 0, 1, 2, 3 or 5 (got %d)", mt);
    g_debug_positions.store(mt, std::memory_order_relaxed);
    return SATA_OK;
}

sata_status sata_debug_prefill_refresh(int chunks) {
    g_last_error.clear();
    if (chunks < 0 || chunks > 16)
        return fail(SATA_ERR_INVALID, "chunks per state-copy refresh must be 0 (the rule) or 1 .. 16 (got %d)", chunks);
    g_debug_refresh.store(chunks, std::memory_order_relaxed);
    return SATA_OK;
}

int64_t sata_describe_prefill_plan(int d_k, int P, int64_t batch_heads, int64_t n, int chunk, int in_dt,
                                   int64_t work_cap, int64_t *seg_chunks, int64_t *slices) {
    g_last_error.clear();
    if (check_dims(d_k, d_k, P) != SATA_OK) return -1;
    // chunked plans: d_K <= 64, and d_K = 128 on the fp16-operand scan (bf16 inputs, P <= 4)
    const bool wide = d_k > kMaxPrefillDim && d_k <= kMaxScan16Dim && P <= 4 && in_dt == SATA_BF16;
    if ((d_k > kMaxPrefillDim && !wide) || batch_heads < 1 || n < 1 || !valid_dtype(in_dt) || work_cap < 1 ||
        (chunk != 0 && chunk != 64 && chunk != 128)) {
        fail(SATA_ERR_INVALID, "no chunked prefill plan for these arguments");
        return -1;
    }
    // the plan reads only the index's shape and quad count: a host-only stand-in suffices
    sata_index idx;
    idx.dk = idx.dv = d_k;
    idx.P = P;
    std::vector<sata::QuadRec> quads;
    std::vector<uint32_t> flags;
    if (!wide) build_quads(d_k, P, quads, flags);
    idx.nq = (int64_t)quads.size();
    idx.nq_tab = round_up(std::max<int64_t>(idx.nq, 1), sata::kQuadPad);
    if (P <= 4 && d_k >= 16) {
        std::vector<sata::QuadRec> q16;
        std::vector<uint32_t> f16;
        build_quads16(d_k, P, q16, f16);
        idx.np16 = (int64_t)f16.size();
    }
    const sata::PrefillPlan plan = sata::plan_prefill(&idx, batch_heads, n, chunk, (sata_dtype)in_dt, work_cap);
    if (!plan.ok) {
        fail(SATA_ERR_UNSUPPORTED, "no prefill plan for this configuration");
        return -1;
    }
    if (seg_chunks) *seg_chunks = plan.seg_chunks;
    if (slices) *slices = plan.slices;
    return plan.work_bytes;
}

sata_status sata_expand_features(const sata_index *idx, const void *x, void *out, int64_t rows, int side,
                                 sata_dtype in_dt, void *stream) {
    g_last_error.clear();
    if (!idx) return fail(SATA_ERR_INVALID, "index is NULL");
    if (rows < 0) return fail(SATA_ERR_INVALID, "rows must be >= 0");
    if (side != 0 && side != 1) return fail(SATA_ERR_INVALID, "side must be 0 (key) or 1 (query)");
    if (!valid_dtype(in_dt)) return fail(SATA_ERR_INVALID, "unknown dtype");
    if (rows > 65535) return fail(SATA_ERR_UNSUPPORTED, "rows <= 65535 per call");
    if (rows == 0) return SATA_OK;
    if (!x || !out) return fail(SATA_ERR_INVALID, "x and out must be non-NULL");
    if (overlaps(out, rows * idx->m_pad * 4, x, rows * idx->dk * dtype_bytes(in_dt)))
        return fail(SATA_ERR_INVALID, "out overlaps x");
    DeviceGuard g(idx->device);
    hipError_t e = sata::launch_expand(idx, x, out, rows, side, in_dt, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "expand launch");
    return SATA_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- profiling

#include <mutex>

namespace {

struct ProfRecord {
    int kernel;
    hipEvent_t a, b;
};

std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRecord> g_prof;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
    // caller holds g_prof_mu
    if (!g_prof_pool.empty()) {
        hipEvent_t e = g_prof_pool.back();
        g_prof_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    return e;
}

void prof_clear_locked() {
    for (auto &r : g_prof) {
        g_prof_pool.push_back(r.a);
        g_prof_pool.push_back(r.b);
    }
    g_prof.clear();
}

const char *const kProfNames[sata::kProfCount] = {"prefill_scan", "prefill_combine", "decode_stream",
                                                   "decode_finish", "decode_read", "decode_fold", "decode_low"};

}  // namespace

namespace sata {

ProfScope::ProfScope(int k, hipStream_t s) : kernel(k), stream(s) {
    if (t_prof_off) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on) return;
    start = prof_event();
    if (start && hipEventRecord(start, stream) != hipSuccess) {
        (void)hipGetLastError();
        g_prof_pool.push_back(start);
        start = nullptr;
    }
}

ProfScope::~ProfScope() {
    if (!start) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    hipEvent_t stop = prof_event();
    if (!stop || hipEventRecord(stop, stream) != hipSuccess) {
        (void)hipGetLastError();
        g_prof_pool.push_back(start);
        if (stop) g_prof_pool.push_back(stop);
        return;
    }
    g_prof.push_back({kernel, start, stop});
}

}  // namespace sata

extern "C" {

sata_status sata_profile_enable(int on) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (on) prof_clear_locked();
    g_prof_on = on != 0;
    return SATA_OK;
}

sata_status sata_profile_query(int kernel, double *total_ms, int64_t *launches) {
    if (kernel < 0 || kernel >= sata::kProfCount) return fail(SATA_ERR_INVALID, "unknown kernel id %d", kernel);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    double tot = 0.0;
    int64_t cnt = 0;
    for (auto &r : g_prof) {
        if (r.kernel != kernel) continue;
        hipError_t e = hipEventSynchronize(r.b);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
        if (e != hipSuccess) return fail_hip(e, "profile event");
        tot += ms;
        ++cnt;
    }
    if (total_ms) *total_ms = tot;
    if (launches) *launches = cnt;
    return SATA_OK;
}

const char *sata_profile_kernel_name(int kernel) {
    if (kernel < 0 || kernel >= sata::kProfCount) return nullptr;
    return kProfNames[kernel];
}

}  // extern "C"
