// Backward pass of the causal prefill, in the state form.
//
// With x_ij = q_i.k_j / sqrt(d), w(x) = sum_{p<P} x^p/p!, z_i = sum_{j<=i} w(x_ij)
// and o_i = sum_{j<=i} w(x_ij) v_j / z_i, the gradients of a loss L with
// dO_i = dL/do_i are, with g_i = [dO_i, -dO_i.o_i] / z_i (d_V + 1 values) and
// w'(x) = sum_{p<P-1} x^p/p! (the derivative of the truncated series):
//
//   dv_j = sum_{i>=j} w(x_ij) g_i[:d_V]
//   dk_j = (1/sqrt d) sum_c [v_j, 1][c] sum_{i>=j} w'(x_ij) g_i[c] q_i
//   dq_i = (1/sqrt d) sum_c g_i[c] sum_{j<=i} w'(x_ij) [v_j, 1][c] k_j
//
// Each inner sum is a causal Taylor attention without the normalisation: dq's
// with P-1 orders, keys k and values [v_j,1][c] k_j; dv's and dk's are
// anti-causal (i >= j), which is causal on the time-reversed sequences with
// the roles of q and k exchanged.  So the whole backward runs on the forward
// prefill kernels (a fixed state per head, constant work per token [hotdry,
// "Engineering realisation of the constant compute cost"]): one forward pass
// to recover o and z, one for dv, and for dk and dq one pass each over
// (d_V + 1) pseudo-heads per head (one per column c, in groups that bound the
// temporary memory), followed by element-wise contractions over c.
//
//   [hotdry] blog.hotdry.top, "Symmetry-aware Taylor approximation attention:
//            engineering a constant per-token cost" (2026-02-05).
#include <algorithm>
#include <vector>

#include "sata_device.h"
#include "sata_internal.h"

namespace sata {

namespace {

constexpr int kBwThreads = 256;

inline unsigned bw_grid(int64_t n) { return (unsigned)std::min<int64_t>((n + kBwThreads - 1) / kBwThreads, 1 << 20); }
// Grid of the per-element kernels over [heads][n][D] (D a power of two): x strides one head's
// n x D elements, y is the head, so element indices need shifts and masks, no division.
inline dim3 bw_grid2(int64_t n, int D, int64_t heads) {
    return dim3((unsigned)std::min<int64_t>((n * D + kBwThreads - 1) / kBwThreads, 4096), (unsigned)heads);
}
#define BW_ELEMENTS(j, n, lgD) \
    for (int64_t j = (int64_t)blockIdx.x * kBwThreads + threadIdx.x; j < ((n) << (lgD)); j += (int64_t)gridDim.x * kBwThreads)

// g_i = [dO_i / z_i, -(dO_i . o_i) / z_i], one thread per token.
template <typename TIn>
__global__ __launch_bounds__(kBwThreads) void bw_prep_g(const TIn *__restrict__ dout, const float *__restrict__ o,
                                                        const float *__restrict__ z, float *__restrict__ g,
                                                        int64_t tokens, int D) {
    for (int64_t t = (int64_t)blockIdx.x * kBwThreads + threadIdx.x; t < tokens; t += (int64_t)gridDim.x * kBwThreads) {
        const float rz = 1.f / z[t];
        float dot = 0.f;
        for (int c = 0; c < D; ++c) {
            const float d = to_f32(dout[t * D + c]);
            dot += d * o[t * D + c];
            g[t * (D + 1) + c] = d * rz;
        }
        g[t * (D + 1) + D] = -dot * rz;
    }
}

// out[h][t][:] = in[h][n-1-t][:] (the time-reversed sequence of every head); grid bw_grid2.
template <typename T>
__global__ __launch_bounds__(kBwThreads) void bw_reverse(const T *__restrict__ in, T *__restrict__ out, int64_t n,
                                                         int lgD) {
    const int64_t base = (int64_t)blockIdx.y * n << lgD;
    BW_ELEMENTS(j, n, lgD) {
        const int64_t t = j >> lgD, d = j & ((1 << lgD) - 1);
        out[base + j] = in[base + ((n - 1 - t) << lgD) + d];
    }
}

// Largest |g| of the call into *bits (the bit pattern of a non-negative float, which orders like
// an unsigned integer; *bits starts at 0).
__global__ __launch_bounds__(kBwThreads) void bw_absmax(const float *__restrict__ g, int64_t total,
                                                        unsigned *__restrict__ bits) {
    __shared__ unsigned part[kBwThreads / 64];
    unsigned m = 0;
    for (int64_t i = (int64_t)blockIdx.x * kBwThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kBwThreads)
        m = max(m, __float_as_uint(fabsf(g[i])));
    for (int off = 32; off > 0; off >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, off));
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kBwThreads / 64; ++w) m = max(m, part[w]);
        atomicMax(bits, m);
    }
}

// The power of two that the gradient-weighted values of the dv and dk passes are multiplied by
// before they are rounded to the input type: it brings the largest |g| into [2^8, 2^9), so that
// the fp16 operands of the fp16-operand scan hold them in their normal range (g = dout / z
// shrinks with the token count).  Scaling by a power of two commutes with every rounding of the
// passes; the results are multiplied back by the inverse.  1 when g is zero or not finite.
constexpr int kBwValueExp = 9;
__device__ __forceinline__ float bw_value_scale(const unsigned *bits, bool inverse) {
    const float m = __uint_as_float(*bits);
    if (!(m > 0.f) || !(m < INFINITY)) return 1.f;
    const int e = __builtin_amdgcn_frexp_expf(m);   // m in [2^(e-1), 2^e)
    return __builtin_amdgcn_ldexpf(1.f, inverse ? e - kBwValueExp : kBwValueExp - e);
}

// values of the dv pass: out[h][t][d] = g[h][n-1-t][d] (scaled), d < D; TV is the input type,
// or binary16 for a pass on the fp16-operand scan.
template <typename TV>
__global__ __launch_bounds__(kBwThreads) void bw_rev_g(const float *__restrict__ g, const unsigned *__restrict__ gmax,
                                                       TV *__restrict__ out, int64_t n, int lgD) {
    const int64_t h = blockIdx.y, D = 1 << lgD;
    const float vs = bw_value_scale(gmax, false);
    BW_ELEMENTS(j, n, lgD) {
        const int64_t t = j >> lgD, d = j & (D - 1);
        out[(h * n << lgD) + j] = from_f32<TV>(g[(h * n + (n - 1 - t)) * (D + 1) + d] * vs);
    }
}

// Inputs of one column group [c0, c0 + cg) of the dk pass (kdk = 1) or the dq
// pass (kdk = 0), pseudo-head ph = h * cg + cc for column c = c0 + cc:
//   dk: q' = rev(k), k' = rev(q), v'[t] = g[n-1-t][c] q[n-1-t] (scaled)
//   dq: q' = q,      k' = k,      v'[t] = [v, 1][t][c] k[t]
// q' and k' are written only when qo is given (a pass whose pseudo-heads read the head's
// own q' and k' in place needs v' alone); v' is of TV (the input type, or binary16 for a pass
// on the fp16-operand scan).
template <typename TIn, typename TV>
__global__ __launch_bounds__(kBwThreads) void bw_group_inputs(const TIn *__restrict__ q, const TIn *__restrict__ k,
                                                              const TIn *__restrict__ v, const float *__restrict__ g,
                                                              const unsigned *__restrict__ gmax,
                                                              TIn *__restrict__ qo, TIn *__restrict__ ko,
                                                              TV *__restrict__ vo, int64_t n, int lgD, int c0, int cg,
                                                              int kdk) {
    const int ph = blockIdx.y;                                  // grid bw_grid2 over the pseudo-heads
    const int64_t h = ph / cg, D = 1 << lgD;
    const int c = c0 + ph % cg;
    const float vs = bw_value_scale(gmax, false);
    BW_ELEMENTS(j, n, lgD) {
        const int64_t i = ((int64_t)ph * n << lgD) + j;
        const int64_t t = j >> lgD, d = j & (D - 1);
        const int64_t ts = kdk ? n - 1 - t : t;                 // source token
        const int64_t src = (h * n + ts) * D + d;
        if (kdk) {
            if (qo) {
                qo[i] = k[src];
                ko[i] = q[src];
            }
            vo[i] = from_f32<TV>(g[(h * n + ts) * (D + 1) + c] * vs * to_f32(q[src]));
        } else {
            if (qo) {
                qo[i] = q[src];
                ko[i] = k[src];
            }
            const float vc = c < D ? to_f32(v[(h * n + ts) * D + c]) : 1.f;
            vo[i] = from_f32<TV>(vc * to_f32(k[src]));
        }
    }
}

// Contraction over a column group into the fp32 accumulator acc[h][t][d]:
//   dk (kdk = 1): acc[h][j] += s sum_cc [v, 1][j][c] r[h*cg+cc][n-1-j]   (r unscaled here)
//   dq (kdk = 0): acc[h][i] += s sum_cc g[i][c] r[h*cg+cc][i]
template <typename TIn>
__global__ __launch_bounds__(kBwThreads) void bw_contract(const float *__restrict__ r, const TIn *__restrict__ v,
                                                          const float *__restrict__ g, const unsigned *__restrict__ gmax,
                                                          float *__restrict__ acc, int64_t n, int lgD, int c0, int cg,
                                                          int kdk, float s) {
    const int64_t h = blockIdx.y, D = 1 << lgD;                 // grid bw_grid2 over the heads
    if (kdk) s *= bw_value_scale(gmax, true);
    BW_ELEMENTS(j, n, lgD) {
        const int64_t i = (h * n << lgD) + j;
        const int64_t t = j >> lgD, d = j & (D - 1);
        const int64_t tr = kdk ? n - 1 - t : t;                 // row of the pass's output
        float sum = 0.f;
        for (int cc = 0; cc < cg; ++cc) {
            const int c = c0 + cc;
            const float w = kdk ? (c < D ? to_f32(v[(h * n + t) * D + c]) : 1.f) : g[(h * n + t) * (D + 1) + c];
            sum += w * r[((h * cg + cc) * n + tr) * D + d];
        }
        acc[i] += s * sum;
    }
}

// dv[h][j] = r[h][n-1-j] (the dv pass ran on reversed time, on scaled values).
template <typename TOut>
__global__ __launch_bounds__(kBwThreads) void bw_finish_dv(const float *__restrict__ r, const unsigned *__restrict__ gmax,
                                                           TOut *__restrict__ dv, int64_t n, int lgD) {
    const int64_t base = (int64_t)blockIdx.y * n << lgD;        // grid bw_grid2 over the heads
    const float inv = bw_value_scale(gmax, true);
    BW_ELEMENTS(j, n, lgD) {
        const int64_t t = j >> lgD, d = j & ((1 << lgD) - 1);
        dv[base + j] = from_f32<TOut>(r[base + ((n - 1 - t) << lgD) + d] * inv);
    }
}

template <typename TOut>
__global__ __launch_bounds__(kBwThreads) void bw_cast(const float *__restrict__ a, TOut *__restrict__ out, int64_t total) {
    for (int64_t i = (int64_t)blockIdx.x * kBwThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kBwThreads)
        out[i] = from_f32<TOut>(a[i]);
}

// Device buffers of one backward call, taken in order from the index's pool: the calls on an
// index request the same sequence of sizes for the same shapes, so after the first call nothing is
// allocated.  (Allocating and freeing the tens of GB of a call each time slowed later calls down
// to several times the first, and the device's free memory fell, once other indexes had come and
// gone in the process.)  A request larger than its pool entry replaces the entry; when an
// allocation fails, the entries this call has not reached yet are released and it is tried once
// more.  The buffers stay in the pool when the call returns (its stream drained).
struct Arena {
    std::vector<std::pair<void *, size_t>> &pool;
    size_t next = 0;
    hipError_t err = hipSuccess;
    explicit Arena(std::vector<std::pair<void *, size_t>> &p) : pool(p) {}
    template <typename T> T *get(int64_t count) {
        if (err != hipSuccess) return nullptr;
        const size_t bytes = (size_t)std::max<int64_t>(count, 1) * sizeof(T);
        if (next < pool.size() && pool[next].first && pool[next].second >= bytes)
            return static_cast<T *>(pool[next++].first);
        if (next < pool.size() && pool[next].first) {
            (void)hipFree(pool[next].first);
            pool[next] = {nullptr, 0};
        }
        void *p = nullptr;
        err = hipMalloc(&p, bytes);
        if (err != hipSuccess) {
            (void)hipGetLastError();
            for (size_t i = next; i < pool.size(); ++i)
                if (pool[i].first) {
                    (void)hipFree(pool[i].first);
                    pool[i] = {nullptr, 0};
                }
            err = hipMalloc(&p, bytes);
            if (err != hipSuccess) return nullptr;
        }
        if (next < pool.size()) pool[next] = {p, bytes};
        else pool.push_back({p, bytes});
        ++next;
        return static_cast<T *>(p);
    }
};

}  // namespace

void free_backward_pool(const sata_index *idx) {
    for (auto &b : idx->bw_pool)
        if (b.first) (void)hipFree(b.first);
    idx->bw_pool.clear();
}

namespace {

// A temporary state (and workspace) for up to `heads` heads of idx, reused by
// every pass of one backward call and cleared before each.
struct TempState {
    sata_state st;
    int64_t max_heads = 0;
    hipError_t make(Arena &ar, const sata_index *idx, int64_t heads, int64_t n, int chunk, sata_dtype in_dt,
                    uint32_t *err) {
        const PrefillPlan plan = plan_prefill(idx, heads, n, chunk, in_dt, kWorkCap, scan16_covers(idx, in_dt));
        if (!plan.ok) return hipErrorInvalidValue;
        st.d_err = err;
        st.idx = idx;
        st.batch = 1;
        st.device = idx->device;
        st.dtype = SATA_F32;
        max_heads = heads;
        st.d_state = ar.get<float>(heads * (idx->dv + 1) * idx->m_pad);
        st.d_work = ar.get<char>(plan.work_bytes);
        st.work_bytes = plan.work_bytes;
        return ar.err;
    }
};

// One unnormalised (raw) or normalised prefill of `heads` heads from a zero state; heads read
// q and k of head h / qk_div (the fp16-operand scan only).
hipError_t run_pass(TempState &ts, int64_t heads, const void *q, const void *k, const void *v, float *out, float *den,
                    int64_t n, int chunk, sata_dtype in_dt, bool raw, hipStream_t s, int qk_div = 1,
                    bool v_f16 = false) {
    const sata_index *idx = ts.st.idx;
    // bf16 inputs run on the fp16-operand scan where it covers the index (the gradient-weighted
    // values arrive scaled into fp16's normal range), like the forward prefill
    const bool s16 = scan16_covers(idx, in_dt);
    PrefillPlan plan = plan_prefill(idx, heads, n, chunk, in_dt, kWorkCap, s16);
    // fewer heads than the state was made for can fit more chunks under the default cap than
    // its workspace holds: plan again under the workspace it has (shorter segments)
    if (plan.ok && plan.work_bytes > ts.st.work_bytes)
        plan = plan_prefill(idx, heads, n, chunk, in_dt, ts.st.work_bytes, s16);
    if (!plan.ok || heads > ts.max_heads || plan.work_bytes > ts.st.work_bytes) return hipErrorInvalidValue;
    if ((qk_div != 1 || v_f16) && !plan.s16) return hipErrorInvalidValue;
    plan.raw = raw;
    plan.den_out = den;
    plan.qk_div = qk_div;
    plan.v_f16 = v_f16;
    ts.st.heads = (int)heads;
    ts.st.state_bytes = heads * (idx->dv + 1) * idx->m_pad * (int64_t)sizeof(float);
    hipError_t e = launch_zero(static_cast<float *>(ts.st.d_state), ts.st.state_bytes / 4, s);
    if (e != hipSuccess) return e;
    return launch_prefill(idx, &ts.st, plan, q, k, v, out, n, in_dt, SATA_F32, s);
}

// The step of the running backward call (per host thread), for the error message of a failure.
thread_local const char *t_bw_step = "";

template <typename TIn, typename TOut>
hipError_t backward_t(const sata_index *idx, const sata_index *lower, int64_t bh, const void *qv, const void *kv,
                      const void *vv, const void *doutv, void *dqv, void *dkv, void *dvv, int64_t n, int chunk,
                      sata_dtype in_dt, int64_t mem_budget, hipStream_t s) {
    const int D = idx->dk;
    const int lgD = __builtin_ctz((unsigned)D);   // head sizes are powers of two
    const TIn *q = static_cast<const TIn *>(qv), *k = static_cast<const TIn *>(kv), *v = static_cast<const TIn *>(vv);
    const int64_t elems = bh * n * D;
    t_bw_step = "temporaries";
    Arena ar(idx->bw_pool);
    float *o = ar.get<float>(elems), *z = ar.get<float>(bh * n), *g = ar.get<float>(bh * n * (D + 1));
    float *r = ar.get<float>(elems);
    TIn *rq = ar.get<TIn>(elems), *rk = ar.get<TIn>(elems), *rg = ar.get<TIn>(elems);
    if (ar.err != hipSuccess) return ar.err;
    // error word of every pass's scan (a timed-out wait for a predecessor item), read back at the
    // end, and the largest |g| (bits of a float)
    uint32_t *err = ar.get<uint32_t>(2);
    if (ar.err != hipSuccess) return ar.err;
    uint32_t *gmax = err + 1;
    hipError_t e = launch_zero(reinterpret_cast<float *>(err), 2, s);
    if (e != hipSuccess) return e;
    TempState top;
    t_bw_step = "state of the P-order passes";
    if ((e = top.make(ar, idx, bh, n, chunk, in_dt, err)) != hipSuccess) return e;
    // 1. forward: o and z
    t_bw_step = "forward pass";
    if ((e = run_pass(top, bh, q, k, v, o, z, n, chunk, in_dt, false, s)) != hipSuccess) return e;
    t_bw_step = "inputs of the dv pass";
    hipLaunchKernelGGL(bw_prep_g<TIn>, dim3(bw_grid(bh * n)), dim3(kBwThreads), 0, s,
                       static_cast<const TIn *>(doutv), o, z, g, bh * n, D);
    hipLaunchKernelGGL(bw_absmax, dim3(std::min<unsigned>(bw_grid(bh * n * (D + 1)), 4096)), dim3(kBwThreads), 0, s, g,
                       bh * n * (D + 1), gmax);
    // 2. dv: reversed time, queries k, keys q, values g[:d_V], P orders
    hipLaunchKernelGGL(bw_reverse<TIn>, bw_grid2(n, D, bh), dim3(kBwThreads), 0, s, k, rq, n, lgD);
    hipLaunchKernelGGL(bw_reverse<TIn>, bw_grid2(n, D, bh), dim3(kBwThreads), 0, s, q, rk, n, lgD);
    // on the fp16-operand scan the gradient-weighted values go in as binary16 (rg has the width)
    const bool top16 = scan16_covers(idx, in_dt);
    if (top16)
        hipLaunchKernelGGL(bw_rev_g<f16_t>, bw_grid2(n, D, bh), dim3(kBwThreads), 0, s, g, gmax,
                           reinterpret_cast<f16_t *>(rg), n, lgD);
    else
        hipLaunchKernelGGL(bw_rev_g<TIn>, bw_grid2(n, D, bh), dim3(kBwThreads), 0, s, g, gmax, rg, n, lgD);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    t_bw_step = "dv pass";
    if ((e = run_pass(top, bh, rq, rk, rg, r, nullptr, n, chunk, in_dt, true, s, 1, top16)) != hipSuccess) return e;
    t_bw_step = "dk and dq accumulators";
    hipLaunchKernelGGL(bw_finish_dv<TOut>, bw_grid2(n, D, bh), dim3(kBwThreads), 0, s, r, gmax,
                       static_cast<TOut *>(dvv), n, lgD);
    // 3. dk and dq: P - 1 orders, one pseudo-head per column c in groups of cg
    float *acc_k = ar.get<float>(elems), *acc_q = ar.get<float>(elems);
    if (ar.err != hipSuccess) return ar.err;
    if ((e = launch_zero(acc_k, elems, s)) != hipSuccess) return e;
    if ((e = launch_zero(acc_q, elems, s)) != hipSuccess) return e;
    if (lower) {
        // on the fp16-operand scan the pseudo-heads of a head read its q' and k' in place (q and k
        // for dq, the reversed copies of the dv pass for dk): only v' is written per column
        const bool shared = scan16_covers(lower, in_dt);
        const int64_t per_col = elems * ((shared ? 1 : 3) * (int64_t)sizeof(TIn) + (int64_t)sizeof(float));
        // columns per pass: within the memory budget, and bh * cg pseudo-heads within the grid's y limit
        const int cg = (int)std::max<int64_t>(1, std::min<int64_t>({(int64_t)D + 1, mem_budget / std::max<int64_t>(per_col, 1),
                                                                   65535 / bh}));
        TIn *gq = shared ? nullptr : ar.get<TIn>(elems * cg), *gk = shared ? nullptr : ar.get<TIn>(elems * cg);
        TIn *gv = ar.get<TIn>(elems * cg);
        float *gr = ar.get<float>(elems * cg);
        if (ar.err != hipSuccess) return ar.err;
        TempState low;
        t_bw_step = "state of the (P-1)-order passes";
        if ((e = low.make(ar, lower, bh * cg, n, chunk, in_dt, err)) != hipSuccess) return e;
        const float sc = 1.0f / sqrtf((float)D);
        for (int pass = 0; pass < 2; ++pass) {
            const int kdk = pass == 0 ? 1 : 0;
            for (int c0 = 0; c0 <= D; c0 += cg) {
                const int n_c = std::min(cg, D + 1 - c0);
                t_bw_step = kdk ? "inputs of a dk pass" : "inputs of a dq pass";
                if (shared)
                    hipLaunchKernelGGL((bw_group_inputs<TIn, f16_t>), bw_grid2(n, D, bh * n_c), dim3(kBwThreads), 0,
                                       s, q, k, v, g, gmax, gq, gk, reinterpret_cast<f16_t *>(gv), n, lgD, c0, n_c,
                                       kdk);
                else
                    hipLaunchKernelGGL((bw_group_inputs<TIn, TIn>), bw_grid2(n, D, bh * n_c), dim3(kBwThreads), 0, s,
                                       q, k, v, g, gmax, gq, gk, gv, n, lgD, c0, n_c, kdk);
                if ((e = hipGetLastError()) != hipSuccess) return e;
                t_bw_step = kdk ? "dk pass" : "dq pass";
                const void *pq = shared ? (kdk ? (const void *)rq : (const void *)q) : (const void *)gq;
                const void *pk = shared ? (kdk ? (const void *)rk : (const void *)k) : (const void *)gk;
                if ((e = run_pass(low, bh * n_c, pq, pk, gv, gr, nullptr, n, chunk, in_dt, true, s,
                                  shared ? n_c : 1, shared)) != hipSuccess)
                    return e;
                t_bw_step = "contraction";
                hipLaunchKernelGGL(bw_contract<TIn>, bw_grid2(n, D, bh), dim3(kBwThreads), 0, s, gr, v, g, gmax,
                                   kdk ? acc_k : acc_q, n, lgD, c0, n_c, kdk, sc);
                if ((e = hipGetLastError()) != hipSuccess) return e;
            }
        }
    }
    t_bw_step = "gradient output";
    hipLaunchKernelGGL(bw_cast<TOut>, dim3(bw_grid(elems)), dim3(kBwThreads), 0, s, acc_k, static_cast<TOut *>(dkv), elems);
    hipLaunchKernelGGL(bw_cast<TOut>, dim3(bw_grid(elems)), dim3(kBwThreads), 0, s, acc_q, static_cast<TOut *>(dqv), elems);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // the temporaries go back to the pool on return, for a later call on any stream: let this
    // stream drain first
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
    uint32_t bits = 0;
    if ((e = hipMemcpy(&bits, err, sizeof(bits), hipMemcpyDeviceToHost)) != hipSuccess) return e;
    return bits ? hipErrorLaunchTimeOut : hipSuccess;   // a scan's wait ran out: the gradients are invalid
}

}  // namespace

const char *backward_last_step() { return t_bw_step; }

hipError_t launch_backward(const sata_index *idx, const sata_index *lower, int64_t bh, const void *q, const void *k,
                           const void *v, const void *dout, void *dq, void *dk, void *dv, int64_t n, int chunk,
                           sata_dtype in_dt, sata_dtype out_dt, int64_t mem_budget, hipStream_t s) {
    if (in_dt == SATA_F32 && out_dt == SATA_F32)
        return backward_t<float, float>(idx, lower, bh, q, k, v, dout, dq, dk, dv, n, chunk, in_dt, mem_budget, s);
    if (in_dt == SATA_F32 && out_dt == SATA_BF16)
        return backward_t<float, bf16_t>(idx, lower, bh, q, k, v, dout, dq, dk, dv, n, chunk, in_dt, mem_budget, s);
    if (in_dt == SATA_BF16 && out_dt == SATA_F32)
        return backward_t<bf16_t, float>(idx, lower, bh, q, k, v, dout, dq, dk, dv, n, chunk, in_dt, mem_budget, s);
    return backward_t<bf16_t, bf16_t>(idx, lower, bh, q, k, v, dout, dq, dk, dv, n, chunk, in_dt, mem_budget, s);
}

}  // namespace sata
