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

// out[h][t][:] = in[h][n-1-t][:] (the time-reversed sequence of every head).
template <typename T>
__global__ __launch_bounds__(kBwThreads) void bw_reverse(const T *__restrict__ in, T *__restrict__ out, int64_t heads,
                                                         int64_t n, int D) {
    const int64_t total = heads * n * D;
    for (int64_t i = (int64_t)blockIdx.x * kBwThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kBwThreads) {
        const int64_t d = i % D, t = (i / D) % n, h = i / (D * n);
        out[i] = in[(h * n + (n - 1 - t)) * D + d];
    }
}

// values of the dv pass: out[h][t][d] = g[h][n-1-t][d], d < D.
template <typename TIn>
__global__ __launch_bounds__(kBwThreads) void bw_rev_g(const float *__restrict__ g, TIn *__restrict__ out, int64_t heads,
                                                       int64_t n, int D) {
    const int64_t total = heads * n * D;
    for (int64_t i = (int64_t)blockIdx.x * kBwThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kBwThreads) {
        const int64_t d = i % D, t = (i / D) % n, h = i / (D * n);
        out[i] = from_f32<TIn>(g[(h * n + (n - 1 - t)) * (D + 1) + d]);
    }
}

// Inputs of one column group [c0, c0 + cg) of the dk pass (kdk = 1) or the dq
// pass (kdk = 0), pseudo-head ph = h * cg + cc for column c = c0 + cc:
//   dk: q' = rev(k), k' = rev(q), v'[t] = g[n-1-t][c] q[n-1-t]
//   dq: q' = q,      k' = k,      v'[t] = [v, 1][t][c] k[t]
template <typename TIn>
__global__ __launch_bounds__(kBwThreads) void bw_group_inputs(const TIn *__restrict__ q, const TIn *__restrict__ k,
                                                              const TIn *__restrict__ v, const float *__restrict__ g,
                                                              TIn *__restrict__ qo, TIn *__restrict__ ko,
                                                              TIn *__restrict__ vo, int64_t heads, int64_t n, int D,
                                                              int c0, int cg, int kdk) {
    const int64_t total = heads * cg * n * D;
    for (int64_t i = (int64_t)blockIdx.x * kBwThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kBwThreads) {
        const int64_t d = i % D, t = (i / D) % n, ph = i / (D * n);
        const int64_t h = ph / cg;
        const int c = c0 + (int)(ph % cg);
        const int64_t ts = kdk ? n - 1 - t : t;                 // source token
        const int64_t src = (h * n + ts) * D + d;
        if (kdk) {
            qo[i] = k[src];
            ko[i] = q[src];
            vo[i] = from_f32<TIn>(g[(h * n + ts) * (D + 1) + c] * to_f32(q[src]));
        } else {
            qo[i] = q[src];
            ko[i] = k[src];
            const float vc = c < D ? to_f32(v[(h * n + ts) * D + c]) : 1.f;
            vo[i] = from_f32<TIn>(vc * to_f32(k[src]));
        }
    }
}

// Contraction over a column group into the fp32 accumulator acc[h][t][d]:
//   dk (kdk = 1): acc[h][j] += s sum_cc [v, 1][j][c] r[h*cg+cc][n-1-j]
//   dq (kdk = 0): acc[h][i] += s sum_cc g[i][c] r[h*cg+cc][i]
template <typename TIn>
__global__ __launch_bounds__(kBwThreads) void bw_contract(const float *__restrict__ r, const TIn *__restrict__ v,
                                                          const float *__restrict__ g, float *__restrict__ acc,
                                                          int64_t heads, int64_t n, int D, int c0, int cg, int kdk,
                                                          float s) {
    const int64_t total = heads * n * D;
    for (int64_t i = (int64_t)blockIdx.x * kBwThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kBwThreads) {
        const int64_t d = i % D, t = (i / D) % n, h = i / (D * n);
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

// dv[h][j] = r[h][n-1-j] (the dv pass ran on reversed time).
template <typename TOut>
__global__ __launch_bounds__(kBwThreads) void bw_finish_dv(const float *__restrict__ r, TOut *__restrict__ dv,
                                                           int64_t heads, int64_t n, int D) {
    const int64_t total = heads * n * D;
    for (int64_t i = (int64_t)blockIdx.x * kBwThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kBwThreads) {
        const int64_t d = i % D, t = (i / D) % n, h = i / (D * n);
        dv[i] = from_f32<TOut>(r[(h * n + (n - 1 - t)) * D + d]);
    }
}

template <typename TOut>
__global__ __launch_bounds__(kBwThreads) void bw_cast(const float *__restrict__ a, TOut *__restrict__ out, int64_t total) {
    for (int64_t i = (int64_t)blockIdx.x * kBwThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kBwThreads)
        out[i] = from_f32<TOut>(a[i]);
}

// Device buffers of one backward call, freed (after the stream drains) when
// the call returns.
struct Arena {
    std::vector<void *> ptrs;
    hipError_t err = hipSuccess;
    template <typename T> T *get(int64_t count) {
        void *p = nullptr;
        if (err == hipSuccess) err = hipMalloc(&p, (size_t)std::max<int64_t>(count, 1) * sizeof(T));
        if (err != hipSuccess) return nullptr;
        ptrs.push_back(p);
        return static_cast<T *>(p);
    }
    ~Arena() {
        for (void *p : ptrs) (void)hipFree(p);
    }
};

// A temporary state (and workspace) for up to `heads` heads of idx, reused by
// every pass of one backward call and cleared before each.
struct TempState {
    sata_state st;
    int64_t max_heads = 0;
    hipError_t make(Arena &ar, const sata_index *idx, int64_t heads, int64_t n, int chunk, sata_dtype in_dt) {
        const PrefillPlan plan = plan_prefill(idx, heads, n, chunk, in_dt);
        if (!plan.ok) return hipErrorInvalidValue;
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

// One unnormalised (raw) or normalised prefill of `heads` heads from a zero state.
hipError_t run_pass(TempState &ts, int64_t heads, const void *q, const void *k, const void *v, float *out, float *den,
                    int64_t n, int chunk, sata_dtype in_dt, bool raw, hipStream_t s) {
    const sata_index *idx = ts.st.idx;
    PrefillPlan plan = plan_prefill(idx, heads, n, chunk, in_dt);
    if (!plan.ok || heads > ts.max_heads || plan.work_bytes > ts.st.work_bytes) return hipErrorInvalidValue;
    plan.raw = raw;
    plan.den_out = den;
    ts.st.heads = (int)heads;
    ts.st.state_bytes = heads * (idx->dv + 1) * idx->m_pad * (int64_t)sizeof(float);
    hipError_t e = launch_zero(static_cast<float *>(ts.st.d_state), ts.st.state_bytes / 4, s);
    if (e != hipSuccess) return e;
    return launch_prefill(idx, &ts.st, plan, q, k, v, out, n, in_dt, SATA_F32, s);
}

template <typename TIn, typename TOut>
hipError_t backward_t(const sata_index *idx, const sata_index *lower, int64_t bh, const void *qv, const void *kv,
                      const void *vv, const void *doutv, void *dqv, void *dkv, void *dvv, int64_t n, int chunk,
                      sata_dtype in_dt, int64_t mem_budget, hipStream_t s) {
    const int D = idx->dk;
    const TIn *q = static_cast<const TIn *>(qv), *k = static_cast<const TIn *>(kv), *v = static_cast<const TIn *>(vv);
    const int64_t elems = bh * n * D;
    Arena ar;
    float *o = ar.get<float>(elems), *z = ar.get<float>(bh * n), *g = ar.get<float>(bh * n * (D + 1));
    float *r = ar.get<float>(elems);
    TIn *rq = ar.get<TIn>(elems), *rk = ar.get<TIn>(elems), *rg = ar.get<TIn>(elems);
    if (ar.err != hipSuccess) return ar.err;
    TempState top;
    hipError_t e = top.make(ar, idx, bh, n, chunk, in_dt);
    if (e != hipSuccess) return e;
    // 1. forward: o and z
    if ((e = run_pass(top, bh, q, k, v, o, z, n, chunk, in_dt, false, s)) != hipSuccess) return e;
    hipLaunchKernelGGL(bw_prep_g<TIn>, dim3(bw_grid(bh * n)), dim3(kBwThreads), 0, s,
                       static_cast<const TIn *>(doutv), o, z, g, bh * n, D);
    // 2. dv: reversed time, queries k, keys q, values g[:d_V], P orders
    hipLaunchKernelGGL(bw_reverse<TIn>, dim3(bw_grid(elems)), dim3(kBwThreads), 0, s, k, rq, bh, n, D);
    hipLaunchKernelGGL(bw_reverse<TIn>, dim3(bw_grid(elems)), dim3(kBwThreads), 0, s, q, rk, bh, n, D);
    hipLaunchKernelGGL(bw_rev_g<TIn>, dim3(bw_grid(elems)), dim3(kBwThreads), 0, s, g, rg, bh, n, D);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = run_pass(top, bh, rq, rk, rg, r, nullptr, n, chunk, in_dt, true, s)) != hipSuccess) return e;
    hipLaunchKernelGGL(bw_finish_dv<TOut>, dim3(bw_grid(elems)), dim3(kBwThreads), 0, s, r, static_cast<TOut *>(dvv),
                       bh, n, D);
    // 3. dk and dq: P - 1 orders, one pseudo-head per column c in groups of cg
    float *acc_k = ar.get<float>(elems), *acc_q = ar.get<float>(elems);
    if (ar.err != hipSuccess) return ar.err;
    if ((e = launch_zero(acc_k, elems, s)) != hipSuccess) return e;
    if ((e = launch_zero(acc_q, elems, s)) != hipSuccess) return e;
    if (lower) {
        const int64_t per_col = elems * (3 * (int64_t)sizeof(TIn) + (int64_t)sizeof(float));
        // columns per pass: within the memory budget, and bh * cg pseudo-heads within the grid's y limit
        const int cg = (int)std::max<int64_t>(1, std::min<int64_t>({(int64_t)D + 1, mem_budget / std::max<int64_t>(per_col, 1),
                                                                   65535 / bh}));
        TIn *gq = ar.get<TIn>(elems * cg), *gk = ar.get<TIn>(elems * cg), *gv = ar.get<TIn>(elems * cg);
        float *gr = ar.get<float>(elems * cg);
        if (ar.err != hipSuccess) return ar.err;
        TempState low;
        if ((e = low.make(ar, lower, bh * cg, n, chunk, in_dt)) != hipSuccess) return e;
        const float sc = 1.0f / sqrtf((float)D);
        for (int pass = 0; pass < 2; ++pass) {
            const int kdk = pass == 0 ? 1 : 0;
            for (int c0 = 0; c0 <= D; c0 += cg) {
                const int n_c = std::min(cg, D + 1 - c0);
                hipLaunchKernelGGL(bw_group_inputs<TIn>, dim3(bw_grid(elems * n_c)), dim3(kBwThreads), 0, s, q, k, v,
                                   g, gq, gk, gv, bh, n, D, c0, n_c, kdk);
                if ((e = hipGetLastError()) != hipSuccess) return e;
                if ((e = run_pass(low, bh * n_c, gq, gk, gv, gr, nullptr, n, chunk, in_dt, true, s)) != hipSuccess)
                    return e;
                hipLaunchKernelGGL(bw_contract<TIn>, dim3(bw_grid(elems)), dim3(kBwThreads), 0, s, gr, v, g,
                                   kdk ? acc_k : acc_q, bh, n, D, c0, n_c, kdk, sc);
                if ((e = hipGetLastError()) != hipSuccess) return e;
            }
        }
    }
    hipLaunchKernelGGL(bw_cast<TOut>, dim3(bw_grid(elems)), dim3(kBwThreads), 0, s, acc_k, static_cast<TOut *>(dkv), elems);
    hipLaunchKernelGGL(bw_cast<TOut>, dim3(bw_grid(elems)), dim3(kBwThreads), 0, s, acc_q, static_cast<TOut *>(dqv), elems);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // the temporaries are freed on return: let the stream drain first
    return hipStreamSynchronize(s);
}

}  // namespace

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
