// Wavefront-per-row band attention: the fp32 path (any 1 <= D <= 256), the
// chunk continuation of a ring, and the fallback for shapes the bf16 fast
// kernels do not cover.
//
// One 64-lane wavefront owns one output row and walks only that row's
// visible keys, 64 at a time: lane j scores key c0 + j, the chunk max and
// sum are wave reductions, and the running max / sum of an online softmax
// rescale the output accumulator between chunks (lanes own output columns
// d = lane + 64 r).  For prefill the visible keys of query i are
// [max(0, i - W + 1), i] ("27. Sliding-Window Attention", step 2); for decode
// they are the occupied ring slots [0, min(pos + 1, W)).  Scores are the
// fp32 dot product times 1/sqrt(D); the exponent argument is s - m with both
// terms in the same (unscaled) units, so W = 1 yields exactly v.

#include "swa_internal.h"

namespace swa {
namespace {

constexpr int kRowMaxD = 256;
constexpr int kRowDPL = kRowMaxD / 64;

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ inline T from_f32(float x);
template <> __device__ inline float from_f32<float>(float x) { return x; }
template <> __device__ inline bf16 from_f32<bf16>(float x) { return (bf16)x; }

__device__ inline float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// Online-softmax state of one wavefront's output row.  A row's visible keys
// may come in several contiguous segments (ring slots that wrap, then the
// rows of a new chunk); segments are folded in one after another.
template <typename T>
struct RowAttn {
    float m = -__builtin_inff();
    float l = 0.f;
    float o[kRowDPL];
    float* qs;
    float* ps;
    int D;
    float scale;

    __device__ void init(const T* __restrict__ qrow, float* qs_, float* ps_, int D_, float scale_) {
        qs = qs_;
        ps = ps_;
        D = D_;
        scale = scale_;
        for (int d = threadIdx.x; d < D; d += 64) qs[d] = to_f32(qrow[d]);
#pragma unroll
        for (int r = 0; r < kRowDPL; ++r) o[r] = 0.f;
        __syncthreads();
    }

    // Fold in keys [kbeg, kend) of the matrices K, V (row strides ks, vs).
    __device__ void segment(const T* __restrict__ K, int64_t ks, const T* __restrict__ V,
                            int64_t vs, int64_t kbeg, int64_t kend) {
        const int lane = threadIdx.x;
        for (int64_t c0 = kbeg; c0 < kend; c0 += 64) {
            const int64_t j = c0 + lane;
            const bool valid = j < kend;
            float s = -__builtin_inff();
            if (valid) {
                const T* kr = K + j * ks;
                float acc = 0.f;
                for (int d = 0; d < D; ++d) acc = fmaf(qs[d], to_f32(kr[d]), acc);
                s = acc * scale;
            }
            const float m_new = fmaxf(m, wave_max(s));   // finite: key c0 is valid
            const float alpha = expf(m - m_new);          // 0 while nothing was seen
            const float p = valid ? expf(s - m_new) : 0.f;
            l = l * alpha + wave_sum(p);
            ps[lane] = p;
            __syncthreads();
            const int nk = (int)((kend - c0) < 64 ? (kend - c0) : 64);
#pragma unroll
            for (int r = 0; r < kRowDPL; ++r) {
                const int d = lane + 64 * r;
                if (d < D) {
                    float acc = o[r] * alpha;
                    const T* vc = V + c0 * vs + d;
                    for (int jj = 0; jj < nk; ++jj) acc = fmaf(ps[jj], to_f32(vc[(int64_t)jj * vs]), acc);
                    o[r] = acc;
                }
            }
            m = m_new;
            __syncthreads();
        }
    }

    // ln(sum_j exp(s_j)) of the scaled scores seen (-inf if none)
    __device__ float lse() const { return m + logf(l); }

    __device__ void finish(T* __restrict__ orow) const {
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int r = 0; r < kRowDPL; ++r) {
            const int d = threadIdx.x + 64 * r;
            if (d < D) orow[d] = from_f32<T>(o[r] * inv);
        }
    }
};

// Attend query row `qrow` to keys [kbeg, kend) of the matrices K, V (row
// strides ks, vs).
template <typename T>
__device__ void attend_row(const T* __restrict__ qrow, const T* __restrict__ K, int64_t ks,
                           const T* __restrict__ V, int64_t vs, int64_t kbeg, int64_t kend,
                           int D, float scale, T* __restrict__ orow) {
    __shared__ float qs[kRowMaxD];
    __shared__ float ps[64];
    RowAttn<T> st;
    st.init(qrow, qs, ps, D, scale);
    st.segment(K, ks, V, vs, kbeg, kend);
    st.finish(orow);
}

template <typename T>
__global__ __launch_bounds__(64) void rowwise_prefill_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    T* __restrict__ out, int64_t H, int64_t Tn, int D, int64_t W, Layout L, float scale,
    float* __restrict__ lse) {
    const int64_t row = blockIdx.x;            // (b*H + h)*T + i
    const int64_t bh = row / Tn;
    const int64_t i = row - bh * Tn;
    const int64_t b = bh / H, h = bh - b * H;
    const int64_t kbeg = i - W + 1 > 0 ? i - W + 1 : 0;
    __shared__ float qs[kRowMaxD];
    __shared__ float ps[64];
    RowAttn<T> st;
    st.init(q + b * L.q.b + h * L.q.h + i * L.q.t, qs, ps, D, scale);
    st.segment(k + b * L.k.b + h * L.k.h, L.k.t, v + b * L.v.b + h * L.v.h, L.v.t, kbeg, i + 1);
    st.finish(out + b * L.o.b + h * L.o.h + i * L.o.t);
    if (lse != nullptr && threadIdx.x == 0) lse[row] = st.lse();
}

template <typename T>
__global__ __launch_bounds__(64) void rowwise_decode_kernel(
    const T* __restrict__ q, const T* __restrict__ kring, const T* __restrict__ vring,
    const int64_t* __restrict__ pos, T* __restrict__ out, int64_t H, int D, int64_t W,
    float scale) {
    const int64_t sh = blockIdx.x;             // s*H + h
    const int64_t s = sh / H;
    const int64_t p = pos[s];
    int64_t n = p + 1;
    n = n < 0 ? 0 : (n > W ? W : n);
    const int64_t rbase = sh * W * D;
    attend_row<T>(q + sh * D, kring + rbase, D, vring + rbase, D, 0, n, D, scale, out + sh * D);
}

// Chunk continuation: query c of the chunk sits at absolute position
// p = pos0 + c and sees tokens (p - W, p]: those before pos0 live in the
// ring at slot t mod W (a slot range that may wrap), the rest are chunk rows.
template <typename T>
__global__ __launch_bounds__(64) void rowwise_chunk_kernel(
    const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
    const T* __restrict__ kring, const T* __restrict__ vring, const int64_t* __restrict__ pos0,
    T* __restrict__ out, int64_t H, int64_t C, int D, int64_t W, float scale) {
    const int64_t row = blockIdx.x;            // (s*H + h)*C + c
    const int64_t sh = row / C;
    const int64_t c = row - sh * C;
    const int64_t s = sh / H;
    int64_t p0 = pos0[s];
    p0 = p0 < 0 ? 0 : p0;                      // outside the contract; stay in bounds
    const int64_t p = p0 + c;
    const int64_t lo = p - W + 1 > 0 ? p - W + 1 : 0;
    const int64_t cbase = sh * C * D;
    const int64_t rbase = sh * W * D;
    __shared__ float qs[kRowMaxD];
    __shared__ float ps[64];
    RowAttn<T> st;
    st.init(q + cbase + c * D, qs, ps, D, scale);
    if (lo < p0) {                             // ring tokens [lo, p0): slots from lo mod W
        const int64_t n = p0 - lo;             // < W
        const int64_t a = lo % W;
        const int64_t first = a + n <= W ? n : W - a;
        st.segment(kring + rbase, D, vring + rbase, D, a, a + first);
        if (first < n) st.segment(kring + rbase, D, vring + rbase, D, 0, n - first);
    }
    const int64_t cb = lo > p0 ? lo - p0 : 0;  // chunk rows [cb, c]
    st.segment(kc + cbase, D, vc + cbase, D, cb, c + 1);
    st.finish(out + cbase + c * D);
}

// ---- backward ---------------------------------------------------------------
//
// Gradients of out = P v with P = softmax over the band of S = q k^T * scale:
//   dV = P^T dout, dP = dout v^T, dS = P (dP - delta), delta_i = dout_i . out_i
//   (= sum_j P_ij dP_ij), dQ = dS k * scale, dK = dS^T q * scale.
// bwd_query_kernel: one wavefront per query row i: the row's log-sum-exp of
// the scores and delta_i = sum_j P_ij dP_ij (one online pass over its band,
// in fp32: taken from a bf16 output, delta would carry that rounding into
// dS = P (dP - delta) where dP of a dominant key cancels it), then a second
// pass accumulating dQ_i.  bwd_key_kernel: one wavefront per key row j, over the
// queries i in [j, j + W - 1] that see it, accumulating dK_j and dV_j from
// the per-row log-sum-exp and delta the first kernel left in the workspace.

template <typename T>
__global__ __launch_bounds__(64) void bwd_query_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ o, const T* __restrict__ dout, T* __restrict__ dq,
    float* __restrict__ lse, float* __restrict__ delta, int64_t Tn, int D, int64_t W,
    float scale) {
    __shared__ float qs[kRowMaxD];
    __shared__ float ds_[kRowMaxD];
    __shared__ float ps[64];
    const int lane = threadIdx.x;
    const int64_t row = blockIdx.x;            // (b*H + h)*T + i
    const int64_t bh = row / Tn;
    const int64_t i = row - bh * Tn;
    const int64_t base = bh * Tn * D;
    const T* K = k + base;
    const T* V = v + base;
    (void)o;
    for (int d = lane; d < D; d += 64) {
        qs[d] = to_f32(q[base + i * D + d]);
        ds_[d] = to_f32(dout[base + i * D + d]);
    }
    __syncthreads();
    const int64_t kbeg = i - W + 1 > 0 ? i - W + 1 : 0, kend = i + 1;
    auto score = [&](int64_t j) {
        const T* kr = K + j * D;
        float acc = 0.f;
        for (int d = 0; d < D; ++d) acc = fmaf(qs[d], to_f32(kr[d]), acc);
        return acc * scale;
    };
    auto dprod = [&](int64_t j) {                // dP_ij = dout_i . v_j
        const T* vr = V + j * D;
        float dp = 0.f;
        for (int d = 0; d < D; ++d) dp = fmaf(ds_[d], to_f32(vr[d]), dp);
        return dp;
    };
    // pass 1: log-sum-exp of the row's scores and sum_j e_j dP_ij, both
    // against the running max
    float m = -__builtin_inff(), l = 0.f, y = 0.f;
    for (int64_t c0 = kbeg; c0 < kend; c0 += 64) {
        const int64_t j = c0 + lane;
        const float s = j < kend ? score(j) : -__builtin_inff();
        const float mn = fmaxf(m, wave_max(s));      // finite: key c0 is valid
        const float e = j < kend ? expf(s - mn) : 0.f;
        const float r = expf(m - mn);
        l = l * r + wave_sum(e);
        y = y * r + wave_sum(j < kend ? e * dprod(j) : 0.f);
        m = mn;
    }
    const float L = m + logf(l);
    const float dl = y / l;
    // pass 2: dQ_i = scale * sum_j dS_ij k_j (lanes own columns d = lane + 64 r)
    float acc[kRowDPL];
#pragma unroll
    for (int r = 0; r < kRowDPL; ++r) acc[r] = 0.f;
    for (int64_t c0 = kbeg; c0 < kend; c0 += 64) {
        const int64_t j = c0 + lane;
        float dsv = 0.f;
        if (j < kend) {
            const float p = expf(score(j) - L);
            dsv = p * (dprod(j) - dl);
        }
        ps[lane] = dsv;
        __syncthreads();
        const int nk = (int)((kend - c0) < 64 ? (kend - c0) : 64);
#pragma unroll
        for (int r = 0; r < kRowDPL; ++r) {
            const int d = lane + 64 * r;
            if (d < D)
                for (int jj = 0; jj < nk; ++jj)
                    acc[r] = fmaf(ps[jj], to_f32(K[(c0 + jj) * D + d]), acc[r]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < kRowDPL; ++r) {
        const int d = lane + 64 * r;
        if (d < D) dq[base + i * D + d] = from_f32<T>(acc[r] * scale);
    }
    if (lane == 0) {
        lse[row] = L;
        delta[row] = dl;
    }
}

template <typename T>
__global__ __launch_bounds__(64) void bwd_key_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, T* __restrict__ dk, T* __restrict__ dv,
    const float* __restrict__ lse, const float* __restrict__ delta, int64_t Tn, int D, int64_t W,
    float scale) {
    __shared__ float ks[kRowMaxD];
    __shared__ float vs[kRowMaxD];
    __shared__ float pp[64];
    __shared__ float dd[64];
    const int lane = threadIdx.x;
    const int64_t row = blockIdx.x;            // (b*H + h)*T + j
    const int64_t bh = row / Tn;
    const int64_t j = row - bh * Tn;
    const int64_t base = bh * Tn * D;
    const T* Q = q + base;
    const T* DO = dout + base;
    for (int d = lane; d < D; d += 64) {
        ks[d] = to_f32(k[base + j * D + d]);
        vs[d] = to_f32(v[base + j * D + d]);
    }
    __syncthreads();
    const int64_t qbeg = j, qend = j + W < Tn ? j + W : Tn;
    float ak[kRowDPL], av[kRowDPL];
#pragma unroll
    for (int r = 0; r < kRowDPL; ++r) ak[r] = av[r] = 0.f;
    for (int64_t c0 = qbeg; c0 < qend; c0 += 64) {
        const int64_t i = c0 + lane;
        float p = 0.f, dsv = 0.f;
        if (i < qend) {
            const T* qr = Q + i * D;
            const T* dr = DO + i * D;
            float s = 0.f, dp = 0.f;
            for (int d = 0; d < D; ++d) {
                s = fmaf(ks[d], to_f32(qr[d]), s);
                dp = fmaf(vs[d], to_f32(dr[d]), dp);
            }
            p = expf(s * scale - lse[bh * Tn + i]);
            dsv = p * (dp - delta[bh * Tn + i]);
        }
        pp[lane] = p;
        dd[lane] = dsv;
        __syncthreads();
        const int nq = (int)((qend - c0) < 64 ? (qend - c0) : 64);
#pragma unroll
        for (int r = 0; r < kRowDPL; ++r) {
            const int d = lane + 64 * r;
            if (d < D)
                for (int ii = 0; ii < nq; ++ii) {
                    av[r] = fmaf(pp[ii], to_f32(DO[(c0 + ii) * D + d]), av[r]);
                    ak[r] = fmaf(dd[ii], to_f32(Q[(c0 + ii) * D + d]), ak[r]);
                }
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < kRowDPL; ++r) {
        const int d = lane + 64 * r;
        if (d < D) {
            dk[base + j * D + d] = from_f32<T>(ak[r] * scale);
            dv[base + j * D + d] = from_f32<T>(av[r]);
        }
    }
}

}  // namespace

template <typename T>
hipError_t launch_rowwise_backward(const T* q, const T* k, const T* v, const T* o, const T* dout,
                                   T* dq, T* dk, T* dv, float* lse, float* delta, int64_t B,
                                   int64_t H, int64_t Tn, int D, int64_t W, float scale,
                                   hipStream_t stream) {
    const int64_t rows = B * H * Tn;
    void* a1[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&o, (void*)&dout, (void*)&dq,
                  (void*)&lse, (void*)&delta, (void*)&Tn, (void*)&D, (void*)&W, (void*)&scale};
    hipError_t e = hipLaunchKernel((const void*)bwd_query_kernel<T>, dim3((unsigned)rows),
                                   dim3(64), a1, 0, stream);
    if (e != hipSuccess) return e;
    const float* lc = lse;
    const float* dc = delta;
    void* a2[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&dout, (void*)&dk, (void*)&dv,
                  (void*)&lc, (void*)&dc, (void*)&Tn, (void*)&D, (void*)&W, (void*)&scale};
    return hipLaunchKernel((const void*)bwd_key_kernel<T>, dim3((unsigned)rows), dim3(64), a2, 0,
                           stream);
}

template <typename T>
hipError_t launch_rowwise_chunk(const T* q, const T* kc, const T* vc, const T* kring,
                                const T* vring, const int64_t* pos0, T* out, int64_t S, int64_t H,
                                int64_t C, int D, int64_t W, hipStream_t stream) {
    const int64_t rows = S * H * C;
    float scale = 1.0f / sqrtf((float)D);
    void* args[] = {(void*)&q, (void*)&kc, (void*)&vc, (void*)&kring, (void*)&vring,
                    (void*)&pos0, (void*)&out, (void*)&H, (void*)&C, (void*)&D, (void*)&W,
                    (void*)&scale};
    return hipLaunchKernel((const void*)rowwise_chunk_kernel<T>, dim3((unsigned)rows), dim3(64),
                           args, 0, stream);
}

template <typename T>
hipError_t launch_rowwise_prefill(const T* q, const T* k, const T* v, T* out, int64_t B,
                                  int64_t H, int64_t Tn, int D, int64_t W, const Layout& L,
                                  float scale, hipStream_t stream, float* lse) {
    const int64_t rows = B * H * Tn;
    Layout lay = L;
    void* args[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&out, (void*)&H, (void*)&Tn,
                    (void*)&D, (void*)&W, (void*)&lay, (void*)&scale, (void*)&lse};
    return hipLaunchKernel((const void*)rowwise_prefill_kernel<T>, dim3((unsigned)rows),
                           dim3(64), args, 0, stream);
}

template <typename T>
hipError_t launch_rowwise_decode(const T* q, const T* kring, const T* vring,
                                 const int64_t* pos, T* out, int64_t S, int64_t H, int D,
                                 int64_t W, hipStream_t stream) {
    const int64_t rows = S * H;
    float scale = 1.0f / sqrtf((float)D);
    void* args[] = {(void*)&q, (void*)&kring, (void*)&vring, (void*)&pos, (void*)&out,
                    (void*)&H, (void*)&D, (void*)&W, (void*)&scale};
    return hipLaunchKernel((const void*)rowwise_decode_kernel<T>, dim3((unsigned)rows),
                           dim3(64), args, 0, stream);
}

template hipError_t launch_rowwise_prefill<float>(const float*, const float*, const float*,
                                                  float*, int64_t, int64_t, int64_t, int,
                                                  int64_t, const Layout&, float, hipStream_t,
                                                  float*);
template hipError_t launch_rowwise_prefill<bf16>(const bf16*, const bf16*, const bf16*, bf16*,
                                                 int64_t, int64_t, int64_t, int, int64_t,
                                                 const Layout&, float, hipStream_t, float*);
template hipError_t launch_rowwise_chunk<float>(const float*, const float*, const float*,
                                                const float*, const float*, const int64_t*, float*,
                                                int64_t, int64_t, int64_t, int, int64_t, hipStream_t);
template hipError_t launch_rowwise_chunk<bf16>(const bf16*, const bf16*, const bf16*, const bf16*,
                                               const bf16*, const int64_t*, bf16*, int64_t, int64_t,
                                               int64_t, int, int64_t, hipStream_t);
template hipError_t launch_rowwise_backward<float>(const float*, const float*, const float*,
                                                   const float*, const float*, float*, float*,
                                                   float*, float*, float*, int64_t, int64_t,
                                                   int64_t, int, int64_t, float, hipStream_t);
template hipError_t launch_rowwise_backward<bf16>(const bf16*, const bf16*, const bf16*,
                                                  const bf16*, const bf16*, bf16*, bf16*, bf16*,
                                                  float*, float*, int64_t, int64_t, int64_t, int,
                                                  int64_t, float, hipStream_t);
template hipError_t launch_rowwise_decode<float>(const float*, const float*, const float*,
                                                 const int64_t*, float*, int64_t, int64_t,
                                                 int, int64_t, hipStream_t);
template hipError_t launch_rowwise_decode<bf16>(const bf16*, const bf16*, const bf16*,
                                                const int64_t*, bf16*, int64_t, int64_t, int,
                                                int64_t, hipStream_t);

}  // namespace swa
