// Backward of the causal sliding-window attention prefill in fp32 on gfx950
// matrix cores (v_mfma_f32_32x32x2_f32).
//
// The gradients are the chain rule through the forward ("NNX Sliding-Window
// Attention", Mask before softmax: masked weights are zero, so no gradient
// reaches a key outside a query's window):
//   P = exp(S - L) over the band (L the row's log-sum-exp), dV = P^T dout,
//   dP = dout v^T, dS = P (dP - delta) with delta_i = dout_i . out_i,
//   dQ = dS k * scale, dK = dS^T q * scale.
// Two kernels, each a wavefront per 32 rows walking the 32-wide tiles of
// their band, with the operand order of the fp32 forward (contraction slot
// l / 32 of lane l; 16-byte loads of whole row slices; the probabilities and
// dS feed the next product from their own accumulator lanes):
//   query rows  S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T
//               (3 D/2 MFMAs per tile); also writes L log2(e) and delta
//   key rows    S = Q K^T, dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS
//               (2 D MFMAs per tile)
// Masked entries get weight 0 by a select after the exponential, so any
// finite scale, negative included, works unchanged.  Consecutive workgroups
// (consecutive 32-row tiles of a head) run on one XCD, sharing its L2.

#include "swa_mfma.h"

namespace swa {
namespace {


struct BF32Args {
    const float* q;
    const float* k;
    const float* v;
    const float* o;
    const float* dout;
    float* dq;
    float* dk;
    float* dv;
    const float* lse;   // [B * H * T] natural-log row normalisers (forward)
    float* l2;          // [B * H * T] the same in log2 units (written by the query kernel)
    float* delta;       // [B * H * T] dout . out (written by the query kernel)
    int T, W;           // W = min(W, T)
    int ntile;          // 32-row tiles per (b, h)
    int nwaves;         // B * H * ntile
    int remap;          // 1: consecutive workgroups on one XCD (xcd_logical_tile)
    float cs;           // log2(e) * scale (signed)
    float scale;
};

__device__ inline f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_f32_query_kernel(BF32Args a) {
    const int lane = threadIdx.x & 63;
    const int lr = lane & 31, hf = lane >> 5;
    const int gw = xcd_logical_tile(blockIdx.x, gridDim.x, a.remap, 1, -1) * 4 + (threadIdx.x >> 6);
    if (gw >= a.nwaves) return;
    const int bh = gw / a.ntile;
    const int q0 = (gw - bh * a.ntile) * 32;
    const int T = a.T, W = a.W;
    const int64_t off = (int64_t)bh * T * D;
    const float* __restrict__ K = a.k + off;
    const float* __restrict__ V = a.v + off;
    const int qi = q0 + lr;
    const int rc = min(qi, T - 1);
    // q and dout rows as B operands (d = 8 g + 4 hf + e); delta = dout . out
    f32x4 qf[D / 8], df[D / 8];
    float dl = 0.f;
#pragma unroll
    for (int g = 0; g < D / 8; ++g) {
        const int64_t e0 = off + (int64_t)rc * D + 8 * g + 4 * hf;
        qf[g] = ld4(a.q + e0);
        df[g] = ld4(a.dout + e0);
        const f32x4 of = ld4(a.o + e0);
        dl = __builtin_fmaf(df[g][0], of[0], dl);
        dl = __builtin_fmaf(df[g][1], of[1], dl);
        dl = __builtin_fmaf(df[g][2], of[2], dl);
        dl = __builtin_fmaf(df[g][3], of[3], dl);
    }
    const float delta = swap_sum(dl);
    const float L2 = a.lse[(int64_t)bh * T + rc] * kLog2e;
    if (hf == 0 && qi < T) {
        a.l2[(int64_t)bh * T + qi] = L2;
        a.delta[(int64_t)bh * T + qi] = delta;
    }
    const float cs = a.cs;
    const int t0 = max(q0 - W + 1, 0) / 32;
    const int t1 = (min(q0 + 32, T) + 31) / 32;
    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

    for (int t = t0; t < t1; ++t) {
        const int k0 = 32 * t;
        f32x16 s = f32x16{}, dp = f32x16{};
        {
            const int64_t r = (int64_t)min(k0 + lr, T - 1) * D + 4 * hf;
#pragma unroll
            for (int g = 0; g < D / 8; ++g) {
                const f32x4 kf = ld4(K + r + 8 * g);
                const f32x4 vf = ld4(V + r + 8 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[e], qf[g][e], s, 0, 0, 0);
                    dp = __builtin_amdgcn_mfma_f32_32x32x2f32(vf[e], df[g][e], dp, 0, 0, 0);
                }
            }
        }
        // lane: query qi, keys k0 + 8 (vv/4) + 4 hf + vv%4
        const bool interior = k0 + 31 <= q0 && q0 + 31 - k0 < W;
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) {
            const int key = k0 + 8 * (vv >> 2) + 4 * hf + (vv & 3);
            const bool ok = interior || (unsigned)(qi - key) < (unsigned)W;
            const float p = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[vv], cs, -L2)) : 0.f;
            s[vv] = p * (dp[vv] - delta);
        }
        // dQ^T += K^T dS^T: slot hf of MFMA (i, e) is key k0 + 8 i + 4 hf + e
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float* kp = K + (int64_t)min(k0 + 8 * i + 4 * hf + e, T - 1) * D + lr;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(kp[32 * db], s[4 * i + e], acc[db],
                                                                   0, 0, 0);
            }
    }
    if (qi >= T) return;
    float* row = a.dq + off + (int64_t)qi * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            *reinterpret_cast<f32x4*>(row + 32 * db + 8 * g + 4 * hf) =
                f32x4{acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]} *
                a.scale;
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_f32_key_kernel(BF32Args a) {
    const int lane = threadIdx.x & 63;
    const int lr = lane & 31, hf = lane >> 5;
    const int gw = xcd_logical_tile(blockIdx.x, gridDim.x, a.remap, 1, -1) * 4 + (threadIdx.x >> 6);
    if (gw >= a.nwaves) return;
    const int bh = gw / a.ntile;
    const int k0 = (gw - bh * a.ntile) * 32;
    const int T = a.T, W = a.W;
    const int64_t off = (int64_t)bh * T * D;
    const float* __restrict__ Q = a.q + off;
    const float* __restrict__ DO = a.dout + off;
    const float* __restrict__ L2 = a.l2 + (int64_t)bh * T;
    const float* __restrict__ DL = a.delta + (int64_t)bh * T;
    const int kr = k0 + lr;                     // this lane's key (accumulator column)
    const int64_t krow = (int64_t)min(kr, T - 1) * D + 4 * hf;
    const float cs = a.cs;
    // queries that see keys [k0, k0 + 32): [k0, k0 + 31 + W - 1]
    const int u0 = k0 / 32;
    const int u1 = (min(k0 + 31 + W, T) + 31) / 32;
    f32x16 adv[D / 32], adk[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        adv[db] = f32x16{};
        adk[db] = f32x16{};
    }

    for (int u = u0; u < u1; ++u) {
        const int q0 = 32 * u;
        // S = Q K^T and dP = dO V^T: rows = queries q0 + lr (A), column = key kr (B)
        f32x16 s = f32x16{}, dp = f32x16{};
        {
            const int64_t r = (int64_t)min(q0 + lr, T - 1) * D + 4 * hf;
#pragma unroll
            for (int g = 0; g < D / 8; ++g) {
                const f32x4 qf = ld4(Q + r + 8 * g);
                const f32x4 of = ld4(DO + r + 8 * g);
                const f32x4 kf = ld4(a.k + off + krow + 8 * g);
                const f32x4 vf = ld4(a.v + off + krow + 8 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    s = __builtin_amdgcn_mfma_f32_32x32x2f32(qf[e], kf[e], s, 0, 0, 0);
                    dp = __builtin_amdgcn_mfma_f32_32x32x2f32(of[e], vf[e], dp, 0, 0, 0);
                }
            }
        }
        // lane: key kr, queries q0 + 8 (vv/4) + 4 hf + vv%4
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) {
            const int qq = q0 + 8 * (vv >> 2) + 4 * hf + (vv & 3);
            const int qc = min(qq, T - 1);
            const bool ok = (unsigned)(qq - kr) < (unsigned)W && qq < T;
            const float p = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[vv], cs, -L2[qc])) : 0.f;
            s[vv] = p;
            dp[vv] = p * (dp[vv] - DL[qc]);
        }
        // dV^T += dO^T P and dK^T += Q^T dS: slot hf of MFMA (i, e) is query
        // q0 + 8 i + 4 hf + e
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t r = (int64_t)min(q0 + 8 * i + 4 * hf + e, T - 1) * D + lr;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    adv[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(DO[r + 32 * db], s[4 * i + e],
                                                                   adv[db], 0, 0, 0);
                    adk[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(Q[r + 32 * db], dp[4 * i + e],
                                                                   adk[db], 0, 0, 0);
                }
                // bound the operand loads in flight (two waves per SIMD)
                if (D == 128 && (e & 1)) __builtin_amdgcn_sched_barrier(0);
            }
    }
    if (kr >= T) return;
    float* rv = a.dv + off + (int64_t)kr * D;
    float* rk = a.dk + off + (int64_t)kr * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = 32 * db + 8 * g + 4 * hf;
            *reinterpret_cast<f32x4*>(rv + d) =
                f32x4{adv[db][4 * g], adv[db][4 * g + 1], adv[db][4 * g + 2], adv[db][4 * g + 3]};
            *reinterpret_cast<f32x4*>(rk + d) =
                f32x4{adk[db][4 * g], adk[db][4 * g + 1], adk[db][4 * g + 2], adk[db][4 * g + 3]} *
                a.scale;
        }
}

template <int D>
hipError_t launch_both(BF32Args a, hipStream_t st) {
    const dim3 grid((unsigned)((a.nwaves + 3) / 4));
    a.remap = grid.x % 8 == 0 ? 1 : 0;
    void* args[] = {(void*)&a};
    hipError_t e = hipLaunchKernel((const void*)bwd_f32_query_kernel<D>, grid, dim3(256), args, 0, st);
    if (e != hipSuccess) return e;
    return hipLaunchKernel((const void*)bwd_f32_key_kernel<D>, grid, dim3(256), args, 0, st);
}

}  // namespace

bool backward_f32_supports(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const void* dq, const void* dk, const void* dv,
                           int64_t T, int64_t D) {
    if (D != 32 && D != 64 && D != 128) return false;
    for (const void* p : {q, k, v, o, dout, dq, dk, dv})
        if (((uintptr_t)p & 15) != 0) return false;
    return T < ((int64_t)1 << 30);
}

hipError_t launch_backward_f32(const float* q, const float* k, const float* v, const float* o,
                               const float* dout, float* dq, float* dk, float* dv,
                               const float* lse_in, float* lse, float* delta, int64_t B,
                               int64_t H, int64_t T, int D, int64_t W, float scale,
                               hipStream_t stream) {
    if (lse_in == nullptr) {
        // the forward again for each row's log-sum-exp (into lse); its
        // output goes to dq, which the query kernel overwrites
        hipError_t e = launch_prefill_f32(q, k, v, dq, B, H, T, D, W, contiguous_layout(H, T, D),
                                          scale, stream, lse);
        if (e != hipSuccess) return e;
        lse_in = lse;
    }
    BF32Args a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dout = dout;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.lse = lse_in;
    // the log2 normalisers go to the lse workspace (the same array as
    // lse_in after a rerun: each row is read and rewritten by the lane that
    // owns it; rows past T, which read row T - 1, are never stored)
    a.l2 = lse;
    a.delta = delta;
    a.T = (int)T;
    a.W = (int)(W < T ? W : T);
    a.ntile = (int)((T + 31) / 32);
    a.nwaves = (int)(B * H * a.ntile);
    a.cs = kLog2e * scale;
    a.scale = scale;
    if (D == 128) return launch_both<128>(a, stream);
    if (D == 64) return launch_both<64>(a, stream);
    return launch_both<32>(a, stream);
}

}  // namespace swa
