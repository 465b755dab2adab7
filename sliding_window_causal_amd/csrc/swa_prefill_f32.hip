// Causal sliding-window attention prefill in fp32 on gfx950 matrix cores
// (v_mfma_f32_32x32x2_f32: fp32 operands, fp32 products and sums).
//
// Band-only iteration as in the bf16 kernel ("NNX Sliding-Window
// Attention", A local mask is not a sparse implementation): a wavefront owns
// 32 consecutive queries of one (batch, head) and walks the 32-key tiles
// that meet their band, keys j with i - W < j <= i ("27. Sliding-Window
// Attention", step 2), masking (a select to -inf) only the tiles that
// straddle an edge of the band.  Per tile:
//   S^T = K Q^T     D/2 MFMAs.  Lane l supplies row l % 32 (key, or for Q^T
//                   the query) and contraction slot l / 32; MFMA (g, e)
//                   pairs head dimension 8 g + e (slot 0) with 8 g + 4 + e
//                   (slot 1), so each lane loads 16 contiguous bytes per four
//                   MFMAs.  The accumulator gives lane l query l % 32 and
//                   keys 8 (v/4) + 4 (l/32) + v%4 (the layout of the bf16
//                   kernel's score tile).
//   softmax         online: row max over the tile (in-lane, then the lane
//                   pair l, l ^ 32), O and the row sum rescaled when the max
//                   grows, p = exp2((s - m) c) with c = log2(e) * scale.
//   O^T += V^T P^T  D/2 MFMAs: MFMA (i, e) takes key 8 i + e in slot 0 and
//                   8 i + 4 + e in slot 1, so the B operand is the lane's own
//                   probability p[4 i + e] (no exchange) and the A operand
//                   one element of a v row (32 lanes read 128 contiguous
//                   bytes).
// The four wavefronts of a workgroup are independent (no LDS, no barrier):
// they take consecutive query tiles of one (batch, head), and consecutive
// workgroups run on one XCD (xcd_logical_tile), so a head's key tiles are
// shared through that XCD's L2 (23% faster than the hardware's round-robin
// over the XCDs at [1, 32, 8192, 128]).
//
// CHUNK: the continuation of a ring ("25. Sliding-Window Causal Attention
// for Streaming Inference", Problem: the bounded cache; "27. Sliding-Window
// Attention", Problem, the rolling buffer).  Stream s's chunk holds
// positions p0 .. p0 + C - 1 (q, k, v, out [S, H, C, D]); keys before p0
// come from ring slot (position mod W).  Each lane addresses its own key
// rows, so a tile may straddle the ring and the chunk.

#include "swa_mfma.h"

namespace swa {
namespace {

struct F32Args {
    const float* q;
    const float* k;
    const float* v;
    float* out;
    float* lse;     // optional: ln(sum_j exp(s_ij * scale)) at lse[bh * T + i]
    Layout L;       // element strides (D axis contiguous)
    int H, T, W;    // rows of q (T, or C for a chunk); W = min(W, T) (a chunk: the ring's W)
    const float* kring;       // chunk continuation: [S, H, W, D] rings
    const float* vring;
    const int64_t* pos0;      // chunk continuation: first position of stream s's chunk
    int nqt;        // 32-query tiles per (b, h)
    int nwaves;     // B * H * nqt
    int remap;      // 1: consecutive workgroups on one XCD (xcd_logical_tile)
    float c;        // log2(e) * |scale|
    int qneg;       // scale < 0: q negated (exact) and |scale| used
};

template <int D, bool CHUNK>
__global__ __launch_bounds__(256) void prefill_f32_kernel(F32Args a) {
    static_assert(D % 32 == 0 && D <= 128, "head size");
    const int lane = threadIdx.x & 63;
    const int lr = lane & 31, hf = lane >> 5;
    const int blk = xcd_logical_tile(blockIdx.x, gridDim.x, a.remap, 1, -1);
    const int gw = blk * 4 + (threadIdx.x >> 6);
    if (gw >= a.nwaves) return;
    const int bh = gw / a.nqt;
    const int qt = gw - bh * a.nqt;
    const int b = bh / a.H, h = bh - b * a.H;
    const int T = a.T, W = a.W;
    const float* __restrict__ Q = a.q + b * a.L.q.b + h * a.L.q.h;
    const float* __restrict__ K = a.k + b * a.L.k.b + h * a.L.k.h;
    const float* __restrict__ V = a.v + b * a.L.v.b + h * a.L.v.h;
    const int64_t qrs = a.L.q.t, krs = a.L.k.t, vrs = a.L.v.t;

    const int q0 = qt * 32;
    const int qi = q0 + lr;                 // this lane's row of q and out
    // positions: row r of the chunk is position p0 + r (p0 = 0 for a prefill)
    // (chunk: relative to an origin at least W + 32 below the chunk, so
    // positions stay in int whatever the stream's length; omod is the
    // origin's ring slot)
    int p0 = 0, omod = 0;
    const float* __restrict__ Kr = nullptr;
    const float* __restrict__ Vr = nullptr;
    if constexpr (CHUNK) {
        int64_t x = a.pos0[b];
        x = x < 0 ? 0 : x;
        const int64_t origin = x >= (int64_t)W + 32 ? x - W - 32 : 0;
        p0 = (int)(x - origin);
        omod = (int)(origin % W);
        Kr = a.kring + (int64_t)bh * W * D;
        Vr = a.vring + (int64_t)bh * W * D;
    }
    const int qpos = p0 + qi;
    // row of key position x: ring slot (x + omod) mod W below p0, else row
    // x - p0 of k / v (past the last row: the last row, above every valid
    // query's diagonal)
    auto key_row = [&](const float* __restrict__ M, const float* __restrict__ R, int64_t rs,
                       int x) -> const float* {
        if constexpr (CHUNK)
            if (x < p0) return R + (int64_t)((x + omod) % W) * D;
        return M + (int64_t)min(x - p0, T - 1) * rs;
    };
    // Q^T operand: q[qi][8 g + 4 hf .. + 3] (rows past T read row T - 1 and
    // are never stored)
    f32x4 qf[D / 8];
    {
        const float* qp = Q + (int64_t)min(qi, T - 1) * qrs + 4 * hf;
#pragma unroll
        for (int g = 0; g < D / 8; ++g) {
            qf[g] = *reinterpret_cast<const f32x4*>(qp + 8 * g);
            if (a.qneg) qf[g] = -qf[g];
        }
    }
    const float c = a.c;
    // key positions [kbeg, kend): the band of the wave's valid rows, in
    // 32-key tiles from kbeg (tile-aligned for a prefill)
    const int kbeg = CHUNK ? max(p0 + q0 - W + 1, 0) : max(q0 - W + 1, 0) / 32 * 32;
    const int kend = p0 + min(q0 + 32, T);

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    float m = -__builtin_inff();     // running row max (raw score units)
    float lsum = 0.f;                // this lane's half of the row sum

    for (int k0 = kbeg; k0 < kend; k0 += 32) {
        // S^T = K Q^T
        f32x16 s = f32x16{};
        {
            const float* kp = key_row(K, Kr, krs, k0 + lr) + 4 * hf;
#pragma unroll
            for (int g = 0; g < D / 8; ++g) {
                const f32x4 kf = *reinterpret_cast<const f32x4*>(kp + 8 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[e], qf[g][e], s, 0, 0, 0);
            }
        }
        // band mask on tiles that straddle an edge (keys past T lie above
        // every valid query's diagonal)
        const bool interior = k0 + 31 <= p0 + q0 && p0 + q0 + 31 - k0 < W;
        if (!interior) {
#pragma unroll
            for (int vv = 0; vv < 16; ++vv) {
                const int key = k0 + 8 * (vv >> 2) + 4 * hf + (vv & 3);
                s[vv] = (unsigned)(qpos - key) < (unsigned)W ? s[vv] : -__builtin_inff();
            }
        }
        float mx = s[0];
#pragma unroll
        for (int vv = 1; vv < 16; ++vv) mx = fmaxf(mx, s[vv]);
        mx = swap_max(mx);
        if (mx > m) {
            // m = -inf before the row's first key: nothing to rescale
            const float alpha = m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f((m - mx) * c);
            m = mx;
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
        }
        // (s - m) c: the row's max key gets exp2(0) = 1 exactly (a fused
        // s c - m c would leave the rounding of m c), so W = 1 returns v
        const float mr = m == -__builtin_inff() ? 0.f : m;
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) {
            s[vv] = __builtin_amdgcn_exp2f((s[vv] - mr) * c);
            lsum += s[vv];
        }
        // O^T += V^T P^T
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float* vp = key_row(V, Vr, vrs, k0 + 8 * i + 4 * hf + e) + lr;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vp[32 * db], s[4 * i + e], o[db], 0,
                                                                 0, 0);
            }
    }

    if (qi >= T) return;
    const float l = swap_sum(lsum);
    const float inv = 1.f / l;
    if (!CHUNK && a.lse != nullptr && hf == 0)
        a.lse[(int64_t)bh * T + qi] = (m * c + __builtin_amdgcn_logf(l)) * kLn2;
    // lane holds d = 32 db + 8 g + 4 hf + 0..3 of query qi
    float* orow = a.out + b * a.L.o.b + h * a.L.o.h + (int64_t)qi * a.L.o.t;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * g + 4 * hf) =
                f32x4{o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                      o[db][4 * g + 3] * inv};
}

bool strides_ok4(const Strides& s) {
    return s.b >= 0 && s.h >= 0 && s.t >= 0 && s.b % 4 == 0 && s.h % 4 == 0 && s.t % 4 == 0;
}

}  // namespace

bool prefill_f32_supports(const void* q, const void* k, const void* v, const void* out,
                          int64_t T, int64_t D, const Layout& L) {
    if (D != 32 && D != 64 && D != 128) return false;
    for (const void* p : {q, k, v, out})
        if (((uintptr_t)p & 15) != 0) return false;
    for (const Strides* s : {&L.q, &L.k, &L.v, &L.o})
        if (!strides_ok4(*s)) return false;
    return T < ((int64_t)1 << 30);
}

hipError_t launch_prefill_f32(const float* q, const float* k, const float* v, float* out,
                              int64_t B, int64_t H, int64_t T, int D, int64_t W, const Layout& L,
                              float scale, hipStream_t stream, float* lse) {
    F32Args a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.lse = lse;
    a.L = L;
    a.H = (int)H;
    a.T = (int)T;
    a.W = (int)(W < T ? W : T);
    a.nqt = (int)((T + 31) / 32);
    const int64_t nwaves = B * H * a.nqt;
    a.nwaves = (int)nwaves;
    a.c = kLog2e * fabsf(scale);
    a.qneg = scale < 0.f ? 1 : 0;
    const dim3 grid((unsigned)((nwaves + 3) / 4));
    a.remap = grid.x % 8 == 0 ? 1 : 0;
    void* args[] = {(void*)&a};
    const void* kern = D == 128 ? (const void*)prefill_f32_kernel<128, false>
                     : D == 64  ? (const void*)prefill_f32_kernel<64, false>
                                : (const void*)prefill_f32_kernel<32, false>;
    return hipLaunchKernel(kern, grid, dim3(256), args, 0, stream);
}

bool chunk_f32_supports(const void* q, const void* kc, const void* vc, const void* kring,
                        const void* vring, const void* out, int64_t C, int64_t D, int64_t W) {
    if (D != 32 && D != 64 && D != 128) return false;
    for (const void* p : {q, kc, vc, kring, vring, out})
        if (((uintptr_t)p & 15) != 0) return false;
    // positions (below 2^30 past the chunk start) in int
    return C < ((int64_t)1 << 29) && W < ((int64_t)1 << 29);
}

hipError_t launch_chunk_f32(const float* q, const float* kc, const float* vc, const float* kring,
                            const float* vring, const int64_t* pos0, float* out, int64_t S,
                            int64_t H, int64_t C, int D, int64_t W, hipStream_t stream) {
    F32Args a = {};
    a.q = q;
    a.k = kc;
    a.v = vc;
    a.out = out;
    a.L = contiguous_layout(H, C, D);
    a.H = (int)H;
    a.T = (int)C;
    a.W = (int)W;
    a.kring = kring;
    a.vring = vring;
    a.pos0 = pos0;
    a.nqt = (int)((C + 31) / 32);
    const int64_t nwaves = S * H * a.nqt;
    a.nwaves = (int)nwaves;
    a.c = kLog2e / sqrtf((float)D);
    const dim3 grid((unsigned)((nwaves + 3) / 4));
    a.remap = grid.x % 8 == 0 ? 1 : 0;
    void* args[] = {(void*)&a};
    const void* kern = D == 128 ? (const void*)prefill_f32_kernel<128, true>
                     : D == 64  ? (const void*)prefill_f32_kernel<64, true>
                                : (const void*)prefill_f32_kernel<32, true>;
    return hipLaunchKernel(kern, grid, dim3(256), args, 0, stream);
}

}  // namespace swa
