// Causal sliding-window attention prefill, bf16 in / bf16 out, fp32
// accumulation, on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Band-only iteration.  A workgroup owns a tile of BM = 32 * NW consecutive
// queries [i0, i0 + BM) of one (batch, head) and walks only the 64-key tiles
// that intersect the tile's band [max(0, i0 - W + 1), min(T, i0 + BM)), so the
// work is O(T * min(W, T) * D) and never the dense O(T^2 * D) of the masked
// recipe ("NNX Sliding-Window Attention", A local mask is not a sparse
// implementation).  Each wavefront owns 32 queries and additionally skips the
// key tiles that miss its own band.  The band predicate j <= i and i - j < W
// ("27. Sliding-Window Attention", step 2) is evaluated, as a select to -inf,
// only on the tiles that straddle an edge of the wavefront's band.
//
// Per wavefront and key tile (everything fp32 except the MFMA operands):
//   S^T = K Q^T        32x32 output blocks: lane l holds query l % 32 and 16
//                      keys of it, so row maxima and sums are mostly in-lane
//                      plus one exchange with lane l ^ 32 (v_permlane32_swap)
//   online softmax     running max m and sum l per query (exp2 with the
//                      1/sqrt(D) * log2(e) scale folded into one FMA), the
//                      output rescaled by exp2(m_old - m_new)
//   O^T += V^T P^T     P^T goes from the S^T accumulator straight into the
//                      B operand (converted to bf16, round to nearest even);
//                      V^T comes from LDS, where V is stored transposed with
//                      its keys permuted to match the accumulator's key order.
// K and V^T tiles are staged in LDS, double buffered: the global loads of the
// next tile are in flight while the current one is computed.

#include "swa_internal.h"

namespace swa {
namespace {

template <int D, int NW>
struct Cfg {
    static constexpr int BM = 32 * NW;          // queries per workgroup
    static constexpr int BN = 64;               // keys per tile
    static constexpr int NT = 64 * NW;          // threads
    static constexpr int KSTR = D + 8;          // K tile row stride (elements), +16 B breaks bank aliasing
    static constexpr int VSTR = BN + 8;         // V^T tile row stride (elements)
    static constexpr int KTILE = BN * KSTR;     // elements
    static constexpr int VTILE = D * VSTR;      // elements
    static constexpr int STAGE = KTILE + VTILE; // elements per pipeline stage
    static constexpr int LDS_BYTES = 2 * STAGE * 2;
    static constexpr int CPR = D / 8;           // 16-byte chunks per K/V row
    static constexpr int KCHUNKS = BN * CPR;
    static constexpr int KPT = (KCHUNKS + NT - 1) / NT;
    // V items: (4-key group g, 8-d chunk cc) with g fastest across lanes, so
    // 16 consecutive lanes store one contiguous 128-byte run of a V^T row
    // (no LDS bank conflicts) and load 64-byte runs of 16 key rows.
    static constexpr int VITEMS = (BN / 4) * CPR;
    static constexpr int VPT = (VITEMS + NT - 1) / NT;
    static_assert(D == 64 || D == 128, "head size");
};

struct Args {
    const bf16* q;
    const bf16* k;
    const bf16* v;
    bf16* out;
    int T;
    int W;          // min(W, T)
    int nqt;        // query tiles per (b, h)
    int nblocks;    // grid size
    int remap;      // 1: spread consecutive logical tiles over one XCD
    float c;        // log2(e) / sqrt(D)
};

__device__ inline float swap_max(float x) {
    // v_permlane32_swap exchanges the two 32-lane halves between its two
    // outputs; max over both outputs is the max over lanes l and l ^ 32.
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float swap_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Position, inside a 64-key V^T row, of tile key 4 g + r.  Within each
// 16-key chunk the key offset 8 a + 4 h + r is stored at 8 h + 4 a + r, so
// that lane half h reads its eight B-operand keys as one 16-byte vector.
__device__ inline int vt_pos(int g) {
    const int c16 = g >> 2, gg = g & 3;
    return 16 * c16 + 8 * (gg & 1) + 4 * (gg >> 1);
}

// Global -> registers for key tile [k0, k0 + 64).  Rows past the sequence
// are clamped to row T - 1: those keys lie above every valid query's
// diagonal, so the band mask sends their scores to -inf and their values are
// multiplied by an exact zero.  No branch, so the loads stay in flight while
// the current tile is computed.
template <int D, int NW>
__device__ inline void load_tile(const bf16* __restrict__ Kbh, const bf16* __restrict__ Vbh,
                                 int k0, int Tm1, int tid, u32x4 (&kreg)[Cfg<D, NW>::KPT],
                                 u32x4 (&vreg)[Cfg<D, NW>::VPT][4]) {
    using C = Cfg<D, NW>;
#pragma unroll
    for (int r = 0; r < C::KPT; ++r) {
        const int c = tid + r * C::NT;
        if (C::KCHUNKS % C::NT == 0 || c < C::KCHUNKS) {
            const int key = min(k0 + c / C::CPR, Tm1);
            kreg[r] = *reinterpret_cast<const u32x4*>(Kbh + key * D + (c % C::CPR) * 8);
        }
    }
#pragma unroll
    for (int r = 0; r < C::VPT; ++r) {
        const int it = tid + r * C::NT;
        if (C::VITEMS % C::NT == 0 || it < C::VITEMS) {
            const int g = it % (C::BN / 4), cc = it / (C::BN / 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int key = min(k0 + 4 * g + e, Tm1);
                vreg[r][e] = *reinterpret_cast<const u32x4*>(Vbh + key * D + cc * 8);
            }
        }
    }
}

template <int D, int NW>
__device__ inline void store_tile(bf16* __restrict__ stage, int tid,
                                  const u32x4 (&kreg)[Cfg<D, NW>::KPT],
                                  const u32x4 (&vreg)[Cfg<D, NW>::VPT][4]) {
    using C = Cfg<D, NW>;
    bf16* Ks = stage;
    bf16* Vs = stage + C::KTILE;
#pragma unroll
    for (int r = 0; r < C::KPT; ++r) {
        const int c = tid + r * C::NT;
        if (C::KCHUNKS % C::NT == 0 || c < C::KCHUNKS)
            *reinterpret_cast<u32x4*>(Ks + (c / C::CPR) * C::KSTR + (c % C::CPR) * 8) = kreg[r];
    }
#pragma unroll
    for (int r = 0; r < C::VPT; ++r) {
        const int it = tid + r * C::NT;
        if (C::VITEMS % C::NT == 0 || it < C::VITEMS) {
            const int g = it % (C::BN / 4), cc = it / (C::BN / 4);
            bf16* dst = Vs + (cc * 8) * C::VSTR + vt_pos(g);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // keys 4g..4g+3 of d = 8cc + 2j (low halves) and 8cc + 2j + 1
                const uint32_t r0 = vreg[r][0][j], r1 = vreg[r][1][j];
                const uint32_t r2 = vreg[r][2][j], r3 = vreg[r][3][j];
                const uint32_t lo_e = __builtin_amdgcn_perm(r1, r0, 0x05040100u);
                const uint32_t hi_e = __builtin_amdgcn_perm(r3, r2, 0x05040100u);
                const uint32_t lo_o = __builtin_amdgcn_perm(r1, r0, 0x07060302u);
                const uint32_t hi_o = __builtin_amdgcn_perm(r3, r2, 0x07060302u);
                *reinterpret_cast<u32x2*>(dst + (2 * j) * C::VSTR) = u32x2{lo_e, hi_e};
                *reinterpret_cast<u32x2*>(dst + (2 * j + 1) * C::VSTR) = u32x2{lo_o, hi_o};
            }
        }
    }
}

// Lazy rescale threshold, in log2 units: the reference max of a row is only
// raised when a new score exceeds it by more than this, so probabilities stay
// below 2^8 and the output accumulator is rarely rescaled.  The final O / l
// is the same quotient whichever reference is used.
constexpr float kRescaleLog2 = 8.0f;

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_bf16_kernel(Args a) {
    using C = Cfg<D, NW>;
    extern __shared__ __attribute__((aligned(16))) bf16 lds[];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 31, hh = lane >> 5;

    // Logical tile: consecutive logical tiles land on one XCD (the hardware
    // deals workgroups round-robin over 8 XCDs), heads stay together, and
    // within a head the tiles with the longest bands (the last ones) go first.
    const int bid = blockIdx.x;
    const int logical = a.remap ? (bid & 7) * (a.nblocks >> 3) + (bid >> 3) : bid;
    const int bh = logical / a.nqt;
    const int qt = a.nqt - 1 - (logical - bh * a.nqt);
    const int T = a.T, W = a.W;        // W is clamped to T on the host (W >= T is causal)
    const int i0 = qt * C::BM;
    const int64_t off = (int64_t)bh * T * D;
    const bf16* __restrict__ Qbh = a.q + off;
    const bf16* __restrict__ Kbh = a.k + off;
    const bf16* __restrict__ Vbh = a.v + off;

    const int qw0 = i0 + 32 * wave;                  // this wave's first query
    const int qi = qw0 + lr;                         // this lane's query
    const bool wave_active = qw0 < T;
    const int wlo = max(qw0 - W + 1, 0);             // wave's lowest visible key
    const int whi = min(qw0 + 32, T);                // one past its highest

    // Q^T operand: lane holds q[qi][16 dc + 8 hh .. + 7] for every 16-wide d
    // chunk (rows past T read row T - 1; their outputs are never stored).
    bf16x8 qf[D / 16];
    {
        const bf16* qp = Qbh + min(qi, T - 1) * D + 8 * hh;
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) qf[dc] = *reinterpret_cast<const bf16x8*>(qp + 16 * dc);
    }

    const int klo = max(i0 - W + 1, 0);
    const int khi = min(i0 + C::BM, T);
    const int t0 = klo / C::BN;
    const int t1 = (khi + C::BN - 1) / C::BN;

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    float m = -__builtin_inff();      // reference max (raw score units)
    float lsum = 0.f;                 // this lane's half of the row sum
    const float c = a.c;
    const float tau = kRescaleLog2 / c;

    u32x4 kreg[C::KPT];
    u32x4 vreg[C::VPT][4];
    load_tile<D, NW>(Kbh, Vbh, t0 * C::BN, T - 1, tid, kreg, vreg);
    store_tile<D, NW>(lds, tid, kreg, vreg);
    // Everything loaded so far (Q fragments, first tile) has landed: the
    // in-loop waits then only concern the prefetch of the next tile.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int t = t0; t < t1; ++t) {
        const int cur = (t - t0) & 1;
        // Prefetch the next tile (the last iteration re-reads its own tile
        // into the idle buffer, which keeps the loop free of branches).
        load_tile<D, NW>(Kbh, Vbh, min(t + 1, t1 - 1) * C::BN, T - 1, tid, kreg, vreg);

        const int k0 = t * C::BN;
        if (wave_active && k0 < whi && k0 + C::BN > wlo) {
            const bf16* Ks = lds + cur * C::STAGE;
            const bf16* Vs = Ks + C::KTILE;
            // ---- S^T = K Q^T, two 32-key blocks; K fragments are read ahead
            constexpr int NF = 2 * (D / 16);
            const bf16* kp = Ks + lr * C::KSTR + 8 * hh;
            bf16x8 kf[NF];
#pragma unroll
            for (int f = 0; f < NF; ++f)
                kf[f] = *reinterpret_cast<const bf16x8*>(kp + (f & 1) * 32 * C::KSTR + 16 * (f >> 1));
            f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
            for (int dc = 0; dc < D / 16; ++dc) {
                s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[2 * dc], qf[dc], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[2 * dc + 1], qf[dc], s1, 0, 0, 0);
            }
            // ---- band mask where the tile straddles an edge of this wave's band:
            // key j is visible iff 0 <= qi - j < W (one unsigned compare)
            const bool interior = (k0 + C::BN - 1 <= qw0) && (qw0 + 31 - k0 < W);
            if (!interior) {
                const int base = qi - k0 - 4 * hh;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int kof = 8 * (v >> 2) + (v & 3);
                    s0[v] = (unsigned)(base - kof) < (unsigned)W ? s0[v] : -__builtin_inff();
                    s1[v] = (unsigned)(base - kof - 32) < (unsigned)W ? s1[v] : -__builtin_inff();
                }
            }
            // ---- online softmax with a lazily raised reference max
            float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
            for (int v = 1; v < 16; ++v) mx = fmaxf(mx, fmaxf(s0[v], s1[v]));
            mx = swap_max(mx);
            const bool raise = mx > m + tau;           // false while the row is fully masked
            if (__any(raise)) {
                // 1 for rows keeping their reference (also rows still fully
                // masked, where m - m would be NaN); 0 when m = -inf.
                const float alpha = raise ? __builtin_amdgcn_exp2f((m - mx) * c) : 1.f;
                const float m_new = raise ? mx : m;
                lsum *= alpha;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
                m = m_new;
            }
            const float mc = m == -__builtin_inff() ? 0.f : m * c;
            float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                s0[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[v], c, -mc));
                s1[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[v], c, -mc));
                ps[v & 3] += s0[v] + s1[v];
            }
            lsum += (ps[0] + ps[1]) + (ps[2] + ps[3]);
            // ---- O^T += V^T P^T, four 16-key chunks
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) {
                const f32x16& sb = (ch >> 1) ? s1 : s0;
                const int e0 = 8 * (ch & 1);
                bf16x8 pf;
#pragma unroll
                for (int e = 0; e < 8; ++e) pf[e] = (bf16)sb[e0 + e];
                const bf16* vp = Vs + lr * C::VSTR + 16 * ch + 8 * hh;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const bf16x8 va = *reinterpret_cast<const bf16x8*>(vp + 32 * db * C::VSTR);
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf, o[db], 0, 0, 0);
                }
            }
        }

        store_tile<D, NW>(lds + (cur ^ 1) * C::STAGE, tid, kreg, vreg);
        __syncthreads();
    }

    // ---- finalise: O / l, bf16, store (lane holds d = 32 db + 8 g + 4 hh + 0..3)
    const float l = swap_sum(lsum);
    const float inv = 1.f / l;
    if (qi < T) {
        bf16* orow = a.out + off + (int64_t)qi * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = (bf16)(o[db][4 * g + e] * inv);
                *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * g + 4 * hh) = w;
            }
    }
}

template <int D, int NW>
hipError_t launch(const bf16* q, const bf16* k, const bf16* v, bf16* out, int64_t B,
                  int64_t H, int64_t T, int64_t W, hipStream_t stream) {
    using C = Cfg<D, NW>;
    static bool attr_set = false;   // per process; the attribute is per function
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)prefill_bf16_kernel<D, NW>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           C::LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    Args a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.T = (int)T;
    a.W = (int)(W < T ? W : T);
    a.nqt = (int)((T + C::BM - 1) / C::BM);
    const int64_t nblocks = B * H * a.nqt;
    a.nblocks = (int)nblocks;
    a.remap = (nblocks % 8 == 0) ? 1 : 0;
    a.c = kLog2e / sqrtf((float)D);
    void* args[] = {(void*)&a};
    return hipLaunchKernel((const void*)prefill_bf16_kernel<D, NW>, dim3((unsigned)nblocks),
                           dim3(C::NT), args, C::LDS_BYTES, stream);
}

}  // namespace

hipError_t launch_prefill_bf16(const bf16* q, const bf16* k, const bf16* v, bf16* out,
                               int64_t B, int64_t H, int64_t T, int D, int64_t W,
                               hipStream_t stream) {
    if (D == 128) return launch<128, 4>(q, k, v, out, B, H, T, W, stream);
    return launch<64, 4>(q, k, v, out, B, H, T, W, stream);
}

}  // namespace swa
