// Backward of the causal sliding-window attention prefill, bf16 in / out,
// fp32 accumulation, on gfx950 matrix cores.
//
// With S = q k^T * scale over the band, P = softmax(S) and out = P v, the
// gradients are (the pages define the forward only; "NNX Sliding-Window
// Attention", Mask before softmax, notes that masked weights are zero and
// gradients stay defined):
//   dV = P^T dout, dP = dout v^T, dS = P (dP - delta), delta_i = dout_i . out_i,
//   dQ = dS k * scale, dK = dS^T q * scale.
// P is rebuilt tile by tile as exp2(s * c - L_i log2(e)) from the forward's
// per-row log-sum-exp L_i (c = log2(e) * scale), so no T x T array exists.
//
// Sharper softmaxes (an explicit |scale| above 1/sqrt(D)) raise two roundings
// above the bf16 bar: delta taken from the bf16 output cancels against dP
// of the dominant key, and so does any common error of the rebuilt P (the
// forward's row sums run over bf16 weights).  There the precise variant
// first runs ST (below) for each row's z_i = sum_j P_ij and
// y_i = sum_j P_ij dP_ij in fp32, replaces L_i by L_i + ln z_i (so the
// rebuilt weights sum to one) and takes delta_i = y_i / z_i, and DQ and DK
// feed dS to the matrix cores as two bf16 terms (hi + lo) instead of one.
//
// Two kernels.  The query-row kernel (DQ, and ST for the precise variant):
// a workgroup of 4 wavefronts owns 128 queries (32 per wavefront) and walks
// the 32-key tiles of its band through an LDS ring (HBM -> LDS buffer loads,
// 3 tiles ahead, one barrier per tile).  Per wavefront and tile:
//   DQ  S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - delta),
//       dQ^T += K^T dS^T                                  (24 MFMAs)
//   ST  S^T = K Q^T, dP^T = V dO^T, z += P, y += P dP     (16)
// (DQ issues 8 more with the split dS.)  dV and dK come from one key-row
// kernel, bwd_kv_kernel (below), on 16x16x32 MFMAs: S, dP, dV and dK in
// 32 MFMAs of half the size per 16 keys and 32 queries, so it rebuilds S
// once for both gradients.
// The accumulator layout of v_mfma_f32_32x32x16_bf16 gives lane l column
// l % 32 (a row item) and 16 column-tile items 8 (v/4) + 4 (l/32) + v%4, so
// the packed probabilities feed the next product's B operand directly, as in
// the forward kernel, and transposed operands come from ds_read_b64_tr_b16.
// DQ reads its k tile, and the key-row kernel its q and dout tiles, both
// whole and transposed, from one LDS copy each (swizzles bswz and qswz, one
// per operand layout), which serves both reads without bank conflicts.

#include "swa_mfma.h"

#include <type_traits>

namespace swa {
namespace {

enum Mode { kDQ = 0, kST = 1 };

template <int D, int MODE>
struct BCfg {
    static constexpr int NW = 4;                // wavefronts per workgroup
    static constexpr int BM = 32 * NW;          // query rows per workgroup
    static constexpr int BN = 32;               // keys per tile
    static constexpr int TILEB = BN * 2 * D;    // bytes per tile
    static constexpr int NTL = 2;               // tile kinds per step (k, v)
    static constexpr int PF = 3;                // tiles in flight ahead
    static constexpr int R = PF + 1;            // ring slots per tile kind
    static constexpr int NLD_W = TILEB / 1024 / NW;
    static constexpr int NLD_T = NTL * NLD_W;   // loads per wave per tile
    static constexpr int VM_WAIT = (PF - 1) * NLD_T;
    static_assert(D == 64 || D == 128, "head size");
    static_assert(VM_WAIT < 64, "vmcnt range");
};

struct BArgs {
    const bf16* q;
    const bf16* k;
    const bf16* v;
    const bf16* o;        // forward output (DQ: delta)
    const bf16* dout;
    bf16* grad;           // DQ: dq; key kernel: dv   ([B, H, T, D])
    bf16* grad2;          // key kernel: dk
    const float* lse;     // [B * H * T] log-sum-exp of the scaled scores (forward;
                          // precise DQ: ST's lse_w)
    float* delta;         // [B * H * T] -(dout . out) (written by DQ; precise: by ST)
    float* lse_w;         // [B * H * T] log2 normaliser of the rebuilt weights, read
                          // by the key kernel (written by DQ; precise: by ST)
    int T, W, nrt, nblocks, remap;
    int nfull;            // longest-first dispatch (xcd_logical_tile); -1: plain order
    float c;              // log2(e) * scale
    float scale;
};

// Eight values as a bf16 B operand.
__device__ inline bf16x8 pack8(const f32x16& s, int e0) {
    bf16x8 p;
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = (bf16)s[e0 + e];
    return p;
}

// Eight values as two bf16 B operands whose sum is them to about 2^-16
// relative: hi = bf16(x), lo = bf16(x - hi).
__device__ inline void pack8_split(const f32x16& s, int e0, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        hi[e] = (bf16)s[e0 + e];
        lo[e] = (bf16)(s[e0 + e] - (float)hi[e]);
    }
}

// Query-row kernel (rows = queries, columns = keys): DQ, or ST (the row
// statistics of the precise variant).  PREC: DQ takes ST's delta and splits dS.
template <int D, int MODE, bool PREC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_bf16_kernel(BArgs a) {
    using C = BCfg<D, MODE>;
    __shared__ __attribute__((aligned(1024))) char ring[C::NTL * C::R * C::TILEB];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lr = lane & 31, hh = lane >> 5;

    const int bid = blockIdx.x;
    const int logical = xcd_logical_tile(bid, a.nblocks, a.remap, a.nrt, a.nfull);
    const int bh = logical / a.nrt;
    const int rti = logical - bh * a.nrt;
    const int rt = a.nrt - 1 - rti;             // longest bands (the last query tiles) first
    const int T = a.T, W = a.W;
    const int64_t off = (int64_t)bh * T * D;
    const bf16* Q = a.q + off;
    const bf16* K = a.k + off;
    const bf16* V = a.v + off;
    const bf16* DO = a.dout + off;

    const int r0 = rt * C::BM;                  // workgroup's queries [r0, r0 + BM)
    const int rw0 = r0 + 32 * wave;             // this wave's queries
    const int ri = rw0 + lr;                    // this lane's query
    // keys j with 0 <= i - j < W, for the workgroup and for this wave
    const int c_lo = max(r0 - W + 1, 0), c_hi = min(r0 + C::BM, T);
    const int w_lo = max(rw0 - W + 1, 0), w_hi = min(rw0 + 32, T);
    const int t0 = c_lo / C::BN, t1 = (c_hi + C::BN - 1) / C::BN;
    const bool live = rw0 < T;
    const int wt0 = live ? w_lo / C::BN : t1, wt1 = live ? (w_hi + C::BN - 1) / C::BN : t1;
    auto needs = [&](int t) { return t >= wt0 && t < wt1; };
    // every (query, key) pair of the tile inside the band
    auto interior = [&](int t) {
        const int k0 = t * C::BN;
        return k0 + 31 <= rw0 && rw0 + 31 - k0 < W;
    };

    // register operands: the wave's 32 q and dout rows (B operands of S^T and
    // dP^T), clamped to the last row past the end
    const int rc = min(ri, T - 1);
    bf16x8 f0[D / 16], f1[D / 16];
    {
        const bf16* p0 = Q + (int64_t)rc * D + 8 * hh;
        const bf16* p1 = DO + (int64_t)rc * D + 8 * hh;
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) {
            f0[dc] = *reinterpret_cast<const bf16x8*>(p0 + 16 * dc);
            f1[dc] = *reinterpret_cast<const bf16x8*>(p1 + 16 * dc);
        }
    }
    // this row's log2 normaliser (the forward's natural-log lse, or for the
    // precise DQ ST's log2 output); DQ: delta = dout . out (published with
    // the normaliser for the key kernel), or (precise) ST's delta
    const float Lrow = (MODE == kDQ && PREC) ? a.lse[(int64_t)bh * T + rc]
                                             : a.lse[(int64_t)bh * T + rc] * kLog2e;
    // nd = -delta (the delta arrays hold -delta: it starts the dP products'
    // accumulation, so they yield dP - delta directly)
    float nd = 0.f;
    if (MODE == kDQ && PREC) {
        nd = a.delta[(int64_t)bh * T + rc];
    } else if (MODE == kDQ) {
        const bf16* po = a.o + off + (int64_t)rc * D + 8 * hh;
        float d = 0.f;
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) {
            const bf16x8 ov = *reinterpret_cast<const bf16x8*>(po + 16 * dc);
#pragma unroll
            for (int e = 0; e < 8; ++e) d = fmaf((float)f1[dc][e], (float)ov[e], d);
        }
        nd = -swap_sum(d);
        if (hh == 0 && ri < T) {
            a.delta[(int64_t)bh * T + ri] = nd;
            a.lse_w[(int64_t)bh * T + ri] = Lrow;
        }
    }
    // land the register operands before any tile load is counted
    __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));

    // ---- tile ring: kind x of tile t in slot x * R + (t - t0) % R
    // 0 = K (DQ: read whole and transposed; ST: whole), 1 = V (rows whole)
    constexpr int SW0 = MODE == kST ? kSwzK : kSwzB;   // swizzle of kind 0
    // Ring slot s of kind x (tile t lives in slot (t - t0) mod R); slot numbers
    // are compile-time constants at every call site (the key loop is unrolled
    // over the R = 4 slots), so LDS addresses carry them as immediates.
    static_assert(C::R == 4, "the loop is unrolled over 4 ring slots");
    auto slot = [&](int x, int s) { return ring + (x * C::R + s % C::R) * C::TILEB; };
    uint32_t off0[C::NLD_W], off1[C::NLD_W];
    tile_offsets<D, C::NW, SW0>(off0, wave, lane, 2 * D);
    tile_offsets<D, C::NW, kSwzK>(off1, wave, lane, 2 * D);
    const int slab = T * D * 2;
    auto load = [&](int t, int s) {   // tile t into ring slot s
        const int tt = min(t, t1 - 1);
        const int boff = tt * C::TILEB;
        dma_tile(rows_rsrc(K, boff, slab), lds_addr(slot(0, s)), wave, off0);
        dma_tile(rows_rsrc(V, boff, slab), lds_addr(slot(1, s)), wave, off1);
    };
    // Wait until this wave's loads of the next tile have landed (at most the
    // PF - 1 newer tiles' loads in flight) and its LDS reads are done, then
    // barrier: the next tile is visible to every wave and the slots of the
    // current one are free.
    auto publish = [&]() {
        __builtin_amdgcn_s_waitcnt((C::VM_WAIT & 15) | ((C::VM_WAIT >> 4) << 14) | (7 << 4) | (0 << 8));
        __builtin_amdgcn_s_barrier();
    };

    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
    const float c = a.c;
    // masked scores: -inf, or +inf for a negative scale (s * c is then -inf)
    const float sfill = c >= 0.f ? -__builtin_inff() : __builtin_inff();
    float zsum = 0.f, ysum = 0.f;               // ST: this lane's share of z and y

#pragma unroll
    for (int i = 0; i < C::PF; ++i) load(t0 + i, i);
    publish();                // tile t0 has landed
    // one key tile j, in ring slot KS = (j - t0) mod 4
    auto step = [&](auto ks, int j) {
        constexpr int KS = decltype(ks)::value;
        load(j + C::PF, KS + C::PF);   // into the slot of tile j - 1, released by the last barrier
        if (needs(j)) {
            const int k0 = j * C::BN;
            const char* A0 = slot(0, KS);
            const char* A1 = slot(1, KS);
            // S^T = K Q^T and dP^T = V dO^T
            f32x16 s = f32x16{}, dp;
#pragma unroll
            for (int vv = 0; vv < 16; ++vv) dp[vv] = nd;
#pragma unroll
            for (int dc = 0; dc < D / 16; ++dc) {
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_row_frag<D, SW0>(A0, lr, hh, dc),
                                                            f0[dc], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_row_frag<D, kSwzK>(A1, lr, hh, dc),
                                                             f1[dc], dp, 0, 0, 0);
            }
            // band mask: query ri against keys k0 + 8 (v/4) + 4 hh + v%4
            if (!interior(j)) {
#pragma unroll
                for (int vv = 0; vv < 16; ++vv) {
                    const int col = k0 + 8 * (vv >> 2) + 4 * hh + (vv & 3);
                    const bool ok = (unsigned)(ri - col) < (unsigned)W && ri < T;
                    s[vv] = ok ? s[vv] : sfill;
                }
            }
            // P and (DQ) dS; (ST) the row sums of P and P dP
#pragma unroll
            for (int vv = 0; vv < 16; ++vv) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[vv], c, -Lrow));
                if (MODE == kST) {
                    zsum += p;
                    ysum = __builtin_fmaf(p, dp[vv], ysum);
                } else {
                    s[vv] = p * dp[vv];
                }
            }
            if constexpr (MODE == kDQ) {
                // dQ^T += K^T dS^T (k transposed from the same LDS copy)
                bf16x8 t0f[D / 32], t1f[D / 32];
                read_v_chunk<D, kSwzB>(A0, 0, lane, t0f);
                read_v_chunk<D, kSwzB>(A0, 1, lane, t1f);
                if constexpr (PREC) {
                    bf16x8 h0, l0, h1, l1;
                    pack8_split(s, 0, h0, l0);
                    pack8_split(s, 8, h1, l1);
#pragma unroll
                    for (int db = 0; db < D / 32; ++db) {
                        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t0f[db], h0, acc[db], 0, 0, 0);
                        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t0f[db], l0, acc[db], 0, 0, 0);
                    }
#pragma unroll
                    for (int db = 0; db < D / 32; ++db) {
                        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t1f[db], h1, acc[db], 0, 0, 0);
                        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t1f[db], l1, acc[db], 0, 0, 0);
                    }
                } else {
                    const bf16x8 b0 = pack8(s, 0), b1 = pack8(s, 8);
#pragma unroll
                    for (int db = 0; db < D / 32; ++db)
                        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t0f[db], b0, acc[db], 0, 0, 0);
#pragma unroll
                    for (int db = 0; db < D / 32; ++db)
                        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t1f[db], b1, acc[db], 0, 0, 0);
                }
            }
        }
        publish();            // tile j + 1 has landed; tile j's slots are free
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    for (int j = t0; j < t1;) {
        step(I0{}, j);
        if (++j >= t1) break;
        step(I1{}, j);
        if (++j >= t1) break;
        step(I2{}, j);
        if (++j >= t1) break;
        step(I3{}, j);
        ++j;
    }
    __builtin_amdgcn_s_waitcnt(0);   // no LDS load may outlive the workgroup

    if constexpr (MODE == kST) {
        // each row's z and y over its band (lanes l, l ^ 32 hold halves)
        const float z = swap_sum(zsum), y = swap_sum(ysum);
        if (hh == 0 && ri < T) {
            a.lse_w[(int64_t)bh * T + ri] = Lrow + __builtin_amdgcn_logf(z);
            a.delta[(int64_t)bh * T + ri] = -(y / z);
        }
        return;
    }

    // store (lane holds d = 32 db + 8 g + 4 hh + 0..3 of query ri)
    if (ri < T) {
        bf16* row = a.grad + off + (int64_t)ri * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = (bf16)(acc[db][4 * g + e] * a.scale);
                *reinterpret_cast<bf16x4*>(row + 32 * db + 8 * g + 4 * hh) = w;
            }
    }
}

typedef float f32x4v __attribute__((ext_vector_type(4)));

// Key-row kernel computing dV and dK together (rows = keys, columns =
// queries), 16 key rows per wavefront on v_mfma_f32_16x16x32_bf16 so that
// both accumulators fit beside the operands at two wavefronts per SIMD.  Per
// wavefront and 32-query tile (two 16-query blocks):
//   S^T = Q K^T, dP^T = dO V^T           (2 x D/32 MFMAs each; k, v rows of
//                                          the wavefront stay in registers)
//   P^T = exp2(S^T c - L), dS^T = P^T (dP^T - delta)
//   dV^T += dO^T P^T, dK^T += Q^T dS^T    (D/16 MFMAs each, the transposed
//                                          operands from ds_read_b64_tr_b16;
//                                          the precise variant adds D/16 for
//                                          the lo term of dS)
// 16x16x32 operand layout: lane l gives row (or column) l % 16 and the eight
// contraction items 8 (l / 16) .. + 7; the accumulator gives lane l column
// l % 16 and rows 4 (l / 16) .. + 3.  A lane of group g = l / 16 thus holds
// P^T, dS^T for its key and the queries 4g .. 4g+3 of both 16-query blocks,
// which is the (permuted) contraction order of the B operand; the
// transposed A operands are read in that same query order.  At 162 registers
// three wavefronts fit a SIMD, so three workgroups share a CU, with a
// three-slot ring (tiles two steps ahead) to fit their LDS.
template <int D, bool PREC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void bwd_kv_kernel(BArgs a) {
    constexpr int NW = 4, RW = 16, BM = NW * RW, BN = 32;
    constexpr int TILEB = BN * 2 * D;
    constexpr int PF = 2, R = PF + 1;
    constexpr int NLD_W = TILEB / 1024 / NW;
    constexpr int NLD_T = 2 * NLD_W + 2;            // Q, dout tiles; L and delta
    constexpr int VM_WAIT = (PF - 1) * NLD_T;
    constexpr int KC = D / 32;                      // 32-wide contraction steps over D
    constexpr int DB = D / 16;                      // 16-row blocks of D
    static_assert(VM_WAIT < 64, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) char ring[2 * R * TILEB];
    __shared__ __attribute__((aligned(16))) float stats[R][64];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15, g = lane >> 4;

    const int logical = xcd_logical_tile(blockIdx.x, a.nblocks, a.remap, a.nrt, a.nfull);
    const int bh = logical / a.nrt;
    const int rt = logical - bh * a.nrt;            // longest bands (first key tiles) first
    const int T = a.T, W = a.W;
    const int64_t off = (int64_t)bh * T * D;
    const bf16* Q = a.q + off;
    const bf16* K = a.k + off;
    const bf16* V = a.v + off;
    const bf16* DO = a.dout + off;

    const int r0 = rt * BM;                         // workgroup's keys [r0, r0 + BM)
    const int rw0 = r0 + RW * wave;                 // this wave's keys
    const int kr = rw0 + l16;                       // this lane's key
    const int c_hi = min(r0 + BM - 1 + W, T);       // queries i with 0 <= i - j < W
    const int t0 = r0 / BN, t1 = (c_hi + BN - 1) / BN;
    const bool live = rw0 < T;
    const int wt0 = live ? rw0 / BN : t1;
    const int wt1 = live ? (min(rw0 + RW - 1 + W, T) + BN - 1) / BN : t1;
    auto needs = [&](int t) { return t >= wt0 && t < wt1; };
    auto interior = [&](int t) {
        const int q0 = t * BN;
        return q0 >= rw0 + RW - 1 && q0 + BN - 1 - rw0 < W && q0 + BN - 1 < T;
    };

    // B operands of S^T and dP^T: this lane's key row of k and of v,
    // d = 32 kc + 8 g .. + 7 (rows past T read row T - 1; never stored)
    bf16x8 kb[KC], vb[KC];
    {
        const int rc = min(kr, T - 1);
        const bf16* pk = K + (int64_t)rc * D + 8 * g;
        const bf16* pv = V + (int64_t)rc * D + 8 * g;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            kb[kc] = *reinterpret_cast<const bf16x8*>(pk + 32 * kc);
            vb[kc] = *reinterpret_cast<const bf16x8*>(pv + 32 * kc);
        }
    }
    __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));

    // ring: kind 0 = Q, kind 1 = dout, both read whole rows and transposed
    // Ring slot s of kind x (tile t lives in slot (t - t0) mod R); the loop
    // is unrolled over the R = 3 slots, so slot addresses are immediates.
    static_assert(R == 3, "the loop is unrolled over 3 ring slots");
    auto slot = [&](int x, int s) { return ring + (x * R + s % R) * TILEB; };
    uint32_t offs[NLD_W];
    tile_offsets<D, NW, kSwzQ>(offs, wave, lane, 2 * D);
    const int slab = T * D * 2;
    const __amdgpu_buffer_rsrc_t lse_rs = __builtin_amdgcn_make_buffer_rsrc(
        a.lse_w + (int64_t)bh * T, 0, T * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t del_rs = __builtin_amdgcn_make_buffer_rsrc(
        a.delta + (int64_t)bh * T, 0, T * 4, 0x00020000);
    auto load = [&](int t, int s) {
        const int tt = min(t, t1 - 1);
        const int boff = tt * TILEB;
        dma_tile(rows_rsrc(Q, boff, slab), lds_addr(slot(0, s)), wave, offs);
        dma_tile(rows_rsrc(DO, boff, slab), lds_addr(slot(1, s)), wave, offs);
        const uint32_t sbase = lds_addr(&stats[s % R][0]);
        const uint32_t soff = (tt * BN + 4 * (lane & 7)) * 4;
        if (lane < 8) lds_load16(lse_rs, sbase, soff);
        if (lane >= 8 && lane < 16) lds_load16(del_rs, sbase, soff);
    };
    auto publish = [&]() {
        __builtin_amdgcn_s_waitcnt((VM_WAIT & 15) | ((VM_WAIT >> 4) << 14) | (7 << 4) | (0 << 8));
        __builtin_amdgcn_s_barrier();
    };
    // A operand rows of a tile: row 16 blk + l16, 16-byte chunk 4 kc + g
    auto row_frag = [&](const char* tile, int blk, int kc) {
        const int row = 16 * blk + l16;
        return *reinterpret_cast<const bf16x8*>(tile + row * (2 * D) +
                                                (((4 * kc + g) ^ qswz<D>(row)) << 4));
    };
    // Transposed A operand: lane l16 of group g gets tile[16 blk + 4 g + e][16 db + l16]
    // for e = 0..3 (elements 4 blk + e of the bf16x8); source lane j reads row
    // 16 blk + 4 g + j / 4 at columns 16 db + 4 (j % 4) .. + 3.
    auto tr_frag = [&](const char* tile, int db) {
        i16x4 part[2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int row = 16 * blk + 4 * g + (l16 >> 2);
            const int col = 16 * db + 4 * (l16 & 3);
            const int chunk = col >> 3;
            part[blk] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4_t*)(tile + row * (2 * D) + ((chunk ^ qswz<D>(row)) << 4) + 2 * (col & 7)));
        }
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4,
                                                                  5, 6, 7));
    };

    f32x4v adv[DB], adk[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        adv[db] = f32x4v{};
        adk[db] = f32x4v{};
    }
    const float c = a.c;
    const float sfill = c >= 0.f ? -__builtin_inff() : __builtin_inff();

#pragma unroll
    for (int i = 0; i < PF; ++i) load(t0 + i, i);
    publish();
    auto step = [&](auto ks, int j) {
        constexpr int KS = decltype(ks)::value;
        load(j + PF, KS + PF);
        if (needs(j)) {
            const char* TQ = slot(0, KS);
            const char* TD = slot(1, KS);
            const float* st = &stats[KS][0];
            f32x4v Ls[2], Ds[2];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                Ls[blk] = *reinterpret_cast<const f32x4v*>(st + 16 * blk + 4 * g);
                Ds[blk] = *reinterpret_cast<const f32x4v*>(st + 32 + 16 * blk + 4 * g);
            }
            f32x4v s[2], dp[2];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                s[blk] = f32x4v{};
                dp[blk] = Ds[blk];   // -delta: the products give dP - delta
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    s[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(row_frag(TQ, blk, kc), kb[kc],
                                                                     s[blk], 0, 0, 0);
                    dp[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(row_frag(TD, blk, kc), vb[kc],
                                                                      dp[blk], 0, 0, 0);
                }
            }
            // this lane: key kr, queries q0 + 16 blk + 4 g + i
            const int q0 = j * BN;
            if (!interior(j)) {
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int qq = q0 + 16 * blk + 4 * g + i;
                        const bool ok = (unsigned)(qq - kr) < (unsigned)W && qq < T;
                        s[blk][i] = ok ? s[blk][i] : sfill;
                    }
            }
            float pv[8], dsv[8];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[blk][i], c, -Ls[blk][i]));
                    pv[4 * blk + i] = p;
                    dsv[4 * blk + i] = p * dp[blk][i];
                }
            bf16x8 pp, ph, pl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pp[e] = (bf16)pv[e];
                ph[e] = (bf16)dsv[e];
                if constexpr (PREC) pl[e] = (bf16)(dsv[e] - (float)ph[e]);
            }
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                adv[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tr_frag(TD, db), pp, adv[db], 0, 0, 0);
                const bf16x8 tq = tr_frag(TQ, db);
                adk[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tq, ph, adk[db], 0, 0, 0);
                if constexpr (PREC)
                    adk[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tq, pl, adk[db], 0, 0, 0);
            }
            // issue order: the first two operand sets, then each set's
            // products followed by the reads of the set after next
            constexpr int MF = PREC ? 3 : 2;
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
            for (int i = 0; i < DB - 2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, MF, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, MF, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, MF, 0);
        }
        publish();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    for (int j = t0; j < t1;) {
        step(I0{}, j);
        if (++j >= t1) break;
        step(I1{}, j);
        if (++j >= t1) break;
        step(I2{}, j);
        ++j;
    }
    __builtin_amdgcn_s_waitcnt(0);   // no LDS load may outlive the workgroup

    // store: lane holds d = 16 db + 4 g + 0..3 of key kr
    if (kr < T) {
        bf16* rv = a.grad + off + (int64_t)kr * D;       // dv
        bf16* rk = a.grad2 + off + (int64_t)kr * D;      // dk
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            bf16x4 wv, wk;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                wv[e] = (bf16)adv[db][e];
                wk[e] = (bf16)(adk[db][e] * a.scale);
            }
            *reinterpret_cast<bf16x4*>(rv + 16 * db + 4 * g) = wv;
            *reinterpret_cast<bf16x4*>(rk + 16 * db + 4 * g) = wk;
        }
    }
}

template <int D, bool PREC>
hipError_t launch_kv(BArgs a, int64_t B, int64_t H, hipStream_t st) {
    constexpr int BM = 64;
    a.nrt = (a.T + BM - 1) / BM;
    const int64_t nblocks = B * H * a.nrt;
    a.nblocks = (int)nblocks;
    a.remap = nblocks % 8 == 0 ? 1 : 0;
    a.nfull = xcd_longest_first_nfull(nblocks, a.nrt, (a.W - 1 + BM - 1) / BM);
    void* args[] = {(void*)&a};
    return hipLaunchKernel((const void*)bwd_kv_kernel<D, PREC>, dim3((unsigned)nblocks), dim3(256),
                           args, 0, st);
}

template <int D, int MODE, bool PREC>
hipError_t launch_mode(BArgs a, int64_t B, int64_t H, hipStream_t st) {
    using C = BCfg<D, MODE>;
    a.nrt = (a.T + C::BM - 1) / C::BM;
    const int64_t nblocks = B * H * a.nrt;
    a.nblocks = (int)nblocks;
    a.remap = nblocks % 8 == 0 ? 1 : 0;
    // query tiles within W - 1 of the sequence's start have shorter bands
    a.nfull = xcd_longest_first_nfull(nblocks, a.nrt, (a.W - 1 + C::BM - 1) / C::BM);
    void* args[] = {(void*)&a};
    return hipLaunchKernel((const void*)bwd_bf16_kernel<D, MODE, PREC>, dim3((unsigned)nblocks),
                           dim3(256), args, 0, st);
}

// lse_ws: workspace log2 row normalisers for the key kernel, written by DQ
// (precise: by ST) from a.lse.  It may be a.lse itself (the forward rerun
// writes its lse there): each row is read and rewritten by the lane that
// owns it, and rows past T, which read row T - 1, are never stored.
template <int D, bool PREC>
hipError_t launch_all(BArgs a, float* lse_ws, bf16* dq, bf16* dk, bf16* dv, int64_t B, int64_t H,
                      hipStream_t st) {
    hipError_t e;
    a.lse_w = lse_ws;
    if constexpr (PREC) {
        e = launch_mode<D, kST, true>(a, B, H, st);
        if (e != hipSuccess) return e;
        a.lse = lse_ws;
    }
    a.grad = dq;
    e = launch_mode<D, kDQ, PREC>(a, B, H, st);
    if (e != hipSuccess) return e;
    a.grad = dv;
    a.grad2 = dk;
    return launch_kv<D, PREC>(a, B, H, st);
}

}  // namespace

bool backward_bf16_supports(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, int64_t T, int64_t D, double scale) {
    if (D != 64 && D != 128) return false;
    for (const void* p : {q, k, v, o, dout})
        if (((uintptr_t)p & 15) != 0) return false;
    return T * D * 2 < ((int64_t)1 << 31);
}

bool backward_bf16_precise(double scale, int64_t D) {
    return fabs(scale) * sqrt((double)D) > kBwdFastSharpness;
}

hipError_t launch_backward_bf16(const bf16* q, const bf16* k, const bf16* v, const bf16* o,
                                const bf16* dout, bf16* dq, bf16* dk, bf16* dv,
                                const float* lse_in, float* lse, float* delta, int64_t B,
                                int64_t H, int64_t T, int D, int64_t W, float scale,
                                hipStream_t stream) {
    if (lse_in == nullptr) {
        // the forward again, for the per-row log-sum-exp; its output goes to
        // dq, which the DQ kernel overwrites
        hipError_t e = launch_prefill_bf16(q, k, v, dq, B, H, T, D, W,
                                           contiguous_layout(H, T, D), scale, stream, lse);
        if (e != hipSuccess) return e;
        lse_in = lse;
    }
    BArgs a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dout = dout;
    a.lse = lse_in;
    a.delta = delta;
    a.T = (int)T;
    a.W = (int)(W < T ? W : T);
    a.c = kLog2e * scale;
    a.scale = scale;
    if (backward_bf16_precise(scale, D)) {
        if (D == 128) return launch_all<128, true>(a, lse, dq, dk, dv, B, H, stream);
        return launch_all<64, true>(a, lse, dq, dk, dv, B, H, stream);
    }
    if (D == 128) return launch_all<128, false>(a, lse, dq, dk, dv, B, H, stream);
    return launch_all<64, false>(a, lse, dq, dk, dv, B, H, stream);
}

}  // namespace swa
