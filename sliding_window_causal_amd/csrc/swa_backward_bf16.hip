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
// The kernels share one skeleton: a workgroup of 4 wavefronts owns 128
// "row" items (32 per wavefront) and walks 32-item "column" tiles of its band
// through an LDS ring (HBM -> LDS buffer loads, 3 tiles ahead, one barrier
// per tile).  Per wavefront and tile:
//   DQ  rows = queries, columns = keys:  S^T = K Q^T, dP^T = V dO^T,
//       dS^T = P^T (dP^T - delta), dQ^T += K^T dS^T      (24 MFMAs)
//   DV  rows = keys, columns = queries:  S = Q K^T, dV^T += dO^T P   (16)
//   DK  rows = keys, columns = queries:  S = Q K^T, dP = dO V^T,
//       dS = P (dP - delta), dK^T += Q^T dS                           (24)
//   ST  rows = queries, columns = keys:  S^T = K Q^T, dP^T = V dO^T,
//       z += P, y += P dP                                             (16)
// (DQ and DK issue 8 more with the split dS.)
// The accumulator layout of v_mfma_f32_32x32x16_bf16 gives lane l column
// l % 32 (a row item) and 16 column-tile items 8 (v/4) + 4 (l/32) + v%4, so
// the packed probabilities feed the next product's B operand directly, as in
// the forward kernel, and transposed operands come from ds_read_b64_tr_b16.
// DQ reads its k tile, and DK its q tile, both whole and transposed, from one
// LDS copy laid out with the bswz swizzle, which serves both reads without
// bank conflicts.

#include "swa_mfma.h"

#include <type_traits>

namespace swa {
namespace {

enum Mode { kDQ = 0, kDV = 1, kDK = 2, kST = 3 };

template <int D, int MODE>
struct BCfg {
    static constexpr int NW = 4;                // wavefronts per workgroup
    static constexpr int BM = 32 * NW;          // row items per workgroup
    static constexpr int BN = 32;               // column items per tile
    static constexpr int TILEB = BN * 2 * D;    // bytes per tile
    static constexpr int NTL = 2;               // tile kinds per step
    static constexpr int PF = 3;                // tiles in flight ahead
    static constexpr int R = PF + 1;            // ring slots per tile kind
    static constexpr int NLD_W = TILEB / 1024 / NW;
    // loads per wave per tile: the tiles, plus (DV, DK) one for the column
    // items' statistics
    static constexpr int NLD_T = NTL * NLD_W + (MODE == kDV ? 1 : MODE == kDK ? 2 : 0);
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
    bf16* grad;           // dq, dk or dv, [B, H, T, D]
    const float* lse;     // [B * H * T] log-sum-exp of the scaled scores (forward)
    float* delta;         // [B * H * T] dout . out (written by DQ; precise: by ST)
    float* lse_w;         // ST: [B * H * T] log normaliser of the rebuilt weights
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

// Per-row statistics of the 16 column items a lane holds in an accumulator
// (items 8 g + 4 hh + 0..3 of a tile), from the tile's 32 values in LDS.
__device__ inline void read_stats(const float* st, int hh, float (&x)[16]) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(st + 8 * g + 4 * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * g + e] = w[e];
    }
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

// PREC: the precise variant (DQ: delta from ST; DQ, DK: split dS).
template <int D, int MODE, bool PREC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_bf16_kernel(BArgs a) {
    using C = BCfg<D, MODE>;
    constexpr bool ROWQ = MODE == kDQ || MODE == kST;   // rows are queries (else keys)
    __shared__ __attribute__((aligned(1024))) char ring[C::NTL * C::R * C::TILEB];
    // DV, DK: log2 normaliser and delta of the 32 column items of a tile
    // (128 bytes each) per ring slot
    __shared__ __attribute__((aligned(16))) float stats[C::R][64];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lr = lane & 31, hh = lane >> 5;

    const int bid = blockIdx.x;
    const int logical = xcd_logical_tile(bid, a.nblocks, a.remap, a.nrt, a.nfull);
    const int bh = logical / a.nrt;
    const int rti = logical - bh * a.nrt;
    // longest bands first: the last query tiles (DQ), the first key tiles (DV, DK)
    const int rt = ROWQ ? a.nrt - 1 - rti : rti;
    const int T = a.T, W = a.W;
    const int64_t off = (int64_t)bh * T * D;
    const bf16* Q = a.q + off;
    const bf16* K = a.k + off;
    const bf16* V = a.v + off;
    const bf16* DO = a.dout + off;

    const int r0 = rt * C::BM;                  // workgroup's row items [r0, r0 + BM)
    const int rw0 = r0 + 32 * wave;             // this wave's rows
    const int ri = rw0 + lr;                    // this lane's row item
    // column band of the workgroup and of this wave
    int c_lo, c_hi, w_lo, w_hi;
    if (ROWQ) {                                 // keys j with 0 <= i - j < W
        c_lo = max(r0 - W + 1, 0);
        c_hi = min(r0 + C::BM, T);
        w_lo = max(rw0 - W + 1, 0);
        w_hi = min(rw0 + 32, T);
    } else {                                    // queries i with 0 <= i - j < W
        c_lo = r0;
        c_hi = min(r0 + C::BM - 1 + W, T);
        w_lo = rw0;
        w_hi = min(rw0 + 31 + W, T);
    }
    const int t0 = c_lo / C::BN, t1 = (c_hi + C::BN - 1) / C::BN;
    const bool live = rw0 < T;
    const int wt0 = live ? w_lo / C::BN : t1, wt1 = live ? (w_hi + C::BN - 1) / C::BN : t1;
    auto needs = [&](int t) { return t >= wt0 && t < wt1; };
    // every (row, column) pair of the tile inside the band and the sequence
    auto interior = [&](int t) {
        const int k0 = t * C::BN;
        if (ROWQ) return k0 + 31 <= rw0 && rw0 + 31 - k0 < W;
        return k0 >= rw0 + 31 && k0 + 31 - rw0 < W && k0 + 31 < T;
    };

    // register operands: the wave's 32 row items (B operands of the first
    // products), clamped to the last row past the end
    const int rc = min(ri, T - 1);
    bf16x8 f0[D / 16], f1[D / 16];              // DQ: q, dout rows; DV/DK: k, v rows
    {
        const bf16* p0 = (ROWQ ? Q : K) + (int64_t)rc * D + 8 * hh;
        const bf16* p1 = (ROWQ ? DO : V) + (int64_t)rc * D + 8 * hh;
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) {
            f0[dc] = *reinterpret_cast<const bf16x8*>(p0 + 16 * dc);
            if (MODE != kDV) f1[dc] = *reinterpret_cast<const bf16x8*>(p1 + 16 * dc);
        }
    }
    // DQ, ST: this row's log2 normaliser; DQ: delta = dout . out (also
    // published for the DK kernel), or (precise) ST's delta
    float Lrow = 0.f, drow = 0.f;
    if (ROWQ) {
        Lrow = a.lse[(int64_t)bh * T + rc] * kLog2e;
        if (MODE == kDQ && PREC) {
            drow = a.delta[(int64_t)bh * T + rc];
        } else if (MODE == kDQ) {
            const bf16* po = a.o + off + (int64_t)rc * D + 8 * hh;
            float d = 0.f;
#pragma unroll
            for (int dc = 0; dc < D / 16; ++dc) {
                const bf16x8 ov = *reinterpret_cast<const bf16x8*>(po + 16 * dc);
#pragma unroll
                for (int e = 0; e < 8; ++e) d = fmaf((float)f1[dc][e], (float)ov[e], d);
            }
            drow = swap_sum(d);
            if (hh == 0 && ri < T) a.delta[(int64_t)bh * T + ri] = drow;
        }
    }
    // land the register operands before any tile load is counted
    __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));

    // ---- tile ring: kind x of tile t in slot x * R + (t - t0) % R
    // DQ: 0 = K (read whole and transposed), 1 = V (rows whole)
    // DV: 0 = Q (rows whole), 1 = dout (transposed reads)
    // DK: 0 = Q (read whole and transposed), 1 = dout (rows whole)
    // ST: 0 = K, 1 = V (rows whole)
    constexpr int SW0 = MODE == kDV || MODE == kST ? kSwzK : kSwzB;   // swizzle of kind 0
    constexpr int SW1 = MODE == kDV ? kSwzV : kSwzK;   // swizzle of kind 1
    // Ring slot s of kind x (tile t lives in slot (t - t0) mod R); slot numbers
    // are compile-time constants at every call site (the key loop is unrolled
    // over the R = 4 slots), so LDS addresses carry them as immediates.
    static_assert(C::R == 4, "the loop is unrolled over 4 ring slots");
    auto slot = [&](int x, int s) { return ring + (x * C::R + s % C::R) * C::TILEB; };
    const bf16* src[2];
    src[0] = ROWQ ? K : Q;
    src[1] = ROWQ ? V : DO;
    uint32_t off0[C::NLD_W], off1[C::NLD_W];
    tile_offsets<D, C::NW, SW0>(off0, wave, lane, 2 * D);
    tile_offsets<D, C::NW, SW1>(off1, wave, lane, 2 * D);
    const int slab = T * D * 2;
    // DV, DK: lanes 0..7 of every wave copy the tile's 32 log2 normalisers
    // and (DK) lanes 8..15 its 32 deltas into the slot's stats (all waves
    // write the same bytes); past the sequence end the buffer range check
    // gives 0.
    const __amdgpu_buffer_rsrc_t lse_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.lse) + (int64_t)bh * T, 0, T * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t del_rs = __builtin_amdgcn_make_buffer_rsrc(
        a.delta + (int64_t)bh * T, 0, T * 4, 0x00020000);
    auto load = [&](int t, int s) {   // tile t into ring slot s
        const int tt = min(t, t1 - 1);
        const int boff = tt * C::TILEB;
#pragma unroll
        for (int x = 0; x < C::NTL; ++x)
            dma_tile(rows_rsrc(src[x], boff, slab), lds_addr(slot(x, s)), wave, x == 1 ? off1 : off0);
        if (!ROWQ) {
            const uint32_t sbase = lds_addr(&stats[s % C::R][0]);
            // lane l < 8 (l < 16) fetches items 4 (l % 8) .. + 3 of L (delta)
            const uint32_t soff = (tt * C::BN + 4 * (lane & 7)) * 4;
            if (lane < 8) lds_load16(lse_rs, sbase, soff);
            if (MODE == kDK && lane >= 8 && lane < 16) lds_load16(del_rs, sbase, soff);
        }
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
    // one column tile j, in ring slot KS = (j - t0) mod 4
    auto step = [&](auto ks, int j) {
        constexpr int KS = decltype(ks)::value;
        load(j + C::PF, KS + C::PF);   // into the slot of tile j - 1, released by the last barrier
        if (needs(j)) {
            const int k0 = j * C::BN;
            const char* A0 = slot(0, KS);
            const char* A1 = slot(1, KS);
            float Ls[16], Ds[16];
            if (!ROWQ) {
                const float* st = &stats[KS][0];
                read_stats(st, hh, Ls);
                if (MODE == kDK) read_stats(st + 32, hh, Ds);
            }
            // first products: scores and, for DQ / DK, dP
            f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int dc = 0; dc < D / 16; ++dc) {
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_row_frag<D, SW0>(A0, lr, hh, dc),
                                                            f0[dc], s, 0, 0, 0);
                if (MODE != kDV)
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        read_row_frag<D, kSwzK>(A1, lr, hh, dc), f1[dc], dp, 0, 0, 0);
            }
            // band mask: row item ri against column items k0 + 8 (v/4) + 4 hh + v%4
            if (!interior(j)) {
#pragma unroll
                for (int vv = 0; vv < 16; ++vv) {
                    const int col = k0 + 8 * (vv >> 2) + 4 * hh + (vv & 3);
                    const int qq = ROWQ ? ri : col, kk = ROWQ ? col : ri;
                    const bool ok = (unsigned)(qq - kk) < (unsigned)W && qq < T;
                    s[vv] = ok ? s[vv] : sfill;
                }
            }
            // P and (DQ, DK) dS; (ST) the row sums of P and P dP
#pragma unroll
            for (int vv = 0; vv < 16; ++vv) {
                const float L = ROWQ ? Lrow : Ls[vv] * kLog2e;
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[vv], c, -L));
                if (MODE == kST) {
                    zsum += p;
                    ysum = __builtin_fmaf(p, dp[vv], ysum);
                } else if (MODE == kDV) {
                    s[vv] = p;
                } else {
                    s[vv] = p * (dp[vv] - (ROWQ ? drow : Ds[vv]));
                }
            }
            if constexpr (MODE != kST) {
                // accumulate: (DQ) dQ^T += K^T dS^T, (DV) dV^T += dO^T P, (DK) dK^T += Q^T dS
                bf16x8 t0f[D / 32], t1f[D / 32];
                // transposed operand: kind 0 (k or q) for DQ, DK; kind 1 (dout) for DV
                const char* At = MODE == kDV ? A1 : A0;
                read_v_chunk<D, MODE == kDV ? kSwzV : kSwzB>(At, 0, lane, t0f);
                read_v_chunk<D, MODE == kDV ? kSwzV : kSwzB>(At, 1, lane, t1f);
                if constexpr (PREC && MODE != kDV) {
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
            a.lse_w[(int64_t)bh * T + ri] = (Lrow + __builtin_amdgcn_logf(z)) * kLn2;
            a.delta[(int64_t)bh * T + ri] = y / z;
        }
        return;
    }

    // store (lane holds d = 32 db + 8 g + 4 hh + 0..3 of row item ri)
    const float f = MODE == kDV ? 1.f : a.scale;
    if (ri < T) {
        bf16* row = a.grad + off + (int64_t)ri * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = (bf16)(acc[db][4 * g + e] * f);
                *reinterpret_cast<bf16x4*>(row + 32 * db + 8 * g + 4 * hh) = w;
            }
    }
}

template <int D, int MODE, bool PREC>
hipError_t launch_mode(BArgs a, int64_t B, int64_t H, hipStream_t st) {
    using C = BCfg<D, MODE>;
    a.nrt = (a.T + C::BM - 1) / C::BM;
    const int64_t nblocks = B * H * a.nrt;
    a.nblocks = (int)nblocks;
    a.remap = nblocks % 8 == 0 ? 1 : 0;
    // row tiles within W - 1 of the sequence's far end (DQ: its start; DV, DK:
    // its end) have shorter bands
    a.nfull = xcd_longest_first_nfull(nblocks, a.nrt, (a.W - 1 + C::BM - 1) / C::BM);
    void* args[] = {(void*)&a};
    return hipLaunchKernel((const void*)bwd_bf16_kernel<D, MODE, PREC>, dim3((unsigned)nblocks),
                           dim3(256), args, 0, st);
}

// lse_ws: workspace row normalisers (precise: written by ST from a.lse)
template <int D, bool PREC>
hipError_t launch_all(BArgs a, float* lse_ws, bf16* dq, bf16* dk, bf16* dv, int64_t B, int64_t H,
                      hipStream_t st) {
    hipError_t e;
    if constexpr (PREC) {
        a.lse_w = lse_ws;
        e = launch_mode<D, kST, true>(a, B, H, st);
        if (e != hipSuccess) return e;
        a.lse = lse_ws;
    }
    a.grad = dq;
    e = launch_mode<D, kDQ, PREC>(a, B, H, st);
    if (e != hipSuccess) return e;
    a.grad = dv;
    e = launch_mode<D, kDV, false>(a, B, H, st);
    if (e != hipSuccess) return e;
    a.grad = dk;
    return launch_mode<D, kDK, PREC>(a, B, H, st);
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
