// Causal sliding-window attention prefill, bf16 in / bf16 out, fp32
// accumulation, on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Band-only iteration.  A workgroup owns BM = 32 * NW consecutive queries
// [i0, i0 + BM) of one (batch, head) and walks only the 32-key tiles that
// intersect their band [max(0, i0 - W + 1), min(T, i0 + BM)), so the work is
// O(T * min(W, T) * D) rather than the dense O(T^2 * D) of the masked recipe
// ("NNX Sliding-Window Attention", A local mask is not a sparse
// implementation).  Each wavefront owns 32 queries and skips the key tiles
// that miss its own band.  The band predicate j <= i and i - j < W
// ("27. Sliding-Window Attention", step 2) is applied, as a select to -inf,
// only on tiles that straddle an edge of the wavefront's band.
//
// Per wavefront and key tile (fp32 everywhere except the MFMA operands):
//   S^T = K Q^T      32x32 blocks: lane l holds query l % 32 and 16 of its
//                    keys, so row max / sum are in-lane plus one exchange with
//                    lane l ^ 32 (v_permlane32_swap).
//   softmax          running reference max m and sum l per query; exp2 with
//                    the scale 1/sqrt(D) * log2(e) folded into one FMA.  The
//                    reference is raised, and O rescaled by exp2(m_old -
//                    m_new), only when a row max grows by more than 2^8; the
//                    prefill's fast pass takes row maxima only on edge tiles
//                    and the first interior tile where a row's window starts
//                    on it, and redoes just the rows that overflow (see the
//                    kernel).
//   O^T += V^T P^T   P^T goes from the S^T accumulator straight into the B
//                    operand (bf16, round to nearest even); the row sum is
//                    taken over those same bf16 weights (v_dot2 with ones).
//                    V stays row-major in LDS; the key-contiguous A operand
//                    comes from transposing LDS reads (ds_read_b64_tr_b16).
//
// Data movement: K and V tiles go HBM -> LDS directly (buffer loads with an
// LDS destination; the hardware range check returns zeros past the sequence
// end) through rings of PF + 1 slots, issued PF tiles ahead, with K one tile
// ahead of V.  Iteration j issues S(j+1) = K(j+1) Q^T on the matrix cores
// while the vector ALUs run the softmax of tile j, then O += V(j)^T P(j)^T.
// The K operands of S(j+1) were read from LDS during iteration j-1, so an
// iteration starts its matrix work right after the barrier.  The LDS layouts
// are XOR swizzled on 16-byte chunks so every LDS read is bank-conflict free;
// the loop is unrolled over the ring's 4 slots, so slot addresses are
// immediate offsets.

#include "swa_mfma.h"

#include <type_traits>

namespace swa {
namespace {

template <int D, int NW>
struct Cfg {
    static constexpr int BM = 32 * NW;          // queries per workgroup
    static constexpr int BN = 32;               // keys per tile
    static constexpr int NT = 64 * NW;          // threads
    static constexpr int ROWB = D * 2;          // bytes per K / V row
    static constexpr int TILEB = BN * ROWB;     // bytes per K or V tile
    static constexpr int PF = 3;                // prefetch distance in tiles
    static constexpr int R = PF + 1;            // LDS ring slots per matrix
    static constexpr int LDS_BYTES = 2 * R * TILEB;
    static constexpr int NLD_W = TILEB / 1024 / NW;   // 1-KiB LDS loads per wave per tile
    // vmcnt that leaves only the two most recent tile loads (those of the
    // current step) in flight (see the issue order in the kernel)
    static constexpr int VM_WAIT = (2 * PF - 4) * NLD_W;
    static_assert(R == 4, "the key loop is unrolled over the 4 ring slots");
    static_assert(VM_WAIT < 64, "vmcnt range");
    static_assert(D == 64 || D == 128, "head size");
    static_assert((TILEB / 1024) % NW == 0, "tile loads split evenly over waves");
};

struct Args {
    const bf16* q;
    const bf16* k;
    const bf16* v;
    bf16* out;
    Layout L;       // element strides (D axis contiguous)
    int H;
    int T;
    int W;          // min(W, T)
    int nqt;        // query tiles per (b, h)
    int nblocks;    // grid size
    int remap;      // 1: spread consecutive logical tiles over one XCD
    int nfull;      // longest-first dispatch (xcd_logical_tile); -1: plain order
    float c;        // log2(e) * |scale| (scale defaults to 1 / sqrt(D))
    int qneg;       // 1: scale < 0, applied as -q (exact) times |scale|
    // chunk continuation only: q, k, v, out are the chunk [S, H, C, D]
    // (contiguous), the W-slot rings hold the earlier tokens, pos0[s] is the
    // chunk's first position
    const bf16* kring;
    const bf16* vring;
    const int64_t* pos0;
    int C;
    // chunk continuation split over the key range (nsplit > 1): partial
    // unnormalised outputs, maxima (log2 units) and sums per (row, split)
    int nsplit;
    float* ws_o;          // [S * H * C * nsplit, D]
    float* ws_ml;         // [S * H * C * nsplit, 2]
    // prefill only, optional: each row's log-sum-exp of its scaled scores,
    // ln(sum_j exp(s_ij * scale)), at lse[bh * T + i] (for the backward)
    float* lse;
};

// S^T for a 32-key tile: s holds keys 8 (v/4) + 4 hh + v%4 of query lr
// (v = register index).
template <int D>
__device__ inline void qk_tile(const char* Kt, const bf16x8 (&qf)[D / 16], int lr, int hh,
                               int ksw, f32x16& s) {
    const char* r0 = Kt + lr * (2 * D);
    s = f32x16{};
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
        const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(r0 + (((2 * dc + hh) ^ ksw) << 4));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[dc], s, 0, 0, 0);
    }
}

// Lazy rescale threshold in log2 units: where the max is taken, probabilities
// stay below 2^8 and the output accumulator is rarely rescaled.  O / l is the
// same quotient for any reference.
constexpr float kRescaleLog2 = 8.0f;

// CHUNK = false: prefill of [B, H, T, D].  CHUNK = true: the chunk
// continuation of a ring ("27. Sliding-Window Attention", Problem, the
// rolling buffer; "25. Sliding-Window Causal Attention for Streaming
// Inference", Problem).  Stream b's chunk holds positions p0 .. p0 + C - 1;
// keys before p0 live in ring slot (position mod W).  Positions are taken
// relative to an origin (a multiple of 32 at least W + 32 below p0), so the
// kernel sees a sequence of length p0r + C whose queries are its last C rows
// and whose key tiles come from the ring below p0r and from the chunk above.
template <int D, int NW, bool CHUNK>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_bf16_kernel(Args a) {
    using C = Cfg<D, NW>;
    // Tile t lives in slot (t - t0) % R of the K ring and of the V ring.
    __shared__ __attribute__((aligned(1024))) char ring[2 * C::R * C::TILEB];
    __shared__ int rerun;            // set when the fast pass must be redone
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS load bases go to M0
    const int lane = tid & 63;
    const int lr = lane & 31, hh = lane >> 5;

    // Logical tile bh * nqt + r is rank r of head bh; rank 0 is the last
    // query tile, and ranks past the full-band ones (the query tiles near the
    // sequence start) have ever shorter bands.  xcd_logical_tile spreads the
    // logical tiles over the XCDs, longest first where that pays.
    const int bid = blockIdx.x;
    int logical = xcd_logical_tile(bid, a.nblocks, a.remap, CHUNK ? a.nqt * a.nsplit : a.nqt,
                                   CHUNK ? -1 : a.nfull);
    int sp = 0;                                      // key-range split (chunk continuation)
    if constexpr (CHUNK) {
        sp = logical % a.nsplit;
        logical /= a.nsplit;
    }
    const int bh = logical / a.nqt;
    const int qt = a.nqt - 1 - (logical - bh * a.nqt);
    const int W = a.W;
    const int b = bh / a.H, h = bh - b * a.H;
    int T = a.T;                    // sequence length (relative positions)
    int p0r = 0;                    // first query position (relative)
    int omod = 0;                   // origin mod W (ring slot of relative position 0)
    if constexpr (CHUNK) {
        int64_t p0 = a.pos0[b];
        p0 = p0 < 0 ? 0 : p0;
        const int64_t origin = p0 >= (int64_t)W + 32 ? ((p0 - W - 32) & ~(int64_t)31) : 0;
        p0r = (int)(p0 - origin);
        omod = (int)(origin % W);
        T = p0r + a.C;
    }
    const int nrow = CHUNK ? a.C : T;   // rows of q and out
    const int i0 = p0r + qt * C::BM;
    const bf16* __restrict__ Qbh = a.q + b * a.L.q.b + h * a.L.q.h;
    const bf16* __restrict__ Kbh = a.k + b * a.L.k.b + h * a.L.k.h;
    const bf16* __restrict__ Vbh = a.v + b * a.L.v.b + h * a.L.v.h;
    const int qrs = (int)a.L.q.t, krs = (int)a.L.k.t, vrs = (int)a.L.v.t;

    const int qw0 = i0 + 32 * wave;                  // this wave's first query
    const int qi = qw0 + lr;                         // this lane's query
    const int klo = max(i0 - W + 1, 0);
    const int khi = min(i0 + C::BM, T);
    int t0 = klo / C::BN;                            // workgroup's key tiles [t0, t1)
    int t1 = (khi + C::BN - 1) / C::BN;
    if constexpr (CHUNK) {
        // split sp of nsplit takes its share of the band's tiles
        const int per = (t1 - t0 + a.nsplit - 1) / a.nsplit;
        const int s0 = t0 + sp * per;
        t1 = min(t1, s0 + per);
        t0 = s0;
    }
    int wt0 = t1, wt1 = t1;                          // this wave's key tiles [wt0, wt1)
    if (qw0 < T) {
        wt0 = max(qw0 - W + 1, 0) / C::BN;
        wt1 = (min(qw0 + 32, T) + C::BN - 1) / C::BN;
    }
    // Tile tests as one unsigned range compare each (uniform, scalar ALU).
    auto needs = [&](int t) { return (unsigned)(t - wt0) < (unsigned)(wt1 - wt0); };
    // Interior tiles [ia, ia + ilen): every key at or below the wave's first
    // query and inside its last query's window, so no key is masked.
    const int xa = qw0 + 32 - W;                     // first key in every row's window
    const int ia = xa <= 0 ? 0 : (xa + C::BN - 1) / C::BN;
    const int ib = qw0 >= C::BN - 1 ? (qw0 - (C::BN - 1)) / C::BN + 1 : 0;
    const int ilen = max(ib - ia, 0);
    auto interior = [&](int t) { return (unsigned)(t - ia) < (unsigned)ilen; };
    // Fast-pass tiles [fa, fa + flen): interior tiles that every row of the
    // wave reaches with a key already seen in an earlier tile, i.e. all
    // interior tiles but the first when the last row's window starts on it
    // (xa a multiple of the tile, or xa <= 0).  Fixed by positions alone,
    // so which tiles take the row max never depends on data.
    const int fa = ia + ((xa <= 0 || xa % C::BN == 0) ? 1 : 0);
    const int flen = max(ib - fa, 0);
    // a split's partial row: unnormalised output o, max m (raw units) and
    // this lane's half of the sum; the merge rescales partials to a common max
    auto write_partial = [&](const f32x16 (&o)[D / 32], float m, float lsum) {
        const int crow = qi - p0r;
        if (crow >= a.C) return;
        const int64_t idx = ((int64_t)bh * a.C + crow) * a.nsplit + sp;
        float* po = a.ws_o + idx * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<f32x4*>(po + 32 * db + 8 * g + 4 * hh) =
                    f32x4{o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
        const float l = swap_sum(lsum);
        if (hh == 0) {
            a.ws_ml[2 * idx] = m * a.c;                  // -inf for a row with no key here
            a.ws_ml[2 * idx + 1] = l;
        }
    };
    if constexpr (CHUNK) {
        if (t0 >= t1) {                              // an empty split
            f32x16 z[D / 32];
#pragma unroll
            for (int db = 0; db < D / 32; ++db) z[db] = f32x16{};
            write_partial(z, -__builtin_inff(), 0.f);
            return;
        }
    }

    // Q^T operand: q[qi][16 dc + 8 hh .. + 7] (rows past T read row T - 1;
    // their outputs are never stored).
    bf16x8 qf[D / 16];
    {
        const bf16* qp = Qbh + (int64_t)min(qi - p0r, nrow - 1) * qrs + 8 * hh;
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) qf[dc] = *reinterpret_cast<const bf16x8*>(qp + 16 * dc);
    }
    // Q is not waited for here: the prologue's tile loads are issued behind
    // it and one wait covers both, so they share one memory round trip.  A
    // negative scale flips q after that wait.
    bool negate_q = a.qneg != 0;
    const int ksw = kswz<D>(lr);

    f32x16 o[D / 32];
    float m;                          // reference max (raw score units)
    float lsum;                       // this lane's half of the row sum
    float mref;                       // m * c, 0 while m = -inf
    // Fast pass (prefill, careful = false): the reference m only has to keep
    // the exponents in range, so the fast-pass tiles [fa, fa + flen) skip the
    // row max.  A row whose scores there exceed its reference by more than
    // the fp32 exponent range gets a non-finite probability, row sum or
    // output; such rows (and only they) are redone with the max taken on
    // every tile (careful pass) and stored from it, while every other row
    // keeps its fast-pass result.  Each row's result therefore depends on
    // its own window only, bit for bit.  The chunk continuation always runs
    // careful.
    bool careful = CHUNK;
    bool redo = true;                 // careful pass: this row is stored from it
    // Tiles that skip the row max: [fa, fa + flen) in the fast pass, none in
    // the careful pass.
    int f_lo, f_len;
    // Cleared before the prologue's tile loads (asm with memory clobbers
    // keep the store ahead of them) and so before its first barrier.
    if (tid == 0) rerun = 0;
    const float c = a.c;
    const float tau = kRescaleLog2 / c;

    // ---- prologue.  Tile loads are issued in the order K(t0) V(t0) K(t0+1)
    // V(t0+1) ... K(t0+PF-1) V(t0+PF-1) K(t0+PF), and then, in step j,
    // V(j+PF) K(j+1+PF).  Tiles past the band are issued too (into a free
    // slot, never read: zeros in the prefill, the band's last tile again in
    // the chunk continuation), so every step issues the same number of
    // loads and a fixed vmcnt waits for exactly the oldest.
    // Ring slot s of K and of V (tile t lives in slot (t - t0) mod R).  Slot
    // numbers are compile-time constants at every call site, so the LDS
    // reads carry the slot in their immediate offset.
    auto kslot_n = [&](int s) { return ring + (s % C::R) * C::TILEB; };
    auto vslot_n = [&](int s) { return ring + (C::R + s % C::R) * C::TILEB; };
    uint32_t koff[C::NLD_W], voff[C::NLD_W];
    tile_offsets<D, NW, kSwzK>(koff, wave, lane, 2 * krs);
    tile_offsets<D, NW, kSwzV>(voff, wave, lane, 2 * vrs);
    // bytes per key tile and per slab (the last row ends after D elements)
    // (capped: a tile step at or past the slab end only has to empty it)
    const int ktb = (int)min((int64_t)C::BN * 2 * krs, (int64_t)INT32_MAX);
    const int vtb = (int)min((int64_t)C::BN * 2 * vrs, (int64_t)INT32_MAX);
    const int kslab = ((nrow - 1) * krs + D) * 2, vslab = ((nrow - 1) * vrs + D) * 2;
    // Chunk continuation: the ring slot of relative position x (x < 3 W
    // whenever W >= 64, which the two subtractions cover).
    auto ring_slot = [&](int x) {
        if (W < 64) return x % W;
        x -= x >= W ? W : 0;
        x -= x >= W ? W : 0;
        return x;
    };
    const int rslab = W * D * 2;
    const bf16* Krh = nullptr;
    const bf16* Vrh = nullptr;
    if constexpr (CHUNK) {
        Krh = a.kring + (int64_t)bh * W * D;
        Vrh = a.vring + (int64_t)bh * W * D;
    }
    // A tile of the chunk continuation: all chunk rows (zero-filled past
    // the chunk), all ring rows in consecutive slots, or (the tile holding
    // position p0r, or the one where the ring wraps) one source address per
    // lane, with rows past the chunk clamped to its last row: those keys lie
    // above every query's diagonal and get weight 0.
    auto load_chunk_tile = [&](int t, const bf16* Cbh, const bf16* Rbh, int tb, int cslab,
                               const uint32_t (&off)[C::NLD_W], uint32_t lds, bool isv) {
        const int k0 = min(t, t1 - 1) * C::BN;
        if (k0 >= p0r) {
            dma_tile(rows_rsrc(Cbh, (k0 - p0r) * (tb / C::BN), cslab), lds, wave, off);
            return;
        }
        const int s0 = ring_slot(k0 + omod);
        if (k0 + C::BN <= p0r && s0 + C::BN <= W) {
            dma_tile(rows_rsrc(Rbh, s0 * 2 * D, rslab), lds, wave, off);
            return;
        }
#pragma unroll
        for (int i = 0; i < C::NLD_W; ++i) {
            const int pb = (wave * C::NLD_W + i) * 1024 + lane * 16;
            const int row = pb / C::ROWB;
            const int phys = (pb % C::ROWB) >> 4;
            const int logical = phys ^ (isv ? vswz<D>(row) : kswz<D>(row));
            const int pos = k0 + row;
            const bf16* src = pos < p0r ? Rbh + (int64_t)ring_slot(pos + omod) * D
                                        : Cbh + (int64_t)min(pos - p0r, a.C - 1) * D;
            lds_load16_global(lds + (wave * C::NLD_W + i) * 1024, src + logical * 8);
        }
    };
    // Chunk continuation: the tiles of a stream (K or V) are loaded in order,
    // and away from the tile holding p0r and a ring wrap they are whole rows
    // at consecutive addresses (a run of ring slots, then the chunk).  A
    // cursor holds the next tile's address while tiles stay regular, and ev,
    // the first tile from which the general per-tile logic takes over again.
    struct Cursor {
        const char* p;      // next tile's first row
        int left;           // bytes from p to the end of its slab (0 past it)
        int ev;             // first tile index that needs the general path
    };
    // cursor for tile t as the first of a regular run, or ev = t if tile t
    // itself needs the general path
    auto cursor_at = [&](int t, const bf16* Cbh, const bf16* Rbh, int tb, int cslab, Cursor& cu) {
        const int k0 = t * C::BN;
        if (k0 >= p0r) {
            const int off = (k0 - p0r) * (tb / C::BN);
            cu.p = reinterpret_cast<const char*>(Cbh) + off;
            cu.left = max(cslab - off, 0);
            cu.ev = INT32_MAX;
            return;
        }
        const int s0 = ring_slot(k0 + omod);
        if (k0 + C::BN <= p0r && s0 + C::BN <= W) {
            cu.p = reinterpret_cast<const char*>(Rbh) + s0 * 2 * D;
            cu.left = rslab - s0 * 2 * D;
            // regular ring tiles run until the slots reach W or the tile
            // holding p0r
            cu.ev = min(t + (W - s0) / C::BN, p0r / C::BN);
            return;
        }
        cu.ev = t;
    };
    auto load_cursor = [&](int t, const bf16* Cbh, const bf16* Rbh, int tb, int cslab,
                           const uint32_t (&off)[C::NLD_W], uint32_t lds, bool isv, Cursor& cu) {
        if (t < cu.ev) {
            dma_tile(__builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(cu.p), 0, cu.left,
                                                       0x00020000),
                     lds, wave, off);
            cu.p += tb;
            cu.left = max(cu.left - tb, 0);
        } else {
            load_chunk_tile(t, Cbh, Rbh, tb, cslab, off, lds, isv);
            cursor_at(t + 1, Cbh, Rbh, tb, cslab, cu);
        }
    };
    Cursor kcur = {}, vcur = {};
    // Prefill: the next K and V tiles to load, as an address and the bytes
    // left from there to the end of the band's last tile (0 past it: such
    // loads read nothing and write zeros).  Tiles are loaded in order, so
    // each load just advances these by one tile.
    const char* kp = nullptr;
    const char* vp = nullptr;
    int kr = 0, vr = 0;
    // tile t into ring slot s (s = t - t0 modulo the ring)
    auto load_k = [&](int t, int s) {
        if constexpr (CHUNK) {
            load_cursor(t, Kbh, Krh, ktb, kslab, koff, lds_addr(kslot_n(s)), false, kcur);
        } else {
            dma_tile(rows_rsrc(reinterpret_cast<const bf16*>(kp), 0, kr), lds_addr(kslot_n(s)),
                     wave, koff);
            kp += ktb;
            kr = max(kr - ktb, 0);
        }
    };
    auto load_v = [&](int t, int s) {
        if constexpr (CHUNK) {
            load_cursor(t, Vbh, Vrh, vtb, vslab, voff, lds_addr(vslot_n(s)), true, vcur);
        } else {
            dma_tile(rows_rsrc(reinterpret_cast<const bf16*>(vp), 0, vr), lds_addr(vslot_n(s)),
                     wave, voff);
            vp += vtb;
            vr = max(vr - vtb, 0);
        }
    };
    // Publish loads: wait until at most VM_WAIT of this wave's loads are in
    // flight and its LDS reads are done, then barrier.  No fence is needed:
    // the only LDS writes are the tile loads, covered by the count.
    auto publish = [&]() {
        __builtin_amdgcn_s_waitcnt((C::VM_WAIT & 15) | ((C::VM_WAIT >> 4) << 14) | (7 << 4) | (0 << 8));
        __builtin_amdgcn_s_barrier();
    };
    // Row max of a score tile (in-lane over 16 keys, then across the lane
    // pair l, l ^ 32 that shares the query).
    auto tile_max = [&](const f32x16& s) {
        float mx = fmaxf(s[0], s[1]);
#pragma unroll
        for (int v = 2; v < 16; v += 2) mx = fmaxf(fmaxf(mx, s[v]), s[v + 1]);
        return swap_max(mx);
    };
    // Scores of a tile outside this wave's band: all -inf, so its
    // probabilities are exact zeros whatever its keys hold (a finite key can
    // still overflow the fp32 dot product).  The empty asm keeps this a
    // branch taken on those few tiles rather than selects on every tile.
    auto kill_tile = [&](f32x16& s) {
        asm volatile("");
#pragma unroll
        for (int v = 0; v < 16; ++v) s[v] = -__builtin_inff();
    };
    // Reference update for a freshly computed (and masked) score tile whose
    // row max is mx: raise m if mx exceeds it by more than 2^8 and rescale
    // what has been accumulated so far.  Runs between tiles, outside the
    // MFMA/VALU overlap regions.
    auto raise_ref = [&](float mx) {
        const bool raise = mx > m + tau;               // false while the row is fully masked
        if (__any(raise)) {
            // 1 for rows keeping their reference (also rows still fully
            // masked, where m - m would be NaN); 0 when m = -inf.
            const float alpha = __builtin_amdgcn_exp2f(raise ? (m - mx) * c : 0.f);
            // A row whose reference was -inf has accumulated nothing (every
            // score so far was -inf), so only rows raising a finite
            // reference need the rescale; a wavefront's first keys skip it.
            const bool rescale = __any(raise && m != -__builtin_inff());
            m = raise ? mx : m;
            mref = m == -__builtin_inff() ? 0.f : m * c;
            if (rescale) {
                lsum *= alpha;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
            }
        }
    };

  for (;;) {   // fast pass, then (rarely) the careful pass
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    m = -__builtin_inff();
    mref = 0.f;
    lsum = 0.f;
    f_lo = careful ? 0 : fa;
    f_len = careful ? 0 : flen;
    if constexpr (CHUNK) {
        cursor_at(t0, Kbh, Krh, ktb, kslab, kcur);
        cursor_at(t0, Vbh, Vrh, vtb, vslab, vcur);
    } else {
        // t0 * 32 < T, so the first tile starts inside both slabs.  The
        // range ends with the band: tiles past it are zeros, not reads.
        kp = reinterpret_cast<const char*>(Kbh) + (int64_t)t0 * ktb;
        vp = reinterpret_cast<const char*>(Vbh) + (int64_t)t0 * vtb;
        kr = (int)(min((int64_t)kslab, (int64_t)t1 * ktb) - (int64_t)t0 * ktb);
        vr = (int)(min((int64_t)vslab, (int64_t)t1 * vtb) - (int64_t)t0 * vtb);
    }
#pragma unroll
    for (int i = 0; i < C::PF; ++i) {
        load_k(t0 + i, i);
        load_v(t0 + i, i);
    }
    load_k(t0 + C::PF, C::PF);
    // Every load so far has landed (Q and all of the prologue's tiles): a
    // full wait, which also tells the compiler that Q is in registers on
    // every path, so it adds no waits of its own inside the key loop.
    __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (0 << 8));
    __builtin_amdgcn_s_barrier();
    if (negate_q) {
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) qf[dc] = -qf[dc];
        negate_q = false;
    }

    f32x16 sA, sB;
    if (needs(t0)) {
        qk_tile<D>(kslot_n(0), qf, lr, hh, ksw, sA);
        if (!interior(t0)) mask_tile(sA, qi, t0 * C::BN, hh, W);
        raise_ref(tile_max(sA));
    } else {
        kill_tile(sA);
    }
    // K operands of the next score tile live in registers one step ahead:
    // step j computes S(j+1) from kf of K(j+1) and reads K(j+2) into the
    // other set, so no step waits on LDS before its first MFMA.
    bf16x8 kfA[D / 16], kfB[D / 16];
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) kfA[dc] = read_row_frag<D>(kslot_n(1), lr, hh, dc);
    __builtin_amdgcn_s_waitcnt((7 << 4) | (0 << 8) | 15 | (3 << 14));   // LDS reads done
    __builtin_amdgcn_s_barrier();   // every wave is done with K(t0) before its slot is reloaded

    // ---- one key tile j: S(j+1) on the matrix cores alongside softmax(j).
    // KS = (j - t0) mod 4 is a compile-time constant, so every ring slot
    // address below is one.
    auto body = [&](auto ks, f32x16& sc, f32x16& sn, bf16x8 (&kc)[D / 16],
                    bf16x8 (&kn)[D / 16], int j) {
        constexpr int KS = decltype(ks)::value;
        // Slots released by the barrier that ended the previous step:
        // V(j+PF) replaces V(j-1), K(j+1+PF) replaces K(j) (whose operands
        // were read two steps ago).
        load_v(j + C::PF, KS + C::PF);
        load_k(j + 1 + C::PF, KS + 1 + C::PF);
        const bool nj = needs(j), nn = needs(j + 1);
        const char* Vc = vslot_n(KS);
        float mxn = 0.f;   // chunk continuation: the row max of S(j+1)

        // Every wave runs every tile of the workgroup, so the accumulator
        // path has no branches; a tile outside this wave's band arrives with
        // scores -inf (kill_tile) and so gets probabilities exp2(-inf) = 0.
        {
            const float mc = mref;
            // The schedule is written out slice by slice; each sched_barrier
            // closes a slice, so the MFMAs at the top of a slice run on the
            // matrix core while the slice's (independent) vector ALU work
            // issues behind them.
            constexpr int ND = D / 16;
            constexpr int NEA = 12;                 // exps issued in region A
            constexpr int NPRE = 2;                 // of which before the first MFMA
            bf16x8 p0, p1;
            // The V(j) operands of chunk 0 are read up front, so their
            // latency hides behind region A.
            bf16x8 va0[D / 32], va1[D / 32];
            read_v_chunk<D>(Vc, 0, lane, va0);
            // The first probabilities need no LDS data: they cover the
            // latency of the first operand reads.
#pragma unroll
            for (int v = 0; v < NPRE; ++v) sc[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[v], c, -mc));
            __builtin_amdgcn_sched_barrier(0);
            // Region A: S(j+1) = K(j+1) Q^T, one MFMA per 16-wide d slice, with
            // the probabilities of keys NPRE..NEA-1 of tile j and the operand
            // p0 of keys 0..15.  S(j+1) is computed even where this wave does
            // not need it (at the end from a stale buffer); kill_tile then
            // replaces its scores.
            sn = f32x16{};
#pragma unroll
            for (int dc = 0; dc < ND; ++dc) {
                sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc[dc], qf[dc], sn, 0, 0, 0);
#pragma unroll
                for (int v = NPRE + dc * (NEA - NPRE) / ND; v < NPRE + (dc + 1) * (NEA - NPRE) / ND; ++v)
                    sc[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[v], c, -mc));
                if (dc == ND - 1) {
                    p0 = pack_p(sc, 0, lsum);
                    read_v_chunk<D>(Vc, 1, lane, va1);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // Region B: O += V(j) P(j), two 16-key chunks of D/32 MFMAs, with
            // the rest of the probabilities produced alongside chunk 0 and the
            // row max of S(j+1) alongside chunk 1.
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va0[db], p0, o[db], 0, 0, 0);
            // K(j+2), published by the barrier that ended the previous step
#pragma unroll
            for (int dc = 0; dc < ND; ++dc) kn[dc] = read_row_frag<D>(kslot_n(KS + 2), lr, hh, dc);
#pragma unroll
            for (int v = NEA; v < 16; ++v) sc[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[v], c, -mc));
            p1 = pack_p(sc, 8, lsum);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va1[db], p1, o[db], 0, 0, 0);
            if constexpr (CHUNK) mxn = tile_max(sn);
            __builtin_amdgcn_sched_barrier(0);
        }
        // Edge tiles are masked; the max of every tile outside the fast-pass
        // range (all tiles in the careful pass) updates m.
        if (!nn) {
            kill_tile(sn);
        } else if constexpr (CHUNK) {
            {
                if (!interior(j + 1)) {
                    mask_tile(sn, qi, (j + 1) * C::BN, hh, W);
                    mxn = tile_max(sn);
                }
                raise_ref(mxn);
            }
        } else if ((unsigned)(j + 1 - f_lo) >= (unsigned)f_len) {
            if (!interior(j + 1)) mask_tile(sn, qi, (j + 1) * C::BN, hh, W);
            raise_ref(tile_max(sn));
        }
        publish();   // V(j+2) and K(j+3) have landed
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    for (int j = t0;;) {
        body(I0{}, sA, sB, kfA, kfB, j);
        if (++j >= t1) break;
        body(I1{}, sB, sA, kfB, kfA, j);
        if (++j >= t1) break;
        body(I2{}, sA, sB, kfA, kfB, j);
        if (++j >= t1) break;
        body(I3{}, sB, sA, kfB, kfA, j);
        if (++j >= t1) break;
    }

    __builtin_amdgcn_s_waitcnt(0);   // every tile load has landed
    if constexpr (CHUNK) {
        if (a.nsplit > 1) {
            write_partial(o, m, lsum);
            return;
        }
    }
    // Fast pass: a row is redone when its row sum or any output of either
    // lane that holds it is inf or NaN.  Any such value shows in this lane's
    // sum: its exponent field is all ones.  The empty asm hides the bits'
    // origin, so the test is not folded into a float compare, which this
    // file's no-NaN float model would reduce to an infinity test.
    bool row_bad = false;
    if (!careful) {
        float chk = lsum;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) chk += o[db][v];
        uint32_t bits = __float_as_uint(chk);
        asm volatile("" : "+v"(bits));
        const uint32_t bad = (bits & 0x7f800000u) == 0x7f800000u ? 1u : 0u;
        const auto pr = __builtin_amdgcn_permlane32_swap(bad, bad, false, false);
        row_bad = (pr[0] | pr[1]) != 0u && qi < T;
    }

    // ---- finalise the rows this pass owns: the fast pass stores its good
    // rows, the careful pass the rows the fast pass could not finish.  O / l,
    // bf16, store (lane holds d = 32 db + 8 g + 4 hh + 0..3).
    if (careful ? redo : !row_bad) {
        const float l = swap_sum(lsum);
        const float inv = 1.f / l;
        if (!CHUNK && a.lse != nullptr && qi < T && hh == 0)
            a.lse[(int64_t)bh * T + qi] = (m * c + __builtin_amdgcn_logf(l)) * kLn2;
        if (qi < T) {
            bf16* orow = a.out + b * a.L.o.b + h * a.L.o.h + (int64_t)(qi - p0r) * a.L.o.t;
            // All packs first, each in registers of its own, then the
            // stores: a store's data registers are not rewritten while it is
            // queued.
            bf16x4 w[D / 32][4];
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[db][g][e] = (bf16)(o[db][4 * g + e] * inv);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * g + 4 * hh) = w[db][g];
        }
    }
    if (careful) break;
    if (__any(row_bad) && lane == 0) rerun = 1;
    __syncthreads();
    if (rerun == 0) break;
    redo = row_bad;
    careful = true;
  }
}

template <int D, int NW, bool CHUNK>
hipError_t launch(Args a, int64_t B, int64_t H, int64_t rows, hipStream_t stream) {
    using C = Cfg<D, NW>;
    a.H = (int)H;
    a.nqt = (int)((rows + C::BM - 1) / C::BM);
    const int64_t nblocks = B * H * a.nqt * (CHUNK ? a.nsplit : 1);
    a.nblocks = (int)nblocks;
    a.remap = (nblocks % 8 == 0) ? 1 : 0;
    // the query tiles that start before row W - 1 (W = min(W, T) here) have
    // shorter bands (measured: longest first 4.4% faster at 4 heads per XCD,
    // 1.5% slower at 32)
    a.nfull = CHUNK ? -1 : xcd_longest_first_nfull(nblocks, a.nqt, (a.W - 1 + C::BM - 1) / C::BM);
    void* args[] = {(void*)&a};
    return hipLaunchKernel((const void*)prefill_bf16_kernel<D, NW, CHUNK>,
                           dim3((unsigned)nblocks), dim3(C::NT), args, 0, stream);
}

Args make_args(const bf16* q, const bf16* k, const bf16* v, bf16* out, const Layout& L,
               float scale) {
    Args a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.L = L;
    a.c = kLog2e * fabsf(scale);
    a.qneg = scale < 0.f ? 1 : 0;
    return a;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

bool strides_ok(const Strides& s) {
    return s.b >= 0 && s.h >= 0 && s.t >= 0 && s.b % 8 == 0 && s.h % 8 == 0 && s.t % 8 == 0 &&
           s.t < ((int64_t)1 << 30);
}

}  // namespace

bool prefill_bf16_supports(const void* q, const void* k, const void* v, const void* out,
                           int64_t T, int64_t D, const Layout& L) {
    if (D != 64 && D != 128) return false;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return false;
    if (!strides_ok(L.q) || !strides_ok(L.k) || !strides_ok(L.v) || !strides_ok(L.o)) return false;
    // rows past T must fall outside the buffer range of a k / v slab, and the
    // slab must be addressable with 32-bit byte offsets
    for (const Strides* s : {&L.k, &L.v}) {
        if (s->t < D) return false;
        if (((T - 1) * s->t + D) * 2 >= ((int64_t)1 << 31)) return false;
    }
    return T < ((int64_t)1 << 31);
}

hipError_t launch_prefill_bf16(const bf16* q, const bf16* k, const bf16* v, bf16* out,
                               int64_t B, int64_t H, int64_t T, int D, int64_t W,
                               const Layout& L, float scale, hipStream_t stream, float* lse) {
    Args a = make_args(q, k, v, out, L, scale);
    a.lse = lse;
    a.T = (int)T;
    a.W = (int)(W < T ? W : T);
    if (D == 128) return launch<128, 4, false>(a, B, H, T, stream);
    return launch<64, 4, false>(a, B, H, T, stream);
}

bool chunk_bf16_supports(const void* q, const void* kc, const void* vc, const void* kring,
                         const void* vring, const void* out, int64_t C, int64_t D, int64_t W) {
    if (D != 64 && D != 128) return false;
    for (const void* p : {q, kc, vc, kring, vring, out})
        if (!aligned16(p)) return false;
    // 32-bit byte offsets inside one chunk slab and one ring slab, and
    // relative positions (below W + 64 + C) in int
    return C * D * 2 < ((int64_t)1 << 31) && W * D * 2 < ((int64_t)1 << 31) &&
           W + C + 64 < ((int64_t)1 << 30);
}

int chunk_splits(int64_t S, int64_t H, int64_t C, int64_t W) {
    // Splitting the key range pays while S * H * (C / 128) workgroups leave
    // the GPU mostly idle; each split keeps at least 8 key tiles (256 keys).
    const int64_t wgs = S * H * ((C + 127) / 128);
    if (wgs >= kChunkSplitTargetWGs / 2) return 1;
    const int64_t tiles = (W + 128 + 31) / 32;
    int64_t p = (kChunkSplitTargetWGs + wgs - 1) / wgs;
    p = p < tiles / 8 ? p : tiles / 8;
    p = p < kChunkMaxSplits ? p : kChunkMaxSplits;
    return p < 1 ? 1 : (int)p;
}

int64_t chunk_workspace_bytes(int64_t S, int64_t H, int64_t C, int64_t D, int64_t W) {
    const int P = chunk_splits(S, H, C, W);
    return P == 1 ? 0 : S * H * C * P * (D + 2) * (int64_t)sizeof(float);
}

hipError_t launch_chunk_bf16(const bf16* q, const bf16* kc, const bf16* vc, const bf16* kring,
                             const bf16* vring, const int64_t* pos0, bf16* out, int64_t S,
                             int64_t H, int64_t C, int D, int64_t W, void* workspace,
                             hipStream_t stream) {
    Args a = make_args(q, kc, vc, out, contiguous_layout(H, C, D), 1.0f / sqrtf((float)D));
    a.kring = kring;
    a.vring = vring;
    a.pos0 = pos0;
    a.C = (int)C;
    a.W = (int)W;
    a.nsplit = workspace ? chunk_splits(S, H, C, W) : 1;
    if (a.nsplit > 1) {
        a.ws_o = (float*)workspace;
        a.ws_ml = a.ws_o + S * H * C * a.nsplit * D;
    }
    hipError_t e = D == 128 ? launch<128, 4, true>(a, S, H, C, stream)
                            : launch<64, 4, true>(a, S, H, C, stream);
    if (e != hipSuccess || a.nsplit == 1) return e;
    return launch_combine_bf16(a.ws_o, a.ws_ml, out, S * H * C, a.nsplit, D, stream);
}

}  // namespace swa
