// Matrix-core and LDS helpers shared by the bf16 band kernels (gfx950):
// lane exchanges, LDS tile swizzles, HBM -> LDS tile loads, the band mask on
// a score accumulator, P packing and the transposing operand reads.
#pragma once

#include "swa_internal.h"

namespace swa {
namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

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

// K tile: 16-byte chunk c of row r is stored at chunk c ^ kswz(r), so the 16
// lanes that read one chunk column of 16 consecutive rows (the S MFMA A
// operand) touch 16 different bank groups.
template <int D> __device__ inline int kswz(int row) {
    return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
// V tile: chunk c of row r is stored at c ^ vswz(r).  A transposing read
// covers 4 consecutive rows x 32 bytes per 16 lanes; XOR with 4 (r & 3)
// spreads the two 16-lane groups of a pass over 16 distinct chunks.
template <int D> __device__ inline int vswz(int row) {
    return D == 128 ? 4 * (row & 3) : 4 * (row & 1);
}
// Tile read both ways (whole rows, and transposed): chunk c of row r is
// stored at c ^ bswz(r), the bit reversal of r's low four bits (D = 128) or
// of bits 1..3 (D = 64).  It spreads the 16 lanes of a whole-row read over
// 16 bank groups and the 32 lanes of a transposing read over all 64 banks,
// so one copy of the tile serves both reads without conflicts.
template <int D> __device__ inline int bswz(int row) {
    if (D == 128) {
        const int r = row & 15;
        return ((r & 1) << 3) | ((r & 2) << 1) | ((r & 4) >> 1) | ((r & 8) >> 3);
    }
    const int r = (row >> 1) & 7;
    return ((r & 1) << 2) | (r & 2) | ((r & 4) >> 2);
}

// Buffer resource over the bytes [off, slab_bytes) of one (batch, head)
// slab whose rows are at least D elements apart: loads past the sequence
// end return zeros.  Keys past the end lie above every valid query's
// diagonal, so their scores are masked to -inf and their (zero) values get
// weight 0.
__device__ inline __amdgpu_buffer_rsrc_t rows_rsrc(const bf16* slab, int off, int slab_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(reinterpret_cast<const char*>(slab) + off), 0, slab_bytes - off,
        0x00020000);
}

// One 16-byte-per-lane buffer load into LDS: lane l's 16 bytes land at
// lds_base + 16 l (lds_base goes to M0).  Written as asm so the compiler
// does not see an LDS write: otherwise it cannot tell later LDS reads of
// other ring slots apart from the loads still streaming in and drains all
// in-flight loads before them.  The kernel orders these loads itself
// (counted vmcnt waits and a barrier before a slot is read).  No register
// is written, so nothing is left in flight into a VGPR.
__device__ inline void lds_load16(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_base, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_base), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

__device__ inline uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Tile read both ways in the 16x16x32 operand layout (whole rows: 16 lanes
// over 16 rows of one chunk column; transposed: 4 rows x 32 bytes per 16
// lanes).  The LDS services a wavefront's lanes in passes that pair lanes
// l and l + 32 (16 of them per pass for 16-byte reads, 32 for 8-byte
// reads), which the bit reversal above does not spread for this layout;
// XOR-ing the chunk with 4, 8, 3 and 2 for row bits 0..3 (D = 128; 4, 3, 2
// for bits 1..3 at D = 64) puts every pass of both reads on distinct banks.
template <int D> __device__ inline int qswz(int row) {
    if (D == 128)
        return ((row & 1) ? 4 : 0) ^ ((row & 2) ? 8 : 0) ^ ((row & 4) ? 3 : 0) ^ ((row & 8) ? 2 : 0);
    return ((row & 2) ? 4 : 0) ^ ((row & 4) ? 3 : 0) ^ ((row & 8) ? 2 : 0);
}

// Swizzle selectors for tile layouts in LDS.
constexpr int kSwzK = 0;   // kswz: rows read whole (16 lanes over 16 rows of one chunk column)
constexpr int kSwzV = 1;   // vswz: rows read through ds_read_b64_tr_b16
constexpr int kSwzB = 2;   // bswz: rows read both ways
constexpr int kSwzQ = 3;   // qswz: rows read both ways, 16x16x32 layout
template <int D, int SW> __device__ inline int swz(int row) {
    return SW == kSwzV   ? vswz<D>(row)
           : SW == kSwzB ? bswz<D>(row)
           : SW == kSwzQ ? qswz<D>(row)
                         : kswz<D>(row);
}

// Source offsets of one tile's loads (N 1-KiB loads per wave, NW waves).
// Load n of this wave writes tile bytes [1024 n, 1024 n + 1024), lane l the
// 16 bytes at 1024 n + 16 l; it fetches the chunk that the swizzle stores
// there, from a row rsb bytes apart from the previous one.
template <int D, int NW, int SW, int N>
__device__ inline void tile_offsets(uint32_t (&voff)[N], int wave, int lane, int rsb) {
    constexpr int ROWB = 2 * D;
    static_assert(N * NW * 1024 == 32 * ROWB, "loads cover one 32-row tile");
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int p = (wave * N + i) * 1024 + lane * 16;
        const int row = p / ROWB;
        const int phys = (p % ROWB) >> 4;
        const int logical = phys ^ swz<D, SW>(row);
        voff[i] = row * rsb + logical * 16;
    }
}

// One 16-byte-per-lane global load into LDS (per-lane source addresses),
// written as asm for the same reason as lds_load16.
__device__ inline void lds_load16_global(uint32_t lds_base, const void* src) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_base), "v"(src)
                 : "memory", "m0");
}

// Start the HBM -> LDS copy of one tile.
template <int N>
__device__ inline void dma_tile(__amdgpu_buffer_rsrc_t rsrc, uint32_t buf, int wave,
                                const uint32_t (&voff)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) lds_load16(rsrc, buf + (wave * N + i) * 1024, voff[i]);
}

// Dispatch order of a grid of nblocks workgroups, nper per (b, h) slab, rank
// r of a slab's workgroups having the r-th longest band (ranks below nfull
// full length, later ranks ever shorter).  The hardware deals workgroups
// round-robin over the 8 XCDs and each XCD dispatches its share in order;
// with remap, an XCD's share is consecutive logical tiles (logical tile
// bh * nper + r), so a slab's keys stay in one XCD's L2.  With nfull >= 0
// (each share is whole slabs) the share goes out longest first: the
// full-length ranks slab by slab, then the shorter ranks rank by rank across
// the share's slabs, so the last workgroups of an XCD are its shortest.
__device__ inline int xcd_logical_tile(int bid, int nblocks, int remap, int nper, int nfull) {
    if (!remap) return bid;
    const int per = nblocks >> 3;               // workgroups per XCD
    const int p = bid >> 3;                     // dispatch position on the XCD
    if (nfull < 0) return (bid & 7) * per + p;
    const int G = per / nper;                   // slabs per XCD
    int slab, rank;
    if (p < G * nfull) {
        slab = p / nfull;
        rank = p - slab * nfull;
    } else {
        const int pr = p - G * nfull;
        rank = nfull + pr / G;
        slab = pr - (rank - nfull) * G;
    }
    return (bid & 7) * per + slab * nper + rank;
}

// nfull for xcd_logical_tile on the host: nshort of a slab's nper ranks have
// shorter bands; -1 (plain order) unless every XCD's share is whole slabs and
// at most 8 of them.  Longest-first pays where an XCD holds few slabs (a late
// slab's full-length workgroups otherwise overrun the others at the end of
// the grid); with many, the tail is short already and the short workgroups of
// many slabs at once reuse L2 less.
inline int xcd_longest_first_nfull(int64_t nblocks, int64_t nper, int64_t nshort) {
    if (nblocks % 8 != 0 || (nblocks / 8) % nper != 0 || (nblocks / 8) / nper > 8) return -1;
    return (int)(nper - (nshort < nper ? nshort : nper));
}

// Band mask of a tile starting at key k0: key j is visible to query qi iff
// 0 <= qi - j < W; the other scores become -inf (bit for bit, whatever they
// held, +inf and NaN included).
__device__ inline void mask_tile(f32x16& s, int qi, int k0, int hh, int W) {
    // Register v holds key offset kof = 8 (v / 4) + v % 4 (0 .. 27) past
    // k0 + 4 hh.  The visible offsets, base - W < kof <= base, are one range
    // of bits of vis, and each score keeps its bits or becomes -inf by a
    // bitwise select on its bit: 42 vector instructions per masked tile
    // against 48 and 16 wait states for compare-and-select, whose lane-mask
    // results cannot be read back to back.
    const int base = qi - k0 - 4 * hh;
    const int h1 = min(max(base + 1, 0), 29);
    const int l0 = min(max(base - W + 1, 0), 28);
    uint32_t vis = (1u << h1) - (1u << l0);
    // keeps the per-score masks from being computed ahead, out of a loop,
    // into registers of their own
    asm volatile("" : "+v"(vis));
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int kof = 8 * (v >> 2) + (v & 3);
        // keep: bit kof of vis, sign-extended (all ones or zero)
        const int keep = __builtin_amdgcn_sbfe((int)vis, kof, 1);
        s[v] = __int_as_float((__float_as_int(s[v]) & keep) | ((int)0xff800000u & ~keep));
    }
}

// Eight probabilities as the bf16 B operand; their sum is added to acc with
// v_dot2 against ones, so l sums exactly the weights the MFMA applies.
__device__ inline bf16x8 pack_p(const f32x16& s, int e0, float& acc) {
    bf16x8 pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[e] = (bf16)s[e0 + e];
    const u32x4 pw = __builtin_bit_cast(u32x4, pf);
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t w = pw[j];   // scalar copy: bit_cast of a vector element reads element 0
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, acc, false);
    }
    return pf;
}

// A operands of O^T += V^T P^T for the 16-key chunk ch.  Lane l (i = l % 16,
// group half dh = (l / 16) % 2, hh = l / 32) needs, for d = 32 db + l % 32,
// the keys 16 ch + 8 a + 4 hh + e (a = 0, 1; e = 0..3).  One
// ds_read_b64_tr_b16 over the 16 lanes of a group hands lane i column
// (group base + i) of the 4 x 16 block whose row r0 + i/4, columns
// 4 (i % 4) .. + 3, lane i addresses.  SW is the tile's storage swizzle
// (kSwzV makes these reads conflict free).
template <int D, int SW = kSwzV>
__device__ inline void read_v_chunk(const char* Vt, int ch, int lane, bf16x8 (&va)[D / 32]) {
    const int i = lane & 15, hh = lane >> 5, dh = (lane >> 4) & 1;
    const int row = 16 * ch + 4 * hh + (i >> 2);           // + 8 a
    const int sw0 = swz<D, SW>(row), sw1 = swz<D, SW>(row + 8);
    const char* rp = Vt + row * (2 * D) + 8 * (i & 1);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        const int chunk = 4 * db + 2 * dh + ((i & 3) >> 1);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(rp + ((chunk ^ sw0) << 4)));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(rp + 8 * 2 * D + ((chunk ^ sw1) << 4)));
        va[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
}

// A operand rows of a tile read whole: lane l reads row l % 32, 16-byte
// chunk 2 dc + l / 32 (the K operand of S^T = K Q^T).
template <int D, int SW = kSwzK>
__device__ inline bf16x8 read_row_frag(const char* tile, int lr, int hh, int dc) {
    return *reinterpret_cast<const bf16x8*>(tile + lr * (2 * D) +
                                            (((2 * dc + hh) ^ swz<D, SW>(lr)) << 4));
}
}  // namespace
}  // namespace swa
