// One-token decode against a bounded W-slot ring of keys and values, bf16
// (or fp32: the kernel's element type E) in and out, fp32 arithmetic.  The
// ring is the bounded cache that keeps only the window ("25. Sliding-Window
// Causal Attention for Streaming Inference", Problem; "Sliding Window
// Attention", Key Advantages: a KV cache of size W).
//
// The path is bound by HBM: every occupied slot's k and v row is read once
// (2 * n * D * sizeof(E) bytes per (stream, head)) for 4 * n * D flops.  One
// workgroup of 256 threads owns one (stream, head); LPR lanes own one slot
// row, lane c of them its 16-byte chunks LPR i + c (8 bf16 or 4 fp32
// elements each).
//   phase 1  scores: each lane dots its chunks against the query's
//            (v_dot2_f32_bf16; fp32 FMAs), the LPR lanes of a row sum with
//            DPP steps, and the row's score goes to LDS, pre-scaled by
//            log2(e)/sqrt(D).
//   softmax  exact two-pass over the n LDS scores (max, then exp2 and sum).
//   phase 2  output: the same lane/slot mapping streams v rows, each lane
//            accumulating p * v for its columns; partial outputs are reduced
//            across the 256 / LPR row slots through LDS.
// Two mappings.  Row-contiguous (LPR = D / 8 for bf16, D / 4 for fp32, one
// chunk per lane): one wavefront load covers whole consecutive rows, a
// contiguous KiB, and the loads are non-temporal (the ring is read once).
// Quad (LPR = 4, several chunks per lane): fewer vector instructions per
// byte.  Measured on 16 GiB reads, 1-KiB-contiguous non-temporal loads reach
// 7.05-7.1 TB/s, ordinary loads 6.2-6.35 TB/s whatever the pattern, and
// non-temporal loads that cover 64 bytes of 16 rows per instruction (the
// quad mapping) 6.36-6.48.  With at least one workgroup per compute unit the
// launch is bound by HBM and takes the row-contiguous mapping (7.0-7.1 TB/s
// against 6.2-6.3 for the quad one from 512 workgroups on); with fewer, each
// workgroup's own issue rate bounds it and the quad mapping is faster (46
// against 62 us for one stream of 32 heads, W = 4096).
// Occupied slots are [0, min(pos + 1, W)): unoccupied slots are never read.

#include "swa_internal.h"

#include <atomic>

namespace swa {
namespace {

constexpr int kDecThreads = 256;
// launches of at least this many workgroups (one per compute unit) take
// the row-contiguous mapping
constexpr int64_t kDecRowsMinWGs = 256;

// Sum over the 4 lanes of a quad (DPP quad_perm; no LDS traffic).
__device__ inline float quad_sum(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
    return x;
}

// Sum over the N lanes (4, 8, 16 or 32) that hold one row, left in all of
// them (DPP: quad exchanges, then the half-row and row mirrors; a lane
// exchange for the two 16-lane rows of 32).
template <int N>
__device__ inline float row_sum(float x) {
    x = quad_sum(x);
    if constexpr (N >= 8)
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, true));
    if constexpr (N >= 16)
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, true));
    if constexpr (N >= 32) x += __shfl_xor(x, 16, 64);
    return x;
}

__device__ inline float dot8(const u32x4& k, const u32x4& q, float acc) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // Copy the lanes out first: a bit_cast of a vector-element lvalue
        // reads element 0 whatever the index.
        const uint32_t kj = k[j], qj = q[j];
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kj),
                                              __builtin_bit_cast(bf16x2, qj), acc, false);
    }
    return acc;
}

__device__ inline float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// One 16-byte chunk of a row (8 bf16 or 4 fp32 elements): its dot product
// with the query's chunk, and acc[e] += p * element e.
template <typename E>
__device__ inline float chunk_dot(const u32x4& k, const u32x4& q, float acc) {
    if constexpr (sizeof(E) == 2) {
        return dot8(k, q, acc);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t kj = k[j], qj = q[j];
            acc = fmaf(__uint_as_float(kj), __uint_as_float(qj), acc);
        }
        return acc;
    }
}
template <typename E>
__device__ inline void chunk_axpy(float p, const u32x4& v, float (&acc)[16 / sizeof(E)]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t vj = v[j];
        if constexpr (sizeof(E) == 2) {
            acc[2 * j] = fmaf(p, bf_lo(vj), acc[2 * j]);
            acc[2 * j + 1] = fmaf(p, bf_hi(vj), acc[2 * j + 1]);
        } else {
            acc[j] = fmaf(p, __uint_as_float(vj), acc[j]);
        }
    }
}

// Arguments of one decode launch.  A launch has S * H * P workgroups: split
// sp of (stream, head) sh covers the occupied slots [sp * chunk,
// min(n, (sp + 1) * chunk)).  With P = 1 the workgroup writes the output;
// otherwise it writes its unnormalised partial output, max and sum to the
// workspace and decode_combine_kernel merges the P partials.
template <typename E>
struct DecArgs {
    const E* q;
    const E* kring;
    const E* vring;
    const int64_t* pos;
    E* out;
    const E* knew;        // fused append: k, v of the current token ([S, H, D]), else null
    const E* vnew;
    E* kring_w;           // the rings again, writable (fused append only)
    E* vring_w;
    float* ws_o;          // [S * H * P, D] partial outputs (P > 1)
    float* ws_ml;         // [S * H * P, 2] partial (max, sum) (P > 1)
    int64_t H, W;
    int P, chunk;
    float c;              // log2(e) / sqrt(D)
};

template <typename E, int D, bool ROWS>
__global__ __launch_bounds__(kDecThreads) void decode_bf16_kernel(DecArgs<E> a) {
    constexpr int EPC = 16 / (int)sizeof(E);   // elements per 16-byte chunk
    constexpr int LPR = ROWS ? D / EPC : 4;     // lanes per row
    constexpr int CPL = D / (EPC * LPR);        // 16-byte chunks per lane per row
    constexpr int RPG = kDecThreads / LPR;      // rows per workgroup and load
    // loads per lane in flight (x CPL)
    constexpr int UN = ROWS ? 16 : (sizeof(E) == 2 ? 4 : 2);
    auto ld = [](const E* p) {
        const u32x4* v = reinterpret_cast<const u32x4*>(p);
        if constexpr (ROWS) return __builtin_nontemporal_load(v);
        else return *v;
    };
    extern __shared__ __attribute__((aligned(16))) float sm[];
    float* sc = sm;                             // scores / probabilities, later partial outputs
    __shared__ float red[kDecThreads / 64];

    const int tid = threadIdx.x;
    const int cl = tid % LPR, rw = tid / LPR;   // chunk lane, row slot
    const int wave = tid >> 6, lane = tid & 63;
    const int64_t bid = blockIdx.x;
    const int64_t sh = bid / a.P;
    const int sp = (int)(bid - sh * a.P);
    const int64_t s = sh / a.H;
    const int64_t p = a.pos[s];
    const int64_t W = a.W;
    int64_t n64 = p + 1;
    n64 = n64 < 0 ? 0 : (n64 > W ? W : n64);
    const int n = (int)n64;
    const int lo = sp * a.chunk;
    const int hi = min(n, lo + a.chunk);       // rows [lo, hi); empty when lo >= hi
    const int cnt = hi > lo ? hi - lo : 0;
    const E* __restrict__ Kr = a.kring + sh * W * D;
    const E* __restrict__ Vr = a.vring + sh * W * D;
    // Fused append: slot p mod W holds the current token, read from knew /
    // vnew instead of the ring (which this launch writes).
    // The slot is written by the one split that covers it (split 0 for a
    // negative position, which has no occupied slots: the slot index is
    // reduced into [0, W) as the plain append does).
    int wslot = -1;
    const E* __restrict__ Kn = nullptr;
    const E* __restrict__ Vn = nullptr;
    if (a.knew != nullptr) {
        int64_t w64 = p % W;
        w64 = w64 < 0 ? w64 + W : w64;
        const int wsl = (int)w64;
        Kn = a.knew + sh * D;
        Vn = a.vnew + sh * D;
        if (p >= 0) wslot = wsl;                // always inside [0, n)
        const bool owner = p >= 0 ? (wsl >= lo && wsl < hi) : sp == 0;
        if (owner && tid < D / EPC) {
            const int64_t dst = (sh * W + wsl) * D + tid * EPC;
            *reinterpret_cast<u32x4*>(a.kring_w + dst) = *reinterpret_cast<const u32x4*>(Kn + tid * EPC);
            *reinterpret_cast<u32x4*>(a.vring_w + dst) = *reinterpret_cast<const u32x4*>(Vn + tid * EPC);
        }
    }

    // query chunks LPR i + cl
    u32x4 qv[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
        qv[i] = *reinterpret_cast<const u32x4*>(a.q + sh * D + (LPR * i + cl) * EPC);

    // ---- phase 1: scores
    for (int r0 = lo; r0 < hi; r0 += RPG * UN) {
        u32x4 kv[UN][CPL];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int row = r0 + rw + RPG * u;
            const E* src = row == wslot ? Kn : Kr + (int64_t)row * D;
#pragma unroll
            for (int i = 0; i < CPL; ++i)
                kv[u][i] = row < hi ? ld(src + (LPR * i + cl) * EPC) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int row = r0 + rw + RPG * u;
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < CPL; ++i) acc = chunk_dot<E>(kv[u][i], qv[i], acc);
            acc = row_sum<LPR>(acc);
            if (cl == 0 && row < hi) sc[row - lo] = acc * a.c;
        }
    }
    __syncthreads();

    // ---- softmax over the cnt scores: max, then exp2 and sum
    float mx = -__builtin_inff();
    for (int r = tid; r < cnt; r += kDecThreads) mx = fmaxf(mx, sc[r]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float ls = 0.f;
    for (int r = tid; r < cnt; r += kDecThreads) {
        const float e = __builtin_amdgcn_exp2f(sc[r] - mx);
        sc[r] = e;
        ls += e;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ls += __shfl_xor(ls, o, 64);
    if (lane == 0) red[wave] = ls;
    __syncthreads();
    const float l = (red[0] + red[1]) + (red[2] + red[3]);

    // ---- phase 2: o = sum_r p_r v_r over this lane's columns
    float acc[CPL][EPC];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[i][e] = 0.f;
    for (int r0 = lo; r0 < hi; r0 += RPG * UN) {
        u32x4 vv[UN][CPL];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int row = r0 + rw + RPG * u;
            const E* src = row == wslot ? Vn : Vr + (int64_t)row * D;
#pragma unroll
            for (int i = 0; i < CPL; ++i)
                vv[u][i] = row < hi ? ld(src + (LPR * i + cl) * EPC) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int row = r0 + rw + RPG * u;
            const float pr = row < hi ? sc[row - lo] : 0.f;
#pragma unroll
            for (int i = 0; i < CPL; ++i) chunk_axpy<E>(pr, vv[u][i], acc[i]);
        }
    }
    __syncthreads();   // every lane is done with the probabilities

    // ---- reduce partial outputs over the RPG row slots: sm[rw][d]
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
        for (int e = 0; e < EPC; ++e) sm[rw * D + (LPR * i + cl) * EPC + e] = acc[i][e];
    __syncthreads();
    if (tid < D) {
        float t = 0.f;
        for (int r = 0; r < RPG; ++r) t += sm[r * D + tid];
        if (a.P == 1) {
            a.out[sh * D + tid] = (E)(cnt > 0 ? t / l : 0.f);
        } else {
            a.ws_o[bid * D + tid] = t;
            if (tid == 0) {
                a.ws_ml[2 * bid] = mx;          // -inf for an empty split
                a.ws_ml[2 * bid + 1] = l;
            }
        }
    }
}

// Merge the P partials of each (stream, head): with M the largest partial
// max, o = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.  Empty splits
// (m_p = -inf) get weight 0; a stream with no occupied slot gets 0.  One
// wavefront per row: lane p holds split p's (max, sum) (P <= 64), M and the
// weighted sum come from wave reductions, and the output loop takes each
// split's weight from its lane and keeps eight splits' loads in flight.
template <typename E, int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ ws_o,
                                                            const float* __restrict__ ws_ml,
                                                            E* __restrict__ out, int P) {
    constexpr int R = (D + 63) / 64;            // columns lane + 64 r (those below D)
    const int64_t sh = blockIdx.x;
    const int lane = threadIdx.x;
    const float* ml = ws_ml + 2 * sh * P;
    float mp = -__builtin_inff(), lp = 0.f;
    if (lane < P) {
        mp = ml[2 * lane];
        lp = ml[2 * lane + 1];
    }
    float M = mp;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float wp = mp == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mp - M);
    float L = wp * lp;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
    float o[R];
#pragma unroll
    for (int r = 0; r < R; ++r) o[r] = 0.f;
    const float* po = ws_o + sh * P * D + lane;
    for (int p = 0; p < P; p += 8) {
        float y[8][R];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int r = 0; r < R; ++r)
                y[u][r] = p + u < P && lane + 64 * r < D ? po[(int64_t)(p + u) * D + 64 * r] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            // weight of split p + u: 0 for an empty split, whose row is never used
            const float w = p + u < P
                ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wp), p + u)) : 0.f;
            if (w != 0.f) {
#pragma unroll
                for (int r = 0; r < R; ++r) o[r] = fmaf(w, y[u][r], o[r]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (lane + 64 * r < D) out[sh * D + lane + 64 * r] = (E)(L > 0.f ? o[r] / L : 0.f);
}

// Raise the kernel's dynamic-LDS limit to the largest score array, once
// per device (bit dev of done).
template <typename E, int D, bool ROWS>
hipError_t allow_lds() {
    static std::atomic<uint64_t> done{0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    const uint64_t bit = 1ull << (dev & 63);
    if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
    hipError_t e = hipFuncSetAttribute((const void*)decode_bf16_kernel<E, D, ROWS>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)(kDecodeMaxW * sizeof(float)));
    if (e == hipSuccess) done.fetch_or(bit, std::memory_order_release);
    return e;
}

template <typename E, int D, bool ROWS>
hipError_t launch_mapping(const DecArgs<E>& a, int64_t wgs, hipStream_t stream) {
    // scores (one float per slot of the split), later the partial outputs
    // of the RPG row slots
    const int64_t red = (int64_t)(kDecThreads / (ROWS ? D / (16 / (int)sizeof(E)) : 4)) * D;
    const int64_t floats = a.chunk > red ? (int64_t)a.chunk : red;
    hipError_t e = allow_lds<E, D, ROWS>();
    if (e != hipSuccess) return e;
    void* args[] = {(void*)&a};
    return hipLaunchKernel((const void*)decode_bf16_kernel<E, D, ROWS>, dim3((unsigned)wgs),
                           dim3(kDecThreads), args, (unsigned)(floats * sizeof(float)), stream);
}

template <typename E, int D>
hipError_t launch(DecArgs<E> a, int64_t S, hipStream_t stream) {
    a.c = kLog2e / sqrtf((float)D);
    const int64_t wgs = S * a.H * a.P;
    hipError_t e = wgs >= kDecRowsMinWGs ? launch_mapping<E, D, true>(a, wgs, stream)
                                         : launch_mapping<E, D, false>(a, wgs, stream);
    if (e != hipSuccess || a.P == 1) return e;
    const float* wo = a.ws_o;
    const float* wml = a.ws_ml;
    int P = a.P;
    void* cargs[] = {(void*)&wo, (void*)&wml, (void*)&a.out, (void*)&P};
    return hipLaunchKernel((const void*)decode_combine_kernel<E, D>, dim3((unsigned)(S * a.H)),
                           dim3(64), cargs, 0, stream);
}

// ---- ring append -----------------------------------------------------------

template <typename U>
__global__ __launch_bounds__(256) void ring_append_kernel(
    const U* __restrict__ knew, const U* __restrict__ vnew, U* __restrict__ kring,
    U* __restrict__ vring, const int64_t* __restrict__ pos, int64_t H, int64_t D, int64_t W) {
    const int64_t sh = blockIdx.x;
    const int64_t s = sh / H;
    int64_t slot = pos[s] % W;
    if (slot < 0) slot += W;
    const int64_t dst = (sh * W + slot) * D;
    for (int64_t d = threadIdx.x; d < D; d += blockDim.x) {
        kring[dst + d] = knew[sh * D + d];
        vring[dst + d] = vnew[sh * D + d];
    }
}

// Chunk append: tokens pos0 + c for c in [cfirst, C) go to slot
// (pos0 + c) mod W.  Only the last min(C, W) tokens of a chunk can survive,
// so cfirst = max(0, C - W) and no two writes of one call share a slot.
template <typename U>
__global__ __launch_bounds__(256) void ring_append_chunk_kernel(
    const U* __restrict__ kc, const U* __restrict__ vc, U* __restrict__ kring,
    U* __restrict__ vring, const int64_t* __restrict__ pos0, int64_t H, int64_t C, int64_t D,
    int64_t W, int64_t cfirst) {
    const int64_t sh = blockIdx.x;
    const int64_t s = sh / H;
    const int64_t p0 = pos0[s] < 0 ? 0 : pos0[s];     // same clamp as the chunk forward
    for (int64_t c = cfirst + blockIdx.y; c < C; c += gridDim.y) {
        const int64_t slot = (p0 + c) % W;
        const int64_t dst = (sh * W + slot) * D;
        const int64_t src = (sh * C + c) * D;
        for (int64_t d = threadIdx.x; d < D; d += blockDim.x) {
            kring[dst + d] = kc[src + d];
            vring[dst + d] = vc[src + d];
        }
    }
}

}  // namespace

hipError_t launch_ring_append_chunk(const void* kc, const void* vc, void* kring, void* vring,
                                    const int64_t* pos0, int64_t S, int64_t H, int64_t C,
                                    int64_t D, int64_t W, int elem_bytes, hipStream_t stream) {
    int64_t cfirst = C > W ? C - W : 0;
    const int64_t n = C - cfirst;
    const dim3 grid((unsigned)(S * H), (unsigned)(n < 65535 ? n : 65535));
    const dim3 block(D >= 256 ? 256 : (unsigned)((D + 63) / 64 * 64));
    if (elem_bytes == 4) {
        const uint32_t* kn = (const uint32_t*)kc;
        const uint32_t* vn = (const uint32_t*)vc;
        uint32_t* kr = (uint32_t*)kring;
        uint32_t* vr = (uint32_t*)vring;
        void* args[] = {(void*)&kn, (void*)&vn, (void*)&kr, (void*)&vr, (void*)&pos0,
                        (void*)&H, (void*)&C, (void*)&D, (void*)&W, (void*)&cfirst};
        return hipLaunchKernel((const void*)ring_append_chunk_kernel<uint32_t>, grid, block, args,
                               0, stream);
    }
    const uint16_t* kn = (const uint16_t*)kc;
    const uint16_t* vn = (const uint16_t*)vc;
    uint16_t* kr = (uint16_t*)kring;
    uint16_t* vr = (uint16_t*)vring;
    void* args[] = {(void*)&kn, (void*)&vn, (void*)&kr, (void*)&vr, (void*)&pos0,
                    (void*)&H, (void*)&C, (void*)&D, (void*)&W, (void*)&cfirst};
    return hipLaunchKernel((const void*)ring_append_chunk_kernel<uint16_t>, grid, block, args, 0,
                           stream);
}

static_assert(kDecMaxSplits <= 64 && kChunkMaxSplits <= 64, "one combine lane per split");

hipError_t launch_combine_bf16(const float* ws_o, const float* ws_ml, bf16* out, int64_t rows,
                               int P, int D, hipStream_t stream) {
    if (P < 1 || P > 64) return hipErrorInvalidValue;
    void* cargs[] = {(void*)&ws_o, (void*)&ws_ml, (void*)&out, (void*)&P};
    const void* k = D == 128 ? (const void*)decode_combine_kernel<bf16, 128>
                             : (const void*)decode_combine_kernel<bf16, 64>;
    return hipLaunchKernel(k, dim3((unsigned)rows), dim3(64), cargs, 0, stream);
}

int decode_splits(int64_t S, int64_t H, int64_t W) {
    // Splitting pays while S * H workgroups leave most compute units idle
    // (measured at D = 128, W = 4096: 2.9x at S * H = 32, 1.8x at 64, 1.14x
    // at 128, 1.01x at 256, none from 512 on).  Aim for kDecSplitTargetWGs
    // workgroups with at least kDecSplitMinSlots slots each (smaller splits
    // measured slower, and so did a target of 4096 at S * H = 256 and 512).
    const int64_t sh = S * H;
    if (sh >= kDecSplitTargetWGs / 4) return 1;
    int64_t p = (kDecSplitTargetWGs + sh - 1) / sh;
    const int64_t pmax = (W + kDecSplitMinSlots - 1) / kDecSplitMinSlots;
    p = p < pmax ? p : pmax;
    p = p < kDecMaxSplits ? p : kDecMaxSplits;
    return p < 1 ? 1 : (int)p;
}

int64_t decode_workspace_bytes(int64_t S, int64_t H, int64_t D, int64_t W) {
    const int P = decode_splits(S, H, W);
    return P == 1 ? 0 : S * H * P * (D + 2) * (int64_t)sizeof(float);
}

hipError_t launch_decode_bf16(const bf16* q, const bf16* kring, const bf16* vring,
                              const int64_t* pos, bf16* out, int64_t S, int64_t H, int D,
                              int64_t W, const bf16* knew, const bf16* vnew, void* workspace,
                              hipStream_t stream) {
    DecArgs<bf16> a = {};
    a.q = q;
    a.kring = kring;
    a.vring = vring;
    a.pos = pos;
    a.out = out;
    a.knew = knew;
    a.vnew = vnew;
    a.kring_w = const_cast<bf16*>(kring);
    a.vring_w = const_cast<bf16*>(vring);
    a.H = H;
    a.W = W;
    a.P = workspace ? decode_splits(S, H, W) : 1;
    a.chunk = (int)((W + a.P - 1) / a.P);
    if (a.P > 1) {
        a.ws_o = (float*)workspace;
        a.ws_ml = a.ws_o + S * H * a.P * D;
    }
    if (D == 128) return launch<bf16, 128>(a, S, stream);
    return launch<bf16, 64>(a, S, stream);
}

bool decode_f32_supports(const void* q, const void* kring, const void* vring, const void* out,
                         const void* knew, const void* vnew, int64_t D, int64_t W) {
    if ((D != 32 && D != 64 && D != 128) || W > kDecodeMaxW) return false;
    for (const void* p : {q, kring, vring, out, knew, vnew})
        if (((uintptr_t)p & 15) != 0) return false;    // (null passes)
    return true;
}

hipError_t launch_decode_f32(const float* q, const float* kring, const float* vring,
                             const int64_t* pos, float* out, int64_t S, int64_t H, int D,
                             int64_t W, const float* knew, const float* vnew, void* workspace,
                             hipStream_t stream) {
    DecArgs<float> a = {};
    a.q = q;
    a.kring = kring;
    a.vring = vring;
    a.pos = pos;
    a.out = out;
    a.knew = knew;
    a.vnew = vnew;
    a.kring_w = const_cast<float*>(kring);
    a.vring_w = const_cast<float*>(vring);
    a.H = H;
    a.W = W;
    a.P = workspace ? decode_splits(S, H, W) : 1;
    a.chunk = (int)((W + a.P - 1) / a.P);
    if (a.P > 1) {
        a.ws_o = (float*)workspace;
        a.ws_ml = a.ws_o + S * H * a.P * D;
    }
    if (D == 128) return launch<float, 128>(a, S, stream);
    if (D == 64) return launch<float, 64>(a, S, stream);
    return launch<float, 32>(a, S, stream);
}

hipError_t launch_ring_append(const void* knew, const void* vnew, void* kring, void* vring,
                              const int64_t* pos, int64_t S, int64_t H, int64_t D, int64_t W,
                              int elem_bytes, hipStream_t stream) {
    const dim3 grid((unsigned)(S * H)), block(D >= 256 ? 256 : (unsigned)((D + 63) / 64 * 64));
    if (elem_bytes == 4) {
        const uint32_t* kn = (const uint32_t*)knew;
        const uint32_t* vn = (const uint32_t*)vnew;
        uint32_t* kr = (uint32_t*)kring;
        uint32_t* vr = (uint32_t*)vring;
        void* args[] = {(void*)&kn, (void*)&vn, (void*)&kr, (void*)&vr, (void*)&pos,
                        (void*)&H, (void*)&D, (void*)&W};
        return hipLaunchKernel((const void*)ring_append_kernel<uint32_t>, grid, block, args, 0, stream);
    }
    const uint16_t* kn = (const uint16_t*)knew;
    const uint16_t* vn = (const uint16_t*)vnew;
    uint16_t* kr = (uint16_t*)kring;
    uint16_t* vr = (uint16_t*)vring;
    void* args[] = {(void*)&kn, (void*)&vn, (void*)&kr, (void*)&vr, (void*)&pos,
                    (void*)&H, (void*)&D, (void*)&W};
    return hipLaunchKernel((const void*)ring_append_kernel<uint16_t>, grid, block, args, 0, stream);
}

}  // namespace swa
