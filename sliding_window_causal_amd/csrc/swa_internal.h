// Internal declarations shared by the libswa translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element strides of a [B, H, T, D] operand whose D axis is contiguous:
// element (b, h, t, d) sits at b * b + h * h + t * t + d.
struct Strides {
    int64_t b, h, t;
};
// Strides of q, k, v and out of one prefill call.
struct Layout {
    Strides q, k, v, o;
};
inline Layout contiguous_layout(int64_t H, int64_t T, int64_t D) {
    const Strides s = {H * T * D, T * D, D};
    return {s, s, s, s};
}

// ---- launchers (each returns the hipError_t of its launch) -----------------

// Generic wavefront-per-row kernels; T is float or bf16; 1 <= D <= 256.
template <typename T>
hipError_t launch_rowwise_prefill(const T* q, const T* k, const T* v, T* out,
                                  int64_t B, int64_t H, int64_t Tn, int D, int64_t W,
                                  const Layout& L, float scale, hipStream_t stream,
                                  float* lse = nullptr);
template <typename T>
hipError_t launch_rowwise_decode(const T* q, const T* kring, const T* vring,
                                 const int64_t* pos, T* out, int64_t S, int64_t H, int D,
                                 int64_t W, hipStream_t stream);

// Band attention backward, wavefront per query row (dq, log-sum-exp and
// delta into lse / delta, B*H*T floats each), then per key row (dk, dv).
template <typename T>
hipError_t launch_rowwise_backward(const T* q, const T* k, const T* v, const T* o, const T* dout,
                                   T* dq, T* dk, T* dv, float* lse, float* delta, int64_t B,
                                   int64_t H, int64_t Tn, int D, int64_t W, float scale,
                                   hipStream_t stream);

// bf16 matrix-core backward (contiguous [B, H, T, D], D in {64, 128},
// 16-byte aligned, any finite scale): unless lse_in is given, the forward
// again for the per-row log-sum-exp (into lse; its output goes to dq); then
// dq (and delta), dv, dk kernels.  With |scale| sqrt(D) above
// kBwdFastSharpness (a softmax sharper than the default scale's) the precise
// variant runs: a row-statistics kernel first (normalisers into lse, delta),
// and dS split into two bf16 terms.
constexpr double kBwdFastSharpness = 1.001;
bool backward_bf16_supports(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, int64_t T, int64_t D, double scale);
bool backward_bf16_precise(double scale, int64_t D);
hipError_t launch_backward_bf16(const bf16* q, const bf16* k, const bf16* v, const bf16* o,
                                const bf16* dout, bf16* dq, bf16* dk, bf16* dv,
                                const float* lse_in, float* lse, float* delta, int64_t B,
                                int64_t H, int64_t T, int D, int64_t W, float scale,
                                hipStream_t stream);

// Chunk continuation of a ring, wavefront per row; T is float or bf16.
template <typename T>
hipError_t launch_rowwise_chunk(const T* q, const T* kc, const T* vc, const T* kring,
                                const T* vring, const int64_t* pos0, T* out, int64_t S, int64_t H,
                                int64_t C, int D, int64_t W, hipStream_t stream);

// bf16 MFMA band prefill; D in {64, 128}.  Every pointer 16-byte aligned,
// every stride a multiple of 8 elements, row strides >= D, and each
// (batch, head) slab of k and v within 2^31 bytes (prefill_bf16_supports).
bool prefill_bf16_supports(const void* q, const void* k, const void* v, const void* out,
                           int64_t T, int64_t D, const Layout& L);
// With lse non-null, row i of (batch, head) bh also gets the log-sum-exp of
// its scaled scores, ln(sum_j exp(s_ij * scale)), at lse[bh * T + i].
hipError_t launch_prefill_bf16(const bf16* q, const bf16* k, const bf16* v, bf16* out,
                               int64_t B, int64_t H, int64_t T, int D, int64_t W,
                               const Layout& L, float scale, hipStream_t stream,
                               float* lse = nullptr);

// fp32 MFMA prefill (v_mfma_f32_32x32x2_f32): D in {32, 64, 128}, 16-byte
// aligned pointers, every stride a multiple of 4 elements
// (prefill_f32_supports); lse as for launch_prefill_bf16.
bool prefill_f32_supports(const void* q, const void* k, const void* v, const void* out,
                          int64_t T, int64_t D, const Layout& L);
hipError_t launch_prefill_f32(const float* q, const float* k, const float* v, float* out,
                              int64_t B, int64_t H, int64_t T, int D, int64_t W, const Layout& L,
                              float scale, hipStream_t stream, float* lse = nullptr);

// fp32 MFMA chunk continuation of a ring (q, kc, vc, out contiguous
// [S, H, C, D], rings [S, H, W, D]); D in {32, 64, 128}, 16-byte aligned.
bool chunk_f32_supports(const void* q, const void* kc, const void* vc, const void* kring,
                        const void* vring, const void* out, int64_t C, int64_t D, int64_t W);
hipError_t launch_chunk_f32(const float* q, const float* kc, const float* vc, const float* kring,
                            const float* vring, const int64_t* pos0, float* out, int64_t S,
                            int64_t H, int64_t C, int D, int64_t W, hipStream_t stream);

// fp32 matrix-core backward (contiguous [B, H, T, D], D in {32, 64, 128},
// 16-byte aligned): unless lse_in is given, the fp32 forward again for the
// per-row log-sum-exp (into lse; its output goes to dq); then a query-row
// kernel (dq; writes the log2 normalisers to lse and dout . out to delta)
// and a key-row kernel (dk, dv).
bool backward_f32_supports(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const void* dq, const void* dk, const void* dv,
                           int64_t T, int64_t D);
hipError_t launch_backward_f32(const float* q, const float* k, const float* v, const float* o,
                               const float* dout, float* dq, float* dk, float* dv,
                               const float* lse_in, float* lse, float* delta, int64_t B,
                               int64_t H, int64_t T, int D, int64_t W, float scale,
                               hipStream_t stream);

// bf16 MFMA chunk continuation of a ring (q, kc, vc, out contiguous
// [S, H, C, D], rings [S, H, W, D]); D in {64, 128}, 16-byte aligned
// pointers, slabs under 2 GiB (chunk_bf16_supports).
bool chunk_bf16_supports(const void* q, const void* kc, const void* vc, const void* kring,
                         const void* vring, const void* out, int64_t C, int64_t D, int64_t W);
// With a workspace of chunk_workspace_bytes() the key range of each query
// tile may be split over chunk_splits() workgroups and the partials merged by
// launch_combine_bf16.
constexpr int64_t kChunkSplitTargetWGs = 512;
constexpr int64_t kChunkMaxSplits = 16;
int chunk_splits(int64_t S, int64_t H, int64_t C, int64_t W);
int64_t chunk_workspace_bytes(int64_t S, int64_t H, int64_t C, int64_t D, int64_t W);
hipError_t launch_chunk_bf16(const bf16* q, const bf16* kc, const bf16* vc, const bf16* kring,
                             const bf16* vring, const int64_t* pos0, bf16* out, int64_t S,
                             int64_t H, int64_t C, int D, int64_t W, void* workspace,
                             hipStream_t stream);
// Merge P partial rows (ws_o [rows * P, D], ws_ml [rows * P, 2]: max in log2
// units, sum) into out [rows, D]; D in {64, 128}, 1 <= P <= 64.
hipError_t launch_combine_bf16(const float* ws_o, const float* ws_ml, bf16* out, int64_t rows,
                               int P, int D, hipStream_t stream);

// bf16 ring decode; D in {64, 128}, W <= kDecodeMaxW.  With a workspace of
// decode_workspace_bytes(S, H, D, W) bytes the window may be split over
// decode_splits(S, H, W) workgroups per (stream, head) and merged by a second
// kernel; with knew / vnew the current token's k, v are read from there and
// written into slot pos mod W by the same launch.
constexpr int64_t kDecodeMaxW = 16384;
constexpr int64_t kDecSplitTargetWGs = 2048;
constexpr int64_t kDecSplitMinSlots = 256;
constexpr int64_t kDecMaxSplits = 64;
int decode_splits(int64_t S, int64_t H, int64_t W);
int64_t decode_workspace_bytes(int64_t S, int64_t H, int64_t D, int64_t W);
hipError_t launch_decode_bf16(const bf16* q, const bf16* kring, const bf16* vring,
                              const int64_t* pos, bf16* out, int64_t S, int64_t H, int D,
                              int64_t W, const bf16* knew, const bf16* vnew, void* workspace,
                              hipStream_t stream);

// Chunk append into the ring; any D >= 1; elem_bytes is 2 or 4.
// fp32 ring decode on the same kernel (split and fused append as for bf16):
// D in {32, 64, 128}, W <= kDecodeMaxW, 16-byte aligned pointers (knew and
// vnew may be null).
bool decode_f32_supports(const void* q, const void* kring, const void* vring, const void* out,
                         const void* knew, const void* vnew, int64_t D, int64_t W);
hipError_t launch_decode_f32(const float* q, const float* kring, const float* vring,
                             const int64_t* pos, float* out, int64_t S, int64_t H, int D,
                             int64_t W, const float* knew, const float* vnew, void* workspace,
                             hipStream_t stream);

hipError_t launch_ring_append_chunk(const void* kc, const void* vc, void* kring, void* vring,
                                    const int64_t* pos0, int64_t S, int64_t H, int64_t C,
                                    int64_t D, int64_t W, int elem_bytes, hipStream_t stream);

// Ring append; any D >= 1; elem_bytes is 2 or 4.
hipError_t launch_ring_append(const void* knew, const void* vnew, void* kring, void* vring,
                              const int64_t* pos, int64_t S, int64_t H, int64_t D, int64_t W,
                              int elem_bytes, hipStream_t stream);

}  // namespace swa
