// libswa C ABI: argument validation and kernel dispatch.  Declarations and
// the contract of every entry point are in include/swa.h.

#include "../../include/swa.h"
#include "swa_internal.h"

#include <cmath>

namespace {

constexpr int kAbiVersion = 2;
constexpr int64_t kMaxRowD = 256;

bool positive(int64_t x) { return x >= 1; }

// Element counts must stay addressable with 64-bit offsets and grid sizes
// must fit a 32-bit launch.
bool fits(int64_t a, int64_t b, int64_t c, int64_t d) {
    const int64_t lim = (int64_t)1 << 62;
    int64_t x = a;
    for (int64_t y : {b, c, d}) {
        if (x > lim / y) return false;
        x *= y;
    }
    return true;
}

int from_hip(hipError_t e) { return e == hipSuccess ? SWA_OK : SWA_ERR_LAUNCH; }

// Prefill dispatch once arguments are known to be non-null and positive.
// scale == 0 selects 1 / sqrt(D).
int forward(const void* q, const void* k, const void* v, void* out, int64_t B, int64_t H,
            int64_t T, int64_t D, int64_t W, const swa::Layout& L, double scale, int dtype,
            hipStream_t st, float* lse = nullptr) {
    if (B * H * T >= ((int64_t)1 << 31)) return SWA_ERR_UNSUPPORTED;
    const float sc = scale == 0.0 ? 1.0f / sqrtf((float)D) : (float)scale;
    if (dtype == SWA_BF16) {
        if (D != 64 && D != 128) return SWA_ERR_UNSUPPORTED;
        const swa::bf16 *qb = (const swa::bf16*)q, *kb = (const swa::bf16*)k,
                        *vb = (const swa::bf16*)v;
        if (swa::prefill_bf16_supports(q, k, v, out, T, D, L))
            return from_hip(swa::launch_prefill_bf16(qb, kb, vb, (swa::bf16*)out, B, H, T, (int)D,
                                                     W, L, sc, st, lse));
        // alignment or offsets the matrix-core kernel does not take
        return from_hip(swa::launch_rowwise_prefill<swa::bf16>(qb, kb, vb, (swa::bf16*)out, B, H,
                                                               T, (int)D, W, L, sc, st, lse));
    }
    if (dtype == SWA_F32) {
        if (D > kMaxRowD) return SWA_ERR_UNSUPPORTED;
        if (swa::prefill_f32_supports(q, k, v, out, T, D, L))
            return from_hip(swa::launch_prefill_f32((const float*)q, (const float*)k,
                                                    (const float*)v, (float*)out, B, H, T, (int)D,
                                                    W, L, sc, st, lse));
        // other head sizes, alignment or strides: one wavefront per row
        return from_hip(swa::launch_rowwise_prefill<float>((const float*)q, (const float*)k,
                                                           (const float*)v, (float*)out, B, H, T,
                                                           (int)D, W, L, sc, st, lse));
    }
    return SWA_ERR_UNSUPPORTED;
}

}  // namespace

extern "C" {

int swa_abi_version(void) { return kAbiVersion; }

const char* swa_status_string(int status) {
    switch (status) {
        case SWA_OK: return "ok";
        case SWA_ERR_INVALID_ARG: return "invalid argument (null pointer, size < 1 or window < 1)";
        case SWA_ERR_UNSUPPORTED: return "unsupported dtype or head size for this entry point";
        case SWA_ERR_LAUNCH: return "kernel launch failed";
        case SWA_ERR_SCRATCH_LIMIT:
            return "sizes need more scratch than the allocation-free entry point holds "
                   "(SWA_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

int swa_forward(const void* q, const void* k, const void* v, void* out, int64_t B, int64_t H,
                int64_t T, int64_t D, int64_t W, int dtype, void* stream) {
    if (!q || !k || !v || !out) return SWA_ERR_INVALID_ARG;
    if (!positive(B) || !positive(H) || !positive(T) || !positive(D) || !positive(W))
        return SWA_ERR_INVALID_ARG;
    if (!fits(B, H, T, D)) return SWA_ERR_UNSUPPORTED;
    return forward(q, k, v, out, B, H, T, D, W, swa::contiguous_layout(H, T, D), 0.0, dtype,
                   (hipStream_t)stream);
}

int swa_forward_lse(const void* q, const void* k, const void* v, void* out, float* lse,
                    int64_t B, int64_t H, int64_t T, int64_t D, int64_t W, double scale,
                    int dtype, void* stream) {
    if (!q || !k || !v || !out || !lse) return SWA_ERR_INVALID_ARG;
    if (!positive(B) || !positive(H) || !positive(T) || !positive(D) || !positive(W))
        return SWA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return SWA_ERR_INVALID_ARG;
    if (!fits(B, H, T, D)) return SWA_ERR_UNSUPPORTED;
    return forward(q, k, v, out, B, H, T, D, W, swa::contiguous_layout(H, T, D), scale, dtype,
                   (hipStream_t)stream, lse);
}

int swa_forward_strided(const void* q, const void* k, const void* v, void* out, int64_t B,
                        int64_t H, int64_t T, int64_t D, int64_t W, const int64_t* strides,
                        double scale, int dtype, void* stream) {
    if (!q || !k || !v || !out || !strides) return SWA_ERR_INVALID_ARG;
    if (!positive(B) || !positive(H) || !positive(T) || !positive(D) || !positive(W))
        return SWA_ERR_INVALID_ARG;
    for (int i = 0; i < 12; ++i)
        if (strides[i] < 0) return SWA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return SWA_ERR_INVALID_ARG;
    if (!fits(B, H, T, D)) return SWA_ERR_UNSUPPORTED;
    swa::Layout L;
    swa::Strides* dst[4] = {&L.q, &L.k, &L.v, &L.o};
    for (int i = 0; i < 4; ++i) *dst[i] = {strides[3 * i], strides[3 * i + 1], strides[3 * i + 2]};
    return forward(q, k, v, out, B, H, T, D, W, L, scale, dtype, (hipStream_t)stream);
}

int swa_decode(const void* q, const void* kring, const void* vring, const int64_t* pos, void* out,
               int64_t S, int64_t H, int64_t D, int64_t W, int dtype, void* stream) {
    if (!q || !kring || !vring || !pos || !out) return SWA_ERR_INVALID_ARG;
    if (!positive(S) || !positive(H) || !positive(D) || !positive(W)) return SWA_ERR_INVALID_ARG;
    if (!fits(S, H, W, D) || S * H >= ((int64_t)1 << 31)) return SWA_ERR_UNSUPPORTED;
    hipStream_t st = (hipStream_t)stream;
    if (dtype == SWA_BF16) {
        if (D != 64 && D != 128) return SWA_ERR_UNSUPPORTED;
        if (W <= swa::kDecodeMaxW)
            return from_hip(swa::launch_decode_bf16((const swa::bf16*)q, (const swa::bf16*)kring,
                                                    (const swa::bf16*)vring, pos, (swa::bf16*)out,
                                                    S, H, (int)D, W, nullptr, nullptr, nullptr,
                                                    st));
        return from_hip(swa::launch_rowwise_decode<swa::bf16>(
            (const swa::bf16*)q, (const swa::bf16*)kring, (const swa::bf16*)vring, pos,
            (swa::bf16*)out, S, H, (int)D, W, st));
    }
    if (dtype == SWA_F32) {
        if (D > kMaxRowD) return SWA_ERR_UNSUPPORTED;
        if (swa::decode_f32_supports(q, kring, vring, out, nullptr, nullptr, D, W))
            return from_hip(swa::launch_decode_f32((const float*)q, (const float*)kring,
                                                   (const float*)vring, pos, (float*)out, S, H,
                                                   (int)D, W, nullptr, nullptr, nullptr, st));
        return from_hip(swa::launch_rowwise_decode<float>((const float*)q, (const float*)kring,
                                                          (const float*)vring, pos, (float*)out, S,
                                                          H, (int)D, W, st));
    }
    return SWA_ERR_UNSUPPORTED;
}

int64_t swa_backward_workspace_bytes(int64_t B, int64_t H, int64_t T) {
    if (!positive(B) || !positive(H) || !positive(T)) return -SWA_ERR_INVALID_ARG;
    if (!fits(B, H, T, 8)) return -SWA_ERR_UNSUPPORTED;
    return B * H * T * 2 * (int64_t)sizeof(float);
}

int swa_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H,
                 int64_t T, int64_t D, int64_t W, double scale, int dtype, void* workspace,
                 int64_t workspace_bytes, void* stream) {
    if (!q || !k || !v || !out || !dout || !dq || !dk || !dv || !workspace)
        return SWA_ERR_INVALID_ARG;
    if (!positive(B) || !positive(H) || !positive(T) || !positive(D) || !positive(W))
        return SWA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || workspace_bytes < 0) return SWA_ERR_INVALID_ARG;
    if (!fits(B, H, T, D) || B * H * T >= ((int64_t)1 << 31)) return SWA_ERR_UNSUPPORTED;
    if (dtype != SWA_F32 && dtype != SWA_BF16) return SWA_ERR_UNSUPPORTED;
    if (D > kMaxRowD) return SWA_ERR_UNSUPPORTED;
    const int64_t need = swa_backward_workspace_bytes(B, H, T);
    if (workspace_bytes < need || ((uintptr_t)workspace & 3) != 0) return SWA_ERR_INVALID_ARG;
    const float sc = scale == 0.0 ? 1.0f / sqrtf((float)D) : (float)scale;
    float* lse_ws = (float*)workspace;
    float* delta = lse_ws + B * H * T;
    hipStream_t st = (hipStream_t)stream;
    if (dtype == SWA_BF16 && swa::backward_bf16_supports(q, k, v, out, dout, T, D, scale) &&
        B * H * ((T + 127) / 128) < ((int64_t)1 << 31)) {
        using bf = swa::bf16;
        return from_hip(swa::launch_backward_bf16(
            (const bf*)q, (const bf*)k, (const bf*)v, (const bf*)out, (const bf*)dout, (bf*)dq,
            (bf*)dk, (bf*)dv, lse, lse_ws, delta, B, H, T, (int)D, W, sc, st));
    }
    if (dtype == SWA_BF16) {
        using bf = swa::bf16;
        return from_hip(swa::launch_rowwise_backward<bf>(
            (const bf*)q, (const bf*)k, (const bf*)v, (const bf*)out, (const bf*)dout, (bf*)dq,
            (bf*)dk, (bf*)dv, lse_ws, delta, B, H, T, (int)D, W, sc, st));
    }
    if (swa::backward_f32_supports(q, k, v, out, dout, dq, dk, dv, T, D))
        return from_hip(swa::launch_backward_f32(
            (const float*)q, (const float*)k, (const float*)v, (const float*)out,
            (const float*)dout, (float*)dq, (float*)dk, (float*)dv, lse, lse_ws, delta, B, H, T,
            (int)D, W, sc, st));
    return from_hip(swa::launch_rowwise_backward<float>(
        (const float*)q, (const float*)k, (const float*)v, (const float*)out, (const float*)dout,
        (float*)dq, (float*)dk, (float*)dv, lse_ws, delta, B, H, T, (int)D, W, sc, st));
}

int64_t swa_decode_workspace_bytes(int64_t S, int64_t H, int64_t D, int64_t W, int dtype) {
    if (!positive(S) || !positive(H) || !positive(D) || !positive(W)) return -SWA_ERR_INVALID_ARG;
    if (!fits(S, H, W, D)) return -SWA_ERR_UNSUPPORTED;
    if (W > swa::kDecodeMaxW) return 0;
    if (dtype == SWA_BF16 && (D == 64 || D == 128)) return swa::decode_workspace_bytes(S, H, D, W);
    if (dtype == SWA_F32 && (D == 32 || D == 64 || D == 128))
        return swa::decode_workspace_bytes(S, H, D, W);
    return 0;
}

namespace {

// Shared checks of the workspace-taking decode entries; returns SWA_OK or a
// status, and sets *split when the split-window kernel applies (bf16; fp32
// with the alignment decode_f32_supports asks for, knew / vnew included).
int check_decode_ws(const void* q, const void* kring, const void* vring, const void* out,
                    const void* knew, const void* vnew, int64_t S, int64_t H, int64_t D,
                    int64_t W, int dtype, const void* ws, int64_t ws_bytes, bool* split) {
    if (!positive(S) || !positive(H) || !positive(D) || !positive(W)) return SWA_ERR_INVALID_ARG;
    if (ws_bytes < 0) return SWA_ERR_INVALID_ARG;
    if (!fits(S, H, W, D) || S * H * swa::kDecMaxSplits >= ((int64_t)1 << 31))
        return SWA_ERR_UNSUPPORTED;
    if (dtype != SWA_F32 && dtype != SWA_BF16) return SWA_ERR_UNSUPPORTED;
    if (dtype == SWA_BF16 && D != 64 && D != 128) return SWA_ERR_UNSUPPORTED;
    if (dtype == SWA_F32 && D > kMaxRowD) return SWA_ERR_UNSUPPORTED;
    const int64_t need = swa_decode_workspace_bytes(S, H, D, W, dtype);
    if (need > 0 && (!ws || ws_bytes < need || ((uintptr_t)ws & 15) != 0))
        return SWA_ERR_INVALID_ARG;
    *split = (dtype == SWA_BF16 && W <= swa::kDecodeMaxW) ||
             (dtype == SWA_F32 && swa::decode_f32_supports(q, kring, vring, out, knew, vnew, D, W));
    return SWA_OK;
}

}  // namespace

int swa_decode_split(const void* q, const void* kring, const void* vring, const int64_t* pos,
                     void* out, int64_t S, int64_t H, int64_t D, int64_t W, int dtype,
                     void* workspace, int64_t workspace_bytes, void* stream) {
    if (!q || !kring || !vring || !pos || !out) return SWA_ERR_INVALID_ARG;
    bool split = false;
    const int rc = check_decode_ws(q, kring, vring, out, nullptr, nullptr, S, H, D, W, dtype,
                                   workspace, workspace_bytes, &split);
    if (rc != SWA_OK) return rc;
    if (!split) return swa_decode(q, kring, vring, pos, out, S, H, D, W, dtype, stream);
    void* ws = swa_decode_workspace_bytes(S, H, D, W, dtype) > 0 ? workspace : nullptr;
    if (dtype == SWA_F32)
        return from_hip(swa::launch_decode_f32((const float*)q, (const float*)kring,
                                               (const float*)vring, pos, (float*)out, S, H,
                                               (int)D, W, nullptr, nullptr, ws,
                                               (hipStream_t)stream));
    return from_hip(swa::launch_decode_bf16(
        (const swa::bf16*)q, (const swa::bf16*)kring, (const swa::bf16*)vring, pos,
        (swa::bf16*)out, S, H, (int)D, W, nullptr, nullptr,
        swa_decode_workspace_bytes(S, H, D, W, dtype) > 0 ? workspace : nullptr,
        (hipStream_t)stream));
}

int swa_decode_append(const void* q, const void* knew, const void* vnew, void* kring, void* vring,
                      const int64_t* pos, void* out, int64_t S, int64_t H, int64_t D, int64_t W,
                      int dtype, void* workspace, int64_t workspace_bytes, void* stream) {
    if (!q || !knew || !vnew || !kring || !vring || !pos || !out) return SWA_ERR_INVALID_ARG;
    bool split = false;
    const int rc = check_decode_ws(q, kring, vring, out, knew, vnew, S, H, D, W, dtype, workspace,
                                   workspace_bytes, &split);
    if (rc != SWA_OK) return rc;
    if (!split) {
        // no fused kernel for this shape: append, then decode, in stream order
        const int r = swa_ring_append(knew, vnew, kring, vring, pos, S, H, D, W, dtype, stream);
        if (r != SWA_OK) return r;
        return swa_decode(q, kring, vring, pos, out, S, H, D, W, dtype, stream);
    }
    if (dtype == SWA_F32)
        return from_hip(swa::launch_decode_f32(
            (const float*)q, (const float*)kring, (const float*)vring, pos, (float*)out, S, H,
            (int)D, W, (const float*)knew, (const float*)vnew,
            swa_decode_workspace_bytes(S, H, D, W, dtype) > 0 ? workspace : nullptr,
            (hipStream_t)stream));
    return from_hip(swa::launch_decode_bf16(
        (const swa::bf16*)q, (const swa::bf16*)kring, (const swa::bf16*)vring, pos,
        (swa::bf16*)out, S, H, (int)D, W, (const swa::bf16*)knew, (const swa::bf16*)vnew,
        swa_decode_workspace_bytes(S, H, D, W, dtype) > 0 ? workspace : nullptr,
        (hipStream_t)stream));
}

int swa_ring_append(const void* knew, const void* vnew, void* kring, void* vring,
                    const int64_t* pos, int64_t S, int64_t H, int64_t D, int64_t W, int dtype,
                    void* stream) {
    if (!knew || !vnew || !kring || !vring || !pos) return SWA_ERR_INVALID_ARG;
    if (!positive(S) || !positive(H) || !positive(D) || !positive(W)) return SWA_ERR_INVALID_ARG;
    if (!fits(S, H, W, D) || S * H >= ((int64_t)1 << 31)) return SWA_ERR_UNSUPPORTED;
    if (dtype != SWA_F32 && dtype != SWA_BF16) return SWA_ERR_UNSUPPORTED;
    return from_hip(swa::launch_ring_append(knew, vnew, kring, vring, pos, S, H, D, W,
                                            dtype == SWA_F32 ? 4 : 2, (hipStream_t)stream));
}

int64_t swa_chunk_workspace_bytes(int64_t S, int64_t H, int64_t C, int64_t D, int64_t W,
                                  int dtype) {
    if (!positive(S) || !positive(H) || !positive(C) || !positive(D) || !positive(W))
        return -SWA_ERR_INVALID_ARG;
    if (!fits(S, H, C, D) || !fits(S, H, W, D)) return -SWA_ERR_UNSUPPORTED;
    if (dtype != SWA_BF16 || (D != 64 && D != 128)) return 0;
    return swa::chunk_workspace_bytes(S, H, C, D, W);
}

namespace {

int chunk_forward(const void* q, const void* kc, const void* vc, const void* kring,
                  const void* vring, const int64_t* pos0, void* out, int64_t S, int64_t H,
                  int64_t C, int64_t D, int64_t W, int dtype, void* workspace, void* stream);

}  // namespace

int swa_chunk_forward(const void* q, const void* kc, const void* vc, const void* kring,
                      const void* vring, const int64_t* pos0, void* out, int64_t S, int64_t H,
                      int64_t C, int64_t D, int64_t W, int dtype, void* stream) {
    return chunk_forward(q, kc, vc, kring, vring, pos0, out, S, H, C, D, W, dtype, nullptr,
                         stream);
}

int swa_chunk_forward_split(const void* q, const void* kc, const void* vc, const void* kring,
                            const void* vring, const int64_t* pos0, void* out, int64_t S,
                            int64_t H, int64_t C, int64_t D, int64_t W, int dtype,
                            void* workspace, int64_t workspace_bytes, void* stream) {
    if (workspace_bytes < 0) return SWA_ERR_INVALID_ARG;
    const int64_t need = swa_chunk_workspace_bytes(S, H, C, D, W, dtype);
    if (need < 0) return (int)-need;
    if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 15) != 0))
        return SWA_ERR_INVALID_ARG;
    return chunk_forward(q, kc, vc, kring, vring, pos0, out, S, H, C, D, W, dtype,
                         need > 0 ? workspace : nullptr, stream);
}

namespace {

int chunk_forward(const void* q, const void* kc, const void* vc, const void* kring,
                  const void* vring, const int64_t* pos0, void* out, int64_t S, int64_t H,
                  int64_t C, int64_t D, int64_t W, int dtype, void* workspace, void* stream) {
    if (!q || !kc || !vc || !kring || !vring || !pos0 || !out) return SWA_ERR_INVALID_ARG;
    if (!positive(S) || !positive(H) || !positive(C) || !positive(D) || !positive(W))
        return SWA_ERR_INVALID_ARG;
    if (!fits(S, H, C, D) || !fits(S, H, W, D) || S * H * C >= ((int64_t)1 << 31))
        return SWA_ERR_UNSUPPORTED;
    if (D > kMaxRowD) return SWA_ERR_UNSUPPORTED;
    hipStream_t st = (hipStream_t)stream;
    if (dtype == SWA_BF16 && swa::chunk_bf16_supports(q, kc, vc, kring, vring, out, C, D, W) &&
        S * H * ((C + 127) / 128) < ((int64_t)1 << 31))
        return from_hip(swa::launch_chunk_bf16(
            (const swa::bf16*)q, (const swa::bf16*)kc, (const swa::bf16*)vc,
            (const swa::bf16*)kring, (const swa::bf16*)vring, pos0, (swa::bf16*)out, S, H, C,
            (int)D, W, workspace, st));
    if (dtype == SWA_BF16)
        return from_hip(swa::launch_rowwise_chunk<swa::bf16>(
            (const swa::bf16*)q, (const swa::bf16*)kc, (const swa::bf16*)vc,
            (const swa::bf16*)kring, (const swa::bf16*)vring, pos0, (swa::bf16*)out, S, H, C,
            (int)D, W, st));
    if (dtype == SWA_F32 && swa::chunk_f32_supports(q, kc, vc, kring, vring, out, C, D, W))
        return from_hip(swa::launch_chunk_f32((const float*)q, (const float*)kc,
                                              (const float*)vc, (const float*)kring,
                                              (const float*)vring, pos0, (float*)out, S, H, C,
                                              (int)D, W, st));
    if (dtype == SWA_F32)
        return from_hip(swa::launch_rowwise_chunk<float>((const float*)q, (const float*)kc,
                                                         (const float*)vc, (const float*)kring,
                                                         (const float*)vring, pos0, (float*)out, S,
                                                         H, C, (int)D, W, st));
    return SWA_ERR_UNSUPPORTED;
}

}  // namespace

int swa_ring_append_chunk(const void* kc, const void* vc, void* kring, void* vring,
                          const int64_t* pos0, int64_t S, int64_t H, int64_t C, int64_t D,
                          int64_t W, int dtype, void* stream) {
    if (!kc || !vc || !kring || !vring || !pos0) return SWA_ERR_INVALID_ARG;
    if (!positive(S) || !positive(H) || !positive(C) || !positive(D) || !positive(W))
        return SWA_ERR_INVALID_ARG;
    if (!fits(S, H, C, D) || !fits(S, H, W, D) || S * H >= ((int64_t)1 << 31))
        return SWA_ERR_UNSUPPORTED;
    if (dtype != SWA_F32 && dtype != SWA_BF16) return SWA_ERR_UNSUPPORTED;
    return from_hip(swa::launch_ring_append_chunk(kc, vc, kring, vring, pos0, S, H, C, D, W,
                                                  dtype == SWA_F32 ? 4 : 2, (hipStream_t)stream));
}

}  // extern "C"
