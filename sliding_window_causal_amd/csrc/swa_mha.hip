// Multi-head sliding-window self-attention module forward ("NNX Sliding-
// Window Attention", A complete example with moving averages: q, k, v and
// output projections around the banded attention).
//
// The four projections are plain GEMMs and go to rocBLAS (bf16 or fp32
// operands, fp32 accumulation).  Their bias is written into the output
// first and the GEMM accumulates onto it (beta = 1).  The q, k and v
// projections write side by side into one [B*T, 3 d_model] workspace, which
// the banded attention reads in place as three strided [B, H, T, Dh] views;
// the attention writes [B*T, d_model] (heads side by side, the concatenation
// of the page's module), which the output projection consumes.

#include "../../include/swa.h"
#include "swa_internal.h"

#include <rocblas/rocblas.h>

#include <mutex>

namespace {

constexpr int kMaxDevices = 64;

// One rocBLAS handle per device, created on first use and kept until the
// process ends (the library's only state besides cached device properties).
// A handle carries the stream its calls go to, so a caller holds the
// device's lock (taken here) from setting the stream until its last rocBLAS
// call has been issued: module calls on other host threads and streams then
// cannot redirect its products.  Launches are asynchronous, so the lock is
// held only for the time it takes to issue them.
struct LockedHandle {
    std::unique_lock<std::mutex> lock;
    rocblas_handle h = nullptr;
};

LockedHandle device_handle() {
    static std::mutex create_mu;
    static std::mutex use_mu[kMaxDevices];
    static rocblas_handle handles[kMaxDevices] = {};
    LockedHandle r;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return r;
    rocblas_handle h = nullptr;
    {
        std::lock_guard<std::mutex> lock(create_mu);
        if (!handles[dev] && rocblas_create_handle(&handles[dev]) != rocblas_status_success)
            handles[dev] = nullptr;
        h = handles[dev];
    }
    if (h) {
        r.lock = std::unique_lock<std::mutex>(use_mu[dev]);
        r.h = h;
    }
    return r;
}

// C[r, c] = bias[c] (0 without a bias) for r < rows, c < cols; row stride ldc.
template <typename T>
__global__ __launch_bounds__(256) void fill_bias_kernel(T* __restrict__ C,
                                                        const T* __restrict__ bias, int64_t rows,
                                                        int64_t cols, int64_t ldc) {
    const int64_t n = rows * cols;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / cols, c = i - r * cols;
        C[r * ldc + c] = bias ? bias[c] : T(0.f);
    }
}

template <typename T>
hipError_t fill_bias(void* C, const void* bias, int64_t rows, int64_t cols, int64_t ldc,
                     hipStream_t st) {
    const int64_t n = rows * cols;
    const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    T* c = (T*)C;
    const T* b = (const T*)bias;
    void* args[] = {(void*)&c, (void*)&b, (void*)&rows, (void*)&cols, (void*)&ldc};
    return hipLaunchKernel((const void*)fill_bias_kernel<T>, dim3((unsigned)blocks), dim3(256),
                           args, 0, st);
}

// Row-major C[rows, N] += A[rows, K] @ B[K, N] (leading dimensions lda, ldb,
// ldc in elements), as the column-major product C^T = B^T A^T.
rocblas_status gemm_acc(rocblas_handle h, int dtype, const void* A, int64_t lda, const void* B,
                        int64_t ldb, void* C, int64_t ldc, int64_t rows, int64_t N, int64_t K) {
    const float one = 1.f;
    const rocblas_datatype t = dtype == SWA_BF16 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r;
    return rocblas_gemm_ex(h, rocblas_operation_none, rocblas_operation_none, (rocblas_int)N,
                           (rocblas_int)rows, (rocblas_int)K, &one, B, t, (rocblas_int)ldb, A, t,
                           (rocblas_int)lda, &one, C, t, (rocblas_int)ldc, C, t, (rocblas_int)ldc,
                           rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
}

int64_t elem_bytes(int dtype) { return dtype == SWA_BF16 ? 2 : 4; }

}  // namespace

extern "C" {

int64_t swa_mha_workspace_bytes(int64_t B, int64_t T, int64_t d_model, int dtype) {
    if (B < 1 || T < 1 || d_model < 1) return -SWA_ERR_INVALID_ARG;
    if (dtype != SWA_F32 && dtype != SWA_BF16) return -SWA_ERR_UNSUPPORTED;
    if (B > ((int64_t)1 << 40) / T || B * T > ((int64_t)1 << 40) / (4 * d_model))
        return -SWA_ERR_UNSUPPORTED;
    // q | k | v side by side, then the attention output
    return B * T * 4 * d_model * elem_bytes(dtype);
}

int swa_mha_forward(const void* x, const void* wq, const void* bq, const void* wk, const void* bk,
                    const void* wv, const void* bv, const void* wo, const void* bo, void* out,
                    int64_t B, int64_t T, int64_t d_model, int64_t H, int64_t W, int dtype,
                    void* workspace, int64_t workspace_bytes, void* stream) {
    if (!x || !wq || !wk || !wv || !wo || !out || !workspace) return SWA_ERR_INVALID_ARG;
    if (B < 1 || T < 1 || d_model < 1 || H < 1 || W < 1 || workspace_bytes < 0)
        return SWA_ERR_INVALID_ARG;
    if (d_model % H != 0) return SWA_ERR_INVALID_ARG;
    if (dtype != SWA_F32 && dtype != SWA_BF16) return SWA_ERR_UNSUPPORTED;
    const int64_t dh = d_model / H;
    if (dtype == SWA_BF16 && dh != 64 && dh != 128) return SWA_ERR_UNSUPPORTED;
    if (dtype == SWA_F32 && dh > 256) return SWA_ERR_UNSUPPORTED;
    const int64_t need = swa_mha_workspace_bytes(B, T, d_model, dtype);
    if (need < 0) return (int)-need;
    // rocBLAS takes 32-bit sizes and leading dimensions
    const int64_t rows = B * T;
    if (rows >= ((int64_t)1 << 31) || 3 * d_model >= ((int64_t)1 << 31)) return SWA_ERR_UNSUPPORTED;
    if (workspace_bytes < need || ((uintptr_t)workspace & 15) != 0) return SWA_ERR_INVALID_ARG;

    hipStream_t st = (hipStream_t)stream;
    LockedHandle lh = device_handle();   // held until this call returns
    rocblas_handle h = lh.h;
    if (!h || rocblas_set_stream(h, st) != rocblas_status_success) return SWA_ERR_LAUNCH;
    const int64_t eb = elem_bytes(dtype);
    char* qkv = (char*)workspace;                       // [rows, 3 d_model]
    char* att = qkv + rows * 3 * d_model * eb;          // [rows, d_model]
    auto fill = dtype == SWA_BF16 ? fill_bias<swa::bf16> : fill_bias<float>;

    const void* w3[3] = {wq, wk, wv};
    const void* b3[3] = {bq, bk, bv};
    for (int i = 0; i < 3; ++i) {
        char* dst = qkv + i * d_model * eb;
        if (fill(dst, b3[i], rows, d_model, 3 * d_model, st) != hipSuccess) return SWA_ERR_LAUNCH;
        if (gemm_acc(h, dtype, x, d_model, w3[i], d_model, dst, 3 * d_model, rows, d_model,
                     d_model) != rocblas_status_success)
            return SWA_ERR_LAUNCH;
    }
    // q, k, v as [B, H, T, Dh] views of the packed projections; the output
    // as a [B, H, T, Dh] view of [B, T, d_model]
    const int64_t s3[3] = {T * 3 * d_model, dh, 3 * d_model};
    const int64_t strides[12] = {s3[0], s3[1], s3[2], s3[0], s3[1], s3[2],
                                 s3[0], s3[1], s3[2], T * d_model, dh, d_model};
    const int rc = swa_forward_strided(qkv, qkv + d_model * eb, qkv + 2 * d_model * eb, att, B, H,
                                       T, dh, W, strides, 0.0, dtype, stream);
    if (rc != SWA_OK) return rc;
    if (fill(out, bo, rows, d_model, d_model, st) != hipSuccess) return SWA_ERR_LAUNCH;
    if (gemm_acc(h, dtype, att, d_model, wo, d_model, out, d_model, rows, d_model, d_model) !=
        rocblas_status_success)
        return SWA_ERR_LAUNCH;
    return SWA_OK;
}

}  // extern "C"
