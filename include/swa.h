/*
 * swa.h -- C ABI of libswa, causal sliding-window attention for AMD gfx950.
 *
 * Operation.  For every query position i, attention over the W most recent
 * keys including i itself:
 *
 *     out[i] = sum_{j in J(i)} softmax_j( q[i] . k[j] / sqrt(D) ) v[j],
 *     J(i)   = { j : j <= i  and  i - j < W }.
 *
 * This is the band of "27. Sliding-Window Attention" (Step-by-Step Approach,
 * step 2), "25. Sliding-Window Causal Attention for Streaming Inference"
 * (step 3: a strict lower bound j > i - W), "Implementation: Sliding Window
 * Attention" (Step 1, the printed 8-token mask) and "NNX Sliding-Window
 * Attention" (Build the band by index difference).  W >= T is ordinary causal
 * attention; W = 1 returns v.  The scale is 1/sqrt(D) as on every page.
 *
 * Conventions shared by every entry point:
 *  - All tensors are device memory, dense and row-major (C-contiguous) in the
 *    stated layout; element type is the `dtype` argument (SWA_F32 = float,
 *    SWA_BF16 = bfloat16).  Output has the input dtype.
 *  - The caller owns every buffer.  The library never allocates, frees or
 *    synchronises; it keeps no state beyond cached device attributes and the
 *    static device scratch array of swa_decode_split_noalloc.
 *  - `out` must not alias any input.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  A launch failure returns SWA_ERR_LAUNCH; faults surface when
 *    the caller synchronises.
 *  - Argument errors are reported before any HIP call: SWA_ERR_INVALID_ARG for
 *    a NULL pointer, a size < 1, or W < 1 (a positive window keeps the
 *    diagonal, so no row is ever fully masked: "NNX Sliding-Window
 *    Attention", Mask before softmax); SWA_ERR_UNSUPPORTED for a dtype or
 *    head size the kernels do not cover.
 *  - Sizes are int64_t; element offsets are computed in 64 bits.
 */
#ifndef SWA_H
#define SWA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SWA_F32 = 0,   /* IEEE binary32 */
    SWA_BF16 = 1   /* bfloat16, rounded to nearest even on output */
} swa_dtype_t;

typedef enum {
    SWA_OK = 0,
    SWA_ERR_INVALID_ARG = 1,
    SWA_ERR_UNSUPPORTED = 2,
    SWA_ERR_LAUNCH = 3,
    SWA_ERR_SCRATCH_LIMIT = 4   /* swa_decode_split_noalloc: sizes need more than its static scratch */
} swa_status_t;

/* Version of this ABI (bumped on any signature or semantic change). */
int swa_abi_version(void);

/* Human-readable text for a status code (static storage, never NULL). */
const char* swa_status_string(int status);

/*
 * Prefill: out = band attention of q, k, v.
 *
 *   q, k, v, out : [B, H, T, D]  (the (batch, heads, seq, head_dim) layout of
 *                  "27. Sliding-Window Attention", Reference solution)
 *   W            : window in keys including the query itself (W >= 1)
 *   dtype        : SWA_BF16 needs D in {64, 128}; SWA_F32 takes 1 <= D <= 256.
 *                  B * H * T < 2^31 for either (else SWA_ERR_UNSUPPORTED).  bf16
 *                  runs on the matrix cores when each (b, h) slab of k and v is
 *                  under 2 GiB (T * D < 2^30 here) and every pointer is 16-byte
 *                  aligned, otherwise on the (slower) row kernel.
 *
 * Work is O(B * H * T * min(W, T) * D): only key tiles that intersect a
 * query tile's band are read ("NNX Sliding-Window Attention", A local mask is
 * not a sparse implementation).
 */
int swa_forward(const void* q, const void* k, const void* v, void* out,
                int64_t B, int64_t H, int64_t T, int64_t D, int64_t W,
                int dtype, void* stream);

/*
 * Prefill as swa_forward, with an explicit scale (0 selects 1 / sqrt(D)),
 * also writing each row's log-sum-exp of its scaled scores,
 *   lse[(b * H + h) * T + i] = ln(sum over the row's band of exp(s_ij)),
 * s_ij = q_i . k_j * scale: the softmax normaliser of "Implementation:
 * Sliding Window Attention", Step 2, that swa_backward can take instead of
 * recomputing it.
 *
 *   lse : device float[B * H * T], written; other arguments as swa_forward
 * Returns SWA_ERR_INVALID_ARG also for a null lse or a non-finite scale.
 */
int swa_forward_lse(const void* q, const void* k, const void* v, void* out, float* lse,
                    int64_t B, int64_t H, int64_t T, int64_t D, int64_t W, double scale,
                    int dtype, void* stream);

/*
 * Prefill with arbitrary strides and an optional score scale: the layouts of
 * "Implementation: Sliding Window Attention", Step 2 (queries, keys and
 * values as (batch, seq_len, num_heads, head_dim), and its scale argument
 * that defaults to 1 / sqrt(head_dim)) and of "25. Sliding-Window Causal
 * Attention for Streaming Inference" ((batch, seq_len, d_model), one head),
 * without copies.  The computation is that of swa_forward with the scores
 * multiplied by `scale` instead of divided by sqrt(D).
 *
 *   q, k, v, out : logical [B, H, T, D]; element (b, h, t, d) of tensor X
 *                  sits at X + b * sb + h * sh + t * st + d, elements of dtype
 *   strides      : host int64[12] = {q_sb, q_sh, q_st, k_sb, k_sh, k_st,
 *                  v_sb, v_sh, v_st, out_sb, out_sh, out_st}, in elements,
 *                  each >= 0 (0 broadcasts, e.g. one key/value head shared
 *                  by all query heads).  Read during the call only.
 *   scale        : finite; 0 selects 1 / sqrt(D)
 *   dtype        : as swa_forward.  bf16 with 16-byte aligned pointers,
 *                  strides that are multiples of 8, k/v row strides >= D and
 *                  k/v (batch, head) slabs under 2 GiB runs on the matrix
 *                  cores; other bf16 layouts run on the row-wise kernel.
 *   out must not overlap itself or an input.
 * Returns SWA_ERR_INVALID_ARG also for a null `strides`, a negative stride
 * or a non-finite scale.
 */
int swa_forward_strided(const void* q, const void* k, const void* v, void* out, int64_t B,
                        int64_t H, int64_t T, int64_t D, int64_t W, const int64_t* strides,
                        double scale, int dtype, void* stream);

/*
 * Decode: one query per stream against a bounded W-slot ring of keys/values
 * (the bounded cache that drops anything older than the window,
 * "25. Sliding-Window Causal Attention for Streaming Inference", Problem; a
 * KV cache of size W, "Sliding Window Attention", Key Advantages).
 *
 *   q, out       : [S, H, D]
 *   kring, vring : [S, H, W, D]; the token at absolute position p lives in
 *                  slot p mod W
 *   pos          : device int64[S]; absolute position of each stream's
 *                  current query, whose own k/v are already in the ring.  The
 *                  visible keys are the occupied slots [0, min(pos + 1, W)),
 *                  i.e. tokens (pos - W, pos], so the result equals prefill
 *                  row pos.  Unoccupied slots are never read.  pos < 0 is
 *                  outside the contract: the kernel stays in bounds and writes
 *                  zeros for that stream.
 *   dtype        : SWA_BF16 needs D in {64, 128}; SWA_F32 takes 1 <= D <= 256
 */
int swa_decode(const void* q, const void* kring, const void* vring,
               const int64_t* pos, void* out,
               int64_t S, int64_t H, int64_t D, int64_t W,
               int dtype, void* stream);

/*
 * Bytes of device workspace that swa_decode_split and swa_decode_append need
 * for these sizes (0: none), or a negative status (-SWA_ERR_INVALID_ARG for
 * sizes < 1, -SWA_ERR_UNSUPPORTED for sizes too large to address).  The
 * amount depends on the sizes and dtype only.
 */
int64_t swa_decode_workspace_bytes(int64_t S, int64_t H, int64_t D, int64_t W, int dtype);

/*
 * Decode as swa_decode, for few streams: when S * H workgroups would leave
 * most of the GPU idle, each (stream, head)'s occupied slots are split over
 * several workgroups that write partial (max, sum, unnormalised output)
 * triples to `workspace`, and a second kernel merges them by rescaling each
 * partial to the largest max (the running-max identity of the stable
 * softmax in "Implementation: Sliding Window Attention", Step 2, applied to
 * slot ranges instead of single keys).  Same result as swa_decode up to
 * rounding order.
 *
 *   workspace       : device memory of at least swa_decode_workspace_bytes()
 *                     bytes, 16-byte aligned, owned by the caller; may be
 *                     null when that size is 0.  Contents on entry are
 *                     ignored; concurrent calls need separate workspaces.
 *   workspace_bytes : its size; too small (or null when needed) returns
 *                     SWA_ERR_INVALID_ARG.
 * Other arguments, layouts and dtypes as swa_decode.  bf16 (D in {64, 128})
 * and fp32 with D in {32, 64, 128} and 16-byte aligned pointers split;
 * other fp32 shapes, and windows over 16384 slots, run swa_decode's kernels
 * and use no workspace.
 */
int swa_decode_split(const void* q, const void* kring, const void* vring, const int64_t* pos,
                     void* out, int64_t S, int64_t H, int64_t D, int64_t W, int dtype,
                     void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Append and decode in one launch: the current token's knew, vnew
 * ([S, H, D]) go into ring slot pos mod W, as swa_ring_append does, and its
 * query q attends to the ring including that token, as swa_decode does after
 * the append (the bounded cache that evicts what falls out of the window,
 * "25. Sliding-Window Causal Attention for Streaming Inference", Problem).
 * The attention reads the current token from knew / vnew rather than from
 * the slot being written, so the result does not depend on write ordering.
 *
 *   kring, vring : [S, H, W, D], written at slot pos[s] mod W of each stream
 *   workspace    : as swa_decode_split
 * A negative pos[s] writes slot pos mod W reduced into [0, W), as
 * swa_ring_append does, and gives a zero output (no occupied slots).
 * Shapes that do not split (see swa_decode_split; for fp32 also unaligned
 * knew / vnew) run the append kernel and then swa_decode's kernels, in
 * stream order.
 */
int swa_decode_append(const void* q, const void* knew, const void* vnew, void* kring, void* vring,
                      const int64_t* pos, void* out, int64_t S, int64_t H, int64_t D, int64_t W,
                      int dtype, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Decode as swa_decode_split, allocating nothing: for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  The split's
 * partial results live in a static device array of
 * SWA_NOALLOC_SCRATCH_BYTES bytes inside the library, one copy per GPU, held
 * until the process ends; it covers every size swa_decode_workspace_bytes()
 * asks for (at most about 1.3 MiB: the split stops at 512 (stream, head)
 * pairs and 2048 workgroups).  Same kernels and bit-identical results as
 * swa_decode_split with a workspace of its own.
 *
 *   arguments    : as swa_decode_split without the workspace; `stream` must
 *                  belong to the GPU that holds q, the rings and out
 * Calls that overlap on one GPU (concurrent streams, or threads) share that
 * GPU's array and race: serialise them.  Nothing needs to be zero on entry.
 * Returns SWA_ERR_SCRATCH_LIMIT (before any HIP call) if the sizes would
 * need more than SWA_NOALLOC_SCRATCH_BYTES, and SWA_ERR_LAUNCH if the
 * array's device address cannot be found.
 */
#define SWA_NOALLOC_SCRATCH_BYTES (2 * 1024 * 1024)
int swa_decode_split_noalloc(const void* q, const void* kring, const void* vring,
                             const int64_t* pos, void* out, int64_t S, int64_t H, int64_t D,
                             int64_t W, int dtype, void* stream);

/*
 * Ring append (not part of the timed path): for every stream s and head h,
 * kring[s, h, pos[s] mod W, :] = knew[s, h, :] and the same for v.
 *
 *   knew, vnew   : [S, H, D];  kring, vring : [S, H, W, D];  pos : device int64[S]
 *   dtype        : SWA_F32 or SWA_BF16, any D >= 1
 * A negative pos is reduced into [0, W) (the kernel never writes outside
 * the ring).
 */
int swa_ring_append(const void* knew, const void* vnew, void* kring, void* vring,
                    const int64_t* pos, int64_t S, int64_t H, int64_t D, int64_t W,
                    int dtype, void* stream);

/*
 * Chunked prefill continuing a stream held in a W-slot ring (the rolling
 * buffer that "27. Sliding-Window Attention", Problem, names as the follow-up
 * to the dense version; the bounded cache of "25. Sliding-Window Causal
 * Attention for Streaming Inference", Problem).  C new tokens per stream sit
 * at absolute positions pos0[s] .. pos0[s] + C - 1; the ring holds the
 * stream's earlier tokens (pos0 - W, pos0) in slots p mod W (slots of
 * negative positions are never read).  Query p attends to the tokens
 * (p - W, p]: those before pos0 from the ring, the rest from the chunk, so
 * the result equals prefill rows pos0 .. pos0 + C - 1 of the whole sequence.
 *
 *   q, kc, vc, out : [S, H, C, D]
 *   kring, vring   : [S, H, W, D]  read only
 *   pos0           : device int64[S], >= 0 (negative values are treated as 0)
 *   dtype          : SWA_F32 or SWA_BF16, 1 <= D <= 256
 * Append the chunk afterwards with swa_ring_append_chunk (the attention of
 * the chunk still needs ring slots the append overwrites).
 */
int swa_chunk_forward(const void* q, const void* kc, const void* vc,
                      const void* kring, const void* vring, const int64_t* pos0,
                      void* out, int64_t S, int64_t H, int64_t C, int64_t D, int64_t W,
                      int dtype, void* stream);

/*
 * Chunk continuation as swa_chunk_forward, for few streams: when the
 * S * H * ceil(C / 128) workgroups of the matrix-core kernel would leave most
 * of the GPU idle, each query tile's key range is split over several
 * workgroups that write partial (max, sum, unnormalised output) rows to
 * `workspace`, merged by a second kernel (the running-max identity of the
 * stable softmax, "Implementation: Sliding Window Attention", Step 2).
 *
 *   workspace       : device memory of swa_chunk_workspace_bytes() bytes,
 *                     16-byte aligned, owned by the caller; may be null when
 *                     that size is 0 (no split applies; then this call is
 *                     swa_chunk_forward).  Concurrent calls need separate
 *                     workspaces.
 *   workspace_bytes : its size; too small returns SWA_ERR_INVALID_ARG.
 * The size query returns a negative status for invalid or oversized sizes.
 */
int64_t swa_chunk_workspace_bytes(int64_t S, int64_t H, int64_t C, int64_t D, int64_t W,
                                  int dtype);
int swa_chunk_forward_split(const void* q, const void* kc, const void* vc, const void* kring,
                            const void* vring, const int64_t* pos0, void* out, int64_t S,
                            int64_t H, int64_t C, int64_t D, int64_t W, int dtype,
                            void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Chunk append (not part of the timed path): the last min(C, W) tokens of
 * the chunk, at positions pos0 + c, go to ring slots (pos0 + c) mod W.
 *
 *   kc, vc : [S, H, C, D];  kring, vring : [S, H, W, D]
 *   pos0   : device int64[S], >= 0 (negative values are treated as 0)
 *   dtype  : SWA_F32 or SWA_BF16, any D >= 1
 */
int swa_ring_append_chunk(const void* kc, const void* vc, void* kring, void* vring,
                          const int64_t* pos0, int64_t S, int64_t H, int64_t C, int64_t D,
                          int64_t W, int dtype, void* stream);

/*
 * Backward of the prefill: gradients dq, dk, dv of a loss with respect to
 * q, k, v, given dout = d loss / d out.  The pages define the forward only;
 * "NNX Sliding-Window Attention", Mask before softmax, notes that masked
 * weights are zero and gradients stay well defined for finite allowed
 * scores.  With P = softmax over the band of S = q k^T * scale:
 *   dv = P^T dout, dS = P * (dout v^T - rowsum(dout * out)),
 *   dq = dS k * scale, dk = dS^T q * scale.
 *
 *   q, k, v, out, dout, dq, dk, dv : [B, H, T, D] contiguous, one dtype;
 *                    out must be swa_forward's output for q, k, v, W, scale
 *   lse            : NULL, or swa_forward_lse's lse for the same call; the
 *                    matrix-core path then skips rerunning the forward
 *   scale          : finite; 0 selects 1 / sqrt(D)
 *   dtype          : SWA_F32 or SWA_BF16 (fp32 accumulation), 1 <= D <= 256
 *   workspace      : device memory of swa_backward_workspace_bytes() bytes
 *                    (per-row log normaliser and delta), 4-byte aligned,
 *                    owned by the caller
 * bf16 with D in {64, 128} and 16-byte aligned pointers runs on the matrix
 * cores.  There delta_i = dout_i . out_i at scales up to 1 / sqrt(D) in
 * magnitude; for a sharper softmax (|scale| sqrt(D) > 1.001) a first kernel
 * takes each row's sum of the rebuilt weights and delta_i = sum_j P_ij dP_ij
 * in fp32 (rows renormalised), and dS reaches the matrix cores as two bf16
 * terms, which keeps the gradients within the bf16 tolerance at any scale.
 * fp32 with D in {32, 64, 128} and 16-byte aligned pointers runs on the fp32
 * matrix cores (delta_i = dout_i . out_i).  Other shapes run row-wise
 * kernels (one wavefront per query row, then per key row; fp32 arithmetic,
 * delta as the band sum above).
 */
int64_t swa_backward_workspace_bytes(int64_t B, int64_t H, int64_t T);
int swa_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H,
                 int64_t T, int64_t D, int64_t W, double scale, int dtype, void* workspace,
                 int64_t workspace_bytes, void* stream);

/*
 * Multi-head sliding-window self-attention module, forward ("NNX
 * Sliding-Window Attention", A complete example with moving averages):
 *   q = x wq + bq, k = x wk + bk, v = x wv + bv   (x: [B, T, d_model])
 *   heads h of width Dh = d_model / H: o_h = swa(q_h, k_h, v_h, W) with
 *   scores divided by sqrt(Dh) (the computation of swa_forward)
 *   out = concat_h(o_h) wo + bo
 * The projections are plain GEMMs (rocBLAS, fp32 accumulation).
 *
 *   x, out          : [B, T, d_model]
 *   wq, wk, wv, wo  : [d_model, d_model], applied as x @ w (rows = input
 *                     features), row-major
 *   bq, bk, bv, bo  : [d_model] or NULL for a zero bias
 *   H               : heads, d_model % H == 0 (else SWA_ERR_INVALID_ARG);
 *                     bf16 needs Dh in {64, 128}, fp32 Dh <= 256
 *   workspace       : device memory of swa_mha_workspace_bytes() bytes,
 *                     16-byte aligned, owned by the caller (q, k, v and the
 *                     attention output live there)
 * All device pointers; dtype SWA_F32 or SWA_BF16 for every tensor.  Returns
 * SWA_ERR_LAUNCH also when rocBLAS fails.
 */
int64_t swa_mha_workspace_bytes(int64_t B, int64_t T, int64_t d_model, int dtype);
int swa_mha_forward(const void* x, const void* wq, const void* bq, const void* wk, const void* bk,
                    const void* wv, const void* bv, const void* wo, const void* bo, void* out,
                    int64_t B, int64_t T, int64_t d_model, int64_t H, int64_t W, int dtype,
                    void* workspace, int64_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SWA_H */
