/*
 * dsa.h -- C ABI of the sparse index selection in libfa.so (status codes and fa_last_error()
 * from fa.h).
 *
 * The operation is that of the onnx-runtime-ep-cuda page `src/kernels/dsa_index_select.rs`
 * (module documentation; shapes from the checks of its host code; attributes top_k, scale and
 * weights_scale):
 *
 *   for batch b, query row s, key position t:
 *     allowed(t) iff bias[b, 0, s, t] > -1e30   (a NaN bias is not allowed)
 *     score(t)   = sum_h relu(scale * dot_h) * (weights[b, s, h] * weights_scale) + bias[b, 0, s, t]
 *                  with dot_h = sum_d query[b, s, h, d] * key[b, t, d],
 *                  all in float32, the sums taken in ascending d, then ascending h, every product
 *                  and sum rounded on its own (no fused multiply-add); relu of NaN is 0; a NaN
 *                  score is replaced by the quiet NaN 0x7fc00000.
 *   out[b, 0, s, :] = the min(#allowed, top_k) allowed positions with the largest scores in
 *                  IEEE-754 total order (a tie goes to the lower position), in ascending
 *                  position order, then -1 up to top_k entries.
 *
 * The result is integer: it matches the CPU reference of that definition exactly.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#include "fa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * dsa_index_select -- enqueue the selection above (a scoring kernel, then the selection's
 * histogram, candidate and write kernels).
 *
 *   query      [batch, q_seq, heads, head_dim] elements of `dtype`
 *   key        [batch, key_seq, head_dim] elements of `dtype` (one key head shared by all heads)
 *   weights    [batch, q_seq, heads] elements of `dtype`
 *   bias       [batch, 1, q_seq, key_seq] float32
 *   out        [batch, 1, q_seq, top_k] int64
 *   batch, q_seq, heads, key_seq >= 0; 0 <= head_dim <= 128; top_k >= 1
 *   scale, weights_scale   finite and > 0
 *   dtype      FA_DTYPE_F32, FA_DTYPE_F16 or FA_DTYPE_BF16 (query, key and weights alike)
 *   workspace  caller-owned device memory of at least
 *              dsa_index_select_workspace_bytes(batch, q_seq, key_seq) bytes, 16-byte aligned
 *              (may be NULL when that is 0); overwritten, and in use until the call's work on
 *              `stream` has finished; calls that overlap in time must not share it
 *   stream     hipStream_t (NULL: the default stream)
 *
 * Every pointer is caller-owned device memory, dense and contiguous.  Asynchronous: no
 * allocation, memset or synchronisation, so the call may be captured into a HIP graph.  An
 * empty problem (batch * q_seq == 0) returns FA_OK without touching the device; key_seq == 0
 * writes rows of -1.  Errors: FA_ERR_UNSUPPORTED (dtype, head_dim > 128),
 * FA_ERR_INVALID_ARGUMENT (negative sizes, top_k < 1, scale or weights_scale not finite and
 * positive, a required NULL pointer, a missing, misaligned or short workspace), FA_ERR_OVERFLOW
 * (element counts or grid), FA_ERR_HIP (launch); nothing is enqueued on error except after a
 * failed launch.  fa_last_error() describes the failure.
 */
int dsa_index_select(const void* query, const void* key, const void* weights, const float* bias,
                     int64_t* out, int batch, int q_seq, int heads, int head_dim, int key_seq,
                     int top_k, float scale, float weights_scale, int dtype, void* workspace,
                     size_t workspace_bytes, void* stream);

/* The validation dsa_index_select performs, without enqueuing anything or touching the HIP
 * runtime.  Same arguments (minus the stream), same status codes. */
int dsa_check_args(const void* query, const void* key, const void* weights, const float* bias,
                   const int64_t* out, int batch, int q_seq, int heads, int head_dim, int key_seq,
                   int top_k, float scale, float weights_scale, int dtype, const void* workspace,
                   size_t workspace_bytes);

/* Workspace bytes dsa_index_select needs: 4 per (batch, query row, key position) cell (the
 * cells' order keys, first), then for every query row 16416 bytes of histograms and counters and
 * 4 bytes per 2048 key positions, then 8 bytes per cell (threshold candidates and positions); 0 when key_seq or batch * q_seq is 0, for
 * negative sizes or on overflow.  Host only. */
size_t dsa_index_select_workspace_bytes(int batch, int q_seq, int key_seq);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
