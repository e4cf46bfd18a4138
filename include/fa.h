/*
 * fa.h — C ABI of the MI355X (gfx950) tiled online-softmax attention forward library (libfa.so).
 *
 * The operation is the prefill attention forward pass stated on the onnx-runtime-ep-cuda page
 * `src/kernels/flash_attention.rs` (kernel argument list of `flash_attention_body`, host
 * function `run`), with the token-major output of the pictor-kernels page
 * `src/gpu_backend/cuda_imagen_attn_kernels.rs` (module documentation, "the op"):
 *
 *   for batch b, query head h, query row i:
 *     kvh  = h / (heads / kv_heads)                      (consecutive heads share a KV head)
 *     L    = total_lengths ? min(total_lengths[b], sk) : sk
 *     cmax = past_lengths  ? past_lengths[b] + i : L - sq + i      (bottom-right causal)
 *     lo   = local_window > 0 ? max(0, cmax + 1 - local_window) : 0
 *     key j is attended iff j < L, (causal == 0 or j <= cmax) and j >= lo
 *     x_j  = scale * <q[b,h,i,:], k[b,kvh,j,:]>
 *            then, if softcap > 0:     x_j = softcap * tanh(x_j / softcap)
 *            then, if mask_planes > 0: x_j += mask[plane, i, j]
 *     out[b,h,i,:] = sum_j softmax_j(x) * v[b,kvh,j,:] over attended keys with x_j != -inf,
 *                    or 0 when no such key exists.
 *   plane = 0 when mask_planes == 1, b when mask_planes == batch, b*heads + h when
 *   mask_planes == batch*heads (checked in that order).
 *
 *   Reading of total_lengths[b] > sk: the page's kernels never score a key at or past sk, so
 *   L is capped at sk; without past_lengths the causal base is that capped L (L - sq + i),
 *   whereas the page's kernel body subtracts sq from the uncapped total.  The two agree
 *   whenever total_lengths[b] <= sk.
 *
 * Threading and ownership: every pointer is caller-owned DEVICE memory, dense and contiguous
 * in the layout stated per argument; the library never allocates, frees, copies to the host
 * or synchronises on the call path and keeps no state between calls except the thread-local
 * error text.  Work is enqueued on `stream` (a hipStream_t; NULL means the default stream)
 * and the call returns before it runs.  `out` must not alias any input.  Device-side
 * length values are not checked on the host (that would need a device-to-host copy); any
 * int32 value is handled by the rule above.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  F16 is IEEE binary16, BF16 is bfloat16, both accumulated in fp32. */
typedef enum fa_dtype { FA_DTYPE_F32 = 0, FA_DTYPE_F16 = 1, FA_DTYPE_BF16 = 2 } fa_dtype;

/* Output layouts. */
typedef enum fa_out_layout {
    FA_OUT_HEAD_MAJOR = 0,  /* out [batch, heads, sq, dim]                                  */
    FA_OUT_TOKEN_MAJOR = 1  /* out [batch, sq, heads*dim], out[b, i, h*dim + d]             */
} fa_out_layout;

/* Status codes. */
enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARGUMENT = -1, /* inconsistent sizes, null required pointer, bad enum     */
    FA_ERR_UNSUPPORTED = -2,      /* dtype, mask dtype or head dim outside what is built     */
    FA_ERR_OVERFLOW = -3,         /* an element count, byte size or grid exceeds its range   */
    FA_ERR_HIP = -4               /* the HIP runtime rejected the launch                     */
};

/*
 * flash_attn_fwd — enqueue the attention forward pass described above.
 *
 *   q              [batch, heads, sq, dim] elements of `dtype`
 *   k, v           [batch, kv_heads, kv_capacity, dim] elements of `dtype`; only rows j < L of
 *                  each (b, kv head) plane are read (rows past L may hold anything, NaN included)
 *   mask           NULL, or [mask_planes, sq, sk] elements of `mask_dtype` (row stride sk);
 *                  -inf entries remove a key
 *   total_lengths  NULL, or device int32[batch]: keys per batch entry (capped at sk)
 *   past_lengths   NULL, or device int32[batch]: cache rows before this call's first query
 *   out            output in `out_layout`, elements of `dtype`, rounded to nearest even
 *   batch, sq, sk, kv_capacity >= 0; heads >= 0; kv_heads >= 1 and divides heads;
 *   sk <= kv_capacity; 1 <= dim <= 128 (16-bit dtypes) or 1 <= dim <= 384 (FA_DTYPE_F32)
 *   causal         nonzero enables bottom-right aligned causal masking
 *   mask_planes    0 (no mask), 1, batch or batch*heads; nonzero needs a non-NULL mask
 *   local_window   <= 0 disables the window; otherwise keys j < cmax + 1 - local_window drop
 *   scale          any finite value (typically 1/sqrt(dim))
 *   softcap        <= 0 disables; otherwise finite
 *   dtype          FA_DTYPE_F32, FA_DTYPE_F16 or FA_DTYPE_BF16
 *   mask_dtype     FA_DTYPE_F32 or `dtype` (ignored without a mask)
 *   out_layout     FA_OUT_HEAD_MAJOR or FA_OUT_TOKEN_MAJOR
 *   stream         hipStream_t to enqueue on
 *
 * An empty problem (batch*heads*sq == 0) returns FA_OK without touching the device.  With
 * sk == 0 (or every key removed) the output rows are written as 0.  On error nothing is
 * enqueued (except FA_ERR_HIP, which reports a failed launch) and fa_last_error() describes
 * the failure.
 *
 * Graph capture: a call enqueues one kernel (none for an empty problem) and neither allocates,
 * clears memory with a memset node, nor synchronises, so it may be captured into a HIP graph
 * and replayed.  The graph keeps the pointers and sizes of the capture: a replay reads the
 * buffers' contents at replay time.  Make one call outside capture first on each device (it
 * queries and caches the device's compute-unit count).
 */
int flash_attn_fwd(const void* q, const void* k, const void* v, const void* mask,
                   const int32_t* total_lengths, const int32_t* past_lengths, void* out,
                   int batch, int heads, int kv_heads, int sq, int sk, int kv_capacity, int dim,
                   int causal, int mask_planes, int local_window, float scale, float softcap,
                   int dtype, int mask_dtype, int out_layout, void* stream);

/*
 * fa_check_args — the argument validation flash_attn_fwd performs, without enqueuing
 * anything or touching the HIP runtime.  Same arguments (minus the stream), same status
 * codes.  Pointers are only checked for NULL where they are required.
 *
 * This is the claim-time gate of the flash_attention.rs page: its `supported` function (which
 * accepts head dims 1..128 and routes single-query calls elsewhere) and the checks `run` makes
 * before it launches (dtype dispatch, checked narrowing of sizes to the kernel's integer
 * types, grid overflow).  Here the head-dim range is 1..128 for 16-bit inputs and 1..384 for
 * FA_DTYPE_F32, sq == 1 is accepted, and the layout sizes are checked as well.
 */
int fa_check_args(const void* q, const void* k, const void* v, const void* mask,
                  const int32_t* total_lengths, const int32_t* past_lengths, const void* out,
                  int batch, int heads, int kv_heads, int sq, int sk, int kv_capacity, int dim,
                  int causal, int mask_planes, int local_window, float scale, float softcap,
                  int dtype, int mask_dtype, int out_layout);

/*
 * flash_attn_fwd_splitkv — the operation of flash_attn_fwd (same arguments, same result up to
 * rounding order) for few query rows per KV head, such as decode steps: the key range is cut
 * into `num_splits` spans processed in parallel, and a second kernel merges the spans' partial
 * states (running maximum, denominator, unnormalised output) exactly as the online softmax
 * merges tiles.  The onnx-runtime-ep-cuda page gates one-query calls of its prefill kernel to a
 * separate decode kernel (`supported`, and the decode parity test it names); this is that path.
 *
 *   Takes:    dtype FA_DTYPE_BF16 or FA_DTYPE_F16, dim 64 or 128, (heads / kv_heads) * sq <= 32
 *             (the query rows of one KV head form one 32-row block), 16-byte aligned q, k, v and
 *             out, and kv_capacity * dim * 2 < 2^31; masks as for flash_attn_fwd.  Anything else
 *             returns FA_ERR_UNSUPPORTED; flash_attn_fwd covers it.
 *   num_splits  a positive multiple of 4 (fa_splitkv_suggested_splits gives one that fills the
 *             device); spans are ceil(sk / 32 / num_splits) 32-key tiles long.
 *   workspace   caller-owned device memory, 16-byte aligned, at least
 *             fa_splitkv_workspace_bytes(batch, kv_heads, dim, num_splits) bytes; overwritten,
 *             and in use until the call's work on `stream` has finished.  Calls that overlap in
 *             time must not share a workspace.
 *
 * Enqueues two kernels on `stream` (none for an empty problem); no allocation, memset or
 * synchronisation, so it may be captured into a HIP graph like flash_attn_fwd.  Errors: those
 * of flash_attn_fwd, FA_ERR_UNSUPPORTED as above, FA_ERR_INVALID_ARGUMENT for num_splits or a
 * missing, misaligned or short workspace, FA_ERR_OVERFLOW when the workspace size or grid
 * overflows.
 */
int flash_attn_fwd_splitkv(const void* q, const void* k, const void* v, const void* mask,
                           const int32_t* total_lengths, const int32_t* past_lengths, void* out,
                           int batch, int heads, int kv_heads, int sq, int sk, int kv_capacity,
                           int dim, int causal, int mask_planes, int local_window, float scale,
                           float softcap, int dtype, int mask_dtype, int out_layout,
                           int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/* Size of the static device scratch of flash_attn_fwd_splitkv_noalloc (16 MiB per device). */
#define FA_SPLITKV_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * flash_attn_fwd_splitkv_noalloc — flash_attn_fwd_splitkv for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments minus the workspace, same kernels, same result (bit for bit, at
 * the same num_splits).  The spans' partial states go to a static device array of
 * FA_SPLITKV_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs on until the
 * process ends; nothing is allocated, freed or cleared per call.
 *
 *   Limit:    fa_splitkv_workspace_bytes(batch, kv_heads, dim, num_splits) must not exceed
 *             FA_SPLITKV_NOALLOC_SCRATCH_BYTES; larger calls return FA_ERR_UNSUPPORTED (use
 *             fewer spans, or flash_attn_fwd_splitkv with a workspace).
 *   Sharing:  every call on one device uses the same scratch, which keeps the last call's
 *             contents.  Calls whose work overlaps in time on one device (two streams, two
 *             host threads) race on it and give wrong results: serialise them, e.g. on one
 *             stream.  Nothing in the scratch needs to start at zero: every span writes its
 *             state before the merge reads it.
 *   Set-up:   the first call on each device looks up the scratch's device address once
 *             (hipGetSymbolAddress; no stream work) and caches it; make that first call
 *             outside graph capture.  FA_ERR_HIP if the lookup fails.
 *   Other errors: those of flash_attn_fwd_splitkv except the workspace checks.
 */
int flash_attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, const void* mask,
                                   const int32_t* total_lengths, const int32_t* past_lengths, void* out,
                                   int batch, int heads, int kv_heads, int sq, int sk, int kv_capacity,
                                   int dim, int causal, int mask_planes, int local_window, float scale,
                                   float softcap, int dtype, int mask_dtype, int out_layout, int num_splits,
                                   void* stream);

/* Workspace bytes flash_attn_fwd_splitkv needs: num_splits * batch * kv_heads * 32 rows of
 * (dim + 2) floats.  0 for invalid arguments or on overflow.  Host only. */
size_t fa_splitkv_workspace_bytes(int batch, int kv_heads, int dim, int num_splits);

/* A num_splits for flash_attn_fwd_splitkv that gives the current device about one workgroup of
 * four spans per compute unit (a multiple of 4, at most one span per 32-key tile).  Queries the
 * device's compute-unit count once (cached); no stream work. */
int fa_splitkv_suggested_splits(int batch, int kv_heads, int sk);

/* Thread-local text describing the most recent non-FA_OK status on this thread ("" if none).
 * The pointer stays valid until the next call into the library on the same thread.
 *
 * The flash_attention.rs page's host function `run` reports failures as typed errors carrying
 * a message: "not implemented" for shapes and dtypes outside the kernels (FA_ERR_UNSUPPORTED
 * here), and a kernel failure for sizes that do not narrow to the kernel's integer types and
 * for a failed launch (FA_ERR_OVERFLOW and FA_ERR_HIP here).  A C ABI returns the status as an
 * integer and keeps the message here. */
const char* fa_last_error(void);

/* Library version, e.g. "0.1.0". */
const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
