// C ABI of libfa.so: argument validation, kernel selection and launch (declared in fa.h).
//
// Mirrors the host function `run` of the onnx-runtime-ep-cuda page
// `src/kernels/flash_attention.rs` (support gate, dtype dispatch, checked narrowing of sizes,
// grid computation, launch), with these differences: the call is asynchronous on the caller's
// stream, sizes are validated against the stated layouts, mask planes outside {1, B, B*H} are
// rejected instead of silently reading plane 0, and an empty key range writes zeros.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "../../include/dsa.h"
#include "../../include/fa.h"
#include "dsa_kernels.h"
#include "fa_launch.h"
#include "fa_params.h"
#include "fa_fwd16_ring_consts.h"

namespace {

thread_local char g_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_error, sizeof(g_error), fmt, ap);
    va_end(ap);
    return status;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

// Element count a*b*c*d with overflow detection; false on overflow.
bool count4(int64_t a, int64_t b, int64_t c, int64_t d, int64_t* out) {
    int64_t t;
    return mul_ok(a, b, &t) && mul_ok(t, c, &t) && mul_ok(t, d, out);
}

int elem_bytes(int dtype) { return dtype == FA_DTYPE_F32 ? 4 : 2; }

bool aligned(const void* ptr, uintptr_t n) { return ((uintptr_t)ptr % n) == 0; }

struct Plan {
    fa::FwdParams p;
    int dp;
    int grid;
    int maskk;  // 0 none, 1 fp32 mask, 2 mask of the input type
    bool ring;  // 256-row LDS-ring kernel (16-bit, head dim 64/128, aligned rows)
    bool wide;  // fp32 kernel for head dims 129..384
    bool empty;
    // fp32 (head dim <= 128) in 32-row workgroups with the key range split in two halves: grid
    // and tile counts (grid_split 0 where that form is not available)
    int grid_split, q_tiles_split, pairs_split;
};

int validate(const void* q, const void* k, const void* v, const void* mask, const void* out,
             int batch, int heads, int kv_heads, int sq, int sk, int kv_capacity, int dim,
             int mask_planes, float scale, float softcap, int dtype, int mask_dtype,
             int out_layout, Plan* plan) {
    g_error[0] = '\0';
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16)
        return fail(FA_ERR_UNSUPPORTED, "dtype %d is not one of F32 (0), F16 (1), BF16 (2)", dtype);
    // fp32 goes up to the pages' wide variant (384); the 16-bit kernels to 128
    const int max_dim = dtype == FA_DTYPE_F32 ? 384 : 128;
    if (dim < 1 || dim > max_dim)
        return fail(FA_ERR_UNSUPPORTED, "head dim %d outside the supported range 1..%d for this dtype", dim, max_dim);
    if (out_layout != FA_OUT_HEAD_MAJOR && out_layout != FA_OUT_TOKEN_MAJOR)
        return fail(FA_ERR_INVALID_ARGUMENT, "out_layout %d is neither head-major (0) nor token-major (1)", out_layout);
    if (batch < 0 || heads < 0 || sq < 0 || sk < 0 || kv_capacity < 0)
        return fail(FA_ERR_INVALID_ARGUMENT, "negative size (batch %d, heads %d, sq %d, sk %d, kv_capacity %d)",
                    batch, heads, sq, sk, kv_capacity);
    if (kv_heads < 1) return fail(FA_ERR_INVALID_ARGUMENT, "kv_heads must be >= 1 (got %d)", kv_heads);
    if (heads % kv_heads != 0)
        return fail(FA_ERR_INVALID_ARGUMENT, "heads %d is not a multiple of kv_heads %d", heads, kv_heads);
    if (sk > kv_capacity)
        return fail(FA_ERR_INVALID_ARGUMENT, "sk %d exceeds kv_capacity %d", sk, kv_capacity);
    const int64_t bh = (int64_t)batch * heads;
    if (mask_planes != 0 && mask_planes != 1 && mask_planes != batch && (int64_t)mask_planes != bh)
        return fail(FA_ERR_INVALID_ARGUMENT, "mask_planes %d is not 0, 1, batch (%d) or batch*heads (%lld)",
                    mask_planes, batch, (long long)bh);
    if (mask_planes < 0) return fail(FA_ERR_INVALID_ARGUMENT, "negative mask_planes %d", mask_planes);
    if (mask_planes > 0 && mask == nullptr)
        return fail(FA_ERR_INVALID_ARGUMENT, "mask_planes %d but the mask pointer is null", mask_planes);
    if (mask_planes > 0 && mask_dtype != FA_DTYPE_F32 && mask_dtype != dtype)
        return fail(FA_ERR_UNSUPPORTED, "mask dtype %d must be F32 (0) or the input dtype (%d)", mask_dtype, dtype);
    if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARGUMENT, "scale must be finite");
    if (std::isnan(softcap) || std::isinf(softcap))
        return fail(FA_ERR_INVALID_ARGUMENT, "softcap must be finite (<= 0 disables it)");

    // element counts and byte sizes must fit in 63 bits
    const int64_t esz = elem_bytes(dtype);
    int64_t n_q, n_kv, n_mask, bytes;
    if (!count4(batch, heads, sq, dim, &n_q) || !mul_ok(n_q, esz, &bytes))
        return fail(FA_ERR_OVERFLOW, "q/out element count overflows");
    if (!count4(batch, kv_heads, kv_capacity, dim, &n_kv) || !mul_ok(n_kv, esz, &bytes))
        return fail(FA_ERR_OVERFLOW, "k/v element count overflows");
    if (!count4(mask_planes, sq, sk, 1, &n_mask) || !mul_ok(n_mask, 4, &bytes))
        return fail(FA_ERR_OVERFLOW, "mask element count overflows");

    plan->empty = (n_q == 0);
    if (plan->empty) return FA_OK;
    if (q == nullptr || out == nullptr) return fail(FA_ERR_INVALID_ARGUMENT, "q and out must not be null");
    if (sk > 0 && (k == nullptr || v == nullptr))
        return fail(FA_ERR_INVALID_ARGUMENT, "k and v must not be null when sk > 0");

    // kernel choice: the LDS-ring kernel takes 16-bit inputs with head dim 64 or 128 whose rows
    // (and the output rows) sit on 16-byte boundaries
    // (a mask must have 16-byte aligned rows there: sk a multiple of 4 and an aligned base)
    const int maskk = mask_planes == 0 ? 0 : (mask_dtype == FA_DTYPE_F32 ? 1 : 2);
    const bool mask_vec = mask_planes > 0 && sk % 4 == 0 && aligned(mask, maskk == 1 ? 16 : 8);
    // (its K/V loads address one (batch, KV head) cache through 32-bit byte offsets)
    plan->ring = dtype != FA_DTYPE_F32 && (dim == 64 || dim == 128) && aligned(q, 16) &&
                 aligned(out, 16) && (sk == 0 || (aligned(k, 16) && aligned(v, 16))) &&
                 (mask_planes == 0 || mask_vec) && (int64_t)kv_capacity * dim * 2 < 0x7fffffffLL;
    plan->wide = dtype == FA_DTYPE_F32 && dim > 128;
    const int block_rows = plan->ring ? fa::kRingBlockRows
                           : plan->wide ? fa::kWideRows
                           : dtype == FA_DTYPE_F32 ? fa::kF32Rows : fa::kBlockRows;
    if (mask_planes > 0 && (int64_t)block_rows * sk * 4 >= 0x7fffffffLL)
        return fail(FA_ERR_UNSUPPORTED, "sk %d is too long for a masked launch (a workgroup's mask rows "
                    "must span less than 2 GiB)", sk);
    const int64_t q_tiles = ((int64_t)sq + block_rows - 1) / block_rows;
    const int64_t pairs = (int64_t)batch * q_tiles;
    const int64_t pairs_padded = (pairs + 7) / 8 * 8;
    // group-major workgroup order when no mask plane is shared across heads and the (batch, KV
    // head) groups split evenly over the 8 XCDs; the grid then needs no padding
    const bool xcd_groups = mask_planes == 0 && ((int64_t)batch * kv_heads) % 8 == 0;
    int64_t grid;
    if (!mul_ok(xcd_groups ? (int64_t)batch * q_tiles : pairs_padded, heads, &grid) || grid > 0x7fffffffLL)
        return fail(FA_ERR_OVERFLOW, "grid of %lld x %d workgroups exceeds the launch limit",
                    (long long)pairs_padded, heads);

    plan->grid_split = 0;
    if (dtype == FA_DTYPE_F32 && !plan->wide) {
        const int64_t qt2 = ((int64_t)sq + fa::kF32SplitRows - 1) / fa::kF32SplitRows;
        const int64_t pairs2 = (int64_t)batch * qt2;
        int64_t grid2;
        if (mul_ok(xcd_groups ? pairs2 : (pairs2 + 7) / 8 * 8, heads, &grid2) && grid2 <= 0x7fffffffLL) {
            plan->grid_split = (int)grid2;
            plan->q_tiles_split = (int)qt2;
            plan->pairs_split = (int)pairs2;
        }
    }

    fa::FwdParams& p = plan->p;
    p.q = q; p.k = k; p.v = v; p.out = (void*)out;
    p.mask = mask_planes > 0 ? mask : nullptr;
    p.batch = batch; p.heads = heads; p.kv_heads = kv_heads; p.sq = sq; p.sk = sk; p.dim = dim;
    p.group = heads / kv_heads;
    p.mask_planes = mask_planes;
    p.q_tiles = (int)q_tiles;
    p.pairs = (int)pairs;
    p.xcd_groups = xcd_groups ? 1 : 0;
    p.kv_capacity = kv_capacity;
    const uintptr_t vec_align = 16;
    p.vec_kv = (dim % (dtype == FA_DTYPE_F32 ? 4 : 8) == 0) && aligned(q, vec_align) &&
               (sk == 0 || (aligned(k, vec_align) && aligned(v, vec_align)));
    p.vec_out = (dim % 4 == 0) && aligned(out, dtype == FA_DTYPE_F32 ? 16 : 8);
    plan->maskk = maskk;
    p.vec_mask = mask_vec;
    if (out_layout == FA_OUT_HEAD_MAJOR) {
        p.o_stride_b = (int64_t)heads * sq * dim;
        p.o_stride_h = (int64_t)sq * dim;
        p.o_stride_i = dim;
    } else {
        p.o_stride_b = (int64_t)sq * heads * dim;
        p.o_stride_h = dim;
        p.o_stride_i = (int64_t)heads * dim;
    }
    p.scale = scale;
    p.softcap = softcap > 0.0f ? softcap : 0.0f;
    const bool has_cap = softcap > 0.0f;
    p.cap_y = has_cap ? scale / softcap : 0.0f;
    // Units of the tracked score x and the log2(e) factor that turns them into base-2 exponents.
    const float raw_k = scale * 1.4426950408889634f;
    p.raw_scores = (!has_cap && mask_planes == 0 && scale > 0.0f && std::isnormal(raw_k) && raw_k >= 1e-30f) ? 1 : 0;
    if (has_cap && mask_planes == 0) p.kfac = softcap * 1.4426950408889634f;  // x = tanh(.)
    else if (p.raw_scores) p.kfac = raw_k;                                    // x = raw dot
    else p.kfac = 1.4426950408889634f;                                        // x in natural units
    if (!std::isfinite(p.kfac) || !(p.kfac > 0.0f))
        return fail(FA_ERR_UNSUPPORTED, "softcap %g is too large for fp32 exponent scaling", (double)softcap);
    {
        // tanh y = y - y^3 / 3 + 2 y^5 / 15 + O(y^7), taken for |y| < 1/8 (y = cap_y * s)
        const double k = p.kfac, c = p.cap_y;
        p.tc_b1 = (float)(k * c);
        p.tc_b3 = (float)(-k * c * c * c / 3.0);
        p.tc_b5 = (float)(2.0 * k * c * c * c * c * c / 15.0);
        p.tc_slim = c != 0.0 ? (float)(1.0 / (8.0 * std::fabs(c))) : INFINITY;
    }
    // Ring launches with bf16 inputs, head dim 64, an fp32 mask and a scale that is a power of two
    // in [2^-20, 1] (the default 1/8 included): the kernel multiplies Q by the scale, which only moves bf16 exponents
    // (exact unless a scaled value falls below 2^-126, the smallest normal bf16), and starts the
    // Q.K products from the mask values.
    int scale_exp = 0;
    const float scale_mant = std::frexp(scale, &scale_exp);
    p.mask_in_acc = (plan->ring && dtype == FA_DTYPE_BF16 && mask_planes > 0 && mask_dtype == FA_DTYPE_F32 &&
                     !has_cap && dim == 64 && scale_mant == 0.5f && scale_exp >= -19 && scale_exp <= 1) ? 1 : 0;
    plan->dp = plan->wide ? 384 : (dim + 31) / 32 * 32;
    plan->grid = (int)grid;
    return FA_OK;
}

// Compute units of the current device, queried once per device (no synchronisation).
int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Scratch for flash_attn_fwd_splitkv_noalloc: the split-key spans' partial states, for callers
// that cannot allocate.  One copy per device, held until the process ends; every call on a
// device shares it (calls that overlap in time on one device race on it).  Host code never
// passes this name to a kernel: on the host it is only a stand-in for the symbol, and the
// device address comes from hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) char scratch[FA_SPLITKV_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on the current device, looked up once per device and cached.
// Returns nullptr (with the error text set) when the lookup fails.
void* scratch_address() {
    static std::mutex mu;
    static void* cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        fail(FA_ERR_HIP, "cannot determine the current device for the static scratch");
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == nullptr) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr) {
            fail(FA_ERR_HIP, "hipGetSymbolAddress of the static scratch failed on device %d: %s", dev,
                 hipGetErrorString(e));
            return nullptr;
        }
        cache[dev] = ptr;
    }
    return cache[dev];
}

// flash_attn_fwd_splitkv with a caller workspace, or (static_scratch) with the static scratch.
int splitkv_run(const void* q, const void* k, const void* v, const void* mask,
                const int32_t* total_lengths, const int32_t* past_lengths, void* out,
                int batch, int heads, int kv_heads, int sq, int sk, int kv_capacity, int dim,
                int causal, int mask_planes, int local_window, float scale, float softcap,
                int dtype, int mask_dtype, int out_layout, int num_splits, void* workspace,
                size_t workspace_bytes, bool static_scratch, void* stream) {
    Plan plan;
    const int st = validate(q, k, v, mask, out, batch, heads, kv_heads, sq, sk, kv_capacity, dim,
                            mask_planes, scale, softcap, dtype, mask_dtype, out_layout, &plan);
    if (st != FA_OK) return st;
    if (dtype == FA_DTYPE_F32 || (dim != 64 && dim != 128))
        return fail(FA_ERR_UNSUPPORTED, "the split-key path takes bf16/f16 inputs with head dim 64 or 128");
    if ((int64_t)(heads / kv_heads) * sq > 32)
        return fail(FA_ERR_UNSUPPORTED, "the split-key path needs (heads / kv_heads) * sq <= 32, got %lld",
                    (long long)(heads / kv_heads) * sq);
    if (!aligned(q, 16) || !aligned(out, 16) || (sk > 0 && (!aligned(k, 16) || !aligned(v, 16))))
        return fail(FA_ERR_UNSUPPORTED, "the split-key path needs 16-byte aligned q, k, v and out");
    if ((int64_t)kv_capacity * dim * 2 >= 0x7fffffffLL)
        return fail(FA_ERR_UNSUPPORTED, "a (batch, KV head) cache of %lld bytes exceeds the 2 GiB the split-key "
                    "path addresses", (long long)kv_capacity * dim * 2);
    if (num_splits < 4 || num_splits % 4 != 0)
        return fail(FA_ERR_INVALID_ARGUMENT, "num_splits must be a positive multiple of 4, got %d", num_splits);
    if (plan.empty) return FA_OK;
    const size_t need = fa_splitkv_workspace_bytes(batch, kv_heads, dim, num_splits);
    if (need == 0) return fail(FA_ERR_OVERFLOW, "the split-key workspace size overflows");
    if (static_scratch) {
        if (need > (size_t)FA_SPLITKV_NOALLOC_SCRATCH_BYTES)
            return fail(FA_ERR_UNSUPPORTED, "the split-key state of this call needs %zu bytes, more than the "
                        "%zu-byte static scratch of flash_attn_fwd_splitkv_noalloc (use fewer spans, or "
                        "flash_attn_fwd_splitkv with a workspace)", need,
                        (size_t)FA_SPLITKV_NOALLOC_SCRATCH_BYTES);
        workspace = scratch_address();
        if (workspace == nullptr) return FA_ERR_HIP;
        workspace_bytes = FA_SPLITKV_NOALLOC_SCRATCH_BYTES;
    }
    if (workspace == nullptr || !aligned(workspace, 16) || workspace_bytes < need)
        return fail(FA_ERR_INVALID_ARGUMENT, "the split-key path needs a 16-byte aligned workspace of %zu bytes "
                    "(got %zu at %p)", need, workspace_bytes, workspace);
    int64_t grid1;
    if (!mul_ok((int64_t)batch * kv_heads, num_splits / 4, &grid1) || grid1 > 0x7fffffffLL)
        return fail(FA_ERR_OVERFLOW, "split-key grid exceeds the launch limit");

    fa::FwdParams& p = plan.p;
    p.total_lengths = total_lengths;
    p.past_lengths = past_lengths;
    p.causal = causal != 0;
    p.window = local_window > 0 ? local_window : 0;
    fa::SplitParams sp;
    const int64_t ws_rows = (int64_t)num_splits * batch * kv_heads * 32;
    sp.ws_o = (float*)workspace;
    sp.ws_m = sp.ws_o + ws_rows * dim;
    sp.ws_l = sp.ws_m + ws_rows;
    sp.num_splits = num_splits;
    const int64_t tiles = ((int64_t)sk + 31) / 32;
    sp.span = (int)(((tiles + num_splits - 1) / num_splits) * 32);
    if (sp.span < 32) sp.span = 32;
    sp.rows = (heads / kv_heads) * sq;

    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    const hipError_t err = dtype == FA_DTYPE_BF16 ? fa::launch_bf16_splitkv(p, sp, dim, plan.maskk, s)
                                                  : fa::launch_f16_splitkv(p, sp, dim, plan.maskk, s);
    if (err != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return FA_OK;
}

}  // namespace

extern "C" {

int fa_check_args(const void* q, const void* k, const void* v, const void* mask,
                  const int32_t* total_lengths, const int32_t* past_lengths, const void* out,
                  int batch, int heads, int kv_heads, int sq, int sk, int kv_capacity, int dim,
                  int causal, int mask_planes, int local_window, float scale, float softcap,
                  int dtype, int mask_dtype, int out_layout) {
    (void)total_lengths; (void)past_lengths; (void)causal; (void)local_window;
    Plan plan;
    return validate(q, k, v, mask, out, batch, heads, kv_heads, sq, sk, kv_capacity, dim,
                    mask_planes, scale, softcap, dtype, mask_dtype, out_layout, &plan);
}

int flash_attn_fwd(const void* q, const void* k, const void* v, const void* mask,
                   const int32_t* total_lengths, const int32_t* past_lengths, void* out,
                   int batch, int heads, int kv_heads, int sq, int sk, int kv_capacity, int dim,
                   int causal, int mask_planes, int local_window, float scale, float softcap,
                   int dtype, int mask_dtype, int out_layout, void* stream) {
    Plan plan;
    const int st = validate(q, k, v, mask, out, batch, heads, kv_heads, sq, sk, kv_capacity, dim,
                            mask_planes, scale, softcap, dtype, mask_dtype, out_layout, &plan);
    if (st != FA_OK || plan.empty) return st;
    fa::FwdParams& p = plan.p;
    p.total_lengths = total_lengths;
    p.past_lengths = past_lengths;
    p.causal = causal != 0;
    p.window = local_window > 0 ? local_window : 0;

    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();  // a stale error from unrelated work must not be reported as ours
    p.items_per_xcd = plan.grid / 8;
    int grid = plan.grid;
    if (plan.ring) {
        // the ring kernel is persistent: one workgroup per CU (rounded down to whole XCDs)
        // walks the work items; small problems keep one workgroup per item
        const int cus = device_cu_count();
        if (cus <= 0) return fail(FA_ERR_HIP, "cannot query the compute-unit count of the current device");
        const int persist = cus / 8 * 8;
        if (persist >= 8 && grid > persist) grid = persist;
    }
    // fp32: the key-split form when its twice as many half-size workgroups spread more evenly
    // over the CUs.  Per CU, in units of one 64-row workgroup's work: ceil(n / cus) whole ones
    // against ceil(2n / cus) halves, a half costing about 0.58 of a whole one (its K/V tiles
    // serve 32 rows instead of 64: measured on the fp32 DiT problem, 24 heads x 1536 rows, where
    // 2.25 whole workgroups per CU take 297 us and 4.5 halves 290 us).
    bool split = false;
    if (dtype == FA_DTYPE_F32 && !plan.wide && plan.grid_split > 0 &&
        fa::fwd32_split_built(plan.dp, plan.maskk != 0)) {
        const int cus = device_cu_count();
        if (cus <= 0) return fail(FA_ERR_HIP, "cannot query the compute-unit count of the current device");
        const int64_t whole = ((int64_t)plan.grid + cus - 1) / cus;
        const int64_t halves = ((int64_t)plan.grid_split + cus - 1) / cus;
        if (7 * halves < 12 * whole) {
            split = true;
            grid = plan.grid_split;
            p.q_tiles = plan.q_tiles_split;
            p.pairs = plan.pairs_split;
        }
    }
    hipError_t err;
    if (dtype == FA_DTYPE_BF16)
        err = plan.ring ? fa::launch_bf16_ring(p, plan.dp, grid, plan.maskk, p.softcap > 0.0f, s)
                        : fa::launch_bf16(p, plan.dp, grid, plan.maskk, p.softcap > 0.0f, s);
    else if (dtype == FA_DTYPE_F16)
        err = plan.ring ? fa::launch_f16_ring(p, plan.dp, grid, plan.maskk, p.softcap > 0.0f, s)
                        : fa::launch_f16(p, plan.dp, grid, plan.maskk, p.softcap > 0.0f, s);
    else if (plan.wide) err = fa::launch_f32_wide(p, grid, plan.maskk != 0, p.softcap > 0.0f, s);
    else err = fa::launch_f32(p, plan.dp, grid, plan.maskk != 0, p.softcap > 0.0f, split, s);
    if (err != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return FA_OK;
}

size_t fa_splitkv_workspace_bytes(int batch, int kv_heads, int dim, int num_splits) {
    if (batch < 0 || kv_heads < 1 || dim < 1 || num_splits < 1) return 0;
    int64_t rows, bytes;
    if (!count4(num_splits, batch, kv_heads, 32, &rows) || !mul_ok(rows, (int64_t)(dim + 2) * 4, &bytes)) return 0;
    return (size_t)bytes;
}

int fa_splitkv_suggested_splits(int batch, int kv_heads, int sk) {
    const int cus = device_cu_count();
    const int64_t groups = (int64_t)(batch > 0 ? batch : 1) * (kv_heads > 0 ? kv_heads : 1);
    // one workgroup of four spans per CU (its registers and LDS fit one per CU; a second round
    // of workgroups costs more in start-up latency than it gains), spans of at least one tile
    int64_t want = 4 * (((int64_t)(cus > 0 ? cus : 256) + groups - 1) / groups);
    const int64_t tiles = ((int64_t)(sk > 0 ? sk : 1) + 31) / 32;
    const int64_t cap = 4 * ((tiles + 3) / 4);
    if (want > cap) want = cap;
    if (want < 4) want = 4;
    if (want > 4096) want = 4096;
    return (int)want;
}

int flash_attn_fwd_splitkv(const void* q, const void* k, const void* v, const void* mask,
                           const int32_t* total_lengths, const int32_t* past_lengths, void* out,
                           int batch, int heads, int kv_heads, int sq, int sk, int kv_capacity, int dim,
                           int causal, int mask_planes, int local_window, float scale, float softcap,
                           int dtype, int mask_dtype, int out_layout, int num_splits, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return splitkv_run(q, k, v, mask, total_lengths, past_lengths, out, batch, heads, kv_heads, sq, sk,
                       kv_capacity, dim, causal, mask_planes, local_window, scale, softcap, dtype, mask_dtype,
                       out_layout, num_splits, workspace, workspace_bytes, false, stream);
}

int flash_attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, const void* mask,
                                   const int32_t* total_lengths, const int32_t* past_lengths, void* out,
                                   int batch, int heads, int kv_heads, int sq, int sk, int kv_capacity,
                                   int dim, int causal, int mask_planes, int local_window, float scale,
                                   float softcap, int dtype, int mask_dtype, int out_layout, int num_splits,
                                   void* stream) {
    return splitkv_run(q, k, v, mask, total_lengths, past_lengths, out, batch, heads, kv_heads, sq, sk,
                       kv_capacity, dim, causal, mask_planes, local_window, scale, softcap, dtype, mask_dtype,
                       out_layout, num_splits, nullptr, 0, true, stream);
}

size_t dsa_index_select_workspace_bytes(int batch, int q_seq, int key_seq) {
    if (batch < 0 || q_seq < 0 || key_seq < 0) return 0;
    int64_t keys, rows;
    if (!count4(batch, q_seq, key_seq, 4, &keys) || !count4(batch, q_seq, 1, 1, &rows)) return 0;
    if (key_seq == 0 || rows == 0) return 0;
    // keys, then per row kAuxInts words and one word per chunk of kSelChunkKeys positions, then
    // two words per cell (the candidates)
    const int64_t chunks = ((int64_t)key_seq + dsa::kSelChunkKeys - 1) / dsa::kSelChunkKeys;
    int64_t aux, cnt, total;
    if (!mul_ok(rows, (int64_t)dsa::kAuxInts * 4, &aux) || !mul_ok(rows, chunks * 4, &cnt)) return 0;
    total = keys + aux + cnt;
    if (total < keys || total > INT64_MAX - 2 * keys) return 0;
    total += 2 * keys;
    return (size_t)total;
}

int dsa_check_args(const void* query, const void* key, const void* weights, const float* bias,
                   const int64_t* out, int batch, int q_seq, int heads, int head_dim, int key_seq,
                   int top_k, float scale, float weights_scale, int dtype, const void* workspace,
                   size_t workspace_bytes) {
    g_error[0] = '\0';
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16)
        return fail(FA_ERR_UNSUPPORTED, "dtype %d is not one of FA_DTYPE_F32/F16/BF16", dtype);
    if (batch < 0 || q_seq < 0 || heads < 0 || head_dim < 0 || key_seq < 0)
        return fail(FA_ERR_INVALID_ARGUMENT, "negative size (batch %d, q_seq %d, heads %d, head_dim %d, key_seq %d)",
                    batch, q_seq, heads, head_dim, key_seq);
    if (head_dim > 128) return fail(FA_ERR_UNSUPPORTED, "head_dim %d exceeds 128", head_dim);
    if (top_k < 1) return fail(FA_ERR_INVALID_ARGUMENT, "top_k must be >= 1, got %d", top_k);
    if (!std::isfinite(scale) || !(scale > 0.0f))
        return fail(FA_ERR_INVALID_ARGUMENT, "scale must be finite and > 0, got %g", (double)scale);
    if (!std::isfinite(weights_scale) || !(weights_scale > 0.0f))
        return fail(FA_ERR_INVALID_ARGUMENT, "weights_scale must be finite and > 0, got %g", (double)weights_scale);
    const int64_t esz = dtype == FA_DTYPE_F32 ? 4 : 2;
    int64_t n, bytes;
    if (!count4(batch, q_seq, heads, head_dim, &n) || !mul_ok(n, esz, &bytes) ||
        !count4(batch, key_seq, head_dim, 1, &n) || !mul_ok(n, esz, &bytes) ||
        !count4(batch, q_seq, heads, 1, &n) || !mul_ok(n, esz, &bytes) ||
        !count4(batch, q_seq, key_seq, 4, &bytes) || !count4(batch, q_seq, top_k, 8, &bytes))
        return fail(FA_ERR_OVERFLOW, "an element count or byte size overflows");
    const int64_t rows = (int64_t)batch * q_seq;
    if (rows == 0) return FA_OK;
    if (out == nullptr || !aligned(out, 8)) return fail(FA_ERR_INVALID_ARGUMENT, "out is NULL or not 8-byte aligned");
    if (key_seq > 0) {
        if (bias == nullptr || !aligned(bias, 4)) return fail(FA_ERR_INVALID_ARGUMENT, "bias is NULL or not 4-byte aligned");
        if (heads > 0 && weights == nullptr) return fail(FA_ERR_INVALID_ARGUMENT, "weights is NULL");
        if (heads > 0 && head_dim > 0 && (query == nullptr || key == nullptr))
            return fail(FA_ERR_INVALID_ARGUMENT, "query or key is NULL");
        const int64_t tiles = ((int64_t)key_seq + 255) / 256;
        int64_t grid;
        if (!mul_ok(rows, tiles, &grid) || grid > 0x7fffffffLL)
            return fail(FA_ERR_OVERFLOW, "scoring grid exceeds the launch limit");
    }
    int64_t sel_grid;
    if (!mul_ok(rows, ((int64_t)key_seq + dsa::kSelChunkKeys - 1) / dsa::kSelChunkKeys, &sel_grid) ||
        rows > 0x7fffffffLL || sel_grid > 0x7fffffffLL)
        return fail(FA_ERR_OVERFLOW, "selection grid exceeds the launch limit");
    const size_t need = dsa_index_select_workspace_bytes(batch, q_seq, key_seq);
    if (need > 0 && (workspace == nullptr || !aligned(workspace, 16) || workspace_bytes < need))
        return fail(FA_ERR_INVALID_ARGUMENT, "the index selection needs a 16-byte aligned workspace of %zu bytes "
                    "(got %zu at %p)", need, workspace_bytes, workspace);
    return FA_OK;
}

int dsa_index_select(const void* query, const void* key, const void* weights, const float* bias,
                     int64_t* out, int batch, int q_seq, int heads, int head_dim, int key_seq,
                     int top_k, float scale, float weights_scale, int dtype, void* workspace,
                     size_t workspace_bytes, void* stream) {
    const int st = dsa_check_args(query, key, weights, bias, out, batch, q_seq, heads, head_dim, key_seq,
                                  top_k, scale, weights_scale, dtype, workspace, workspace_bytes);
    if (st != FA_OK || (int64_t)batch * q_seq == 0) return st;
    dsa::DsaParams p;
    p.query = query;
    p.key = key;
    p.weights = weights;
    p.bias = bias;
    p.keys = (uint32_t*)workspace;
    p.aux = (int*)((char*)workspace + (size_t)batch * q_seq * key_seq * 4);
    p.counts = p.aux + (size_t)batch * q_seq * dsa::kAuxInts;
    p.cand = p.counts + (size_t)batch * q_seq * (((size_t)key_seq + dsa::kSelChunkKeys - 1) / dsa::kSelChunkKeys);
    p.out = out;
    p.batch = batch;
    p.q_seq = q_seq;
    p.heads = heads;
    p.head_dim = head_dim;
    p.key_seq = key_seq;
    p.top_k = top_k;
    p.scale = scale;
    p.weights_scale = weights_scale;
    (void)hipGetLastError();
    const hipError_t err = dsa::launch_index_select(p, dtype == FA_DTYPE_F32 ? 0 : (dtype == FA_DTYPE_F16 ? 1 : 2),
                                                    (hipStream_t)stream);
    if (err != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return FA_OK;
}

const char* fa_last_error(void) { return g_error; }

const char* fa_version(void) { return "0.1.0"; }

}  // extern "C"
