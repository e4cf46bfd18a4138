/*
 * Attention-forward oracle in double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  The test-suite, the smoke check and the benchmark's CPU-baseline
 * leg are the only callers.  The GPU library never links, loads or calls this code, and this
 * file shares no source with it.
 *
 * What it computes, for every batch b, query head h and query row i (sources are the
 * onnx-runtime-ep-cuda page `src/kernels/flash_attention.rs` and the pictor-kernels page
 * `src/gpu_backend/cuda_imagen_attn_kernels.rs`):
 *
 *   1. GQA head map: consecutive query heads share one KV head, kvh = h / (H / Hkv)
 *      (flash_attention.rs, `flash_attention_body`, plane decomposition).
 *   2. Per-row key rule (flash_attention.rs, `flash_attention_body`, the `logical_sk`,
 *      `causal_max` and `local_min` definitions and the masking test in the key loop):
 *        L    = total_lengths ? min(total_lengths[b], Sk) : Sk
 *        cmax = past_lengths  ? past_lengths[b] + i : L - Sq + i
 *        lo   = W > 0 ? max(0, cmax + 1 - W) : 0
 *      key j is attended iff  j < L  and  (!causal or j <= cmax)  and  j >= lo.
 *      Capping L at Sk is a reading: the scalar kernel never scores keys past Sk.
 *   3. Score epilogue in the pages' order (`flash_attention_body`, score branch):
 *        x = scale * <q, k_j>;  if softcap > 0: x = softcap * tanh(x / softcap);
 *        if mask_planes > 0:    x += mask[plane, i, j]
 *      with plane = 0, or b when mask_planes == B, or b*H + h when mask_planes == B*H
 *      (tested in that order).  Mask rows have stride Sk.
 *   4. Full-row, max-subtracted softmax over the attended keys whose x is not -inf, then the
 *      probability-weighted sum of V rows (the test oracle `cpu_reference` on the
 *      flash_attention.rs page, and the "op" section of the cuda_imagen_attn_kernels.rs
 *      module documentation).  No attended finite key -> the output row is 0 (the
 *      `denominator > 0` rule of the pages' final store).
 *   5. Output layout: head-major [B, H, Sq, D], or token-major [B, Sq, H*D] with
 *      out[b, i, h*D + d] (cuda_imagen_attn_kernels.rs module documentation, "then transpose
 *      to token-major").
 *
 * Inputs are float32 arrays holding the exact stored values (bf16/f16/f32 all widen exactly);
 * every operation above is carried out in double.  Threads split the rows; each row is
 * computed independently, so the result does not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct fa_oracle_problem {
    const float* q;                /* [batch, heads, sq, dim]                      */
    const float* k;                /* [batch, kv_heads, kv_capacity, dim]          */
    const float* v;                /* [batch, kv_heads, kv_capacity, dim]          */
    const float* mask;             /* [mask_planes, sq, sk] or NULL                */
    const int32_t* total_lengths;  /* [batch] or NULL                              */
    const int32_t* past_lengths;   /* [batch] or NULL                              */
    int64_t batch, heads, kv_heads, sq, sk, kv_capacity, dim;
    int64_t causal, mask_planes, local_window;
    double scale, softcap;
} fa_oracle_problem;

static int problem_ok(const fa_oracle_problem* p) {
    if (p->batch < 0 || p->heads < 0 || p->kv_heads < 1 || p->sq < 0 || p->sk < 0) return 0;
    if (p->dim < 1 || p->sk > p->kv_capacity) return 0;
    if (p->heads % p->kv_heads != 0) return 0;
    if (p->mask_planes != 0 && p->mask == NULL) return 0;
    return 1;
}

/* Which mask plane row (b, h) reads; -1 when there is no mask. */
static int64_t mask_plane(const fa_oracle_problem* p, int64_t b, int64_t h) {
    if (p->mask_planes <= 0) return -1;
    if (p->mask_planes == p->batch) return b;
    if (p->mask_planes == p->batch * p->heads) return b * p->heads + h;
    return 0;
}

/*
 * One output row (b, h, i) into o[0..dim).  x and keep are caller scratch of sk entries.
 */
static void oracle_row(const fa_oracle_problem* p, int64_t b, int64_t h, int64_t i,
                       double* o, double* x, unsigned char* keep) {
    const int64_t group = p->heads / p->kv_heads;
    const int64_t kvh = h / group;
    const int64_t D = p->dim;

    int64_t L = p->sk;
    if (p->total_lengths != NULL && (int64_t)p->total_lengths[b] < L) L = p->total_lengths[b];
    const int64_t cmax = p->past_lengths != NULL ? (int64_t)p->past_lengths[b] + i : L - p->sq + i;
    int64_t lo = 0;
    if (p->local_window > 0) {
        lo = cmax + 1 - p->local_window;
        if (lo < 0) lo = 0;
    }

    const float* qrow = p->q + ((b * p->heads + h) * p->sq + i) * D;
    const float* kbase = p->k + (b * p->kv_heads + kvh) * p->kv_capacity * D;
    const float* vbase = p->v + (b * p->kv_heads + kvh) * p->kv_capacity * D;
    const int64_t plane = mask_plane(p, b, h);

    /* scores of the attended keys */
    for (int64_t j = 0; j < p->sk; ++j) {
        int attended = 1;
        if (j >= L) attended = 0;
        if (p->causal && j > cmax) attended = 0;
        if (j < lo) attended = 0;
        keep[j] = 0;
        if (!attended) continue;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += (double)qrow[d] * (double)kbase[j * D + d];
        double s = p->scale * dot;
        if (p->softcap > 0.0) s = p->softcap * tanh(s / p->softcap);
        if (plane >= 0) s += (double)p->mask[(plane * p->sq + i) * p->sk + j];
        x[j] = s;
        keep[j] = (s != -INFINITY);
    }

    /* full-row max-subtracted softmax */
    int any = 0;
    double m = -INFINITY;
    for (int64_t j = 0; j < p->sk; ++j) {
        if (!keep[j]) continue;
        if (!any || x[j] > m) m = x[j];
        any = 1;
    }
    for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
    if (!any) return;

    double denom = 0.0;
    for (int64_t j = 0; j < p->sk; ++j) {
        if (!keep[j]) continue;
        x[j] = exp(x[j] - m);
        denom += x[j];
    }
    for (int64_t j = 0; j < p->sk; ++j) {
        if (!keep[j]) continue;
        const double w = x[j] / denom;
        for (int64_t d = 0; d < D; ++d) o[d] += w * (double)vbase[j * D + d];
    }
}

/* ------------------------------------------------------------------------------------------ */
/* threading: rows are dealt round-robin to the workers                                        */

typedef struct {
    const fa_oracle_problem* p;
    const int64_t* rows;  /* NULL -> all rows, in (b, h, i) order */
    int64_t nrows;
    double* out;
    int64_t out_layout;   /* all-rows mode: 0 head-major, 1 token-major; rows mode: packed */
    int64_t first, step;
    int failed;
} worker_args;

static void* worker(void* arg) {
    worker_args* w = (worker_args*)arg;
    const fa_oracle_problem* p = w->p;
    const int64_t sk = p->sk > 0 ? p->sk : 1;
    double* x = (double*)malloc((size_t)sk * sizeof(double));
    unsigned char* keep = (unsigned char*)malloc((size_t)sk);
    double* o = (double*)malloc((size_t)p->dim * sizeof(double));
    if (x == NULL || keep == NULL || o == NULL) {
        w->failed = 1;
        free(x); free(keep); free(o);
        return NULL;
    }
    for (int64_t r = w->first; r < w->nrows; r += w->step) {
        int64_t b, h, i;
        double* dst;
        if (w->rows != NULL) {
            b = w->rows[3 * r]; h = w->rows[3 * r + 1]; i = w->rows[3 * r + 2];
            dst = w->out + r * p->dim;
        } else {
            i = r % p->sq;
            h = (r / p->sq) % p->heads;
            b = r / (p->sq * p->heads);
            if (w->out_layout == 1)
                dst = w->out + ((b * p->sq + i) * p->heads + h) * p->dim;
            else
                dst = w->out + ((b * p->heads + h) * p->sq + i) * p->dim;
        }
        oracle_row(p, b, h, i, o, x, keep);
        memcpy(dst, o, (size_t)p->dim * sizeof(double));
    }
    free(x); free(keep); free(o);
    return NULL;
}

static int run_rows(const fa_oracle_problem* p, const int64_t* rows, int64_t nrows, double* out,
                    int64_t out_layout, int nthreads) {
    if (nthreads <= 0) {
        long n = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = n > 0 ? (int)n : 1;
    }
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > nrows) nthreads = nrows > 0 ? (int)nrows : 1;
    pthread_t tid[256];
    worker_args args[256];
    for (int t = 0; t < nthreads; ++t) {
        args[t].p = p; args[t].rows = rows; args[t].nrows = nrows; args[t].out = out;
        args[t].out_layout = out_layout; args[t].first = t; args[t].step = nthreads;
        args[t].failed = 0;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tid[t], NULL, worker, &args[t]) != 0) break;
        started = t;
    }
    /* workers that could not be started are run on this thread */
    for (int t = started + 1; t < nthreads; ++t) worker(&args[t]);
    worker(&args[0]);
    int failed = args[0].failed;
    for (int t = 1; t <= started; ++t) {
        pthread_join(tid[t], NULL);
        failed |= args[t].failed;
    }
    for (int t = started + 1; t < nthreads; ++t) failed |= args[t].failed;
    return failed ? -2 : 0;
}

/* Every output row, in head-major (out_layout 0) or token-major (1) order.
 * Returns 0, -1 for an inconsistent problem, -2 when scratch memory is unavailable. */
int fa_oracle_forward(const fa_oracle_problem* p, double* out, int64_t out_layout, int nthreads) {
    if (!problem_ok(p)) return -1;
    return run_rows(p, NULL, p->batch * p->heads * p->sq, out, out_layout, nthreads);
}

/* Selected rows: rows holds nrows (b, h, i) triples; out receives nrows * dim values. */
int fa_oracle_rows(const fa_oracle_problem* p, const int64_t* rows, int64_t nrows, double* out,
                   int nthreads) {
    if (!problem_ok(p)) return -1;
    for (int64_t r = 0; r < nrows; ++r) {
        if (rows[3 * r] < 0 || rows[3 * r] >= p->batch || rows[3 * r + 1] < 0 ||
            rows[3 * r + 1] >= p->heads || rows[3 * r + 2] < 0 || rows[3 * r + 2] >= p->sq)
            return -1;
    }
    return run_rows(p, rows, nrows, out, 0, nthreads);
}

/* Number of worker threads a call with nthreads <= 0 would use. */
int fa_oracle_default_threads(void) {
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}
