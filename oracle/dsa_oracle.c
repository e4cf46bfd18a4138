/*
 * dsa_oracle.c -- CPU reference of the sparse index-selection operation of the
 * onnx-runtime-ep-cuda page `src/kernels/dsa_index_select.rs` (module documentation, first
 * paragraph and "Determinism / bit-parity"; input and output shapes from the shape checks of its
 * host code).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by tests/, by the smoke check and by the benchmark's
 * CPU-baseline leg.  The GPU library never links or loads it, and it shares no code with it.
 *
 * Shapes (all dense, row-major):
 *   query [B, S, H, D], key [B, T, D], weights [B, S, H]  (float32 here; 16-bit inputs are
 *   widened exactly by the caller), bias [B, 1, S, T] float32, out int64 [B, 1, S, top_k].
 *
 * For query row (b, s) and key position t:
 *   allowed  iff  bias[b, s, t] > -1e30            (the page's allow rule; NaN bias is not allowed)
 *   dot_h    = sum over d = 0, 1, ..., D-1 of fl(q[b,s,h,d] * k[b,t,d]), added left to right in
 *              float32 starting from +0, every product and every sum rounded on its own (no
 *              fused multiply-add): the page fixes this ascending-D, un-fused order for bit parity
 *   term_h   = fl( relu(fl(scale * dot_h)) * fl(w[b,s,h] * weights_scale) ), where relu(x) is the
 *              larger of x and 0 with a NaN x giving 0 (the maximum-with-zero the page applies)
 *   score    = fl( (sum over h = 0..H-1 of term_h, left to right from +0) + bias[b,s,t] ), a NaN
 *              result replaced by the canonical quiet NaN 0x7fc00000
 * Selection: keep = min(number of allowed positions, top_k) positions, the largest scores in
 * IEEE-754 total order (-inf < ... < -0 < +0 < ... < +inf < +NaN), a tie going to the lower
 * position; they are written in ascending position order, followed by -1 up to width top_k.
 *
 * Built with gcc -O2 -ffp-contract=off on x86-64 (SSE arithmetic: every float operation rounds
 * to float32, and no multiply-add is contracted).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static float canonical_nan(void) {
    const uint32_t bits = 0x7fc00000u;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

static float relu(float x) {
    /* the larger of x and 0; a NaN x gives 0 */
    return x > 0.0f ? x : 0.0f;
}

/* Scores of every cell: scores[b,s,t] (float32) and allowed[b,s,t] (0/1).  Returns 0. */
int dsa_oracle_scores(const float* query, const float* key, const float* weights, const float* bias,
                      int64_t B, int64_t S, int64_t H, int64_t D, int64_t T, float scale,
                      float weights_scale, float* scores, uint8_t* allowed) {
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t s = 0; s < S; ++s) {
            const int64_t row = b * S + s;
            const float* qrow = query + row * H * D;
            const float* wrow = weights + row * H;
            for (int64_t t = 0; t < T; ++t) {
                const int64_t cell = row * T + t;
                const float bt = bias[cell];
                if (!(bt > -1e30f)) {
                    allowed[cell] = 0;
                    scores[cell] = -INFINITY;
                    continue;
                }
                const float* krow = key + (b * T + t) * D;
                float total = 0.0f;
                for (int64_t h = 0; h < H; ++h) {
                    float dot = 0.0f;
                    for (int64_t d = 0; d < D; ++d) {
                        const float prod = qrow[h * D + d] * krow[d];
                        dot = dot + prod;
                    }
                    const float scaled = scale * dot;
                    const float wgt = wrow[h] * weights_scale;
                    const float term = relu(scaled) * wgt;
                    total = total + term;
                }
                float sc = total + bt;
                if (isnan(sc)) sc = canonical_nan();
                scores[cell] = sc;
                allowed[cell] = 1;
            }
        }
    }
    return 0;
}

/* Unsigned integer whose ordinary order is the IEEE-754 total order of the float. */
static uint32_t total_order_key(float x) {
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

typedef struct {
    uint32_t key;
    int64_t pos;
} Cand;

/* larger key first, then lower position */
static int by_rank(const void* a, const void* b) {
    const Cand* x = (const Cand*)a;
    const Cand* y = (const Cand*)b;
    if (x->key != y->key) return x->key > y->key ? -1 : 1;
    return (x->pos > y->pos) - (x->pos < y->pos);
}

static int by_pos(const void* a, const void* b) {
    const int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
    return (x > y) - (x < y);
}

/* Selection of every row from precomputed scores.  out [rows, top_k].  Returns 0, or -1 when
 * memory runs out. */
int dsa_oracle_select(const float* scores, const uint8_t* allowed, int64_t rows, int64_t T,
                      int64_t top_k, int64_t* out) {
    Cand* cand = (Cand*)malloc((size_t)(T > 0 ? T : 1) * sizeof(Cand));
    int64_t* pick = (int64_t*)malloc((size_t)(top_k > 0 ? top_k : 1) * sizeof(int64_t));
    if (!cand || !pick) {
        free(cand);
        free(pick);
        return -1;
    }
    for (int64_t r = 0; r < rows; ++r) {
        int64_t n = 0;
        for (int64_t t = 0; t < T; ++t) {
            if (allowed[r * T + t]) {
                cand[n].key = total_order_key(scores[r * T + t]);
                cand[n].pos = t;
                ++n;
            }
        }
        qsort(cand, (size_t)n, sizeof(Cand), by_rank);
        const int64_t keep = n < top_k ? n : top_k;
        for (int64_t i = 0; i < keep; ++i) pick[i] = cand[i].pos;
        qsort(pick, (size_t)keep, sizeof(int64_t), by_pos);
        for (int64_t i = 0; i < top_k; ++i) out[r * top_k + i] = i < keep ? pick[i] : -1;
    }
    free(cand);
    free(pick);
    return 0;
}
