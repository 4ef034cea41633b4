/* Memory and undefined-behaviour check of the CPU oracle (test infrastructure).
 *
 * Built by tests/test_oracle_sanitize.py with -fsanitize=address,undefined
 * and linked with oracle/moe_oracle.cpp (whose functions have C linkage), and
 * run on the host.  Every output buffer
 * is allocated at exactly the size the oracle's header comments state, so an
 * access one element past it stops the program; each call's results are also
 * checked against the invariants that hold for any input (every valid entry
 * placed once or reported, src and pos inverse to each other, counts adding
 * up).  The oracle's prototypes are declared here; nothing is shared with the
 * GPU library.  Exit status 0 means every case passed.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t oracle_max_recv_rows(int S, int K, int E, int R, int pad_mode, int pad_rows);
int oracle_layout(const int32_t *topk_idx, int S, int K, int E, int R, int pad_mode, int pad_rows,
                  int32_t *tokens_per_expert, int32_t *tokens_per_rank, int32_t *expert_offset,
                  int32_t *rank_offset, int32_t *pos, int32_t *src, int32_t *status);
int oracle_dispatch_bf16(const uint16_t *hidden, int S, int H, int K, const int32_t *pos,
                         const float *topk_w, uint16_t *recv, float *recv_w);
int oracle_dispatch_fp8(const uint16_t *hidden, int S, int H, int K, const int32_t *pos,
                        const float *topk_w, uint8_t *recv, float *recv_scales, float *recv_w);
int oracle_combine(const uint16_t *expert_out, int S, int H, int K, const int32_t *pos,
                   const float *w, const uint16_t *shared, uint16_t *out);
void oracle_dequant_identity(const uint8_t *codes, const float *scales, int64_t rows, int H, uint16_t *y);
void oracle_zero_padding(const int32_t *src, int64_t rows, int64_t row_bytes, uint8_t *recv, float *scales,
                         int nsc);
int oracle_layout_balanced(const int32_t *topk_idx, int S, int K, int E, int R, int B,
                           int32_t *tokens_per_expert, int32_t *tokens_per_rank,
                           int32_t *expert_offset, int32_t *rank_offset, int32_t *pos,
                           int32_t *src, int32_t *seg_offset, int32_t *slot_expert,
                           int32_t *status);
float oracle_f32_from_bf16(uint16_t h);
uint16_t oracle_bf16_from_f32(float v);
float oracle_f32_from_e4m3(uint8_t c);
uint8_t oracle_e4m3_from_f32(float v);

/* splitmix64 (Steele, Lea and Flood, 2014) */
static uint64_t rng_state;
static uint64_t next_u64(void) {
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static int below(int n) { return (int)(next_u64() % (uint64_t)n); }

static int failures = 0;
#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                  \
            fputc('\n', stderr);                           \
            ++failures;                                    \
        }                                                  \
    } while (0)

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}

/* layout + dispatch (both formats) + combine + zero padding on one shape */
static void run_shape(int S, int K, int E, int R, int pad_mode, int pad_rows, int H, int bad) {
    const int64_t rows = oracle_max_recv_rows(S, K, E, R, pad_mode, pad_rows);
    CHECK(rows >= 0, "shape S=%d K=%d E=%d R=%d pad=%d/%d refused", S, K, E, R, pad_mode, pad_rows);
    if (rows < 0) return;
    const int n = S * K;
    int32_t *idx = xmalloc(sizeof(int32_t) * n);
    for (int i = 0; i < n; ++i) idx[i] = below(E);
    for (int b = 0; b < bad && n > 0; ++b) idx[below(n)] = below(2) ? -1 - below(3) : E + below(3);
    int32_t *tpe = xmalloc(sizeof(int32_t) * E), *tpr = xmalloc(sizeof(int32_t) * R);
    int32_t *eoff = xmalloc(sizeof(int32_t) * (E + 1)), *roff = xmalloc(sizeof(int32_t) * (R + 1));
    int32_t *pos = xmalloc(sizeof(int32_t) * n), *src = xmalloc(sizeof(int32_t) * rows), status = -7;
    int rc = oracle_layout(idx, S, K, E, R, pad_mode, pad_rows, tpe, tpr, eoff, roff, pos, src, &status);
    CHECK(rc == 0, "oracle_layout rc %d", rc);
    int64_t placed = 0, total = 0;
    for (int e = 0; e < E; ++e) total += tpe[e];
    for (int i = 0; i < n; ++i) {
        if (pos[i] < 0) continue;
        ++placed;
        CHECK(pos[i] < rows && src[pos[i]] == i, "pos/src not inverse at entry %d", i);
    }
    CHECK(placed == total, "placed %lld, counts add to %lld", (long long)placed, (long long)total);
    CHECK(eoff[E] <= rows && roff[R] == eoff[E], "offsets past the buffer");
    CHECK(bad == 0 || (status & 1), "bad ids not reported");

    uint16_t *hid = xmalloc(sizeof(uint16_t) * (size_t)S * H);
    for (int64_t i = 0; i < (int64_t)S * H; ++i) hid[i] = (uint16_t)(0x3000 + below(0x2000)) ^ (uint16_t)(below(2) << 15);
    float *w = xmalloc(sizeof(float) * n);
    for (int i = 0; i < n; ++i) w[i] = (float)below(1000) / 1000.0f;
    uint16_t *recv = xmalloc(sizeof(uint16_t) * (size_t)rows * H);
    float *recv_w = xmalloc(sizeof(float) * rows);
    rc = oracle_dispatch_bf16(hid, S, H, K, pos, w, recv, recv_w);
    CHECK(rc == 0, "oracle_dispatch_bf16 rc %d", rc);
    for (int i = 0; i < n; ++i)
        if (pos[i] >= 0) CHECK(memcmp(recv + (size_t)pos[i] * H, hid + (size_t)(i / K) * H, 2 * (size_t)H) == 0,
                               "bf16 row of entry %d", i);
    uint16_t *out = xmalloc(sizeof(uint16_t) * (size_t)S * H);
    rc = oracle_combine(recv, S, H, K, pos, w, NULL, out);
    CHECK(rc == 0, "oracle_combine rc %d", rc);
    rc = oracle_combine(recv, S, H, K, pos, NULL, hid, out);
    CHECK(rc == 0, "oracle_combine (shared, no weights) rc %d", rc);
    oracle_zero_padding(src, rows, 2 * (int64_t)H, (uint8_t *)recv, NULL, 0);
    for (int64_t r = 0; r < rows; ++r)
        if (src[r] < 0)
            for (int c = 0; c < H; ++c) CHECK(recv[(size_t)r * H + c] == 0, "padding row %lld not zero", (long long)r);

    if (H % 128 == 0) {
        const int nsc = H / 128;
        uint8_t *rq = xmalloc((size_t)rows * H);
        float *rs = xmalloc(sizeof(float) * (size_t)rows * nsc);
        rc = oracle_dispatch_fp8(hid, S, H, K, pos, w, rq, rs, recv_w);
        CHECK(rc == 0, "oracle_dispatch_fp8 rc %d", rc);
        uint16_t *y = xmalloc(sizeof(uint16_t) * (size_t)rows * H);
        oracle_dequant_identity(rq, rs, rows, H, y);
        oracle_zero_padding(src, rows, H, rq, rs, nsc);
        free(rq); free(rs); free(y);
    }
    free(idx); free(tpe); free(tpr); free(eoff); free(roff); free(pos); free(src);
    free(hid); free(w); free(recv); free(recv_w); free(out);
}

static void run_balanced(int S, int K, int E, int R, int B, int bad) {
    const int n = S * K, epr = E / R, ngrp = R * (epr + B);
    int32_t *idx = xmalloc(sizeof(int32_t) * n);
    for (int i = 0; i < n; ++i) idx[i] = below(3) ? below(E > 4 ? E / 4 : E) : below(E);  /* skewed */
    for (int b = 0; b < bad && n > 0; ++b) idx[below(n)] = E + 1;
    int32_t *tpe = xmalloc(sizeof(int32_t) * E), *tpr = xmalloc(sizeof(int32_t) * R);
    int32_t *eoff = xmalloc(sizeof(int32_t) * (E + 1)), *roff = xmalloc(sizeof(int32_t) * (R + 1));
    int32_t *pos = xmalloc(sizeof(int32_t) * n), *src = xmalloc(sizeof(int32_t) * n);
    int32_t *seg = xmalloc(sizeof(int32_t) * (ngrp + 1)), *slot = xmalloc(sizeof(int32_t) * (R * B)), status = -7;
    const int rc = oracle_layout_balanced(idx, S, K, E, R, B, tpe, tpr, eoff, roff, pos, src, seg, slot, &status);
    CHECK(rc == 0, "oracle_layout_balanced rc %d (S=%d K=%d E=%d R=%d B=%d)", rc, S, K, E, R, B);
    int64_t placed = 0;
    for (int i = 0; i < n; ++i) {
        if (pos[i] < 0) continue;
        ++placed;
        CHECK(pos[i] < n && src[pos[i]] == i, "balanced pos/src not inverse at entry %d", i);
    }
    int64_t per_rank = 0;
    for (int r = 0; r < R; ++r) per_rank += tpr[r];
    CHECK(per_rank == placed, "balanced rank totals %lld, placed %lld", (long long)per_rank, (long long)placed);
    free(idx); free(tpe); free(tpr); free(eoff); free(roff); free(pos); free(src); free(seg); free(slot);
}

int main(void) {
    rng_state = 20261203u;
    /* every bf16 pattern through both converters */
    for (uint32_t h = 0; h < 65536; ++h) {
        const float v = oracle_f32_from_bf16((uint16_t)h);
        (void)oracle_bf16_from_f32(v);
        (void)oracle_f32_from_e4m3(oracle_e4m3_from_f32(v));
    }
    /* fixed edge shapes: empty batch, one entry, K = E, capacity overflow, bad ids */
    run_shape(0, 4, 8, 2, 0, 0, 128, 0);
    run_shape(0, 4, 8, 2, 2, 3, 128, 0);
    run_shape(1, 1, 1, 1, 0, 0, 8, 0);
    run_shape(5, 4, 4, 2, 1, 3, 16, 0);
    run_shape(40, 8, 16, 4, 2, 4, 128, 3);
    run_shape(33, 3, 12, 3, 1, 5, 256, 2);
    /* seeded random shapes in every pad mode */
    for (int c = 0; c < 2000; ++c) {
        const int R = 1 + below(8), E = R * (1 + below(16)), K = 1 + below(8);
        const int S = below(40), pad_mode = below(3);
        const int pad_rows = pad_mode == 0 ? 0 : 1 + below(12);
        const int H = below(2) ? 128 * (1 + below(2)) : 8 * (1 + below(6));
        run_shape(S, K, E, R, pad_mode, pad_rows, H, below(3) == 0 ? 1 + below(3) : 0);
    }
    for (int c = 0; c < 2000; ++c) {
        const int R = 1 + below(8), E = R * (1 + below(8)), K = 1 + below(6);
        run_balanced(below(60), K, E, R, below(9), below(4) == 0);
    }
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer run: all cases passed\n");
    return 0;
}
