/*
 * moe_oracle.cpp -- plain, slow, single-threaded CPU oracle for MoE expert-parallel
 * layout, dispatch and combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  It shares no
 * code, header, table or constant generator with the GPU library: every
 * routine here is written out from the definition of the operation.
 *
 * Build: g++ -O2 -std=c++17 -ffp-contract=off -fno-fast-math -shared -fPIC
 *        (IEEE fp32 with no contraction: every fused multiply-add below is an
 *        explicit fmaf call).  Written in the plain C subset of C++: loops,
 *        arrays and the C math library, nothing that hides a step; every
 *        exported function has C linkage (extern "C") for the test harnesses.
 *
 * What is computed, and the passage each step follows:
 *   - Expert parallelism spreads the experts of one MoE layer over the ranks of
 *     a group; the number of experts must divide evenly by the group size, and
 *     each rank holds E/R local experts (delect.ru glossary "Expert parallelism
 *     (EP)", confirmed-facts section, the DeepSpeed v0.14.5 example with 8
 *     experts over 4 ranks).  Ranks own contiguous expert ids (MoonEP article,
 *     section 3, Fig. 3: rows [0,E) of the weight buffer are all ranks' local
 *     experts in order).
 *   - Dispatch moves each token's activations to its experts, combine brings
 *     the results back and merges them (same glossary, the MOELayer.forward
 *     fact; DeepEP analysis: "dispatch and combine" kernels).
 *   - Tokens are written straight into their final expert-grouped slot on the
 *     receiving rank, with static shapes and no host sync (MoonEP article,
 *     section 2, zero-copy and static layout); per-expert padding to a static
 *     shape is one of the two ways to handle dynamic routing (search-results
 *     page, the snippet on dynamic-routing limits: drop tokens or zero-pad).
 *   - Dispatch is FP8 and combine is BF16 (DeepEP analysis, feature list and
 *     both benchmark set-ups).
 *
 * Readings where the pages are silent (each listed with its reason in the
 * design notes): stable (t*K+k) order inside an expert segment; rank-major
 * then expert-ascending partitions; padding rows are neither written nor read;
 * capacity overflow and out-of-range ids are flagged, not dropped silently;
 * OCP E4M3FN with saturation to +-448 and round-to-nearest-even; q = x / scale
 * with scale = amax / 448 (both IEEE fp32 divisions); combine is an fp32 fma
 * chain over k ascending from +0.0, the shared output added after, one bf16
 * round-to-nearest-even at the end.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

extern "C" {

enum { OR_OK = 0, OR_ERR_NULL = 1, OR_ERR_SHAPE = 2 };
enum { OR_PAD_NONE = 0, OR_PAD_MULTIPLE = 1, OR_PAD_CAPACITY = 2 };
enum { OR_FLAG_BAD_EXPERT = 1, OR_FLAG_CAPACITY = 2 };

/* ------------------------------------------------------------------------ */
/* Number formats                                                             */
/* ------------------------------------------------------------------------ */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 is the upper half of an IEEE fp32 pattern. */
float oracle_f32_from_bf16(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* fp32 -> bf16, round to nearest, ties to the even pattern.
 * Written as the definition: the two bf16 neighbours of v (truncation toward
 * zero and one step away from zero), the exact distance to each in double,
 * the nearer one wins, a tie goes to the pattern with a zero last bit.
 * NaN keeps its sign and becomes the quiet pattern 0x7FC0. */
uint16_t oracle_bf16_from_f32(float v) {
    uint32_t u = bits_from_f32(v);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)(sign | 0x7FC0u);
    if ((u & 0x7FFFFFFFu) == 0x7F800000u) return (uint16_t)(u >> 16);
    uint16_t lo = (uint16_t)(u >> 16);          /* toward zero */
    if ((u & 0xFFFFu) == 0) return lo;           /* exactly representable */
    uint16_t hi = (uint16_t)(lo + 1);           /* away from zero (may be inf) */
    double av = fabs((double)v);
    double vlo = fabs((double)oracle_f32_from_bf16(lo));
    double vhi;
    if ((hi & 0x7FFFu) == 0x7F80u) vhi = ldexp(1.0, 128);  /* next step past max */
    else vhi = fabs((double)oracle_f32_from_bf16(hi));
    double dlo = av - vlo, dhi = vhi - av;
    if (dlo < dhi) return lo;
    if (dhi < dlo) return hi;
    return (lo & 1u) ? hi : lo;
}

/* Value of an OCP E4M3FN code: 1 sign, 4 exponent (bias 7), 3 mantissa bits;
 * exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no infinities. */
float oracle_f32_from_e4m3(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
    float mag;
    if (e == 0xF && m == 7) return NAN;
    if (e == 0) mag = ldexpf((float)m, -9);
    else mag = ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return s ? -mag : mag;
}

/* fp32 -> E4M3FN, round to nearest with ties to the even mantissa, saturating
 * at +-448 (the largest finite code), sign kept (so -0 and negative values
 * that round to zero give 0x80), NaN -> 0x7F. */
uint8_t oracle_e4m3_from_f32(float v) {
    if (isnan(v)) return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    float a = fabsf(v);
    if (a >= 448.0f) return (uint8_t)(sign | 0x7E);
    /* nearbyintf rounds in the current mode, which is the default
     * round-to-nearest-even; nothing here changes it. */
    if (a < 0.015625f) {                         /* below 2^-6: subnormal grid 2^-9 */
        float q = nearbyintf(a * 512.0f);        /* exact scaling, RNE to integer */
        int m = (int)q;                           /* 0..8; 8 is the smallest normal */
        return (uint8_t)(sign | m);
    }
    int e2;
    frexpf(a, &e2);                               /* a = f * 2^e2, f in [0.5,1) */
    int e = e2 - 1;                               /* a in [2^e, 2^(e+1)) */
    float frac = (ldexpf(a, -e) - 1.0f) * 8.0f;   /* exact: mantissa in eighths */
    int m = (int)nearbyintf(frac);                /* RNE: 0..8 */
    if (m == 8) { m = 0; e += 1; }
    int ef = e + 7;
    if (ef > 15 || (ef == 15 && m == 7)) return (uint8_t)(sign | 0x7E);
    return (uint8_t)(sign | (ef << 3) | m);
}

/* ------------------------------------------------------------------------ */
/* Layout                                                                     */
/* ------------------------------------------------------------------------ */

static int shape_ok(int S, int K, int E, int R, int pad_mode, int pad_rows) {
    if (S < 0 || K < 1 || K > 16 || E < 1 || E > 1024 || R < 1 || E % R) return 0;
    if (pad_mode != OR_PAD_NONE && pad_mode != OR_PAD_MULTIPLE && pad_mode != OR_PAD_CAPACITY) return 0;
    if (pad_mode != OR_PAD_NONE && pad_rows < 1) return 0;
    if ((int64_t)S * K >= ((int64_t)1 << 31)) return 0;
    return 1;
}

/* Rows a receive buffer must hold for every possible routing of S*K entries:
 * S*K without padding, S*K + E*(p-1) when each segment is rounded up to a
 * multiple of p, E*cap with a fixed capacity per expert.  -1 on bad shape. */
int64_t oracle_max_recv_rows(int S, int K, int E, int R, int pad_mode, int pad_rows) {
    if (!shape_ok(S, K, E, R, pad_mode, pad_rows)) return -1;
    int64_t n = (int64_t)S * K, rows = n;
    if (pad_mode == OR_PAD_MULTIPLE) rows = n + (int64_t)E * (pad_rows - 1);
    if (pad_mode == OR_PAD_CAPACITY) rows = (int64_t)E * pad_rows;
    if (rows >= ((int64_t)1 << 31)) return -1;   /* rows are int32 indices */
    return rows;
}

/* Layout of the receive buffer for one batch of top-k routing.
 *   topk_idx [S*K]          expert id of entry (t,k) at t*K+k
 *   tokens_per_expert [E]   rows placed in expert e's segment
 *   tokens_per_rank [R]     sum of tokens_per_expert over the rank's experts
 *   expert_offset [E+1]     start row of each (padded) expert segment
 *   rank_offset [R+1]       start row of each rank's partition
 *   pos [S*K]               receive row of entry (t,k), or -1 if not placed
 *   src [max_recv]          entry t*K+k held by each row, -1 for unused rows
 *   status [1]              OR of OR_FLAG_* seen in the data
 */
int oracle_layout(const int32_t *topk_idx, int S, int K, int E, int R, int pad_mode, int pad_rows,
                  int32_t *tokens_per_expert, int32_t *tokens_per_rank, int32_t *expert_offset,
                  int32_t *rank_offset, int32_t *pos, int32_t *src, int32_t *status) {
    if (oracle_max_recv_rows(S, K, E, R, pad_mode, pad_rows) < 0) return OR_ERR_SHAPE;
    if ((S > 0 && (!topk_idx || !pos)) || !tokens_per_expert || !tokens_per_rank ||
        !expert_offset || !rank_offset || !src || !status)
        return OR_ERR_NULL;
    int64_t max_recv = oracle_max_recv_rows(S, K, E, R, pad_mode, pad_rows);
    int64_t n = (int64_t)S * K;
    int32_t flags = 0;

    /* count[e]: entries routed to e, scanning t ascending then k ascending */
    int64_t *count = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    for (int64_t i = 0; i < n; ++i) {
        int32_t e = topk_idx[i];
        if (e < 0 || e >= E) { flags |= OR_FLAG_BAD_EXPERT; continue; }
        count[e] += 1;
    }

    /* placed rows and padded segment length per expert */
    int64_t *seg = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    for (int e = 0; e < E; ++e) {
        int64_t placed = count[e];
        if (pad_mode == OR_PAD_CAPACITY && placed > pad_rows) {
            flags |= OR_FLAG_CAPACITY;
            placed = pad_rows;
        }
        tokens_per_expert[e] = (int32_t)placed;
        if (pad_mode == OR_PAD_NONE) seg[e] = count[e];
        else if (pad_mode == OR_PAD_MULTIPLE) seg[e] = (count[e] + pad_rows - 1) / pad_rows * pad_rows;
        else seg[e] = pad_rows;
    }

    /* exclusive scan of segment lengths over expert ids */
    int64_t run = 0;
    for (int e = 0; e < E; ++e) { expert_offset[e] = (int32_t)run; run += seg[e]; }
    expert_offset[E] = (int32_t)run;

    /* ranks own E/R consecutive experts */
    int epr = E / R;
    for (int r = 0; r < R; ++r) {
        int64_t s = 0;
        for (int j = 0; j < epr; ++j) s += tokens_per_expert[r * epr + j];
        tokens_per_rank[r] = (int32_t)s;
        rank_offset[r] = expert_offset[r * epr];
    }
    rank_offset[R] = expert_offset[E];

    /* stable placement: entries keep their t*K+k order inside a segment */
    for (int64_t row = 0; row < max_recv; ++row) src[row] = -1;
    int64_t *cursor = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    for (int64_t i = 0; i < n; ++i) {
        int32_t e = topk_idx[i];
        if (e < 0 || e >= E) { pos[i] = -1; continue; }
        if (cursor[e] >= tokens_per_expert[e]) { pos[i] = -1; continue; } /* over capacity */
        int64_t row = expert_offset[e] + cursor[e];
        cursor[e] += 1;
        pos[i] = (int32_t)row;
        src[row] = (int32_t)i;
    }
    status[0] |= flags;
    free(count); free(seg); free(cursor);
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Dispatch                                                                   */
/* ------------------------------------------------------------------------ */

/* bf16 dispatch: recv[pos[t,k]] = hidden[t] bit for bit; recv_w[pos[t,k]] =
 * topk_w[t,k] when both weight pointers are given. */
int oracle_dispatch_bf16(const uint16_t *hidden, int S, int H, int K, const int32_t *pos,
                         const float *topk_w, uint16_t *recv, float *recv_w) {
    if (S < 0 || H < 1 || K < 1) return OR_ERR_SHAPE;
    for (int t = 0; t < S; ++t)
        for (int k = 0; k < K; ++k) {
            int32_t p = pos[(int64_t)t * K + k];
            if (p < 0) continue;
            memcpy(recv + (int64_t)p * H, hidden + (int64_t)t * H, (size_t)H * 2);
            if (topk_w && recv_w) recv_w[p] = topk_w[(int64_t)t * K + k];
        }
    return OR_OK;
}

/* FP8 quantisation of one token row, 128 channels per block:
 *   amax = max |x| over the block; scale = amax / 448 (fp32 division);
 *   code = E4M3FN(x / scale) (fp32 division, then the rounding above);
 *   an all-zero block gets scale 0 and codes 0x00.
 * codes [H], scales [H/128]. */
int oracle_quantize_row_fp8(const uint16_t *x, int H, uint8_t *codes, float *scales) {
    if (H < 128 || H % 128) return OR_ERR_SHAPE;
    for (int b = 0; b < H / 128; ++b) {
        float amax = 0.0f;
        for (int c = 0; c < 128; ++c) {
            float a = fabsf(oracle_f32_from_bf16(x[b * 128 + c]));
            if (a > amax) amax = a;
        }
        if (amax == 0.0f) {
            scales[b] = 0.0f;
            for (int c = 0; c < 128; ++c) codes[b * 128 + c] = 0x00;
            continue;
        }
        float scale = amax / 448.0f;
        scales[b] = scale;
        for (int c = 0; c < 128; ++c)
            codes[b * 128 + c] = oracle_e4m3_from_f32(oracle_f32_from_bf16(x[b * 128 + c]) / scale);
    }
    return OR_OK;
}

/* FP8 dispatch: each token row is quantised once and its codes and scales are
 * written to every row pos[t,k]. recv [max_recv, H] bytes, recv_scales
 * [max_recv, H/128] fp32. */
int oracle_dispatch_fp8(const uint16_t *hidden, int S, int H, int K, const int32_t *pos,
                        const float *topk_w, uint8_t *recv, float *recv_scales, float *recv_w) {
    if (S < 0 || H < 128 || H % 128 || K < 1) return OR_ERR_SHAPE;
    uint8_t *codes = (uint8_t *)malloc((size_t)H);
    float *scales = (float *)malloc((size_t)(H / 128) * sizeof(float));
    for (int t = 0; t < S; ++t) {
        oracle_quantize_row_fp8(hidden + (int64_t)t * H, H, codes, scales);
        for (int k = 0; k < K; ++k) {
            int32_t p = pos[(int64_t)t * K + k];
            if (p < 0) continue;
            memcpy(recv + (int64_t)p * H, codes, (size_t)H);
            memcpy(recv_scales + (int64_t)p * (H / 128), scales, (size_t)(H / 128) * sizeof(float));
            if (topk_w && recv_w) recv_w[p] = topk_w[(int64_t)t * K + k];
        }
    }
    free(codes); free(scales);
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Combine                                                                    */
/* ------------------------------------------------------------------------ */

/* out[t,c] = bf16( fma chain over k = 0..K-1 of w[t,k] * y[pos[t,k], c],
 *                  starting from +0.0, plus shared[t,c] if given ).
 * Entries with pos = -1 are skipped; w = NULL means every weight is 1. */
int oracle_combine(const uint16_t *expert_out, int S, int H, int K, const int32_t *pos,
                   const float *w, const uint16_t *shared, uint16_t *out) {
    if (S < 0 || H < 1 || K < 1) return OR_ERR_SHAPE;
    for (int t = 0; t < S; ++t)
        for (int c = 0; c < H; ++c) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                int32_t p = pos[(int64_t)t * K + k];
                if (p < 0) continue;
                float wk = w ? w[(int64_t)t * K + k] : 1.0f;
                acc = fmaf(wk, oracle_f32_from_bf16(expert_out[(int64_t)p * H + c]), acc);
            }
            if (shared) acc = acc + oracle_f32_from_bf16(shared[(int64_t)t * H + c]);
            out[(int64_t)t * H + c] = oracle_bf16_from_f32(acc);
        }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Array helpers for the tests (loops over the scalar routines above)         */
/* ------------------------------------------------------------------------ */

void oracle_bf16_from_f32_n(const float *v, int64_t n, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_from_f32(v[i]);
}

void oracle_e4m3_from_f32_n(const float *v, int64_t n, uint8_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_from_f32(v[i]);
}

/* Stand-in identity expert for FP8 rows, used to feed combine in round-trip
 * tests: y = bf16(value(code) * scale), one fp32 product and one rounding per
 * element.  codes [rows, H], scales [rows, H/128], y [rows, H]. */
void oracle_dequant_identity(const uint8_t *codes, const float *scales, int64_t rows, int H,
                             uint16_t *y) {
    for (int64_t r = 0; r < rows; ++r)
        for (int c = 0; c < H; ++c) {
            float v = oracle_f32_from_e4m3(codes[r * H + c]) * scales[r * (H / 128) + c / 128];
            y[r * H + c] = oracle_bf16_from_f32(v);
        }
}

/* Zero padding (optional, after dispatch): static per-expert segments are
 * filled up with zeros (search-results page, the snippet on dynamic-routing
 * limits: tokens are dropped or segments zero-padded).  Every receive row that
 * no entry maps to (src[r] = -1: padding inside a segment and the unused tail)
 * becomes all-zero bytes, and with FP8 its scale row becomes 0.0f; rows that
 * hold an entry are left as they are.  recv [rows, row_bytes] bytes,
 * scales [rows, nsc] or NULL. */
void oracle_zero_padding(const int32_t *src, int64_t rows, int64_t row_bytes, uint8_t *recv, float *scales,
                         int nsc) {
    for (int64_t r = 0; r < rows; ++r) {
        if (src[r] >= 0) continue;
        for (int64_t b = 0; b < row_bytes; ++b) recv[r * row_bytes + b] = 0;
        if (scales != NULL)
            for (int j = 0; j < nsc; ++j) scales[r * nsc + j] = 0.0f;
    }
}

/* ------------------------------------------------------------------------ */
/* Balanced layout (redundant expert slots)                                   */
/* ------------------------------------------------------------------------ */
/* Every rank receives the same number of rows however skewed the routing:
 * ranks whose own experts hold more entries than their quota hand the surplus
 * to replicas of those experts placed in free slots of ranks below their quota
 * (MoonEP article, section 1 "perfect balance": each rank receives exactly
 * S*K rows through a few redundant experts planned online; section 3, Fig. 3:
 * each rank holds its local experts followed by B prefetch slots).  The pages
 * do not give the planning rule; this is the plain greedy reading:
 *   quota q[r] = N/R, plus one for the first N%R ranks (N = valid entries);
 *   source ranks in ascending order; inside a rank its experts by count,
 *   largest first (ties: lower id); each expert sheds what its rank still has
 *   to shed, at most all its entries;
 *   each shed amount goes to the lowest destination rank that still has room
 *   (below its quota) and a free slot, as much as that room allows, then the
 *   next destination; each (expert, destination) piece takes one slot;
 *   if no destination is left the rest stays home and the layout is flagged.
 * Entries of an expert keep their t*K+k order: the first ones stay home, the
 * following ones fill the expert's replicas in the order they were created.
 * Rows: rank-major; inside a rank its E/R home segments in expert order, then
 * its B slot segments in slot order.
 *   seg_offset  [R*(E/R+B)+1]  first row of each (rank, segment)
 *   slot_expert [R*B]          expert replicated in each slot, -1 if unused
 *   expert_offset [E+1]        first row of each expert's home segment; [E] = rows
 * Other outputs as in oracle_layout (no padding; max rows = S*K). */
enum { OR_FLAG_UNBALANCED = 4 };

int oracle_layout_balanced(const int32_t *topk_idx, int S, int K, int E, int R, int B,
                           int32_t *tokens_per_expert, int32_t *tokens_per_rank,
                           int32_t *expert_offset, int32_t *rank_offset, int32_t *pos,
                           int32_t *src, int32_t *seg_offset, int32_t *slot_expert,
                           int32_t *status) {
    if (!shape_ok(S, K, E, R, OR_PAD_NONE, 0) || B < 0 || B > 64) return OR_ERR_SHAPE;
    const int64_t n = (int64_t)S * K;
    const int epr = E / R, nseg = epr + B;
    int32_t flags = 0;

    int64_t *count = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    for (int64_t i = 0; i < n; ++i) {
        int32_t e = topk_idx[i];
        if (e < 0 || e >= E) { flags |= OR_FLAG_BAD_EXPERT; continue; }
        count[e] += 1;
    }
    int64_t valid = 0;
    for (int e = 0; e < E; ++e) valid += count[e];

    /* quotas and deficits */
    int64_t *room = (int64_t *)calloc((size_t)R, sizeof(int64_t));   /* quota - load, may be < 0 */
    for (int r = 0; r < R; ++r) {
        int64_t quota = valid / R + (r < valid % R ? 1 : 0);
        int64_t load = 0;
        for (int j = 0; j < epr; ++j) load += count[r * epr + j];
        room[r] = quota - load;
    }

    /* replicas: expert, destination rank, slot, number of entries */
    int max_rep = R * B;
    int *rep_e = (int *)malloc(sizeof(int) * (size_t)(max_rep + 1));
    int *rep_r = (int *)malloc(sizeof(int) * (size_t)(max_rep + 1));
    int *rep_s = (int *)malloc(sizeof(int) * (size_t)(max_rep + 1));
    int64_t *rep_n = (int64_t *)malloc(sizeof(int64_t) * (size_t)(max_rep + 1));
    int nrep = 0;
    int *slots_used = (int *)calloc((size_t)R, sizeof(int));
    int64_t *home = (int64_t *)malloc(sizeof(int64_t) * (size_t)E);
    for (int e = 0; e < E; ++e) home[e] = count[e];
    int *order = (int *)malloc(sizeof(int) * (size_t)epr);

    for (int r = 0; r < R; ++r) {
        int64_t surplus = -room[r];
        if (surplus <= 0) continue;
        /* this rank's experts, largest count first, ties by lower id (insertion sort) */
        for (int j = 0; j < epr; ++j) {
            int e = r * epr + j, at = j;
            while (at > 0 && count[order[at - 1]] < count[e]) { order[at] = order[at - 1]; --at; }
            order[at] = e;
        }
        for (int j = 0; j < epr && surplus > 0; ++j) {
            int e = order[j];
            int64_t shed = home[e] < surplus ? home[e] : surplus;
            while (shed > 0) {
                int d = -1;
                for (int cand = 0; cand < R; ++cand)
                    if (room[cand] > 0 && slots_used[cand] < B) { d = cand; break; }
                if (d < 0) { flags |= OR_FLAG_UNBALANCED; goto planned; }
                int64_t take = shed < room[d] ? shed : room[d];
                rep_e[nrep] = e; rep_r[nrep] = d; rep_s[nrep] = slots_used[d]; rep_n[nrep] = take;
                nrep += 1;
                slots_used[d] += 1;
                room[d] -= take;
                home[e] -= take;
                shed -= take;
                surplus -= take;
                room[r] += take;
            }
        }
    }
planned:;
    /* segment sizes, scan */
    int64_t *seg = (int64_t *)calloc((size_t)R * nseg, sizeof(int64_t));
    for (int e = 0; e < E; ++e) seg[(int64_t)(e / epr) * nseg + (e % epr)] = home[e];
    for (int i = 0; i < R * B; ++i) slot_expert[i] = -1;
    for (int q = 0; q < nrep; ++q) {
        seg[(int64_t)rep_r[q] * nseg + epr + rep_s[q]] = rep_n[q];
        slot_expert[rep_r[q] * B + rep_s[q]] = rep_e[q];
    }
    int64_t run = 0;
    for (int64_t g = 0; g < (int64_t)R * nseg; ++g) { seg_offset[g] = (int32_t)run; run += seg[g]; }
    seg_offset[(int64_t)R * nseg] = (int32_t)run;
    for (int r = 0; r < R; ++r) {
        rank_offset[r] = seg_offset[(int64_t)r * nseg];
        tokens_per_rank[r] = seg_offset[(int64_t)(r + 1) * nseg] - seg_offset[(int64_t)r * nseg];
    }
    rank_offset[R] = (int32_t)run;
    for (int e = 0; e < E; ++e) {
        tokens_per_expert[e] = (int32_t)count[e];
        expert_offset[e] = seg_offset[(int64_t)(e / epr) * nseg + (e % epr)];
    }
    expert_offset[E] = (int32_t)run;

    /* place entries: per expert, the first home[e] stay, the rest fill its replicas in order */
    for (int64_t row = 0; row < n; ++row) src[row] = -1;
    int64_t *seen = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    for (int64_t i = 0; i < n; ++i) {
        int32_t e = topk_idx[i];
        if (e < 0 || e >= E) { pos[i] = -1; continue; }
        int64_t k = seen[e]++;
        int64_t row;
        if (k < home[e]) {
            row = expert_offset[e] + k;
        } else {
            k -= home[e];
            row = -1;
            for (int q = 0; q < nrep && row < 0; ++q) {
                if (rep_e[q] != e) continue;
                if (k < rep_n[q]) row = seg_offset[(int64_t)rep_r[q] * nseg + epr + rep_s[q]] + k;
                else k -= rep_n[q];
            }
        }
        pos[i] = (int32_t)row;
        src[row] = (int32_t)i;
    }
    status[0] |= flags;
    free(count); free(room); free(rep_e); free(rep_r); free(rep_s); free(rep_n); free(slots_used);
    free(home); free(order); free(seg); free(seen);
    return OR_OK;
}

}  // extern "C"
