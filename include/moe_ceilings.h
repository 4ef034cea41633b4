/* moe_ceilings.h -- pattern-ceiling kernels (libmoe_ceilings.so).
 *
 * Measurement infrastructure beside the MoE layout / dispatch / combine
 * library: streaming kernels that move bytes in the access patterns of the
 * dispatch and combine kernels with no arithmetic, so a benchmark can state
 * what HBM sustains for each pattern on the GPU at hand.  The hot path never
 * calls them.
 *
 * Dispatch writes each token row into the K expert-grouped receive rows its
 * routed entries were given, in FP8 or bf16, and combine gathers the K rows
 * back (DeepEP analysis page, the "dispatch" and "combine" kernels and both
 * benchmark set-ups: FP8 dispatch, BF16 combine; MoonEP article, section 2:
 * rows written straight into their final slot).
 *
 * Every call is asynchronous on `stream` (a hipStream_t, NULL for the null
 * stream).  Pointers are device pointers, 16-byte aligned; the caller owns
 * every buffer; nothing is allocated.  Arguments are checked before any
 * launch: MOE_CEIL_ERR_ARG for a bad one, MOE_CEIL_ERR_HIP when the launch
 * fails.
 */
#ifndef MOE_CEILINGS_H
#define MOE_CEILINGS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MOE_CEIL_OK = 0, MOE_CEIL_ERR_ARG = 1, MOE_CEIL_ERR_HIP = 2 };

/* Streaming read of `bytes` from src: each wave reads vec_per_lane KiB
 * contiguously (16 bytes per lane per load, every load issued before any
 * use), waves_per_group waves per workgroup.  load_kind 0 = ordinary load,
 * 1 = non-temporal.  vec_per_lane in {1,2,4,8,16}, waves_per_group in
 * [1,16], bytes a multiple of 1 KiB * vec_per_lane * waves_per_group.  The
 * data is kept live through `sink` (16 bytes), written only if the XOR of the
 * values read equals 0x5EEDF00D in every word. */
int32_t moe_ceiling_read(const void *src, int64_t bytes, int32_t vec_per_lane, int32_t waves_per_group,
                         int32_t load_kind, void *sink, void *stream);

/* Streaming write of `bytes` to dst, the same shapes as moe_ceiling_read.
 * store_kind 0 = ordinary store, 1 = non-temporal, 2 = buffer store with the
 * SC1 cache-policy bit. */
int32_t moe_ceiling_write(void *dst, int64_t bytes, int32_t vec_per_lane, int32_t waves_per_group,
                          int32_t store_kind, void *stream);

/* The dispatch pattern: for each token t < S and each 1 KiB chunk of an output
 * row, one wave reads the matching in_row_bytes/out_row_bytes KiB of src row t
 * ([S, in_row_bytes]) and stores 1 KiB to dst row rows[t*K+k]
 * ([*, out_row_bytes]) for every k with rows[t*K+k] >= 0 (non-temporal
 * stores).  With `scales` ([*, out_row_bytes/128] fp32, or NULL) one lane in 8
 * also stores a 4-byte value per 128 output bytes, as FP8 dispatch does.
 * A workgroup holds waves_per_group (1..4, dividing the chunks per row)
 * waves on consecutive chunks of one token (1: the dispatch kernels' shape).
 * in_row_bytes is out_row_bytes (bf16 dispatch) or twice it (FP8 dispatch);
 * out_row_bytes is a multiple of 1024; K in {1,2,4,6,8}.  Every rows entry
 * must be -1 or a row of dst. */
int32_t moe_ceiling_scatter(const void *src, int32_t S, int32_t in_row_bytes, int32_t K, const int32_t *rows,
                            void *dst, int32_t out_row_bytes, float *scales, int32_t waves_per_group, void *stream);

/* The combine pattern: for each token t < S and each vec_per_lane KiB chunk of
 * a row, one single-wave workgroup issues non-temporal loads of that chunk of
 * y row rows[t*K+k] for every k with rows[t*K+k] >= 0 (all before any use),
 * XORs them and stores the chunk of out row t ([S, row_bytes]) with
 * store_kind as in moe_ceiling_write.  row_bytes a multiple of
 * 1 KiB * vec_per_lane, vec_per_lane in {1,2}, K in {1,2,4,6,8}.  Every rows
 * entry must be -1 or a row of y. */
int32_t moe_ceiling_gather(const void *y, int32_t S, int32_t row_bytes, int32_t K, const int32_t *rows,
                           int32_t vec_per_lane, int32_t store_kind, void *out, void *stream);

/* The dispatch bytes in row order through LDS: one workgroup of K waves per
 * token loads the token row (src row t) into LDS, each wave a 1/K share, then
 * wave k stores the whole out_row_bytes row contiguously to dst row
 * rows[t*K+k] (non-temporal), plus the 4-byte values per 128 output bytes
 * into `scales` when given, as moe_ceiling_scatter does.  Same output as
 * moe_ceiling_scatter.  K in {6, 8}; out_row_bytes a multiple of 1024, at
 * most 64 KiB (the LDS row); in_row_bytes as in moe_ceiling_scatter. */
int32_t moe_ceiling_scatter_rows(const void *src, int32_t S, int32_t in_row_bytes, int32_t K, const int32_t *rows,
                                 void *dst, int32_t out_row_bytes, float *scales, void *stream);

/* The combine pattern with the gathers' cache-policy operand given:
 * load_policy is the buffer load's operand (0 none, 2 NT, 3 NT+SC0, 18 NT+SC1,
 * 19 NT+SC0+SC1); the output store carries SC1.  Same output as
 * moe_ceiling_gather (vec_per_lane 1).  K = 8. */
int32_t moe_ceiling_gather_policy(const void *y, int32_t S, int32_t row_bytes, int32_t K, const int32_t *rows,
                                  int32_t load_policy, void *out, void *stream);

/* The combine pattern in persistent form: `groups` workgroups of
 * waves_per_group waves (1..4) walk the same (token, 1 KiB chunk) units as
 * moe_ceiling_gather (chunk-fastest), each wave keeping the next unit's K row
 * loads in flight while it combines and stores the current one.  Same
 * output as moe_ceiling_gather with vec_per_lane 1.  K in {6, 8}; store_kind
 * as in moe_ceiling_write (K = 6: SC1 only). */
int32_t moe_ceiling_gather_persistent(const void *y, int32_t S, int32_t row_bytes, int32_t K, const int32_t *rows,
                                      int32_t groups, int32_t waves_per_group, int32_t store_kind, void *out,
                                      void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_CEILINGS_H */
