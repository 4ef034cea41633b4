/*
 * moe_ep.h -- C ABI of the MI355X (gfx950) MoE expert-parallel layout,
 * dispatch and combine library (libmoe_ep.so).
 *
 * The three calls are the data-parallel hot path of expert parallelism:
 *
 *   moe_layout    top-k routing -> per-expert / per-rank counts, padded segment
 *                 offsets, and the maps between (token, k) entries and rows of
 *                 the receive buffer.
 *   moe_dispatch  token rows -> rows of the expert-grouped, rank-partitioned
 *                 receive buffer, bit-copied bf16 or FP8 E4M3 with one fp32
 *                 scale per 128 channels.
 *   moe_combine   expert output rows -> token order, as the route-weighted sum
 *                 of each token's K rows (fp32 accumulation), plus an optional
 *                 shared-expert output.
 *
 * Around them: moe_layout_dispatch (layout + dispatch in one launch for
 * decode-sized batches), moe_layout_balanced (every rank receives the same
 * number of rows through redundant-expert slots), moe_zero_padding (optional
 * zero fill of padding rows), moe_stream_create_cu_limited /
 * moe_stream_create_cu_range / moe_stream_destroy (a stream confined to a set
 * of CUs), and the sizing helpers
 * moe_max_recv_rows, moe_layout_workspace_bytes,
 * moe_layout_balanced_workspace_bytes, plus moe_status_str.
 *
 * What the operations are (passages):
 *   - Experts of a layer are spread over the ranks of an EP group; E must
 *     divide by the group size R and each rank holds E/R local experts
 *     (delect.ru glossary "Expert parallelism (EP)", confirmed facts: the
 *     DeepSpeed v0.14.5 example, 8 experts on 4 ranks).  Rank r owns experts
 *     [r*E/R, (r+1)*E/R) (MoonEP article, section 3 and Fig. 3: rows [0,E) of
 *     the weight buffer hold every rank's local experts in order).
 *   - Activations travel to the experts and the results travel back and are
 *     merged (same glossary, the MOELayer.forward fact); the all-to-all pair
 *     is called dispatch and combine (DeepEP analysis, "DeepEP introduction").
 *   - Dispatch sends FP8, combine returns BF16 (DeepEP analysis, feature list
 *     and the set-up of both benchmark tables).
 *   - Each token is written straight into its final expert-grouped row on the
 *     receiving rank; static shapes avoid any per-layer host sync (MoonEP
 *     article, section 2, "zero copy" and static layout).  Per-expert padding
 *     to a static shape (search-results page, the dynamic-routing snippet:
 *     drop tokens or zero-pad; MoonEP basic usage, token_padding=128).
 *
 * The R ranks of one EP group are simulated on one GPU as rank-major
 * partitions of one receive buffer: partition r is exactly what GPU r would
 * receive.
 *
 * Conventions for every call:
 *   - All array arguments are DEVICE pointers, row-major and contiguous, owned
 *     by the caller; the library never allocates, frees or keeps them.
 *     Descriptor structs are HOST pointers read during the call only.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     runs asynchronously; no call copies device -> host or synchronises.
 *   - Argument errors are returned synchronously, before anything is
 *     enqueued.  Data errors (an expert id outside [0,E), a capacity
 *     overflow) are found on the device and written to layout->status[0].
 *   - The library holds no global state: calls are reentrant and thread safe.
 *     Calls on one stream run in order; calls on different streams that share
 *     output buffers race.
 *   - Limits: 0 <= S, 1 <= K <= 16, 1 <= E <= 1024, R divides E,
 *     S*K and every row count below 2^31; dispatch: S*ceil(H/512) (bf16) or
 *     S*ceil(H/1024) (FP8) below 2^31; combine: S*ceil(H/512) below 2^31.
 */
#ifndef MOE_EP_H
#define MOE_EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,      /* a required pointer is NULL */
    MOE_ERR_SHAPE = 2,     /* a size or mode is outside the limits above */
    MOE_ERR_ALIGN = 3,     /* a row buffer is not 16-byte aligned */
    MOE_ERR_WORKSPACE = 4, /* workspace missing or smaller than required */
    MOE_ERR_HIP = 5        /* the HIP runtime refused a launch */
} moe_status;

/* How each expert's segment of the receive buffer is sized. */
typedef enum {
    MOE_PAD_NONE = 0,      /* exactly the expert's entries */
    MOE_PAD_MULTIPLE = 1,  /* rounded up to a multiple of pad_rows (0 stays 0) */
    MOE_PAD_CAPACITY = 2   /* exactly pad_rows; entries beyond are not placed */
} moe_pad_mode;

/* Bits of layout->status[0]. */
enum {
    MOE_FLAG_BAD_EXPERT = 1, /* some topk_idx outside [0,E); that entry got pos = -1 */
    MOE_FLAG_CAPACITY = 2    /* some expert had more than pad_rows entries (CAPACITY);
                                the entries past the capacity got pos = -1 */
};

/* Shape of one batch (host struct). */
typedef struct {
    int32_t S;        /* tokens */
    int32_t K;        /* experts per token */
    int32_t E;        /* experts */
    int32_t R;        /* EP ranks; rank r owns experts [r*E/R, (r+1)*E/R) */
    int32_t pad_mode; /* moe_pad_mode */
    int32_t pad_rows; /* multiple or capacity; ignored for MOE_PAD_NONE */
} moe_layout_desc;

/* The layout of one batch: outputs of moe_layout, inputs of dispatch and
 * combine (host struct holding device pointers, all int32). */
typedef struct {
    int32_t *tokens_per_expert; /* [E]   rows placed in each expert's segment */
    int32_t *tokens_per_rank;   /* [R]   rows placed in each rank's partition */
    int32_t *expert_offset;     /* [E+1] first row of each expert's segment; [E] = rows used */
    int32_t *rank_offset;       /* [R+1] first row of each rank's partition */
    int32_t *pos;               /* [S*K] row of entry (t,k) at t*K+k, or -1 */
    int32_t *src;               /* [moe_max_recv_rows] entry t*K+k held by each row, -1 if none */
    int32_t *status;            /* [1]   MOE_FLAG_* of this batch (overwritten) */
} moe_layout_bufs;

/* Rows the receive buffer (and src) must hold for ANY routing of this shape:
 * S*K (NONE), S*K + E*(pad_rows-1) (MULTIPLE), E*pad_rows (CAPACITY).
 * Host only.  Returns -1 if the shape is invalid. */
int64_t moe_max_recv_rows(const moe_layout_desc *desc);

/* Device workspace bytes moe_layout needs for this shape: 0 when
 * S*K <= 32768 (those batches run as one launch with no scratch), else one
 * histogram of E counts per tile.  Host only.  Returns 0 for an invalid shape
 * too; moe_layout then reports MOE_ERR_SHAPE. */
size_t moe_layout_workspace_bytes(const moe_layout_desc *desc);

/* Layout of one batch from its top-k routing.
 *   topk_idx  [S,K] int32 device: expert of entry (t,k).
 *   out       every pointer required; src has moe_max_recv_rows entries.
 *   workspace device scratch of at least moe_layout_workspace_bytes (may be
 *             NULL when that is 0); 16-byte aligned; contents need no init.
 * Inside each expert's segment, rows follow ascending t*K+k (stable); ranks
 * and experts appear in ascending order (rank-major).  Padding rows are not
 * touched in the row buffers; their src is -1. */
moe_status moe_layout(const moe_layout_desc *desc, const int32_t *topk_idx,
                      const moe_layout_bufs *out, void *workspace, size_t workspace_bytes,
                      void *stream);

/* moe_layout without a workspace argument, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same results as moe_layout.  The two-launch form
 * (S*K > 32768) keeps its per-tile histograms in a device array inside the
 * library, 4 MiB per GPU, held from the first call on a GPU until the process
 * ends: MOE_ERR_WORKSPACE when moe_layout_workspace_bytes exceeds 4 MiB (about
 * 4M entries at E = 1024, 16M at E = 256).  Every call on one GPU shares that
 * array, so calls that overlap in time on one GPU (other streams, other host
 * threads) race; calls on one stream are fine.  The array needs no clearing:
 * each call writes every histogram and flag it reads.  The current device must
 * be the stream's device.  No allocation, free or host sync. */
moe_status moe_layout_noalloc(const moe_layout_desc *desc, const int32_t *topk_idx,
                              const moe_layout_bufs *out, void *stream);

/* Dispatch: row pos[t,k] of the receive buffer gets token t's hidden row.
 *   hidden      [S,H] bf16 device, 16-byte aligned, H % 8 == 0.
 *   topk_idx    [S,K] int32; the expert ids already folded into `layout`
 *               (kept for the calling convention; may be NULL).
 *   topk_w      [S,K] fp32 or NULL; with recv_w, recv_w[pos[t,k]] = topk_w[t,k].
 *   fp8 == 0    recv [max_recv,H] bf16 gets the row bit for bit.
 *   fp8 != 0    H % 128 == 0; recv [max_recv,H] E4M3FN bytes and recv_scales
 *               [max_recv,H/128] fp32: per 128-channel block b of token t,
 *               scale = amax/448 (fp32 division, amax = max |x|) and
 *               code = E4M3FN(x/scale) (fp32 division, round to nearest even,
 *               saturating at +-448); an all-zero block has scale 0 and codes 0.
 *   recv_w      [max_recv] fp32 or NULL.
 * Rows that no entry maps to (padding, unused tail) are not written. */
moe_status moe_dispatch(const moe_layout_desc *desc, const moe_layout_bufs *layout,
                        const void *hidden, int32_t H, const int32_t *topk_idx,
                        const float *topk_w, int32_t fp8, void *recv, float *recv_scales,
                        float *recv_w, void *stream);

/* Layout + dispatch in one call: the same results as moe_layout followed by
 * moe_dispatch with these arguments (every output of both).  Batches with
 * S*K <= 4096 and S <= 512 (decode-sized) run as ONE kernel launch in which
 * each workgroup rebuilds the layout counts it needs in LDS; other batches run
 * the two calls' kernels back to back.  Arguments as in moe_layout and moe_dispatch; the
 * workspace rule is moe_layout's.  This is the low-latency variant for
 * inference decoding (DeepEP analysis, feature list: low-latency kernels for
 * decoding). */
moe_status moe_layout_dispatch(const moe_layout_desc *desc, const int32_t *topk_idx,
                               const moe_layout_bufs *out, void *workspace, size_t workspace_bytes,
                               const void *hidden, int32_t H, const float *topk_w, int32_t fp8,
                               void *recv, float *recv_scales, float *recv_w, void *stream);

/* Combine: out[t,c] = bf16_rne( (fma chain over k = 0..K-1 of
 *                                w[t,k] * expert_out[pos[t,k], c], from +0.0)
 *                               + shared_out[t,c] ).
 *   expert_out  [max_recv,H] bf16 device, 16-byte aligned, H % 8 == 0; only rows
 *               some pos[t,k] points to are read.
 *   w           [S,K] fp32 in token order, or NULL for weight 1.
 *   shared_out  [S,H] bf16 or NULL (then nothing is added).
 *   out         [S,H] bf16, 16-byte aligned.
 * Entries with pos = -1 are skipped: their expert_out row is not read. */
moe_status moe_combine(const moe_layout_desc *desc, const moe_layout_bufs *layout,
                       const void *expert_out, int32_t H, const float *w,
                       const void *shared_out, void *out, void *stream);

/* Zero padding (optional, after dispatch): clears every receive row that no
 * entry maps to -- src[r] = -1: padding inside the segments and the unused
 * tail -- so a consumer that runs over whole padded segments reads zeros
 * there (search-results page, the snippet on the limits of dynamic routing:
 * drop tokens or zero-pad).  Dispatch itself never writes those rows.
 *   layout      moe_layout's output for this batch (its src is read).
 *   H, fp8      as given to moe_dispatch.
 *   recv        [max_recv,H] bf16 or E4M3 bytes, 16-byte aligned.
 *   recv_scales [max_recv,H/128] fp32 (required when fp8, ignored otherwise);
 *               scale rows of cleared rows become 0.0f.
 * Rows that hold an entry are not written.  Cost: one write of every padding
 * row (at the decode shape 31,744 rows x 7 KB). */
moe_status moe_zero_padding(const moe_layout_desc *desc, const moe_layout_bufs *layout, int32_t H, int32_t fp8,
                            void *recv, float *recv_scales, void *stream);

/* Balanced layout: every rank receives the same number of rows (N/R, the
 * first N%R ranks one more; N = entries with a valid expert) however skewed
 * the routing, through redundant copies of experts held in per-rank slots --
 * the perfect-balance scheme of the MoonEP article (section 1: a few
 * redundant experts planned online; section 3, Fig. 3: each rank's local
 * experts followed by B prefetch slots).  The planning rule (the pages give
 * none): overloaded ranks in ascending order shed their surplus from their
 * largest experts first (ties: lower id); each piece goes to the lowest rank
 * still below its quota that has a free slot, as much as its room allows;
 * each (expert, destination) piece takes one slot; an expert's first entries
 * (t*K+k order) stay home, later ones fill its replicas in creation order.
 * If slots run out the rest stays home and status bit 4 is set.
 *   desc       pad_mode must be MOE_PAD_NONE; rows used <= S*K (src has S*K).
 *   slots_per_rank  B, 0..64, R*B <= 512.
 *   out        as moe_layout; expert_offset[e] = first row of e's home segment,
 *              expert_offset[E] = rows used; tokens_per_rank = rows per rank.
 *   bal        seg_offset [R*(E/R+B)+1]: first row of each (rank, segment),
 *              segments per rank = its E/R experts then its B slots;
 *              slot_expert [R*B]: expert copied in each slot, -1 if unused
 *              (the weights a rank must hold in that slot).
 *   workspace  at least moe_layout_balanced_workspace_bytes, 256-byte aligned;
 *              that is 0 for S*K <= 32768 (one launch, no scratch), and
 *              workspace may then be NULL.
 * pos/src are ordinary maps, so moe_dispatch and moe_combine take this
 * layout unchanged. */
enum { MOE_FLAG_UNBALANCED = 4 };
typedef struct {
    int32_t *seg_offset;  /* [R*(E/R+B)+1] */
    int32_t *slot_expert; /* [R*B] */
} moe_balance_bufs;
size_t moe_layout_balanced_workspace_bytes(const moe_layout_desc *desc, int32_t slots_per_rank);
moe_status moe_layout_balanced(const moe_layout_desc *desc, int32_t slots_per_rank,
                               const int32_t *topk_idx, const moe_layout_bufs *out,
                               const moe_balance_bufs *bal, void *workspace, size_t workspace_bytes,
                               void *stream);

/* CU budget for overlap: a new stream whose kernels may run only on
 * `num_cus` compute units, num_cus / (number of XCDs) on every XCD (default
 * priority).  Launching layout / dispatch / combine on it leaves
 * the other CUs to concurrent work, the AMD form of DeepEP's control of the
 * number of SMs its kernels occupy (DeepEP analysis, feature list and the
 * "normal kernels" paragraph; MoonEP basic usage, num_sms=32).  Results do not
 * depend on the budget.  Host call: touches the HIP runtime of the current
 * device, allocates the stream; release it with moe_stream_destroy.
 * MOE_ERR_SHAPE if num_cus is outside [1, CU count] or not a multiple of the
 * XCD count (8 on MI355X). */
moe_status moe_stream_create_cu_limited(int32_t num_cus, void **stream_out);

/* The same with the CU set placed: CUs [first_cu, first_cu + num_cus) in the
 * queue-mask numbering (CU i is on XCD i % XCD count), so two streams with
 * disjoint ranges split the chip -- e.g. layout / dispatch / combine on one
 * half and expert compute on the other.  first_cu and num_cus must be
 * multiples of the XCD count, the range within the CU count; else
 * MOE_ERR_SHAPE.  moe_stream_create_cu_limited(n) is the range [0, n). */
moe_status moe_stream_create_cu_range(int32_t first_cu, int32_t num_cus, void **stream_out);
moe_status moe_stream_destroy(void *stream);

/* Static string naming a moe_status value. */
const char *moe_status_str(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_EP_H */
