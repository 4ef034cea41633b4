// C ABI front end of libmoe_ep.so: argument checks, launch-shape choice, and
// status codes.  Declarations and the meaning of every argument are in
// include/moe_ep.h.  Nothing here allocates, frees or synchronises.
#include <hip/hip_ext.h>
#include <stdint.h>

#include <atomic>
#include <vector>

#include "moe_ep.h"
#include "moe_kernels.h"

namespace moe {
hipError_t launch_zero_padding(const int32_t *src, int rows, int row_bytes, void *recv, float *scales, int nsc,
                               hipStream_t s);  // padding.hip
}

// Scratch of moe_layout_noalloc, for callers that cannot allocate: the
// two-launch layout's per-tile histograms and flags, in a file-scope device
// array.  Each GPU the library runs on holds its own copy until the process
// ends.  Host code never uses the array's name as an address: each device's
// copy is looked up once with hipGetSymbolAddress (scratch_ptr below).
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch` (resolved on the first call on that
// device, with it current), or null with st set.
void *scratch_ptr(moe_status &st) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        st = MOE_ERR_HIP;
        return nullptr;
    }
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            st = MOE_ERR_HIP;
            return nullptr;
        }
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}

bool desc_ok(const moe_layout_desc *d) {
    if (d->S < 0 || d->K < 1 || d->K > moe::kMaxK || d->E < 1 || d->E > moe::kMaxE || d->R < 1 ||
        d->R > d->E || d->E % d->R != 0)
        return false;
    if (d->pad_mode != MOE_PAD_NONE && d->pad_mode != MOE_PAD_MULTIPLE && d->pad_mode != MOE_PAD_CAPACITY)
        return false;
    if (d->pad_mode != MOE_PAD_NONE && d->pad_rows < 1) return false;
    if (static_cast<int64_t>(d->S) * d->K >= (int64_t(1) << 31)) return false;
    return true;
}

int64_t max_rows(const moe_layout_desc *d) {
    const int64_t n = static_cast<int64_t>(d->S) * d->K;
    int64_t rows = n;
    if (d->pad_mode == MOE_PAD_MULTIPLE) rows = n + static_cast<int64_t>(d->E) * (d->pad_rows - 1);
    if (d->pad_mode == MOE_PAD_CAPACITY) rows = static_cast<int64_t>(d->E) * d->pad_rows;
    return rows >= (int64_t(1) << 31) ? -1 : rows;
}

int ceil_log2(int x) {
    int b = 0;
    while ((1 << b) < x) ++b;
    return b;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// moe_layout_dispatch takes its one-launch form up to this many tokens: every
// workgroup of that form (one per token and row slice) recounts all S*K
// entries, so its cost grows with S times S*K.  Measured on MI355X at S*K
// <= 4096: one launch 6.6 / 9.9 us against 7.9 / 12.0 us for layout +
// dispatch at S = 128 / 512; 12.3 against 11.7 at S = 1024 and 36.6 against
// 22.9 at S = 4096 (FP8, H = 7168).
constexpr int kFusedMaxTokens = 512;

}  // namespace

extern "C" {

int64_t moe_max_recv_rows(const moe_layout_desc *desc) {
    if (desc == nullptr || !desc_ok(desc)) return -1;
    return max_rows(desc);
}

size_t moe_layout_workspace_bytes(const moe_layout_desc *desc) {
    if (desc == nullptr || !desc_ok(desc)) return 0;
    return moe::layout_workspace_bytes(static_cast<int64_t>(desc->S) * desc->K, desc->E);
}

}  // extern "C"

namespace {

// Checks shared by moe_layout and moe_layout_dispatch; fills the kernel args.
moe_status prepare_layout(const moe_layout_desc *desc, const int32_t *topk_idx, const moe_layout_bufs *out,
                          void *workspace, size_t workspace_bytes, moe::LayoutArgs &a,
                          bool check_workspace = true) {
    if (desc == nullptr || out == nullptr) return MOE_ERR_NULL;
    if (!desc_ok(desc) || max_rows(desc) < 0) return MOE_ERR_SHAPE;
    const int64_t n = static_cast<int64_t>(desc->S) * desc->K;
    if (out->tokens_per_expert == nullptr || out->tokens_per_rank == nullptr ||
        out->expert_offset == nullptr || out->rank_offset == nullptr || out->status == nullptr)
        return MOE_ERR_NULL;
    if (max_rows(desc) > 0 && out->src == nullptr) return MOE_ERR_NULL;
    if (n > 0 && (topk_idx == nullptr || out->pos == nullptr)) return MOE_ERR_NULL;
    const void *ints[] = {topk_idx, out->tokens_per_expert, out->tokens_per_rank, out->expert_offset,
                          out->rank_offset, out->pos, out->src, out->status};
    for (const void *p : ints)
        if (!aligned(p, 4)) return MOE_ERR_ALIGN;
    const size_t need = moe::layout_workspace_bytes(n, desc->E);
    if (check_workspace && need > 0 && (workspace == nullptr || workspace_bytes < need)) return MOE_ERR_WORKSPACE;
    if (check_workspace && need > 0 && !aligned(workspace, 16)) return MOE_ERR_ALIGN;
    a = moe::LayoutArgs{};
    a.idx = topk_idx;
    a.N = static_cast<int32_t>(n);
    a.E = desc->E;
    a.R = desc->R;
    a.pad_mode = desc->pad_mode;
    a.pad_rows = desc->pad_rows;
    a.nbits = ceil_log2(desc->E);
    a.max_recv = static_cast<int32_t>(max_rows(desc));
    a.tpe = out->tokens_per_expert;
    a.tpr = out->tokens_per_rank;
    a.eoff = out->expert_offset;
    a.roff = out->rank_offset;
    a.pos = out->pos;
    a.src = out->src;
    a.status = out->status;
    a.blk_hist = static_cast<int32_t *>(workspace);
    return MOE_OK;
}

// Checks shared by moe_dispatch and moe_layout_dispatch (pos is checked by the
// caller where it is an input).
moe_status prepare_dispatch(const moe_layout_desc *desc, const void *hidden, int32_t H, const float *topk_w,
                            int32_t fp8, void *recv, float *recv_scales, float *recv_w, moe::DispatchArgs &a) {
    if (!desc_ok(desc) || max_rows(desc) < 0 || H < 8 || H % 8 != 0) return MOE_ERR_SHAPE;
    if (fp8 && H % 128 != 0) return MOE_ERR_SHAPE;
    // one single-wave workgroup per (token, 512- or 1024-channel chunk)
    if (static_cast<int64_t>(desc->S) * ((H / (fp8 ? 16 : 8) + moe::kWave - 1) / moe::kWave) > INT32_MAX)
        return MOE_ERR_SHAPE;
    if (desc->S > 0 && (hidden == nullptr || recv == nullptr)) return MOE_ERR_NULL;
    if (desc->S > 0 && fp8 && recv_scales == nullptr) return MOE_ERR_NULL;
    if (!aligned(hidden, 16) || !aligned(recv, 16) || !aligned(recv_scales, 4) || !aligned(recv_w, 4) ||
        !aligned(topk_w, 4))
        return MOE_ERR_ALIGN;
    a = moe::DispatchArgs{};
    a.hidden = hidden;
    a.S = desc->S;
    a.H = H;
    a.K = desc->K;
    a.topk_w = topk_w;
    a.recv = recv;
    a.recv_scales = recv_scales;
    a.recv_w = recv_w;
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_layout(const moe_layout_desc *desc, const int32_t *topk_idx, const moe_layout_bufs *out,
                      void *workspace, size_t workspace_bytes, void *stream) {
    moe::LayoutArgs a;
    const moe_status st = prepare_layout(desc, topk_idx, out, workspace, workspace_bytes, a);
    if (st != MOE_OK) return st;
    return moe::launch_layout(a, static_cast<hipStream_t>(stream)) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_layout_noalloc(const moe_layout_desc *desc, const int32_t *topk_idx, const moe_layout_bufs *out,
                              void *stream) {
    if (desc == nullptr || out == nullptr) return MOE_ERR_NULL;
    if (!desc_ok(desc) || max_rows(desc) < 0) return MOE_ERR_SHAPE;
    const size_t need = moe::layout_workspace_bytes(static_cast<int64_t>(desc->S) * desc->K, desc->E);
    if (need > kNoAllocScratchBytes) return MOE_ERR_WORKSPACE;
    void *ws = nullptr;
    if (need > 0) {
        moe_status st = MOE_OK;
        ws = scratch_ptr(st);
        if (ws == nullptr) return st;
    }
    moe::LayoutArgs a;
    const moe_status st = prepare_layout(desc, topk_idx, out, ws, need, a);
    if (st != MOE_OK) return st;
    return moe::launch_layout(a, static_cast<hipStream_t>(stream)) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_dispatch(const moe_layout_desc *desc, const moe_layout_bufs *layout, const void *hidden,
                        int32_t H, const int32_t *topk_idx, const float *topk_w, int32_t fp8, void *recv,
                        float *recv_scales, float *recv_w, void *stream) {
    (void)topk_idx;  // already folded into layout->pos
    if (desc == nullptr || layout == nullptr) return MOE_ERR_NULL;
    moe::DispatchArgs a;
    const moe_status st = prepare_dispatch(desc, hidden, H, topk_w, fp8, recv, recv_scales, recv_w, a);
    if (st != MOE_OK) return st;
    if (desc->S == 0) return MOE_OK;
    if (layout->pos == nullptr) return MOE_ERR_NULL;
    if (!aligned(layout->pos, 4)) return MOE_ERR_ALIGN;
    a.pos = layout->pos;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t err = fp8 ? moe::launch_dispatch_fp8(a, s) : moe::launch_dispatch_bf16(a, s);
    return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_layout_dispatch(const moe_layout_desc *desc, const int32_t *topk_idx, const moe_layout_bufs *out,
                               void *workspace, size_t workspace_bytes, const void *hidden, int32_t H,
                               const float *topk_w, int32_t fp8, void *recv, float *recv_scales, float *recv_w,
                               void *stream) {
    moe::LayoutArgs la;
    moe_status st = prepare_layout(desc, topk_idx, out, workspace, workspace_bytes, la);
    if (st != MOE_OK) return st;
    moe::DispatchArgs da;
    st = prepare_dispatch(desc, hidden, H, topk_w, fp8, recv, recv_scales, recv_w, da);
    if (st != MOE_OK) return st;
    da.pos = out->pos;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    if (la.N > 0 && la.N <= moe::kFusedDispatchMaxN && desc->S <= kFusedMaxTokens) {
        err = moe::launch_layout_dispatch_small(la, da, fp8 != 0, s);
    } else {
        err = moe::launch_layout(la, s);
        if (err == hipSuccess && desc->S > 0)
            err = fp8 ? moe::launch_dispatch_fp8(da, s) : moe::launch_dispatch_bf16(da, s);
    }
    return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_combine(const moe_layout_desc *desc, const moe_layout_bufs *layout, const void *expert_out,
                       int32_t H, const float *w, const void *shared_out, void *out, void *stream) {
    if (desc == nullptr || layout == nullptr) return MOE_ERR_NULL;
    if (!desc_ok(desc) || max_rows(desc) < 0 || H < 8 || H % 8 != 0) return MOE_ERR_SHAPE;
    // one workgroup per (token, 512-channel chunk)
    if (static_cast<int64_t>(desc->S) * ((H / 8 + moe::kWave - 1) / moe::kWave) > INT32_MAX) return MOE_ERR_SHAPE;
    if (desc->S == 0) return MOE_OK;
    if (expert_out == nullptr || out == nullptr || layout->pos == nullptr) return MOE_ERR_NULL;
    if (!aligned(expert_out, 16) || !aligned(out, 16) || !aligned(shared_out, 16) || !aligned(w, 4) ||
        !aligned(layout->pos, 4))
        return MOE_ERR_ALIGN;
    moe::CombineArgs a{};
    a.y = expert_out;
    a.S = desc->S;
    a.H = H;
    a.K = desc->K;
    a.pos = layout->pos;
    a.w = w;
    a.shared = shared_out;
    a.out = out;
    return moe::launch_combine(a, static_cast<hipStream_t>(stream)) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

size_t moe_layout_balanced_workspace_bytes(const moe_layout_desc *desc, int32_t slots_per_rank) {
    if (desc == nullptr || !desc_ok(desc) || slots_per_rank < 0) return 0;
    return moe::balance_workspace_bytes(static_cast<int64_t>(desc->S) * desc->K, desc->E, desc->R);
}

moe_status moe_zero_padding(const moe_layout_desc *desc, const moe_layout_bufs *layout, int32_t H, int32_t fp8,
                            void *recv, float *recv_scales, void *stream) {
    if (desc == nullptr || layout == nullptr) return MOE_ERR_NULL;
    if (!desc_ok(desc) || max_rows(desc) < 0 || H < 8 || H % 8 != 0 || (fp8 && H % 128 != 0)) return MOE_ERR_SHAPE;
    const int64_t rows = max_rows(desc);
    if (rows == 0) return MOE_OK;
    if (layout->src == nullptr || recv == nullptr || (fp8 && recv_scales == nullptr)) return MOE_ERR_NULL;
    if (!aligned(layout->src, 4) || !aligned(recv, 16) || !aligned(recv_scales, 4)) return MOE_ERR_ALIGN;
    const int row_bytes = fp8 ? H : 2 * H;
    return moe::launch_zero_padding(layout->src, static_cast<int>(rows), row_bytes, recv,
                                    fp8 ? recv_scales : nullptr, H / 128, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? MOE_OK
               : MOE_ERR_HIP;
}

moe_status moe_layout_balanced(const moe_layout_desc *desc, int32_t slots_per_rank, const int32_t *topk_idx,
                               const moe_layout_bufs *out, const moe_balance_bufs *bal, void *workspace,
                               size_t workspace_bytes, void *stream) {
    if (desc == nullptr || out == nullptr || bal == nullptr) return MOE_ERR_NULL;
    if (!desc_ok(desc) || desc->pad_mode != MOE_PAD_NONE || slots_per_rank < 0 ||
        slots_per_rank > moe::kMaxSlotsPerRank || static_cast<int64_t>(desc->R) * slots_per_rank > moe::kMaxBalanceSlots)
        return MOE_ERR_SHAPE;
    moe::LayoutArgs la;
    // the checks of moe_layout; its own workspace is carved out of ours
    const moe_status st = prepare_layout(desc, topk_idx, out, nullptr, 0, la, false);
    if (st != MOE_OK) return st;
    if (bal->seg_offset == nullptr || (slots_per_rank > 0 && bal->slot_expert == nullptr)) return MOE_ERR_NULL;
    if (!aligned(bal->seg_offset, 4) || !aligned(bal->slot_expert, 4)) return MOE_ERR_ALIGN;
    const size_t need = moe::balance_workspace_bytes(la.N, desc->E, desc->R);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return MOE_ERR_WORKSPACE;
    if (need > 0 && !aligned(workspace, 256)) return MOE_ERR_ALIGN;
    moe::BalanceArgs b{};
    b.idx = topk_idx;
    b.N = la.N;
    b.E = desc->E;
    b.R = desc->R;
    b.B = slots_per_rank;
    b.tpe = out->tokens_per_expert;
    b.tpr = out->tokens_per_rank;
    b.eoff = out->expert_offset;
    b.roff = out->rank_offset;
    b.pos = out->pos;
    b.src = out->src;
    b.status = out->status;
    b.seg_offset = bal->seg_offset;
    b.slot_expert = bal->slot_expert;
    return moe::launch_layout_balanced(la, b, workspace, static_cast<hipStream_t>(stream)) == hipSuccess
               ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_stream_create_cu_range(int32_t first_cu, int32_t num_cus, void **stream_out) {
    if (stream_out == nullptr) return MOE_ERR_NULL;
    int dev = 0, xcc = 1;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_HIP;
    if (hipDeviceGetAttribute(&xcc, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcc < 1) xcc = 1;
    const int total = prop.multiProcessorCount;
    // Bit i of the queue CU mask selects a CU of XCD i % xcc, so a run of bits
    // starting at a multiple of xcc with a length that is a multiple of xcc
    // gives every XCD the same number of CUs; a mask that leaves an XCD
    // without CUs is refused by the runtime.
    if (first_cu < 0 || num_cus < 1 || first_cu % xcc != 0 || num_cus % xcc != 0 || first_cu + num_cus > total)
        return MOE_ERR_SHAPE;
    std::vector<uint32_t> mask((total + 31) / 32, 0u);
    for (int i = first_cu; i < first_cu + num_cus; ++i) mask[i / 32] |= 1u << (i % 32);
    hipStream_t s = nullptr;
    if (hipExtStreamCreateWithCUMask(&s, static_cast<uint32_t>(mask.size()), mask.data()) != hipSuccess) {
        (void)hipGetLastError();
        return MOE_ERR_HIP;
    }
    *stream_out = s;
    return MOE_OK;
}

moe_status moe_stream_create_cu_limited(int32_t num_cus, void **stream_out) {
    return moe_stream_create_cu_range(0, num_cus, stream_out);
}

moe_status moe_stream_destroy(void *stream) {
    if (stream == nullptr) return MOE_ERR_NULL;
    return hipStreamDestroy(static_cast<hipStream_t>(stream)) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

const char *moe_status_str(int32_t status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
        case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: a size or mode is outside the supported limits";
        case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: a buffer is not aligned as required";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
        case MOE_ERR_HIP: return "MOE_ERR_HIP: the HIP runtime refused a launch";
        default: return "unknown moe_status";
    }
}

}  // extern "C"
