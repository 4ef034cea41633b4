// Single-launch layout + dispatch for small (decode-sized) batches.
//
// DeepEP ships separate low-latency kernels for inference decoding, and keeps
// two static buffers that alternate between calls (DeepEP analysis, feature
// list and "code notes": low-latency kernels, double buffer).  Here a decode
// call's layout and dispatch run in one launch instead of two: the results are
// exactly those of moe_layout followed by moe_dispatch.
//
// Every workgroup owns one token and a slice of its row.  It first issues the
// loads of its row slice (they do not depend on the layout), then rebuilds in
// LDS only what its token needs: per-expert counts of all S*K entries and of
// the entries before its token -- with LDS atomics, since only counts matter
// here -- the padded segment offsets (scan over experts), and from these the
// rows of its K entries: start of the expert's segment + entries of that
// expert before the token + earlier k of the token with the same expert.  This
// is the same stable (t*K+k) order the multi-kernel layout produces.  Then it
// scatters (bf16) or quantises and scatters (FP8) its slice.
//
// Shared outputs are split across workgroups: chunk 0 of each token writes its
// entries' pos, src and recv_w; workgroup 0 writes the per-expert and per-rank
// outputs and the status; every workgroup marks its share of padding rows.
// S*K is at most 4096, so each workgroup reads at most 16 KB of routing.
#include "moe_kernels.h"

namespace moe {
namespace {

constexpr int kT = kFusedDispatchThreads;
constexpr int kTW = kT / kWave;
constexpr int kPerThread = kFusedDispatchMaxN / kT;  // routing entries per thread, at most

struct SmallLayoutLds {
    int cnt[kMaxE];       // entries per expert, all tokens
    int pre[kMaxE];       // entries per expert before this workgroup's token
    int off[kMaxE + 1];   // first row of each padded segment
    int pex[kMaxE + 1];   // placed rows before each expert
    int2 tmp[kTW];
    int flags;
};

// This thread's routing entries (tid, tid + kT, ...), all loads in flight
// at once; entries past N read as 0 and are skipped by small_layout.
__device__ __forceinline__ void load_routing(const LayoutArgs &a, int (&ev)[kPerThread]) {
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
        const int i = threadIdx.x + u * kT;
        ev[u] = i < a.N ? a.idx[i] : 0;
    }
}

// Counts, padded offsets, count-only outputs (workgroup 0) and this
// workgroup's share of padding rows, from load_routing's values.  Returns this
// thread's flags.
__device__ int small_layout(const LayoutArgs &a, int t, int K, const int (&ev)[kPerThread], SmallLayoutLds &L) {
    const int tid = threadIdx.x;
    for (int e = tid; e < a.E; e += kT) {
        L.cnt[e] = 0;
        L.pre[e] = 0;
    }
    __syncthreads();
    int flags = 0;
    const int before = t * K;
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
        const int i = tid + u * kT;
        if (i >= a.N) break;
        const int e = ev[u];
        if (e < 0 || e >= a.E) {
            flags |= FLAG_BAD_EXPERT;
            continue;
        }
        atomicAdd(&L.cnt[e], 1);
        if (i < before) atomicAdd(&L.pre[e], 1);
    }
    __syncthreads();

    // thread tid owns experts [tid*ept, tid*ept + ept)
    const int ept = (a.E + kT - 1) / kT;
    const int e0 = tid * ept;
    int seg_sum = 0, placed_sum = 0;
    for (int j = 0; j < ept && e0 + j < a.E; ++j) {
        const int c = L.cnt[e0 + j];
        int seg = c, placed = c;
        if (a.pad_mode == PAD_MULTIPLE) {
            seg = (c + a.pad_rows - 1) / a.pad_rows * a.pad_rows;
        } else if (a.pad_mode == PAD_CAPACITY) {
            seg = a.pad_rows;
            if (c > a.pad_rows) { placed = a.pad_rows; flags |= FLAG_CAPACITY; }
        }
        seg_sum += seg;
        placed_sum += placed;
    }
    int2 total;
    const int2 ex = block_exclusive_scan2<kTW>(make_int2(seg_sum, placed_sum), L.tmp, total);
    const bool write_outputs = blockIdx.x == 0;
    int so = ex.x, sp = ex.y;
    for (int j = 0; j < ept && e0 + j < a.E; ++j) {
        const int e = e0 + j;
        const int c = L.cnt[e];
        int seg = c, placed = c;
        if (a.pad_mode == PAD_MULTIPLE) {
            seg = (c + a.pad_rows - 1) / a.pad_rows * a.pad_rows;
        } else if (a.pad_mode == PAD_CAPACITY) {
            seg = a.pad_rows;
            placed = c > a.pad_rows ? a.pad_rows : c;
        }
        L.off[e] = so;
        L.pex[e] = sp;
        if (write_outputs) {
            a.tpe[e] = placed;
            a.eoff[e] = so;
        }
        so += seg;
        sp += placed;
    }
    if (tid == 0) {
        L.off[a.E] = total.x;
        L.pex[a.E] = total.y;
        if (write_outputs) a.eoff[a.E] = total.x;
    }
    __syncthreads();
    if (write_outputs) {
        const int epr = a.E / a.R;
        for (int r = tid; r < a.R; r += kT) {
            a.roff[r] = L.off[r * epr];
            a.tpr[r] = L.pex[(r + 1) * epr] - L.pex[r * epr];
        }
        if (tid == 0) a.roff[a.R] = L.off[a.E];
    }
    const int part = blockIdx.x, parts = gridDim.x;
    const int wave = tid / kWave, lane = tid & (kWave - 1);
    for (int e = part + wave * parts; e < a.E; e += kTW * parts) {
        const int beg = L.off[e] + (L.pex[e + 1] - L.pex[e]);
        for (int r = beg + lane; r < L.off[e + 1]; r += kWave) a.src[r] = -1;
    }
    for (int r = L.off[a.E] + part * kT + tid; r < a.max_recv; r += kT * parts) a.src[r] = -1;
    return flags;
}

// Token t's K expert ids (wave-uniform loads, issued at kernel entry).
template <int K>
__device__ __forceinline__ void token_experts(const LayoutArgs &a, int t, int (&e)[K]) {
#pragma unroll
    for (int k = 0; k < K; ++k) e[k] = a.idx[static_cast<size_t>(t) * K + k];
}

// Rows of token t's K entries (-1 if not placed) from its expert ids e.
// Wave-uniform.
template <int K>
__device__ __forceinline__ void token_rows(const LayoutArgs &a, const int (&e)[K], const SmallLayoutLds &L,
                                           int (&p)[K]) {
    // all 2K LDS reads first (an invalid id reads expert 0 and is dropped
    // below), so they are in flight together instead of one after another
    int pre[K], off[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int ek = (e[k] >= 0 && e[k] < a.E) ? e[k] : 0;
        pre[k] = L.pre[ek];
        off[k] = L.off[ek];
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
        int within = pre[k];
#pragma unroll
        for (int j = 0; j < k; ++j) within += (e[j] == e[k]) ? 1 : 0;
        const bool placed = e[k] >= 0 && e[k] < a.E && !(a.pad_mode == PAD_CAPACITY && within >= a.pad_rows);
        p[k] = placed ? off[k] + within : -1;
    }
}

// Route weight of token t's entry threadIdx.x (threads below K of chunk 0,
// when recv_w is wanted), loaded at kernel entry with the other inputs.
template <int K>
__device__ __forceinline__ float token_weight(const DispatchArgs &da, int t, int c) {
    const bool mine = c == 0 && threadIdx.x < K && da.recv_w != nullptr && da.topk_w != nullptr;
    return mine ? da.topk_w[static_cast<size_t>(t) * K + threadIdx.x] : 0.0f;
}

// pos, src and recv_w of token t's entries (chunk 0 only); w = token_weight.
template <int K>
__device__ __forceinline__ void write_token_maps(const LayoutArgs &la, const DispatchArgs &da, int t,
                                                 const int (&p)[K], float w) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
        if (threadIdx.x == k) {
            const int i = t * K + k;
            la.pos[i] = p[k];
            if (p[k] >= 0) {
                la.src[p[k]] = i;
                if (da.recv_w != nullptr && da.topk_w != nullptr) da.recv_w[p[k]] = w;
            }
        }
    }
}

template <int K>
__global__ __launch_bounds__(kT) void k_layout_dispatch_fp8(LayoutArgs la, DispatchArgs da, int nchunk) {
    __shared__ SmallLayoutLds L;
    const int t = blockIdx.x / nchunk, c = blockIdx.x % nchunk;
    const int n16 = da.H / 16;
    const int g = c * kT + threadIdx.x;
    const bool active = g < n16;
    const u32x4 *__restrict__ hid = static_cast<const u32x4 *>(da.hidden) + static_cast<size_t>(t) * (da.H / 8);
    u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    if (active) {
        lo = hid[2 * g];
        hi = hid[2 * g + 1];
    }
    int ev[kPerThread], e[K];
    load_routing(la, ev);
    token_experts<K>(la, t, e);
    const float w = token_weight<K>(da, t, c);
    if (threadIdx.x == 0) L.flags = 0;
    const int flags = small_layout(la, t, K, ev, L);
    int p[K];
    token_rows<K>(la, e, L, p);
    if (c == 0) write_token_maps<K>(la, da, t, p, w);

    float scale;
    const u32x4 q = quantize16_e4m3(lo, hi, scale);
    const int nsc = da.H / 128;
    u32x4 *__restrict__ recv = static_cast<u32x4 *>(da.recv);
    if (active) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            if (p[k] >= 0) {
                __builtin_nontemporal_store(q, recv + static_cast<size_t>(p[k]) * n16 + g);
                if ((threadIdx.x & 7) == 0) da.recv_scales[static_cast<size_t>(p[k]) * nsc + g / 8] = scale;
            }
        }
    }
    if (flags) atomicOr(&L.flags, flags);
    __syncthreads();
    if (blockIdx.x == 0 && threadIdx.x == 0) la.status[0] = L.flags;
}

template <int K>
__global__ __launch_bounds__(kT) void k_layout_dispatch_bf16(LayoutArgs la, DispatchArgs da, int nchunk) {
    __shared__ SmallLayoutLds L;
    const int t = blockIdx.x / nchunk, c = blockIdx.x % nchunk;
    const int nvec = da.H / 8;
    const int v = c * kT + threadIdx.x;
    const bool active = v < nvec;
    const u32x4 *__restrict__ hid = static_cast<const u32x4 *>(da.hidden) + static_cast<size_t>(t) * nvec;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (active) x = hid[v];
    int ev[kPerThread], e[K];
    load_routing(la, ev);
    token_experts<K>(la, t, e);
    const float w = token_weight<K>(da, t, c);
    if (threadIdx.x == 0) L.flags = 0;
    const int flags = small_layout(la, t, K, ev, L);
    int p[K];
    token_rows<K>(la, e, L, p);
    if (c == 0) write_token_maps<K>(la, da, t, p, w);

    u32x4 *__restrict__ recv = static_cast<u32x4 *>(da.recv);
    if (active) {
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (p[k] >= 0) __builtin_nontemporal_store(x, recv + static_cast<size_t>(p[k]) * nvec + v);
    }
    if (flags) atomicOr(&L.flags, flags);
    __syncthreads();
    if (blockIdx.x == 0 && threadIdx.x == 0) la.status[0] = L.flags;
}

#define MOE_FUSED_CASES(KERNEL)                                                              \
    switch (da.K) {                                                                          \
        case 1: hipLaunchKernelGGL(KERNEL<1>, grid, block, 0, s, la, da, nchunk); break;     \
        case 2: hipLaunchKernelGGL(KERNEL<2>, grid, block, 0, s, la, da, nchunk); break;     \
        case 3: hipLaunchKernelGGL(KERNEL<3>, grid, block, 0, s, la, da, nchunk); break;     \
        case 4: hipLaunchKernelGGL(KERNEL<4>, grid, block, 0, s, la, da, nchunk); break;     \
        case 5: hipLaunchKernelGGL(KERNEL<5>, grid, block, 0, s, la, da, nchunk); break;     \
        case 6: hipLaunchKernelGGL(KERNEL<6>, grid, block, 0, s, la, da, nchunk); break;     \
        case 7: hipLaunchKernelGGL(KERNEL<7>, grid, block, 0, s, la, da, nchunk); break;     \
        case 8: hipLaunchKernelGGL(KERNEL<8>, grid, block, 0, s, la, da, nchunk); break;     \
        case 9: hipLaunchKernelGGL(KERNEL<9>, grid, block, 0, s, la, da, nchunk); break;     \
        case 10: hipLaunchKernelGGL(KERNEL<10>, grid, block, 0, s, la, da, nchunk); break;   \
        case 11: hipLaunchKernelGGL(KERNEL<11>, grid, block, 0, s, la, da, nchunk); break;   \
        case 12: hipLaunchKernelGGL(KERNEL<12>, grid, block, 0, s, la, da, nchunk); break;   \
        case 13: hipLaunchKernelGGL(KERNEL<13>, grid, block, 0, s, la, da, nchunk); break;   \
        case 14: hipLaunchKernelGGL(KERNEL<14>, grid, block, 0, s, la, da, nchunk); break;   \
        case 15: hipLaunchKernelGGL(KERNEL<15>, grid, block, 0, s, la, da, nchunk); break;   \
        case 16: hipLaunchKernelGGL(KERNEL<16>, grid, block, 0, s, la, da, nchunk); break;   \
        default: return hipErrorInvalidValue;                                                \
    }

}  // namespace

hipError_t launch_layout_dispatch_small(const LayoutArgs &la, const DispatchArgs &da, bool fp8, hipStream_t s) {
    const int groups = fp8 ? da.H / 16 : da.H / 8;
    const int nchunk = (groups + kT - 1) / kT;
    const dim3 grid(static_cast<unsigned>(da.S) * nchunk), block(kT);
    if (fp8) {
        MOE_FUSED_CASES(k_layout_dispatch_fp8)
    } else {
        MOE_FUSED_CASES(k_layout_dispatch_bf16)
    }
    return hipGetLastError();
}

}  // namespace moe
