// Pattern ceilings: streaming kernels that move the same bytes, in the same
// access patterns, as the dispatch and combine kernels, with no arithmetic.
// They measure what HBM sustains for each pattern on the GPU at hand, so the
// product kernels can be read against the ceiling of their own pattern as
// well as against the 8 TB/s peak.  Measurement infrastructure: nothing on the
// hot path calls them.
//
//   read     contiguous 16-byte loads; a wave reads V KiB, a workgroup W waves
//   write    contiguous 16-byte stores, same shapes, plain / NT / SC1 stores
//   scatter  the dispatch pattern: a single-wave workgroup reads 1 or 2 KiB of
//            one source row (bf16 or FP8 dispatch) and stores 1 KiB to each of
//            the token's K receive rows (non-temporal), plus one fp32 scale
//            per 128 bytes when scales are given (FP8 dispatch)
//   gather   the combine pattern: a single-wave workgroup gathers V KiB from
//            each of the token's K rows (non-temporal loads) and stores V KiB
//            of the output row (plain / NT / SC1 store)
// Workgroups are numbered chunk-fastest, as in the product kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_ceilings.h"

namespace {

constexpr int kWave = 64;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// buffer descriptor word 3 on gfx950 (32-bit format, no swizzle, no stride)
// and the cache-policy operand bit that sets SC1 on a buffer store
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kCachePolicySc1 = 1 << 4;

enum { LOAD_PLAIN = 0, LOAD_NT = 1 };
enum { STORE_PLAIN = 0, STORE_NT = 1, STORE_SC1 = 2 };

template <int KIND>
__device__ __forceinline__ u32x4 load16(const u32x4 *p) {
    if constexpr (KIND == LOAD_NT) return __builtin_nontemporal_load(p);
    else return *p;
}

// store of vector `i` (16 bytes) of a region that starts at `base`
template <int KIND>
__device__ __forceinline__ void store16(u32x4 x, u32x4 *base, unsigned int i, unsigned int region_bytes) {
    if constexpr (KIND == STORE_NT) {
        __builtin_nontemporal_store(x, base + i);
    } else if constexpr (KIND == STORE_SC1) {
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(region_bytes), kBufferRsrcWord3);
        __builtin_amdgcn_raw_buffer_store_b128(x, r, static_cast<int>(i * 16u), 0, kCachePolicySc1);
    } else {
        base[i] = x;
    }
}

// Keeps the loaded values live without storing them: the sink is written
// only if the XOR of everything read equals a value the caller chose (the
// data is never made to match it).
__device__ __forceinline__ void sink_if(u32x4 x, u32x4 *sink, unsigned int magic) {
    if (x[0] == magic && x[1] == magic && x[2] == magic && x[3] == magic) *sink = x;
}

template <int V, int KIND>
__global__ void k_read(const u32x4 *__restrict__ src, u32x4 *sink, unsigned int magic) {
    const int W = blockDim.x / kWave;
    const int64_t wave = static_cast<int64_t>(blockIdx.x) * W + threadIdx.x / kWave;
    const u32x4 *p = src + wave * (V * kWave) + (threadIdx.x % kWave);
    u32x4 r[V];
#pragma unroll
    for (int i = 0; i < V; ++i) r[i] = load16<KIND>(p + i * kWave);
    u32x4 x = r[0];
#pragma unroll
    for (int i = 1; i < V; ++i) x ^= r[i];
    sink_if(x, sink, magic);
}

template <int V, int KIND>
__global__ void k_write(u32x4 *__restrict__ dst, unsigned int magic) {
    const int W = blockDim.x / kWave;
    const int64_t wave = static_cast<int64_t>(blockIdx.x) * W + threadIdx.x / kWave;
    u32x4 *base = dst + wave * (V * kWave);
    const u32x4 x = {static_cast<unsigned int>(wave), threadIdx.x, magic, 0u};
#pragma unroll
    for (int i = 0; i < V; ++i) store16<KIND>(x, base, i * kWave + threadIdx.x % kWave, V * kWave * 16u);
}

// IN = 1: a bf16 row chunk goes out as it came in; IN = 2: two input vectors
// make one output vector (the FP8 dispatch's 2:1 byte ratio).
// A workgroup of W waves covers W consecutive 1 KiB chunks of one token's
// output rows (W = 1: the product dispatch kernels' shape).
template <int K, int IN>
__global__ __launch_bounds__(256) void k_scatter(const u32x4 *__restrict__ src, int out_nvec,
                                                 const int32_t *__restrict__ rows, u32x4 *__restrict__ dst,
                                                 float *__restrict__ scales, int nchunk) {
    const int W = blockDim.x / kWave;
    const int groups_per_token = nchunk / W;
    const int t = blockIdx.x / groups_per_token;
    const int c = (blockIdx.x % groups_per_token) * W + static_cast<int>(threadIdx.x / kWave);
    const int v = c * kWave + static_cast<int>(threadIdx.x % kWave);
    const int32_t *pr = rows + static_cast<size_t>(t) * K;
    int p[K];
#pragma unroll
    for (int k = 0; k < K; ++k) p[k] = pr[k];
    const u32x4 *s = src + static_cast<size_t>(t) * out_nvec * IN + static_cast<size_t>(v) * IN;
    u32x4 x = s[0];
    if constexpr (IN == 2) x ^= s[1];
    asm volatile("" : "+v"(x));
#pragma unroll
    for (int k = 0; k < K; ++k) {
        if (p[k] >= 0) {
            __builtin_nontemporal_store(x, dst + static_cast<size_t>(p[k]) * out_nvec + v);
            if (scales != nullptr && (v & 7) == 0)
                scales[static_cast<size_t>(p[k]) * (out_nvec / 8) + v / 8] = __uint_as_float(x[0] & 0x3F7FFFFFu);
        }
    }
}

// The dispatch bytes in row order through LDS: one workgroup of K waves per
// token; the waves load the token row into LDS together (each wave 1/K of
// it), then wave k stores the whole output row, contiguously, to row
// rows[t*K+k] (NT stores; with `scales`, one lane in 8 stores a 4-byte value
// per 128 output bytes).  IN = 2: two input vectors make one output vector.
template <int K, int IN>
__global__ __launch_bounds__(512) void k_scatter_rows(const u32x4 *__restrict__ src, int out_nvec,
                                                      const int32_t *__restrict__ rows, u32x4 *__restrict__ dst,
                                                      float *__restrict__ scales) {
    extern __shared__ u32x4 s_row[];   // [out_nvec] output vectors of the token
    const int t = blockIdx.x;
    const int w = static_cast<int>(threadIdx.x / kWave), lane = static_cast<int>(threadIdx.x % kWave);
    const u32x4 *s = src + static_cast<size_t>(t) * out_nvec * IN;
    for (int j = static_cast<int>(threadIdx.x); j < out_nvec; j += K * kWave) {
        u32x4 x = s[static_cast<size_t>(j) * IN];
        if constexpr (IN == 2) x ^= s[static_cast<size_t>(j) * IN + 1];
        s_row[j] = x;
    }
    __syncthreads();
    const int p = rows[static_cast<size_t>(t) * K + w];
    if (p < 0) return;
    u32x4 *drow = dst + static_cast<size_t>(p) * out_nvec;
    for (int j = lane; j < out_nvec; j += kWave) {
        const u32x4 x = s_row[j];
        __builtin_nontemporal_store(x, drow + j);
        if (scales != nullptr && (j & 7) == 0)
            scales[static_cast<size_t>(p) * (out_nvec / 8) + j / 8] = __uint_as_float(x[0] & 0x3F7FFFFFu);
    }
}

template <int K, int V, int KIND>
__global__ __launch_bounds__(kWave) void k_gather(const u32x4 *__restrict__ y, int nvec,
                                                  const int32_t *__restrict__ rows, u32x4 *__restrict__ out,
                                                  int nchunk) {
    const int t = blockIdx.x / nchunk, c = blockIdx.x % nchunk;
    const int v = c * kWave * V + threadIdx.x;
    const int32_t *pr = rows + static_cast<size_t>(t) * K;
    u32x4 r[K][V];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int p = pr[k];
#pragma unroll
        for (int i = 0; i < V; ++i)
            r[k][i] = p >= 0 ? __builtin_nontemporal_load(y + static_cast<size_t>(p) * nvec + v + i * kWave)
                             : u32x4{0u, 0u, 0u, 0u};
    }
    u32x4 *orow = out + static_cast<size_t>(t) * nvec;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        u32x4 x = r[0][i];
#pragma unroll
        for (int k = 1; k < K; ++k) x ^= r[k][i];
        store16<KIND>(x, orow, static_cast<unsigned int>(v + i * kWave), static_cast<unsigned int>(nvec) * 16u);
    }
}

// The gather pattern with the gathers' cache-policy operand given (buffer
// loads through a descriptor per row: bit 0 SC0, bit 1 NT, bit 4 SC1) and an
// SC1 output store; one single-wave workgroup per (token, 1 KiB chunk).
template <int K, int POL>
__global__ __launch_bounds__(kWave) void k_gather_policy(const u32x4 *__restrict__ y, int nvec,
                                                         const int32_t *__restrict__ rows, u32x4 *__restrict__ out,
                                                         int nchunk) {
    const int t = blockIdx.x / nchunk, c = blockIdx.x % nchunk;
    const int32_t *pr = rows + static_cast<size_t>(t) * K;
    int p[K];
#pragma unroll
    for (int k = 0; k < K; ++k) p[k] = pr[k];
    u32x4 r[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const u32x4 *chunk = y + static_cast<size_t>(p[k] >= 0 ? p[k] : 0) * nvec + c * kWave;
        const __amdgpu_buffer_rsrc_t d = __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4 *>(chunk), 0,
                                                                          p[k] >= 0 ? kWave * 16 : 0, kBufferRsrcWord3);
        r[k] = __builtin_amdgcn_raw_buffer_load_b128(d, threadIdx.x * 16, 0, POL);
    }
    u32x4 x = r[0];
#pragma unroll
    for (int k = 1; k < K; ++k) x ^= r[k];
    store16<STORE_SC1>(x, out + static_cast<size_t>(t) * nvec, static_cast<unsigned int>(c * kWave + threadIdx.x),
                       static_cast<unsigned int>(nvec) * 16u);
}

// The gather pattern in persistent form: every wave walks (token, 1 KiB
// chunk) units u = w, w + nwaves, ... (chunk-fastest, as above) and keeps the
// next unit's K row loads in flight while it combines and stores the current
// one.  A unit is tracked as (t, c) and advanced by whole strides, so no
// division runs in the loop; both stay wave-uniform (scalar registers).
struct Unit {
    int t, c;
};

__device__ __forceinline__ Unit unit_next(Unit x, int dt, int dc, int nchunk) {
    x.c += dc;
    x.t += dt;
    if (x.c >= nchunk) {
        x.c -= nchunk;
        x.t += 1;
    }
    return x;
}

template <int K>
__device__ __forceinline__ void unit_rows(const int32_t *__restrict__ rows, Unit x, int (&p)[K]) {
    const int32_t *pr = rows + static_cast<size_t>(x.t) * K;
#pragma unroll
    for (int k = 0; k < K; ++k) p[k] = pr[k];
}

// Gathers of one unit through buffer loads: each row chunk gets a descriptor
// built in scalar registers (base at the chunk, 1 KiB long), and the lane's
// byte offset is the only vector operand, so the loads need no per-load
// vector address arithmetic.  An entry with no row gets a zero-length
// descriptor: its load returns zeros without touching memory.
constexpr int kCachePolicyNt = 1 << 1;

template <int K>
__device__ __forceinline__ void unit_gather(const u32x4 *__restrict__ y, int nvec, Unit x, const int (&p)[K],
                                            u32x4 (&r)[K]) {
    const int lane_off = static_cast<int>(threadIdx.x % kWave) * 16;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const u32x4 *chunk = y + static_cast<size_t>(p[k] >= 0 ? p[k] : 0) * nvec + x.c * kWave;
        const __amdgpu_buffer_rsrc_t d =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4 *>(chunk), 0, p[k] >= 0 ? kWave * 16 : 0, kBufferRsrcWord3);
        r[k] = __builtin_amdgcn_raw_buffer_load_b128(d, lane_off, 0, kCachePolicyNt);
    }
}

// Combines the K rows of one unit and stores the chunk.
template <int K, int KIND>
__device__ __forceinline__ void unit_store(const u32x4 (&r)[K], u32x4 *__restrict__ out, int nvec, Unit x) {
    u32x4 acc = r[0];
#pragma unroll
    for (int k = 1; k < K; ++k) acc ^= r[k];
    const int v = x.c * kWave + static_cast<int>(threadIdx.x % kWave);
    store16<KIND>(acc, out + static_cast<size_t>(x.t) * nvec, static_cast<unsigned int>(v),
                  static_cast<unsigned int>(nvec) * 16u);
}

template <int K, int KIND>
__global__ __launch_bounds__(256) void k_gather_persistent(const u32x4 *__restrict__ y, int nvec,
                                                           const int32_t *__restrict__ rows,
                                                           u32x4 *__restrict__ out, int nchunk, int S) {
    const int wpg = blockDim.x / kWave;
    const int nwaves = gridDim.x * wpg;
    const int w = blockIdx.x * wpg + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (w >= S * nchunk) return;
    const int dt = nwaves / nchunk, dc = nwaves % nchunk;
    // Two register sets take turns: while one unit's gathers are combined and
    // stored, the next unit's are in flight in the other set.  Past the last
    // unit the prefetches repeat the current one, so no load sits behind a
    // branch and the waits cover only the unit being combined.
    Unit cur = {w / nchunk, w % nchunk};
    int pa[K], pb[K];
    u32x4 ra[K], rb[K];
    unit_rows<K>(rows, cur, pa);
    unit_gather<K>(y, nvec, cur, pa, ra);
    Unit nxt = unit_next(cur, dt, dc, nchunk);
    unit_rows<K>(rows, nxt.t < S ? nxt : cur, pb);
    while (true) {
        nxt = unit_next(cur, dt, dc, nchunk);
        Unit nn = unit_next(nxt, dt, dc, nchunk);
        unit_gather<K>(y, nvec, nxt.t < S ? nxt : cur, pb, rb);
        unit_rows<K>(rows, nn.t < S ? nn : cur, pa);
        __builtin_amdgcn_sched_barrier(0);   // the next unit's loads go out before this unit is combined
        unit_store<K, KIND>(ra, out, nvec, cur);
        if (nxt.t >= S) break;
        cur = nxt;
        nxt = nn;
        nn = unit_next(nxt, dt, dc, nchunk);
        unit_gather<K>(y, nvec, nxt.t < S ? nxt : cur, pa, ra);
        unit_rows<K>(rows, nn.t < S ? nn : cur, pb);
        __builtin_amdgcn_sched_barrier(0);
        unit_store<K, KIND>(rb, out, nvec, cur);
        if (nxt.t >= S) break;
        cur = nxt;
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t launched() { return hipGetLastError() == hipSuccess ? MOE_CEIL_OK : MOE_CEIL_ERR_HIP; }

}  // namespace

#define CEIL_V_CASES(KERNEL, KIND, ...)                                                        \
    switch (vec_per_lane) {                                                                    \
        case 1: hipLaunchKernelGGL((KERNEL<1, KIND>), grid, block, 0, s, __VA_ARGS__); break;  \
        case 2: hipLaunchKernelGGL((KERNEL<2, KIND>), grid, block, 0, s, __VA_ARGS__); break;  \
        case 4: hipLaunchKernelGGL((KERNEL<4, KIND>), grid, block, 0, s, __VA_ARGS__); break;  \
        case 8: hipLaunchKernelGGL((KERNEL<8, KIND>), grid, block, 0, s, __VA_ARGS__); break;  \
        case 16: hipLaunchKernelGGL((KERNEL<16, KIND>), grid, block, 0, s, __VA_ARGS__); break; \
        default: return MOE_CEIL_ERR_ARG;                                                      \
    }

static bool shape_ok(int64_t bytes, int32_t vec_per_lane, int32_t waves_per_group) {
    if (bytes <= 0 || waves_per_group < 1 || waves_per_group > 16) return false;
    if (vec_per_lane != 1 && vec_per_lane != 2 && vec_per_lane != 4 && vec_per_lane != 8 && vec_per_lane != 16)
        return false;
    const int64_t per_group = 16LL * kWave * vec_per_lane * waves_per_group;
    return bytes % per_group == 0 && bytes / per_group <= 0x7FFFFFFFLL;
}

extern "C" int32_t moe_ceiling_read(const void *src, int64_t bytes, int32_t vec_per_lane, int32_t waves_per_group,
                                    int32_t load_kind, void *sink, void *stream) {
    if (src == nullptr || sink == nullptr || !aligned16(src) || !aligned16(sink)) return MOE_CEIL_ERR_ARG;
    if (!shape_ok(bytes, vec_per_lane, waves_per_group) || (load_kind != LOAD_PLAIN && load_kind != LOAD_NT))
        return MOE_CEIL_ERR_ARG;
    const dim3 grid(static_cast<unsigned>(bytes / (16LL * kWave * vec_per_lane * waves_per_group)));
    const dim3 block(kWave * waves_per_group);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4 *in = static_cast<const u32x4 *>(src);
    u32x4 *out = static_cast<u32x4 *>(sink);
    const unsigned int magic = 0x5EEDF00Du;
    if (load_kind == LOAD_NT) {
        CEIL_V_CASES(k_read, LOAD_NT, in, out, magic)
    } else {
        CEIL_V_CASES(k_read, LOAD_PLAIN, in, out, magic)
    }
    return launched();
}

extern "C" int32_t moe_ceiling_write(void *dst, int64_t bytes, int32_t vec_per_lane, int32_t waves_per_group,
                                     int32_t store_kind, void *stream) {
    if (dst == nullptr || !aligned16(dst) || !shape_ok(bytes, vec_per_lane, waves_per_group)) return MOE_CEIL_ERR_ARG;
    const dim3 grid(static_cast<unsigned>(bytes / (16LL * kWave * vec_per_lane * waves_per_group)));
    const dim3 block(kWave * waves_per_group);
    hipStream_t s = static_cast<hipStream_t>(stream);
    u32x4 *out = static_cast<u32x4 *>(dst);
    const unsigned int magic = 0x5EEDF00Du;
    switch (store_kind) {
        case STORE_PLAIN: CEIL_V_CASES(k_write, STORE_PLAIN, out, magic) break;
        case STORE_NT: CEIL_V_CASES(k_write, STORE_NT, out, magic) break;
        case STORE_SC1: CEIL_V_CASES(k_write, STORE_SC1, out, magic) break;
        default: return MOE_CEIL_ERR_ARG;
    }
    return launched();
}

#define CEIL_K_CASES(KERNEL, TAIL, ...)                                                            \
    switch (K) {                                                                                   \
        case 1: hipLaunchKernelGGL((KERNEL<1, TAIL>), grid, block, 0, s, __VA_ARGS__); break;     \
        case 2: hipLaunchKernelGGL((KERNEL<2, TAIL>), grid, block, 0, s, __VA_ARGS__); break;     \
        case 4: hipLaunchKernelGGL((KERNEL<4, TAIL>), grid, block, 0, s, __VA_ARGS__); break;     \
        case 6: hipLaunchKernelGGL((KERNEL<6, TAIL>), grid, block, 0, s, __VA_ARGS__); break;     \
        case 8: hipLaunchKernelGGL((KERNEL<8, TAIL>), grid, block, 0, s, __VA_ARGS__); break;     \
        default: return MOE_CEIL_ERR_ARG;                                                          \
    }

extern "C" int32_t moe_ceiling_scatter(const void *src, int32_t S, int32_t in_row_bytes, int32_t K,
                                       const int32_t *rows, void *dst, int32_t out_row_bytes, float *scales,
                                       int32_t waves_per_group, void *stream) {
    if (src == nullptr || rows == nullptr || dst == nullptr || !aligned16(src) || !aligned16(dst)) return MOE_CEIL_ERR_ARG;
    if (S < 1 || out_row_bytes < 1024 || out_row_bytes % 1024) return MOE_CEIL_ERR_ARG;
    if (in_row_bytes != out_row_bytes && in_row_bytes != 2 * out_row_bytes) return MOE_CEIL_ERR_ARG;
    const int out_nvec = out_row_bytes / 16, nchunk = out_nvec / kWave;
    if (waves_per_group < 1 || waves_per_group > 4 || nchunk % waves_per_group) return MOE_CEIL_ERR_ARG;
    if (static_cast<int64_t>(S) * nchunk > 0x7FFFFFFFLL) return MOE_CEIL_ERR_ARG;
    const dim3 grid(static_cast<unsigned>(S * (nchunk / waves_per_group))), block(kWave * waves_per_group);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4 *in = static_cast<const u32x4 *>(src);
    u32x4 *out = static_cast<u32x4 *>(dst);
    if (in_row_bytes == out_row_bytes) {
        CEIL_K_CASES(k_scatter, 1, in, out_nvec, rows, out, scales, nchunk)
    } else {
        CEIL_K_CASES(k_scatter, 2, in, out_nvec, rows, out, scales, nchunk)
    }
    return launched();
}

#define CEIL_GATHER_K(V, KIND)                                                                        \
    switch (K) {                                                                                     \
        case 1: hipLaunchKernelGGL((k_gather<1, V, KIND>), grid, block, 0, s, in, nvec, rows, o, nchunk); break; \
        case 2: hipLaunchKernelGGL((k_gather<2, V, KIND>), grid, block, 0, s, in, nvec, rows, o, nchunk); break; \
        case 4: hipLaunchKernelGGL((k_gather<4, V, KIND>), grid, block, 0, s, in, nvec, rows, o, nchunk); break; \
        case 6: hipLaunchKernelGGL((k_gather<6, V, KIND>), grid, block, 0, s, in, nvec, rows, o, nchunk); break; \
        case 8: hipLaunchKernelGGL((k_gather<8, V, KIND>), grid, block, 0, s, in, nvec, rows, o, nchunk); break; \
        default: return MOE_CEIL_ERR_ARG;                                                            \
    }

#define CEIL_GATHER_KIND(V)                                            \
    switch (store_kind) {                                              \
        case STORE_PLAIN: CEIL_GATHER_K(V, STORE_PLAIN) break;         \
        case STORE_NT: CEIL_GATHER_K(V, STORE_NT) break;               \
        case STORE_SC1: CEIL_GATHER_K(V, STORE_SC1) break;             \
        default: return MOE_CEIL_ERR_ARG;                              \
    }

extern "C" int32_t moe_ceiling_gather(const void *y, int32_t S, int32_t row_bytes, int32_t K, const int32_t *rows,
                                      int32_t vec_per_lane, int32_t store_kind, void *out, void *stream) {
    if (y == nullptr || rows == nullptr || out == nullptr || !aligned16(y) || !aligned16(out)) return MOE_CEIL_ERR_ARG;
    if (S < 1 || row_bytes < 1024 || (vec_per_lane != 1 && vec_per_lane != 2)) return MOE_CEIL_ERR_ARG;
    if (row_bytes % (1024 * vec_per_lane)) return MOE_CEIL_ERR_ARG;
    const int nvec = row_bytes / 16, nchunk = nvec / (kWave * vec_per_lane);
    if (static_cast<int64_t>(S) * nchunk > 0x7FFFFFFFLL) return MOE_CEIL_ERR_ARG;
    const dim3 grid(static_cast<unsigned>(S * nchunk)), block(kWave);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4 *in = static_cast<const u32x4 *>(y);
    u32x4 *o = static_cast<u32x4 *>(out);
    if (vec_per_lane == 1) {
        CEIL_GATHER_KIND(1)
    } else {
        CEIL_GATHER_KIND(2)
    }
    return launched();
}

extern "C" int32_t moe_ceiling_gather_persistent(const void *y, int32_t S, int32_t row_bytes, int32_t K,
                                                 const int32_t *rows, int32_t groups, int32_t waves_per_group,
                                                 int32_t store_kind, void *out, void *stream) {
    if (y == nullptr || rows == nullptr || out == nullptr || !aligned16(y) || !aligned16(out)) return MOE_CEIL_ERR_ARG;
    if (S < 1 || row_bytes < 1024 || row_bytes % 1024 || groups < 1 || waves_per_group < 1 || waves_per_group > 4)
        return MOE_CEIL_ERR_ARG;
    const int nvec = row_bytes / 16, nchunk = nvec / kWave;
    if (static_cast<int64_t>(S) * nchunk > 0x7FFFFFFFLL) return MOE_CEIL_ERR_ARG;
    const dim3 grid(static_cast<unsigned>(groups)), block(kWave * waves_per_group);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4 *in = static_cast<const u32x4 *>(y);
    u32x4 *o = static_cast<u32x4 *>(out);
#define CEIL_GP(KK, KIND) hipLaunchKernelGGL((k_gather_persistent<KK, KIND>), grid, block, 0, s, in, nvec, rows, o, nchunk, S)
    if (K == 8 && store_kind == STORE_SC1) CEIL_GP(8, STORE_SC1);
    else if (K == 8 && store_kind == STORE_NT) CEIL_GP(8, STORE_NT);
    else if (K == 8 && store_kind == STORE_PLAIN) CEIL_GP(8, STORE_PLAIN);
    else if (K == 6 && store_kind == STORE_SC1) CEIL_GP(6, STORE_SC1);
    else return MOE_CEIL_ERR_ARG;
#undef CEIL_GP
    return launched();
}

extern "C" int32_t moe_ceiling_scatter_rows(const void *src, int32_t S, int32_t in_row_bytes, int32_t K,
                                            const int32_t *rows, void *dst, int32_t out_row_bytes, float *scales,
                                            void *stream) {
    if (src == nullptr || rows == nullptr || dst == nullptr || !aligned16(src) || !aligned16(dst)) return MOE_CEIL_ERR_ARG;
    if (S < 1 || out_row_bytes < 1024 || out_row_bytes % 1024 || out_row_bytes > 64 * 1024) return MOE_CEIL_ERR_ARG;
    if (in_row_bytes != out_row_bytes && in_row_bytes != 2 * out_row_bytes) return MOE_CEIL_ERR_ARG;
    const int out_nvec = out_row_bytes / 16;
    const dim3 grid(static_cast<unsigned>(S));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4 *in = static_cast<const u32x4 *>(src);
    u32x4 *out = static_cast<u32x4 *>(dst);
    const size_t lds = static_cast<size_t>(out_row_bytes);
#define CEIL_SR(KK)                                                                                                \
    {                                                                                                              \
        const dim3 block(kWave * KK);                                                                              \
        if (in_row_bytes == out_row_bytes)                                                                         \
            hipLaunchKernelGGL((k_scatter_rows<KK, 1>), grid, block, lds, s, in, out_nvec, rows, out, scales);    \
        else                                                                                                       \
            hipLaunchKernelGGL((k_scatter_rows<KK, 2>), grid, block, lds, s, in, out_nvec, rows, out, scales);    \
    }
    switch (K) {
        case 6: CEIL_SR(6) break;
        case 8: CEIL_SR(8) break;
        default: return MOE_CEIL_ERR_ARG;
    }
#undef CEIL_SR
    return launched();
}

extern "C" int32_t moe_ceiling_gather_policy(const void *y, int32_t S, int32_t row_bytes, int32_t K, const int32_t *rows,
                                             int32_t load_policy, void *out, void *stream) {
    if (y == nullptr || rows == nullptr || out == nullptr || !aligned16(y) || !aligned16(out)) return MOE_CEIL_ERR_ARG;
    if (S < 1 || row_bytes < 1024 || row_bytes % 1024 || K != 8) return MOE_CEIL_ERR_ARG;
    if (load_policy != 0 && load_policy != 2 && load_policy != 3 && load_policy != 18 && load_policy != 19)
        return MOE_CEIL_ERR_ARG;
    const int nvec = row_bytes / 16, nchunk = nvec / kWave;
    if (static_cast<int64_t>(S) * nchunk > 0x7FFFFFFFLL) return MOE_CEIL_ERR_ARG;
    const dim3 grid(static_cast<unsigned>(S * nchunk));
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const u32x4 *yv = static_cast<const u32x4 *>(y);
    u32x4 *ov = static_cast<u32x4 *>(out);
    switch (load_policy) {
        case 0: hipLaunchKernelGGL((k_gather_policy<8, 0>), grid, dim3(kWave), 0, st, yv, nvec, rows, ov, nchunk); break;
        case 2: hipLaunchKernelGGL((k_gather_policy<8, 2>), grid, dim3(kWave), 0, st, yv, nvec, rows, ov, nchunk); break;
        case 3: hipLaunchKernelGGL((k_gather_policy<8, 3>), grid, dim3(kWave), 0, st, yv, nvec, rows, ov, nchunk); break;
        case 18: hipLaunchKernelGGL((k_gather_policy<8, 18>), grid, dim3(kWave), 0, st, yv, nvec, rows, ov, nchunk); break;
        default: hipLaunchKernelGGL((k_gather_policy<8, 19>), grid, dim3(kWave), 0, st, yv, nvec, rows, ov, nchunk); break;
    }
    return launched();
}
