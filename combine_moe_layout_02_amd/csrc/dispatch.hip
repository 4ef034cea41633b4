// Dispatch kernels: scatter each token's hidden row into the receive rows its
// K routed entries were given by the layout.
//
// Dispatch carries activations to the experts (delect.ru glossary "Expert
// parallelism (EP)", MOELayer.forward fact), written straight into the final
// expert-grouped row (MoonEP article, section 2, zero copy), in FP8 to halve
// the bytes (DeepEP analysis, feature list: native FP8 dispatch; both
// benchmark set-ups: FP8 dispatch, BF16 combine).
//
// Each token row is read from HBM once and written K times.  A workgroup owns
// one token and a slice of its row; its K row indices are wave-uniform and
// live in scalar registers.  They (and the route weight) are read before the
// first store: a read after the stores would be ordered behind them (the
// compiler cannot rule out that a store changes pos), and the wait for it
// would also wait for every store issued before.  Every lane moves 16 bytes per load/store, so each
// wave touches 1 KiB contiguous per instruction.  Workgroups are single waves
// numbered chunk-fastest, so the waves in flight read whole source rows: with
// 4 KiB rows (H=2048) this measured 1.5x faster on MI355X than a token-fastest
// order, which reads one 1 KiB piece of thousands of rows at once; with 14 KiB
// rows both orders measured the same.  Row loads are ordinary (cached) loads,
// the K row stores are non-temporal (measured fastest for this write-heavy
// scatter).
//
// FP8: a lane holds 16 channels (two 16-byte loads); the 8 lanes of one
// 128-channel block reduce |x| with cross-lane swaps, divide amax by 448
// (correctly rounded fp32 division), divide each value by that scale
// (correctly rounded) and convert with the gfx950 OCP E4M3 instruction
// (round to nearest even).  16 codes make one 16-byte store per row copy.
#include "moe_kernels.h"

namespace moe {
namespace {

// The token's K receive rows (wave-uniform: scalar loads).
template <int K>
__device__ __forceinline__ void load_rows(const int32_t *__restrict__ pos, int (&p)[K]) {
#pragma unroll
    for (int k = 0; k < K; ++k) p[k] = pos[k];
}

// Lane k < K: recv_w of entry k (weight w, row p[k]).
template <int K>
__device__ __forceinline__ void write_recv_w(const DispatchArgs &a, const int (&p)[K], float w) {
    int row = -1;
#pragma unroll
    for (int k = 0; k < K; ++k) row = static_cast<int>(threadIdx.x) == k ? p[k] : row;
    if (row >= 0) a.recv_w[row] = w;
}

template <int K>
__global__ __launch_bounds__(kWave) void k_dispatch_bf16(DispatchArgs a, int nchunk) {
    const int t = blockIdx.x / nchunk, c = blockIdx.x % nchunk;
    const int nvec = a.H / 8;
    const int v = c * kWave + threadIdx.x;
    const u32x4 *__restrict__ hid = static_cast<const u32x4 *>(a.hidden) + static_cast<size_t>(t) * nvec;
    u32x4 *__restrict__ recv = static_cast<u32x4 *>(a.recv);
    const int32_t *__restrict__ pos = a.pos + static_cast<size_t>(t) * K;
    const bool maps = a.recv_w != nullptr && a.topk_w != nullptr && c == 0 && threadIdx.x < K;
    int p[K];
    load_rows<K>(pos, p);
    const float w = maps ? a.topk_w[static_cast<size_t>(t) * K + threadIdx.x] : 0.0f;
    if (v < nvec) {
        u32x4 x = hid[v];
        // the row in registers of its own once it has arrived: the stores
        // below then wait for nothing
        asm volatile("" : "+v"(x));
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (p[k] >= 0) __builtin_nontemporal_store(x, recv + static_cast<size_t>(p[k]) * nvec + v);
    }
    if (maps) write_recv_w<K>(a, p, w);
}

template <int K>
__global__ __launch_bounds__(kWave) void k_dispatch_fp8(DispatchArgs a, int nchunk) {
    const int t = blockIdx.x / nchunk, c = blockIdx.x % nchunk;
    const int n16 = a.H / 16;                       // 16-channel groups per row
    const int g = c * kWave + threadIdx.x;
    const bool active = g < n16;
    const u32x4 *__restrict__ hid = static_cast<const u32x4 *>(a.hidden) + static_cast<size_t>(t) * (a.H / 8);
    const int32_t *__restrict__ pos = a.pos + static_cast<size_t>(t) * K;
    const bool maps = a.recv_w != nullptr && a.topk_w != nullptr && c == 0 && threadIdx.x < K;

    u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    if (active) {
        lo = hid[2 * g];
        hi = hid[2 * g + 1];
    }
    int p[K];
    load_rows<K>(pos, p);
    const float w = maps ? a.topk_w[static_cast<size_t>(t) * K + threadIdx.x] : 0.0f;
    float scale;
    const u32x4 q = quantize16_e4m3(lo, hi, scale);
    const int nsc = a.H / 128;
    u32x4 *__restrict__ recv = static_cast<u32x4 *>(a.recv);
    if (active) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            if (p[k] >= 0) {
                __builtin_nontemporal_store(q, recv + static_cast<size_t>(p[k]) * n16 + g);
                if ((threadIdx.x & 7) == 0) a.recv_scales[static_cast<size_t>(p[k]) * nsc + g / 8] = scale;
            }
        }
    }
    if (maps) write_recv_w<K>(a, p, w);
}

#define MOE_DISPATCH_CASES(KERNEL)                                                           \
    switch (a.K) {                                                                           \
        case 1: hipLaunchKernelGGL(KERNEL<1>, grid, block, 0, s, a, nchunk); break;                  \
        case 2: hipLaunchKernelGGL(KERNEL<2>, grid, block, 0, s, a, nchunk); break;                  \
        case 3: hipLaunchKernelGGL(KERNEL<3>, grid, block, 0, s, a, nchunk); break;                  \
        case 4: hipLaunchKernelGGL(KERNEL<4>, grid, block, 0, s, a, nchunk); break;                  \
        case 5: hipLaunchKernelGGL(KERNEL<5>, grid, block, 0, s, a, nchunk); break;                  \
        case 6: hipLaunchKernelGGL(KERNEL<6>, grid, block, 0, s, a, nchunk); break;                  \
        case 7: hipLaunchKernelGGL(KERNEL<7>, grid, block, 0, s, a, nchunk); break;                  \
        case 8: hipLaunchKernelGGL(KERNEL<8>, grid, block, 0, s, a, nchunk); break;                  \
        case 9: hipLaunchKernelGGL(KERNEL<9>, grid, block, 0, s, a, nchunk); break;                  \
        case 10: hipLaunchKernelGGL(KERNEL<10>, grid, block, 0, s, a, nchunk); break;                \
        case 11: hipLaunchKernelGGL(KERNEL<11>, grid, block, 0, s, a, nchunk); break;                \
        case 12: hipLaunchKernelGGL(KERNEL<12>, grid, block, 0, s, a, nchunk); break;                \
        case 13: hipLaunchKernelGGL(KERNEL<13>, grid, block, 0, s, a, nchunk); break;                \
        case 14: hipLaunchKernelGGL(KERNEL<14>, grid, block, 0, s, a, nchunk); break;                \
        case 15: hipLaunchKernelGGL(KERNEL<15>, grid, block, 0, s, a, nchunk); break;                \
        case 16: hipLaunchKernelGGL(KERNEL<16>, grid, block, 0, s, a, nchunk); break;                \
        default: return hipErrorInvalidValue;                                                \
    }

}  // namespace

hipError_t launch_dispatch_bf16(const DispatchArgs &a, hipStream_t s) {
    const int nchunk = (a.H / 8 + kWave - 1) / kWave;
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.S) * nchunk)), block(kWave);
    MOE_DISPATCH_CASES(k_dispatch_bf16)
    return hipGetLastError();
}

hipError_t launch_dispatch_fp8(const DispatchArgs &a, hipStream_t s) {
    const int nchunk = (a.H / 16 + kWave - 1) / kWave;
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.S) * nchunk)), block(kWave);
    MOE_DISPATCH_CASES(k_dispatch_fp8)
    return hipGetLastError();
}

}  // namespace moe
