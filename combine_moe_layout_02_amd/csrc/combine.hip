// Combine kernel: bring each token's K expert-output rows back to token order
// and merge them with the route weights, plus an optional shared-expert output.
//
// Results return from the experts and are merged per token (delect.ru glossary
// "Expert parallelism (EP)", MOELayer.forward fact), in BF16 (DeepEP analysis,
// both benchmark set-ups); DeepSeekMoE adds always-active shared experts next
// to the routed ones (DeepEP analysis, "DeepSeek MoE": 2 shared + 64 routed
// experts in the 16B model).
//
// out[t,c] = bf16_rne( fma-chain over k = 0..K-1 of w[t,k] * y[pos[t,k], c],
//                      starting at +0.0, then + shared[t,c] ).
// One wavefront per 512-channel (1 KiB) chunk of a token row.  A lane owns 8
// channels: it issues all K 16-byte gathers before the first fma (K loads in
// flight), keeps 8 fp32 accumulators, and writes one 16-byte store (with the
// SC1 cache-policy bit; see the end of the kernel).  The K row
// indices and weights are wave-uniform scalars.  Workgroups are numbered
// chunk-fastest, so the waves running at one time cover whole source rows
// rather than one chunk of thousands of rows: on MI355X that DRAM-friendlier
// order measured about 6% faster than a token-fastest order.  The gathers are
// non-temporal loads (ordinary loads measured ~14 % slower in the step).
#include "moe_kernels.h"

namespace moe {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Word 3 of a raw buffer descriptor on gfx950 (32-bit data format, no
// swizzle, no index stride) and the cache-policy operand bit that sets SC1 on
// a buffer store (bit 0 is SC0, bit 1 NT).
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kCachePolicySc1 = 1 << 4;

// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ unsigned int pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    const bf16x2 b = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(unsigned int, b);
}

template <int K>
__global__ __launch_bounds__(kWave) void k_combine(CombineArgs a, int nchunk) {
    const int t = blockIdx.x / nchunk;
    const int nvec = a.H / 8;
    const int v = (blockIdx.x % nchunk) * kWave + threadIdx.x;
    if (v >= nvec) return;
    const u32x4 *__restrict__ y = static_cast<const u32x4 *>(a.y);
    const int32_t *__restrict__ pos = a.pos + static_cast<size_t>(t) * K;

    int p[K];
    u32x4 r[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        p[k] = pos[k];
        // p[k] is the same for the whole wave, so this is a scalar branch; an
        // entry that was not placed reads nothing
        if (p[k] >= 0)
            r[k] = __builtin_nontemporal_load(y + static_cast<size_t>(p[k]) * nvec + v);
        else
            r[k] = u32x4{0u, 0u, 0u, 0u};
    }
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const float wk = a.w != nullptr ? a.w[static_cast<size_t>(t) * K + k] : 1.0f;
        const bool use = p[k] >= 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float c0 = __builtin_fmaf(wk, bf16_lo(r[k][i]), acc[2 * i]);
            const float c1 = __builtin_fmaf(wk, bf16_hi(r[k][i]), acc[2 * i + 1]);
            acc[2 * i] = use ? c0 : acc[2 * i];
            acc[2 * i + 1] = use ? c1 : acc[2 * i + 1];
        }
    }
    if (a.shared != nullptr) {
        const u32x4 sh = __builtin_nontemporal_load(static_cast<const u32x4 *>(a.shared) +
                                                     static_cast<size_t>(t) * nvec + v);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] = acc[2 * i] + bf16_lo(sh[i]);
            acc[2 * i + 1] = acc[2 * i + 1] + bf16_hi(sh[i]);
        }
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    // The output row is stored with the SC1 cache-policy bit (a buffer store
    // through a descriptor based at this token's row): the line goes on past
    // this XCD's L2 instead of staying there dirty among the non-temporal
    // gathers.  In the prefill step on MI355X this took the kernel from
    // ~93 to ~89 us; a plain, non-temporal or SC0 store, or NT together with
    // SC1, measured 92-94 us.
    // The record count and the offset are unsigned 32-bit: 2*H bytes per row
    // is below 2^32 for any int H.
    const unsigned int row_bytes = static_cast<unsigned int>(a.H) * 2u;
    const __amdgpu_buffer_rsrc_t out_row = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<char *>(a.out) + static_cast<size_t>(t) * row_bytes, 0, static_cast<int>(row_bytes),
        kBufferRsrcWord3);
    __builtin_amdgcn_raw_buffer_store_b128(o, out_row, static_cast<int>(static_cast<unsigned int>(v) * 16u), 0,
                                           kCachePolicySc1);
}

}  // namespace

hipError_t launch_combine(const CombineArgs &a, hipStream_t s) {
    const int nvec = a.H / 8;
    const int nchunk = (nvec + kWave - 1) / kWave;
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.S) * nchunk)), block(kWave);
    switch (a.K) {
        case 1: hipLaunchKernelGGL(k_combine<1>, grid, block, 0, s, a, nchunk); break;
        case 2: hipLaunchKernelGGL(k_combine<2>, grid, block, 0, s, a, nchunk); break;
        case 3: hipLaunchKernelGGL(k_combine<3>, grid, block, 0, s, a, nchunk); break;
        case 4: hipLaunchKernelGGL(k_combine<4>, grid, block, 0, s, a, nchunk); break;
        case 5: hipLaunchKernelGGL(k_combine<5>, grid, block, 0, s, a, nchunk); break;
        case 6: hipLaunchKernelGGL(k_combine<6>, grid, block, 0, s, a, nchunk); break;
        case 7: hipLaunchKernelGGL(k_combine<7>, grid, block, 0, s, a, nchunk); break;
        case 8: hipLaunchKernelGGL(k_combine<8>, grid, block, 0, s, a, nchunk); break;
        case 9: hipLaunchKernelGGL(k_combine<9>, grid, block, 0, s, a, nchunk); break;
        case 10: hipLaunchKernelGGL(k_combine<10>, grid, block, 0, s, a, nchunk); break;
        case 11: hipLaunchKernelGGL(k_combine<11>, grid, block, 0, s, a, nchunk); break;
        case 12: hipLaunchKernelGGL(k_combine<12>, grid, block, 0, s, a, nchunk); break;
        case 13: hipLaunchKernelGGL(k_combine<13>, grid, block, 0, s, a, nchunk); break;
        case 14: hipLaunchKernelGGL(k_combine<14>, grid, block, 0, s, a, nchunk); break;
        case 15: hipLaunchKernelGGL(k_combine<15>, grid, block, 0, s, a, nchunk); break;
        case 16: hipLaunchKernelGGL(k_combine<16>, grid, block, 0, s, a, nchunk); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace moe
