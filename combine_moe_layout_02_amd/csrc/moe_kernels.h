// Internal declarations shared by the kernel files and the C-ABI front end.
// Device helpers for wave64 (CDNA4): ballot-based key matching and block scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
constexpr int kLayoutThreads = 1024;              // 16 waves per layout workgroup
constexpr int kLayoutWaves = kLayoutThreads / kWave;
// Layout variant by batch size (entries N = S*K), from measurements on MI355X:
// one workgroup up to 2048 entries; one launch over 1024-entry tiles up to
// 32768; above, two launches over tiles of 1024*J entries, J = 1 up to 65536
// entries, 2 up to 262144, 4 beyond.
constexpr int kSingleMaxN = 2048;
inline int multi_tile_j(int64_t N) { return N <= 65536 ? 1 : (N <= 262144 ? 2 : 4); }
constexpr int kMaxE = 1024;
constexpr int kMaxK = 16;

enum { PAD_NONE = 0, PAD_MULTIPLE = 1, PAD_CAPACITY = 2 };
enum { FLAG_BAD_EXPERT = 1, FLAG_CAPACITY = 2 };

struct LayoutArgs {
    const int32_t *idx;   // [N] expert ids, N = S*K
    int32_t N, E, R, pad_mode, pad_rows, nbits;
    int32_t max_recv;
    int32_t *tpe, *tpr, *eoff, *roff, *pos, *src, *status;
    int32_t *blk_hist;    // [nblk][E] (multi-workgroup path)
    int32_t *blk_flags;   // [nblk]
    int32_t nblk;
};

struct DispatchArgs {
    const void *hidden;   // [S,H] bf16
    int32_t S, H, K;
    const int32_t *pos;   // [S,K]
    const float *topk_w;  // [S,K] or null
    void *recv;           // [max_recv,H] bf16 or e4m3
    float *recv_scales;   // [max_recv,H/128] (fp8)
    float *recv_w;        // [max_recv] or null
};

struct CombineArgs {
    const void *y;        // [max_recv,H] bf16 expert outputs
    int32_t S, H, K;
    const int32_t *pos;   // [S,K]
    const float *w;       // [S,K] or null (weight 1)
    const void *shared;   // [S,H] bf16 or null
    void *out;            // [S,H] bf16
};

// single-launch layout + dispatch for batches of at most this many entries
constexpr int kFusedDispatchMaxN = 4096;
constexpr int kFusedDispatchThreads = 256;

// balanced layout: at most this many redundant-expert slots in total (R*B)
constexpr int kMaxBalanceSlots = 512;
constexpr int kMaxSlotsPerRank = 64;
enum { FLAG_UNBALANCED = 4 };

struct BalanceArgs {
    const int32_t *idx;
    int32_t N, E, R, B;
    const int32_t *pos_std, *tpe_std, *eoff_std, *status_std;  // plain layout (workspace)
    int32_t *tpe, *tpr, *eoff, *roff, *pos, *src, *status;
    int32_t *seg_offset;   // [R*(E/R+B)+1]
    int32_t *slot_expert;  // [R*B]
};

size_t layout_workspace_bytes(int64_t N, int E);
size_t balance_workspace_bytes(int64_t N, int E, int R);
hipError_t launch_layout_balanced(const LayoutArgs &la, BalanceArgs b, void *workspace, hipStream_t stream);
hipError_t launch_layout_dispatch_small(const LayoutArgs &la, const DispatchArgs &da, bool fp8,
                                        hipStream_t stream);
hipError_t launch_layout(const LayoutArgs &a, hipStream_t stream);
hipError_t launch_dispatch_bf16(const DispatchArgs &a, hipStream_t stream);
hipError_t launch_dispatch_fp8(const DispatchArgs &a, hipStream_t stream);
hipError_t launch_combine(const CombineArgs &a, hipStream_t stream);

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte vector

// the two bf16 halves of a 32-bit word, widened exactly to fp32
__device__ __forceinline__ float bf16_lo(unsigned int w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned int w) { return __uint_as_float(w & 0xFFFF0000u); }

// FP8 quantisation of one lane's 16 consecutive bf16 channels (two 16-byte
// vectors), as part of the 8-lane group that holds one 128-channel block:
// amax over the block (cross-lane swaps inside the group), scale = amax / 448
// (correctly rounded fp32 division), code = E4M3(x / scale) (correctly rounded
// division, then v_cvt_pk_fp8_f32: OCP E4M3, round to nearest even).  An
// all-zero block gives scale 0 and codes 0.  Every lane of the wave must call
// it (the swaps are wave-wide); groups are aligned to 8 lanes.
__device__ __forceinline__ u32x4 quantize16_e4m3(u32x4 lo, u32x4 hi, float &scale_out) {
    float f[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_lo(lo[i]);
        f[2 * i + 1] = bf16_hi(lo[i]);
        f[8 + 2 * i] = bf16_lo(hi[i]);
        f[8 + 2 * i + 1] = bf16_hi(hi[i]);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 4, kWave));
    const float scale = amax / 448.0f;
    u32x4 q = {0u, 0u, 0u, 0u};
    if (amax != 0.0f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int w = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * i] / scale, f[4 * i + 1] / scale, 0, false);
            w = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * i + 2] / scale, f[4 * i + 3] / scale, w, true);
            q[i] = static_cast<unsigned int>(w);
        }
    }
    scale_out = scale;
    return q;
}

// Number of set bits of `m` below this lane (v_mbcnt_lo / v_mbcnt_hi).
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

// Mask of the active lanes holding the same key as this lane: one ballot per
// key bit (nbits of them), intersecting "same bit" sets.  Must be called by
// the whole wave in uniform control flow; lanes with active == false take part
// in the ballots but belong to no mask.
__device__ __forceinline__ uint64_t match_key(int key, bool active, int nbits) {
    uint64_t m = __ballot(active);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
    }
    return m;
}

// Inclusive prefix sum of an int pair across the 64 lanes of a wave.
__device__ __forceinline__ int2 wave_inclusive_scan2(int2 v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int ax = __shfl_up(v.x, d, kWave);
        const int ay = __shfl_up(v.y, d, kWave);
        if (lane >= d) { v.x += ax; v.y += ay; }
    }
    return v;
}

// Exclusive prefix sum of an int pair across a workgroup of WAVES waves, in
// thread order.  `s_tmp` holds WAVES entries.  Returns the prefix and the
// workgroup total.  Contains __syncthreads: call from every thread.
template <int WAVES = kLayoutWaves>
__device__ __forceinline__ int2 block_exclusive_scan2(int2 v, int2 *s_tmp, int2 &total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int2 inc = wave_inclusive_scan2(v);
    if (lane == kWave - 1) s_tmp[wave] = inc;
    __syncthreads();
    int2 before = make_int2(0, 0), all = make_int2(0, 0);
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
        const int2 t = s_tmp[w];
        if (w < wave) { before.x += t.x; before.y += t.y; }
        all.x += t.x; all.y += t.y;
    }
    __syncthreads();
    total = all;
    return make_int2(before.x + inc.x - v.x, before.y + inc.y - v.y);
}

}  // namespace moe
