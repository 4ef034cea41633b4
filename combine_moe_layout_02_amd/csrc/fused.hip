// Single-launch layout + dispatch for small (decode-sized) batches.
//
// DeepEP ships separate low-latency kernels for inference decoding, and keeps
// two static buffers that alternate between calls (DeepEP analysis, feature
// list and "code notes": low-latency kernels, double buffer).  Here a decode
// call's layout and dispatch run in one launch instead of two: the results are
// exactly those of moe_layout followed by moe_dispatch.
//
// A workgroup owns one token (or one slice of its row, for very wide rows):
// wave 0 plus D data waves, each data lane 16 channels (FP8) or 8 (bf16).
//   1. Every wave requests what it reads -- the data waves their row slice,
//      every wave a share of the S*K routing entries, wave 0 the token's K
//      expert ids and weights -- and clears a share of the LDS counters.
//   2. Every wave counts its routing share into one packed LDS counter per
//      expert (low half: all entries, high half: entries before this token;
//      LDS atomics, since only counts matter here).
//   3. Wave 0 alone turns the counts into padded segment offsets (one DPP scan
//      over experts) and the token's K rows: segment start + entries of that
//      expert before the token + earlier k of the token with the same expert,
//      the same stable t*K+k order the layout kernels produce.  Meanwhile the
//      data waves wait for their row slice and quantise it (FP8), so the plan
//      overlaps the row loads' latency.
//   4. The data waves scatter their slice to the K rows; wave 0 writes the
//      token's pos, src and recv_w (first slice), the per-expert / per-rank
//      outputs and the status (workgroup 0), and its share of src = -1 on
//      padding rows.
// Three workgroup barriers separate the steps.  Counting runs on every wave
// because one wave's LDS atomics issue several times slower than the same
// number spread over the CU's four SIMDs.
#include "moe_kernels.h"
#include "small_layout.h"

namespace moe {
namespace {

// Data waves per workgroup: 4 (at most 4,096 channels of an FP8 row, 2,048 of a
// bf16 row, per workgroup) measured fastest at the decode shape on MI355X
// (7 or 3 data waves were 0.15-0.5 us slower per launch); at least 3, so a
// workgroup has 256 threads to share the routing entries (at the decode shape
// 1,024 entries: one counting pass per thread).
constexpr int kDataWaves = 4;
constexpr int kMinDataWaves = 3;

struct FusedLds : small::Counts {
    int rows[kMaxK];  // rows of the token's K entries (-1: not placed)
};

// Step 3 (wave 0): offsets into LDS (and, workgroup 0, tpe / eoff), the
// token's rows into L.rows.  `my_e` is lane k's expert id for k < K.
template <int K>
__device__ __forceinline__ int layout_wave(const LayoutArgs &a, int lane, int my_e, FusedLds &L) {
    const int flags = small::plan_offsets(a, lane, L);

    // lane k < K: row of the token's entry k
    int within_tok = 0;
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int ej = __builtin_amdgcn_readlane(my_e, j);
        within_tok += (j < lane && ej == my_e) ? 1 : 0;
    }
    if (lane < K) {
        const bool valid = my_e >= 0 && my_e < a.E;
        const int ek = valid ? my_e : 0;
        const int within = static_cast<int>(L.cnt[ek] >> 16) + within_tok;
        const bool placed = valid && !(a.pad_mode == PAD_CAPACITY && within >= a.pad_rows);
        L.rows[lane] = placed ? L.off[ek] + within : -1;
    }
    return flags;
}

// Wave 0, lane k < K of the token's first slice: pos, src and recv_w of entry k.
template <int K>
__device__ __forceinline__ void write_token_maps(const LayoutArgs &a, const DispatchArgs &da, int t, int lane,
                                                 float w, const FusedLds &L) {
    if (lane < K) {
        const int i = t * K + lane;
        const int row = L.rows[lane];
        a.pos[i] = row;
        if (row >= 0) {
            a.src[row] = i;
            if (da.recv_w != nullptr && da.topk_w != nullptr) da.recv_w[row] = w;
        }
    }
}

// blockDim.x = 64 * (1 + D); grid = S * nchunk.
template <int K, bool FP8>
__global__ __launch_bounds__((kDataWaves + 1) * kWave) void k_layout_dispatch(LayoutArgs la, DispatchArgs da,
                                                                                 int nchunk) {
    __shared__ FusedLds L;
    __shared__ int s_flags;
    const int t = blockIdx.x / nchunk, c = blockIdx.x % nchunk;
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid & (kWave - 1);
    const int per_chunk = nthr - kWave;                 // data lanes
    const int g = c * per_chunk + tid - kWave;          // this data lane's 16 (FP8) / 8 (bf16) channels
    const int ngroups = FP8 ? da.H / 16 : da.H / 8;
    const bool active = wave > 0 && g < ngroups;

    // step 1: requests first
    u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    if (active) {
        if (FP8) {
            const u32x4 *__restrict__ hid = static_cast<const u32x4 *>(da.hidden) + static_cast<size_t>(t) * (da.H / 8);
            lo = hid[2 * g];
            hi = hid[2 * g + 1];
        } else {
            lo = static_cast<const u32x4 *>(da.hidden)[static_cast<size_t>(t) * ngroups + g];
        }
    }
    int ev[small::kShare];
    small::load_share(la, tid, nthr, ev);
    int my_e = -1;
    float w = 0.0f;
    if (wave == 0) {
        if (lane < K) my_e = la.idx[static_cast<size_t>(t) * K + lane];
        if (c == 0 && lane < K && da.recv_w != nullptr && da.topk_w != nullptr)
            w = da.topk_w[static_cast<size_t>(t) * K + lane];
    }
    small::clear(la, tid, nthr, L);
    if (tid == 0) s_flags = 0;
    __syncthreads();

    // step 2: counts
    int flags = small::count(la, tid, nthr, t * K, ev, L);
    if (__ballot(flags) != 0 && lane == 0) atomicOr(&s_flags, FLAG_BAD_EXPERT);
    __syncthreads();

    // step 3: wave 0 plans while the data waves wait for their rows and
    // quantise them
    float scale = 0.0f;
    u32x4 q = {0u, 0u, 0u, 0u};
    if (wave == 0) {
        flags = layout_wave<K>(la, lane, my_e, L);
        if (c == 0) write_token_maps<K>(la, da, t, lane, w, L);
        if (__ballot(flags) != 0 && lane == 0) atomicOr(&s_flags, FLAG_CAPACITY);
    } else if (FP8) {
        q = quantize16_e4m3(lo, hi, scale);  // whole data waves: the block max crosses lanes
    } else {
        // the row as loaded, in registers of its own: once it has arrived
        // here no store below waits for a load
        q = lo;
        asm volatile("" : "+v"(q));
    }
    __syncthreads();

    // step 4: scatter
    if (wave == 0) {
        small::write_outputs(la, lane, s_flags, L);
        return;
    }
    if (!active) return;
    int p[K];
#pragma unroll
    for (int k = 0; k < K; ++k) p[k] = L.rows[k];
    u32x4 *__restrict__ recv = static_cast<u32x4 *>(da.recv);
    const size_t row_vec = FP8 ? da.H / 16 : da.H / 8;
    const int nsc = da.H / 128;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        if (p[k] >= 0) {
            __builtin_nontemporal_store(q, recv + static_cast<size_t>(p[k]) * row_vec + g);
            if (FP8 && (lane & 7) == 0) da.recv_scales[static_cast<size_t>(p[k]) * nsc + g / 8] = scale;
        }
    }
}

#define MOE_FUSED_CASES(FP8)                                                                        \
    switch (da.K) {                                                                                 \
        case 1: hipLaunchKernelGGL((k_layout_dispatch<1, FP8>), grid, block, 0, s, la, da, nchunk); break;   \
        case 2: hipLaunchKernelGGL((k_layout_dispatch<2, FP8>), grid, block, 0, s, la, da, nchunk); break;   \
        case 3: hipLaunchKernelGGL((k_layout_dispatch<3, FP8>), grid, block, 0, s, la, da, nchunk); break;   \
        case 4: hipLaunchKernelGGL((k_layout_dispatch<4, FP8>), grid, block, 0, s, la, da, nchunk); break;   \
        case 5: hipLaunchKernelGGL((k_layout_dispatch<5, FP8>), grid, block, 0, s, la, da, nchunk); break;   \
        case 6: hipLaunchKernelGGL((k_layout_dispatch<6, FP8>), grid, block, 0, s, la, da, nchunk); break;   \
        case 7: hipLaunchKernelGGL((k_layout_dispatch<7, FP8>), grid, block, 0, s, la, da, nchunk); break;   \
        case 8: hipLaunchKernelGGL((k_layout_dispatch<8, FP8>), grid, block, 0, s, la, da, nchunk); break;   \
        case 9: hipLaunchKernelGGL((k_layout_dispatch<9, FP8>), grid, block, 0, s, la, da, nchunk); break;   \
        case 10: hipLaunchKernelGGL((k_layout_dispatch<10, FP8>), grid, block, 0, s, la, da, nchunk); break; \
        case 11: hipLaunchKernelGGL((k_layout_dispatch<11, FP8>), grid, block, 0, s, la, da, nchunk); break; \
        case 12: hipLaunchKernelGGL((k_layout_dispatch<12, FP8>), grid, block, 0, s, la, da, nchunk); break; \
        case 13: hipLaunchKernelGGL((k_layout_dispatch<13, FP8>), grid, block, 0, s, la, da, nchunk); break; \
        case 14: hipLaunchKernelGGL((k_layout_dispatch<14, FP8>), grid, block, 0, s, la, da, nchunk); break; \
        case 15: hipLaunchKernelGGL((k_layout_dispatch<15, FP8>), grid, block, 0, s, la, da, nchunk); break; \
        case 16: hipLaunchKernelGGL((k_layout_dispatch<16, FP8>), grid, block, 0, s, la, da, nchunk); break; \
        default: return hipErrorInvalidValue;                                                       \
    }

}  // namespace

hipError_t launch_layout_dispatch_small(const LayoutArgs &la, const DispatchArgs &da, bool fp8, hipStream_t s) {
    const int groups = fp8 ? da.H / 16 : da.H / 8;
    int dw = (groups + kWave - 1) / kWave;
    if (dw > kDataWaves) dw = kDataWaves;
    if (dw < kMinDataWaves) dw = kMinDataWaves;
    const int nchunk = (groups + dw * kWave - 1) / (dw * kWave);
    const dim3 grid(static_cast<unsigned>(da.S) * nchunk), block((dw + 1) * kWave);
    if (fp8) {
        MOE_FUSED_CASES(true)
    } else {
        MOE_FUSED_CASES(false)
    }
    return hipGetLastError();
}

}  // namespace moe
