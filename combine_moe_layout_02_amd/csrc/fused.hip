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

namespace moe {
namespace {

// Data waves per workgroup: 4 (at most 4,096 channels of an FP8 row, 2,048 of a
// bf16 row, per workgroup) measured fastest at the decode shape on MI355X
// (7 or 3 data waves were 0.15-0.5 us slower per launch); at least 3, so a
// workgroup has 256 threads to share the routing entries.
constexpr int kDataWaves = 4;
constexpr int kMinDataWaves = 3;
// Routing entries per thread per pass: 8 (every thread's share at the decode
// shape, 1,024 entries over 320 threads, fits one pass; 4,096 entries take two).
constexpr int kShare = 8;

struct FusedLds {
    unsigned int cnt[kMaxE];  // per expert: entries (low 16 bits), entries before the token (high 16)
    int off[kMaxE + 1];       // first row of each padded segment
    int pex[kMaxE + 1];       // placed rows before each expert
    int rows[kMaxK];          // rows of the token's K entries (-1: not placed)
};

// Orders this wave's LDS accesses in the compiler's view; the hardware already
// runs one wave's LDS instructions in issue order.
__device__ __forceinline__ void wave_lds_order() {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Routing entries first, first + n, ..., first + (kShare-1)*n (0 past N).
__device__ __forceinline__ void load_share(const LayoutArgs &a, int first, int n, int (&ev)[kShare]) {
#pragma unroll
    for (int u = 0; u < kShare; ++u) {
        const int i = first + u * n;
        ev[u] = i < a.N ? a.idx[i] : 0;
    }
}

// Segment rows (x) and placed rows (y) of an expert with c entries under pad
// mode MODE; sets FLAG_CAPACITY in flags on overflow.
template <int MODE>
__device__ __forceinline__ int2 segment(int c, int pad_rows, int &flags) {
    if (MODE == PAD_MULTIPLE) return make_int2((c + pad_rows - 1) / pad_rows * pad_rows, c);
    if (MODE == PAD_CAPACITY) {
        if (c > pad_rows) flags |= FLAG_CAPACITY;
        return make_int2(pad_rows, c > pad_rows ? pad_rows : c);
    }
    return make_int2(c, c);
}

// Step 3, first half (wave 0): the padded offsets of every expert into LDS
// (and, workgroup 0, tpe / eoff).  Lane l owns experts [l*ept, l*ept + ept).
// One compact loop per pad mode: a generic body unrolled over every mode and
// every possible ept ran several times slower (its ~3,000 instructions are
// fetched once per launch).
template <int MODE>
__device__ __forceinline__ int plan_offsets(const LayoutArgs &a, int lane, FusedLds &L) {
    const int ept = (a.E + kWave - 1) / kWave;
    const int e0 = min(lane * ept, a.E), e1 = min(e0 + ept, a.E);
    int flags = 0;
    int2 sum = make_int2(0, 0);
#pragma unroll 4
    for (int e = e0; e < e1; ++e) {
        const int2 s = segment<MODE>(static_cast<int>(L.cnt[e] & 0xFFFFu), a.pad_rows, flags);
        sum.x += s.x;
        sum.y += s.y;
    }
    const int2 inc = wave_inclusive_scan2(sum);
    const bool wg0 = blockIdx.x == 0;
    int so = inc.x - sum.x, sp = inc.y - sum.y;
#pragma unroll 4
    for (int e = e0; e < e1; ++e) {
        int unused = 0;
        const int2 s = segment<MODE>(static_cast<int>(L.cnt[e] & 0xFFFFu), a.pad_rows, unused);
        L.off[e] = so;
        L.pex[e] = sp;
        if (wg0) {
            a.tpe[e] = s.y;
            a.eoff[e] = so;
        }
        so += s.x;
        sp += s.y;
    }
    if (lane == kWave - 1) {
        L.off[a.E] = inc.x;
        L.pex[a.E] = inc.y;
        if (wg0) a.eoff[a.E] = inc.x;
    }
    return flags;
}

// Step 3 (wave 0): offsets into LDS (and, workgroup 0, tpe / eoff), the
// token's rows into L.rows.  `my_e` is lane k's expert id for k < K.
template <int K>
__device__ __forceinline__ int layout_wave(const LayoutArgs &a, int lane, int my_e, FusedLds &L) {
    int flags;
    if (a.pad_mode == PAD_CAPACITY)
        flags = plan_offsets<PAD_CAPACITY>(a, lane, L);
    else if (a.pad_mode == PAD_MULTIPLE)
        flags = plan_offsets<PAD_MULTIPLE>(a, lane, L);
    else
        flags = plan_offsets<PAD_NONE>(a, lane, L);
    wave_lds_order();

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

// Wave 0, step 4: the per-rank outputs and status (workgroup 0), and this
// workgroup's share of src = -1 on padding rows.  flags: this workgroup's OR.
__device__ __forceinline__ void layout_wave_outputs(const LayoutArgs &a, int lane, int flags, const FusedLds &L) {
    if (blockIdx.x == 0) {
        const int epr = a.E / a.R;
        for (int r = lane; r < a.R; r += kWave) {
            a.roff[r] = L.off[r * epr];
            a.tpr[r] = L.pex[(r + 1) * epr] - L.pex[r * epr];
        }
        if (lane == 0) {
            a.roff[a.R] = L.off[a.E];
            a.status[0] = flags;
        }
    }
    const int part = blockIdx.x, parts = gridDim.x;
    for (int e = part; e < a.E; e += parts) {
        const int beg = L.off[e] + (L.pex[e + 1] - L.pex[e]);
        for (int r = beg + lane; r < L.off[e + 1]; r += kWave) a.src[r] = -1;
    }
    for (int r = L.off[a.E] + part * kWave + lane; r < a.max_recv; r += kWave * parts) a.src[r] = -1;
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
    int ev[kShare];
    load_share(la, tid, nthr, ev);
    int my_e = -1;
    float w = 0.0f;
    if (wave == 0) {
        if (lane < K) my_e = la.idx[static_cast<size_t>(t) * K + lane];
        if (c == 0 && lane < K && da.recv_w != nullptr && da.topk_w != nullptr)
            w = da.topk_w[static_cast<size_t>(t) * K + lane];
    }
    for (int e = tid; e < la.E; e += nthr) L.cnt[e] = 0u;
    if (tid == 0) s_flags = 0;
    __syncthreads();

    // step 2: counts
    const int before = t * K;
    int flags = 0;
    for (int base = tid;;) {
#pragma unroll
        for (int u = 0; u < kShare; ++u) {
            const int i = base + u * nthr;
            const int e = ev[u];
            if (i < la.N) {
                if (e >= 0 && e < la.E)
                    atomicAdd(&L.cnt[e], i < before ? 0x10001u : 1u);
                else
                    flags = FLAG_BAD_EXPERT;
            }
        }
        base += kShare * nthr;
        if (base - tid >= la.N) break;
        load_share(la, base, nthr, ev);
    }
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
        layout_wave_outputs(la, lane, s_flags, L);
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
