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
constexpr int kOnePassMaxN = 32768;  // one launch up to 32 tiles of 1024 entries
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

// Workgroup barrier that orders LDS accesses only.  __syncthreads also waits
// for every global load the wave has in flight; this one lets them stay in
// flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
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

// Inclusive prefix sum of an int across the 64 lanes of a wave, with DPP
// (data-parallel primitives on VALU operands, no LDS round trip): shifts by
// 1, 2, 4 and 8 lanes inside each row of 16 (lanes shifted in from outside the
// row add 0), then lane 15's sum is added to row 1 and lane 47's to row 3,
// then lane 31's to rows 2 and 3.  On MI355X about 100 cycles against ~480 for
// the same scan through six cross-lane shuffles.  All 64 lanes must be active:
// the cross-lane reads do not skip inactive lanes.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
    return v;
}

// Inclusive prefix sum of an int pair across the 64 lanes of a wave.
__device__ __forceinline__ int2 wave_inclusive_scan2(int2 v) {
    return make_int2(wave_inclusive_scan(v.x), wave_inclusive_scan(v.y));
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

// This lane's J entries of the wave's J*64 consecutive ones from `base`
// (expert ids; entries past N read as 0 and are masked later).  Issued before
// the workgroup clears its counters, so the load latency overlaps that work.
template <int J>
__device__ __forceinline__ void load_keys(const int32_t *__restrict__ idx, int N, int base, int (&raw)[J]) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int i = base + j * kWave + lane;
        raw[j] = i < N ? idx[i] : 0;
    }
}

// Ranks the wave's J*64 entries from `base` (raw = load_keys' values).  s_wcnt
// is the wave's [E] counter row (zero on entry; the wave's per-expert totals
// on exit).  key[j] = expert id or -1 (absent / out of range); local[j] =
// number of this wave's earlier entries with the same expert.
template <int J>
__device__ __forceinline__ void wave_rank(const int (&raw)[J], int N, int E, int nbits, int base,
                                          unsigned short *s_wcnt, int (&key)[J], int (&local)[J],
                                          int &flags) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int i = base + j * kWave + lane;
        const bool in = i < N;
        const int e = raw[j];
        const bool ok = in && e >= 0 && e < E;
        if (in && !ok) flags |= FLAG_BAD_EXPERT;
        const uint64_t m = match_key(e, ok, nbits);
        const int r = lanes_below(m);
        const int before = ok ? static_cast<int>(s_wcnt[e]) : 0;
        // every lane of the group has read the counter; the lowest one advances it
        if (ok && r == 0) s_wcnt[e] = static_cast<unsigned short>(before + __popcll(m));
        key[j] = ok ? e : -1;
        local[j] = before + r;
    }
}

// Per-wave counters of expert e -> exclusive prefixes over waves; returns the
// workgroup's total for e.  All 16 counters are read before the first write:
// read, write, read, ... in one loop made the compiler wait for each read in
// turn (it cannot tell the addresses apart), 16 LDS round trips in a row.
__device__ __forceinline__ int column_scan(unsigned short *s_cnt, int E, int e) {
    int c[kLayoutWaves];
#pragma unroll
    for (int w = 0; w < kLayoutWaves; ++w) c[w] = s_cnt[w * E + e];
    int run = 0;
#pragma unroll
    for (int w = 0; w < kLayoutWaves; ++w) {
        s_cnt[w * E + e] = static_cast<unsigned short>(run);
        run += c[w];
    }
    return run;
}

// Counts of the other tiles' entries for the one-launch layouts (one
// workgroup per 1024-entry tile, N <= 65535).  Per expert one packed counter:
// low 16 bits the entries of every tile but the workgroup's own, high 16 bits
// those of the tiles before it, so each entry costs one LDS atomic.  The
// counter has 1 << other_copies_log2(E) copies (8 for E <= 256), copy c taken
// by the threads with tid % copies == c, which spreads one instruction's
// atomics over more banks and addresses; other_total sums the copies.  At the
// prefill shape (32 tiles, E=256) 8 copies counted ~0.3 us faster than one.
constexpr int kOtherWords = 2048 + 8;  // LDS words of the copies for any E <= kMaxE, plus a spare expert
static_assert(kOnePassMaxN <= 65535, "other-tile counts are packed in 16 bits");
__device__ __forceinline__ int other_copies_log2(int E) { return E <= 256 ? 3 : (E <= 512 ? 2 : 1); }

// Zeroes the copies and the spare expert's (every thread of the workgroup;
// synchronise before counting).
__device__ __forceinline__ void other_clear(unsigned int *s_part, int E) {
    for (int x = threadIdx.x; x < ((E + 1) << other_copies_log2(E)); x += kLayoutThreads) s_part[x] = 0u;
}

// The aligned count reads rounds of 4 * 1024 entries, thread tid entries
// 4*tid .. 4*tid+3 of each round with one 16-byte load, kOtherBatch rounds in
// flight; one batch covers every batch the one-launch layouts take.
constexpr int kOtherGroup = 4 * kLayoutThreads;
constexpr int kOtherBatch = 8;
static_assert(kOnePassMaxN <= kOtherGroup * kOtherBatch, "one batch of loads covers a one-launch layout");

// Issues the loads of rounds g0 .. g0 + kOtherBatch - 1 that lie outside tile
// b (idx 16-byte aligned).  Slots past N are loaded as -1 and taken back out
// of nbad here.
__device__ __forceinline__ void other_issue(const int32_t *__restrict__ idx, int N, int b, int g0,
                                            int4 (&q)[kOtherBatch], int &nbad) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < kOtherBatch; ++u) {
        const int i = (g0 + u) * kOtherGroup + 4 * tid;
        if (i + 3 < N && i / kLayoutThreads != b) {
            q[u] = *reinterpret_cast<const int4 *>(idx + i);
        } else if (i < N && i / kLayoutThreads != b) {  // the ragged end of the batch
            q[u].x = idx[i];
            q[u].y = i + 1 < N ? idx[i + 1] : -1;
            q[u].z = i + 2 < N ? idx[i + 2] : -1;
            q[u].w = -1;
            nbad -= i + 4 - N;
        }
    }
}

// Adds what other_issue loaded into the packed counters (1 << CL copies, a
// constant, so the counter address is one shift-and-or).  An id outside
// [0,E) adds one to nbad and is counted into the spare expert E, which
// nothing reads, so every lane takes part in every atomic and the loop has no
// branches per entry.
template <int CL>
__device__ __forceinline__ void other_add(const int4 (&q)[kOtherBatch], int N, int E, int b, int g0,
                                          unsigned int *s_part, int &nbad) {
    const int tid = threadIdx.x;
    unsigned int *__restrict__ part = s_part + (tid & ((1 << CL) - 1));
    const unsigned int uE = static_cast<unsigned>(E);
#pragma unroll
    for (int u = 0; u < kOtherBatch; ++u) {
        const int i = (g0 + u) * kOtherGroup + 4 * tid, t = i / kLayoutThreads;
        if (i >= N || t == b) continue;
        const unsigned int inc = t < b ? 0x10001u : 1u;
        const int e4[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool ok = static_cast<unsigned>(e4[j]) < uE;
            nbad += ok ? 0 : 1;
            atomicAdd(part + ((ok ? e4[j] : E) << CL), inc);
        }
    }
}

// count_other_tiles with 1 << CL copies.
template <int CL, typename Between>
__device__ __forceinline__ void count_other_tiles_cl(const int32_t *__restrict__ idx, int N, int E, int nblk, int b,
                                                     unsigned int *s_part, int &nbad, Between &&between) {
    const int tid = threadIdx.x;
    unsigned int *__restrict__ part = s_part + (tid & ((1 << CL) - 1));
    const unsigned int uE = static_cast<unsigned>(E);
    if (N <= 0 || nblk <= 0) {
        between();
        return;
    }
    if ((reinterpret_cast<uintptr_t>(idx) & 15u) == 0) {
        for (int g0 = 0; g0 * kOtherGroup < N; g0 += kOtherBatch) {
            int4 q[kOtherBatch];
            other_issue(idx, N, b, g0, q, nbad);
            if (g0 == 0) between();
            other_add<CL>(q, N, E, b, g0, s_part, nbad);
        }
    } else {
        // idx not 16-byte aligned: entry t*1024 + tid of every tile t, 16 loads in flight
        constexpr int kBatch = 16;
        for (int t0 = 0; t0 < nblk; t0 += kBatch) {
            int ev[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int t = t0 + u, i = t * kLayoutThreads + tid;
                ev[u] = (t < nblk && t != b && i < N) ? idx[i] : 0;
            }
            if (t0 == 0) between();
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int t = t0 + u, i = t * kLayoutThreads + tid;
                if (t >= nblk || t == b || i >= N) continue;
                const bool ok = static_cast<unsigned>(ev[u]) < uE;
                nbad += ok ? 0 : 1;
                atomicAdd(part + ((ok ? ev[u] : E) << CL), t < b ? 0x10001u : 1u);
            }
        }
    }
}

// Counts every entry outside tile b into s_part (zeroed).  Entries with an
// expert outside [0,E) set FLAG_BAD_EXPERT in flags and are added to bad.
// Redundant work that lets one workgroup per tile know every count without
// talking to the others.  `between()` runs once, after the first loads are
// issued and before their counts: the caller's own work there (ranking its
// own tile) overlaps the load latency.
//
// Thread tid reads entries 4*tid + 4096*g (g = 0, 1, ...), four at a time with
// one 16-byte load when idx is 16-byte aligned, 8 such loads in flight: at 32
// tiles that is every load the thread makes, issued at once, and the count is
// then bound by the LDS atomics alone (one-by-one 4-byte loads in two batches
// of 16 kept the workgroup ~1.5 us longer on MI355X).  Four consecutive
// entries never straddle a tile, so each load's tile is one test.
template <typename Between>
__device__ __forceinline__ void count_other_tiles(const int32_t *__restrict__ idx, int N, int E, int nblk, int b,
                                                  unsigned int *s_part, int &flags, int &bad, Between &&between) {
    int nbad = 0;
    const int cl = other_copies_log2(E);
    if (cl == 3)
        count_other_tiles_cl<3>(idx, N, E, nblk, b, s_part, nbad, between);
    else if (cl == 2)
        count_other_tiles_cl<2>(idx, N, E, nblk, b, s_part, nbad, between);
    else
        count_other_tiles_cl<1>(idx, N, E, nblk, b, s_part, nbad, between);
    if (nbad) flags |= FLAG_BAD_EXPERT;
    bad += nbad;
}

// count_other_tiles for a one-launch layout whose loads other_issue already
// issued (round 0 on, idx 16-byte aligned): the caller issues them before it
// clears its counters, so their latency overlaps that work and its first
// barrier.  `between()` runs before the first count, as in count_other_tiles.
template <typename Between>
__device__ __forceinline__ void count_other_tiles_issued(const int4 (&q)[kOtherBatch], int N, int E, int b,
                                                         unsigned int *s_part, int nbad, int &flags, int &bad,
                                                         Between &&between) {
    between();
    const int cl = other_copies_log2(E);
    if (cl == 3)
        other_add<3>(q, N, E, b, 0, s_part, nbad);
    else if (cl == 2)
        other_add<2>(q, N, E, b, 0, s_part, nbad);
    else
        other_add<1>(q, N, E, b, 0, s_part, nbad);
    if (nbad) flags |= FLAG_BAD_EXPERT;
    bad += nbad;
}

// After count_other_tiles and a workgroup barrier: expert e's packed counter
// summed over its copies (contiguous: one or two 16-byte LDS reads).  s_part
// must be 16-byte aligned.
__device__ __forceinline__ unsigned int other_total(const unsigned int *s_part, int E, int e) {
    const int cl = other_copies_log2(E);
    if (cl == 3) {
        const uint4 x = reinterpret_cast<const uint4 *>(s_part)[2 * e];
        const uint4 y = reinterpret_cast<const uint4 *>(s_part)[2 * e + 1];
        return (x.x + x.y) + (x.z + x.w) + (y.x + y.y) + (y.z + y.w);
    }
    if (cl == 2) {
        const uint4 x = reinterpret_cast<const uint4 *>(s_part)[e];
        return (x.x + x.y) + (x.z + x.w);
    }
    const uint2 x = reinterpret_cast<const uint2 *>(s_part)[e];
    return x.x + x.y;
}

}  // namespace moe
