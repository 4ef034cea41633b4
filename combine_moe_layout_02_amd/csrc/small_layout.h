// Layout pieces for batches small enough (S*K <= 4096, decode-sized) that
// every workgroup recounts all entries itself instead of exchanging counts
// with the others.  Used by the one-launch layout + dispatch (fused.hip) and by
// the small-batch layout (layout.hip).
//
// Counting: one packed LDS counter per expert -- low 16 bits all entries, high
// 16 bits the entries before a given index -- so each entry costs one LDS
// atomic.  One wave then turns the counts into padded segment offsets (a DPP
// scan over experts); a stable row is segment start + entries of that expert
// before the entry, the ascending t*K+k order inside every segment.
#pragma once

#include "moe_kernels.h"

namespace moe {
namespace small {

constexpr int kMaxN = kFusedDispatchMaxN;  // entries a workgroup recounts, at most
constexpr int kShare = 8;                  // routing entries per thread per counting pass

struct Counts {
    unsigned int cnt[kMaxE];  // per expert: entries (low 16 bits), entries before the split (high 16)
    int off[kMaxE + 1];       // first row of each padded segment
    int pex[kMaxE + 1];       // placed rows before each expert
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

// Zeroes the counters (every thread of the workgroup takes a share; the caller
// then synchronises the workgroup).
__device__ __forceinline__ void clear(const LayoutArgs &a, int tid, int nthr, Counts &L) {
    for (int e = tid; e < a.E; e += nthr) L.cnt[e] = 0u;
}

// Thread tid of nthr counts entries tid, tid + nthr, ... into L.cnt (those
// below `split` also into the high half).  ev holds its first pass, requested
// with load_share(a, tid, nthr, ev) before the counters were cleared so the
// loads overlap that.  Returns FLAG_BAD_EXPERT if one of its entries has an id
// outside [0, E) (such entries are not counted).
__device__ __forceinline__ int count(const LayoutArgs &a, int tid, int nthr, int split, int (&ev)[kShare],
                                     Counts &L) {
    int flags = 0;
    for (int base = tid;;) {
#pragma unroll
        for (int u = 0; u < kShare; ++u) {
            const int i = base + u * nthr;
            const int e = ev[u];
            if (i < a.N) {
                if (e >= 0 && e < a.E)
                    atomicAdd(&L.cnt[e], i < split ? 0x10001u : 1u);
                else
                    flags = FLAG_BAD_EXPERT;
            }
        }
        base += kShare * nthr;
        if (base - tid >= a.N) break;
        load_share(a, base, nthr, ev);
    }
    return flags;
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

// One wave: the padded offsets of every expert into L.off / L.pex (and, in
// workgroup 0, tpe / eoff).  Lane l owns experts [l*ept, l*ept + ept).  One
// compact loop per pad mode: these kernels run once per call, so their
// instructions are fetched cold, and a generic body unrolled over every mode
// and every experts-per-lane count ran measurably slower.
template <int MODE>
__device__ __forceinline__ int plan_offsets_mode(const LayoutArgs &a, int lane, Counts &L) {
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

// plan_offsets_mode for the layout's pad mode, followed by wave_lds_order.
// Returns this lane's FLAG_CAPACITY.
__device__ __forceinline__ int plan_offsets(const LayoutArgs &a, int lane, Counts &L) {
    int flags;
    if (a.pad_mode == PAD_CAPACITY)
        flags = plan_offsets_mode<PAD_CAPACITY>(a, lane, L);
    else if (a.pad_mode == PAD_MULTIPLE)
        flags = plan_offsets_mode<PAD_MULTIPLE>(a, lane, L);
    else
        flags = plan_offsets_mode<PAD_NONE>(a, lane, L);
    wave_lds_order();
    return flags;
}

// One wave, after plan_offsets: the per-rank outputs and the status
// (workgroup 0; `flags` = the status word) and this workgroup's share of
// src = -1 on padding rows (experts e with e % gridDim == blockIdx, and every
// gridDim-th 64-row slice of the unused tail).  The padding ranges of 64 such
// experts come from one LDS round trip (one expert per lane); the wave then
// fills them one after another with coalesced stores, so the loop over
// experts waits on no LDS read (one read per expert and iteration made a
// workgroup with 256 experts to mark take over 30 us).
__device__ __forceinline__ void write_outputs(const LayoutArgs &a, int lane, int flags, const Counts &L) {
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
    for (int e0 = part; e0 < a.E; e0 += parts * kWave) {
        const int e = e0 + lane * parts;
        int beg = 0, end = 0;
        if (e < a.E) {
            beg = L.off[e] + (L.pex[e + 1] - L.pex[e]);
            end = L.off[e + 1];
        }
        for (int j = 0; j < kWave && e0 + j * parts < a.E; ++j) {
            const int b = __builtin_amdgcn_readlane(beg, j), en = __builtin_amdgcn_readlane(end, j);
            for (int r = b + lane; r < en; r += kWave) a.src[r] = -1;
        }
    }
    for (int r = L.off[a.E] + part * kWave + lane; r < a.max_recv; r += kWave * parts) a.src[r] = -1;
}

}  // namespace small
}  // namespace moe
