// Layout kernels: expert histogram, padded segment scan and stable positions.
//
// The receive buffer is grouped by expert, experts in ascending id, so rank r's
// partition is the contiguous run of its E/R experts (delect.ru glossary
// "Expert parallelism (EP)": experts spread over the ranks of a group, E/R
// local experts each; MoonEP article, section 3, Fig. 3: every rank's local
// experts in order).  Inside an expert's segment, entries keep ascending
// t*K+k order, so the layout is unique and reproducible.  Segments may be
// padded to a multiple or a fixed capacity (MoonEP basic usage,
// token_padding; search-results page, dynamic-routing snippet: zero-padding).
//
// Stable ranks without atomics on the order: each wave walks a contiguous run
// of entries 64 at a time; lanes holding the same expert id find each other
// with one ballot per key bit, take their rank from the lanes below them
// (mbcnt), and the lowest such lane advances that wave's private LDS counter.
// A column scan over the 16 per-wave counters then orders the waves.  Nothing
// depends on the order in which waves or workgroups run.
//
// Four variants (thresholds measured on MI355X):
//   small  (S*K <= 4096 and E > 64): 64 workgroups, each recounting every
//          entry with LDS atomics and placing 64 of them (k_layout_small).
//   single (S*K <= 2048): one 1024-thread workgroup does everything in one
//          launch.  Above that one CU cannot issue the scattered src stores
//          fast enough.
//   onepass (S*K <= 32768): one launch, one workgroup per 1024-entry tile,
//          each counting all other tiles itself (k_layout_onepass).  Its
//          counting grows with S*K: beyond 32 tiles two launches are faster.
//   multi  : k_layout_local ranks tiles of 1024*J entries, one workgroup per
//          tile, and writes a per-tile histogram; k_layout_place (one
//          workgroup per tile again) rebuilds the expert offsets from all tile
//          histograms -- cheaper than a separate scan launch -- and turns tile
//          ranks into rows.  Small tiles spread the scatter over more CUs.
#include "moe_kernels.h"
#include "small_layout.h"

namespace moe {
namespace {

// From per-expert counts (thread e < E holds count e): placed rows, padded
// segment lengths and their exclusive scans (into s_off / s_pex).  With
// `write_outputs`, also every output that depends only on counts.  Marks
// padding rows and the unused tail with src = -1: this workgroup takes part
// `part` of `parts` (experts e with e % parts == part, and every parts-th
// 1024-row slice of the tail).  Called by all 1024 threads; returns this
// thread's capacity flag.
__device__ int finish_counts(const LayoutArgs &a, int cnt, int *s_off, int *s_pex, int2 *s_tmp,
                             bool write_outputs, int part, int parts) {
    const int tid = threadIdx.x;
    const bool is_e = tid < a.E;
    int placed = is_e ? cnt : 0, seg = placed, flags = 0;
    if (is_e) {
        if (a.pad_mode == PAD_MULTIPLE) {
            seg = (cnt + a.pad_rows - 1) / a.pad_rows * a.pad_rows;
        } else if (a.pad_mode == PAD_CAPACITY) {
            seg = a.pad_rows;
            if (cnt > a.pad_rows) { placed = a.pad_rows; flags = FLAG_CAPACITY; }
        }
    }
    int2 total;
    const int2 ex = block_exclusive_scan2(make_int2(seg, placed), s_tmp, total);
    if (is_e) {
        s_off[tid] = ex.x;
        s_pex[tid] = ex.y;
    }
    if (tid == 0) {
        s_off[a.E] = total.x;
        s_pex[a.E] = total.y;
    }
    __syncthreads();
    if (write_outputs) {
        if (is_e) {
            a.tpe[tid] = placed;
            a.eoff[tid] = ex.x;
        }
        if (tid == 0) a.eoff[a.E] = total.x;
        const int epr = a.E / a.R;
        if (tid < a.R) {
            a.roff[tid] = s_off[tid * epr];
            a.tpr[tid] = s_pex[(tid + 1) * epr] - s_pex[tid * epr];
        }
        if (tid == 0) a.roff[a.R] = s_off[a.E];
    }
    const int wave = tid / kWave, lane = tid & (kWave - 1);
    for (int e = part + wave * parts; e < a.E; e += kLayoutWaves * parts) {
        const int beg = s_off[e] + (s_pex[e + 1] - s_pex[e]);
        const int end = s_off[e + 1];
        for (int r = beg + lane; r < end; r += kWave) a.src[r] = -1;
    }
    for (int r = s_off[a.E] + part * kLayoutThreads + tid; r < a.max_recv; r += kLayoutThreads * parts)
        a.src[r] = -1;
    return flags;
}

template <int J>
__global__ __launch_bounds__(kLayoutThreads) void k_layout_fused(LayoutArgs a) {
    extern __shared__ unsigned short s_cnt[];  // [kLayoutWaves][E]
    __shared__ int s_off[kMaxE + 1], s_pex[kMaxE + 1];
    __shared__ int2 s_tmp[kLayoutWaves];
    __shared__ int s_flags;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
    const int base = wave * kWave * J;
    int raw[J];
    load_keys<J>(a.idx, a.N, base, raw);
    for (int x = tid; x < kLayoutWaves * a.E; x += kLayoutThreads) s_cnt[x] = 0;
    if (tid == 0) s_flags = 0;
    __syncthreads();

    int key[J], local[J], flags = 0;
    wave_rank<J>(raw, a.N, a.E, a.nbits, base, s_cnt + wave * a.E, key, local, flags);
    __syncthreads();
    const int cnt = tid < a.E ? column_scan(s_cnt, a.E, tid) : 0;
    flags |= finish_counts(a, cnt, s_off, s_pex, s_tmp, true, 0, 1);  // synchronises the workgroup

#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int i = base + j * kWave + lane;
        if (i >= a.N) continue;
        int p = -1;
        const int e = key[j];
        if (e >= 0) {
            const int within = s_cnt[wave * a.E + e] + local[j];
            if (!(a.pad_mode == PAD_CAPACITY && within >= a.pad_rows)) p = s_off[e] + within;
        }
        a.pos[i] = p;
        if (p >= 0) a.src[p] = i;
    }
    if (flags) atomicOr(&s_flags, flags);
    __syncthreads();
    if (tid == 0) a.status[0] = s_flags;
}

// Small batches (S*K <= 4096, more than 64 experts): 64 workgroups of 256
// threads, workgroup b owning entries [64b, 64b + 64), so the scattered pos /
// src stores and the padding rows' src = -1 spread over 64 CUs.  All four
// waves recount every entry into packed counters (all entries / entries
// before this workgroup's first), then wave 0 scans them into padded offsets
// and places its 64 entries: row = segment start + entries of that expert
// before this workgroup + lanes below with the same expert (one ballot per key
// bit), the stable t*K+k order.  Workgroup 0 writes the count outputs and the
// status; every workgroup marks its share of padding rows.  64 workgroups even
// for a few entries: at fixed capacity a decode batch has ~31,000 padding rows
// to mark, and fewer workgroups took longer (16: +0.7 us, 1: +24 us).
constexpr int kPlaceShare = 16;  // threads per expert reading tile histograms in k_layout_place
constexpr int kSmallMinE = 64;  // with fewer experts the single workgroup measured faster
constexpr int kSmallThreads = 256;
constexpr int kSmallBlocks = small::kMaxN / kWave;

__global__ __launch_bounds__(kSmallThreads) void k_layout_small(LayoutArgs a) {
    __shared__ small::Counts L;
    __shared__ int s_flags;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int first = blockIdx.x * kWave;  // this workgroup's entries: [first, first + 64)
    int ev[small::kShare];
    small::load_share(a, tid, kSmallThreads, ev);
    const int i = first + lane;
    const int mine = (wave == 0 && i < a.N) ? a.idx[i] : -1;
    small::clear(a, tid, kSmallThreads, L);
    if (tid == 0) s_flags = 0;
    __syncthreads();

    const int bad = small::count(a, tid, kSmallThreads, first, ev, L);
    if (__ballot(bad) != 0 && lane == 0) atomicOr(&s_flags, FLAG_BAD_EXPERT);
    __syncthreads();
    if (wave != 0) return;

    const int cap = small::plan_offsets(a, lane, L);
    const bool in = i < a.N;
    const bool ok = in && mine >= 0 && mine < a.E;
    const uint64_t m = match_key(mine, ok, a.nbits);
    const int within = ok ? static_cast<int>(L.cnt[mine] >> 16) + lanes_below(m) : 0;
    const bool placed = ok && !(a.pad_mode == PAD_CAPACITY && within >= a.pad_rows);
    const int row = placed ? L.off[mine] + within : -1;
    if (in) {
        a.pos[i] = row;
        if (row >= 0) a.src[row] = i;
    }
    small::write_outputs(a, lane, s_flags | (__ballot(cap) != 0 ? FLAG_CAPACITY : 0), L);
}

template <int J>
__global__ __launch_bounds__(kLayoutThreads) void k_layout_local(LayoutArgs a) {
    extern __shared__ unsigned short s_cnt[];  // [kLayoutWaves][E]
    __shared__ int s_flags;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
    const int base = blockIdx.x * kLayoutThreads * J + wave * kWave * J;
    int raw[J];
    load_keys<J>(a.idx, a.N, base, raw);
    for (int x = tid; x < kLayoutWaves * a.E; x += kLayoutThreads) s_cnt[x] = 0;
    if (tid == 0) s_flags = 0;
    __syncthreads();

    int key[J], local[J], flags = 0;
    wave_rank<J>(raw, a.N, a.E, a.nbits, base, s_cnt + wave * a.E, key, local, flags);
    if (flags) atomicOr(&s_flags, flags);
    __syncthreads();
    if (tid < a.E) a.blk_hist[static_cast<size_t>(blockIdx.x) * a.E + tid] = column_scan(s_cnt, a.E, tid);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int i = base + j * kWave + lane;
        if (i < a.N) a.pos[i] = key[j] >= 0 ? s_cnt[wave * a.E + key[j]] + local[j] : -1;
    }
    if (tid == 0) a.blk_flags[blockIdx.x] = s_flags;
}

// Placement pass of the multi-workgroup layout; workgroup b owns tile b
// (tiles of J*1024 entries, as in k_layout_local<J>).
template <int J>
__global__ __launch_bounds__(kLayoutThreads) void k_layout_place(LayoutArgs a) {
    __shared__ int s_off[kMaxE + 1], s_pex[kMaxE + 1], s_pre[kMaxE];
    __shared__ int2 s_tmp[kLayoutWaves];
    __shared__ int2 s_part[kLayoutThreads];  // [P][E] partial (before b, all) sums
    __shared__ int s_flags;
    const int tid = threadIdx.x, b = blockIdx.x;
    // this tile's expert ids and tile ranks, loaded first: nothing below
    // changes them before they are used
    int e_in[J], rank_in[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int i = b * kLayoutThreads * J + j * kLayoutThreads + tid;
        e_in[j] = i < a.N ? a.idx[i] : -1;
        rank_in[j] = i < a.N ? a.pos[i] : -1;
    }
    if (tid == 0) s_flags = 0;
    // Per expert, the entries in the tiles before b and in all tiles, from the
    // per-tile histograms.  P threads share an expert (thread tid: expert
    // tid % E, tiles tid / E, tid / E + P, ...) and meet in LDS: the
    // histograms were written by other XCDs, so every load misses this L2,
    // and one thread per expert took two rounds of 32 such loads at 48 tiles.
    const int P = min(kLayoutThreads / a.E, kPlaceShare);
    if (tid < P * a.E) {
        const int e = tid % a.E, q = tid / a.E;
        int2 part = make_int2(0, 0);
        constexpr int kBatch = 16;
        for (int t0 = q; t0 < a.nblk; t0 += kBatch * P) {
            int c[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int t = t0 + u * P;
                c[u] = t < a.nblk ? a.blk_hist[static_cast<size_t>(t) * a.E + e] : 0;
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                part.x += (t0 + u * P < b) ? c[u] : 0;
                part.y += c[u];
            }
        }
        s_part[q * a.E + e] = part;
    }
    int flags = 0;
    if (b == 0)
        for (int t = tid; t < a.nblk; t += kLayoutThreads) flags |= a.blk_flags[t];
    __syncthreads();
    int cnt = 0;
    if (tid < a.E) {
        int pre = 0;
        for (int q = 0; q < P; ++q) {
            const int2 v = s_part[q * a.E + tid];
            pre += v.x;
            cnt += v.y;
        }
        s_pre[tid] = pre;
    }
    flags |= finish_counts(a, cnt, s_off, s_pex, s_tmp, b == 0, b, a.nblk);  // synchronises the workgroup
    // tile b's entries: tile rank -> row
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int i = b * kLayoutThreads * J + j * kLayoutThreads + tid;
        if (i >= a.N) break;
        const int e = e_in[j];
        if (e < 0 || e >= a.E) continue;  // already -1
        const int within = s_pre[e] + rank_in[j];
        int p = -1;
        if (!(a.pad_mode == PAD_CAPACITY && within >= a.pad_rows)) p = s_off[e] + within;
        a.pos[i] = p;
        if (p >= 0) a.src[p] = i;
    }
    if (b == 0) {
        if (flags) atomicOr(&s_flags, flags);
        __syncthreads();
        if (tid == 0) a.status[0] = s_flags;
    }
}

// One-launch layout for mid-sized batches (tiles of 1024 entries, one
// workgroup each).  Workgroup b ranks its own tile as k_layout_local does and
// counts every other tile's entries itself (count_other_tiles: one packed
// counter per expert, entries of all other tiles and of the tiles before b),
// so without any exchange between workgroups it knows the per-expert totals
// and the entries of earlier tiles; then it places its tile as k_layout_place
// does.  The redundant counting costs one 16-byte load per thread per four
// tiles, served from L2 once the first workgroups have touched topk_idx, and
// one LDS atomic per entry; the own tile is ranked while those loads are out.
// They are issued first, before the counters are cleared: after a kernel that
// streamed hundreds of MB, topk_idx comes from HBM, and that wait is the
// longest in the kernel (issuing them after the first barrier instead cost
// ~0.8 us per call on MI355X in that sequence).
__global__ __launch_bounds__(kLayoutThreads) void k_layout_onepass(LayoutArgs a) {
    extern __shared__ unsigned short s_cnt[];  // [kLayoutWaves][E]
    __shared__ int s_off[kMaxE + 1], s_pex[kMaxE + 1], s_before[kMaxE];
    __shared__ __align__(16) unsigned int s_part[kOtherWords];
    __shared__ int2 s_tmp[kLayoutWaves];
    __shared__ int s_flags;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1), b = blockIdx.x;
    const int nblk = gridDim.x;
    const int base = b * kLayoutThreads + wave * kWave;
    int raw[1];
    load_keys<1>(a.idx, a.N, base, raw);
    // the other tiles' entries, loaded before anything else when idx allows
    // 16-byte loads (one batch covers every one-launch size)
    const bool issued = (reinterpret_cast<uintptr_t>(a.idx) & 15u) == 0;
    int4 q[kOtherBatch];
    int nbad = 0;
    if (issued) other_issue(a.idx, a.N, b, 0, q, nbad);
    for (int x = tid; x < kLayoutWaves * a.E; x += kLayoutThreads) s_cnt[x] = 0;
    other_clear(s_part, a.E);
    if (tid == 0) s_flags = 0;
    lds_barrier();  // the loads above stay in flight
    // nothing that reads the own key may move above the barrier: a use
    // there makes the wave wait for every load issued before it
    asm volatile("" : "+v"(raw[0]));

    int flags = 0, bad = 0;
    int key[1], local[1];
    const auto rank_own = [&] { wave_rank<1>(raw, a.N, a.E, a.nbits, base, s_cnt + wave * a.E, key, local, flags); };
    if (issued)
        count_other_tiles_issued(q, a.N, a.E, b, s_part, nbad, flags, bad, rank_own);
    else
        count_other_tiles(a.idx, a.N, a.E, nblk, b, s_part, flags, bad, rank_own);
    __syncthreads();
    int cnt = 0;
    if (tid < a.E) {
        const unsigned int other = other_total(s_part, a.E, tid);
        s_before[tid] = static_cast<int>(other >> 16);
        cnt = column_scan(s_cnt, a.E, tid) + static_cast<int>(other & 0xFFFFu);
    }
    flags |= finish_counts(a, cnt, s_off, s_pex, s_tmp, b == 0, b, nblk);  // synchronises the workgroup

    const int i = base + lane;
    if (i < a.N) {
        int p = -1;
        const int e = key[0];
        if (e >= 0) {
            const int within = s_before[e] + s_cnt[wave * a.E + e] + local[0];
            if (!(a.pad_mode == PAD_CAPACITY && within >= a.pad_rows)) p = s_off[e] + within;
        }
        a.pos[i] = p;
        if (p >= 0) a.src[p] = i;
    }
    if (b == 0) {  // workgroup 0 has seen every entry: it reports the status
        if (flags) atomicOr(&s_flags, flags);
        __syncthreads();
        if (tid == 0) a.status[0] = s_flags;
    }
}

hipError_t launch_onepass(const LayoutArgs &a, size_t lds, hipStream_t s) {
    const int nblk = (a.N + kLayoutThreads - 1) / kLayoutThreads;
    hipLaunchKernelGGL(k_layout_onepass, dim3(nblk), dim3(kLayoutThreads), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_small(const LayoutArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_layout_small, dim3(kSmallBlocks), dim3(kSmallThreads), 0, s, a);
    return hipGetLastError();
}

template <int J>
hipError_t launch_fused(const LayoutArgs &a, size_t lds, hipStream_t s) {
    hipLaunchKernelGGL(k_layout_fused<J>, dim3(1), dim3(kLayoutThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace

size_t layout_workspace_bytes(int64_t N, int E) {
    if (N <= kOnePassMaxN) return 0;
    const int64_t tile = static_cast<int64_t>(kLayoutThreads) * multi_tile_j(N);
    const int64_t nblk = (N + tile - 1) / tile;
    const size_t bytes = static_cast<size_t>(nblk) * E * sizeof(int32_t) + static_cast<size_t>(nblk) * sizeof(int32_t);
    return (bytes + 255) / 256 * 256;
}

template <int J>
hipError_t launch_multi(LayoutArgs a, size_t lds, hipStream_t s) {
    const int tile = kLayoutThreads * J;
    a.nblk = (a.N + tile - 1) / tile;
    a.blk_flags = a.blk_hist + static_cast<size_t>(a.nblk) * a.E;
    hipLaunchKernelGGL(k_layout_local<J>, dim3(a.nblk), dim3(kLayoutThreads), lds, s, a);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_layout_place<J>, dim3(a.nblk), dim3(kLayoutThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_layout(const LayoutArgs &a, hipStream_t s) {
    const size_t lds = static_cast<size_t>(kLayoutWaves) * a.E * sizeof(unsigned short);
    if (a.N <= small::kMaxN && a.E > kSmallMinE) return launch_small(a, s);
    if (a.N <= kSingleMaxN) {
        if (a.N <= kLayoutThreads) return launch_fused<1>(a, lds, s);
        return launch_fused<2>(a, lds, s);
    }
    if (a.N <= kOnePassMaxN) return launch_onepass(a, lds, s);
    switch (multi_tile_j(a.N)) {
        case 1: return launch_multi<1>(a, lds, s);
        case 2: return launch_multi<2>(a, lds, s);
        default: return launch_multi<4>(a, lds, s);
    }
}

}  // namespace moe
