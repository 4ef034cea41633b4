// Balanced layout: every rank receives the same number of rows, however skewed
// the routing, by moving the surplus of overloaded ranks into redundant copies
// of their experts held in per-rank slots (MoonEP article, section 1: perfect
// balance through a few redundant experts planned online; section 3 and
// Fig. 3: each rank's local experts followed by B prefetch slots).
//
// The pages give the invariant, not the planning rule.  The rule here (the
// plain greedy reading):
//   quota q[r] = N/R, plus one for the first N%R ranks (N = valid entries);
//   overloaded ranks in ascending order shed their surplus from their largest
//   experts first (ties: lower id), each expert at most all of its entries;
//   every shed piece goes to the lowest rank still below its quota that has a
//   free slot, as much as that rank's room allows, then to the next one; each
//   (expert, destination) piece takes one slot; if no rank is left the rest
//   stays home and status bit 2 is set.
// An expert's first entries (t*K+k order) stay home; the following ones fill
// its replicas in creation order.  Rows are rank-major: the rank's E/R home
// segments in expert order, then its B slot segments.
//
// Implementation: the plain layout is computed first (into workspace); it
// gives each entry's stable rank inside its expert (pos - expert_offset).
// k_balance_place then runs on G workgroups; each one rebuilds the plan --
// counts and loads, the per-rank size order of experts (each thread counts the
// experts ahead of its own), every expert's shed amount (parallel: it depends
// only on its rank's surplus and larger experts), the compacted list of shed
// pieces (workgroup scan), their merge into destinations (one thread, a
// forward-only destination cursor held in registers: O(pieces + replicas)
// steps), segment offsets (workgroup scan) -- and remaps its share of entries.
// Workgroup 0 writes the per-expert / per-rank / per-segment outputs.
#include "moe_kernels.h"

namespace moe {
namespace {

// Entries of the strictly increasing a[0..n) below v / not above v.
__device__ __forceinline__ int count_below(const int *a, int n, int v) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] < v) lo = mid + 1; else hi = mid;
    }
    return lo;
}
__device__ __forceinline__ int count_upto(const int *a, int n, int v) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] <= v) lo = mid + 1; else hi = mid;
    }
    return lo;
}

struct BalanceLds {
    int cnt[kMaxE];           // entries per expert
    int eoff_std[kMaxE];      // plain layout's expert offsets
    int home[kMaxE];          // entries that stay on the owner
    int order[kMaxE];         // experts of each rank, largest first
    int first_rep[kMaxE];     // first replica of each expert (creation order)
    int nrep_e[kMaxE];
    int room[kMaxE];          // quota - load, per rank (R <= E)
    int piece_e[kMaxE];       // shed pieces in planning order: expert, amount
    int piece_n[kMaxE];
    int dest_r[kMaxE];        // ranks below their quota, ascending, and their room
    int dest_room[kMaxE];
    int rep_e[kMaxBalanceSlots];
    int rep_n[kMaxBalanceSlots];
    int rep_rs[kMaxBalanceSlots];    // (destination rank << 8) | slot
    int slot_rep[kMaxBalanceSlots];  // replica held by (rank, slot), -1 if none
    int mrep[kMaxBalanceSlots];      // parallel merge: replicas before each merged breakpoint
    int A[kMaxE];             // start of each piece in the shed stream
    int C[kMaxE];             // start of each destination in the room stream
    int shed[kMaxE];          // entries shed by the expert at each planning position
    int seg_off[kMaxE + kMaxBalanceSlots + 1];
    int2 tmp[kLayoutWaves];
    int4 tmp4[kLayoutWaves];
    int flags;
};

// Exclusive prefix sums of four ints at once across the workgroup, in thread
// order (the four component scans of one pass share its two barriers).
// Returns the prefix; `total` gets the workgroup totals.
__device__ __forceinline__ int4 block_exclusive_scan4(int4 v, int4 *s_tmp, int4 &total) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int4 inc = make_int4(wave_inclusive_scan(v.x), wave_inclusive_scan(v.y), wave_inclusive_scan(v.z),
                               wave_inclusive_scan(v.w));
    if (lane == kWave - 1) s_tmp[wave] = inc;
    __syncthreads();
    int4 before = make_int4(0, 0, 0, 0), all = make_int4(0, 0, 0, 0);
#pragma unroll
    for (int w = 0; w < kLayoutWaves; ++w) {
        const int4 t = s_tmp[w];
        if (w < wave) {
            before.x += t.x; before.y += t.y; before.z += t.z; before.w += t.w;
        }
        all.x += t.x; all.y += t.y; all.z += t.z; all.w += t.w;
    }
    __syncthreads();
    total = all;
    return make_int4(before.x + inc.x - v.x, before.y + inc.y - v.y, before.z + inc.z - v.z,
                     before.w + inc.w - v.w);
}

// The plan, from L.cnt (entries per expert, visible to every thread) and
// L.flags; valid = entries with an expert in range.  Called by all threads of
// the workgroup (it synchronises).  Leaves home, first_rep, nrep_e, the
// replica lists, slot_rep and the segment offsets seg_off in L.
__device__ __forceinline__ void plan_balance(BalanceLds &L, int E, int R, int B, int valid) {
    const int tid = threadIdx.x;
    const int epr = E / R, nseg = epr + B, ngrp = R * nseg;
    // Step 1, from the counts alone: initial results, and for every expert its
    // place in its rank's size order (count descending, id ascending) and the
    // entries it sheds -- its rank's surplus (load - quota) minus the counts
    // of the rank's larger experts, clamped to [0, count]: what the sequential
    // plan takes from it as long as destinations do not run out.  One walk
    // over the rank's experts gives the place, the larger experts' counts and
    // the rank's load.  Results go to the expert's planning position (ranks
    // ascending, size order); the first expert of each rank stores its room.
    for (int e = tid; e < E; e += kLayoutThreads) {
        L.home[e] = L.cnt[e];
        L.first_rep[e] = 0;
        L.nrep_e[e] = 0;
    }
    for (int q = tid; q < R * B; q += kLayoutThreads) L.slot_rep[q] = -1;
    if (tid < E) {
        const int e = tid, r = e / epr, r0 = r * epr, c = L.cnt[e];
        int before = 0, larger = 0, load = 0, j = r0;
        for (; j + 8 <= r0 + epr; j += 8) {   // 8 LDS reads in flight
            int c8[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) c8[u] = L.cnt[j + u];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const bool ahead = c8[u] > c || (c8[u] == c && j + u < e);
                before += ahead ? 1 : 0;
                larger += ahead ? c8[u] : 0;
                load += c8[u];
            }
        }
        for (; j < r0 + epr; ++j) {
            const int cj = L.cnt[j];
            const bool ahead = cj > c || (cj == c && j < e);
            before += ahead ? 1 : 0;
            larger += ahead ? cj : 0;
            load += cj;
        }
        const int room = valid / R + (r < valid % R ? 1 : 0) - load;
        const int my = -room - larger;
        L.order[r0 + before] = e;
        L.shed[r0 + before] = my < 0 ? 0 : (my > c ? c : my);
        if (e == r0) L.room[r] = room;
    }
    __syncthreads();
    const int my = tid < E ? L.shed[tid] : 0;

    // Step 2, one scan for four things: the non-zero pieces compacted in
    // planning order with their starts in the shed stream (A), and the ranks
    // below their quota (destinations, ascending) with their starts in the
    // room stream (C).
    const int room = tid < R ? L.room[tid] : 0;
    int4 tot4;
    const int4 ex4 = block_exclusive_scan4(make_int4(my > 0 ? 1 : 0, my, room > 0 ? 1 : 0, room > 0 ? room : 0),
                                          L.tmp4, tot4);
    if (my > 0) {
        L.piece_e[ex4.x] = L.order[tid];
        L.piece_n[ex4.x] = my;
        L.A[ex4.x] = ex4.y;
    }
    if (room > 0) {
        L.dest_r[ex4.z] = tid;
        L.dest_room[ex4.z] = room;
        L.C[ex4.z] = ex4.w;
    }
    const int npiece = tot4.x, T = tot4.y, ndest = B > 0 ? tot4.z : 0;
    __syncthreads();

    // Step 3: merge of pieces into destinations.  Laid end to end, the pieces
    // and the destinations' rooms both cover [0, T): the overloaded ranks'
    // surpluses add up to the other ranks' rooms.  A replica is a non-empty
    // overlap of one piece's span with one destination's span, numbered in
    // stream order -- what the sequential greedy below produces whenever no
    // destination needs more than B slots.  If one would, or the totals differ,
    // the parallel results are undone and the sequential loop runs instead.
    bool merged = false;
    if (npiece > 0 && ndest > 0 && npiece + ndest <= kMaxBalanceSlots) {  // uniform
        const int *A = L.A, *C = L.C;
        // merged breakpoints, ties: piece start first (its interval is then empty)
        const int M = npiece + ndest;
        int *mval = L.seg_off;  // scratch until the segment scan
        if (tid < npiece) mval[tid + count_below(C, ndest, A[tid])] = A[tid];
        if (tid < ndest) mval[tid + count_upto(A, npiece, C[tid])] = C[tid];
        __syncthreads();
        const int len = tid < M ? (tid + 1 < M ? mval[tid + 1] : T) - mval[tid] : 0;
        int2 rtot;
        const int2 rex = block_exclusive_scan2(make_int2(len > 0 ? 1 : 0, 0), L.tmp, rtot);
        if (tid < M) L.mrep[tid] = rex.x;
        __syncthreads();
        bool bad = false;
        if (len > 0) {
            const int q = rex.x;
            const int d = count_upto(C, ndest, mval[tid]) - 1;                    // destination holding it
            const int slot = q - L.mrep[d + count_upto(A, npiece, C[d])];          // its first replica is slot 0
            if (slot < B) {
                const int pc = count_upto(A, npiece, mval[tid]) - 1;              // piece holding it
                const int dr = L.dest_r[d];
                L.rep_e[q] = L.piece_e[pc];
                L.rep_n[q] = len;
                L.rep_rs[q] = (dr << 8) | slot;
                L.slot_rep[dr * B + slot] = q;
            } else {
                bad = true;
            }
        }
        if (tid < npiece) {
            const int e = L.piece_e[tid];
            const int first = L.mrep[tid + count_below(C, ndest, A[tid])];
            const int next = tid + 1 < npiece ? L.mrep[tid + 1 + count_below(C, ndest, A[tid + 1])] : rtot.x;
            L.home[e] = L.cnt[e] - L.piece_n[tid];
            L.first_rep[e] = first;
            L.nrep_e[e] = next - first;
        }
        merged = !__syncthreads_or(bad || T != tot4.w);
        if (!merged) {  // undo: the sequential loop starts from the initial results
            for (int e = tid; e < E; e += kLayoutThreads) {
                L.home[e] = L.cnt[e];
                L.first_rep[e] = 0;
                L.nrep_e[e] = 0;
            }
            for (int q = tid; q < R * B; q += kLayoutThreads) L.slot_rep[q] = -1;
            __syncthreads();
        }
    }

    // Sequential merge (one thread), used when the parallel form does not
    // apply.  The cursors only move forward; the next piece and the next
    // destination are read one step ahead, so the loop carries no LDS read
    // latency, and each expert's results are written once, when its piece ends.
    if (!merged && tid == 0) {
        int flags = L.flags, nrep = 0;
        int pc = 0, e = 0, left = 0, moved = 0, first = 0;
        int ne = 0, nleft = 0;
        if (npiece > 0) {
            e = L.piece_e[0];
            left = L.piece_n[0];
            if (npiece > 1) { ne = L.piece_e[1]; nleft = L.piece_n[1]; }
        }
        int di = 0, dr = 0, droom = 0, dslots = 0, ndr = 0, ndroom = 0;
        if (ndest > 0) {
            dr = L.dest_r[0];
            droom = L.dest_room[0];
            if (ndest > 1) { ndr = L.dest_r[1]; ndroom = L.dest_room[1]; }
        }
        while (pc < npiece) {
            if (di >= ndest) {
                flags |= FLAG_UNBALANCED;
                break;
            }
            const int take = left < droom ? left : droom;
            L.rep_e[nrep] = e;
            L.rep_n[nrep] = take;
            L.rep_rs[nrep] = (dr << 8) | dslots;
            L.slot_rep[dr * B + dslots] = nrep;
            ++nrep;
            ++dslots;
            droom -= take;
            left -= take;
            moved += take;
            if (droom == 0 || dslots == B) {        // destination full: next one
                ++di;
                dr = ndr;
                droom = ndroom;
                dslots = 0;
                if (di + 1 < ndest) { ndr = L.dest_r[di + 1]; ndroom = L.dest_room[di + 1]; }
            }
            if (left == 0) {                         // piece done: record, next piece
                L.home[e] = L.cnt[e] - moved;
                L.first_rep[e] = first;
                L.nrep_e[e] = nrep - first;
                ++pc;
                e = ne;
                left = nleft;
                moved = 0;
                first = nrep;
                if (pc + 1 < npiece) { ne = L.piece_e[pc + 1]; nleft = L.piece_n[pc + 1]; }
            }
        }
        if (pc < npiece && moved > 0) {              // stopped inside a piece
            L.home[e] = L.cnt[e] - moved;
            L.first_rep[e] = first;
            L.nrep_e[e] = nrep - first;
        }
        L.flags = flags;
    }
    __syncthreads();

    // Step 4: segment sizes -> offsets.
    auto seg_size = [&](int g) -> int {
        const int r = g / nseg, j = g % nseg;
        if (j < epr) return L.home[r * epr + j];
        const int q = L.slot_rep[r * B + (j - epr)];
        return q >= 0 ? L.rep_n[q] : 0;
    };
    if (!(L.flags & FLAG_UNBALANCED)) {  // uniform
        // Every rank holds exactly its quota, so rank r starts after the
        // quotas of the ranks before it; one wave scans each rank's segments.
        const int wave = tid / kWave, lane = tid & (kWave - 1);
        const int c = (nseg + kWave - 1) / kWave;  // segments per lane
        for (int r = wave; r < R; r += kLayoutWaves) {
            const int start = r * (valid / R) + min(r, valid % R);
            const int j0 = min(lane * c, nseg), j1 = min(j0 + c, nseg);
            int sum = 0;
            for (int j = j0; j < j1; ++j) sum += seg_size(r * nseg + j);
            int run = start + wave_inclusive_scan(sum) - sum;
            for (int j = j0; j < j1; ++j) {
                const int n = seg_size(r * nseg + j);
                L.seg_off[r * nseg + j] = run;
                run += n;
            }
        }
        if (tid == 0) L.seg_off[ngrp] = valid;
    } else {
        // each thread scans a run of consecutive segments
        const int per = (ngrp + kLayoutThreads - 1) / kLayoutThreads;
        const int g0 = tid * per;
        int local = 0;
        for (int g = g0; g < g0 + per && g < ngrp; ++g) local += seg_size(g);
        int2 total;
        const int2 ex = block_exclusive_scan2(make_int2(local, 0), L.tmp, total);
        int run = ex.x;
        for (int g = g0; g < g0 + per && g < ngrp; ++g) {
            L.seg_off[g] = run;
            run += seg_size(g);
        }
        if (tid == 0) L.seg_off[ngrp] = total.x;
    }
    __syncthreads();
}

// Row of the k-th entry (stable t*K+k order) of expert e under the plan:
// the first home[e] stay in the home segment, the rest fill the replicas in
// creation order.
__device__ __forceinline__ int balanced_row(const BalanceLds &L, int e, int k, int epr, int nseg) {
    if (k < L.home[e]) return L.seg_off[(e / epr) * nseg + (e % epr)] + k;
    k -= L.home[e];
    const int q0 = L.first_rep[e], q1 = q0 + L.nrep_e[e];
    for (int q = q0; q < q1; ++q) {
        if (k < L.rep_n[q]) {
            const int rs = L.rep_rs[q];
            return L.seg_off[(rs >> 8) * nseg + epr + (rs & 0xFF)] + k;
        }
        k -= L.rep_n[q];
    }
    return -1;
}

// Outputs that depend only on the plan (one workgroup writes them).
__device__ __forceinline__ void write_balance_counts(const BalanceLds &L, const BalanceArgs &b) {
    const int tid = threadIdx.x;
    const int E = b.E, R = b.R, B = b.B, epr = E / R, nseg = epr + B, ngrp = R * nseg;
    for (int g = tid; g <= ngrp; g += kLayoutThreads) b.seg_offset[g] = L.seg_off[g];
    for (int e = tid; e < E; e += kLayoutThreads) {
        b.tpe[e] = L.cnt[e];
        b.eoff[e] = L.seg_off[(e / epr) * nseg + (e % epr)];
    }
    for (int r = tid; r < R; r += kLayoutThreads) {
        b.roff[r] = L.seg_off[r * nseg];
        b.tpr[r] = L.seg_off[(r + 1) * nseg] - L.seg_off[r * nseg];
    }
    for (int q = tid; q < R * B; q += kLayoutThreads) {
        const int rep = L.slot_rep[q];
        b.slot_expert[q] = rep >= 0 ? L.rep_e[rep] : -1;
    }
    if (tid == 0) {
        b.eoff[E] = L.seg_off[ngrp];
        b.roff[R] = L.seg_off[ngrp];
        b.status[0] = L.flags;
    }
}

// Two-step form: the plain layout ran first (into workspace) and gives each
// entry's stable rank inside its expert (pos - expert_offset).  G workgroups
// each rebuild the plan and remap their share of entries.
__global__ __launch_bounds__(kLayoutThreads) void k_balance_place(BalanceArgs b) {
    __shared__ BalanceLds L;
    const int tid = threadIdx.x;
    const int E = b.E, R = b.R, B = b.B, epr = E / R, nseg = epr + B, ngrp = R * nseg;
    // Everything read from global memory is requested up front, so the plan
    // overlaps one round trip: this workgroup's first entries (expert, plain
    // row) and the valid-entry total.
    const int stride = gridDim.x * kLayoutThreads;
    const int i0 = blockIdx.x * kLayoutThreads + tid;
    const int e_first = i0 < b.N ? b.idx[i0] : -1;
    const int p_first = i0 < b.N ? b.pos_std[i0] : 0;
    const int valid = b.eoff_std[E];
    for (int e = tid; e < E; e += kLayoutThreads) {
        L.cnt[e] = b.tpe_std[e];
        L.eoff_std[e] = b.eoff_std[e];
    }
    if (tid == 0) L.flags = b.status_std[0];
    __syncthreads();
    plan_balance(L, E, R, B, valid);
    if (blockIdx.x == 0) write_balance_counts(L, b);

    // this workgroup's entries: stable rank inside the expert -> balanced row
    for (int i = i0; i < b.N; i += stride) {
        const int e = i == i0 ? e_first : b.idx[i];
        int row = -1;
        if (e >= 0 && e < E) row = balanced_row(L, e, (i == i0 ? p_first : b.pos_std[i]) - L.eoff_std[e], epr, nseg);
        b.pos[i] = row;
        if (row >= 0) b.src[row] = i;
    }
    // rows past the valid ones (only when some ids were out of range)
    for (int r = L.seg_off[ngrp] + blockIdx.x * kLayoutThreads + tid; r < b.N; r += stride) b.src[r] = -1;
}

// One-launch form for batches of up to 32 tiles of 1024 entries, one
// workgroup per tile.  Each workgroup counts the other tiles itself and ranks
// its own tile (as the one-launch plain layout does), so it holds every
// expert's count and each of its entries' stable rank inside its expert with
// no exchange between workgroups; then it builds the plan and places its own
// entries.  No plain layout is written or read back.
__global__ __launch_bounds__(kLayoutThreads) void k_layout_balanced_onepass(LayoutArgs a, BalanceArgs b) {
    extern __shared__ unsigned short s_cnt[];  // [kLayoutWaves][E]
    __shared__ int s_before[kMaxE];
    __shared__ __align__(16) unsigned int s_part[kOtherWords];
    __shared__ BalanceLds L;
    __shared__ int s_bad;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1), tb = blockIdx.x;
    const int E = a.E, epr = E / b.R, nseg = epr + b.B, ngrp = b.R * nseg, nblk = gridDim.x;
    const int base = tb * kLayoutThreads + wave * kWave;
    int raw[1];
    load_keys<1>(a.idx, a.N, base, raw);
    // the other tiles' entries, loaded before anything else when idx allows
    // 16-byte loads (one batch covers every one-launch size)
    const bool issued = (reinterpret_cast<uintptr_t>(a.idx) & 15u) == 0;
    int4 q[kOtherBatch];
    int nbad = 0;
    if (issued) other_issue(a.idx, a.N, tb, 0, q, nbad);
    for (int x = tid; x < kLayoutWaves * E; x += kLayoutThreads) s_cnt[x] = 0;
    other_clear(s_part, E);
    if (tid == 0) {
        s_bad = 0;
        L.flags = 0;
    }
    lds_barrier();  // the loads above stay in flight
    // nothing that reads the own key may move above the barrier: a use
    // there makes the wave wait for every load issued before it
    asm volatile("" : "+v"(raw[0]));

    int flags = 0, bad = 0;
    int key[1], local[1];
    const auto rank_own = [&] { wave_rank<1>(raw, a.N, E, a.nbits, base, s_cnt + wave * E, key, local, flags); };
    if (issued)
        count_other_tiles_issued(q, a.N, E, tb, s_part, nbad, flags, bad, rank_own);
    else
        count_other_tiles(a.idx, a.N, E, nblk, tb, s_part, flags, bad, rank_own);
    if (base + lane < a.N && key[0] < 0) ++bad;
    if (flags) atomicOr(&L.flags, flags);
    if (bad) atomicAdd(&s_bad, bad);
    __syncthreads();
    if (tid < E) {
        const unsigned int other = other_total(s_part, E, tid);
        s_before[tid] = static_cast<int>(other >> 16);
        L.cnt[tid] = column_scan(s_cnt, E, tid) + static_cast<int>(other & 0xFFFFu);
    }
    __syncthreads();
    plan_balance(L, E, b.R, b.B, a.N - s_bad);
    if (tb == 0) write_balance_counts(L, b);

    const int i = base + lane;
    if (i < a.N) {
        const int e = key[0];
        const int row = e >= 0 ? balanced_row(L, e, s_before[e] + s_cnt[wave * E + e] + local[0], epr, nseg) : -1;
        b.pos[i] = row;
        if (row >= 0) b.src[row] = i;
    }
    // rows past the valid ones (only when some ids were out of range)
    for (int r = L.seg_off[ngrp] + tb * kLayoutThreads + tid; r < a.N; r += nblk * kLayoutThreads) b.src[r] = -1;
}

}  // namespace

size_t balance_workspace_bytes(int64_t N, int E, int R) {
    if (N <= kOnePassMaxN) return 0;  // one launch, no plain layout to hold
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    return up(static_cast<size_t>(N) * 4) * 2 + up(static_cast<size_t>(E) * 4) + up(static_cast<size_t>(R) * 4) +
           up(static_cast<size_t>(E + 1) * 4) + up(static_cast<size_t>(R + 1) * 4) + up(4) +
           layout_workspace_bytes(N, E);
}

hipError_t launch_layout_balanced(const LayoutArgs &la_in, BalanceArgs b, void *workspace, hipStream_t s) {
    if (la_in.N <= kOnePassMaxN) {
        const int nblk = la_in.N > 0 ? (la_in.N + kLayoutThreads - 1) / kLayoutThreads : 1;
        const size_t lds = static_cast<size_t>(kLayoutWaves) * la_in.E * sizeof(unsigned short);
        hipLaunchKernelGGL(k_layout_balanced_onepass, dim3(nblk), dim3(kLayoutThreads), lds, s, la_in, b);
        return hipGetLastError();
    }
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    char *ws = static_cast<char *>(workspace);
    const int64_t N = la_in.N;
    LayoutArgs la = la_in;  // the plain layout, written to workspace
    la.pos = reinterpret_cast<int32_t *>(ws); ws += up(static_cast<size_t>(N) * 4);
    la.src = reinterpret_cast<int32_t *>(ws); ws += up(static_cast<size_t>(N) * 4);
    la.tpe = reinterpret_cast<int32_t *>(ws); ws += up(static_cast<size_t>(la.E) * 4);
    la.tpr = reinterpret_cast<int32_t *>(ws); ws += up(static_cast<size_t>(la.R) * 4);
    la.eoff = reinterpret_cast<int32_t *>(ws); ws += up(static_cast<size_t>(la.E + 1) * 4);
    la.roff = reinterpret_cast<int32_t *>(ws); ws += up(static_cast<size_t>(la.R + 1) * 4);
    la.status = reinterpret_cast<int32_t *>(ws); ws += up(4);
    la.blk_hist = reinterpret_cast<int32_t *>(ws);
    la.pad_mode = PAD_NONE;
    la.pad_rows = 0;
    la.max_recv = static_cast<int32_t>(N);
    hipError_t err = launch_layout(la, s);
    if (err != hipSuccess) return err;
    b.pos_std = la.pos;
    b.tpe_std = la.tpe;
    b.eoff_std = la.eoff;
    b.status_std = la.status;
    const int64_t wgs = (N + kLayoutThreads - 1) / kLayoutThreads;
    const int grid = static_cast<int>(wgs < 1 ? 1 : (wgs > 256 ? 256 : wgs));
    hipLaunchKernelGGL(k_balance_place, dim3(grid), dim3(kLayoutThreads), 0, s, b);
    return hipGetLastError();
}

}  // namespace moe
