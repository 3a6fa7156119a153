// Deterministic device-wide sparse map for gfx950.
//
// Computes, for flat routes f = 0 .. N-1 (N = S*k) with expert ids[f]:
//   counts[e]      = #{f : ids[f] = e}                  (histogram)
//   offsets[e]     = sum_{e' < e} counts[e']            (exclusive scan)
//   sparse_rows[f] = offsets[e] + #{f' < f : ids[f'] = e}
//   slot_src[sparse_rows[f]] = f
// following the Histogram(e) / Offsets(e) equations of the ScatterMoE guide
// ("2. Grouped Coordinate Indexing Without Padding") and the pass structure
// of the Fast-LLM scalable sparse map (histogram pass, then assignment).
// Unlike that pull request's atomic slot claim, the assignment here is a
// stable rank, so the map is identical on every run.
//
// Layout of the work: routes are taken 64 at a time by a wavefront; a lane's
// rank among the lanes of its group holding the same expert is a popcount of
// their lane mask, and the group's count per expert goes to a per-wave LDS
// counter. No global atomics are used anywhere. Large maps:
//   pass 1 (hist):    per chunk of routes, counts by LDS atomic adds (the
//                     sum does not depend on their order) -> cnt[e][chunk]
//   pass 2 (rowscan): per expert, exclusive scan over chunks, total
//   pass 3 (assign):  offsets from the totals, then per chunk a local stable
//                     sort by expert in LDS (lane masks built by OR-ing each
//                     lane's bit into one LDS word per wave and expert) ->
//                     slots, written out in runs
// Small maps (at most 8192 routes) take all three steps in one workgroup,
// with the lane masks from one ballot per id bit (match-any).
#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "launch.hpp"
#include "profile.hpp"

namespace smoe {

constexpr int kMaxExperts = 1024;

__device__ __forceinline__ unsigned long long match_any(int key, int nbits) {
    unsigned long long m = __ballot(1);
    for (int b = 0; b < nbits; ++b) {
        const int bit = (key >> b) & 1;
        const unsigned long long bb = __ballot(bit);
        m &= bit ? bb : ~bb;
    }
    return m;
}

// Block-wide exclusive scan of one int per thread (WAVES wavefronts); returns
// the exclusive prefix and writes the block total to *total. s_tmp holds
// WAVES ints.
template <int WAVES>
__device__ int block_exscan(int v, int *s_tmp, int *total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d);
        if (lane >= d) x += y;
    }
    if (lane == 63) s_tmp[w] = x;
    __syncthreads();
    int wave_base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < WAVES; ++i) {
        if (i < w) wave_base += s_tmp[i];
        tot += s_tmp[i];
    }
    __syncthreads();
    *total = tot;
    return wave_base + x - v;
}

__global__ __launch_bounds__(256) void smap_rowscan_kernel(int32_t *__restrict__ cnt, int nsub,
                                                            int32_t *__restrict__ totals) {
    __shared__ int s_tmp[4];
    const int e = blockIdx.x;
    int32_t *row = cnt + (size_t)e * nsub;
    int running = 0;
    for (int base = 0; base < nsub; base += 256 * 4) {
        int v[4], s = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = base + threadIdx.x * 4 + i;
            v[i] = idx < nsub ? row[idx] : 0;
            s += v[i];
        }
        int tot;
        int pre = block_exscan<4>(s, s_tmp, &tot) + running;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = base + threadIdx.x * 4 + i;
            if (idx < nsub) row[idx] = pre;
            pre += v[i];
        }
        running += tot;
    }
    if (threadIdx.x == 0) totals[e] = running;
}

// The whole map in one workgroup of 1024 threads, for maps of at most
// kSmallMapRoutes routes (decode-sized batches), where the three launches
// of the general path cost more than the work. Wave w takes the contiguous
// chunk [w L, (w + 1) L) of routes (L a multiple of 64), so a route's rank
// among the routes of its expert is: earlier waves' counts of that expert,
// then earlier groups of 64 in its own wave, then lower lanes of its own
// group -- the same stable slot as the general path. A lane loads its ids
// once, all in one round, and keeps them for both passes.
constexpr int kSmallMapRoutes = 8192;
constexpr int kSmallMapWaves = 16;
constexpr int kSmallPerLane = kSmallMapRoutes / (kSmallMapWaves * 64);  // groups of 64 per wave, at most
static_assert(kSmallMapRoutes % (kSmallMapWaves * 64) == 0, "a wave's chunk of at most kSmallMapRoutes / 16 routes fits kSmallPerLane groups");

__global__ __launch_bounds__(1024) void smap_small_kernel(const int32_t *__restrict__ ids, int N, int E, int nbits,
                                                          int L, int32_t *__restrict__ expert_counts,
                                                          int32_t *__restrict__ expert_offsets,
                                                          int32_t *__restrict__ sparse_rows,
                                                          int32_t *__restrict__ slot_src) {
    __shared__ int32_t s_cnt[kSmallMapWaves * kMaxExperts];  // [wave][expert]: count, then base
    __shared__ int s_tmp[kSmallMapWaves];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int base = w * L;
    // route base + 64 j + lane, or the sentinel E past the wave's chunk, past N or out of range
    int ev[kSmallPerLane];
#pragma unroll
    for (int j = 0; j < kSmallPerLane; ++j) {
        const int f = base + 64 * j + lane;
        int e = (64 * j < L && f < N) ? ids[f] : E;
        if ((unsigned)e >= (unsigned)E) e = E;
        ev[j] = e;
    }
    int32_t *my = s_cnt + w * E;
    for (int e = lane; e < E; e += 64) my[e] = 0;
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    // pass 1: per-wave counts (only a group's lowest lane of an expert writes)
#pragma unroll
    for (int j = 0; j < kSmallPerLane; ++j) {
        if (64 * j < L) {
            const int e = ev[j];
            const unsigned long long m = match_any(e, nbits);
            const int leader = __ffsll(m) - 1;
            if (lane == leader && e < E) my[e] += __popcll(m);
        }
    }
    __syncthreads();
    // totals and their exclusive scan (thread e owns expert e; E <= 1024), then
    // each wave's starting slot per expert, in wave order
    const int e = threadIdx.x;
    int tot_e = 0;
    if (e < E)
        for (int i = 0; i < kSmallMapWaves; ++i) tot_e += s_cnt[i * E + e];
    int x = tot_e;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d);
        if (lane >= d) x += y;
    }
    if (lane == 63) s_tmp[w] = x;
    __syncthreads();
    int off = x - tot_e, total = 0;
#pragma unroll
    for (int i = 0; i < kSmallMapWaves; ++i) {
        if (i < w) off += s_tmp[i];
        total += s_tmp[i];
    }
    if (e < E) {
        expert_counts[e] = tot_e;
        expert_offsets[e] = off;
        int run = off;
        for (int i = 0; i < kSmallMapWaves; ++i) {
            const int c = s_cnt[i * E + e];
            s_cnt[i * E + e] = run;
            run += c;
        }
    }
    if (e == 0) expert_offsets[E] = total;
    __syncthreads();
    // pass 2: slots
#pragma unroll
    for (int j = 0; j < kSmallPerLane; ++j) {
        if (64 * j < L) {
            const int f = base + 64 * j + lane;
            const int ex = ev[j];
            const unsigned long long m = match_any(ex, nbits);
            const int leader = __ffsll(m) - 1;
            int b = (lane == leader && ex < E) ? my[ex] : 0;
            b = __shfl(b, leader);
            if (ex < E) {
                const int slot = b + __popcll(m & lt);
                sparse_rows[f] = slot;
                slot_src[slot] = f;
            } else if (f < N) {
                sparse_rows[f] = -1;
            }
            if (lane == leader && ex < E) my[ex] = b + __popcll(m);
        }
    }
}

// ---- large maps: chunks of routes per workgroup ----
//
// The routes are cut into chunks of C consecutive routes, one chunk per
// workgroup. The histogram pass counts each chunk's routes per expert with
// LDS atomic adds (cnt[e][chunk]; counts commute, so the order of the adds
// does not matter). After the row scan over chunks, the assignment pass
// walks its chunk in rounds of kAssignWaves waves x RG groups of 64 routes
// (wave w takes the round's w-th run of RG * 64 routes), ranks each round's
// routes stably by expert (match-any ranks within a group of 64, per-wave
// counters over the wave's groups, the waves' prefix per expert and the
// prefix over experts), places them in that order in LDS, writes
// sparse_rows in route order and then slot_src from the local order: the
// routes of one expert in one round have consecutive slots, so slot_src
// leaves as runs of consecutive words instead of one scattered word per
// lane. The next round's ids are loaded while the current round is ranked.
constexpr int kHistThreads = 256;
constexpr int kHistUnroll = 8;  // routes per thread whose ids are in flight together
constexpr int kAssignWaves = 8;
constexpr int kAssignThreads = kAssignWaves * 64;

template <int U>
__global__ __launch_bounds__(kHistThreads) void smap_chunk_hist_kernel(const int32_t *__restrict__ ids, int N, int E,
                                                                       int C, int nchunks, int32_t *__restrict__ cnt) {
    extern __shared__ int32_t s_hist[];  // [E]
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kHistThreads) s_hist[e] = 0;
    __syncthreads();
    // offsets within the chunk, so that no index passes N (N < 2^31)
    const int *chunk = ids + (size_t)blockIdx.x * C;
    const int len = min(N - (int)blockIdx.x * C, C);
    for (int o = 0; o < len; o += kHistThreads * U) {
        int v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = o + u * kHistThreads + tid;
            v[u] = i < len ? chunk[i] : -1;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if ((unsigned)v[u] < (unsigned)E) atomicAdd(&s_hist[v[u]], 1);  // ids outside [0, E) get no slot
    }
    __syncthreads();
    for (int e = tid; e < E; e += kHistThreads) cnt[(size_t)e * nchunks + blockIdx.x] = s_hist[e];
}

constexpr size_t chunk_hist_lds_bytes(int E) { return (size_t)E * sizeof(int32_t); }
constexpr size_t chunk_assign_lds_bytes(int E, int RG) {
    return (size_t)kAssignThreads * RG * sizeof(int2) + (size_t)kAssignWaves * E * sizeof(unsigned long long) +
           (size_t)(kAssignWaves + 2) * E * sizeof(int32_t);
}

template <int RG>
__global__ __launch_bounds__(kAssignThreads) void smap_chunk_assign_kernel(
    const int32_t *__restrict__ ids, int N, int E, int C, int nchunks, const int32_t *__restrict__ cnt,
    const int32_t *__restrict__ totals, int32_t *__restrict__ expert_counts, int32_t *__restrict__ expert_offsets,
    int32_t *__restrict__ sparse_rows, int32_t *__restrict__ slot_src) {
    constexpr int T = kAssignThreads, W = kAssignWaves, ROUND = T * RG;
    constexpr int EPT = (kMaxExperts + T - 1) / T;
    // LDS (chunk_assign_lds_bytes):
    //   s_pair [ROUND]  the round's (slot, route) pairs in local order (sorted by expert)
    //   s_peer [W][E]   per-wave 64-bit lane masks
    //   s_wc   [W][E]   per-wave counts of the round, then each wave's first
    //                   local position for expert e
    //   s_base [E]      next slot of expert e in this chunk
    //   s_delta[E]      slot - local position, for the round's routes of expert e
    extern __shared__ int2 s_pair[];
    unsigned long long *s_peer = reinterpret_cast<unsigned long long *>(s_pair + ROUND);
    int32_t *s_wc = reinterpret_cast<int32_t *>(s_peer + W * E);
    int32_t *s_base = s_wc + W * E;
    int32_t *s_delta = s_base + E;
    __shared__ int s_tmp[W];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    unsigned long long *peer = s_peer + w * E;
    int32_t *my = s_wc + w * E;
    // route f = base + i of the chunk, 0 <= i < len; indices are formed as
    // offsets within the chunk, so that none passes N (N < 2^31)
    const int base = blockIdx.x * C;
    const int len = min(N - base, C);
    const int *chunk = ids + base;
    int32_t *rows = sparse_rows + base;

    // the first round's ids are in flight while the offsets are formed
    int ev[RG];
#pragma unroll
    for (int u = 0; u < RG; ++u) {
        const int i = (w * RG + u) * 64 + lane;
        ev[u] = i < len ? chunk[i] : -1;
    }
    // offsets = exclusive scan of the per-expert totals; thread t owns experts
    // t * EPT .. t * EPT + EPT - 1 (E <= 1024)
    {
        int tv[EPT], cv[EPT], sum = 0;
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = tid * EPT + i;
            tv[i] = e < E ? totals[e] : 0;
            cv[i] = e < E ? cnt[(size_t)e * nchunks + blockIdx.x] : 0;  // scanned over chunks
            sum += tv[i];
        }
        int tot;
        int off = block_exscan<W>(sum, s_tmp, &tot);
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = tid * EPT + i;
            if (e < E) {
                s_base[e] = off + cv[i];
                if (blockIdx.x == 0) {
                    expert_counts[e] = tv[i];
                    expert_offsets[e] = off;
                }
            }
            off += tv[i];
        }
        if (blockIdx.x == 0 && tid == 0) expert_offsets[E] = tot;
    }
    for (int o = 0; o < len; o += ROUND) {
        for (int e = lane; e < E; e += 64) my[e] = 0;
        // ranks within the wave (groups in order, lanes in order); only lanes
        // with an id in [0, E) take part. The lanes of one group holding the
        // same expert find each other through the wave's LDS word peer[e]:
        // cleared, then each such lane ORs in its own bit, then read back
        // (a wave's LDS operations complete in issue order, and OR commutes,
        // so the mask does not depend on the order of the lanes' ORs).
        int rk[RG];
#pragma unroll
        for (int u = 0; u < RG; ++u) {
            const int e = ev[u];
            const bool valid = (unsigned)e < (unsigned)E;
            unsigned long long m = 0;
            int c = 0;
            if (valid) peer[e] = 0;
            __builtin_amdgcn_wave_barrier();
            if (valid) atomicOr(&peer[e], 1ull << lane);
            __builtin_amdgcn_wave_barrier();
            if (valid) {
                m = peer[e];
                c = my[e];
            }
            __builtin_amdgcn_wave_barrier();
            rk[u] = c + __popcll(m & lt);
            if (valid && lane == __ffsll(m) - 1) my[e] = c + __popcll(m);
            __builtin_amdgcn_wave_barrier();
        }
        // the next round's ids
        int nx[RG];
#pragma unroll
        for (int u = 0; u < RG; ++u) {
            const int i = o + ROUND + (w * RG + u) * 64 + lane;
            nx[u] = i < len ? chunk[i] : -1;
        }
        __syncthreads();
        // per expert: the run length over the waves, the runs' starts (scan
        // over experts), then each wave's first position and the slot offset
        int wc[EPT][W], te[EPT], sum = 0;
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = tid * EPT + i;
            te[i] = 0;
#pragma unroll
            for (int v = 0; v < W; ++v) {
                wc[i][v] = e < E ? s_wc[v * E + e] : 0;
                te[i] += wc[i][v];
            }
            sum += te[i];
        }
        int round_total;
        int lofs = block_exscan<W>(sum, s_tmp, &round_total);
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = tid * EPT + i;
            if (e < E) {
                int p = lofs;
#pragma unroll
                for (int v = 0; v < W; ++v) {
                    s_wc[v * E + e] = p;
                    p += wc[i][v];
                }
                const int b = s_base[e];
                s_delta[e] = b - lofs;
                s_base[e] = b + te[i];  // read again in the next round's transform
            }
            lofs += te[i];
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < RG; ++u) {
            const int i = o + (w * RG + u) * 64 + lane;
            const int e = ev[u];
            if ((unsigned)e < (unsigned)E) {  // only loaded lanes (i < len) hold ids in [0, E)
                const int lpos = my[e] + rk[u];
                const int slot = s_delta[e] + lpos;
                s_pair[lpos] = make_int2(slot, base + i);
                rows[i] = slot;
            } else if (i < len) {
                rows[i] = -1;  // id outside [0, E): the route gets no slot
            }
        }
        __syncthreads();
        // slot_src from the local order: consecutive positions of one expert are consecutive slots
        for (int q = tid; q < round_total; q += T) {
            const int2 pr = s_pair[q];
            slot_src[pr.x] = pr.y;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < RG; ++u) ev[u] = nx[u];
    }
}

__global__ void smap_empty_kernel(int E, int32_t *expert_counts, int32_t *expert_offsets) {
    for (int e = threadIdx.x; e <= E; e += blockDim.x) {
        if (e < E) expert_counts[e] = 0;
        expert_offsets[e] = 0;
    }
}

SparseMapPlan sparse_map_plan(int64_t N, int E) {
    SparseMapPlan pl;
    // rounds of kAssignThreads * RG routes (RG = 8 from 2^18 routes, else 1
    // so that mid-sized maps still spread over many workgroups), one round
    // per chunk, chunks doubled while there would be more than
    // max(2048, 2^20 / E) of them, so that the per-chunk count matrix stays
    // within 4 MiB for E <= 512
    const int64_t max_chunks = std::max<int64_t>(2048, ((int64_t)1 << 20) / std::max(E, 1));
    pl.rg = N >= ((int64_t)1 << 18) ? 8 : 1;
    int64_t C = (int64_t)kAssignThreads * pl.rg;
    while ((N + C - 1) / C > max_chunks) C *= 2;
    pl.L = (int)C;
    pl.nsub = (int)((N + C - 1) / C);
    pl.ws_bytes = (size_t)E * (size_t)pl.nsub * sizeof(int32_t) + (size_t)E * sizeof(int32_t);
    return pl;
}

// ---- no-allocation form ----
// Scratch of the no-allocation entry point: one copy per GPU in the code
// object's static device memory, held until the process ends. Host code never
// uses this name as an address (on the host it is only a stand-in for the
// symbol): the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) char scratch[kSparseMapNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t sparse_map_noalloc_scratch(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_sparse_map(const int32_t *ids, int N, int E, int32_t *expert_counts, int32_t *expert_offsets,
                             int32_t *sparse_rows, int32_t *slot_src, void *workspace, hipStream_t stream) {
    if (N == 0) {
        prof_begin(stream, kKMapEmpty);
        smap_empty_kernel<<<1, 256, 0, stream>>>(E, expert_counts, expert_offsets);
        prof_end(stream, kKMapEmpty);
        return hipGetLastError();
    }
    if (N <= kSmallMapRoutes) {
        // chunks of whole groups of 64 routes, one per wave (L <= 64 * kSmallPerLane)
        const int L = ((N + kSmallMapWaves - 1) / kSmallMapWaves + 63) / 64 * 64;
        prof_begin(stream, kKMapSmall);
        const int sbits = 32 - __builtin_clz((unsigned)E);  // bits to hold 0..E (E is the sentinel)
        smap_small_kernel<<<1, 1024, 0, stream>>>(ids, N, E, sbits, L, expert_counts, expert_offsets, sparse_rows,
                                                  slot_src);
        prof_end(stream, kKMapSmall);
        return hipGetLastError();
    }
    const SparseMapPlan pl = sparse_map_plan(N, E);
    int32_t *cnt = reinterpret_cast<int32_t *>(workspace);
    int32_t *totals = cnt + (size_t)E * pl.nsub;
    const size_t hist_lds = chunk_hist_lds_bytes(E), assign_lds = chunk_assign_lds_bytes(E, pl.rg);
    prof_begin(stream, kKMapHist);
    smap_chunk_hist_kernel<kHistUnroll><<<pl.nsub, kHistThreads, hist_lds, stream>>>(ids, N, E, pl.L, pl.nsub, cnt);
    prof_end(stream, kKMapHist);
    prof_begin(stream, kKMapRowscan);
    smap_rowscan_kernel<<<E, 256, 0, stream>>>(cnt, pl.nsub, totals);
    prof_end(stream, kKMapRowscan);
    prof_begin(stream, kKMapAssign);
    if (pl.rg == 8)
        smap_chunk_assign_kernel<8><<<pl.nsub, kAssignThreads, assign_lds, stream>>>(
            ids, N, E, pl.L, pl.nsub, cnt, totals, expert_counts, expert_offsets, sparse_rows, slot_src);
    else
        smap_chunk_assign_kernel<1><<<pl.nsub, kAssignThreads, assign_lds, stream>>>(
            ids, N, E, pl.L, pl.nsub, cnt, totals, expert_counts, expert_offsets, sparse_rows, slot_src);
    prof_end(stream, kKMapAssign);
    return hipGetLastError();
}

}  // namespace smoe
