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
// Layout of the work: the routes are cut into sub-chunks of L routes, one
// per wavefront, processed 64 at a time. Within a group of 64, a lane finds
// the lanes holding the same expert with one ballot per id bit (match-any),
// so its rank among them is a popcount and the group's count per expert is
// known to the lowest such lane, which updates a per-wave LDS counter. No
// global atomics are used anywhere.
//   pass 1 (hist):    per sub-chunk counts  -> cnt[e][sub]       (workspace)
//   pass 2 (rowscan): per expert, exclusive scan over sub-chunks, total
//   pass 3 (assign):  offsets from the totals, then rank -> slot
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"
#include "profile.hpp"

namespace smoe {

constexpr int kMapWaves = 4;
constexpr int kMaxExperts = 1024;
constexpr int kMapUnroll = 4;  // groups of 64 routes whose ids are loaded together

__device__ __forceinline__ unsigned long long match_any(int key, int nbits) {
    unsigned long long m = __ballot(1);
    for (int b = 0; b < nbits; ++b) {
        const int bit = (key >> b) & 1;
        const unsigned long long bb = __ballot(bit);
        m &= bit ? bb : ~bb;
    }
    return m;
}

__global__ __launch_bounds__(256) void smap_hist_kernel(const int32_t *__restrict__ ids, int N, int E, int nbits,
                                                         int L, int nsub, int32_t *__restrict__ cnt) {
    __shared__ int32_t s_cnt[kMapWaves * kMaxExperts];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int sub = blockIdx.x * kMapWaves + w;
    int32_t *my = s_cnt + w * E;
    for (int e = lane; e < E; e += 64) my[e] = 0;
    __syncthreads();
    if (sub < nsub) {
        const int base = sub * L;
        for (int g0 = 0; g0 < L; g0 += 64 * kMapUnroll) {
            int ev[kMapUnroll];  // the ids of kMapUnroll groups are loaded before any is used
#pragma unroll
            for (int u = 0; u < kMapUnroll; ++u) {
                const int f = base + g0 + 64 * u + lane;
                ev[u] = f < N ? ids[f] : E;  // E = sentinel: lanes past the end, ids outside [0, E)
            }
#pragma unroll
            for (int u = 0; u < kMapUnroll; ++u) {
                int e = ev[u];
                if ((unsigned)e >= (unsigned)E) e = E;
                const unsigned long long m = match_any(e, nbits);
                const int leader = __ffsll(m) - 1;
                if (lane == leader && e < E) my[e] += __popcll(m);
            }
        }
        for (int e = lane; e < E; e += 64) cnt[(size_t)e * nsub + sub] = my[e];
    }
}

// Block-wide exclusive scan of one int per thread (256 threads); returns the
// exclusive prefix and writes the block total to *total.
__device__ int block_exscan_256(int v, int *s_tmp, int *total) {
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
    for (int i = 0; i < 4; ++i) {
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
        int pre = block_exscan_256(s, s_tmp, &tot) + running;
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

__global__ __launch_bounds__(256) void smap_assign_kernel(const int32_t *__restrict__ ids, int N, int E, int nbits,
                                                           int L, int nsub, const int32_t *__restrict__ cnt,
                                                           const int32_t *__restrict__ totals,
                                                           int32_t *__restrict__ expert_counts,
                                                           int32_t *__restrict__ expert_offsets,
                                                           int32_t *__restrict__ sparse_rows,
                                                           int32_t *__restrict__ slot_src) {
    __shared__ int32_t s_off[kMaxExperts];
    __shared__ int32_t s_ctr[kMapWaves * kMaxExperts];
    __shared__ int s_tmp[4];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;

    // offsets = exclusive scan of the per-expert totals (E <= 1024: 4 per thread)
    {
        int v[4], s = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = threadIdx.x * 4 + i;
            v[i] = e < E ? totals[e] : 0;
            s += v[i];
        }
        int tot;
        int pre = block_exscan_256(s, s_tmp, &tot);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = threadIdx.x * 4 + i;
            if (e < E) {
                s_off[e] = pre;
                if (blockIdx.x == 0) {
                    expert_counts[e] = v[i];
                    expert_offsets[e] = pre;
                }
            }
            pre += v[i];
        }
        if (blockIdx.x == 0 && threadIdx.x == 0) expert_offsets[E] = tot;
    }
    __syncthreads();

    const int sub = blockIdx.x * kMapWaves + w;
    if (sub >= nsub) return;
    int32_t *my = s_ctr + w * E;
    for (int e = lane; e < E; e += 64) my[e] = s_off[e] + cnt[(size_t)e * nsub + sub];
    const int base = sub * L;
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int g0 = 0; g0 < L; g0 += 64 * kMapUnroll) {
        int ev[kMapUnroll];
#pragma unroll
        for (int u = 0; u < kMapUnroll; ++u) {
            const int f = base + g0 + 64 * u + lane;
            ev[u] = f < N ? ids[f] : E;
        }
#pragma unroll
        for (int u = 0; u < kMapUnroll; ++u) {
            const int f = base + g0 + 64 * u + lane;
            int e = ev[u];
            if ((unsigned)e >= (unsigned)E) e = E;
            const unsigned long long m = match_any(e, nbits);
            const int leader = __ffsll(m) - 1;
            int b = (lane == leader && e < E) ? my[e] : 0;
            b = __shfl(b, leader);
            if (e < E) {
                const int slot = b + __popcll(m & lt);
                sparse_rows[f] = slot;
                slot_src[slot] = f;
            } else if (f < N) {
                sparse_rows[f] = -1;  // id outside [0, E): the route gets no slot
            }
            if (lane == leader && e < E) my[e] = b + __popcll(m);
        }
    }
}

// The whole map in one workgroup of 1024 threads, for maps of at most
// kSmallMapRoutes routes (decode-sized batches), where the three launches
// of the general path cost more than the work. Wave w takes the contiguous
// chunk [w L, (w + 1) L) of routes, so a route's rank among the routes of its
// expert is: earlier waves' counts of that expert, then earlier groups of 64
// in its own wave, then lower lanes of its own group -- the same stable slot
// as the general path.
constexpr int kSmallMapRoutes = 8192;
constexpr int kSmallMapWaves = 16;

__global__ __launch_bounds__(1024) void smap_small_kernel(const int32_t *__restrict__ ids, int N, int E, int nbits,
                                                          int L, int32_t *__restrict__ expert_counts,
                                                          int32_t *__restrict__ expert_offsets,
                                                          int32_t *__restrict__ sparse_rows,
                                                          int32_t *__restrict__ slot_src) {
    __shared__ int32_t s_cnt[kSmallMapWaves * kMaxExperts];  // [wave][expert]: count, then base
    __shared__ int s_tmp[kSmallMapWaves];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int32_t *my = s_cnt + w * E;
    for (int e = lane; e < E; e += 64) my[e] = 0;
    const int base = w * L;
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    // pass 1: per-wave counts (only a group's lowest lane of an expert writes)
    for (int g0 = 0; g0 < L; g0 += 64 * kMapUnroll) {
        int ev[kMapUnroll];
#pragma unroll
        for (int u = 0; u < kMapUnroll; ++u) {
            const int f = base + g0 + 64 * u + lane;
            ev[u] = f < N ? ids[f] : E;
        }
#pragma unroll
        for (int u = 0; u < kMapUnroll; ++u) {
            int e = ev[u];
            if ((unsigned)e >= (unsigned)E) e = E;
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
    for (int g0 = 0; g0 < L; g0 += 64 * kMapUnroll) {
        int ev[kMapUnroll];
#pragma unroll
        for (int u = 0; u < kMapUnroll; ++u) {
            const int f = base + g0 + 64 * u + lane;
            ev[u] = f < N ? ids[f] : E;
        }
#pragma unroll
        for (int u = 0; u < kMapUnroll; ++u) {
            const int f = base + g0 + 64 * u + lane;
            int ex = ev[u];
            if ((unsigned)ex >= (unsigned)E) ex = E;
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

__global__ void smap_empty_kernel(int E, int32_t *expert_counts, int32_t *expert_offsets) {
    for (int e = threadIdx.x; e <= E; e += blockDim.x) {
        if (e < E) expert_counts[e] = 0;
        expert_offsets[e] = 0;
    }
}

SparseMapPlan sparse_map_plan(int64_t N, int E) {
    SparseMapPlan pl;
    // sub-chunks of L = 256 * 2^j routes (a multiple of 64 * kMapUnroll); up
    // to max(2048, 2^20 / E) of them, so large maps keep many waves busy (a
    // wave's loop over its L routes is latency-bound) while the per-sub-chunk
    // count matrix stays within 4 MB
    const int64_t max_sub = std::max<int64_t>(2048, ((int64_t)1 << 20) / std::max(E, 1));
    int64_t L = 256;
    while ((N + L - 1) / L > max_sub) L *= 2;
    pl.L = (int)L;
    pl.nsub = (int)((N + L - 1) / L);
    pl.nbits = 32 - __builtin_clz((unsigned)E);  // bits to hold 0..E (E is the sentinel)
    pl.ws_bytes = (size_t)E * (size_t)pl.nsub * sizeof(int32_t) + (size_t)E * sizeof(int32_t);
    return pl;
}

hipError_t launch_sparse_map(const int32_t *ids, int N, int E, int32_t *expert_counts, int32_t *expert_offsets,
                             int32_t *sparse_rows, int32_t *slot_src, void *workspace, hipStream_t stream) {
    if (N == 0) {
        prof_begin(stream, kKMapEmpty);
        smap_empty_kernel<<<1, 256, 0, stream>>>(E, expert_counts, expert_offsets);
        prof_end(stream, kKMapEmpty);
        return hipGetLastError();
    }
    const SparseMapPlan pl = sparse_map_plan(N, E);
    if (N <= kSmallMapRoutes) {
        // chunks of whole 64 * kMapUnroll groups, one per wave
        constexpr int G = 64 * kMapUnroll;
        const int L = ((N + kSmallMapWaves - 1) / kSmallMapWaves + G - 1) / G * G;
        prof_begin(stream, kKMapSmall);
        smap_small_kernel<<<1, 1024, 0, stream>>>(ids, N, E, pl.nbits, L, expert_counts, expert_offsets, sparse_rows,
                                                  slot_src);
        prof_end(stream, kKMapSmall);
        return hipGetLastError();
    }
    int32_t *cnt = reinterpret_cast<int32_t *>(workspace);
    int32_t *totals = cnt + (size_t)E * pl.nsub;
    const int blocks = (pl.nsub + kMapWaves - 1) / kMapWaves;
    prof_begin(stream, kKMapHist);
    smap_hist_kernel<<<blocks, 256, 0, stream>>>(ids, N, E, pl.nbits, pl.L, pl.nsub, cnt);
    prof_end(stream, kKMapHist);
    prof_begin(stream, kKMapRowscan);
    smap_rowscan_kernel<<<E, 256, 0, stream>>>(cnt, pl.nsub, totals);
    prof_end(stream, kKMapRowscan);
    prof_begin(stream, kKMapAssign);
    smap_assign_kernel<<<blocks, 256, 0, stream>>>(ids, N, E, pl.nbits, pl.L, pl.nsub, cnt, totals, expert_counts,
                                                   expert_offsets, sparse_rows, slot_src);
    prof_end(stream, kKMapAssign);
    return hipGetLastError();
}

}  // namespace smoe
