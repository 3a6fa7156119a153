// Router: H(X) = Softmax(TopK(X W_gate, k)) (ScatterMoE Guide, section
// "1. The Dynamic Routing Imbalance Dilemma", equation H(X)).
//
//   logits   fp32 [S, E] = x W_gate on bf16 MFMA (the grouped GEMM kernel in
//            its plain-rows mode), kept in the caller's workspace
//   top-k    one wavefront per token: k rounds of a wave-wide arg-max
//            (larger logit wins, equal logits -> lower expert id), then the
//            softmax of the k chosen logits in fp32 with the maximum
//            subtracted.
#include <math.h>

#include "gemm.hpp"
#include "launch.hpp"
#include "profile.hpp"

namespace smoe {

constexpr int kRouteMaxE = 256;
constexpr int kRouteMaxK = 16;

__global__ __launch_bounds__(256) void topk_softmax_kernel(const float *__restrict__ logits, int S, int E, int k,
                                                           int32_t *__restrict__ ids, float *__restrict__ weights) {
    const int lane = threadIdx.x & 63;
    const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (s >= S) return;
    const float *l = logits + (size_t)s * E;
    float v[kRouteMaxE / 64];
    unsigned taken = 0;
#pragma unroll
    for (int i = 0; i < kRouteMaxE / 64; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? l[e] : -INFINITY;
        if (e >= E) taken |= 1u << i;
    }
    float top[kRouteMaxK];
    int topi[kRouteMaxK];
#pragma unroll
    for (int j = 0; j < kRouteMaxK; ++j) {
        top[j] = -INFINITY;
        topi[j] = 0;
        if (j < k) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
#pragma unroll
            for (int i = 0; i < kRouteMaxE / 64; ++i) {
                const int e = lane + 64 * i;
                if (!((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && e < bi))) {
                    bv = v[i];
                    bi = e;
                }
            }
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) {
                const float ov = __shfl_xor(bv, d);
                const int oi = __shfl_xor(bi, d);
                if (ov > bv || (ov == bv && oi < bi)) {
                    bv = ov;
                    bi = oi;
                }
            }
            if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
            top[j] = bv;
            topi[j] = bi;
        }
    }
    const float m = top[0];
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < kRouteMaxK; ++j)
        if (j < k) z += expf(top[j] - m);
#pragma unroll
    for (int j = 0; j < kRouteMaxK; ++j) {
        if (j < k && lane == j) {
            ids[(size_t)s * k + j] = topi[j];
            weights[(size_t)s * k + j] = expf(top[j] - m) / z;
        }
    }
}

size_t route_ws_bytes(int64_t S, int64_t E) { return align_up((size_t)S * (size_t)E * sizeof(float)); }

template <int BM, int BN, int WM, int WN>
static void launch_logits(const uint16_t *x, const uint16_t *w_gate, int S, int D, int E, float *logits,
                          hipStream_t stream) {
    GemmParams p{};
    p.A = x;
    p.B0 = w_gate;
    p.C = logits;
    p.M = S;
    p.A_rows = S;
    p.N = E;
    p.K = D;
    p.topk = 1;
    p.n_mtiles = (S + BM - 1) / BM;
    p.n_ntiles = (E + BN - 1) / BN;
    p.group_m = 8;
    prof_begin(stream, kKRouteLogits);
    grouped_gemm_kernel<BM, BN, WM, WN, kLogits><<<p.n_mtiles * p.n_ntiles, 256, 0, stream>>>(p);
    prof_end(stream, kKRouteLogits);
}

hipError_t launch_route(const uint16_t *x, const uint16_t *w_gate, int S, int D, int E, int k, int32_t *topk_ids,
                        float *topk_weights, void *workspace, hipStream_t stream) {
    float *logits = reinterpret_cast<float *>(workspace);
    if (E <= 64) launch_logits<16, 64, 1, 4>(x, w_gate, S, D, E, logits, stream);
    else launch_logits<32, 128, 2, 2>(x, w_gate, S, D, E, logits, stream);
    prof_begin(stream, kKRouteTopk);
    topk_softmax_kernel<<<(S + 3) / 4, 256, 0, stream>>>(logits, S, E, k, topk_ids, topk_weights);
    prof_end(stream, kKRouteTopk);
    return hipGetLastError();
}

}  // namespace smoe
