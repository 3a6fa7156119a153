// Shared definitions of the grouped, gathered bf16 GEMMs of the expert FFN
// and the router (kernels in gemm_pp.hpp).
//
// A GEMM tile computes, for the rows r of one expert's tile,
//   C[r, n] = sum_k A[row(r), k] * B_e[k, n]
// where rows r are slots [row_begin, row_end) of that expert (from a tile
// table built from the scanned expert offsets) and row(r) is either the slot
// itself (contiguous A) or the token of the slot (gathered A: token rows of
// X read in place, never copied).
//
// The epilogues (MODE):
//   kGateUp   two B matrices (W1, W3) share every A tile; the tile writes
//             h = bf16(SiLU(A W1) * (A W3)) in slot order (fused gate+up).
//   kDown     one B matrix (W2); the tile scales each row by its route's
//             router weight and atomically adds into the fp32 token
//             accumulator (scatter-add combine).
//   kDownRows one B matrix (W2); the tile scales each row by its route's
//             router weight and stores it, fp32, to row f of a per-route
//             buffer (f = the slot's flat route index, so the k rows of a
//             token are adjacent); a combine pass sums them per token.
//   kLogits   one B matrix (W_gate), no experts; fp32 store (router logits).
//   kLinBf16  one B matrix; the tile scales each row by its route's gate
//             (1 when gate is NULL) and stores it, bf16, to row r of C in
//             slot order (ParallelLinear with grouped output).
//   kGateUpSave  as kGateUp (gathered A, W1 and W3), for the backward's
//             recomputation: stores a = bf16(A W1) and b = bf16(A W3) side by
//             side in C ([rows, 2N]: a in columns [0, N), b in [N, 2N)) and
//             h = bf16(SiLU(a) * b) from the fp32 sums in C2 ([rows, N]).
//   kSwigluBwd  one B matrix (W2 used transposed: kFlagBT), gathered A (the
//             output gradient rows of the tokens): c = dout[t] W2[e]^T; with
//             the route's gate g and the saved a, b of C it writes, in place,
//             da = g c b SiLU'(a) over a and db = g c SiLU(a) over b, and adds
//             <h, c> over the tile's columns into part[(nt * 4 + wn) * M + f]
//             (the router-gate gradient, summed later in a fixed order).
// kDownRows also treats a NULL gate as 1.
//
// Weights are [E, K, N] with N contiguous; with kFlagBT they are [E, N, K]
// with K contiguous (a weight [E, D_in, D_out] used transposed: the product
// with W^T that the input gradient needs). gather_a != 0 makes the kDownRows
// and kLinBf16 tiles read token rows of A in place (row = slot_src[r] / topk),
// as kGateUp always does. kFlagKSplit (with kFlagBT) splits K in two halves:
// k < K/2 reads B0 and k >= K/2 reads B1, each [E, N, K/2] (the input
// gradient of the SwiGLU experts: [da | db] times [W1 ; W3]^T).
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace smoe {

enum GemmMode { kGateUp = 0, kDown = 1, kLogits = 2, kDownRows = 3, kLinBf16 = 4, kGateUpSave = 5, kSwigluBwd = 6 };
// kFlagSplitDma: the two wave groups share the DMA issue (see pp_dma_split)
enum GemmFlags { kFlagBT = 1, kFlagKSplit = 2, kFlagSplitDma = 4 };

struct GemmParams {
    const uint16_t *A;        // X [S, K] (kGateUp, kLogits) or h [S*k, K] (kDown, kDownRows)
    const uint16_t *B0;       // W1 / W2 / W_gate: [E, K, N]
    const uint16_t *B1;       // W3 (kGateUp only)
    const int32_t *slot_src;  // [S*k] slot -> flat route index
    const float *gate;        // [S*k] router weights (kDown, kDownRows, kLinBf16; may be NULL except kDown)
    const int4 *tiles;        // [n_mtiles] (expert, row_begin, row_end, -) ; expert < 0 = empty
    const uint32_t *order;    // [n_mtiles * n_ntiles] block order: mt | nt << kOrderMtBits, valid blocks first
    const int *valid_mtiles;  // device count of non-empty M tiles
    int *queue;               // per-XCD tile claim counters, kQueueStride ints apart (zeroed by the
                              // tile table), for the persistent kernel's dynamic form
    void *C;                  // h bf16 [S*k, N] / acc fp32 [S, N] / y fp32 [S*k, N] / logits fp32 [S, N]
                              // / a|b bf16 [S*k, 2N] (kGateUpSave, kSwigluBwd)
    void *C2;                 // h bf16 [S*k, N] (kGateUpSave)
    float *part;              // router-gate partial sums (kSwigluBwd)
    int M;                    // rows (kLogits: S); A has M rows unless gathered
    int A_rows;               // rows of A (gathered: S)
    int N;                    // output columns
    int K;                    // reduction length (multiple of 64)
    int topk;                 // k (token = flat route index / k)
    int gather_a;             // kDownRows / kLinBf16: A rows are token rows read by index
    int n_mtiles;             // M tiles (upper bound over all experts)
    int n_ntiles;             // N tiles
};

}  // namespace smoe
