// Grouped, gathered bf16 GEMM tile kernel for gfx950 (MFMA 16x16x32).
//
// One workgroup (4 waves) computes a BM x BN output tile of one expert:
//   C[r, n] = sum_k A[row(r), k] * B_e[k, n]
// where rows r are slots [row_begin, row_end) of that expert (from a tile
// table built from the scanned expert offsets) and row(r) is either the slot
// itself (contiguous A) or the token of the slot (gathered A: token rows of
// X read in place, never copied).
//
// Four epilogues:
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
//
// Weights are [E, K, N] with N contiguous. MFMA wants K-contiguous operands,
// so each thread loads an 8x8 block of B (8 rows of 16 B), transposes it in
// registers and writes 8 K-contiguous 16 B chunks to LDS. Both A and B live
// in LDS as rows of 64 K values (BK = 64) with an XOR chunk swizzle, double
// buffered: global loads for step k+1 are in flight while step k computes.
// All global reads are buffer loads: rows past the end of a buffer read as
// zero, and rows or columns outside the tile only feed outputs that are
// never stored, so the loads need no per-element masking.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace smoe {

enum GemmMode { kGateUp = 0, kDown = 1, kLogits = 2, kDownRows = 3 };

struct GemmParams {
    const uint16_t *A;        // X [S, K] (kGateUp, kLogits) or h [S*k, K] (kDown, kDownRows)
    const uint16_t *B0;       // W1 / W2 / W_gate: [E, K, N]
    const uint16_t *B1;       // W3 (kGateUp only)
    const int32_t *slot_src;  // [S*k] slot -> flat route index
    const float *gate;        // [S*k] router weights (kDown, kDownRows)
    const int4 *tiles;        // [n_mtiles] (expert, row_begin, row_end, -) ; expert < 0 = empty
    const uint32_t *order;    // [n_mtiles * n_ntiles] logical block -> mt | nt << kOrderMtBits (nullptr: grouped)
    const int *valid_mtiles;  // device count of non-empty M tiles (stream-K kernels)
    void *C;                  // h bf16 [S*k, N] / acc fp32 [S, N] / y fp32 [S*k, N] / logits fp32 [S, N]
    int M;                    // rows (kLogits: S); A has M rows unless gathered
    int A_rows;               // rows of A (gathered: S)
    int N;                    // output columns
    int K;                    // reduction length (multiple of 64)
    int topk;                 // k (token = flat route index / k)
    int n_mtiles;
    int n_ntiles;
    int group_m;              // M tiles per tile group (L2 reuse order)
};

// Block -> (M tile, N tile). Logical ids are XCD-contiguous (xcd_remap). With
// an order table (built next to the tile table) the logical order is
// expert-major, then N tile, then the expert's M tiles: the blocks that share
// one expert's weight panel run back to back on one XCD. Without it, M tiles
// are taken in groups of group_m per N tile. Returns false for an empty slot.
__device__ __forceinline__ bool decode_tile(const GemmParams &p, int &mt, int &nt) {
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    if (p.order != nullptr) {
        const uint32_t v = p.order[L];
        mt = (int)(v & kOrderMtMask);
        nt = (int)(v >> kOrderMtBits);
        return mt < p.n_mtiles;
    }
    const int per_group = p.group_m * p.n_ntiles;
    const int grp = L / per_group;
    const int within = L - grp * per_group;
    const int m_first = grp * p.group_m;
    const int gm = min(p.group_m, p.n_mtiles - m_first);
    nt = within / gm;
    mt = m_first + (within - nt * gm);
    return true;
}

template <int BM, int BN, int WM, int WN, int MODE>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(const GemmParams p) {
    constexpr int NB = (MODE == kGateUp) ? 2 : 1;
    constexpr int BK = 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int MT = WTM / 16, NT = WTN / 16;
    static_assert(WM * WN == 4, "4 waves per workgroup");
    static_assert(MT >= 1 && NT >= 1 && WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be 16-aligned");
    constexpr int A_BYTES = BM * BK * 2;
    constexpr int B_BYTES = BN * BK * 2;
    constexpr int STAGE = A_BYTES + NB * B_BYTES;
    constexpr int A_CHUNKS = BM * 8;             // 16 B chunks per A stage
    constexpr int A_ITERS = (A_CHUNKS + 255) / 256;
    constexpr int B_BLOCKS = NB * BN;            // 8x8 blocks per B stage (BK/8 * BN/8 * NB)
    constexpr int B_ITERS = (B_BLOCKS + 255) / 256;

    __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    int mt, nt;
    if (!decode_tile(p, mt, nt)) return;

    int expert, row0, row1;
    if (MODE == kLogits) {
        expert = 0;
        row0 = mt * BM;
        row1 = min(p.M, row0 + BM);
    } else {
        const int4 t = p.tiles[mt];
        expert = t.x;
        row0 = t.y;
        row1 = t.z;
    }
    if (expert < 0 || row0 >= row1) return;
    const int n0 = nt * BN;
    const int N = p.N, K = p.K;
    const uint32_t ldb = (uint32_t)N * 2u;  // bytes per B row

    // ---- A: buffer over the rows this tile may touch ----
    // gathered: the whole X; contiguous: rows [row0, row0 + BM) of A
    const uint16_t *a_base = (MODE == kGateUp) ? p.A : p.A + (size_t)row0 * K;
    const uint32_t a_bytes = (MODE == kGateUp) ? (uint32_t)((size_t)p.A_rows * K * 2)
                                               : (uint32_t)((size_t)(row1 - row0) * K * 2);
    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(a_base, a_bytes);
    uint32_t a_voff[A_ITERS];
    int a_lds[A_ITERS];
#pragma unroll
    for (int i = 0; i < A_ITERS; ++i) {
        const int idx = tid + 256 * i;
        const int r = (idx >> 3) < BM ? (idx >> 3) : 0;
        const int c = idx & 7;
        int slot = row0 + r;
        if (slot >= row1) slot = row1 - 1;  // rows past the expert's end load a valid row, never stored
        const uint32_t arow = (MODE == kGateUp) ? (uint32_t)(p.slot_src[slot] / p.topk) : (uint32_t)(slot - row0);
        a_voff[i] = arow * (uint32_t)K * 2u + (uint32_t)c * 16u;
        a_lds[i] = lds_off(r, c);
    }
    // ---- B: thread -> 8x8 block (k rows kb*8.., n cols nb*8..) of one matrix ----
    const size_t b_off = (size_t)expert * (size_t)K * (size_t)N;
    const uint32_t b_bytes = (uint32_t)((size_t)K * N * 2);
    const __amdgpu_buffer_rsrc_t b_rsrc0 = make_rsrc(p.B0 + b_off, b_bytes);
    const __amdgpu_buffer_rsrc_t b_rsrc1 = make_rsrc((NB == 2 ? p.B1 : p.B0) + b_off, b_bytes);
    static_assert(BN % 64 == 0, "a wave's 64 B blocks must come from one matrix");
    uint32_t b_voff[B_ITERS];
    int b_lds_row[B_ITERS], b_kb[B_ITERS];
    __amdgpu_buffer_rsrc_t b_rsrc[B_ITERS];
#pragma unroll
    for (int i = 0; i < B_ITERS; ++i) {
        const int blk = (tid + 256 * i) % B_BLOCKS;
        const int kb = blk & 7, nb = blk >> 3;
        // which matrix (W1 or W3) is uniform across the wave: make that explicit
        const int which = __builtin_amdgcn_readfirstlane(nb / (BN / 8));
        const int ncol = (nb % (BN / 8)) * 8;
        const int gcol = min(n0 + ncol, N - 8);  // columns past N only feed unstored outputs
        b_rsrc[i] = (NB == 2 && which == 1) ? b_rsrc1 : b_rsrc0;
        b_voff[i] = (uint32_t)(kb * 8) * ldb + (uint32_t)gcol * 2u;
        b_lds_row[i] = which * BN + ncol;
        b_kb[i] = kb;
    }

    uint4 ra[A_ITERS];
    uint4 rb[B_ITERS][8];
    constexpr bool A_FULL = (A_CHUNKS % 256) == 0;
    constexpr bool B_FULL = (B_BLOCKS % 256) == 0;

#define SMOE_LOAD_GLOBAL(KT)                                                                      \
    {                                                                                            \
        const uint32_t a_soff = (uint32_t)(KT) * (BK * 2);                                       \
        _Pragma("unroll") for (int i = 0; i < A_ITERS; ++i) if (A_FULL || tid + 256 * i < A_CHUNKS) \
            ra[i] = buf_load16(a_rsrc, a_voff[i], a_soff);                                       \
        const uint32_t b_soff = (uint32_t)(KT) * BK * ldb;                                       \
        _Pragma("unroll") for (int i = 0; i < B_ITERS; ++i) if (B_FULL || tid + 256 * i < B_BLOCKS) { \
            _Pragma("unroll") for (int r = 0; r < 8; ++r)                                        \
                rb[i][r] = buf_load16(b_rsrc[i], b_voff[i] + r * ldb, b_soff); \
        }                                                                                        \
    }
#define SMOE_STORE_LDS(STG)                                                                       \
    {                                                                                            \
        char *sa = smem + (STG) * STAGE;                                                         \
        char *sb = sa + A_BYTES;                                                                 \
        _Pragma("unroll") for (int i = 0; i < A_ITERS; ++i) if (A_FULL || tid + 256 * i < A_CHUNKS) \
            *reinterpret_cast<uint4 *>(sa + a_lds[i]) = ra[i];                                   \
        _Pragma("unroll") for (int i = 0; i < B_ITERS; ++i) if (B_FULL || tid + 256 * i < B_BLOCKS) { \
            uint4 t[8];                                                                          \
            transpose8x8(rb[i], t);                                                              \
            _Pragma("unroll") for (int c = 0; c < 8; ++c)                                        \
                *reinterpret_cast<uint4 *>(sb + lds_off(b_lds_row[i] + c, b_kb[i])) = t[c];      \
        }                                                                                        \
    }

    f32x4 acc[NB][MT][NT];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j) acc[b][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int KT = K / BK;
    SMOE_LOAD_GLOBAL(0);
    SMOE_STORE_LDS(0);
    __syncthreads();

    const int frag_row = lane & 15;
    const int frag_chunk = lane >> 4;
    for (int kt = 0; kt < KT; ++kt) {
        const int stage = kt & 1;
        const bool more = kt + 1 < KT;
        if (more) SMOE_LOAD_GLOBAL(kt + 1);
        const char *sa = smem + stage * STAGE;
        const char *sb = sa + A_BYTES;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            uint4 af[MT];
            uint4 bfr[NB][NT];
#pragma unroll
            for (int i = 0; i < MT; ++i)
                af[i] = *reinterpret_cast<const uint4 *>(sa + lds_off(wm * WTM + i * 16 + frag_row, kk * 4 + frag_chunk));
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    bfr[b][j] = *reinterpret_cast<const uint4 *>(
                        sb + b * B_BYTES + lds_off(wn * WTN + j * 16 + frag_row, kk * 4 + frag_chunk));
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int i = 0; i < MT; ++i)
#pragma unroll
                    for (int j = 0; j < NT; ++j) acc[b][i][j] = mfma_16x16x32(af[i], bfr[b][j], acc[b][i][j]);
        }
        if (more) SMOE_STORE_LDS(stage ^ 1);
        __syncthreads();
    }
#undef SMOE_LOAD_GLOBAL
#undef SMOE_STORE_LDS

    // ---- epilogue ----
    const int col_in_tile = lane & 15;
    const int row_grp = (lane >> 4) * 4;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = wm * WTM + i * 16 + row_grp + r;
            const int slot = row0 + row;
            if (slot >= row1) continue;
            if (MODE == kGateUp) {
                uint16_t *h = reinterpret_cast<uint16_t *>(p.C) + (size_t)slot * N + n0;
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const int col = wn * WTN + j * 16 + col_in_tile;
                    if (n0 + col < N) {
                        const float g = acc[0][i][j][r], u = acc[1][i][j][r];
                        const float s = g / (1.0f + __expf(-g));
                        h[col] = f32_to_bf16_bits(s * u);
                    }
                }
            } else if (MODE == kDown) {
                const int f = p.slot_src[slot];
                const int tok = f / p.topk;
                const float w = p.gate[f];
                float *accp = reinterpret_cast<float *>(p.C) + (size_t)tok * N + n0;
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const int col = wn * WTN + j * 16 + col_in_tile;
                    if (n0 + col < N) atomicAdd(accp + col, w * acc[0][i][j][r]);
                }
            } else if (MODE == kDownRows) {
                const int f = p.slot_src[slot];
                const float w = p.gate[f];
                float *yp = reinterpret_cast<float *>(p.C) + (size_t)f * N + n0;
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const int col = wn * WTN + j * 16 + col_in_tile;
                    if (n0 + col < N) yp[col] = w * acc[0][i][j][r];
                }
            } else {
                float *out = reinterpret_cast<float *>(p.C) + (size_t)slot * N + n0;
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const int col = wn * WTN + j * 16 + col_in_tile;
                    if (n0 + col < N) out[col] = acc[0][i][j][r];
                }
            }
        }
    }
}

}  // namespace smoe
