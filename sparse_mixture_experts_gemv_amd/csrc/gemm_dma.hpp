// Grouped, gathered bf16 GEMM for gfx950 with direct global->LDS loads.
//
// Same contract as grouped_gemm_kernel (gemm.hpp): one workgroup of 4 waves
// computes a BM x BN tile of one expert (or of the router logits), with the
// fused SwiGLU gate+up, the router-weighted scatter-add, or a plain fp32
// store as epilogue. What differs is how operands reach the matrix cores:
//
//  * Both operands move HBM -> LDS with buffer_load ... lds (no VGPR
//    staging). Each wave instruction fills 1 KB of LDS: 8 rows of the A tile
//    (64 bf16 of K each) or 1024 / (2 BN) rows of a B tile (BN bf16 of N
//    each). Which global 16-byte piece a lane fetches is chosen so that the
//    LDS image comes out swizzled.
//  * A stays K-contiguous: a lane's MFMA A operand (8 consecutive K of one
//    row) is one ds_read_b128.
//  * B stays N-contiguous, exactly as the weights are stored; the MFMA B
//    operand (8 consecutive K of one column) is assembled by two
//    ds_read_b64_tr_b16 transposing reads. Within each 16-lane group that
//    instruction hands lane i element (i % 4) of the 8-byte piece addressed
//    by lane 4 r + i / 4, for r = 0..3. So lane q of group g addresses row
//    k = 8 g + 4 h + q / 4 and columns 4 (q % 4) .. + 3 of its 16-column
//    fragment, and reads h = 0, 1 give K = 8 g .. 8 g + 7 in order, the same
//    K order as the A operand.
//  * Pipeline (two LDS stages): wait for this step's tile, barrier, read
//    every MFMA fragment of the step into registers, issue the next step's
//    loads into the other stage, then run the step's MFMAs while those
//    loads are in flight.
#pragma once

#include "gemm.hpp"

namespace smoe {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char *lds_wave_base, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds_wave_base, 16, (int)voff, (int)soff, 0, 0);
}

__device__ __forceinline__ uint2 lds_read_tr(const char *p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(p));
    return __builtin_bit_cast(uint2, v);
}

// A tile: rows of 64 bf16 (8 chunks of 16 B); chunk XOR-swizzled by row.
__device__ __forceinline__ int a_swz(int row) { return row & 7; }
// B tile: rows of BN bf16 cut into 32-byte segments (16 columns); segment
// XOR-swizzled by k so the 4 (or 8) rows one transposing read touches land
// in different banks.
template <int BN>
__device__ __forceinline__ int b_swz(int k) {
    constexpr int SEGS = BN / 16;
    return (SEGS >= 8) ? ((k & 3) | (((k >> 3) & 1) << 2)) : (k & (SEGS - 1));
}

template <int BM, int BN, int WM, int WN, int MODE>
__global__ __launch_bounds__(256) void grouped_gemm_dma_kernel(const GemmParams p) {
    constexpr int NB = (MODE == kGateUp) ? 2 : 1;
    constexpr int BK = 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int MT = WTM / 16, NT = WTN / 16;
    static_assert(WM * WN == 4, "4 waves per workgroup");
    static_assert(MT >= 1 && NT >= 1 && WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be 16-aligned");
    static_assert(BN % 64 == 0 && BN <= 512, "B rows are 128..1024 bytes");
    constexpr int A_BYTES = BM * BK * 2;
    constexpr int B_ROW = BN * 2;                  // bytes per B row in LDS
    constexpr int B_BYTES = BK * B_ROW;
    constexpr int STAGE = A_BYTES + NB * B_BYTES;
    constexpr int A_INSTR = A_BYTES / 1024;        // wave instructions per stage
    constexpr int B_INSTR = NB * B_BYTES / 1024;
    constexpr int B_INSTR_PER_MAT = B_BYTES / 1024;
    constexpr int B_ROWS_PER_INSTR = 1024 / B_ROW;
    constexpr int B_LANES_PER_ROW = B_ROW / 16;
    static_assert(A_BYTES % 1024 == 0, "BM must be a multiple of 8");
    constexpr int A_PER_WAVE = (A_INSTR + 3) / 4;
    constexpr int B_PER_WAVE = (B_INSTR + 3) / 4;

    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps DMA targets in SGPRs
    const int wm = wave / WN, wn = wave % WN;

    // ---- tile decode (same order as grouped_gemm_kernel) ----
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int per_group = p.group_m * p.n_ntiles;
    const int grp = L / per_group;
    const int within = L - grp * per_group;
    const int m_first = grp * p.group_m;
    const int gm = min(p.group_m, p.n_mtiles - m_first);
    const int nt = within / gm;
    const int mt = m_first + (within - nt * gm);

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
    const uint32_t ldb = (uint32_t)N * 2u;

    // ---- A loads: wave instruction j fills rows 8 j .. 8 j + 7 ----
    const uint16_t *a_base = (MODE == kGateUp) ? p.A : p.A + (size_t)row0 * K;
    const uint32_t a_bytes = (MODE == kGateUp) ? (uint32_t)((size_t)p.A_rows * K * 2)
                                               : (uint32_t)((size_t)(row1 - row0) * K * 2);
    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(a_base, a_bytes);
    uint32_t a_voff[A_PER_WAVE];
#pragma unroll
    for (int i = 0; i < A_PER_WAVE; ++i) {
        const int j = wave + 4 * i;
        const int r = (j < A_INSTR ? j : 0) * 8 + (lane >> 3);
        const int pc = lane & 7;               // physical chunk this lane fills
        const int c = pc ^ a_swz(r);           // logical K chunk it must hold
        int slot = row0 + r;
        if (slot >= row1) slot = row1 - 1;     // never stored; keeps gathered reads in range
        const uint32_t arow = (MODE == kGateUp) ? (uint32_t)(p.slot_src[slot] / p.topk) : (uint32_t)(slot - row0);
        a_voff[i] = arow * (uint32_t)K * 2u + (uint32_t)c * 16u;
    }
    // ---- B loads: wave instruction j fills B_ROWS_PER_INSTR rows of one matrix ----
    const size_t b_off = (size_t)expert * (size_t)K * (size_t)N;
    const uint32_t b_bytes = (uint32_t)((size_t)K * N * 2);
    const __amdgpu_buffer_rsrc_t b_rsrc0 = make_rsrc(p.B0 + b_off, b_bytes);
    const __amdgpu_buffer_rsrc_t b_rsrc1 = make_rsrc((NB == 2 ? p.B1 : p.B0) + b_off, b_bytes);
    uint32_t b_voff[B_PER_WAVE];
#pragma unroll
    for (int i = 0; i < B_PER_WAVE; ++i) {
        const int j = wave + 4 * i;
        const int jj = (j < B_INSTR ? j : 0) % B_INSTR_PER_MAT;
        const int k = jj * B_ROWS_PER_INSTR + lane / B_LANES_PER_ROW;
        const int pos = lane % B_LANES_PER_ROW;       // 16-byte piece within the LDS row
        const int pseg = pos >> 1, half = pos & 1;
        const int seg = pseg ^ b_swz<BN>(k);          // logical 16-column segment
        const int col = min(n0 + seg * 16 + half * 8, N - 8);  // columns past N feed unstored outputs
        b_voff[i] = (uint32_t)k * ldb + (uint32_t)col * 2u;
    }

#define SMOE_DMA_ISSUE(KT, STG)                                                                   \
    {                                                                                            \
        char *sbase = smem + (STG) * STAGE;                                                      \
        const uint32_t a_soff = (uint32_t)(KT) * (BK * 2);                                       \
        _Pragma("unroll") for (int i = 0; i < A_PER_WAVE; ++i) {                                 \
            const int j = wave + 4 * i;                                                          \
            if (A_INSTR % 4 == 0 || j < A_INSTR) dma16(a_rsrc, sbase + j * 1024, a_voff[i], a_soff); \
        }                                                                                        \
        const uint32_t b_soff = (uint32_t)(KT) * BK * ldb;                                       \
        _Pragma("unroll") for (int i = 0; i < B_PER_WAVE; ++i) {                                 \
            const int j = wave + 4 * i;                                                          \
            if (B_INSTR % 4 == 0 || j < B_INSTR) {                                               \
                const int b = j / B_INSTR_PER_MAT;                                               \
                dma16(b == 1 ? b_rsrc1 : b_rsrc0, sbase + A_BYTES + j * 1024, b_voff[i], b_soff); \
            }                                                                                    \
        }                                                                                        \
    }

    f32x4 acc[NB][MT][NT];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j) acc[b][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // per-lane fragment geometry
    const int fr = lane & 15, fg = lane >> 4;  // A: row in tile / K chunk; B: lane in group / group
    const int tr_k = 8 * fg + (fr >> 2);       // + 4 h + 32 kk
    const int tr_n = 4 * (fr & 3);             // + 16 j (within the wave's columns)

    const int KT = K / BK;
    SMOE_DMA_ISSUE(0, 0);
    for (int kt = 0; kt < KT; ++kt) {
        const int stage = kt & 1;
        __syncthreads();  // this step's tile landed (all waves), last step's reads done
        const char *sa = smem + stage * STAGE;
        const char *sb = sa + A_BYTES;
        uint4 af[2][MT];
        uint4 bfr[2][NB][NT];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int row = wm * WTM + i * 16 + fr;
                const int chunk = kk * 4 + fg;
                af[kk][i] = *reinterpret_cast<const uint4 *>(sa + row * 128 + ((chunk ^ a_swz(row)) << 4));
            }
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const int n = wn * WTN + j * 16 + tr_n;
                    uint2 v[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int k = kk * 32 + tr_k + 4 * h;
                        const int seg = (n >> 4) ^ b_swz<BN>(k);
                        v[h] = lds_read_tr(sb + b * B_BYTES + k * B_ROW + seg * 32 + (n & 15) * 2);
                    }
                    bfr[kk][b][j] = make_uint4(v[0].x, v[0].y, v[1].x, v[1].y);
                }
        }
        if (kt + 1 < KT) SMOE_DMA_ISSUE(kt + 1, stage ^ 1);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int i = 0; i < MT; ++i)
#pragma unroll
                    for (int j = 0; j < NT; ++j)
                        acc[b][i][j] = mfma_16x16x32(af[kk][i], bfr[kk][b][j], acc[b][i][j]);
    }

#undef SMOE_DMA_ISSUE

    // ---- epilogue (C layout: lane holds column lane % 16, rows 4 (lane / 16) + r) ----
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
