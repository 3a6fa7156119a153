// Pipelined grouped, gathered bf16 GEMM for gfx950 (MFMA 16x16x32).
//
// Contract as grouped_gemm_kernel (gemm.hpp): one workgroup of 4 waves
// computes a BM x BN tile of one expert, with the fused SwiGLU gate+up
// (two weight matrices sharing each A tile), the router-weighted
// scatter-add, or a plain fp32 store as epilogue.
//
// Data movement:
//  * HBM -> LDS by buffer_load_dwordx4 ... lds (LDS DMA, no VGPR staging).
//    Each wave instruction fills 1 KB of LDS; the global piece a lane
//    fetches is chosen so that the LDS image comes out swizzled. The DMA is
//    issued from inline assembly with explicit s_waitcnt vmcnt bookkeeping,
//    so loads can run STAGES - 1 k-steps ahead of the MFMAs (the compiler's
//    automatic waits would drain every DMA before each LDS read).
//  * A (token rows, K-contiguous): one ds_read_b128 per MFMA operand.
//  * B (weights, N-contiguous as stored): two ds_read_b64_tr_b16 per MFMA
//    operand. Within a 16-lane group that instruction gives lane i element
//    (i % 4) of the 8-byte piece addressed by lane 4 r + i / 4 (r = 0..3):
//    lane q of group g addresses row k = 8 g + 4 h + q / 4, columns
//    4 (q % 4) .. + 3 of its 16-column fragment, so reads h = 0, 1 deliver
//    K = 8 g .. 8 g + 7 in the same order as the A operand.
//
// Schedule of k-step t (BK = 32, ring of STAGES LDS buffers):
//   wait for my DMA of step t+1, barrier        (step t+1 visible to all)
//   issue DMA of step t+STAGES-1 into the buffer step t-1 used
//   MFMAs of step t on fragments already in registers, interleaved with the
//   LDS reads of step t+1's fragments into the other register set.
#pragma once

#include "gemm.hpp"

namespace smoe {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4p_t;

// Raw buffer descriptor (CDNA format word 3: 32-bit data, no swizzle) in
// SGPRs; loads at offsets >= bytes return zero.
__device__ __forceinline__ i32x4_t make_desc(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    i32x4_t d;
    d[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    d[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
    d[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    d[3] = 0x00020000;
    return d;
}

// One wave instruction: 64 lanes x 16 bytes into LDS [lds, lds + 1024).
// No VGPR is written, so nothing can be overwritten while it is in flight;
// completion is tracked by vmcnt and waited for explicitly.
__device__ __forceinline__ void dma_b128(const i32x4_t &desc, uint32_t lds_byte_addr, uint32_t voff, uint32_t soff) {
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(desc), "s"(soff), "{m0}"(lds_byte_addr)
                 : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint2 lds_tr_b64(const char *p) {
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4p_t *)(p));
    return __builtin_bit_cast(uint2, v);
}

// A rows are 32 bf16 (64 B, four 16-byte chunks). The chunk index is XORed
// with a function of the row that makes the 16 rows one ds_read_b128 touches
// (one chunk each) hit distinct banks whether the LDS serves 128 or 256
// bytes per cycle.
__device__ __forceinline__ int pipe_a_swz(int r) { return (((r >> 1) ^ (r >> 3)) & 1) | (((r >> 2) & 1) << 1); }
// B rows are BN bf16 cut into 32-byte segments (16 columns); the segment
// index is XORed with a function of k so the 4 (or 8) rows one transposing
// read touches land in different banks.
template <int SEGS>
__device__ __forceinline__ int pipe_b_swz(int k) {
    return (SEGS >= 8) ? ((k & 3) | (((k >> 3) & 1) << 2)) : (k & (SEGS - 1));
}

template <int BM, int BN, int WM, int WN, int MODE, int STAGES>
__global__ __launch_bounds__(256) void grouped_gemm_pipe_kernel(const GemmParams p) {
    constexpr int NB = (MODE == kGateUp) ? 2 : 1;
    constexpr int BK = 32;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int MT = WTM / 16, NT = WTN / 16;
    static_assert(WM * WN == 4, "4 waves per workgroup");
    static_assert(MT >= 1 && NT >= 1 && WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be 16-aligned");
    static_assert(BN % 64 == 0 && BN <= 512, "B rows are 128..1024 bytes");
    static_assert(STAGES >= 3 && STAGES <= 6, "ring depth");
    constexpr int A_ROW = BK * 2;                  // 64 B
    constexpr int A_BYTES = BM * A_ROW;
    constexpr int B_ROW = BN * 2;
    constexpr int B_BYTES = BK * B_ROW;
    constexpr int STAGE = A_BYTES + NB * B_BYTES;
    static_assert(A_BYTES % 1024 == 0 && B_BYTES % 1024 == 0, "whole 1 KB DMA blocks");
    constexpr int A_INSTR = A_BYTES / 1024;        // 16 rows each
    constexpr int B_INSTR_PER_MAT = B_BYTES / 1024;
    constexpr int B_INSTR = NB * B_INSTR_PER_MAT;
    constexpr int B_ROWS_PER_INSTR = 1024 / B_ROW;
    constexpr int B_LANES_PER_ROW = B_ROW / 16;
    constexpr int SEGS = BN / 16;
    static_assert(A_INSTR % 4 == 0 && B_INSTR % 4 == 0, "DMA instructions split evenly over 4 waves");
    constexpr int A_PER_WAVE = A_INSTR / 4;
    constexpr int B_PER_WAVE = B_INSTR / 4;
    constexpr int DMA_PER_WAVE = A_PER_WAVE + B_PER_WAVE;
    static_assert(DMA_PER_WAVE * (STAGES - 2) < 64, "vmcnt range");

    __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];
    const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // ---- tile decode: XCD-contiguous logical id, grouped M-major order ----
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

    // ---- DMA sources ----
    const uint16_t *a_base = (MODE == kGateUp) ? p.A : p.A + (size_t)row0 * K;
    const uint32_t a_bytes = (MODE == kGateUp) ? (uint32_t)((size_t)p.A_rows * K * 2)
                                               : (uint32_t)((size_t)(row1 - row0) * K * 2);
    const i32x4_t a_desc = make_desc(a_base, a_bytes);
    uint32_t a_voff[A_PER_WAVE];
#pragma unroll
    for (int i = 0; i < A_PER_WAVE; ++i) {
        const int j = wave + 4 * i;               // instruction: rows 16 j .. 16 j + 15
        const int r = 16 * j + (lane >> 2);
        const int c = (lane & 3) ^ pipe_a_swz(r);  // logical 16-byte K chunk this lane must hold
        int slot = row0 + r;
        if (slot >= row1) slot = row1 - 1;        // never stored; keeps gathered reads in range
        const uint32_t arow = (MODE == kGateUp) ? (uint32_t)(p.slot_src[slot] / p.topk) : (uint32_t)(slot - row0);
        a_voff[i] = arow * (uint32_t)K * 2u + (uint32_t)c * 16u;
    }
    const size_t b_off = (size_t)expert * (size_t)K * (size_t)N;
    const uint32_t b_bytes = (uint32_t)((size_t)K * N * 2);
    const i32x4_t b_desc0 = make_desc(p.B0 + b_off, b_bytes);
    const i32x4_t b_desc1 = make_desc((NB == 2 ? p.B1 : p.B0) + b_off, b_bytes);
    uint32_t b_voff[B_PER_WAVE];
#pragma unroll
    for (int i = 0; i < B_PER_WAVE; ++i) {
        const int j = wave + 4 * i;
        const int jj = j % B_INSTR_PER_MAT;
        const int k = jj * B_ROWS_PER_INSTR + lane / B_LANES_PER_ROW;
        const int pos = lane % B_LANES_PER_ROW;
        const int seg = (pos >> 1) ^ pipe_b_swz<SEGS>(k);
        const int col = min(n0 + seg * 16 + (pos & 1) * 8, N - 8);  // columns past N feed unstored outputs
        b_voff[i] = (uint32_t)k * ldb + (uint32_t)col * 2u;
    }

    auto issue = [&](int kt) __attribute__((always_inline)) {
        const uint32_t sbase = smem_addr + (uint32_t)((kt % STAGES) * STAGE);
        const uint32_t a_soff = (uint32_t)kt * (BK * 2);
#pragma unroll
        for (int i = 0; i < A_PER_WAVE; ++i) dma_b128(a_desc, sbase + (wave + 4 * i) * 1024, a_voff[i], a_soff);
        const uint32_t b_soff = (uint32_t)kt * BK * ldb;
#pragma unroll
        for (int i = 0; i < B_PER_WAVE; ++i) {
            const int j = wave + 4 * i;
            dma_b128((j / B_INSTR_PER_MAT) == 1 ? b_desc1 : b_desc0, sbase + A_BYTES + j * 1024, b_voff[i], b_soff);
        }
    };

    // ---- fragment geometry ----
    const int fr = lane & 15, fg = lane >> 4;
    int a_rd[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int row = wm * WTM + i * 16 + fr;
        a_rd[i] = row * A_ROW + ((fg ^ pipe_a_swz(row)) << 4);
    }
    int b_rd[NT][2];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = 8 * fg + 4 * h + (fr >> 2);
            const int n = wn * WTN + j * 16 + 4 * (fr & 3);
            b_rd[j][h] = A_BYTES + k * B_ROW + (((n >> 4) ^ pipe_b_swz<SEGS>(k)) << 5) + (n & 15) * 2;
        }

    auto read_frags = [&](int kt, uint4 (&af)[MT], uint4 (&bf)[NB][NT]) __attribute__((always_inline)) {
        const char *s = smem + (kt % STAGES) * STAGE;
#pragma unroll
        for (int i = 0; i < MT; ++i) af[i] = *reinterpret_cast<const uint4 *>(s + a_rd[i]);
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const uint2 lo = lds_tr_b64(s + b * B_BYTES + b_rd[j][0]);
                const uint2 hi = lds_tr_b64(s + b * B_BYTES + b_rd[j][1]);
                bf[b][j] = make_uint4(lo.x, lo.y, hi.x, hi.y);
            }
    };

    f32x4 acc[NB][MT][NT];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j) acc[b][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto mfmas = [&](const uint4 (&af)[MT], const uint4 (&bf)[NB][NT]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int j = 0; j < NT; ++j) acc[b][i][j] = mfma_16x16x32(af[i], bf[b][j], acc[b][i][j]);
    };

    const int KT = K / BK;
    // prologue: steps 0 .. STAGES-2 in flight, step 0 landed and read
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < KT) issue(s);
    if (KT >= STAGES - 1) wait_vmcnt<DMA_PER_WAVE * (STAGES - 2)>();
    else wait_vmcnt<0>();
    block_barrier();
    uint4 afA[MT], afB[MT];
    uint4 bfA[NB][NT], bfB[NB][NT];
    read_frags(0, afA, bfA);

    // one k-step; `cur` holds step t's fragments, `nxt` receives step t+1's
#define SMOE_PIPE_STEP(T, CUR_A, CUR_B, NXT_A, NXT_B)                                              \
    {                                                                                              \
        const int t_ = (T);                                                                        \
        if (t_ + 1 < KT) {                                                                         \
            if (t_ + STAGES - 1 <= KT) wait_vmcnt<DMA_PER_WAVE * (STAGES - 3)>();                  \
            else wait_vmcnt<0>();                                                                  \
            block_barrier();                                                                       \
            if (t_ + STAGES - 1 < KT) issue(t_ + STAGES - 1);                                      \
            read_frags(t_ + 1, NXT_A, NXT_B);                                                      \
        }                                                                                          \
        mfmas(CUR_A, CUR_B);                                                                       \
    }

    int t = 0;
    for (; t + 1 < KT; t += 2) {
        SMOE_PIPE_STEP(t, afA, bfA, afB, bfB);
        SMOE_PIPE_STEP(t + 1, afB, bfB, afA, bfA);
    }
    if (t < KT) SMOE_PIPE_STEP(t, afA, bfA, afB, bfB);
#undef SMOE_PIPE_STEP

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
