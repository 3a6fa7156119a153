// Grouped weight-gradient GEMM for gfx950 (MFMA 16x16x32), the weight half
// of the ParallelLinear backward (ScatterMoE Guide, "3. Fused Backward Pass
// Dynamics": dW_e accumulates g x^T dY over the tokens routed to expert e):
//
//   C_b[e][m, n] = sum over the slots r of expert e of A[r, m] * B_b[r, n]
//
// A [rows, M] and B_b [rows, N] (b < NB) hold one row per slot in slot
// order, so an expert's rows are the contiguous range [off_e, off_{e+1});
// the router gate is already folded into B. The reduction runs over the
// expert's rows, which makes both operands row-major in the reduction
// dimension: their LDS images are [BK rows][BM or BN columns] and the MFMA
// operands (8 consecutive reduction indices of one column) come from
// ds_read_b64_tr_b16 transposing reads, as the forward GEMM's weights do.
//
// Each output tile (e, M tile, N tile) is owned by one workgroup that runs
// the whole reduction in registers and stores plain fp32: no atomics and no
// partial sums in memory (the per-expert reduction stays on chip). The last
// k-step of an expert is ragged: the buffer descriptors of a tile cover only
// that expert's rows, so DMA lanes past them read zero (the buffer range
// check), and an expert with no rows stores a zero tile.
//
// The wave schedule (two groups of four waves one barrier phase apart, group
// 0 issuing the DMA with explicit vmcnt waits) is the one of gemm_pp.hpp.
#pragma once

#include "gemm_pp.hpp"

namespace smoe {

struct WgradParams {
    const uint16_t *A;        // [rows, M] slot order
    const uint16_t *B0, *B1;  // [rows, N] slot order, row stride ldb (B1 only when NB = 2)
    const int32_t *offsets;   // [E + 1] expert row ranges
    void *C0, *C1;            // [E, M, N] fp32, or bf16 with out_bf16
    int out_bf16;             // store the fp32 tile sums rounded to bf16 (RNE)
    int M, N, E;
    int ldb;                  // row stride of B0 / B1 in elements (>= N)
    int n_mt, n_nt;           // tiles per expert
};

template <int BM, int BN, int NB, int BK, int STAGES>
struct WgGeom {
    static constexpr int SMEM = STAGES * (BK * BM * 2 + NB * BK * BN * 2);
};

template <int BM, int BN, int NB, int BK, int STAGES>
__device__ __forceinline__ void wg_tile(const WgradParams &p, char *smem, int e, int mt, int nt) {
    static_assert(BK == 32 || BK == 64, "K step");
    constexpr int KK = BK / 32;
    constexpr int WM = 2, WN = 4;  // 8 waves: 2 row blocks x 4 column blocks
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int MT = WTM / 16, NT = WTN / 16;
    static_assert(MT >= 1 && NT >= 1 && WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be 16-aligned");
    constexpr int A_ROW = BM * 2, B_ROW = BN * 2;
    static_assert(A_ROW >= 128 && A_ROW <= 1024 && B_ROW >= 128 && B_ROW <= 1024, "rows of 128..1024 bytes");
    constexpr int A_BYTES = BK * A_ROW, B_BYTES = BK * B_ROW;
    constexpr int A_INSTR = A_BYTES / 1024, B_INSTR_PER_MAT = B_BYTES / 1024, B_INSTR = NB * B_INSTR_PER_MAT;
    constexpr int A_ROWS_PER_INSTR = 1024 / A_ROW, B_ROWS_PER_INSTR = 1024 / B_ROW;
    constexpr int A_LANES_PER_ROW = A_ROW / 16, B_LANES_PER_ROW = B_ROW / 16;
    constexpr int ASEGS = BM / 16, BSEGS = BN / 16;
    static_assert(A_INSTR % 4 == 0 && B_INSTR % 4 == 0, "DMA split evenly over the 4 loading waves");
    constexpr int A_PER_WAVE = A_INSTR / 4, B_PER_WAVE = B_INSTR / 4, DMA_PER_WAVE = A_PER_WAVE + B_PER_WAVE;
    static_assert(WgGeom<BM, BN, NB, BK, STAGES>::SMEM <= 160 * 1024, "LDS ring");
    constexpr int B_RING = STAGES * A_BYTES;
    // both rings have STAGES slots and each step issues A then B, so a wait
    // for step s leaves exactly the (STAGES - 2) later steps outstanding
    constexpr int WAIT = (STAGES - 2) * DMA_PER_WAVE;
    static_assert(WAIT < 64, "vmcnt range");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int group = wave >> 2;
    const int wl = wave & 3;
    const int wm = wave & 1, wn = wave >> 1;

    const int M = p.M, N = p.N;
    const int off = p.offsets[e];
    const int rows = max(p.offsets[e + 1] - off, 0);
    const int KT = (rows + BK - 1) / BK;
    const int m0 = mt * BM, n0 = nt * BN;

    // descriptors cover exactly this expert's rows: later rows read as zero
    const pp_i32x4 a_rsrc = pp_desc(p.A + (size_t)off * M, (uint32_t)((size_t)rows * M * 2));
    const int ldb = p.ldb;
    const pp_i32x4 b_rsrc0 = pp_desc(p.B0 + (size_t)off * ldb, (uint32_t)((size_t)rows * ldb * 2));
    const pp_i32x4 b_rsrc1 = pp_desc((NB == 2 ? p.B1 : p.B0) + (size_t)off * ldb, (uint32_t)((size_t)rows * ldb * 2));
    const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;
    uint32_t a_voff[A_PER_WAVE], b_voff[B_PER_WAVE];
    if (group == 0) {
#pragma unroll
        for (int i = 0; i < A_PER_WAVE; ++i) {
            const int j = wl + 4 * i;
            const int k = j * A_ROWS_PER_INSTR + lane / A_LANES_PER_ROW;
            const int pos = lane % A_LANES_PER_ROW;
            const int seg = (pos >> 1) ^ pp_b_swz<ASEGS>(k);
            const int col = min(m0 + seg * 16 + (pos & 1) * 8, M - 8);  // columns past M feed unstored outputs
            a_voff[i] = (uint32_t)k * (uint32_t)M * 2u + (uint32_t)col * 2u;
        }
#pragma unroll
        for (int i = 0; i < B_PER_WAVE; ++i) {
            const int j = wl + 4 * i;
            const int jj = j % B_INSTR_PER_MAT;
            const int k = jj * B_ROWS_PER_INSTR + lane / B_LANES_PER_ROW;
            const int pos = lane % B_LANES_PER_ROW;
            const int seg = (pos >> 1) ^ pp_b_swz<BSEGS>(k);
            const int col = min(n0 + seg * 16 + (pos & 1) * 8, N - 8);
            b_voff[i] = (uint32_t)k * (uint32_t)ldb * 2u + (uint32_t)col * 2u;
        }
    }
    // The whole offset goes in the VGPR operand (scalar offset 0) so that the
    // range check sees it.
#define SMOE_WG_ISSUE(KT_)                                                                          \
    {                                                                                               \
        const int slot_ = (KT_) % STAGES;                                                           \
        const uint32_t sa_ = smem_addr + slot_ * A_BYTES;                                           \
        const uint32_t astep_ = (uint32_t)(KT_) * BK * (uint32_t)M * 2u;                            \
        _Pragma("unroll") for (int i = 0; i < A_PER_WAVE; ++i)                                      \
            pp_dma16(a_rsrc, sa_ + (wl + 4 * i) * 1024, a_voff[i] + astep_, 0u);                    \
        const uint32_t sb_ = smem_addr + B_RING + slot_ * (NB * B_BYTES);                           \
        const uint32_t bstep_ = (uint32_t)(KT_) * BK * (uint32_t)ldb * 2u;                          \
        _Pragma("unroll") for (int i = 0; i < B_PER_WAVE; ++i) {                                    \
            const int j = wl + 4 * i;                                                               \
            pp_dma16((j / B_INSTR_PER_MAT) == 1 ? b_rsrc1 : b_rsrc0, sb_ + j * 1024, b_voff[i] + bstep_, 0u); \
        }                                                                                           \
    }

    // fragment offsets: both operands through transposing reads of [k][col] images
    const int fr = lane & 15, fg = lane >> 4;
    int a_rd[KK][MT][2];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = kk * 32 + 8 * fg + 4 * h + (fr >> 2);
                const int m = (WM * i + wm) * 16 + 4 * (fr & 3);
                a_rd[kk][i][h] = k * A_ROW + (((m >> 4) ^ pp_b_swz<ASEGS>(k)) << 5) + (m & 15) * 2;
            }
    int b_rd[KK][NT][2];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = kk * 32 + 8 * fg + 4 * h + (fr >> 2);
                const int n = wn * WTN + j * 16 + 4 * (fr & 3);
                b_rd[kk][j][h] = k * B_ROW + (((n >> 4) ^ pp_b_swz<BSEGS>(k)) << 5) + (n & 15) * 2;
            }

    f32x4 acc[NB][MT][NT];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j) acc[b][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (group == 0) {
#pragma unroll
        for (int st = 0; st < STAGES - 1; ++st)
            if (st < KT) SMOE_WG_ISSUE(st);
        if (KT >= STAGES - 1) pp_wait_dma<WAIT>();
        else pp_wait_dma<0>();
    }
    pp_barrier();
    if (group == 1) pp_barrier();  // group 1 runs one phase behind

    for (int kt = 0; kt < KT; ++kt) {
        if (group == 0 && kt + STAGES - 1 < KT) SMOE_WG_ISSUE(kt + STAGES - 1);
        const char *sa = smem + (kt % STAGES) * A_BYTES;
        const char *sb = smem + B_RING + (kt % STAGES) * (NB * B_BYTES);
        uint4 af[KK][MT];
        uint4 bf[KK][NB][NT];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const uint2 lo = pp_tr(sa + a_rd[kk][i][0]);
                const uint2 hi = pp_tr(sa + a_rd[kk][i][1]);
                af[kk][i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
            }
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const uint2 lo = pp_tr(sb + b * B_BYTES + b_rd[kk][j][0]);
                    const uint2 hi = pp_tr(sb + b * B_BYTES + b_rd[kk][j][1]);
                    bf[kk][b][j] = make_uint4(lo.x, lo.y, hi.x, hi.y);
                }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        pp_barrier();
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int j = 0; j < NT; ++j)
                        acc[b][i][j] = mfma_16x16x32(af[kk][i], bf[kk][b][j], acc[b][i][j]);
        __builtin_amdgcn_s_setprio(0);
        if (group == 0) {
            if (kt + STAGES - 1 < KT) pp_wait_dma<WAIT>();
            else pp_wait_dma<0>();
        }
        pp_barrier();
    }
    if (group == 0) pp_barrier();
#undef SMOE_WG_ISSUE

    // Epilogue through LDS (the ring is free once every wave is past the
    // loop): each wave writes a slice of its accumulators to its own LDS
    // region in the MFMA layout (lane holds column lane % 16 and rows
    // 4 (lane / 16) + r of a 16x16 block) and reads it back as rows, so the
    // fp32 gradient leaves in 16-byte stores covering WTN-column row
    // segments (128 or 256 bytes) instead of 64-byte pieces of four rows.
    // The stores are non-temporal (measured: GPT-OSS weight gradients, 128
    // experts of ~256 rows, 2.06 -> 1.88 ms; neutral on Mixtral and DS-V3).
    constexpr int STRIDE = WTN + 4;  // floats per LDS row (+4: distinct banks for the 4 row groups)
    constexpr int WAVE_BYTES_FULL = MT * 16 * STRIDE * 4;
    constexpr int LDS_BYTES = WgGeom<BM, BN, NB, BK, STAGES>::SMEM;
    constexpr int PASSES = (8 * WAVE_BYTES_FULL <= LDS_BYTES) ? 1 : (8 * WAVE_BYTES_FULL / 2 <= LDS_BYTES) ? 2 : 4;
    static_assert(MT % PASSES == 0 && 8 * (WAVE_BYTES_FULL / PASSES) <= LDS_BYTES, "epilogue staging fits the ring");
    constexpr int MT_P = MT / PASSES;          // 16-row blocks per pass
    constexpr int ROWS_P = MT_P * 16;          // LDS rows per wave per pass
    constexpr int LANES_PER_ROW = WTN / 4;     // 16-byte pieces per row
    constexpr int ROWS_PER_READ = 64 / LANES_PER_ROW;
    float *reg = reinterpret_cast<float *>(smem) + wave * (ROWS_P * STRIDE);
    const int col_in_tile = lane & 15;
    const int row_grp = (lane >> 4) * 4;
    const int rd_row = lane / LANES_PER_ROW, rd_col = (lane % LANES_PER_ROW) * 4;
    __syncthreads();  // every wave is done reading the operand ring
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const size_t c_off = (size_t)e * M * N;
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
#pragma unroll
            for (int il = 0; il < MT_P; ++il)
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int j = 0; j < NT; ++j)
                        reg[(il * 16 + row_grp + r) * STRIDE + j * 16 + col_in_tile] = acc[b][ps * MT_P + il][j][r];
#pragma unroll
            for (int q = 0; q < ROWS_P / ROWS_PER_READ; ++q) {
                const int rl = q * ROWS_PER_READ + rd_row;  // LDS row: block il = rl / 16, row rl % 16
                const int m = m0 + (WM * (ps * MT_P + rl / 16) + wm) * 16 + (rl % 16);
                const int n = n0 + wn * WTN + rd_col;
                const f32x4 v = *reinterpret_cast<const f32x4 *>(reg + rl * STRIDE + rd_col);
                // streaming store: the gradient is not read again by this pass
                if (m < M && n < N) {
                    const size_t o = c_off + (size_t)m * N + n;
                    if (p.out_bf16) {
                        const u32x2 w2 = {(uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16),
                                          (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16)};
                        __builtin_nontemporal_store(w2, reinterpret_cast<u32x2 *>(
                                                            static_cast<uint16_t *>(b == 0 ? p.C0 : p.C1) + o));
                    } else {
                        __builtin_nontemporal_store(
                            v, reinterpret_cast<f32x4 *>(static_cast<float *>(b == 0 ? p.C0 : p.C1) + o));
                    }
                }
            }
        }
    }
    __syncthreads();  // the next tile's DMA may overwrite the staging area
}

// Persistent: one workgroup per CU walks the tiles (expert major, then N
// tile, M tile minor, so consecutive tiles share the expert's B panel) with
// stride gridDim.x over an XCD-contiguous numbering.
template <int BM, int BN, int NB, int BK, int STAGES>
__global__ __launch_bounds__(512) void grouped_wgrad_kernel(const WgradParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[WgGeom<BM, BN, NB, BK, STAGES>::SMEM];
    const int per_e = p.n_mt * p.n_nt;
    const int total = p.E * per_e;
    const int G = gridDim.x;
    for (int L = xcd_remap(blockIdx.x, G); L < total; L += G) {
        const int e = L / per_e, rem = L - e * per_e;
        const int nt = rem / p.n_mt, mt = rem - nt * p.n_mt;
        wg_tile<BM, BN, NB, BK, STAGES>(p, smem, e, mt, nt);
    }
}

// One persistent launch with 32-row k-steps. The reduction runs over an
// expert's rows: with fewer than ~256 rows per expert a 3-deep ring fills
// sooner (DS-V3 dW -5 %); with long experts the 4-deep ring keeps more in
// flight (Mixtral dW 4 % faster than 3-deep).
template <int BM, int BN, int NB>
inline void launch_grouped_wgrad(const WgradParams &q, int64_t rows, int64_t experts, int grid, hipStream_t stream) {
    if (rows < 256 * experts) grouped_wgrad_kernel<BM, BN, NB, 32, 3><<<grid, 512, 0, stream>>>(q);
    else grouped_wgrad_kernel<BM, BN, NB, 32, 4><<<grid, 512, 0, stream>>>(q);
}

}  // namespace smoe
