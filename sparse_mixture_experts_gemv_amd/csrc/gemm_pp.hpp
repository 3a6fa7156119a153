// Ping-pong grouped, gathered bf16 GEMM for gfx950 (MFMA 16x16x32).
//
// The GEMM contract and the epilogue modes (kGateUp, kDown, kDownRows,
// kLogits, kLinBf16, kGateUpSave, kSwigluBwd) are described in gemm.hpp. One
// workgroup of 8 waves (two per SIMD) computes a BM x BN tile of one expert
// (pp_tile); the persistent and stream-K kernels at the end of this file walk
// the tiles of a device-built block order.
//
// Operand path: HBM -> LDS by LDS DMA (buffer_load ... lds), A read back as
// K-contiguous ds_read_b128 operands, B (weights, N-contiguous as stored)
// read back with ds_read_b64_tr_b16 transposing reads. Within a 16-lane
// group that instruction gives lane i element (i % 4) of the 8-byte piece
// addressed by lane 4 r + i / 4 (r = 0..3), so lane q of group g addresses
// row k = 8 g + 4 h + q / 4, columns 4 (q % 4) .. + 3 of its 16-column
// fragment and reads h = 0, 1 deliver K = 8 g .. 8 g + 7, the A operand's
// K order.
//
// Schedule (k-steps of BK = 32 or 64): the waves form two groups of four (one wave
// of each per SIMD), running the same sequence "read fragments of step k
// from LDS | barrier | MFMAs of step k | barrier" one barrier phase apart,
// so on every SIMD one wave feeds the matrix core while the other reads LDS.
// The LDS holds two rings: STAGES steps of B and STAGES_A steps of A. During
// its read phase for step k, a group issues the DMA of step k + STAGES_A - 1
// of A and/or of step k + STAGES - 1 of B, each into the slot of step k - 1
// of its ring (both groups finished reading it at least one phase earlier),
// spread among its fragment reads, so up to STAGES - 1 steps of weights are
// in flight per CU. Either group 0 issues both rings and, at the end of its
// MFMA phase, waits until step k + 1 has landed; or (the gate+up tiles and
// the launches that pass kFlagSplitDma: the 64-deep down, input-gradient
// and ParallelLinear tiles listed at pp_dma_split)
// group 0 issues A and waits for it there, and group 1 issues B and waits,
// at the end of its read phase, for the B of step k + 1. Both waits come
// before the barrier that opens step k + 1 to readers. The DMA is plain
// assembly with explicit vmcnt bookkeeping because the compiler would drain
// every DMA before each LDS read (it cannot prove the ring slots disjoint).
#pragma once

#include <type_traits>

#include "gemm.hpp"

namespace smoe {

typedef short pp_s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void pp_lds_void;
typedef __attribute__((address_space(3))) pp_s16x4 pp_lds_s16x4;

typedef int pp_i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (CDNA word 3: 32-bit data, no swizzle) in SGPRs;
// loads at offsets >= bytes return zero.
__device__ __forceinline__ pp_i32x4 pp_desc(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    pp_i32x4 d;
    d[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    d[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
    d[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    d[3] = 0x00020000;
    return d;
}

// LDS DMA of one wave instruction: 64 lanes x 16 bytes into LDS
// [lds, lds + 1024). Written as assembly so that the compiler does not drain
// it before every later LDS read (it cannot prove the stages disjoint);
// completion is waited for explicitly with s_waitcnt vmcnt. The instruction
// writes no VGPR, so nothing can be overwritten while it is in flight.
__device__ __forceinline__ void pp_dma16(const pp_i32x4 &desc, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(desc), "s"(soff), "{m0}"(lds)
                 : "memory");
}

__device__ __forceinline__ uint2 pp_tr(const char *p) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((pp_lds_s16x4 *)(p)));
}

// Barrier that the compiler may move neither memory accesses nor other
// instructions across.
__device__ __forceinline__ void pp_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <int N>
__device__ __forceinline__ void pp_wait_dma() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// A tile rows are BK bf16 = CH chunks of 16 B (CH = 4 or 8). The chunk index
// is XORed with a function of the row so that the fragment reads (16
// consecutive rows, one chunk each, per 16-lane group) hit distinct banks;
// both forms were checked with the LDS bank-conflict counter on gfx950 (the
// 64-byte-row form r & 3 / (r >> 2) & 3 variants conflict, (r >> 1) & 3 does
// not).
template <int CH>
__device__ __forceinline__ int pp_a_swz(int r) {
    return (CH == 8) ? (((r >> 1) ^ ((r & 1) << 2)) & 7) : ((r >> 1) & 3);
}
// B tile rows: BN bf16 in 32-byte segments (16 columns); segment XOR by k.
template <int SEGS>
__device__ __forceinline__ int pp_b_swz(int k) {
    return (SEGS >= 8) ? ((k & 3) | (((k >> 3) & 1) << 2)) : (k & (SEGS - 1));
}

// LDS: a ring of STAGES_A k-steps of A and a ring of STAGES k-steps of B.
template <int BM, int BN, int MODE, int BK, int STAGES, int STAGES_A = STAGES>
struct PPGeom {
    static constexpr int NB = (MODE == kGateUp || MODE == kGateUpSave) ? 2 : 1;
    static constexpr int RING = STAGES_A * BM * BK * 2 + STAGES * NB * BK * BN * 2;
    // the bf16 epilogues stage a whole BM x (BN + 8) tile in the same LDS
    static constexpr int STAGE_BF16 =
        (MODE == kGateUp || MODE == kGateUpSave || MODE == kLinBf16) ? BM * (BN + 8) * 2 : 0;
    static constexpr int SMEM = RING > STAGE_BF16 ? RING : STAGE_BF16;
};

// Whether the two wave groups share the DMA issue (group 0 the token rows,
// group 1 the weights, each in its own read phase) rather than group 0
// issuing both. Measured against group 0 alone (both with the instructions
// spread among the reads): the gate+up GEMM 1524 -> 1490 us on Mixtral, 1245
// -> 1198 us on GPT-OSS, 1111 -> 1083 us on Qwen2 S = 4096. On the down GEMM's
// 32-deep tiles sharing was 1-3 % slower, but on its 192 x 256 tile with
// 64-deep k-steps (3/2 rings) it pays: Mixtral 885-888 -> 842-844 us,
// Qwen2 S = 4096 748-762 -> 693-696 us, which beats the 32-deep 4/4 tile
// without sharing. Launches opt in with kFlagSplitDma: that down tile, the
// backward's 192- and 128-row transposed-weight tiles, the ParallelLinear
// input-gradient 192-row tile and its 256-row forward tile (with a 3-deep
// weight ring). The 128-row and short-tile down launches, the router's
// logits tile, the decode-size tiles and the stream-K down GEMM measured
// 0-1 % slower or unchanged with it.
constexpr bool pp_dma_split(int mode, int flags) {
    return mode == kGateUp || mode == kGateUpSave || (flags & kFlagSplitDma) != 0;
}

// One tile (mt, nt), k-steps [k_begin, k_end) of BK, epilogue included. All
// 512 threads of the workgroup call it together; on return every LDS read of
// the ring has completed, so the caller may start another tile.
//
// The A (token rows) and B (weights) rings may have different depths: with
// STAGES_A < STAGES the weights, which mostly come from HBM, are requested
// STAGES - 1 steps ahead and the token rows, mostly L2 hits, STAGES_A - 1
// steps ahead, within the same LDS budget.
template <int BM, int BN, int MODE, int BK, int STAGES, int STAGES_A = STAGES, bool PARTIAL = false, int FLAGS = 0>
__device__ __forceinline__ void pp_tile(const GemmParams &p, char *smem, int mt, int nt, int k_begin, int k_end) {
    constexpr int NB = (MODE == kGateUp || MODE == kGateUpSave) ? 2 : 1;
    constexpr bool BT = (FLAGS & kFlagBT) != 0;          // B stored [N, K]
    constexpr bool KSPLIT = (FLAGS & kFlagKSplit) != 0;  // k < K/2 from B0, k >= K/2 from B1
    static_assert(!KSPLIT || (BT && NB == 1), "K split is for one transposed B");
    static_assert(BK == 32 || BK == 64, "K step");
    constexpr int KK = BK / 32;                     // MFMA K sub-steps per step
    constexpr int CH = BK / 8;                      // 16-byte chunks per A row
    constexpr int WM = 2, WN = 4;                   // 8 waves: 2 row blocks x 4 column blocks
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int MT = WTM / 16, NT = WTN / 16;
    static_assert(MT >= 1 && NT >= 1 && WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be 16-aligned");
    static_assert(BN % 64 == 0 && BN <= 512, "B rows are 128..1024 bytes");
    constexpr int A_ROW = BK * 2;                   // 64 or 128 B
    constexpr int A_BYTES = BM * A_ROW;
    constexpr int B_ROW = BN * 2;
    constexpr int B_BYTES = BK * B_ROW;
    constexpr int A_INSTR = A_BYTES / 1024;
    constexpr int A_ROWS_PER_INSTR = 1024 / A_ROW;
    constexpr int B_INSTR_PER_MAT = B_BYTES / 1024;
    constexpr int B_INSTR = NB * B_INSTR_PER_MAT;
    constexpr int B_ROWS_PER_INSTR = 1024 / B_ROW;
    constexpr int B_LANES_PER_ROW = B_ROW / 16;
    constexpr int SEGS = BN / 16;
    static_assert(A_INSTR % 4 == 0 && B_INSTR % 4 == 0, "DMA split evenly over the 4 loading waves");
    constexpr int A_PER_WAVE = A_INSTR / 4;
    constexpr int B_PER_WAVE = B_INSTR / 4;
    constexpr int DMA_PER_WAVE = A_PER_WAVE + B_PER_WAVE;
    static_assert(STAGES_A >= 2 && STAGES_A <= STAGES, "A ring no deeper than the B ring");
    static_assert(STAGES_A * A_BYTES + STAGES * NB * B_BYTES <= 160 * 1024, "LDS rings");
    constexpr int B_RING = STAGES_A * A_BYTES;  // byte offset of the B ring
    // ops a group-0 wave may leave outstanding when the next step is needed:
    // those issued after that step's A and after its B (steady state)
    constexpr int WAIT_A = B_PER_WAVE + (STAGES_A - 2) * DMA_PER_WAVE;
    constexpr int WAIT_B = (STAGES - 2) * DMA_PER_WAVE;
    constexpr int WAIT_STEADY = WAIT_A < WAIT_B ? WAIT_A : WAIT_B;
    constexpr int WAIT_FIRST = (STAGES_A - 2) * A_PER_WAVE + (STAGES - 2) * B_PER_WAVE;
    static_assert(WAIT_FIRST < 64 && WAIT_STEADY < 64, "vmcnt range");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int group = wave >> 2;                    // waves w and w + 4 share a SIMD
    const int wl = wave & 3;                        // index within the group
    const int wm = wave & 1, wn = wave >> 1;        // group 0: column blocks 0, 1; group 1: 2, 3

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
    // Tiles with fewer than BM rows (PARTIAL) skip work on the missing rows.
    // 16-row blocks are dealt to the two row halves of the waves alternately
    // (block b to wm = b % WM), so a short tile still spreads its rows over
    // every SIMD; a wave skips the MFMAs of its groups of MQ blocks that lie
    // wholly past row1.
    const int mlim = min(MT, max(0, (((row1 - row0 + 15) >> 4) - wm + WM - 1) / WM));
    // A DMA instructions whose rows all lie past row1 are not issued either.
    // This is only done with a 2-deep A ring: then no A instruction is ever
    // issued between the last one a wait needs and that wait, so the vmcnt
    // targets below (counts of later B instructions) stay exact. LDS rows
    // past row1 keep stale values; they only feed output rows that are not
    // stored.
    constexpr bool SKIP_A = PARTIAL && STAGES_A == 2;
    const int a_cnt = min(A_PER_WAVE, max(0, ((row1 - row0 + A_ROWS_PER_INSTR - 1) / A_ROWS_PER_INSTR - wl + 3) / 4));
    constexpr int MQ = (MT % 2 == 0) ? 2 : 1;  // blocks per MFMA group that is skipped as a whole
    const int n0 = nt * BN;
    const int N = p.N, K = p.K;
    const uint32_t ldb = (uint32_t)N * 2u;

    // ---- DMA sources (group 0 only) ----
    // token rows of A read by index (kGateUp always; kDownRows / kLinBf16 on request)
    const bool gather = (MODE == kGateUp || MODE == kGateUpSave) ||
                        ((MODE == kDownRows || MODE == kLinBf16 || MODE == kSwigluBwd) && p.gather_a);
    const uint16_t *a_base = gather ? p.A : p.A + (size_t)row0 * K;
    const uint32_t a_bytes = gather ? (uint32_t)((size_t)p.A_rows * K * 2) : (uint32_t)((size_t)(row1 - row0) * K * 2);
    const pp_i32x4 a_rsrc = pp_desc(a_base, a_bytes);
    const int KB = KSPLIT ? K / 2 : K;  // K extent of one B matrix
    const size_t b_off = (size_t)expert * (size_t)KB * (size_t)N;
    const uint32_t b_bytes = (uint32_t)((size_t)KB * N * 2);
    const pp_i32x4 b_rsrc0 = pp_desc(p.B0 + b_off, b_bytes);
    const pp_i32x4 b_rsrc1 = pp_desc((NB == 2 || KSPLIT ? p.B1 : p.B0) + b_off, b_bytes);
    const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;
    // Who issues the DMA (measured per epilogue, see pp_dma_split): with SPLIT,
    // group 0 the A (token row) DMA and group 1 the B (weight) DMA, each
    // during its own read phase; otherwise group 0 issues both.
    constexpr bool SPLIT = pp_dma_split(MODE, FLAGS);
    uint32_t a_voff[A_PER_WAVE], b_voff[B_PER_WAVE];
    if (group == 0) {
#pragma unroll
        for (int i = 0; i < A_PER_WAVE; ++i) {
            const int j = wl + 4 * i;               // instruction: A_ROWS_PER_INSTR rows
            const int r = A_ROWS_PER_INSTR * j + lane / CH;
            const int c = (lane % CH) ^ pp_a_swz<CH>(r);
            int slot = row0 + r;
            if (slot >= row1) slot = row1 - 1;      // never stored; keeps gathered reads in range
            const uint32_t arow = gather ? (uint32_t)(p.slot_src[slot] / p.topk) : (uint32_t)(slot - row0);
            a_voff[i] = arow * (uint32_t)K * 2u + (uint32_t)c * 16u;
        }
    }
    if (group == (SPLIT ? 1 : 0)) {
#pragma unroll
        for (int i = 0; i < B_PER_WAVE; ++i) {
            const int j = wl + 4 * i;
            const int jj = j % B_INSTR_PER_MAT;
            if constexpr (BT) {
                // B^T image like the A image: BN rows (weight rows n), BK K-contiguous
                const int r = A_ROWS_PER_INSTR * jj + lane / CH;
                const int c = (lane % CH) ^ pp_a_swz<CH>(r);
                const int n = min(n0 + r, N - 1);  // rows past N feed unstored outputs
                b_voff[i] = (uint32_t)n * (uint32_t)KB * 2u + (uint32_t)c * 16u;
            } else {
                const int k = jj * B_ROWS_PER_INSTR + lane / B_LANES_PER_ROW;
                const int pos = lane % B_LANES_PER_ROW;
                const int seg = (pos >> 1) ^ pp_b_swz<SEGS>(k);
                const int col = min(n0 + seg * 16 + (pos & 1) * 8, N - 8);  // columns past N feed unstored outputs
                b_voff[i] = (uint32_t)k * ldb + (uint32_t)col * 2u;
            }
        }
    }

#define SMOE_PP_ISSUE_A(KT)                                                                        \
    {                                                                                              \
        const uint32_t sbase = smem_addr + SMOE_SLOT_A(KT) * A_BYTES;                              \
        const uint32_t a_soff = (uint32_t)(KT) * (BK * 2);                                         \
        _Pragma("unroll") for (int i = 0; i < A_PER_WAVE; ++i)                                     \
            if (!SKIP_A || i < a_cnt) pp_dma16(a_rsrc, sbase + (wl + 4 * i) * 1024, a_voff[i], a_soff); \
    }
#define SMOE_PP_ISSUE_B(KT)                                                                        \
    {                                                                                              \
        const uint32_t sbase = smem_addr + B_RING + SMOE_SLOT_B(KT) * (NB * B_BYTES);              \
        const bool hi_ = KSPLIT && (KT) * BK >= KB;                                                \
        const uint32_t b_soff = (uint32_t)((KT) - (hi_ ? KB / BK : 0)) * (BT ? BK * 2u : BK * ldb); \
        _Pragma("unroll") for (int i = 0; i < B_PER_WAVE; ++i) {                                   \
            const int j = wl + 4 * i;                                                              \
            pp_dma16(((j / B_INSTR_PER_MAT) == 1 || hi_) ? b_rsrc1 : b_rsrc0, sbase + j * 1024,    \
                     b_voff[i], b_soff);                                                           \
        }                                                                                          \
    }

    // ---- fragment read offsets within a stage ----
    const int fr = lane & 15, fg = lane >> 4;
    // The swizzles depend only on the low four bits of a row (A, B^T) or on
    // bits 0, 1 and 3 of a k index (B), so offsets that differ by a multiple
    // of 16 rows, or by 32 k and by 4 k, differ by a constant: one register
    // per kk (A, B^T) or per j (B) and the rest as immediate offsets.
    int a_rd[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        const int row = wm * 16 + fr;
        a_rd[kk] = row * A_ROW + (((kk * 4 + fg) ^ pp_a_swz<CH>(row)) << 4);
    }
    constexpr int A_RD_I = WM * 16 * A_ROW;  // + i * A_RD_I for block i
    int b_rd[BT ? KK : NT];
    if constexpr (BT) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int row = wn * WTN + fr;
            b_rd[kk] = row * A_ROW + (((kk * 4 + fg) ^ pp_a_swz<CH>(row)) << 4);
        }
    } else {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int k = 8 * fg + (fr >> 2);
            const int n = wn * WTN + j * 16 + 4 * (fr & 3);
            b_rd[j] = k * B_ROW + (((n >> 4) ^ pp_b_swz<SEGS>(k)) << 5) + (n & 15) * 2;
        }
    }
    // B^T: + j * B_RD_J for column block j; B: + kk * B_RD_KK + h * B_RD_H
    constexpr int B_RD_J = 16 * A_ROW, B_RD_KK = 32 * B_ROW, B_RD_H = 4 * B_ROW;

    f32x4 acc[NB][MT][NT];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j) acc[b][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // k-steps [k_begin, k_end); ring slots of step kt are (kt - k_begin) % STAGES_A
    // (A) and (kt - k_begin) % STAGES (B). Per step, group 0 issues A first,
    // then B.
    const int KT = k_end;
#define SMOE_SLOT_A(KT_) (((KT_) - k_begin) % STAGES_A)
#define SMOE_SLOT_B(KT_) (((KT_) - k_begin) % STAGES)
    if (SPLIT) {
        if (group == 0) {
#pragma unroll
            for (int st = 0; st < STAGES_A - 1; ++st)
                if (k_begin + st < KT) SMOE_PP_ISSUE_A(k_begin + st);
            if (KT - k_begin >= STAGES_A - 1) pp_wait_dma<(STAGES_A - 2) * A_PER_WAVE>();  // first step landed
            else pp_wait_dma<0>();
        } else {
#pragma unroll
            for (int st = 0; st < STAGES - 1; ++st)
                if (k_begin + st < KT) SMOE_PP_ISSUE_B(k_begin + st);
            if (KT - k_begin >= STAGES - 1) pp_wait_dma<(STAGES - 2) * B_PER_WAVE>();
            else pp_wait_dma<0>();
        }
    } else if (group == 0) {
#pragma unroll
        for (int st = 0; st < STAGES - 1; ++st) {
            if (st < STAGES_A - 1 && k_begin + st < KT) SMOE_PP_ISSUE_A(k_begin + st);
            if (k_begin + st < KT) SMOE_PP_ISSUE_B(k_begin + st);
        }
        if (KT - k_begin >= STAGES - 1) pp_wait_dma<WAIT_FIRST>();  // first step landed
        else pp_wait_dma<0>();
    }
    pp_barrier();
    if (group == 1) pp_barrier();  // group 1 runs one phase behind

    for (int kt = k_begin; kt < KT; ++kt) {
        // ---- read phase: refill the slots of step kt-1, then read step kt ----
        const char *sa = smem + SMOE_SLOT_A(kt) * A_BYTES;
        const char *sb = smem + B_RING + SMOE_SLOT_B(kt) * (NB * B_BYTES);
        // one register per fragment column block holds slot base + lane
        // offset; where there are many (kk, b, h) combinations per column
        // block, the opaque move keeps the compiler from hoisting each into
        // a register of its own, so the constants go into the reads' offset
        // fields (with few, the hoisted form schedules better)
        constexpr bool B_LANE_REG = !BT && (KK * NB >= 4 || (BN == 256 && KK == 2 && BM == 256 && STAGES == 3));
        // (the 256 x 256 x 64 3-deep tile also needs it: 14 spilled VGPRs with it, 74 without)
        int b_lane[BT ? 1 : NT];
        if constexpr (!BT) {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                b_lane[j] = (int)(sb - smem) + b_rd[j];
                if constexpr (B_LANE_REG) asm volatile("" : "+v"(b_lane[j]));
            }
        }
        uint4 af[KK][MT];
        uint4 bf[KK][NB][NT];
        // DMA instruction d of step kt's refill: d < A_PER_WAVE the A ring's
        // instruction d, else the B ring's instruction d - A_PER_WAVE (A
        // before B: the order the vmcnt targets assume). Only in steady state,
        // when this wave's ring(s) are refilled at all.
        auto dma_one = [&](const int d) {
            if (d < A_PER_WAVE) {
                const int ia = d < A_PER_WAVE ? d : 0;
                if (!SKIP_A || ia < a_cnt)
                    pp_dma16(a_rsrc, smem_addr + SMOE_SLOT_A(kt + STAGES_A - 1) * A_BYTES + (wl + 4 * ia) * 1024,
                             a_voff[ia], (uint32_t)(kt + STAGES_A - 1) * (BK * 2));
            } else if (d < DMA_PER_WAVE) {
                const int ib = (d >= A_PER_WAVE && d < DMA_PER_WAVE) ? d - A_PER_WAVE : 0;
                const int ktb = kt + STAGES - 1;
                const int jb = wl + 4 * ib;
                const bool hi = KSPLIT && ktb * BK >= KB;
                const uint32_t b_soff = (uint32_t)(ktb - (hi ? KB / BK : 0)) * (BT ? BK * 2u : BK * ldb);
                pp_dma16(((jb / B_INSTR_PER_MAT) == 1 || hi) ? b_rsrc1 : b_rsrc0,
                         smem_addr + B_RING + SMOE_SLOT_B(ktb) * (NB * B_BYTES) + jb * 1024, b_voff[ib], b_soff);
            }
        };
        // The fragment reads of step kt, with the DMA instructions d0 ..
        // d0 + ND - 1 of the refill spread among them: instruction d0 + i
        // follows read (i + 1) RP - 1. A wave that issues a run of DMA
        // instructions stalls until the CU's vector memory unit has taken them
        // (about 16 cycles per 1 KB instruction), so issued all at once, as
        // before the reads, they delay every read behind them; spread, the
        // reads and the DMA proceed together.
        constexpr int PER_KK = MT + NB * NT * (BT ? 1 : 2);
        constexpr int READS = KK * PER_KK;
        auto reads = [&](auto d0_tag, auto nd_tag) {
            constexpr int D0 = decltype(d0_tag)::value, ND = decltype(nd_tag)::value;
            constexpr int RP = (ND > 0 && READS >= ND) ? READS / (ND > 0 ? ND : 1) : 1;
            auto hook = [&](const int r) {
                if (ND > 0 && (r % RP) == RP - 1 && r / RP < ND) dma_one(D0 + r / RP);
            };
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    af[kk][i] = *reinterpret_cast<const uint4 *>(sa + a_rd[kk] + i * A_RD_I);
                    hook(kk * PER_KK + i);
                }
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int j = 0; j < NT; ++j) {
                        if constexpr (BT) {
                            bf[kk][b][j] = *reinterpret_cast<const uint4 *>(sb + b * B_BYTES + b_rd[kk] + j * B_RD_J);
                            hook(kk * PER_KK + MT + b * NT + j);
                        } else {
                            const char *bp = smem + b_lane[j] + b * B_BYTES + kk * B_RD_KK;
                            const uint2 lo = pp_tr(bp);
                            hook(kk * PER_KK + MT + 2 * (b * NT + j));
                            const uint2 hi = pp_tr(bp + B_RD_H);
                            hook(kk * PER_KK + MT + 2 * (b * NT + j) + 1);
                            bf[kk][b][j] = make_uint4(lo.x, lo.y, hi.x, hi.y);
                        }
                    }
            }
#pragma unroll
            for (int d = READS / RP; d < ND; ++d) dma_one(D0 + d);
        };
        using I0 = std::integral_constant<int, 0>;
        using IA = std::integral_constant<int, A_PER_WAVE>;
        using IB = std::integral_constant<int, B_PER_WAVE>;
        using ID = std::integral_constant<int, DMA_PER_WAVE>;
        if constexpr (SPLIT) {
            if (group == 0) {
                if (kt + STAGES_A - 1 < KT) reads(I0{}, IA{});
                else reads(I0{}, I0{});
            } else {
                if (kt + STAGES - 1 < KT) reads(IA{}, IB{});
                else reads(I0{}, I0{});
            }
        } else if (group == 0 && kt + STAGES - 1 < KT) {  // steady state: both rings refilled
            reads(I0{}, ID{});
        } else {
            // the last steps: the refills still due (the A ring's, when it is
            // shallower than the B ring), then the reads
            if (group == 0) {
                if (kt + STAGES_A - 1 < KT) SMOE_PP_ISSUE_A(kt + STAGES_A - 1);
                if (kt + STAGES - 1 < KT) SMOE_PP_ISSUE_B(kt + STAGES - 1);
            }
            reads(I0{}, I0{});
        }
        // reads complete before the barrier: after it the slots may be refilled
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (SPLIT && group == 1) {  // B of step kt+1 must have landed before the barrier that opens it
            if (kt + STAGES - 1 < KT) pp_wait_dma<(STAGES - 2) * B_PER_WAVE>();
            else pp_wait_dma<0>();
        }
        pp_barrier();
        // ---- MFMA phase ----
        __builtin_amdgcn_s_setprio(1);
        if constexpr (!PARTIAL) {
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
#pragma unroll
                for (int i = 0; i < MT; ++i)
#pragma unroll
                    for (int b = 0; b < NB; ++b)
#pragma unroll
                        for (int j = 0; j < NT; ++j)
                            acc[b][i][j] = mfma_16x16x32(af[kk][i], bf[kk][b][j], acc[b][i][j]);
        } else {
#pragma unroll
            for (int c = 0; c < MT; c += MQ) {
                if (c == 0 || c < mlim) {
#pragma unroll
                    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
                        for (int i = c; i < c + MQ; ++i)
#pragma unroll
                            for (int b = 0; b < NB; ++b)
#pragma unroll
                                for (int j = 0; j < NT; ++j)
                                    acc[b][i][j] = mfma_16x16x32(af[kk][i], bf[kk][b][j], acc[b][i][j]);
                }
            }
        }
        __builtin_amdgcn_s_setprio(0);
        if (SPLIT && group == 0) {  // A of step kt+1 must have landed before the barrier that opens it
            if (kt + STAGES_A - 1 < KT) pp_wait_dma<(STAGES_A - 2) * A_PER_WAVE>();
            else pp_wait_dma<0>();
        } else if (group == 0) {  // step kt+1 must have landed before the barrier that opens it
            if (kt + STAGES - 1 < KT) pp_wait_dma<WAIT_STEADY>();
            else pp_wait_dma<0>();
        }
        pp_barrier();
    }
    if (group == 0) pp_barrier();
#undef SMOE_PP_ISSUE_A
#undef SMOE_PP_ISSUE_B
#undef SMOE_SLOT_A
#undef SMOE_SLOT_B

    // ---- epilogue (C layout: lane holds column lane % 16, rows 4 (lane / 16) + r) ----
    const int col_in_tile = lane & 15;
    const int row_grp = (lane >> 4) * 4;
    if constexpr (MODE == kGateUp || MODE == kGateUpSave || MODE == kLinBf16) {
        // bf16 outputs are staged through LDS (the operand ring is free once
        // every wave is past the loop) and leave in 16-byte stores of whole
        // tile rows instead of 2-byte stores that touch 32-byte pieces of four
        // rows: h (kGateUp), a, b and h (kGateUpSave, one after the other),
        // or the gated product (kLinBf16, the gate applied while staging).
        constexpr int HS = BN + 8;  // bf16 per staged row (16-byte pad)
        static_assert(BM * HS * 2 <= PPGeom<BM, BN, MODE, BK, STAGES, STAGES_A>::SMEM, "tile fits the ring");
        constexpr int NOUT = (MODE == kGateUpSave) ? 3 : 1;
        uint16_t *sh = reinterpret_cast<uint16_t *>(smem);
        constexpr int TPR = BN / 8;  // threads per row, 8 bf16 each
        const int c = (tid % TPR) * 8;
#pragma unroll
        for (int q = 0; q < NOUT; ++q) {
            __syncthreads();  // the loop's reads, or the previous output's stores, are done
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = (WM * i + wm) * 16 + row_grp + r;
                    float w = 1.0f;
                    if constexpr (MODE == kLinBf16) {
                        const int slot = min(row0 + row, row1 - 1);
                        w = p.gate ? p.gate[p.slot_src[slot]] : 1.0f;
                    }
#pragma unroll
                    for (int j = 0; j < NT; ++j) {
                        float v;
                        if constexpr (MODE == kLinBf16) {
                            v = w * acc[0][i][j][r];
                        } else {
                            const float g = acc[0][i][j][r], u = acc[1][i][j][r];
                            if (q == 0 && MODE == kGateUpSave) v = g;
                            else if (q == 1) v = u;
                            else v = (g / (1.0f + __expf(-g))) * u;  // SiLU(a) * b, as stored in h
                        }
                        sh[row * HS + wn * WTN + j * 16 + col_in_tile] = f32_to_bf16_bits(v);
                    }
                }
            __syncthreads();
            // destination: h / y rows [rows, N] (kGateUp, kLinBf16, q = 2 of kGateUpSave: C2),
            // a | b rows [rows, 2N] (kGateUpSave q = 0, 1: C)
            uint16_t *dst;
            size_t ld;
            if (MODE == kGateUpSave && q < 2) {
                dst = reinterpret_cast<uint16_t *>(p.C) + (size_t)q * N;
                ld = 2 * (size_t)N;
            } else {
                dst = reinterpret_cast<uint16_t *>(MODE == kGateUpSave ? p.C2 : p.C);
                ld = N;
            }
            for (int rb = tid / TPR; rb < BM; rb += 512 / TPR) {
                const int slot = row0 + rb;
                if (slot < row1 && n0 + c < N)
                    *reinterpret_cast<uint4 *>(dst + (size_t)slot * ld + n0 + c) =
                        *reinterpret_cast<const uint4 *>(sh + rb * HS + c);
            }
        }
        __syncthreads();  // the next tile's DMA may overwrite the staging area
        return;
    }
    if constexpr (MODE == kSwigluBwd) {
        // c = dout W2^T is staged through LDS as fp32 rows (as for kDownRows);
        // then each thread takes 8 consecutive columns of a route row: a and b
        // come in, da and db go out, as 16-byte accesses, and the row's
        // <SiLU(a) * b, c> over the tile's columns is summed over the row's
        // threads into one partial per (column tile, route)
        constexpr int YS = BN + 4;
        constexpr int SMEM = PPGeom<BM, BN, MODE, BK, STAGES, STAGES_A>::SMEM;
        constexpr int PASSES = (BM * YS * 4 <= SMEM) ? 1 : (MT % 2 == 0 && BM / 2 * YS * 4 <= SMEM) ? 2 : MT;
        static_assert(MT % PASSES == 0 && BM / PASSES * YS * 4 <= SMEM, "staged rows fit the ring");
        constexpr int MTP = MT / PASSES;
        constexpr int RP = BM / PASSES;
        constexpr int TPR = BN / 8;  // threads per row, 8 columns each (a power of two <= 64)
        static_assert(TPR <= 64 && (TPR & (TPR - 1)) == 0, "a row's threads share one wave");
        float *sy = reinterpret_cast<float *>(smem);
        const int c0 = (tid % TPR) * 8;
        __syncthreads();
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
#pragma unroll
            for (int il = 0; il < MTP; ++il)
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int j = 0; j < NT; ++j)
                        sy[((WM * il + wm) * 16 + row_grp + r) * YS + wn * WTN + j * 16 + col_in_tile] =
                            acc[0][ps * MTP + il][j][r];
            __syncthreads();
            // every thread of a row runs the same number of iterations (rows
            // are whole groups of TPR threads), so the shuffles below see all
            // of the row's lanes
            for (int rl = tid / TPR; rl < RP; rl += 512 / TPR) {
                const int slot = row0 + ps * RP + rl;
                const bool live = slot < row1 && n0 + c0 < N;  // F % 8 == 0: all 8 columns or none
                float part = 0.f;
                int f = 0;
                if (live) {
                    f = p.slot_src[slot];
                    const float w = p.gate[f];
                    uint16_t *ab = reinterpret_cast<uint16_t *>(p.C) + (size_t)slot * (2 * N) + n0 + c0;
                    const uint4 av = *reinterpret_cast<const uint4 *>(ab);
                    const uint4 bv = *reinterpret_cast<const uint4 *>(ab + N);
                    const float4 c_lo = *reinterpret_cast<const float4 *>(sy + rl * YS + c0);
                    const float4 c_hi = *reinterpret_cast<const float4 *>(sy + rl * YS + c0 + 4);
                    const uint32_t aw[4] = {av.x, av.y, av.z, av.w}, bw[4] = {bv.x, bv.y, bv.z, bv.w};
                    const float cc[8] = {c_lo.x, c_lo.y, c_lo.z, c_lo.w, c_hi.x, c_hi.y, c_hi.z, c_hi.w};
                    uint32_t da[4], db[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        uint32_t lo_a, hi_a, lo_b, hi_b;
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const float a = bf16_bits_to_f32((uint16_t)(aw[q] >> (16 * h)));
                            const float b = bf16_bits_to_f32((uint16_t)(bw[q] >> (16 * h)));
                            const float c = cc[2 * q + h];
                            const float s = 1.0f / (1.0f + __expf(-a));
                            const float silu = a * s;
                            part += silu * b * c;
                            const float dh = w * c;
                            const uint32_t xa = f32_to_bf16_bits(dh * b * s * (1.0f + a * (1.0f - s)));
                            const uint32_t xb = f32_to_bf16_bits(dh * silu);
                            if (h == 0) {
                                lo_a = xa;
                                lo_b = xb;
                            } else {
                                hi_a = xa;
                                hi_b = xb;
                            }
                        }
                        da[q] = lo_a | (hi_a << 16);
                        db[q] = lo_b | (hi_b << 16);
                    }
                    *reinterpret_cast<uint4 *>(ab) = make_uint4(da[0], da[1], da[2], da[3]);
                    *reinterpret_cast<uint4 *>(ab + N) = make_uint4(db[0], db[1], db[2], db[3]);
                }
#pragma unroll
                for (int d = TPR / 2; d >= 1; d >>= 1) part += __shfl_xor(part, d, TPR);
                if (tid % TPR == 0 && slot < row1) p.part[(size_t)nt * p.M + f] = part;
            }
            __syncthreads();
        }
        return;
    }
    if constexpr (MODE == kDownRows) {
        // the fp32 rows are staged through LDS in passes of whole 32-row
        // groups and leave as 16-byte stores of whole tile rows (BN floats of
        // route row f) instead of 4-byte stores that touch 64-byte pieces of
        // four rows; the route's gate is applied on the way out
        constexpr int YS = BN + 4;  // floats per staged row
        constexpr int SMEM = PPGeom<BM, BN, MODE, BK, STAGES, STAGES_A>::SMEM;
        constexpr int PASSES = (BM * YS * 4 <= SMEM) ? 1 : (MT % 2 == 0 && BM / 2 * YS * 4 <= SMEM) ? 2 : MT;
        static_assert(MT % PASSES == 0 && BM / PASSES * YS * 4 <= SMEM, "staged rows fit the ring");
        constexpr int MTP = MT / PASSES;  // 16-row blocks per wave and pass
        constexpr int RP = BM / PASSES;   // tile rows per pass
        constexpr int TPR = BN / 4;       // threads per row, 4 floats each
        float *sy = reinterpret_cast<float *>(smem);
        float *y = reinterpret_cast<float *>(p.C);
        const int c = (tid % TPR) * 4;
        __syncthreads();
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
#pragma unroll
            for (int il = 0; il < MTP; ++il)
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int j = 0; j < NT; ++j)
                        sy[((WM * il + wm) * 16 + row_grp + r) * YS + wn * WTN + j * 16 + col_in_tile] =
                            acc[0][ps * MTP + il][j][r];
            __syncthreads();
            for (int rl = tid / TPR; rl < RP; rl += 512 / TPR) {
                const int slot = row0 + ps * RP + rl;
                if (slot < row1 && n0 + c < N) {
                    const int f = p.slot_src[slot];
                    const float w = p.gate ? p.gate[f] : 1.0f;
                    float4 v = *reinterpret_cast<const float4 *>(sy + rl * YS + c);
                    v.x *= w;
                    v.y *= w;
                    v.z *= w;
                    v.w *= w;
                    // streaming store (measured: DS-V3 down GEMM -4.6 %, its
                    // combine -4 %; Mixtral's combine +4 us)
                    __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w},
                                                reinterpret_cast<f32x4 *>(y + (size_t)f * N + n0 + c));
                }
            }
            __syncthreads();  // before the next pass or the next tile's DMA reuses the area
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = (WM * i + wm) * 16 + row_grp + r;
            const int slot = row0 + row;
            if (slot >= row1) continue;
            // the remaining modes: the atomic down GEMM and the router logits
            // (every other mode returned from its staged epilogue above)
            if constexpr (MODE == kDown) {
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

// Whether M tile mt holds all BM rows (else pp_tile's PARTIAL form runs).
template <int BM, int MODE>
__device__ __forceinline__ bool pp_full_tile(const GemmParams &p, int mt) {
    if constexpr (MODE == kLogits) return (mt + 1) * BM <= p.M;
    const int4 t = p.tiles[mt];
    return t.z - t.y == BM;
}

// Logical block L of the order: its tile, in the short-tile form where that
// is enabled and the tile holds fewer than BM rows.
template <int BM, int BN, int MODE, int BK, int STAGES, int STAGES_A, bool SKIP_ROWS, int FLAGS>
__device__ __forceinline__ void pp_block(const GemmParams &p, char *smem, int L) {
    const uint32_t v = p.order[L];
    const int mt = (int)(v & kOrderMtMask), nt = (int)(v >> kOrderMtBits);
    if (mt >= p.n_mtiles) return;
    if (!SKIP_ROWS || pp_full_tile<BM, MODE>(p, mt))
        pp_tile<BM, BN, MODE, BK, STAGES, STAGES_A, false, FLAGS>(p, smem, mt, nt, 0, p.K / BK);
    else
        pp_tile<BM, BN, MODE, BK, STAGES, STAGES_A, true, FLAGS>(p, smem, mt, nt, 0, p.K / BK);
}

// Dynamic tile scheduling. The logical blocks 0 .. total-1 of the order are
// cut into kNumXcd contiguous queues, queue x holding [x total / 8,
// (x + 1) total / 8); the workgroups of XCD x (workgroups are dispatched to
// the XCDs round-robin by block index) claim the blocks of queue x in order,
// so the blocks that share a weight panel run together on one XCD's L2. A
// workgroup whose queue is exhausted looks at every queue's counter and
// steals from the nearest one with blocks left. Claims are agent-scope
// atomic adds on counters the tile table zeroed; every block is handed out
// exactly once, whichever workgroup or XCD takes it.
__device__ __forceinline__ int queue_begin(int q, int total) {
    return (int)(((long long)total * q) / kNumXcd);
}

// Called by all 64 lanes of one wave; returns a wave-uniform logical block,
// or total when every queue is exhausted. Each failed claim finds its queue
// exhausted (counters only grow), and the wave's own later loads of that
// counter see at least its own add, so it fails on each queue at most once:
// the loop ends after at most kNumXcd + 1 claims.
__device__ __forceinline__ int queue_claim(int *ctr, int home, int total) {
    const int lane = threadIdx.x & 63;
    int q = home;
    for (int tries = 0; tries < 4 * kNumXcd; ++tries) {
        int c = 0;
        if (lane == 0) c = atomicAdd(ctr + q * kQueueStride, 1);
        c = __builtin_amdgcn_readfirstlane(c);
        const int b = queue_begin(q, total);
        if (c < queue_begin(q + 1, total) - b) return b + c;
        int left = 0;
        if (lane < kNumXcd) {
            const int cq = __hip_atomic_load(ctr + lane * kQueueStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            left = cq < queue_begin(lane + 1, total) - queue_begin(lane, total);
        }
        const unsigned m = (unsigned)__ballot(left) & ((1u << kNumXcd) - 1u);
        if (m == 0) return total;
        const unsigned rot = ((m >> home) | (m << (kNumXcd - home))) & ((1u << kNumXcd) - 1u);
        q = (home + __builtin_ctz(rot)) % kNumXcd;
    }
    return total;
}

// Persistent tile-granular form: one workgroup per CU walks the valid
// blocks of the order, so a tile's epilogue stores drain while the same
// workgroup already streams its next tile. Without QUEUE it takes them with
// stride gridDim.x (each XCD takes one contiguous run of the order per
// round). With QUEUE (p.queue then holds the counters) it claims them
// dynamically as above: wave 4, which issues no LDS DMA (so its wait for
// the claim does not touch the DMA waves' vmcnt bookkeeping), claims the
// next block before each tile while the DMA group waits for the tile's
// first k-step to land, and hands it over through the first word of LDS
// once the tile has finished with the ring.
//
// With SKIP_ROWS, tiles holding fewer than BM rows run pp_tile's PARTIAL form
// (a second copy of the main loop). Measured, that pays where many tiles are
// short (a 192-row tile over experts of ~100-160 rows: -5 to -7 %; 256-row
// tiles over experts of ~210-300 rows: -4 %) and is neutral on the 256-row
// gate+up tile where nearly all tiles are full; other launches over mostly
// full tiles leave it off (the second loop copy has cost up to ~3 % there).
template <int BM, int BN, int MODE, int BK, int STAGES, int STAGES_A = STAGES, bool SKIP_ROWS = false, int FLAGS = 0,
          bool QUEUE = false>
__global__ __launch_bounds__(512) void grouped_gemm_pp_persistent_kernel(const GemmParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[PPGeom<BM, BN, MODE, BK, STAGES, STAGES_A>::SMEM];
    const int total = (*p.valid_mtiles) * p.n_ntiles;
    if constexpr (!QUEUE) {
        const int G = gridDim.x;
        for (int L = xcd_remap(blockIdx.x, G); L < total; L += G)
            pp_block<BM, BN, MODE, BK, STAGES, STAGES_A, SKIP_ROWS, FLAGS>(p, smem, L);
        return;
    }
    const int home = blockIdx.x % kNumXcd;
    const bool claimer = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 4;  // wave-uniform branch
    int *handoff = reinterpret_cast<int *>(smem);
    int next = 0;
    if (claimer) next = queue_claim(p.queue, home, total);
    // every round but the last runs a block no other round runs
    for (;;) {
        if (claimer && (threadIdx.x & 63) == 0) *handoff = next;
        __syncthreads();
        const int L = __builtin_amdgcn_readfirstlane(*handoff);  // uniform: tile fields stay scalar
        __syncthreads();  // the hand-off slot is part of the ring the tile's DMA fills
        if (L >= total) break;
        if (claimer) next = queue_claim(p.queue, home, total);
        pp_block<BM, BN, MODE, BK, STAGES, STAGES_A, SKIP_ROWS, FLAGS>(p, smem, L);
        __syncthreads();  // every wave is done with the ring before the slot is written
    }
}

// Persistent stream-K form for the down GEMM, whose epilogue is an atomic
// add (so a tile's K range may be split between workgroups: each part adds
// its partial sum). The valid blocks of the order table, each cut into
// K / BK k-steps, form one sequence of work units; workgroup b (in
// XCD-contiguous order) takes units [U b / G, U (b + 1) / G) and runs every
// (tile, k-range) piece of it. This removes the idle tail of the last wave of
// tiles and evens out experts of different sizes.
template <int BM, int BN, int BK, int STAGES>
__global__ __launch_bounds__(512) void grouped_gemm_pp_streamk_kernel(const GemmParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[PPGeom<BM, BN, kDown, BK, STAGES>::SMEM];
    const int KT = p.K / BK;
    const int valid_mtiles = min(*p.valid_mtiles, p.n_mtiles);
    const long units = (long)valid_mtiles * p.n_ntiles * KT;
    const int G = gridDim.x;
    const int b = xcd_remap(blockIdx.x, G);
    long u = units * b / G;
    const long u_end = units * (b + 1) / G;
    while (u < u_end) {
        const int L = (int)(u / KT);
        const int ks = (int)(u - (long)L * KT);
        const int ke = (int)min((long)KT, (long)ks + (u_end - u));
        const uint32_t v = p.order[L];
        const int mt = (int)(v & kOrderMtMask), nt = (int)(v >> kOrderMtBits);
        if (mt < p.n_mtiles) pp_tile<BM, BN, kDown, BK, STAGES>(p, smem, mt, nt, ks, ke);
        u += ke - ks;
    }
}

}  // namespace smoe
