// Shared device helpers for the gfx950 (CDNA4) MoE kernels: bf16 packing,
// the bf16 MFMA tile op, the swizzled LDS tile layout and the 8x8 register
// transpose that turns row-major weight blocks into K-contiguous MFMA
// operands.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smoe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, 32 CUs each

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).
// Lane l supplies row (l % 16) of A and column (l % 16) of B, each as 8
// consecutive K values starting at K = 8 * (l / 16) -- any K order works as
// long as A and B use the same one. D: lane l holds column (l % 16), rows
// 4 * (l / 16) + {0, 1, 2, 3}.
__device__ __forceinline__ f32x4 mfma_16x16x32(const uint4 &a, const uint4 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).
// Lane l supplies row (l % 32) of A and column (l % 32) of B, each as 8
// consecutive K values starting at K = 8 * (l / 32). D: lane l holds column
// (l % 32), value v at row 8 (v / 4) + 4 (l / 32) + v % 4.
__device__ __forceinline__ f32x16 mfma_32x32x16(const uint4 &a, const uint4 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// LDS tile of rows that are 64 bf16 (128 B = 8 chunks of 16 B) long. The
// chunk index is XORed with (row & 7) so that 8 lanes reading the same chunk
// of 8 consecutive rows (the MFMA operand pattern) and 8 lanes writing the 8
// chunks of one row both hit 8 distinct 16-byte bank groups.
__device__ __forceinline__ int lds_off(int row, int chunk) { return (row << 7) + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ uint32_t u4_get(const uint4 &v, int i) {
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// 8x8 transpose of 16-bit values held as 8 rows of 8: out[c] = column c.
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t lo = u4_get(in[2 * j], c >> 1);
            const uint32_t hi = u4_get(in[2 * j + 1], c >> 1);
            o[j] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        out[c] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// Buffer resource over [base, base + bytes): loads past the end return zero
// instead of faulting. Word 3 is the CDNA raw-buffer format (32-bit data,
// no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

// Workgroups are dispatched to the 8 XCDs round-robin by block index. Map
// physical block ids so that each XCD receives one contiguous range of
// logical tile ids: neighbouring tiles then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    const int q = nblocks / kNumXcd, r = nblocks % kNumXcd;
    const int xcd = bid % kNumXcd, pos = bid / kNumXcd;
    return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + pos;
}

}  // namespace smoe
