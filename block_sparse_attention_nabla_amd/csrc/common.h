// common.h -- small device helpers shared by the gfx950 NABLA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nabla {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// Native 16-byte vector (HIP's uint4 is a wrapper struct that register
// promotion does not always see through when held in arrays).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kBlockN = 64;  // tokens per block (N)

// log2(e): softmax is evaluated with exp2 and the scale pre-multiplied by it.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// One 32x32x16 bf16 MFMA, fp32 accumulate. Operand layout used throughout:
//   A (32 x 16): lane l supplies row (l % 32), 8 k-slots from k-group (l / 32);
//   B (16 x 32): lane l supplies column (l % 32), 8 k-slots from k-group (l / 32);
//   C (32 x 32): lane l holds column (l % 32), rows 8*(r/4) + 4*(l/32) + r%4, r = 0..15.
// The kernels pair A's and B's (k-group, slot) positions consistently, so the
// contraction is correct whatever order the hardware gives the k index.
__device__ __forceinline__ f32x16_t mfma_32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Pack two fp32 to two bf16 (round-to-nearest-even), low half = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2_t r;
    r[0] = (__bf16)a;
    r[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ f32x16_t zero16() {
    f32x16_t z;
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = 0.f;
    return z;
}

// Row of the 32x32 C tile held in register r by a lane in lane-half h.
__device__ __forceinline__ constexpr int c_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

}  // namespace nabla
