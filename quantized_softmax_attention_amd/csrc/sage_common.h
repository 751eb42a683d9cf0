// sage_common.h -- device-side helpers shared by the gfx950 kernels of
// libsage_mi355x.so.  Constants come from the public header; nothing here is
// shared with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sage_mi355x.h"

namespace sage {

constexpr int kD = SAGE_HEAD_DIM;       // 128 channels per head
constexpr int kQBlock = SAGE_Q_BLOCK;   // 32 tokens per Q scale
constexpr int kKBlock = SAGE_K_BLOCK;   // 64 tokens per K scale
constexpr int kTile = SAGE_P_TILE;      // 64 keys per softmax step
constexpr int kNAlign = SAGE_N_ALIGN;   // code buffers padded to 256 tokens
constexpr int kSumChunk = 64;           // tokens per fp64 partial sum of K
constexpr int kVChunk = 256;            // tokens per partial |V| channel max

static_assert(kKBlock == kTile, "one K scale per softmax tile");

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Strided [B, N, H, D] bf16 view as seen by the kernels (element strides).
struct View {
    const uint16_t *data;
    int64_t sb, sn, sh;
};

struct OutView {
    uint16_t *data;
    int64_t sb, sn, sh;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even fp32 -> bf16 (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// OCP E4M3FN encoding of an fp32 value: round to nearest, ties to even;
// magnitudes >= 448 saturate to 448; the sign of zero is kept.  Integer-only
// so the result does not depend on the conversion unit's rounding modes.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
    uint32_t bits = __float_as_uint(y);
    uint32_t sign = (bits >> 24) & 0x80u;
    uint32_t mag = bits & 0x7FFFFFFFu;
    uint32_t code;
    if (mag >= 0x43E00000u) {                 // |y| >= 448 (and NaN/Inf): saturate
        code = 0x7Eu;
    } else if (mag < 0x3C800000u) {           // |y| < 2^-6: subnormal grid of 2^-9
        float a = __uint_as_float(mag) * 512.0f;   // exact (power-of-two scaling)
        code = (uint32_t)__builtin_rintf(a);       // 0..8; 8 encodes 2^-6
    } else {
        uint32_t e = (mag >> 23) - 127u + 7u;      // biased E4M3 exponent, 1..15
        uint32_t m = mag & 0x7FFFFFu;
        uint32_t r = (m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20;   // RNE to 3 bits, 0..8
        code = (e << 3) + r;                       // r == 8 carries into the exponent
        if (code > 0x7Eu) code = 0x7Eu;
    }
    return sign | code;
}

// Workgroup index remap so that the workgroups one XCD receives (hardware
// dispatch is round-robin over the 8 XCDs) form one contiguous range of the
// logical grid: XCD x works on logical ids [x*n/8, (x+1)*n/8).  Identity when
// n is not a multiple of 8.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t id, uint32_t n) {
    if (n % 8u) return id;
    return (id % 8u) * (n / 8u) + id / 8u;
}

}  // namespace sage
