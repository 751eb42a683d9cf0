// sage_common.h -- device-side helpers shared by the gfx950 kernels of
// libsage_mi355x.so.  Constants come from the public header; nothing here is
// shared with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

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

// ---- OCP microscaling (MX, Microscaling Formats v1.0) blocks of 32 values
// Shared exponent of a block whose largest magnitude is amax (finite, >= 0):
// floor(log2 amax) - emax_elem clamped to [-127, 127], and -127 when amax is 0
// or below the fp32 normal range (the clamp would give -127 there anyway).
__device__ __forceinline__ int mx_shared_exp(float amax, int emax_elem) {
    const uint32_t ebits = __float_as_uint(amax) >> 23;
    if (ebits == 0) return -127;
    return max(-127, min(127, (int)ebits - 127 - emax_elem));
}

// 2^n for n in [-126, 127].
__device__ __forceinline__ float pow2f(int n) { return __uint_as_float((uint32_t)(n + 127) << 23); }

// E2M1 (FP4): nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6, ties to the even code,
// saturating at 6; bit 3 carries the sign (also of zero).
__device__ __forceinline__ uint32_t e2m1_encode(float y) {
    const float a = fabsf(y);
    const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
    return c | ((__float_as_uint(y) >> 28) & 8u);
}

constexpr int kMxE4M3 = SAGE_MX_E4M3, kMxE2M1 = SAGE_MX_E2M1;
constexpr int kMxBlock = 32;

// Workgroup index remap so that the workgroups one XCD receives (hardware
// dispatch is round-robin over the 8 XCDs) form one contiguous range of the
// logical grid: XCD x works on logical ids [x*n/8, (x+1)*n/8).  Identity when
// n is not a multiple of 8.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t id, uint32_t n) {
    if (n % 8u) return id;
    return (id % 8u) * (n / 8u) + id / 8u;
}

// kernel<<<grid, block, shmem, stream>>>(args...) through hipLaunchKernel,
// returning that launch's own status.  (hipGetLastError() after a launch would
// also report, and clear, an error left by the caller's earlier HIP work.)  The
// arguments are converted to the kernel's parameter types first, as a direct
// launch converts them.
template <typename... P, size_t... I>
hipError_t launch_packed(void (*kernel)(P...), dim3 grid, dim3 block, size_t shmem, hipStream_t stream,
                         std::index_sequence<I...>, std::tuple<P...> &args) {
    void *ptrs[sizeof...(P) > 0 ? sizeof...(P) : 1] = {static_cast<void *>(&std::get<I>(args))...};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, ptrs, shmem, stream);
}

template <typename... P, typename... A>
hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, size_t shmem, hipStream_t stream, A &&...args) {
    static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
    std::tuple<P...> packed(std::forward<A>(args)...);
    return launch_packed(kernel, grid, block, shmem, stream, std::index_sequence_for<P...>{}, packed);
}

// In a launcher returning hipError_t: launch, and return the status if it failed.
#define LAUNCH_OR_RETURN(kernel, ...)                                   \
    do {                                                                \
        const hipError_t launch_status_ = ::sage::launch(kernel, __VA_ARGS__); \
        if (launch_status_ != hipSuccess) return launch_status_;        \
    } while (0)

}  // namespace sage
