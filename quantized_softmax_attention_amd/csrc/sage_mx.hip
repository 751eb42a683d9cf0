// sage_mx.hip -- OCP microscaling (MX) blocks of a bf16 tensor for gfx950: the
// format the projection after attention consumes (see sage_mx_quantize in the
// public header).  HBM-bound: each thread reads one 32-channel block (64 bytes)
// and writes its 32 (E4M3) or 16 (E2M1) code bytes and one scale byte.
#include "sage_common.h"

#pragma clang fp contract(off)

namespace sage {

template <int FMT>
__global__ __launch_bounds__(256) void mx_quantize_kernel(View x, int N, int H, int64_t nblocks,
                                                          uint8_t *__restrict__ codes, uint8_t *__restrict__ scales) {
    const int64_t L = (int64_t)blockIdx.x * 256 + threadIdx.x;   // block index, token-major
    if (L >= nblocks) return;
    const int per_token = H * (kD / kMxBlock);
    const int64_t bn = L / per_token;
    const int r = (int)(L % per_token), h = r / (kD / kMxBlock), db = r % (kD / kMxBlock);
    const int64_t b = bn / N, n = bn % N;
    const uint4 *src = reinterpret_cast<const uint4 *>(x.data + b * x.sb + n * x.sn + (int64_t)h * x.sh + kMxBlock * db);
    float v[kMxBlock];
    float amax = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const uint4 raw = src[q];
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int j = 0; j < 8; j++) {
            v[8 * q + j] = bf16_to_f32((j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xFFFFu));
            amax = fmaxf(amax, fabsf(v[8 * q + j]));
        }
    }
    const int X = mx_shared_exp(amax, FMT == kMxE4M3 ? 8 : 2);
    const float sc = pow2f(-X);
    scales[L] = (uint8_t)(X + 127);
    if (FMT == kMxE4M3) {
        uint32_t wd[8];
#pragma unroll
        for (int k = 0; k < 8; k++)
            wd[k] = e4m3_encode(v[4 * k] * sc) | (e4m3_encode(v[4 * k + 1] * sc) << 8) |
                    (e4m3_encode(v[4 * k + 2] * sc) << 16) | (e4m3_encode(v[4 * k + 3] * sc) << 24);
        uint4 *dst = reinterpret_cast<uint4 *>(codes + L * kMxBlock);
        dst[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
        dst[1] = make_uint4(wd[4], wd[5], wd[6], wd[7]);
    } else {
        uint32_t wd[4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            uint32_t acc = 0;
#pragma unroll
            for (int i = 0; i < 8; i++) acc |= e2m1_encode(v[8 * k + i] * sc) << (4 * i);
            wd[k] = acc;
        }
        *reinterpret_cast<uint4 *>(codes + L * (kMxBlock / 2)) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
}

hipError_t launch_mx_quantize(View x, int B, int N, int H, int fmt, uint8_t *codes, uint8_t *scales,
                              hipStream_t stream) {
    const int64_t nblocks = (int64_t)B * N * H * (kD / kMxBlock);
    const dim3 grid((unsigned)((nblocks + 255) / 256));
    if (fmt == kMxE4M3)
        LAUNCH_OR_RETURN(mx_quantize_kernel<kMxE4M3>, grid, dim3(256), 0, stream, x, N, H, nblocks, codes, scales);
    else
        LAUNCH_OR_RETURN(mx_quantize_kernel<kMxE2M1>, grid, dim3(256), 0, stream, x, N, H, nblocks, codes, scales);
    return hipSuccess;
}

}  // namespace sage
