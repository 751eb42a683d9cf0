// sage_quant.hip -- the quantisation stages of the SageAttention2-style forward
// for gfx950: K smoothing statistic, INT8 Q/K blocks, E4M3 V channels.
//
// Stages as named on "gb10-sampling-component-profile-1344x768-124f-seed440420.json",
// attention_internal_p50_milliseconds.sage2 (qk_quantize, v_quantize,
// framework_and_k_smoothing_estimate).  Inputs are strided [B, N, H, D] bf16 views
// ("gb10-sage-strided-nhd-summary-...json", dataflow.qkv_input): every kernel
// reads whole 256-byte head rows, so packed-projection views need no copy.
//
// All kernels here are HBM-bound.  Their results are bit-exact by definition:
// no FMA contraction, IEEE fp32 division, fixed fp64 summation order.
#include "sage_common.h"

#pragma clang fp contract(off)

namespace sage {

// ------------------------------------------------------------------ K mean
// Partial sums: thread (chunk c, channel group seg) adds its 8 channels over the
// chunk's 64 tokens in ascending order in fp64 (bf16 widens exactly).  A
// workgroup covers 16 chunks of one head; the 16 threads of a chunk read whole
// 256-byte head rows.
__global__ __launch_bounds__(256) void kmean_partial_kernel(View k, int N, int H, int nchunk,
                                                            double *__restrict__ ws) {
    const int h = blockIdx.y, b = blockIdx.z;
    const int c = blockIdx.x * 16 + (threadIdx.x >> 4), seg = threadIdx.x & 15;
    if (c >= nchunk) return;
    const uint16_t *base = k.data + (int64_t)b * k.sb + (int64_t)h * k.sh + seg * 8;
    const int n0 = c * kSumChunk, n1 = min(N, n0 + kSumChunk);
    double s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 8
    for (int n = n0; n < n1; n++) {
        const uint4 raw = *reinterpret_cast<const uint4 *>(base + (int64_t)n * k.sn);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int j = 0; j < 8; j++)
            s[j] += (double)bf16_to_f32((j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xFFFFu));
    }
    double *dst = ws + (((int64_t)b * nchunk + c) * H + h) * kD + seg * 8;
#pragma unroll
    for (int j = 0; j < 8; j++) dst[j] = s[j];
}

// Total over chunks in ascending order, one fp64 division by N, one rounding.
// The adds are a dependent chain, so loads are issued 32 at a time ahead of it.
__global__ __launch_bounds__(256) void kmean_final_kernel(const double *__restrict__ ws, int N, int H,
                                                          int nchunk, int B, float *__restrict__ km) {
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    int64_t HD = (int64_t)H * kD;
    if (i >= (int64_t)B * HD) return;
    int64_t b = i / HD, hd = i % HD;
    const double *p = ws + b * nchunk * HD + hd;
    double s = 0.0;
    int c = 0;
    for (; c + 32 <= nchunk; c += 32) {
        double v[32];
#pragma unroll
        for (int j = 0; j < 32; j++) v[j] = p[(int64_t)(c + j) * HD];
#pragma unroll
        for (int j = 0; j < 32; j++) s += v[j];
    }
    for (; c < nchunk; c++) s += p[(int64_t)c * HD];
    km[i] = (float)(s / (double)N);
}

// ------------------------------------------------------------- INT8 blocks
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ uint32_t int8_code(float x, float scale) {
    if (scale == 0.0f) return 0u;
    float r = __builtin_rintf(x / scale);          // IEEE division, ties to even
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (uint32_t)((int32_t)r) & 0xFFu;
}

// One workgroup per (64-token block tb, head h, batch b): two Q blocks of 32
// tokens and one K block of 64.  Thread t holds channels 8*(t%16)..+7 of tokens
// t/16 + 16*i, i = 0..3.  Tokens >= N load as zero, which changes no block
// maximum and yields zero codes, so padded rows need no special case.
__global__ __launch_bounds__(256) void quant_qk_kernel(View q, View k, int N, int H, int64_t Npad,
                                                       const float *__restrict__ km,
                                                       int8_t *__restrict__ qc, float *__restrict__ qs,
                                                       int8_t *__restrict__ kc, float *__restrict__ ks) {
    __shared__ float red[3][4];
    const int tb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int t = threadIdx.x, row = t >> 4, seg = t & 15, lane = t & 63, wave = t >> 6;
    const int64_t bh = (int64_t)b * H + h;
    const uint16_t *qb = q.data + (int64_t)b * q.sb + (int64_t)h * q.sh + seg * 8;
    const uint16_t *kb = k.data + (int64_t)b * k.sb + (int64_t)h * k.sh + seg * 8;
    float mean[8];
#pragma unroll
    for (int j = 0; j < 8; j++) mean[j] = km[bh * kD + seg * 8 + j];

    float xq[4][8], xk[4][8];
    float mq0 = 0.0f, mq1 = 0.0f, mk = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        int n = tb * 64 + row + 16 * i;
        uint4 rq = make_uint4(0, 0, 0, 0), rk = make_uint4(0, 0, 0, 0);
        bool valid = n < N;
        if (valid) {
            rq = *reinterpret_cast<const uint4 *>(qb + (int64_t)n * q.sn);
            rk = *reinterpret_cast<const uint4 *>(kb + (int64_t)n * k.sn);
        }
        uint32_t wq[4] = {rq.x, rq.y, rq.z, rq.w}, wk[4] = {rk.x, rk.y, rk.z, rk.w};
#pragma unroll
        for (int j = 0; j < 8; j++) {
            uint32_t bq = (j & 1) ? (wq[j >> 1] >> 16) : (wq[j >> 1] & 0xFFFFu);
            uint32_t bk = (j & 1) ? (wk[j >> 1] >> 16) : (wk[j >> 1] & 0xFFFFu);
            xq[i][j] = bf16_to_f32(bq);
            xk[i][j] = valid ? bf16_to_f32(bk) - mean[j] : 0.0f;
            if (i < 2) mq0 = fmaxf(mq0, fabsf(xq[i][j]));
            else mq1 = fmaxf(mq1, fabsf(xq[i][j]));
            mk = fmaxf(mk, fabsf(xk[i][j]));
        }
    }
    mq0 = wave_max(mq0);
    mq1 = wave_max(mq1);
    mk = wave_max(mk);
    if (lane == 0) {
        red[0][wave] = mq0;
        red[1][wave] = mq1;
        red[2][wave] = mk;
    }
    __syncthreads();
    float aq0 = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    float aq1 = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
    float ak = fmaxf(fmaxf(red[2][0], red[2][1]), fmaxf(red[2][2], red[2][3]));
    float sq0 = aq0 / 127.0f, sq1 = aq1 / 127.0f, sk = ak / 127.0f;

#pragma unroll
    for (int i = 0; i < 4; i++) {
        int64_t n = (int64_t)tb * 64 + row + 16 * i;
        float sq = i < 2 ? sq0 : sq1;
        uint32_t cq[2] = {0, 0}, ck[2] = {0, 0};
#pragma unroll
        for (int j = 0; j < 8; j++) {
            cq[j >> 2] |= int8_code(xq[i][j], sq) << (8 * (j & 3));
            ck[j >> 2] |= int8_code(xk[i][j], sk) << (8 * (j & 3));
        }
        int64_t off = (bh * Npad + n) * kD + seg * 8;
        *reinterpret_cast<uint2 *>(qc + off) = make_uint2(cq[0], cq[1]);
        *reinterpret_cast<uint2 *>(kc + off) = make_uint2(ck[0], ck[1]);
    }
    if (t == 0) {
        qs[bh * (Npad / kQBlock) + 2 * tb] = sq0;
        qs[bh * (Npad / kQBlock) + 2 * tb + 1] = sq1;
        ks[bh * (Npad / kKBlock) + tb] = sk;
    }
}

// ---------------------------------------------------------- V to E4M3
// Partial channel maxima of |v| over 256-token chunks: ws[b][c][h][d].
__global__ __launch_bounds__(256) void v_amax_partial_kernel(View v, int N, int H, int nchunk,
                                                             float *__restrict__ ws) {
    __shared__ float red[16][kD + 4];
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int t = threadIdx.x, row = t >> 4, seg = t & 15;
    const uint16_t *base = v.data + (int64_t)b * v.sb + (int64_t)h * v.sh + seg * 8;
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 4
    for (int i = 0; i < kVChunk / 16; i++) {
        int n = c * kVChunk + row + 16 * i;
        if (n < N) {
            uint4 raw = *reinterpret_cast<const uint4 *>(base + (int64_t)n * v.sn);
            uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int j = 0; j < 8; j++) {
                uint32_t bits = (j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xFFFFu);
                m[j] = fmaxf(m[j], fabsf(bf16_to_f32(bits)));
            }
        }
    }
#pragma unroll
    for (int j = 0; j < 8; j++) red[row][seg * 8 + j] = m[j];
    __syncthreads();
    if (t < kD) {
        float a = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; r++) a = fmaxf(a, red[r][t]);
        ws[(((int64_t)b * nchunk + c) * H + h) * kD + t] = a;
    }
}

// Channel amax over chunks -> amax[b][h][d] and v_scale = amax / 448.
__global__ __launch_bounds__(256) void v_amax_final_kernel(const float *__restrict__ ws, int H, int nchunk,
                                                           int B, float *__restrict__ amax,
                                                           float *__restrict__ vs) {
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    int64_t HD = (int64_t)H * kD;
    if (i >= (int64_t)B * HD) return;
    int64_t b = i / HD, hd = i % HD;
    const float *p = ws + b * nchunk * HD + hd;
    float a = 0.0f;
    int c = 0;
    for (; c + 32 <= nchunk; c += 32) {   // loads issued 32 at a time (max is exact in any order)
        float v[32];
#pragma unroll
        for (int j = 0; j < 32; j++) v[j] = p[(int64_t)(c + j) * HD];
#pragma unroll
        for (int j = 0; j < 32; j++) a = fmaxf(a, v[j]);
    }
    for (; c < nchunk; c++) a = fmaxf(a, p[(int64_t)c * HD]);
    amax[i] = a;
    vs[i] = a / 448.0f;
}

// One workgroup per (64-key tile t, head h, batch b).  Thread (g = tid/16,
// seg = tid%16) encodes keys 4g..4g+3 of channels 8*seg..+7.  The four codes
// of one channel land in consecutive bytes p0..p0+3 of the tile row, where p0
// inverts kappa (see the public header): keys 4g..4g+3 sit at
// p0 = 32*(g%2) + 16*(g/8) + 4*((g/2)%4).  The 8 KB tile is assembled in LDS
// and written out with coalesced 16-byte stores.
__global__ __launch_bounds__(256) void quant_v_kernel(View v, int N, int H, int64_t Npad,
                                                      const float *__restrict__ vs,
                                                      uint8_t *__restrict__ vc) {
    __shared__ uint32_t tile[kD][kTile / 4];
    const int tt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int t = threadIdx.x, g = t >> 4, seg = t & 15;
    const int64_t bh = (int64_t)b * H + h;
    const uint16_t *base = v.data + (int64_t)b * v.sb + (int64_t)h * v.sh + seg * 8;
    float sv[8];
#pragma unroll
    for (int j = 0; j < 8; j++) sv[j] = vs[bh * kD + seg * 8 + j];
    uint32_t packed[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        int n = tt * kTile + 4 * g + i;
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (n < N) raw = *reinterpret_cast<const uint4 *>(base + (int64_t)n * v.sn);
        uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int j = 0; j < 8; j++) {
            uint32_t bits = (j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xFFFFu);
            uint32_t code = (sv[j] == 0.0f || n >= N) ? 0u : e4m3_encode(bf16_to_f32(bits) / sv[j]);
            packed[j] |= code << (8 * i);
        }
    }
    const int p0 = 32 * (g & 1) + 16 * (g >> 3) + 4 * ((g >> 1) & 3);
#pragma unroll
    for (int j = 0; j < 8; j++) tile[seg * 8 + j][p0 >> 2] = packed[j];
    __syncthreads();
    uint4 *dst = reinterpret_cast<uint4 *>(vc + (bh * (Npad / kTile) + tt) * (int64_t)(kD * kTile));
    const uint4 *src = reinterpret_cast<const uint4 *>(&tile[0][0]);
    dst[t] = src[t];
    dst[t + 256] = src[t + 256];
}

// ------------------------------------------------------------ launchers
hipError_t launch_quantize_qk(View q, View k, int B, int N, int H, int8_t *qc, float *qs, int8_t *kc,
                              float *ks, float *km, void *workspace, hipStream_t stream) {
    const int nchunk = (N + kSumChunk - 1) / kSumChunk;
    const int64_t Npad = ((int64_t)N + kNAlign - 1) / kNAlign * kNAlign;
    double *ws = static_cast<double *>(workspace);
    hipLaunchKernelGGL(kmean_partial_kernel, dim3((nchunk + 15) / 16, H, B), dim3(256), 0, stream, k, N, H, nchunk,
                       ws);
    int64_t total = (int64_t)B * H * kD;
    hipLaunchKernelGGL(kmean_final_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, ws, N,
                       H, nchunk, B, km);
    hipLaunchKernelGGL(quant_qk_kernel, dim3((unsigned)(Npad / 64), H, B), dim3(256), 0, stream, q, k, N, H,
                       Npad, km, qc, qs, kc, ks);
    return hipGetLastError();
}

hipError_t launch_quantize_v(View v, int B, int N, int H, uint8_t *vc, float *vs, void *workspace,
                             hipStream_t stream) {
    const int nchunk = (N + kVChunk - 1) / kVChunk;
    const int64_t Npad = ((int64_t)N + kNAlign - 1) / kNAlign * kNAlign;
    float *part = static_cast<float *>(workspace);
    float *amax = part + (int64_t)nchunk * B * H * kD;
    hipLaunchKernelGGL(v_amax_partial_kernel, dim3(nchunk, H, B), dim3(256), 0, stream, v, N, H, nchunk, part);
    int64_t total = (int64_t)B * H * kD;
    hipLaunchKernelGGL(v_amax_final_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, part, H,
                       nchunk, B, amax, vs);
    hipLaunchKernelGGL(quant_v_kernel, dim3((unsigned)(Npad / kTile), H, B), dim3(256), 0, stream, v, N, H, Npad,
                       vs, vc);
    return hipGetLastError();
}

}  // namespace sage
