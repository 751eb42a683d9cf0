// sage_attn_bf16.hip -- unquantised comparison path for gfx950: the same
// softmax(Q K^T sm_scale) V read straight from strided bf16 Q/K/V views, with
// BF16 MFMA (v_mfma_f32_32x32x16_bf16) for S^T = K Q^T and O^T = V^T P^T and an
// fp32 online softmax over 64-key tiles.  P is rounded to bf16 for the product.
//
// Inputs are the projection-strided NHD views of
// "gb10-sage-strided-nhd-summary-1344x768-124f-seed440420.json" (dataflow:
// no Q/K/V materialisation) or any other [B, N, H, D] view; the output is
// written token-major (dataflow.attention_output).
//
// Layout per wave mirrors the quantised kernel: K is the A operand and Q^T the
// B operand, so each lane holds one query and 16 keys of every 32-key block;
// those values are, unchanged, the P^T B operand of the second product once V
// is staged transposed ([channel][key]) in LDS.  For k-step ks (16 keys) lane
// half u element j pairs with key 16*ks + 8*(j/4) + 4*u + j%4.
#include "sage_common.h"

namespace sage {

namespace {

constexpr int kWaves = 4;
constexpr int kQWg = 32 * kWaves;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2E = 1.4426950408889634f;

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// K tile [64 keys][128 ch] bf16 = 16 chunks of 16 B per row, XOR-swizzled.
__device__ __forceinline__ int k_slot(int r, int c) { return r * 16 + (c ^ (r & 15)); }
// V^T tile [128 ch][64 keys] bf16 = 16 units of 8 B per row, XOR-swizzled.
__device__ __forceinline__ int v_unit(int d, int u) { return d * 16 + (u ^ ((d ^ (d >> 4)) & 15)); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __int_as_float(r[0]) + __int_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    v2bf r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
}

struct Prefetch {
    uint4 k[4];   // K rows t/16 + 16*i, channels 8*(t%16)..+7
    uint4 v[4];   // V keys 4*(t/16) + i, channels 8*(t%16)..+7
};

__device__ __forceinline__ void load_tile(Prefetch &p, const View &K, const View &V, int64_t koff, int64_t voff,
                                          int key0, int N, int t) {
    const int row = t >> 4, seg = t & 15;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        int nk = key0 + row + 16 * i;
        int nv = key0 + 4 * row + i;
        p.k[i] = nk < N ? *reinterpret_cast<const uint4 *>(K.data + koff + (int64_t)nk * K.sn + seg * 8)
                        : make_uint4(0, 0, 0, 0);
        p.v[i] = nv < N ? *reinterpret_cast<const uint4 *>(V.data + voff + (int64_t)nv * V.sn + seg * 8)
                        : make_uint4(0, 0, 0, 0);
    }
}

__device__ __forceinline__ void store_tile(const Prefetch &p, uint4 *lk, uint2 *lv, int t) {
    const int row = t >> 4, seg = t & 15;
#pragma unroll
    for (int i = 0; i < 4; i++) lk[k_slot(row + 16 * i, seg)] = p.k[i];
    // transpose 4 keys x 8 channels: channel c gets keys 4*row..4*row+3 (8 bytes)
    uint32_t w[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        w[i][0] = p.v[i].x; w[i][1] = p.v[i].y; w[i][2] = p.v[i].z; w[i][3] = p.v[i].w;
    }
#pragma unroll
    for (int c = 0; c < 8; c++) {
        const int sh = (c & 1) ? 16 : 0;
        uint32_t e0 = (w[0][c >> 1] >> sh) & 0xFFFFu, e1 = (w[1][c >> 1] >> sh) & 0xFFFFu;
        uint32_t e2 = (w[2][c >> 1] >> sh) & 0xFFFFu, e3 = (w[3][c >> 1] >> sh) & 0xFFFFu;
        lv[v_unit(seg * 8 + c, row)] = make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
    }
}

template <bool TAIL>
__device__ __forceinline__ void tile_step(const uint4 *lk, const uint2 *lv, const v8bf (&qa)[8], float c2,
                                          int nvalid, int hl, int ql, float &m2, float &lsum, v16f (&o)[4]) {
    v16f s[2];
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
        s[kb] = v16f{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int st = 0; st < 8; st++) {
            v8bf ka = __builtin_bit_cast(v8bf, lk[k_slot(32 * kb + ql, 2 * st + hl)]);
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qa[st], s[kb], 0, 0, 0);
        }
    }
    if (TAIL) {
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                int key = 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
                if (key >= nvalid) s[kb][r] = -INFINITY;
            }
    }
    float smax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int r = 0; r < 16; r++) smax = fmaxf(smax, s[kb][r]);
    smax = pair_max(smax);
    const float mnew = fmaxf(m2, c2 * smax);
    const float alpha = fast_exp2(m2 - mnew);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < 4; db++)
#pragma unroll
            for (int r = 0; r < 16; r++) o[db][r] *= alpha;
    }
    m2 = mnew;

    // P^T operand for k-step ks = 2*kb + half: registers 8*half .. 8*half+7 of block kb.
    uint32_t pw[16];
    float part = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            float p0 = fast_exp2(c2 * s[kb][r] - mnew);
            float p1 = fast_exp2(c2 * s[kb][r + 1] - mnew);
            part += p0 + p1;
            pw[(16 * kb + r) >> 1] = pack_bf16(p0, p1);
        }
    lsum += part;

#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
        v8bf pb = __builtin_bit_cast(v8bf, make_uint4(pw[4 * ks], pw[4 * ks + 1], pw[4 * ks + 2], pw[4 * ks + 3]));
#pragma unroll
        for (int db = 0; db < 4; db++) {
            const int d = 32 * db + ql;
            uint2 lo = lv[v_unit(d, 4 * ks + hl)];       // keys 16ks + 4hl + 0..3
            uint2 hi = lv[v_unit(d, 4 * ks + 2 + hl)];   // keys 16ks + 8 + 4hl + 0..3
            v8bf va = __builtin_bit_cast(v8bf, make_uint4(lo.x, lo.y, hi.x, hi.y));
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[db], 0, 0, 0);
        }
    }
}

__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(View Q, View K, View V, int N, int H, float c2,
                                                               OutView out, int nqwg) {
    __shared__ uint4 lk[2][64 * 16];
    __shared__ uint2 lv[2][128 * 16];

    const uint32_t id = xcd_remap(blockIdx.x, gridDim.x);
    const int qb = (int)(id % (uint32_t)nqwg);
    const int64_t bh = id / (uint32_t)nqwg;
    const int b = (int)(bh / H), h = (int)(bh % H);
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, hl = lane >> 5, ql = lane & 31;
    const int q0 = qb * kQWg + 32 * w;
    const int n = q0 + ql;

    v8bf qa[8];
    {
        const uint16_t *qrow = Q.data + (int64_t)b * Q.sb + (int64_t)h * Q.sh + (int64_t)n * Q.sn + 8 * hl;
#pragma unroll
        for (int st = 0; st < 8; st++)
            qa[st] = __builtin_bit_cast(
                v8bf, n < N ? *reinterpret_cast<const uint4 *>(qrow + 16 * st) : make_uint4(0, 0, 0, 0));
    }
    const int64_t koff = (int64_t)b * K.sb + (int64_t)h * K.sh;
    const int64_t voff = (int64_t)b * V.sb + (int64_t)h * V.sh;
    const int ntiles = (N + kTile - 1) / kTile;
    const int tail_valid = N - (ntiles - 1) * kTile;

    v16f o[4];
#pragma unroll
    for (int db = 0; db < 4; db++) o[db] = v16f{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    float m2 = -INFINITY, lsum = 0.0f;

    Prefetch pre;
    load_tile(pre, K, V, koff, voff, 0, N, t);
    store_tile(pre, lk[0], lv[0], t);
    __syncthreads();
    for (int tt = 0; tt < ntiles; tt++) {
        const int buf = tt & 1;
        const bool more = tt + 1 < ntiles;
        if (more) load_tile(pre, K, V, koff, voff, (tt + 1) * kTile, N, t);
        if (more || tail_valid == kTile)
            tile_step<false>(lk[buf], lv[buf], qa, c2, kTile, hl, ql, m2, lsum, o);
        else
            tile_step<true>(lk[buf], lv[buf], qa, c2, tail_valid, hl, ql, m2, lsum, o);
        if (more) store_tile(pre, lk[buf ^ 1], lv[buf ^ 1], t);
        __syncthreads();
    }

    const float inv = 1.0f / pair_sum(lsum);
    if (n < N) {
        uint16_t *orow = out.data + (int64_t)b * out.sb + (int64_t)n * out.sn + (int64_t)h * out.sh;
#pragma unroll
        for (int db = 0; db < 4; db++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int d0 = 32 * db + 8 * g + 4 * hl;
                uint32_t lo = f32_to_bf16(o[db][4 * g] * inv) | (f32_to_bf16(o[db][4 * g + 1] * inv) << 16);
                uint32_t hi = f32_to_bf16(o[db][4 * g + 2] * inv) | (f32_to_bf16(o[db][4 * g + 3] * inv) << 16);
                *reinterpret_cast<uint2 *>(orow + d0) = make_uint2(lo, hi);
            }
    }
}

}  // namespace

hipError_t launch_attn_fwd_bf16(View q, View k, View v, int B, int N, int H, float sm_scale, OutView out,
                                hipStream_t stream) {
    const int nqwg = (N + kQWg - 1) / kQWg;
    const int64_t blocks = (int64_t)nqwg * H * B;
    hipLaunchKernelGGL(attn_bf16_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, q, k, v, N, H,
                       sm_scale * kLog2E, out, nqwg);
    return hipGetLastError();
}

}  // namespace sage
