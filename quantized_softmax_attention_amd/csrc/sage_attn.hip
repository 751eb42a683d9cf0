// sage_attn.hip -- fused quantised attention forward for gfx950:
// INT8 MFMA for S^T = K Q^T, fp32 online softmax, FP8 (E4M3) MFMA for O^T = V^T P^T.
//
// The stage is attention_forward of "gb10-sampling-component-profile-1344x768-
// 124f-seed440420.json" (attention_internal_p50_milliseconds.sage2); the page
// "gb10-sage2-p0-interleave-softmax-latency.json" times it alone and prints the
// GB10 schedule (scheduler: 64-key steps, 32-query warps).  That schedule is prior
// art for another chip; this kernel is laid out for CDNA4's 64-wide waves:
//
//  * Transposed products.  With K as the A operand and Q as the B operand of
//    v_mfma_i32_32x32x32_i8, the 32x32 accumulator gives each lane ONE query
//    (lane % 32) and 16 keys, so row maxima and sums are in-lane reductions plus
//    one exchange between lane l and l^32.  The same lane then holds exactly the
//    P^T values the B operand of v_mfma_scale_f32_32x32x64_f8f6f4 needs (32 keys
//    of one query), so P never travels through LDS.  V codes are stored by the
//    quantiser with the matching key order (kappa in the public header).
//  * One wave = 32 queries (one Q scale block) x 64 keys (one K scale block) per
//    step: the whole QK^T dequantisation is one scalar c = sq * sk * sm_scale *
//    log2(e) per step, and the running maximum is taken on the int32 scores.
//  * Four waves (128 queries) share each 8 KB K tile and 8 KB V tile in LDS,
//    double buffered, XOR-swizzled so the 16-byte fragment reads are free of
//    bank conflicts.  Workgroups are remapped so each XCD streams whole heads.
//
// Reading of the method (tile-relative P rounding, sum of unrounded P): for each
// 64-key tile, p' = 2^(c*a - m + log2 448) ~ 448 * exp(s - m) relative to the
// running maximum m after that tile; p' is summed in fp32 before it is rounded
// to E4M3 for the FP8 product, and the output is acc * sv / sum(p').
#include "sage_common.h"

namespace sage {

namespace {

constexpr int kWaves = 4;                  // waves per workgroup
constexpr int kQWg = 32 * kWaves;          // queries per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kTileBytes = kTile * kD;     // 8 KB per K tile and per V tile
constexpr int kChunks = kTileBytes / 16;   // 512 16-byte chunks per tile
constexpr float kLog2E = 1.4426950408889634f;
constexpr float kLog2_448 = 8.807354922057604f;

// LDS slot of 16-byte chunk c (0..7) of K row r (0..63).
__device__ __forceinline__ int k_slot(int r, int c) { return r * 8 + (c ^ ((r ^ (r >> 3)) & 7)); }
// LDS slot of 16-byte chunk c (0..3) of V channel row d (0..127).
__device__ __forceinline__ int v_slot(int d, int c) { return d * 4 + (c ^ (((d >> 1) ^ (d >> 3)) & 3)); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// v_permlane32_swap exchanges the upper half-wave of its first operand with the
// lower half-wave of its second.  With both operands x, one result holds x of
// lanes 0..31 in every lane position l % 32 and the other x of lanes 32..63, so
// combining the two gives every lane the value of its pair (l, l ^ 32).
__device__ __forceinline__ int pair_max(int x) {
    auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return max((int)r[0], (int)r[1]);
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __int_as_float(r[0]) + __int_as_float(r[1]);
}

struct Prefetch {
    v4i k0, k1, v0, v1;
};

__device__ __forceinline__ void load_tile(Prefetch &p, const int8_t *ktile, const uint8_t *vtile, int t) {
    p.k0 = reinterpret_cast<const v4i *>(ktile)[t];
    p.k1 = reinterpret_cast<const v4i *>(ktile)[t + kThreads];
    p.v0 = reinterpret_cast<const v4i *>(vtile)[t];
    p.v1 = reinterpret_cast<const v4i *>(vtile)[t + kThreads];
}

__device__ __forceinline__ void store_tile(const Prefetch &p, v4i *lk, v4i *lv, int t) {
    int g0 = t, g1 = t + kThreads;
    lk[k_slot(g0 >> 3, g0 & 7)] = p.k0;
    lk[k_slot(g1 >> 3, g1 & 7)] = p.k1;
    lv[v_slot(g0 >> 2, g0 & 3)] = p.v0;
    lv[v_slot(g1 >> 2, g1 & 3)] = p.v1;
}

// One 64-key step for one wave.  TAIL masks keys >= nvalid (last tile only).
template <bool TAIL>
__device__ __forceinline__ void tile_step(const v4i *lk, const v4i *lv, const v4i (&qa)[4], float cq,
                                          float ksc, int nvalid, int hl, int ql, float &m2, float &lsum,
                                          v16f (&o)[4]) {
    // S^T = K Q^T: two 32-key blocks, four 32-channel k-steps each.
    v16i s[2];
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
        s[kb] = v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int st = 0; st < 4; st++) {
            v4i ka = lk[k_slot(32 * kb + ql, 2 * st + hl)];
            s[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka, qa[st], s[kb], 0, 0, 0);
        }
    }
    // Lane (hl, ql) register r of block kb holds key 32*kb + 8*(r/4) + 4*hl + r%4.
    if (TAIL) {
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                int key = 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
                if (key >= nvalid) s[kb][r] = INT32_MIN;
            }
    }
    int imax = INT32_MIN;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int r = 0; r < 16; r++) imax = max(imax, s[kb][r]);
    imax = pair_max(imax);

    const float c2 = cq * ksc;                       // log2-domain scale of this step
    const float mnew = fmaxf(m2, c2 * (float)imax);  // c2 >= 0: monotone in a
    const float alpha = fast_exp2(m2 - mnew);        // 0 on the first step
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {   // wave-uniform; skip when no max moved
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < 4; db++)
#pragma unroll
            for (int r = 0; r < 16; r++) o[db][r] *= alpha;
    }
    m2 = mnew;
    const float bias = mnew - kLog2_448;

    // p' = 448 * exp(s - m) in fp32; sum before rounding; pack to E4M3.
    v8i pf;
    float part = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
            // registers r..r+3 -> operand bytes j = 16*kb + r .. +3 (one dword)
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                p[i] = fast_exp2(c2 * (float)s[kb][r + i] - bias);
                if (TAIL && 32 * kb + 8 * (r >> 2) + 4 * hl + i >= nvalid) p[i] = 0.0f;
            }
            part += (p[0] + p[1]) + (p[2] + p[3]);
            int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
            pf[(16 * kb + r) >> 2] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wd, true);
        }
    lsum += part;

    // O^T += V^T P^T, 32 channels per MFMA.
#pragma unroll
    for (int db = 0; db < 4; db++) {
        const int d = 32 * db + ql;
        v4i lo = lv[v_slot(d, 2 * hl)];
        v4i hi = lv[v_slot(d, 2 * hl + 1)];
        v8i va = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pf, o[db], 0, 0, 0, 127, 0, 127);
    }
}

__global__ __launch_bounds__(kThreads, 2) void attn_i8f8_kernel(
    const int8_t *__restrict__ qc, const float *__restrict__ qs, const int8_t *__restrict__ kc,
    const float *__restrict__ ks, const uint8_t *__restrict__ vc, const float *__restrict__ vs, int N,
    int H, int64_t Npad, float c_base, OutView out, int nqwg) {
    __shared__ v4i lds[2][2][kChunks];   // [buffer][K, V][chunk]

    const uint32_t id = xcd_remap(blockIdx.x, gridDim.x);
    const int qb = (int)(id % (uint32_t)nqwg);
    const int64_t bh = id / (uint32_t)nqwg;
    const int b = (int)(bh / H), h = (int)(bh % H);
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, hl = lane >> 5, ql = lane & 31;
    const int q0 = qb * kQWg + 32 * w;

    // Q^T operand: lane (hl, ql) holds query q0+ql, channels 32*st + 16*hl .. +15.
    const int8_t *qrow = qc + (bh * Npad + q0 + ql) * kD + 16 * hl;
    v4i qa[4];
#pragma unroll
    for (int st = 0; st < 4; st++) qa[st] = *reinterpret_cast<const v4i *>(qrow + 32 * st);
    const float cq = qs[bh * (Npad / kQBlock) + q0 / kQBlock] * c_base;
    const float *ksb = ks + bh * (Npad / kKBlock);
    const int8_t *kbase = kc + bh * Npad * kD;
    const uint8_t *vbase = vc + bh * (Npad / kTile) * (int64_t)kTileBytes;

    const int ntiles = (N + kTile - 1) / kTile;
    const int tail_valid = N - (ntiles - 1) * kTile;

    v16f o[4];
#pragma unroll
    for (int db = 0; db < 4; db++)
        o[db] = v16f{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    float m2 = -INFINITY, lsum = 0.0f;

    Prefetch pre;
    load_tile(pre, kbase, vbase, t);
    store_tile(pre, lds[0][0], lds[0][1], t);
    __syncthreads();

    for (int tt = 0; tt < ntiles; tt++) {
        const int buf = tt & 1;
        const bool more = tt + 1 < ntiles;
        if (more) load_tile(pre, kbase + (int64_t)(tt + 1) * kTileBytes, vbase + (int64_t)(tt + 1) * kTileBytes, t);
        const float ksc = ksb[tt];
        if (tt + 1 < ntiles || tail_valid == kTile)
            tile_step<false>(lds[buf][0], lds[buf][1], qa, cq, ksc, kTile, hl, ql, m2, lsum, o);
        else
            tile_step<true>(lds[buf][0], lds[buf][1], qa, cq, ksc, tail_valid, hl, ql, m2, lsum, o);
        if (more) store_tile(pre, lds[buf ^ 1][0], lds[buf ^ 1][1], t);
        __syncthreads();
    }

    // Epilogue: the two lanes of a query hold different keys' partial sums.
    const float ltot = pair_sum(lsum);
    const float inv = 1.0f / ltot;
    const int n = q0 + ql;
    if (n < N) {
        const float *svp = vs + bh * kD;
        uint16_t *orow = out.data + (int64_t)b * out.sb + (int64_t)n * out.sn + (int64_t)h * out.sh;
#pragma unroll
        for (int db = 0; db < 4; db++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int d0 = 32 * db + 8 * g + 4 * hl;   // registers 4g..4g+3: channels d0..d0+3
                const float sv[4] = {svp[d0], svp[d0 + 1], svp[d0 + 2], svp[d0 + 3]};
                uint32_t lo = f32_to_bf16(o[db][4 * g] * sv[0] * inv) |
                              (f32_to_bf16(o[db][4 * g + 1] * sv[1] * inv) << 16);
                uint32_t hi = f32_to_bf16(o[db][4 * g + 2] * sv[2] * inv) |
                              (f32_to_bf16(o[db][4 * g + 3] * sv[3] * inv) << 16);
                *reinterpret_cast<uint2 *>(orow + d0) = make_uint2(lo, hi);
            }
    }
}

}  // namespace

hipError_t launch_attn_fwd(const int8_t *qc, const float *qs, const int8_t *kc, const float *ks, const uint8_t *vc,
                           const float *vs, int B, int N, int H, float sm_scale, OutView out, hipStream_t stream) {
    const int64_t Npad = ((int64_t)N + kNAlign - 1) / kNAlign * kNAlign;
    const int nqwg = (N + kQWg - 1) / kQWg;
    const int64_t blocks = (int64_t)nqwg * H * B;
    hipLaunchKernelGGL(attn_i8f8_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, qc, qs, kc, ks, vc, vs,
                       N, H, Npad, sm_scale * kLog2E, out, nqwg);
    return hipGetLastError();
}

}  // namespace sage
