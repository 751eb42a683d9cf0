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
#include "sage_norm_rope.h"

#include <utility>

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

// ------------------------------------------- reductions over chunk partials
// The per-chunk partials (fp64 K column sums and/or fp32 V column maxima) are
// rows of H*kD values, one row per chunk of tokens, for each batch entry.  One
// workgroup reduces 32 columns over all chunks: its 256 threads stage 64 chunk
// rows at a time in LDS (thread t loads rows t/32 + 8j of column t%32, so each
// load is a 256-byte row segment per 32 lanes, and sixteen loads per thread are
// in flight), double buffered so the next rows load while this batch is reduced;
// lanes 0..31 of wave 0 add their column's sums in ascending chunk order (the
// order the K mean is defined in), lanes 32..63 take the maxima (exact in any
// order).  Results: km = (float)(sum / N) (one fp64 division, one rounding);
// amax and v_scale = amax / 448.
constexpr int kColsPerWg = 32;
constexpr int kRowsPerBatch = 64;

template <bool SUM, bool MAX>
__global__ __launch_bounds__(256) void chunk_final_kernel(const double *__restrict__ wsk,
                                                          const float *__restrict__ wsv, int N, int H,
                                                          int nchunk, float *__restrict__ km,
                                                          float *__restrict__ amax, float *__restrict__ vs) {
    __shared__ double lk[SUM ? 2 : 1][SUM ? kRowsPerBatch : 1][kColsPerWg];
    __shared__ float lv[MAX ? 2 : 1][MAX ? kRowsPerBatch : 1][kColsPerWg];
    const int t = threadIdx.x, col = t % kColsPerWg, r0 = t / kColsPerWg;
    const int64_t HD = (int64_t)H * kD;
    const int wpb = 4 * H;                                         // workgroups per batch entry
    const int b = (int)(blockIdx.x / wpb);
    const int64_t c0 = (int64_t)(blockIdx.x % wpb) * kColsPerWg;   // first column of this workgroup
    const double *pk = SUM ? wsk + (int64_t)b * nchunk * HD + c0 + col : nullptr;
    const float *pv = MAX ? wsv + (int64_t)b * nchunk * HD + c0 + col : nullptr;
    const int nb = (nchunk + kRowsPerBatch - 1) / kRowsPerBatch;
    double xk[kRowsPerBatch / 8];
    float xv[kRowsPerBatch / 8];
    auto load = [&](int batch) {
#pragma unroll
        for (int j = 0; j < kRowsPerBatch / 8; j++) {
            const int c = batch * kRowsPerBatch + r0 + 8 * j;
            if (SUM) xk[j] = c < nchunk ? pk[(int64_t)c * HD] : 0.0;
            if (MAX) xv[j] = c < nchunk ? pv[(int64_t)c * HD] : 0.0f;
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int j = 0; j < kRowsPerBatch / 8; j++) {
            if (SUM) lk[buf][r0 + 8 * j][col] = xk[j];
            if (MAX) lv[buf][r0 + 8 * j][col] = xv[j];
        }
    };
    load(0);
    store(0);
    __syncthreads();
    double s = 0.0;
    float a = 0.0f;
    for (int i = 0; i < nb; i++) {
        if (i + 1 < nb) load(i + 1);
        const int rows = min(kRowsPerBatch, nchunk - i * kRowsPerBatch);
        if (SUM && t < kColsPerWg)
            for (int r = 0; r < rows; r++) s += lk[i & 1][r][t];
        if (MAX && t >= kColsPerWg && t < 2 * kColsPerWg)
            for (int r = 0; r < rows; r++) a = fmaxf(a, lv[i & 1][r][t - kColsPerWg]);
        if (i + 1 < nb) store((i + 1) & 1);
        __syncthreads();
    }
    const int64_t o = (int64_t)b * HD + c0;
    if (SUM && t < kColsPerWg) km[o + t] = (float)(s / (double)N);
    if (MAX && t >= kColsPerWg && t < 2 * kColsPerWg) {
        amax[o + t - kColsPerWg] = a;
        vs[o + t - kColsPerWg] = a / 448.0f;
    }
}

// 8 consecutive channels of one token row as raw bf16 (a 16-byte load); zeros
// when !valid.
__device__ __forceinline__ uint4 load_raw8(const uint16_t *p, bool valid) {
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (valid) raw = *reinterpret_cast<const uint4 *>(p);
    return raw;
}

// 8 packed bf16 values (channel order) widened exactly to fp32.
__device__ __forceinline__ void widen8(uint4 v, float (&x)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; j++) {
        x[2 * j] = __uint_as_float(w[j] << 16);
        x[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
}

// The raw rows of tokens tb * 64 + row + 16 i (i = 0..3) of head h of a view,
// thread (row, seg) = (t / 16, t % 16) holding channels 8 seg..+7.
__device__ __forceinline__ void load_block_raw(View a, int b, int h, int tb, int N, uint4 (&raw)[4]) {
    const int t = threadIdx.x, row = t >> 4, seg = t & 15;
    const uint16_t *base = a.data + (int64_t)b * a.sb + (int64_t)h * a.sh + seg * 8;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int n = tb * 64 + row + 16 * i;
        raw[i] = load_raw8(base + (int64_t)n * a.sn, n < N);
    }
}

// ------------------------------------------------ RMSNorm + RoPE of Q and K
// "gb10-sage-strided-nhd-summary-1344x768-124f-seed440420.json",
// dataflow.qk_transform: Q and K pass through RMSNorm and rotary embedding on
// their strided views before quantisation.  Per (b, n, h) row of D = 128:
//   ss = sum_d x_d^2, exact, rounded once to fp32 (nearest even),
//   r = 1 / sqrt(ss / D + eps),  y_d = (x_d * r) * gamma_d,
//   channel pairs (2i, 2i+1) turned by the token's angle: (a c - b s, a s + b c),
// rounded once to bf16.  The 16 threads of a row are 16 consecutive lanes
// (seg = lane % 16, channels 8*seg..+7).  No contraction (see the pragma above)
// after ss: every product and sum is rounded to fp32, so the result is
// bit-exactly defined.

// Lane-permuted copy of a within each 16-lane row (DPP; all lanes active).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t a) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, CTRL, 0xF, 0xF, false);
}
// (mov_dpp: every lane is written by these patterns, so no old value is needed.)
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double a) {
    const uint64_t u = __double_as_longlong(a);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Reductions over the 16 lanes of a row with DPP: quad permutations reach the
// xor-1 and xor-2 partners; once each quad holds one value, the half-row mirror
// reaches a lane of the other quad of the half-row, and once each half-row holds
// one value, the row mirror reaches the other half.  Every lane ends with the
// row's result.
__device__ __forceinline__ uint32_t row16_min_u32(uint32_t a) {
    a = min(a, dpp_u32<0xB1>(a));    // quad_perm [1, 0, 3, 2]
    a = min(a, dpp_u32<0x4E>(a));    // quad_perm [2, 3, 0, 1]
    a = min(a, dpp_u32<0x141>(a));   // row_half_mirror
    a = min(a, dpp_u32<0x140>(a));   // row_mirror
    return a;
}
__device__ __forceinline__ double row16_sum_f64(double a) {
    a = a + dpp_f64<0xB1>(a);
    a = a + dpp_f64<0x4E>(a);
    a = a + dpp_f64<0x141>(a);
    a = a + dpp_f64<0x140>(a);
    return a;
}

// ---- ss: the exact sum of a row's squares, rounded once to fp32
// A bf16 value is +-M * 2^(E - 134) with E its exponent field and M <= 255 (the
// hidden bit included; a subnormal reads as E = 1 without it), so its square is
// M^2 * 2^(2E - 268).
//  * Fast path: every square is a multiple of 2^(2 E_min - 268), E_min the
//    smallest exponent among the row's nonzero values, and every partial sum of
//    the squares (all positive) is at most their total, below 2^(e + 1) where e is
//    the binary exponent of the computed fp64 sum (rounding can only raise it).
//    If e + 1 - (2 E_min - 268) <= 53, every partial sum fits 53 bits: the fp64
//    sum was exact, in any order, and one conversion rounds it.
//  * Other rows (a nonzero value about 2^15 or more below the row's largest: about
//    one Gaussian row in a hundred) add the squares as integers in LDS, 18 32-bit
//    words in units of 2^-266 (512 squares of the largest bf16 stay below
//    2^531), by atomic adds whose carries ripple upward, and round the total.
constexpr int kSqWords = 18;

// The exact total of the words at w (this row group's 18 LDS words), rounded
// to fp32: 24 significant bits or the bits at or above 2^-149 (word bit 117),
// nearest even; the fp32 bit pattern (q carries into the exponent by itself).
__device__ uint32_t sq_words_to_f32(const uint32_t *w) {
    int t = -1;
    for (int i = kSqWords - 1; i >= 0 && t < 0; i--) {
        const uint32_t v = w[i];
        if (v) t = 32 * i + 31 - __builtin_clz(v);
    }
    if (t < 0) return 0u;
    const int p = max(t - 23, 117), pm = p - 1;            // pm: the rounding bit
    const int w0 = pm >> 5, sh = pm & 31;
    const uint64_t win = (((uint64_t)w[w0 + 1] << 32) | w[w0]) >> sh;   // bits pm .. pm + 32 + (31 - sh)
    bool sticky = (w[w0] & ((1u << sh) - 1u)) != 0u;
    for (int i = 0; i < w0; i++) sticky = sticky || w[i] != 0u;
    uint32_t q = (uint32_t)(win >> 1) & 0x1FFFFFFu;         // bits p .. t (t - p <= 23)
    if ((win & 1u) && (sticky || (q & 1u))) q++;
    const uint32_t bits = ((uint32_t)(p - 117) << 23) + q;
    return bits >= 0x7F800000u ? 0x7F800000u : bits;
}

// The slow path for one row group (all 16 of its lanes active, 8 values each);
// a call, not inlined per row: it is rare, and its code would otherwise repeat
// in every row of every kernel that normalises.  The row is passed by value
// (registers): an array reference would put it in scratch memory for the call.
struct Row8 {
    float v[8];
};
__device__ __attribute__((noinline)) float ss_exact_lds(Row8 x, uint32_t *w, int seg) {
    w[seg] = 0u;
    if (seg < kSqWords - 16) w[16 + seg] = 0u;
    __builtin_amdgcn_s_waitcnt(0xC07F);                    // lgkmcnt(0): the zeros are in LDS
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const uint32_t u = __float_as_uint(x.v[j]);
        uint32_t e = (u >> 23) & 0xFFu, m = (u >> 16) & 0x7Fu;
        if (e == 0u && m == 0u) continue;
        if (e == 0u) e = 1u;
        else m |= 0x80u;
        const uint32_t sq = m * m;                         // < 2^16
        const int s = 2 * (int)e - 2, wi = s >> 5, off = s & 31;
        const uint32_t lo = sq << off, hi = off > 16 ? sq >> (32 - off) : 0u;
        uint32_t old = atomicAdd(&w[wi], lo);
        uint32_t v = hi + (uint32_t)(old + lo < old);      // the carry out of the low word
        for (int k = wi + 1; v != 0u && k < kSqWords; k++) {
            old = atomicAdd(&w[k], v);
            v = (uint32_t)(old + v < old);
        }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
    return __uint_as_float(sq_words_to_f32(w));
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// The smallest nonzero bf16 magnitude field (15 bits, ordered like the values)
// of 8 packed values, minus one; 0xFFFF when all are zero.  Packed 16-bit
// integer operations, two values per instruction: a zero field minus one wraps
// to 0xFFFF and never sets the minimum.
__device__ __forceinline__ uint32_t min_nonzero_mag_minus1(uint4 raw) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    u16x2 m = u16x2{0xFFFF, 0xFFFF};
#pragma unroll
    for (int j = 0; j < 4; j++)
        m = __builtin_elementwise_min(m, __builtin_bit_cast(u16x2, w[j] & 0x7FFF7FFFu) - u16x2{1, 1});
    return min((uint32_t)m.x, (uint32_t)m.y);
}

// ss of one row whose 8 values this lane holds (all 16 lanes of the row call it).
__device__ __forceinline__ float row_sum_squares(uint4 raw, uint32_t *words, int seg) {
    float x[8];
    widen8(raw, x);
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const double d = (double)x[j];
        s = __builtin_fma(d, d, s);                         // the squares are exact in fp64
    }
    const uint32_t lo = row16_min_u32(min_nonzero_mag_minus1(raw));
    s = row16_sum_f64(s);
    if (lo == 0xFFFFu) return 0.0f;                         // an all-zero row
    const int emin = max((int)((lo + 1u) >> 7), 1);          // subnormals count as exponent 1
    const int e = (int)(__double_as_longlong(s) >> 52) - 1023;   // s >= 2^-266 > 0: a normal fp64
    if (e + 1 - (2 * emin - 268) <= 53) return (float)s;   // exact fp64 sum, rounded once
    Row8 r;
#pragma unroll
    for (int j = 0; j < 8; j++) r.v[j] = x[j];
    return ss_exact_lds(r, words, seg);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// 8 fp32 values as bf16 (round to nearest even: the conversion instruction), packed
// in channel order.
__device__ __forceinline__ uint4 pack_bf16x8(const float (&x)[8]) {
    auto pk = [](float a, float b) { return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a, (__bf16)b}); };
    return make_uint4(pk(x[0], x[1]), pk(x[2], x[3]), pk(x[4], x[5]), pk(x[6], x[7]));
}


// v from lane I of this lane's 16-lane group (ds_swizzle bit mode within 32
// lanes: source lane = (lane & 0x10) | I).
template <int I>
__device__ __forceinline__ float group_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x10 | (I << 5)));
}
template <int... I>
__device__ __forceinline__ void group_bcast_all(float v, float *out, std::integer_sequence<int, I...>) {
    ((out[I] = group_bcast<I>(v)), ...);
}

// This lane's 8 weights (channels 8 seg..+7) of one gamma vector.
struct Gamma8 {
    float g[8];
};
__device__ __forceinline__ Gamma8 load_gamma8(const float *gamma) {
    const int seg = threadIdx.x & 15;
    const float4 g0 = *reinterpret_cast<const float4 *>(gamma + 8 * seg);
    const float4 g1 = *reinterpret_cast<const float4 *>(gamma + 8 * seg + 4);
    return Gamma8{{g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w}};
}

// The rotary (cos, sin) of this lane's channel pairs 4 seg..4 seg+3 for token n;
// tokens >= N read row N - 1 (their outputs are zeros).
struct Rope8 {
    float cs[8];
};
__device__ __forceinline__ Rope8 load_rope8(const NormRope &nr, int n, int N) {
    const int seg = threadIdx.x & 15;
    const int nc = min(n, N - 1);
    const float4 *tr = reinterpret_cast<const float4 *>(nr.rope + ((int64_t)nc * (kD / 2) + 4 * seg) * 2);
    const float4 t0 = tr[0], t1 = tr[1];
    return Rope8{{t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w}};
}

// The transform of R rows held by this lane (8 channels each, raw bf16; row i
// belongs to token n[i], has norm factor r[i] and uses weights ga for i < R / 2,
// gb for the others), as bf16, zeros for tokens >= N.  Each weight vector is loaded once;
// rows of one token share their rotary loads.
template <int R>
__device__ __forceinline__ void rope_rows(const uint4 (&raw)[R], const float (&r)[R], const float *ga,
                                          const float *gb, const int (&n)[R], const NormRope &nr, int N,
                                          uint4 (&out)[R]) {
    const Gamma8 g[2] = {load_gamma8(ga), load_gamma8(gb)};
    Rope8 cs[R];
#pragma unroll
    for (int i = 0; i < R; i++) cs[i] = load_rope8(nr, n[i], N);
#pragma unroll
    for (int i = 0; i < R; i++) {
        const float *gi = g[i < R / 2 ? 0 : 1].g;
        float x[8], y[8], z[8];
        widen8(raw[i], x);
#pragma unroll
        for (int j = 0; j < 8; j++) y[j] = (x[j] * r[i]) * gi[j];
#pragma unroll
        for (int p = 0; p < 4; p++) {
            const float c = cs[i].cs[2 * p], sn = cs[i].cs[2 * p + 1];
            z[2 * p] = y[2 * p] * c - y[2 * p + 1] * sn;
            z[2 * p + 1] = y[2 * p] * sn + y[2 * p + 1] * c;
        }
        const uint4 v = pack_bf16x8(z);
        const uint32_t keep = n[i] < N ? 0xFFFFFFFFu : 0u;      // a mask, not a branch
        out[i] = make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
    }
}

// rope_rows with the norm factors computed here: r = 1/sqrt(ss/D + eps) of each
// row (returned in r).  Must be called by all 16 lanes of the rows' group.  r is
// evaluated once per row rather than once per lane: lane seg computes it for row
// seg % R and every lane reads row i's from lane i of its 16-lane group (a
// ds_swizzle broadcast); the value is the same, as every lane holds the same ss.
template <int R>
__device__ __forceinline__ void norm_rope_rows(const uint4 (&raw)[R], const float *ga, const float *gb,
                                               const int (&n)[R], const NormRope &nr, int N, uint4 (&out)[R],
                                               float (&r)[R]) {
    static_assert(R == 4 || R == 8, "rows per lane");
    __shared__ uint32_t sq_words[16][kSqWords];            // per 16-lane row group (256 threads)
    const int seg = threadIdx.x & 15;
    uint32_t *words = sq_words[(threadIdx.x >> 4) & 15];
    float ss[R];
#pragma unroll
    for (int i = 0; i < R; i++) ss[i] = row_sum_squares(raw[i], words, seg);
    float a = ss[0];
#pragma unroll
    for (int i = 1; i < R; i++) a = (seg % R == i) ? ss[i] : a;
    const float rsel = 1.0f / __builtin_sqrtf(a / (float)kD + nr.eps);
    group_bcast_all(rsel, r, std::make_integer_sequence<int, R>{});
    rope_rows<R>(raw, r, ga, gb, n, nr, N, out);
}

// The (64-token block, head, batch) of a workgroup in a 1-D grid of H * nblk * B
// workgroups: heads vary fastest and the XCD remap hands each XCD a contiguous
// range, so the workgroups of one token block, which read the same rows of the
// rotary table, run on one XCD and find those rows in its L2.
struct TokHead {
    int tb, h, b;
};
__device__ __forceinline__ TokHead tok_head(int H, int nblk) {
    const uint32_t id = xcd_remap(blockIdx.x, gridDim.x);
    return TokHead{(int)((id / (uint32_t)H) % (uint32_t)nblk), (int)(id % (uint32_t)H),
                   (int)(id / ((uint32_t)H * (uint32_t)nblk))};
}

// In place on the Q and K views: one workgroup per (64-token block, head,
// batch); thread (row, seg) transforms tokens row + 16 i of both.  All loads
// are issued before the first store (the views may share a buffer).
__global__ __launch_bounds__(256) void norm_rope_kernel(OutView q, OutView k, int N, int H, NormRope nr) {
    const TokHead w = tok_head(H, (N + 63) / 64);
    const int tb = w.tb, h = w.h, b = w.b;
    const int t = threadIdx.x, row = t >> 4, seg = t & 15;
    uint16_t *qb = q.data + (int64_t)b * q.sb + (int64_t)h * q.sh + seg * 8;
    uint16_t *kb = k.data + (int64_t)b * k.sb + (int64_t)h * k.sh + seg * 8;
    uint4 x[8];             // rows 0-3: Q of tokens row + 16 i; rows 4-7: K of the same tokens
    int n[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        n[i] = n[4 + i] = tb * 64 + row + 16 * i;
        x[i] = load_raw8(qb + (int64_t)n[i] * q.sn, n[i] < N);
        x[4 + i] = load_raw8(kb + (int64_t)n[i] * k.sn, n[i] < N);
    }
    uint4 y[8];
    float r[8];
    norm_rope_rows<8>(x, nr.gamma_q, nr.gamma_k, n, nr, N, y, r);
#pragma unroll
    for (int i = 0; i < 4; i++)
        if (n[i] < N) {
            *reinterpret_cast<uint4 *>(qb + (int64_t)n[i] * q.sn) = y[i];
            *reinterpret_cast<uint4 *>(kb + (int64_t)n[i] * k.sn) = y[4 + i];
        }
}

// ------------------------------------------------------------- INT8 blocks
// The wave's largest value of a non-negative float (no NaN): the bit patterns of
// such floats order like the values, so integer maxima decide it: DPP within each
// 16-lane row, then the four rows' results read as scalars.
__device__ __forceinline__ float wave_max_nonneg(float v) {
    uint32_t a = __float_as_uint(v);
    a = max(a, dpp_u32<0xB1>(a));    // quad_perm [1, 0, 3, 2]
    a = max(a, dpp_u32<0x4E>(a));    // quad_perm [2, 3, 0, 1]
    a = max(a, dpp_u32<0x141>(a));   // row_half_mirror
    a = max(a, dpp_u32<0x140>(a));   // row_mirror
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)a, 0);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)a, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)a, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)a, 48);
    return __uint_as_float(max(max(r0, r1), max(r2, r3)));
}

// The codes are defined on the IEEE quotient x / scale.  Per element it is
// computed as x * inv corrected once (Markstein): with inv = RN(1/scale) (one
// IEEE division per scale), q0 = RN(x * inv) and the exact residual
// r = x - q0 * scale (an fma), RN(q0 + r * inv) is the correctly rounded quotient
// whenever q0 and r stay normal; the sign of zero is restored.  For scales
// >= kFastDivMin the residual can only underflow when |x / scale| < 2^-22, far
// below the first boundary of either encoding (0.5 for INT8, 2^-10 for E4M3), so
// the codes equal those of the IEEE quotient (tests/fast_div_check.c checks it on
// every bf16 value and on random fp32 values, ties and subnormals, for scales
// across the exponent range, codes of both formats).  Smaller scales use the IEEE
// division.
constexpr float kFastDivMin = 0x1p-80f;

__device__ __forceinline__ float div_rn(float x, float scale, float inv) {
    const float q0 = x * inv;
    const float r = __builtin_fmaf(-q0, scale, x);
    return __builtin_copysignf(__builtin_fmaf(r, inv, q0), x);
}

// INT8 code of x / scale (IEEE division): ties to even, clamped to [-127, 127]; 0
// when scale is 0.  The path for blocks whose scale is below kFastDivMin.
__device__ __forceinline__ uint32_t int8_code(float x, float scale) {
    if (scale == 0.0f) return 0u;
    float r = __builtin_rintf(x / scale);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (uint32_t)((int32_t)r) & 0xFFu;
}

// Workgroup-wide maxima of M non-negative per-thread values (256 threads, 4
// waves) with one barrier pair; red is M x 4 floats of LDS.  Every thread gets
// every maximum.
template <int M>
__device__ __forceinline__ void block_maxes(float (&m)[M], float (*red)[4]) {
#pragma unroll
    for (int i = 0; i < M; i++) m[i] = wave_max_nonneg(m[i]);
    if ((threadIdx.x & 63) == 0)
#pragma unroll
        for (int i = 0; i < M; i++) red[i][threadIdx.x >> 6] = m[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < M; i++) m[i] = fmaxf(fmaxf(red[i][0], red[i][1]), fmaxf(red[i][2], red[i][3]));
    __syncthreads();
}

// The INT8 blocks of one 64-token block tb of one head, thread t holding
// channels 8*(t%16)..+7 of tokens t/16 + 16*i, i = 0..3 (tokens >= N hold
// zeros, which changes no block maximum and yields zero codes).  Q: two 32-token
// blocks (i < 2 and i >= 2); K: one 64-token block.
//
// The largest |v| of packed bf16 rows I0 <= i < I1, as fp32: the 15-bit magnitude
// fields compared as 16-bit integers, two per instruction (they order like the
// magnitudes for every non-NaN value).
template <int I0, int I1>
__device__ __forceinline__ float absmax_bf16_rows(const uint4 (&rows)[4]) {
    u16x2 m = u16x2{0, 0};
#pragma unroll
    for (int i = I0; i < I1; i++) {
        const uint32_t w[4] = {rows[i].x, rows[i].y, rows[i].z, rows[i].w};
#pragma unroll
        for (int j = 0; j < 4; j++) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[j] & 0x7FFF7FFFu));
    }
    return __uint_as_float(max((uint32_t)m.x, (uint32_t)m.y) << 16);
}
__device__ __forceinline__ float k_local_max(const float (&x)[4][8]) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 8; j++) m = fmaxf(m, fabsf(x[i][j]));
    return m;
}

// The INT8 code of x / scale for a block scale scale = RN(m / 127) >= kFastDivMin,
// m the largest |x| of the block, in the low byte of the result.  Then
// |x / scale| < 127 (1 + 2^-23), so the correctly rounded quotient q is below
// 127.5 in magnitude and rounds to an integer in [-127, 127] (no clamp), and
// q + 1.5 * 2^23 lies in [2^23, 2^24),
// where fp32 values are the integers: that one addition rounds q to nearest even,
// and the sum is rint(q) + 1.5 * 2^23, whose low byte is rint(q) in two's
// complement.  (The sign of a zero quotient does not matter: both give code 0.)
__device__ __forceinline__ uint32_t int8_code_fast(float x, float scale, float inv) {
    const float q0 = x * inv;
    const float q = __builtin_fmaf(__builtin_fmaf(-q0, scale, x), inv, q0);
    return __float_as_uint(q + 0x1.8p23f);
}

// Codes of the thread's 4 x 8 values with scale sc(i) for token row i.
template <bool FAST>
__device__ __forceinline__ void store_int8_codes_as(const float (&x)[4][8], float s_lo, float s_hi, int tb,
                                                    int64_t bh, int64_t Npad, int8_t *__restrict__ codes) {
    const int t = threadIdx.x, row = t >> 4, seg = t & 15;
    const float i_lo = FAST ? 1.0f / s_lo : 0.0f, i_hi = FAST ? 1.0f / s_hi : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float sc = i < 2 ? s_lo : s_hi, inv = i < 2 ? i_lo : i_hi;
        uint32_t c[2] = {0, 0};
#pragma unroll
        for (int j = 0; j < 8; j++)
            c[j >> 2] |= (FAST ? int8_code_fast(x[i][j], sc, inv) & 0xFFu : int8_code(x[i][j], sc))
                         << (8 * (j & 3));
        const int64_t off = (bh * Npad + (int64_t)tb * 64 + row + 16 * i) * kD + seg * 8;
        *reinterpret_cast<uint2 *>(codes + off) = make_uint2(c[0], c[1]);
    }
}

// The scales are workgroup-uniform, so one of the two paths runs.
__device__ __forceinline__ void store_int8_codes(const float (&x)[4][8], float s_lo, float s_hi, int tb, int64_t bh,
                                                 int64_t Npad, int8_t *__restrict__ codes) {
    if (s_lo >= kFastDivMin && s_hi >= kFastDivMin)
        store_int8_codes_as<true>(x, s_lo, s_hi, tb, bh, Npad, codes);
    else
        store_int8_codes_as<false>(x, s_lo, s_hi, tb, bh, Npad, codes);
}

// K of the block (raw rows from load_block_raw), smoothed: x = fp32(k) - k_mean
// (one fp32 subtraction); zero for tokens >= N.  ROPE: k is first replaced by its
// RMSNorm + RoPE transform, with the rows' norm factors kr[bh * Npad + n] as the
// first pass computed them.
template <bool ROPE>
__device__ __forceinline__ void k_smoothed(const uint4 (&raw)[4], int tb, int N, const float *__restrict__ km,
                                           int64_t bh, const NormRope &nr, const float *__restrict__ kr,
                                           int64_t Npad, float (&x)[4][8]) {
    const int t = threadIdx.x, row = t >> 4, seg = t & 15;
    float mean[8];
#pragma unroll
    for (int j = 0; j < 8; j++) mean[j] = km[bh * kD + seg * 8 + j];
    if (ROPE) {
        const int n[4] = {tb * 64 + row, tb * 64 + row + 16, tb * 64 + row + 32, tb * 64 + row + 48};
        float r[4];
#pragma unroll
        for (int i = 0; i < 4; i++) r[i] = kr[bh * Npad + n[i]];
        uint4 y[4];
        rope_rows<4>(raw, r, nr.gamma_k, nr.gamma_k, n, nr, N, y);
#pragma unroll
        for (int i = 0; i < 4; i++) widen8(y[i], x[i]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; i++) widen8(raw[i], x[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int n = tb * 64 + row + 16 * i;
#pragma unroll
        for (int j = 0; j < 8; j++) x[i][j] = n < N ? x[i][j] - mean[j] : 0.0f;
    }
}

// One workgroup per (64-token block tb, head h, batch b): two Q blocks of 32
// tokens and one K block of 64.
__global__ __launch_bounds__(256) void quant_qk_kernel(View q, View k, int N, int H, int64_t Npad,
                                                       const float *__restrict__ km,
                                                       int8_t *__restrict__ qc, float *__restrict__ qs,
                                                       int8_t *__restrict__ kc, float *__restrict__ ks) {
    __shared__ float red[3][4];
    const int tb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int64_t bh = (int64_t)b * H + h;
    float xq[4][8], xk[4][8];
    uint4 rk[4], rq[4];
    load_block_raw(k, b, h, tb, N, rk);
    load_block_raw(q, b, h, tb, N, rq);
    k_smoothed<false>(rk, tb, N, km, bh, NormRope{}, nullptr, Npad, xk);
#pragma unroll
    for (int i = 0; i < 4; i++) widen8(rq[i], xq[i]);
    float m[3] = {absmax_bf16_rows<0, 2>(rq), absmax_bf16_rows<2, 4>(rq), k_local_max(xk)};
    block_maxes(m, red);
    const float sq0 = m[0] / 127.0f, sq1 = m[1] / 127.0f, sk = m[2] / 127.0f;
    store_int8_codes(xq, sq0, sq1, tb, bh, Npad, qc);
    store_int8_codes(xk, sk, sk, tb, bh, Npad, kc);
    if (threadIdx.x == 0) {
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

// The E4M3 codes of one 64-key tile tt of one head, written tile-major.  Thread
// (g = tid/16, seg = tid%16) encodes keys 4g..4g+3 of channels 8*seg..+7.  The
// four codes of one channel land in consecutive bytes p0..p0+3 of the tile row,
// where p0 inverts kappa (see the public header): keys 4g..4g+3 sit at
// p0 = 32*(g%2) + 16*(g/8) + 4*((g/2)%4).  The 8 KB tile is assembled in LDS
// (tile: kD x 16 words) and written out with coalesced 16-byte stores.
// The raw V rows thread (g, seg) encodes: keys 4g..4g+3 of tile tt.
__device__ __forceinline__ void load_v_tile_raw(View v, int b, int h, int tt, int N, uint4 (&raw)[4]) {
    const int t = threadIdx.x, g = t >> 4, seg = t & 15;
    const uint16_t *base = v.data + (int64_t)b * v.sb + (int64_t)h * v.sh + seg * 8;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int n = tt * kTile + 4 * g + i;
        raw[i] = load_raw8(base + (int64_t)n * v.sn, n < N);
    }
}

__device__ __forceinline__ void v_tile_codes(const uint4 (&raw)[4], int tt, int N, int64_t bh, int64_t Npad,
                                             const float *__restrict__ vs, uint8_t *__restrict__ vc,
                                             uint32_t (*tile)[kTile / 4]) {
    const int t = threadIdx.x, g = t >> 4, seg = t & 15;
    float sv[8];
#pragma unroll
    for (int j = 0; j < 8; j++) sv[j] = vs[bh * kD + seg * 8 + j];
    uint32_t packed[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float x[4][8];
#pragma unroll
    for (int i = 0; i < 4; i++) widen8(raw[i], x[i]);
    bool fast = true;                         // every channel scale of this thread large enough
#pragma unroll
    for (int j = 0; j < 8; j++) fast = fast && sv[j] >= kFastDivMin;
    if (fast) {
        // sv = RN(amax / 448) is normal here, so every quotient has |y| < 448 (1 + 2^-22),
        // below 464: no saturation, and the conversion instruction rounds it as the E4M3 codec does
        // (checked against the codec over that range, both zeros and fp32 subnormals,
        // by the instruction probe tests).  Keys 4g, 4g + 1 fill bytes 0, 1 and keys
        // 4g + 2, 4g + 3 bytes 2, 3.  Rows past N were loaded as +0: their codes are 0.
        float inv[8];
#pragma unroll
        for (int j = 0; j < 8; j++) inv[j] = 1.0f / sv[j];
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(div_rn(x[0][j], sv[j], inv[j]),
                                                          div_rn(x[1][j], sv[j], inv[j]), 0, false);
            packed[j] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(div_rn(x[2][j], sv[j], inv[j]),
                                                                  div_rn(x[3][j], sv[j], inv[j]), lo, true);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int n = tt * kTile + 4 * g + i;
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const uint32_t code = (sv[j] == 0.0f || n >= N) ? 0u : e4m3_encode(x[i][j] / sv[j]);
                packed[j] |= code << (8 * i);
            }
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

// One workgroup per (64-key tile tt, head h, batch b).
__global__ __launch_bounds__(256) void quant_v_kernel(View v, int N, int H, int64_t Npad,
                                                      const float *__restrict__ vs,
                                                      uint8_t *__restrict__ vc) {
    __shared__ uint32_t tile[kD][kTile / 4];
    const int tt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    uint4 rv[4];
    load_v_tile_raw(v, b, h, tt, N, rv);
    v_tile_codes(rv, tt, N, (int64_t)b * H + h, Npad, vs, vc, tile);
}

// ------------------------------------------------- Q, K and V in one call
// The same results as quantize_qk + quantize_v in three passes instead of six:
//   1. per (64-token block, head, batch): the Q codes and scales, the K-mean
//      chunk partial (fp64, per channel, tokens in ascending order) and the
//      block's per-channel max |V|;
//   2. per (b, h, d): k_mean (chunk partials in ascending order, / N) and the V
//      channel maximum and scale;
//   3. per (64-token block, head, batch): the K codes and scale (smoothed) and
//      the block's V codes.
// With the RMSNorm + RoPE transform (qkv_rope_pass1_kernel, qkv_pass3_kernel<true>),
// Q and K are replaced by their transform as they are read: the K block is
// transformed before it is summed and before its codes.

// Per-channel max |V| over this thread's 4 raw rows, into vred[row] (16 rows of
// partial maxima per workgroup; published by the caller's next barrier).
__device__ __forceinline__ void v_block_max(const uint4 (&rv)[4], float (*vred)[kD + 4]) {
    const int t = threadIdx.x, row = t >> 4, seg = t & 15;
    float vm[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        float xv[8];
        widen8(rv[i], xv);
#pragma unroll
        for (int j = 0; j < 8; j++) vm[j] = fmaxf(vm[j], fabsf(xv[j]));
    }
#pragma unroll
    for (int j = 0; j < 8; j++) vred[row][seg * 8 + j] = vm[j];
}

// The two Q blocks' scales (workgroup maxima / 127) and codes of the 64-token
// block held in rq (packed bf16, rows row + 16 i).
__device__ __forceinline__ void q_codes_and_scales(const uint4 (&rq)[4], int tb, int64_t bh, int64_t Npad,
                                                   int8_t *__restrict__ qc, float *__restrict__ qs,
                                                   float (*red)[4]) {
    float m[2] = {absmax_bf16_rows<0, 2>(rq), absmax_bf16_rows<2, 4>(rq)};
    float xq[4][8];
#pragma unroll
    for (int i = 0; i < 4; i++) widen8(rq[i], xq[i]);
    block_maxes(m, red);
    const float sq0 = m[0] / 127.0f, sq1 = m[1] / 127.0f;
    store_int8_codes(xq, sq0, sq1, tb, bh, Npad, qc);
    if (threadIdx.x == 0) {
        qs[bh * (Npad / kQBlock) + 2 * tb] = sq0;
        qs[bh * (Npad / kQBlock) + 2 * tb + 1] = sq1;
    }
}

// The block's chunk partials from LDS: threads 0..127 sum channel t of kbuf over
// the 64 tokens in ascending order (fp64; zeros past N change no sum), threads
// 128..255 reduce the 16 partial V maxima of channel t - 128.
__device__ __forceinline__ void k_sum_v_max_partials(const uint4 (*kbuf)[kD / 8], const float (*vred)[kD + 4],
                                                     int b, int tb, int h, int H, int nchunk,
                                                     double *__restrict__ wsk, float *__restrict__ wsv) {
    const int t = threadIdx.x;
    if (t < kD) {
        const uint16_t *col = reinterpret_cast<const uint16_t *>(&kbuf[0][0]) + t;
        double sum = 0.0;
#pragma unroll 16
        for (int r = 0; r < kKBlock; r++) sum += (double)bf16_to_f32(col[r * kD]);
        wsk[(((int64_t)b * nchunk + tb) * H + h) * kD + t] = sum;
    } else {
        const int d = t - kD;
        float a = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; r++) a = fmaxf(a, vred[r][d]);
        wsv[(((int64_t)b * nchunk + tb) * H + h) * kD + d] = a;
    }
}

__global__ __launch_bounds__(256) void qkv_pass1_kernel(View q, View k, View v, int N, int H, int64_t Npad,
                                                        int nchunk, int8_t *__restrict__ qc, float *__restrict__ qs,
                                                        double *__restrict__ wsk, float *__restrict__ wsv) {
    __shared__ float red[2][4];
    __shared__ uint4 kbuf[kKBlock][kD / 8];      // the block's K rows, bf16 (16 KB)
    __shared__ float vred[16][kD + 4];
    const TokHead w = tok_head(H, (int)(Npad / 64));
    const int tb = w.tb, h = w.h, b = w.b;
    const int t = threadIdx.x, row = t >> 4, seg = t & 15;
    const int64_t bh = (int64_t)b * H + h;
    // K, V and Q rows (raw) of this thread: tokens row + 16 i; tokens >= N read as
    // zero.  Every load is in flight before any compute.
    uint4 rk[4], rv[4], rq[4];
    load_block_raw(k, b, h, tb, N, rk);
    load_block_raw(v, b, h, tb, N, rv);
    load_block_raw(q, b, h, tb, N, rq);
    v_block_max(rv, vred);
#pragma unroll
    for (int i = 0; i < 4; i++) kbuf[row + 16 * i][seg] = rk[i];
    q_codes_and_scales(rq, tb, bh, Npad, qc, qs, red);   // its barriers also publish kbuf and vred
    if (tb >= nchunk) return;                        // a padding block: zero Q codes only
    k_sum_v_max_partials(kbuf, vred, b, tb, h, H, nchunk, wsk, wsv);
}

// The first pass with Q and K replaced by their RMSNorm + RoPE transform.  Two
// workgroups per (64-token block, head, batch), adjacent in the logical grid: the
// odd one transforms the Q block and writes its codes; the even one transforms
// the K block (summed for k_mean; each row's norm factor r kept in kr for the
// last pass, which then skips the sum of squares) and takes the V channel maxima.
// Each holds half the rows of a combined workgroup, so more of them are resident.
__global__ __launch_bounds__(256) void qkv_rope_pass1_kernel(View q, View k, View v, int N, int H, int64_t Npad,
                                                             int nchunk, NormRope nr, int8_t *__restrict__ qc,
                                                             float *__restrict__ qs, double *__restrict__ wsk,
                                                             float *__restrict__ wsv, float *__restrict__ kr) {
    __shared__ float red[2][4];
    __shared__ uint4 kbuf[kKBlock][kD / 8];
    __shared__ float vred[16][kD + 4];
    const uint32_t id = xcd_remap(blockIdx.x, gridDim.x);
    const uint32_t nblk = (uint32_t)(Npad / 64), lid = id >> 1;
    const int tb = (int)((lid / (uint32_t)H) % nblk), h = (int)(lid % (uint32_t)H),
              b = (int)(lid / ((uint32_t)H * nblk));
    const int t = threadIdx.x, row = t >> 4, seg = t & 15;
    const int64_t bh = (int64_t)b * H + h;
    const int n[4] = {tb * 64 + row, tb * 64 + row + 16, tb * 64 + row + 32, tb * 64 + row + 48};
    uint4 y[4];
    float r[4];
    if (id & 1) {
        uint4 rq[4];
        load_block_raw(q, b, h, tb, N, rq);
        norm_rope_rows<4>(rq, nr.gamma_q, nr.gamma_q, n, nr, N, y, r);
        q_codes_and_scales(y, tb, bh, Npad, qc, qs, red);
        return;
    }
    uint4 rk[4], rv[4];
    load_block_raw(k, b, h, tb, N, rk);
    load_block_raw(v, b, h, tb, N, rv);
    v_block_max(rv, vred);
    norm_rope_rows<4>(rk, nr.gamma_k, nr.gamma_k, n, nr, N, y, r);
    // the rows' norm factors: lane seg < 4 of each row group stores row seg's
    // (token row + 16 seg), one store per wave
    float rs = r[0];
#pragma unroll
    for (int i = 1; i < 4; i++) rs = seg == i ? r[i] : rs;
    if (seg < 4) kr[bh * Npad + tb * 64 + row + 16 * seg] = rs;
#pragma unroll
    for (int i = 0; i < 4; i++) kbuf[row + 16 * i][seg] = y[i];
    __syncthreads();                                 // publish kbuf and vred
    if (tb >= nchunk) return;
    k_sum_v_max_partials(kbuf, vred, b, tb, h, H, nchunk, wsk, wsv);
}

template <bool ROPE>
__global__ __launch_bounds__(256) void qkv_pass3_kernel(View k, View v, int N, int H, int64_t Npad, NormRope nr,
                                                        const float *__restrict__ km, const float *__restrict__ vs,
                                                        const float *__restrict__ kr, int8_t *__restrict__ kc,
                                                        float *__restrict__ ks, uint8_t *__restrict__ vc) {
    __shared__ float red[1][4];
    __shared__ uint32_t tile[kD][kTile / 4];
    const TokHead w = tok_head(H, (int)(Npad / 64));
    const int tb = w.tb, h = w.h, b = w.b;
    const int64_t bh = (int64_t)b * H + h;
    uint4 rk[4], rv[4];                              // every row load in flight before any compute
    load_block_raw(k, b, h, tb, N, rk);
    load_v_tile_raw(v, b, h, tb, N, rv);
    float xk[4][8];
    k_smoothed<ROPE>(rk, tb, N, km, bh, nr, kr, Npad, xk);
    float m[1] = {k_local_max(xk)};
    block_maxes(m, red);
    const float sk = m[0] / 127.0f;
    store_int8_codes(xk, sk, sk, tb, bh, Npad, kc);
    if (threadIdx.x == 0) ks[bh * (Npad / kKBlock) + tb] = sk;
    v_tile_codes(rv, tb, N, bh, Npad, vs, vc, tile);
}

// ------------------------------------------------------------ launchers
// chunk_final_kernel: kD / kColsPerWg = 4 workgroups per head and batch entry (the
// shape check bounds B*H by 1e9, so the 1-D grid fits).
static_assert(kD == 4 * kColsPerWg, "four column groups per head");
static dim3 final_grid(int B, int H) { return dim3((unsigned)(4 * (int64_t)H * B)); }

hipError_t launch_quantize_qk(View q, View k, int B, int N, int H, int8_t *qc, float *qs, int8_t *kc,
                              float *ks, float *km, void *workspace, hipStream_t stream) {
    const int nchunk = (N + kSumChunk - 1) / kSumChunk;
    const int64_t Npad = ((int64_t)N + kNAlign - 1) / kNAlign * kNAlign;
    double *ws = static_cast<double *>(workspace);
    LAUNCH_OR_RETURN(kmean_partial_kernel, dim3((nchunk + 15) / 16, H, B), dim3(256), 0, stream, k, N, H, nchunk,
                       ws);
    LAUNCH_OR_RETURN((chunk_final_kernel<true, false>), final_grid(B, H), dim3(256), 0, stream, ws, nullptr, N, H,
                       nchunk, km, nullptr, nullptr);
    LAUNCH_OR_RETURN(quant_qk_kernel, dim3((unsigned)(Npad / 64), H, B), dim3(256), 0, stream, q, k, N, H,
                       Npad, km, qc, qs, kc, ks);
    return hipSuccess;
}

hipError_t launch_quantize_v(View v, int B, int N, int H, uint8_t *vc, float *vs, void *workspace,
                             hipStream_t stream) {
    const int nchunk = (N + kVChunk - 1) / kVChunk;
    const int64_t Npad = ((int64_t)N + kNAlign - 1) / kNAlign * kNAlign;
    float *part = static_cast<float *>(workspace);
    float *amax = part + (int64_t)nchunk * B * H * kD;
    LAUNCH_OR_RETURN(v_amax_partial_kernel, dim3(nchunk, H, B), dim3(256), 0, stream, v, N, H, nchunk, part);
    LAUNCH_OR_RETURN((chunk_final_kernel<false, true>), final_grid(B, H), dim3(256), 0, stream, nullptr, part, N,
                       H, nchunk, nullptr, amax, vs);
    LAUNCH_OR_RETURN(quant_v_kernel, dim3((unsigned)(Npad / kTile), H, B), dim3(256), 0, stream, v, N, H, Npad,
                       vs, vc);
    return hipSuccess;
}

// nr == nullptr: Q and K as given; otherwise their RMSNorm + RoPE transform (the
// workspace then also holds the K rows' norm factors, B * H * Npad floats, after
// the amax block).
hipError_t launch_quantize_qkv(View q, View k, View v, int B, int N, int H, const NormRope *nr, int8_t *qc, float *qs,
                               int8_t *kc, float *ks, float *km, uint8_t *vc, float *vs, void *workspace,
                               hipStream_t stream) {
    const int nchunk = (N + kKBlock - 1) / kKBlock;
    const int64_t Npad = ((int64_t)N + kNAlign - 1) / kNAlign * kNAlign;
    const int64_t total = (int64_t)B * H * kD;
    double *wsk = static_cast<double *>(workspace);
    float *wsv = reinterpret_cast<float *>(wsk + (int64_t)nchunk * total);
    float *amax = wsv + (int64_t)nchunk * total;
    float *kr = nr ? amax + total : nullptr;
    const NormRope p = nr ? *nr : NormRope{};
    const dim3 grid((unsigned)(Npad / 64 * H * B));
    // passes 1 and 3 run over every 64-token block of the padded code buffers
    // (blocks past N write zero codes and scales); the partials exist for the
    // nchunk blocks that hold tokens
    if (nr)
        LAUNCH_OR_RETURN(qkv_rope_pass1_kernel, dim3(2 * grid.x), dim3(256), 0, stream, q, k, v, N, H, Npad, nchunk,
                           p, qc, qs, wsk, wsv, kr);
    else
        LAUNCH_OR_RETURN(qkv_pass1_kernel, grid, dim3(256), 0, stream, q, k, v, N, H, Npad, nchunk, qc, qs, wsk,
                           wsv);
    LAUNCH_OR_RETURN((chunk_final_kernel<true, true>), final_grid(B, H), dim3(256), 0, stream, wsk, wsv, N, H,
                       nchunk, km, amax, vs);
    if (nr)
        LAUNCH_OR_RETURN(qkv_pass3_kernel<true>, grid, dim3(256), 0, stream, k, v, N, H, Npad, p, km, vs, kr, kc,
                           ks, vc);
    else
        LAUNCH_OR_RETURN(qkv_pass3_kernel<false>, grid, dim3(256), 0, stream, k, v, N, H, Npad, p, km, vs, kr, kc,
                           ks, vc);
    return hipSuccess;
}

hipError_t launch_norm_rope(OutView q, OutView k, int B, int N, int H, NormRope nr, hipStream_t stream) {
    LAUNCH_OR_RETURN(norm_rope_kernel, dim3((unsigned)((N + 63) / 64 * H * B)), dim3(256), 0, stream, q, k, N, H,
                       nr);
    return hipSuccess;
}

}  // namespace sage
