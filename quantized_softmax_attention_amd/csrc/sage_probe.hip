// sage_probe.hip -- libsage_probe.so: single-instruction probes used by the GPU
// tests to check the register layouts and conversions the kernels rely on
// (MFMA operand/accumulator layouts, the E4M3 pack instruction, the half-wave
// swap, exp2).  One wave per launch; every access is within the buffers the
// caller passes (sizes fixed below).  Each call synchronises the device and
// returns a hipError_t value.  Not part of the library's ABI.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// a, b: [64 lanes][4 dwords]; d: [64 lanes][16 dwords]
__global__ void probe_i8_kernel(const v4i *a, const v4i *b, v16i *d) {
    int l = threadIdx.x;
    v16i acc = {};
    d[l] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[l], b[l], acc, 0, 0, 0);
}

// a, b: [64][8] dwords of E4M3 codes; d: [64][16] floats; unit scales (E8M0 127)
__global__ void probe_f8_kernel(const v8i *a, const v8i *b, v16f *d) {
    int l = threadIdx.x;
    v16f acc = {};
    d[l] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[l], b[l], acc, 0, 0, 0, 127, 0, 127);
}

// as above with an input accumulator c: [64][16] floats
__global__ void probe_f8_acc_kernel(const v8i *a, const v8i *b, const v16f *c, v16f *d) {
    int l = threadIdx.x;
    d[l] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[l], b[l], c[l], 0, 0, 0, 127, 0, 127);
}

// a, b: [64][4] dwords of bf16 pairs; d: [64][16] floats
__global__ void probe_bf16_kernel(const v4i *a, const v4i *b, v16f *d) {
    int l = threadIdx.x;
    v16f acc = {};
    d[l] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a[l]), __builtin_bit_cast(v8bf, b[l]),
                                                   acc, 0, 0, 0);
}

// x: [n] floats (n even); out[i] = the byte v_cvt_pk_fp8_f32 gives x[i].
// Even pairs go to the low half-word, odd pairs to the high half-word.
__global__ void probe_cvt_fp8_kernel(const float *x, int n, uint8_t *out) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;   // one dword = two pairs
    if (4 * i + 3 < n) {
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * i], x[4 * i + 1], 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * i + 2], x[4 * i + 3], w, true);
        for (int j = 0; j < 4; j++) out[4 * i + j] = (uint8_t)((uint32_t)w >> (8 * j));
    }
}

// x: [64]; out: [2][64] = both results of v_permlane32_swap(x, x)
__global__ void probe_swap_kernel(const int *x, int *out) {
    int l = threadIdx.x;
    auto r = __builtin_amdgcn_permlane32_swap(x[l], x[l], false, false);
    out[l] = r[0];
    out[64 + l] = r[1];
}

// in: 4096 bf16/i16 values staged in LDS; addr: per-lane byte addresses (each
// < 8192 - 8, 8-byte aligned); out: [64 lanes][4] results of ds_read_b64_tr_b16.
typedef short v4s __attribute__((ext_vector_type(4)));
__global__ void probe_tr16_kernel(const short *in, const int *addr, v4s *out) {
    __shared__ short lds[4096];
    for (int i = threadIdx.x; i < 4096; i += 64) lds[i] = in[i];
    __syncthreads();
    int a = addr[threadIdx.x];
    out[threadIdx.x] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(lds + a / 2));
}

__global__ void probe_exp2_kernel(const float *x, int n, float *out) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = __builtin_amdgcn_exp2f(x[i]);
}

// ---- issue-rate probe of the softmax instructions -------------------------
// One workgroup of `waves` waves on one CU (4, 8, 12 or 16 waves: one to four per
// SIMD; each wave reports the SIMD it ran on).  Every wave runs `iters`
// iterations of 4 groups; a group is (optionally) one MFMA followed by 8
// instructions of kind OP on CH independent register chains (8 or 16), so each
// instruction depends on the one issued CH slots earlier.  The two MFMA chains
// alternate, as in the attention kernel.  Lane 0 of each wave writes the
// absolute s_memtime (shader clock) before and after the loop, the
// s_memrealtime (fixed 100 MHz) difference and its SIMD id; the host takes
// per-SIMD throughput from the union of the intervals of the waves on that
// SIMD.  The chains' values are written to `sink` so no work is removed.
// Mixed kinds alternate within each group of 8: kRateMixExpFma exp/fma,
// kRateMixPkFma cvt_pk_fp8/fma, kRateMixSoftmax the per-score mix of the
// attention (sub, fma, exp, add, sub, fma, exp, cvt_pk_fp8).
enum RateOp { kRateFma = 0, kRateAdd, kRateExp, kRateCvtF32I32, kRateCvtPkFp8, kRateMax3, kRateSub, kRateNone,
              kRateMixExpFma, kRateMixPkFma, kRateMixSoftmax };

template <int OP>
__device__ __forceinline__ constexpr int rate_slot_op(int j) {
    if (OP == kRateMixExpFma) return (j & 1) ? kRateFma : kRateExp;
    if (OP == kRateMixPkFma) return (j & 1) ? kRateFma : kRateCvtPkFp8;
    if (OP == kRateMixSoftmax) {
        constexpr int mix[8] = {kRateSub, kRateFma, kRateExp, kRateAdd, kRateSub, kRateFma, kRateExp, kRateCvtPkFp8};
        return mix[j];
    }
    return OP;
}

template <int OP, int CH>
__device__ __forceinline__ void rate_group(float (&x)[CH], int (&w)[CH], int g, float c0, float c1, int i0, int i1) {
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const int k = (8 * g + j) % CH;
        const int op = rate_slot_op<OP>(j);
        if (op == kRateFma) x[k] = __builtin_fmaf(x[k], c0, c1);
        if (op == kRateAdd) x[k] = x[k] + c0;
        if (op == kRateSub) x[k] = x[k] - c1;
        if (op == kRateExp) x[k] = __builtin_amdgcn_exp2f(-x[k]);            // converges to ~0.64
        if (op == kRateCvtF32I32) x[k] = (float)__float_as_int(x[k]);         // bits -> value
        if (op == kRateCvtPkFp8) {
            if (j & 1) w[k] = __builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, w[k], true);
            else w[k] = __builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, w[k], false);
        }
        if (op == kRateMax3) asm volatile("v_max3_i32 %0, %0, %1, %2" : "+v"(w[k]) : "v"(i0), "v"(i1));
    }
}

template <int OP, int MF, int CH>   // MF: 0 none, 1 INT8 32x32x32, 2 FP8 32x32x64 (one per group)
__global__ __launch_bounds__(1024) void rate_kernel(int iters, float seed, unsigned long long *cyc, float *sink) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    float x[CH];
    int w[CH];
#pragma unroll
    for (int k = 0; k < CH; k++) {
        x[k] = seed + 0.01f * (float)(lane + k);
        w[k] = lane * 8 + k;
    }
    const float c0 = seed * 0.5f, c1 = seed * 0.25f;
    const int i0 = lane - 7, i1 = 3 - lane;
    v16i ai[2] = {v16i{}, v16i{}};
    v16f af[2] = {v16f{}, v16f{}};
    const v4i qa = {lane, lane + 1, lane + 2, lane + 3};
    const v8i fa = {lane, lane ^ 0x11, lane ^ 0x22, lane ^ 0x33, lane, lane, lane, lane};
    // HW_ID bits 5:4 = SIMD id (s_getreg_b32 hwreg(HW_REG_HW_ID, 4, 2))
    const unsigned simd = __builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4);
    __builtin_amdgcn_s_waitcnt(0);
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int g = 0; g < 4; g++) {
            if (MF == 1) ai[g & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(qa, qa, ai[g & 1], 0, 0, 0);
            if (MF == 2)
                af[g & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fa, af[g & 1], 0, 0, 0, 0, 0, 0);
            if (OP != kRateNone) rate_group<OP, CH>(x, w, g, c0, c1, i0, i1);
            if (MF) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (OP != kRateNone) __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
            }
        }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < CH; k++) acc += x[k] + (float)w[k];
#pragma unroll
    for (int r = 0; r < 16; r++) acc += (float)(ai[0][r] + ai[1][r]) + af[0][r] + af[1][r];
    sink[threadIdx.x] = acc;
    if (lane == 0) {
        cyc[4 * wv] = t0;
        cyc[4 * wv + 1] = t1;
        cyc[4 * wv + 2] = r1 - r0;
        cyc[4 * wv + 3] = simd;
    }
}

template <int OP, int CH>
static void launch_rate(int mf, int waves, int iters, unsigned long long *cyc, float *sink) {
    const dim3 g(1), b(64 * waves);
    if (mf == 0) hipLaunchKernelGGL((rate_kernel<OP, 0, CH>), g, b, 0, 0, iters, 1.5f, cyc, sink);
    if (mf == 1) hipLaunchKernelGGL((rate_kernel<OP, 1, CH>), g, b, 0, 0, iters, 1.5f, cyc, sink);
    if (mf == 2) hipLaunchKernelGGL((rate_kernel<OP, 2, CH>), g, b, 0, 0, iters, 1.5f, cyc, sink);
}

template <int OP>
static void launch_rate_ch(int mf, int waves, int iters, int chains, unsigned long long *cyc, float *sink) {
    if (chains == 16) launch_rate<OP, 16>(mf, waves, iters, cyc, sink);
    else launch_rate<OP, 8>(mf, waves, iters, cyc, sink);
}

// ---- replay of the quantised attention's per-tile instruction stream ---------
// One wave-tile of attn_i8f8_kernel (32 queries x 64 keys) in its steady state,
// with the kernel's data dependences and interleave but no memory traffic: the
// MFMA A operands stay in registers instead of being read from LDS, and there
// are no HBM -> LDS loads and no barriers.  Per tile t:
//   * 4 FP8 32x32x64 MFMAs (P(t-1) V) interleaved with the running maximum of
//     the biased INT8 scores of tile t (16 three-input maxima, the half-wave
//     swap, one conversion);
//   * 8 INT8 32x32x32 MFMAs of tile t+1 (two alternating chains), each followed
//     by one chunk of 4 scores: int -> float conversion, fma, exp2, the fp32
//     sum and two E4M3 pair packs (SUB: the chains start from the bit pattern
//     of a float bias block and a subtraction replaces the conversion, a form
//     that gives the same values);
//   * the row-sum update, alpha = exp2(m_old - m_new) and RESCALE multiplies of
//     the output accumulators (64 in a tile where some row maximum moved, 0
//     otherwise).
// The cycles per tile per SIMD, at two waves per SIMD as the kernel runs, are
// the issue floor of the kernel's instruction stream on that SIMD (its
// instruction counts per tile equal those of the kernel's loop).
struct ReplayState {
    float m2, lsum, part;
    v8i pf[2];   // packed P: one buffer read by this tile's P.V MFMAs, the other written by its exp chunks
};

template <bool CHAIN, bool SUB>
__device__ __forceinline__ void replay_tile(const v16i (&s)[2], v16i (&sn)[2], v4i (&ka)[2], v8i (&va)[2],
                                            float c2, float f0, int hl, ReplayState &st, v16f (&o)[4],
                                            const v16i &binit) {
    // the operands the kernel reads from LDS for this tile: opaque, so no MFMA is loop-invariant
    asm volatile("" : "+v"(ka[0]), "+v"(ka[1]), "+v"(va[0]), "+v"(va[1]));
#pragma unroll
    for (int db = 0; db < 4; db++)
        o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va[db & 1], st.pf[CHAIN ? 0 : 1], o[db], 0, 0, 0, 0, 0,
                                                               0);
    int imax = max(max(s[0][0], s[0][1]), s[0][2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) imax = max(max(imax, s[0][r]), s[0][r + 1]);
    imax = max(max(imax, s[0][15]), s[1][0]);
#pragma unroll
    for (int r = 1; r < 15; r += 2) imax = max(max(imax, s[1][r]), s[1][r + 1]);
    imax = max(imax, s[1][15]);
    auto sw = __builtin_amdgcn_permlane32_swap(imax, imax, false, false);
    imax = max((int)sw[0], (int)sw[1]);
    // the P.V MFMAs first, spread over the maximum (the kernel's first region)
#pragma unroll
    for (int i = 0; i < 4; i++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    const float mnew = fmaxf(st.m2, c2 * (SUB ? __int_as_float(imax) - f0 : (float)imax));
    const float alpha = __builtin_amdgcn_exp2f(st.m2 - mnew);
    st.m2 = mnew;
    const float bias = mnew - 8.807354922057604f;
#pragma unroll
    for (int c = 0; c < 8; c++) {
        if (SUB)
            sn[c & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka[c & 1], ka[(c >> 1) & 1], c < 2 ? binit : sn[c & 1],
                                                              0, 0, 0);
        else
            sn[c & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka[c & 1], ka[(c >> 1) & 1], c < 2 ? v16i{} : sn[c & 1],
                                                              0, 0, 0);
        const int kb = c >> 2, r = 4 * (c & 3);
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; i++)
            p[i] = __builtin_amdgcn_exp2f(c2 * (SUB ? __int_as_float(s[kb][r + i]) - f0 : (float)s[kb][r + i]) - bias);
        const float chunk = (p[0] + p[1]) + (p[2] + p[3]);
        st.part = c == 0 ? chunk : st.part + chunk;
        v8i &pn = st.pf[CHAIN ? 1 : 0];
        int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], pn[c], false);
        pn[c] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wd, true);
    }
#pragma unroll
    for (int i = 0; i < 8; i++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
    }
    asm volatile("" ::"v"(st.pf[CHAIN ? 1 : 0]), "v"(st.part), "v"(sn[0]), "v"(sn[1]));
    __builtin_amdgcn_sched_barrier(0);
    st.lsum = st.lsum * alpha + st.part;
    (void)hl;
}

template <int RESCALE, bool SUB>
__global__ __launch_bounds__(512) void tile_replay_kernel(int iters, float seed, unsigned long long *cyc,
                                                           float *sink) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, hl = lane >> 5;
    v4i ka[2] = {v4i{lane * 0x01010101, lane ^ 0x5A5A5A5A, lane + 3, 7 - lane}, v4i{lane, 3, 5, -lane}};
    const v8i fa = {0x38383838, 0x30303030, 0x38303830, 0x30383038, 0x38383838, 0x30303030, 0x38303830, 0x30383038};
    v8i va[2] = {fa, fa ^ 0x08080808};
    const int kb0 = 0x3E22F983;
    const v16i binit = {kb0, kb0, kb0, kb0, kb0, kb0, kb0, kb0, kb0, kb0, kb0, kb0, kb0, kb0, kb0, kb0};
    const float c2 = seed * 1e-3f, f0 = 0.15915494f;
    v16i sa[2] = {binit, binit}, sb[2] = {binit, binit};
    v16f o[4] = {v16f{}, v16f{}, v16f{}, v16f{}};
    ReplayState st{-INFINITY, 0.0f, 0.0f, {v8i{}, v8i{}}};
    const unsigned simd = __builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4);
    __builtin_amdgcn_s_waitcnt(0);
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; it++) {        // two tiles per iteration (score buffers alternate)
        replay_tile<true, SUB>(sa, sb, ka, va, c2, f0, hl, st, o, binit);
        if (RESCALE) {
#pragma unroll
            for (int r = 0; r < RESCALE; r++) o[r >> 4][r & 15] *= st.lsum;
        }
        replay_tile<false, SUB>(sb, sa, ka, va, c2, f0, hl, st, o, binit);
        if (RESCALE) {
#pragma unroll
            for (int r = 0; r < RESCALE; r++) o[r >> 4][r & 15] *= st.lsum;
        }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    float acc = st.lsum + st.m2 + (float)(ka[0][0] + ka[1][1] + va[0][2] + va[1][3] + binit[5]);
#pragma unroll
    for (int r = 0; r < 16; r++)
        acc += (float)(sa[0][r] + sa[1][r] + sb[0][r] + sb[1][r]) + o[0][r] + o[1][r] + o[2][r] + o[3][r];
    sink[threadIdx.x] = acc;
    if (lane == 0) {
        cyc[4 * wv] = t0;
        cyc[4 * wv + 1] = t1;
        cyc[4 * wv + 2] = r1 - r0;
        cyc[4 * wv + 3] = simd;
    }
}

extern "C" {
// Replay of the attention's per-tile instruction mix (tile_replay_kernel):
// waves (4 or 8, one workgroup), iters >= 1 (two tiles each), rescale =
// multiplies per tile in the tail (0: no row maximum moved, 64: one did), sub
// (0: int -> float conversion of the scores as the kernel, 1: biased-float
// subtraction); cyc and sink as for sage_probe_rate.
int sage_probe_tile_replay(int waves, int iters, int rescale, int sub, unsigned long long *cyc, float *sink) {
    if ((waves != 4 && waves != 8) || iters < 1) return -1;
    const dim3 g(1), b(64 * waves);
    if (rescale == 0 && !sub) hipLaunchKernelGGL((tile_replay_kernel<0, false>), g, b, 0, 0, iters, 1.5f, cyc, sink);
    else if (rescale == 64 && !sub)
        hipLaunchKernelGGL((tile_replay_kernel<64, false>), g, b, 0, 0, iters, 1.5f, cyc, sink);
    else if (rescale == 0 && sub) hipLaunchKernelGGL((tile_replay_kernel<0, true>), g, b, 0, 0, iters, 1.5f, cyc, sink);
    else if (rescale == 64 && sub)
        hipLaunchKernelGGL((tile_replay_kernel<64, true>), g, b, 0, 0, iters, 1.5f, cyc, sink);
    else return -1;
    hipError_t e = hipGetLastError();
    return e != hipSuccess ? (int)e : (int)hipDeviceSynchronize();
}

// Issue-rate probe: op (RateOp), mf (0: no MFMA, 1: INT8 32x32x32, 2: FP8
// 32x32x64 per 8 instructions), waves (4, 8, 12 or 16, one workgroup), iters >= 1,
// chains (8 or 16).  cyc: [waves][4] u64 (s_memtime at start, at end,
// s_memrealtime difference, SIMD id); sink: [64*waves] floats.
int sage_probe_rate(int op, int mf, int waves, int iters, int chains, unsigned long long *cyc, float *sink) {
    if (op < 0 || op > kRateMixSoftmax || mf < 0 || mf > 2 || waves < 4 || waves > 16 || waves % 4 || iters < 1)
        return -1;
    if ((op == kRateNone && mf == 0) || (chains != 8 && chains != 16)) return -1;
    switch (op) {
        case kRateFma: launch_rate_ch<kRateFma>(mf, waves, iters, chains, cyc, sink); break;
        case kRateAdd: launch_rate_ch<kRateAdd>(mf, waves, iters, chains, cyc, sink); break;
        case kRateExp: launch_rate_ch<kRateExp>(mf, waves, iters, chains, cyc, sink); break;
        case kRateCvtF32I32: launch_rate_ch<kRateCvtF32I32>(mf, waves, iters, chains, cyc, sink); break;
        case kRateCvtPkFp8: launch_rate_ch<kRateCvtPkFp8>(mf, waves, iters, chains, cyc, sink); break;
        case kRateMax3: launch_rate_ch<kRateMax3>(mf, waves, iters, chains, cyc, sink); break;
        case kRateSub: launch_rate_ch<kRateSub>(mf, waves, iters, chains, cyc, sink); break;
        case kRateMixExpFma: launch_rate_ch<kRateMixExpFma>(mf, waves, iters, chains, cyc, sink); break;
        case kRateMixPkFma: launch_rate_ch<kRateMixPkFma>(mf, waves, iters, chains, cyc, sink); break;
        case kRateMixSoftmax: launch_rate_ch<kRateMixSoftmax>(mf, waves, iters, chains, cyc, sink); break;
        default: launch_rate_ch<kRateNone>(mf, waves, iters, chains, cyc, sink); break;
    }
    hipError_t e = hipGetLastError();
    return e != hipSuccess ? (int)e : (int)hipDeviceSynchronize();
}


int sage_probe_mfma_i8(const void *a, const void *b, void *d) {
    hipLaunchKernelGGL(probe_i8_kernel, dim3(1), dim3(64), 0, 0, (const v4i *)a, (const v4i *)b, (v16i *)d);
    hipError_t e = hipGetLastError();
    return e != hipSuccess ? (int)e : (int)hipDeviceSynchronize();
}

int sage_probe_mfma_f8(const void *a, const void *b, void *d) {
    hipLaunchKernelGGL(probe_f8_kernel, dim3(1), dim3(64), 0, 0, (const v8i *)a, (const v8i *)b, (v16f *)d);
    hipError_t e = hipGetLastError();
    return e != hipSuccess ? (int)e : (int)hipDeviceSynchronize();
}

int sage_probe_mfma_f8_acc(const void *a, const void *b, const void *c, void *d) {
    hipLaunchKernelGGL(probe_f8_acc_kernel, dim3(1), dim3(64), 0, 0, (const v8i *)a, (const v8i *)b, (const v16f *)c,
                       (v16f *)d);
    hipError_t e = hipGetLastError();
    return e != hipSuccess ? (int)e : (int)hipDeviceSynchronize();
}

int sage_probe_mfma_bf16(const void *a, const void *b, void *d) {
    hipLaunchKernelGGL(probe_bf16_kernel, dim3(1), dim3(64), 0, 0, (const v4i *)a, (const v4i *)b, (v16f *)d);
    hipError_t e = hipGetLastError();
    return e != hipSuccess ? (int)e : (int)hipDeviceSynchronize();
}

int sage_probe_cvt_fp8(const float *x, int n, uint8_t *out) {
    if (n <= 0 || n % 4) return -1;
    int dwords = n / 4;
    hipLaunchKernelGGL(probe_cvt_fp8_kernel, dim3((dwords + 255) / 256), dim3(256), 0, 0, x, n, out);
    hipError_t e = hipGetLastError();
    return e != hipSuccess ? (int)e : (int)hipDeviceSynchronize();
}

int sage_probe_swap(const int *x, int *out) {
    hipLaunchKernelGGL(probe_swap_kernel, dim3(1), dim3(64), 0, 0, x, out);
    hipError_t e = hipGetLastError();
    return e != hipSuccess ? (int)e : (int)hipDeviceSynchronize();
}

int sage_probe_tr16(const short *in, const int *addr, short *out) {
    hipLaunchKernelGGL(probe_tr16_kernel, dim3(1), dim3(64), 0, 0, in, addr, (v4s *)out);
    hipError_t e = hipGetLastError();
    return e != hipSuccess ? (int)e : (int)hipDeviceSynchronize();
}

int sage_probe_exp2(const float *x, int n, float *out) {
    if (n <= 0) return -1;
    hipLaunchKernelGGL(probe_exp2_kernel, dim3((n + 255) / 256), dim3(256), 0, 0, x, n, out);
    hipError_t e = hipGetLastError();
    return e != hipSuccess ? (int)e : (int)hipDeviceSynchronize();
}

}  // extern "C"
