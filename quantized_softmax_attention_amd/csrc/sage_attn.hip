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
//    P^T values the B operand of the FP8 MFMA (32x32x64, E4M3 x E4M3) needs (32 keys
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
#include "sage_attn_parts.h"

namespace sage {

namespace {

using namespace attn;

constexpr int kTileBytes = kI8TileBytes;   // 8 KB per K tile and per V tile
constexpr int kChunks = kI8Chunks;         // 512 16-byte chunks per tile
constexpr float kLog2_448 = 8.807354922057604f;

// LDS slot of 16-byte chunk c (0..3) of V channel row d (0..127).  ds_read_b128
// serves 16 consecutive lanes per cycle from 64 four-byte banks; with this XOR
// the 32 channel rows x 2 chunks a fragment read touches are conflict-free
// (measured: 4 LDS cycles per read, the minimum).
__device__ __forceinline__ int v_swz(int d) { return (d >> 2) & 3; }
__device__ __forceinline__ int v_slot(int d, int c) { return d * 4 + (c ^ v_swz(d)); }

// HBM -> LDS staging of the K tile (shared INT8 loader) and of the tile-major
// V codes: wave w fills slots [128 w, 128 w + 128) of the 512-slot V tile, lane
// L of load i slot 128 w + 64 i + L, from the per-lane source offsets below.
struct TileLoader {
    K8Loader k;
    int voff[2];
};

__device__ __forceinline__ TileLoader make_loader(int w, int lane) {
    TileLoader L;
    L.k = make_k8_loader(w, lane);
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int slot = 128 * w + 64 * i + lane;
        const int d = slot >> 2, dc = slot & 3;   // LDS slot -> channel, stored chunk
        L.voff[i] = d * 64 + 16 * (dc ^ v_swz(d));
    }
    return L;
}

__device__ __forceinline__ void lds_load_k(v4i *lk, const int8_t *tile, const TileLoader &L, int w) {
    lds_load_k8(lk, tile, L.k, w);
}
__device__ __forceinline__ void lds_load_v(v4i *lv, const uint8_t *tile, const TileLoader &L, int w) {
    const auto r = tile_rsrc(tile, kTileBytes);
#pragma unroll
    for (int i = 0; i < 2; i++)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(lv + 128 * w + 64 * i), 16, L.voff[i], 0, 0, 0);
}

// p' = 448 * exp(s - m) for registers 4c..4c+3 of the tile (c = 0..7), summed
// in fp32 before rounding, packed to E4M3 into operand dword c.
template <bool TAIL>
__device__ __forceinline__ void tile_exp_chunk(const v16i (&s)[2], float c2, float bias, int nvalid, int hl, int c,
                                               v8i &pf, float &part) {
    const int kb = c >> 2, r = 4 * (c & 3);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        p[i] = fast_exp2(c2 * (float)s[kb][r + i] - bias);
        if (TAIL && 32 * kb + 8 * (r >> 2) + 4 * hl + i >= nvalid) p[i] = 0.0f;
    }
    const float chunk = (p[0] + p[1]) + (p[2] + p[3]);
    part = c == 0 ? chunk : part + chunk;   // (no add of the initial zero)
    // the low and then the high half of the dword; the previous tile's value
    // serves as the (fully overwritten) old operand, so no copy is needed
    int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], pf[c], false);
    pf[c] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wd, true);
}

// O^T += V^T P^T, 32 channels per MFMA.  The block-scale operands of the builtin
// are given as 0, which selects the unscaled v_mfma_f32_32x32x64_f8f6f4 (the same
// products as E8M0 scales of 127, i.e. 1.0; the shorter encoding carries no scale
// registers).
__device__ __forceinline__ void pv_tile(const v4i *lv, const v8i &pf, int hl, int ql, v16f (&o)[4]) {
#pragma unroll
    for (int db = 0; db < 4; db++) {
        const int d = 32 * db + ql;
        v4i lo = lv[v_slot(d, 2 * hl)];
        v4i hi = lv[v_slot(d, 2 * hl + 1)];
        v8i va = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pf, o[db], 0, 0, 0, 0, 0, 0);
    }
}

// FP8 MFMA operand of channel block db, read from the tile-major V codes in LDS.
__device__ __forceinline__ v8i v_operand(const v4i *lv, int db, int hl, int ql) {
    const int d = 32 * db + ql;
    v4i lo = lv[v_slot(d, 2 * hl)];
    v4i hi = lv[v_slot(d, 2 * hl + 1)];
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Per-wave running state of the online softmax.
struct RowState {
    float m2;     // running maximum, log2 units
    float lsum;   // running sum of p' over this lane's keys
    v8i pf;       // E4M3 P^T operand of the last processed tile (its P.V is pending)
};

// Step t of the software pipeline, one scheduling region:
//   1. (PV)   O += V(t-1) P(t-1), where O already carries alpha(t-1)
//   2.        running max over tile t; alpha(t); l = alpha(t) * l + sum p'(t)
//   3.        p'(t) -> E4M3, with the 8 QK^T MFMAs of tile t+1 (QK) interleaved
//   4. (PV)   O = alpha(t) * O (a branch, taken only when some row's max moved;
//             by then the P.V MFMAs of step 1 have completed)
// The LDS holds V(t-1) in lv_prev and K(t+1) in lk_next.
template <bool PV, bool QK, bool TAIL>
__device__ __forceinline__ void step(v16i (&s)[2], v16i (&sn)[2], const v4i *lk_next, const v4i *lv_prev,
                                     const v4i (&qa)[4], float c2, int nvalid, int hl, int ql, RowState &st,
                                     v16f (&o)[4]) {
    // MFMA operands are read from LDS ahead of their MFMA (V one MFMA ahead, K
    // two), so an MFMA rarely waits for its LDS read and the VALU work behind
    // it in issue order is not held up.
    v8i va[2];
    v4i ka[3];
    if (PV) va[0] = v_operand(lv_prev, 0, hl, ql);
    else if (QK) {
        ka[0] = k8_operand(lk_next, 0, hl, ql);
        ka[1] = k8_operand(lk_next, 1, hl, ql);
    }
    if (PV) {   // O = alpha(t-1) acc(t-2) + P(t-1) V(t-1)
#pragma unroll
        for (int db = 0; db < 4; db++) {
            if (db < 3) va[(db + 1) & 1] = v_operand(lv_prev, db + 1, hl, ql);
            if (QK && db >= 2) ka[db - 2] = k8_operand(lk_next, db - 2, hl, ql);
            o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va[db & 1], st.pf, o[db], 0, 0, 0, 0, 0, 0);
        }
    }
    const float mnew = tile_max_i32<TAIL>(s, c2, nvalid, hl, st.m2);
    const float alpha = fast_exp2(st.m2 - mnew);   // 0 on the first tile (m2 = -inf)
    st.m2 = mnew;
    const float bias = mnew - kLog2_448;
    float part = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; c++) {
        if (QK) {
            if (c < 6) ka[(c + 2) % 3] = k8_operand(lk_next, c + 2, hl, ql);
            const int kb = c & 1, kst = c >> 1;   // the two accumulation chains alternate
            sn[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka[c % 3], qa[kst], kst ? sn[kb] : v16i{}, 0, 0, 0);
        }
        tile_exp_chunk<TAIL>(s, c2, bias, nvalid, hl, c, st.pf, part);
    }
    // Issue order for the region: the P.V MFMAs spread over the max reduction,
    // then one QK^T MFMA per exp chunk, each LDS read placed before the MFMA
    // that precedes its own.
    if (PV) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);           // V operand 0
#pragma unroll
        for (int i = 0; i < 4; i++) {
            if (i < 3) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);          // V operand i+1
            if (QK && i >= 2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // K operands 0, 1
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // P.V MFMA i
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // 6 VALU
        }
    } else if (QK) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);       // K operands 0, 1
    }
    if (QK) {
#pragma unroll
        for (int i = 0; i < 8; i++) {
            if (i < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // K operand i+2
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // QK^T MFMA i
            __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);  // 16 VALU
        }
    }
    // Everything above is consumed only in the next step, after the rescale
    // branch; this empty statement reads it here so no pass sinks the work
    // (or the MFMAs) out of this step's schedule.
    asm volatile("" ::"v"(st.pf), "v"(part));
    if (QK) asm volatile("" ::"v"(sn[0]), "v"(sn[1]));
    __builtin_amdgcn_sched_barrier(0);
    st.lsum = st.lsum * alpha + part;
    if (PV) rescale(alpha, o);                    // O = alpha(t) acc(t-1); O is 0 before step 1
}

// Software pipeline per wave: while the softmax of tile t runs on the VALU, the
// QK^T MFMAs of tile t+1 and the P.V MFMAs of tile t-1 are in flight.  K tiles
// are staged two steps ahead of the softmax and V tiles one behind: step t
// reads K(t+1), V(t-1) from LDS and writes K(t+2), V(t) (loaded from HBM at the
// start of the step) into the buffers of K(t), V(t-2).
// OUTF: -1 writes the bf16 output through `out`; kMxE4M3 / kMxE2M1 write the MX
// blocks of those bf16 values to mx_codes / mx_scales instead.
template <int OUTF>
__global__ __launch_bounds__(kThreads, 2) void attn_i8f8_kernel(
    const int8_t *__restrict__ qc, const float *__restrict__ qs, const int8_t *__restrict__ kc,
    const float *__restrict__ ks, const uint8_t *__restrict__ vc, const float *__restrict__ vs, int N,
    int H, int64_t Npad, float c_base, OutView out, uint8_t *__restrict__ mx_codes,
    uint8_t *__restrict__ mx_scales, int nqwg) {
    // four separate LDS objects, always selected at compile time, so the
    // compiler can tell the buffers being read from the ones being filled
    __shared__ v4i lk0[kChunks], lk1[kChunks], lv0[kChunks], lv1[kChunks];

    const uint32_t id = xcd_remap(blockIdx.x, gridDim.x);
    const int qb = (int)(id % (uint32_t)nqwg);
    const int64_t bh = id / (uint32_t)nqwg;
    const int b = (int)(bh / H), h = (int)(bh % H);
    const int t = threadIdx.x, lane = t & 63, hl = lane >> 5, ql = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform: LDS addresses stay scalar
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
    const bool partial = tail_valid != kTile;

    v16f o[4];
#pragma unroll
    for (int db = 0; db < 4; db++)
        o[db] = v16f{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    RowState rs{-INFINITY, 0.0f, v8i{}};

    // prologue: K(0), K(1) into LDS; S(0) = K(0) Q^T; K(0)'s buffer is
    // rewritten in step 0, so every wave finishes reading it first.
    const TileLoader ldr = make_loader(w, lane);
    lds_load_k(lk0, kbase, ldr, w);
    if (ntiles > 1) lds_load_k(lk1, kbase + kTileBytes, ldr, w);
    wait_lds_loads_and_sync();
    v16i sa[2], sb[2];
    qk8_tile(lk0, qa, hl, ql, sa);
    __syncthreads();

    // Step t stages K(t+2) and V(t) into the buffers of K(t) and V(t-2), which
    // the previous step finished reading before its barrier.  Buffer parity is
    // t's: even steps fill lk0/lv0 and read lk1/lv1, odd steps the reverse.
    auto prefetch = [&](int tt, v4i *lkw, v4i *lvw) {
        if (tt + 2 < ntiles) lds_load_k(lkw, kbase + (int64_t)(tt + 2) * kTileBytes, ldr, w);
        lds_load_v(lvw, vbase + (int64_t)tt * kTileBytes, ldr, w);
    };

    // step 0 (no P.V yet)
    prefetch(0, lk0, lv0);
    if (ntiles == 1) {
        if (partial) step<false, false, true>(sa, sb, lk1, lv1, qa, cq * ksb[0], tail_valid, hl, ql, rs, o);
        else step<false, false, false>(sa, sb, lk1, lv1, qa, cq * ksb[0], kTile, hl, ql, rs, o);
    } else {
        step<false, true, false>(sa, sb, lk1, lv1, qa, cq * ksb[0], kTile, hl, ql, rs, o);
    }
    wait_lds_loads_and_sync();
    // steps 1 .. ntiles-2, two per iteration (odd then even) so the score
    // registers and LDS buffers alternate statically
    int tt = 1;
    for (; tt + 2 < ntiles; tt += 2) {
        prefetch(tt, lk1, lv1);
        step<true, true, false>(sb, sa, lk0, lv0, qa, cq * ksb[tt], kTile, hl, ql, rs, o);
        wait_lds_loads_and_sync();
        prefetch(tt + 1, lk0, lv0);
        step<true, true, false>(sa, sb, lk1, lv1, qa, cq * ksb[tt + 1], kTile, hl, ql, rs, o);
        wait_lds_loads_and_sync();
    }
    if (tt + 1 < ntiles) {   // one more full odd step: scores in sb
        prefetch(tt, lk1, lv1);
        step<true, true, false>(sb, sa, lk0, lv0, qa, cq * ksb[tt], kTile, hl, ql, rs, o);
        wait_lds_loads_and_sync();
        tt++;
    }
    // last step tt = ntiles - 1 (if >= 1): odd -> scores in sb, reads lv0; even -> sa, lv1
    if (tt < ntiles) {
        const float c2 = cq * ksb[tt];
        if (tt & 1) {
            prefetch(tt, lk1, lv1);
            if (partial) step<true, false, true>(sb, sa, lk0, lv0, qa, c2, tail_valid, hl, ql, rs, o);
            else step<true, false, false>(sb, sa, lk0, lv0, qa, c2, kTile, hl, ql, rs, o);
        } else {
            prefetch(tt, lk0, lv0);
            if (partial) step<true, false, true>(sa, sb, lk1, lv1, qa, c2, tail_valid, hl, ql, rs, o);
            else step<true, false, false>(sa, sb, lk1, lv1, qa, c2, kTile, hl, ql, rs, o);
        }
        wait_lds_loads_and_sync();
    }
    // drain: P.V of the last tile (V(ntiles-1) sits in the buffer of its parity)
    if ((ntiles - 1) & 1) pv_tile(lv1, rs.pf, hl, ql, o);
    else pv_tile(lv0, rs.pf, hl, ql, o);
    const float lsum = rs.lsum;

    // Epilogue: the two lanes of a query hold different keys' partial sums.
    const float ltot = pair_sum(lsum);
    const float inv = 1.0f / ltot;
    const int n = q0 + ql;
    const float *svp = vs + bh * kD;
    if (OUTF < 0) {
        if (n < N) {
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
    } else {
        // MX blocks: channel block db (32 channels) of this query is split over the
        // lane pair (hl = 0, 1), 16 values each; the block maximum needs both.
        const int64_t row = ((int64_t)b * N + n) * H + h;   // token-major (b, n, h) row of 4 blocks
#pragma unroll
        for (int db = 0; db < 4; db++) {
            float x[16];
            float amax = 0.0f;
#pragma unroll
            for (int g = 0; g < 4; g++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int d = 32 * db + 8 * g + 4 * hl + i;
                    x[4 * g + i] = bf16_to_f32(f32_to_bf16(o[db][4 * g + i] * svp[d] * inv));
                    amax = fmaxf(amax, fabsf(x[4 * g + i]));
                }
            amax = pair_max(amax);
            const int X = mx_shared_exp(amax, OUTF == kMxE4M3 ? 8 : 2);
            const float sc = pow2f(-X);
            if (n < N) {
                const int64_t blk = row * (kD / kMxBlock) + db;
                if (hl == 0) mx_scales[blk] = (uint8_t)(X + 127);
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    const int e0 = 8 * g + 4 * hl;   // element index of x[4g] within the block
                    if (OUTF == kMxE4M3) {
                        const uint32_t wd = e4m3_encode(x[4 * g] * sc) | (e4m3_encode(x[4 * g + 1] * sc) << 8) |
                                            (e4m3_encode(x[4 * g + 2] * sc) << 16) |
                                            (e4m3_encode(x[4 * g + 3] * sc) << 24);
                        *reinterpret_cast<uint32_t *>(mx_codes + blk * kMxBlock + e0) = wd;
                    } else {
                        const uint32_t hw = e2m1_encode(x[4 * g] * sc) | (e2m1_encode(x[4 * g + 1] * sc) << 4) |
                                            (e2m1_encode(x[4 * g + 2] * sc) << 8) |
                                            (e2m1_encode(x[4 * g + 3] * sc) << 12);
                        *reinterpret_cast<uint16_t *>(mx_codes + blk * (kMxBlock / 2) + e0 / 2) = (uint16_t)hw;
                    }
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_attn_fwd(const int8_t *qc, const float *qs, const int8_t *kc, const float *ks, const uint8_t *vc,
                           const float *vs, int B, int N, int H, float sm_scale, OutView out, hipStream_t stream) {
    const int64_t Npad = ((int64_t)N + kNAlign - 1) / kNAlign * kNAlign;
    const int nqwg = (N + kQWg - 1) / kQWg;
    const int64_t blocks = (int64_t)nqwg * H * B;
    LAUNCH_OR_RETURN(attn_i8f8_kernel<-1>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, qc, qs, kc, ks, vc,
                       vs, N, H, Npad, sm_scale * kLog2E, out, nullptr, nullptr, nqwg);
    return hipSuccess;
}

hipError_t launch_attn_fwd_mx(const int8_t *qc, const float *qs, const int8_t *kc, const float *ks, const uint8_t *vc,
                              const float *vs, int B, int N, int H, float sm_scale, int fmt, uint8_t *codes,
                              uint8_t *scales, hipStream_t stream) {
    const int64_t Npad = ((int64_t)N + kNAlign - 1) / kNAlign * kNAlign;
    const int nqwg = (N + kQWg - 1) / kQWg;
    const int64_t blocks = (int64_t)nqwg * H * B;
    const OutView none{nullptr, 0, 0, 0};
    if (fmt == kMxE4M3)
        LAUNCH_OR_RETURN(attn_i8f8_kernel<kMxE4M3>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, qc, qs, kc,
                           ks, vc, vs, N, H, Npad, sm_scale * kLog2E, none, codes, scales, nqwg);
    else
        LAUNCH_OR_RETURN(attn_i8f8_kernel<kMxE2M1>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, qc, qs, kc,
                           ks, vc, vs, N, H, Npad, sm_scale * kLog2E, none, codes, scales, nqwg);
    return hipSuccess;
}

}  // namespace sage
