// sage_attn_int8qk.hip -- INT8 Q K^T with an unquantised (bf16) P.V for gfx950:
// the precision split the profile page runs as "sol_int8_qk"
// ("gb10-sampling-component-profile-1344x768-124f-seed440420.json",
// sampling_stage_step_2_seconds.sol_int8_qk_tau_1_3_exact_conditioning_kv:
// Q/K quantised, V left unquantised), used here densely.
//
// Scores come from the INT8 codes and scales sage_quantize_qk writes, exactly as
// in the fully quantised kernel (v_mfma_i32_32x32x32_i8, S^T = K Q^T, one query
// per lane, running maximum on the int32 scores).  P stays in fp32 for the
// normaliser and is rounded to bf16 for the product with the bf16 V read
// straight from its strided [B, N, H, D] view (v_mfma_f32_32x32x16_bf16,
// O^T = V^T P^T), so no V quantisation pass is needed.
//
// Per wave and 64-key tile: the 32x32 INT8 accumulator gives lane (hl, ql)
// register r of block kb = key 32 kb + 8 (r / 4) + 4 hl + r % 4 of query ql;
// taken eight registers at a time these are, unchanged, the bf16 P^T B operand
// of the k-steps of 16 keys (element e of k-step ks = key
// 16 ks + 8 (e / 4) + 4 hl + e % 4), and the matching V^T operand comes from
// ds_read_b64_tr_b16 of the row-major V tile.
#include "sage_attn_parts.h"

namespace sage {

namespace {

using namespace attn;

struct RowState {
    float m2, lsum;    // running maximum (log2 units) and this lane's running sum of p
    uint32_t pw[16];   // bf16 P^T operand of the last processed tile (its P.V is pending)
};

// p = exp(s - m) for registers 4c..4c+3 of the tile (c = 0..7), summed in fp32
// and packed to bf16 pairs in the P^T operand order.
template <bool TAIL>
__device__ __forceinline__ void tile_exp_chunk(const v16i (&s)[2], float c2, float mnew, int nvalid, int hl, int c,
                                               uint32_t (&pw)[16], float &part) {
    const int kb = c >> 2, r = 4 * (c & 3);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        p[i] = fast_exp2(c2 * (float)s[kb][r + i] - mnew);
        if (TAIL && 32 * kb + 8 * (r >> 2) + 4 * hl + i >= nvalid) p[i] = 0.0f;
    }
    const float chunk = (p[0] + p[1]) + (p[2] + p[3]);
    part = c == 0 ? chunk : part + chunk;   // (no add of the initial zero)
    const int ks = 2 * kb + (r >> 3), e0 = r & 7;
    pw[4 * ks + (e0 >> 1)] = pack_bf16(p[0], p[1]);
    pw[4 * ks + (e0 >> 1) + 1] = pack_bf16(p[2], p[3]);
}

// One pipeline step for tile t: P.V of tile t-1 (16 bf16 MFMAs, spread over the
// step), the running maximum and p of tile t with the 8 INT8 QK^T MFMAs of tile
// t+1 interleaved, then the rescale of O (a branch, taken only when some row's
// maximum moved).
template <bool PV, bool QK, bool TAIL>
__device__ __forceinline__ void step(v16i (&s)[2], v16i (&sn)[2], const v4i *lk_next, const v4i *lv_prev,
                                     const v4i (&qa)[4], float c2, int nvalid, int lane, int hl, int ql,
                                     RowState &st, v16f (&o)[4]) {
    // P.V MFMA j (0..15) = k-step j / 4, channel block j % 4.  Six of them run
    // beside the max reduction, the rest two per exp chunk (chunks 0..4), each
    // before the chunk that first overwrites its k-step of the P operand.
    v8bf pb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ks++)
        pb[ks] = __builtin_bit_cast(v8bf, make_uint4(st.pw[4 * ks], st.pw[4 * ks + 1], st.pw[4 * ks + 2],
                                                     st.pw[4 * ks + 3]));
    auto pv = [&](int j) {
        const int ks = j >> 2, db = j & 3;
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v16_operand(lv_prev, lane, ks, db), pb[ks], o[db], 0, 0, 0);
    };
    v4i ka[3];
    if (QK) {
        ka[0] = k8_operand(lk_next, 0, hl, ql);
        ka[1] = k8_operand(lk_next, 1, hl, ql);
    }
    if (PV) {   // O = alpha(t-1) acc(t-2) + P(t-1) V(t-1), first six MFMAs
#pragma unroll
        for (int j = 0; j < 6; j++) pv(j);
    }
    const float mnew = tile_max_i32<TAIL>(s, c2, nvalid, hl, st.m2);
    const float alpha = fast_exp2(st.m2 - mnew);   // 0 on the first tile (m2 = -inf)
    st.m2 = mnew;
    float part = 0.0f;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < 8; c++) {
        if (QK) {
            if (c < 6) ka[(c + 2) % 3] = k8_operand(lk_next, c + 2, hl, ql);
            const int kb = c & 1, kst = c >> 1;
            sn[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka[c % 3], qa[kst], kst ? sn[kb] : v16i{}, 0, 0, 0);
        }
        if (PV && c < 5) {
            pv(6 + 2 * c);
            pv(7 + 2 * c);
        }
        tile_exp_chunk<TAIL>(s, c2, mnew, nvalid, hl, c, st.pw, part);
        asm volatile("" ::"v"(part));
        __builtin_amdgcn_sched_barrier(0);
    }
    // Everything above is consumed only after the rescale branch; reading it
    // here keeps it (and the MFMAs) inside this step's schedule.
#pragma unroll
    for (int i = 0; i < 16; i++) asm volatile("" ::"v"(st.pw[i]));
    asm volatile("" ::"v"(part));
    if (QK) asm volatile("" ::"v"(sn[0]), "v"(sn[1]));
    __builtin_amdgcn_sched_barrier(0);
    st.lsum = st.lsum * alpha + part;
    if (PV) rescale(alpha, o);                    // O = alpha(t) acc(t-1)
}

// Software pipeline per wave as in the fully quantised kernel: step t reads
// K(t+1) (INT8 codes, 8 KB) and V(t-1) (bf16 rows, 16 KB) from LDS and stages
// K(t+2) and V(t) into the buffers of K(t) and V(t-2).
__global__ __launch_bounds__(kThreads, 2) void attn_int8qk_kernel(
    const int8_t *__restrict__ qc, const float *__restrict__ qs, const int8_t *__restrict__ kc,
    const float *__restrict__ ks, View V, int N, int H, int64_t Npad, float c_base, OutView out, int nqwg) {
    __shared__ v4i lk0[kI8Chunks], lk1[kI8Chunks], lv0[kChunks16], lv1[kChunks16];

    const uint32_t id = xcd_remap(blockIdx.x, gridDim.x);
    const int qb = (int)(id % (uint32_t)nqwg);
    const int64_t bh = id / (uint32_t)nqwg;
    const int b = (int)(bh / H), h = (int)(bh % H);
    const int t = threadIdx.x, lane = t & 63, hl = lane >> 5, ql = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform: LDS addresses stay scalar
    const int q0 = qb * kQWg + 32 * w;

    const int8_t *qrow = qc + (bh * Npad + q0 + ql) * kD + 16 * hl;
    v4i qa[4];
#pragma unroll
    for (int st = 0; st < 4; st++) qa[st] = *reinterpret_cast<const v4i *>(qrow + 32 * st);
    const float cq = qs[bh * (Npad / kQBlock) + q0 / kQBlock] * c_base;
    const float *ksb = ks + bh * (Npad / kKBlock);
    const int8_t *kbase = kc + bh * Npad * kD;
    const uint16_t *vbase = V.data + (int64_t)b * V.sb + (int64_t)h * V.sh;
    const int64_t vrow = V.sn * 2;

    const int ntiles = (N + kTile - 1) / kTile;
    const int tail_valid = N - (ntiles - 1) * kTile;
    const bool partial = tail_valid != kTile;
    auto rows = [&](int tt) { return min(kTile, N - tt * kTile); };

    v16f o[4];
#pragma unroll
    for (int db = 0; db < 4; db++) o[db] = v16f{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    RowState rs;
    rs.m2 = -INFINITY;
    rs.lsum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++) rs.pw[i] = 0;

    const K8Loader kl = make_k8_loader(w, lane);
    int voff[4];
    make_v16_offsets(w, lane, vrow, voff);

    lds_load_k8(lk0, kbase, kl, w);
    if (ntiles > 1) lds_load_k8(lk1, kbase + kI8TileBytes, kl, w);
    wait_lds_loads_and_sync();
    v16i sa[2], sb[2];
    qk8_tile(lk0, qa, hl, ql, sa);
    __syncthreads();

    auto prefetch = [&](int tt, v4i *lkw, v4i *lvw) {
        if (tt + 2 < ntiles) lds_load_k8(lkw, kbase + (int64_t)(tt + 2) * kI8TileBytes, kl, w);
        lds_load16(lvw, vbase + (int64_t)tt * kTile * V.sn, rows(tt), vrow, voff, w);
    };

    prefetch(0, lk0, lv0);
    if (ntiles == 1) {
        if (partial) step<false, false, true>(sa, sb, lk1, lv1, qa, cq * ksb[0], tail_valid, lane, hl, ql, rs, o);
        else step<false, false, false>(sa, sb, lk1, lv1, qa, cq * ksb[0], kTile, lane, hl, ql, rs, o);
    } else {
        step<false, true, false>(sa, sb, lk1, lv1, qa, cq * ksb[0], kTile, lane, hl, ql, rs, o);
    }
    wait_lds_loads_and_sync();
    int tt = 1;
    for (; tt + 2 < ntiles; tt += 2) {
        prefetch(tt, lk1, lv1);
        step<true, true, false>(sb, sa, lk0, lv0, qa, cq * ksb[tt], kTile, lane, hl, ql, rs, o);
        wait_lds_loads_and_sync();
        prefetch(tt + 1, lk0, lv0);
        step<true, true, false>(sa, sb, lk1, lv1, qa, cq * ksb[tt + 1], kTile, lane, hl, ql, rs, o);
        wait_lds_loads_and_sync();
    }
    if (tt + 1 < ntiles) {
        prefetch(tt, lk1, lv1);
        step<true, true, false>(sb, sa, lk0, lv0, qa, cq * ksb[tt], kTile, lane, hl, ql, rs, o);
        wait_lds_loads_and_sync();
        tt++;
    }
    if (tt < ntiles) {
        const float c2 = cq * ksb[tt];
        if (tt & 1) {
            prefetch(tt, lk1, lv1);
            if (partial) step<true, false, true>(sb, sa, lk0, lv0, qa, c2, tail_valid, lane, hl, ql, rs, o);
            else step<true, false, false>(sb, sa, lk0, lv0, qa, c2, kTile, lane, hl, ql, rs, o);
        } else {
            prefetch(tt, lk0, lv0);
            if (partial) step<true, false, true>(sa, sb, lk1, lv1, qa, c2, tail_valid, lane, hl, ql, rs, o);
            else step<true, false, false>(sa, sb, lk1, lv1, qa, c2, kTile, lane, hl, ql, rs, o);
        }
        wait_lds_loads_and_sync();
    }
    if ((ntiles - 1) & 1) pv16_tile(lv1, rs.pw, lane, o);
    else pv16_tile(lv0, rs.pw, lane, o);

    const float inv = 1.0f / pair_sum(rs.lsum);
    const int n = q0 + ql;
    if (n < N) {
        uint16_t *orow = out.data + (int64_t)b * out.sb + (int64_t)n * out.sn + (int64_t)h * out.sh;
#pragma unroll
        for (int db = 0; db < 4; db++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int d0 = 32 * db + 8 * g + 4 * hl;   // registers 4g..4g+3: channels d0..d0+3
                uint32_t lo = f32_to_bf16(o[db][4 * g] * inv) | (f32_to_bf16(o[db][4 * g + 1] * inv) << 16);
                uint32_t hi = f32_to_bf16(o[db][4 * g + 2] * inv) | (f32_to_bf16(o[db][4 * g + 3] * inv) << 16);
                *reinterpret_cast<uint2 *>(orow + d0) = make_uint2(lo, hi);
            }
    }
}

}  // namespace

hipError_t launch_attn_fwd_int8qk(const int8_t *qc, const float *qs, const int8_t *kc, const float *ks, View v,
                                  int B, int N, int H, float sm_scale, OutView out, hipStream_t stream) {
    const int64_t Npad = ((int64_t)N + kNAlign - 1) / kNAlign * kNAlign;
    const int nqwg = (N + kQWg - 1) / kQWg;
    const int64_t blocks = (int64_t)nqwg * H * B;
    LAUNCH_OR_RETURN(attn_int8qk_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, qc, qs, kc, ks, v, N,
                       H, Npad, sm_scale * kLog2E, out, nqwg);
    return hipSuccess;
}

}  // namespace sage
