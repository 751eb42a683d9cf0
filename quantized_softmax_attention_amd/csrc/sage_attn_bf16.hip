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
// those values are, unchanged, the P^T B operand of the second product.  For
// k-step ks (16 keys) lane half u element e pairs with key
// 16*ks + 8*(e/4) + 4*u + e%4.  K and V tiles are staged row-major ([key][128
// channels], 256 B per row) straight from HBM into LDS; the V^T operand (one
// channel, 4 keys per lane) comes from ds_read_b64_tr_b16, which within each
// 16-lane group hands lane i element i%4 of the 8-byte reads of lanes
// 4j + i/4, j = 0..3.
#include "sage_attn_parts.h"

namespace sage {

namespace {

using namespace attn;

// QK^T MFMA i (0..15): block i%2, 16-channel k-step i/2.
__device__ __forceinline__ void qk_mfma(const v4i *lk, const v8bf (&qa)[8], int hl, int ql, v16f (&s)[2], int i) {
    const int kb = i & 1, st = i >> 1;
    const int r = 32 * kb + ql;
    v8bf ka = __builtin_bit_cast(v8bf, lk[r * 16 + k_chunk16(r, 2 * st + hl)]);
    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qa[st], st ? s[kb] : v16f{}, 0, 0, 0);
}

template <bool TAIL>
__device__ __forceinline__ float tile_max(v16f (&s)[2], float c2, int nvalid, int hl, float m2) {
    if (TAIL) {
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                if (32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3) >= nvalid) s[kb][r] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) mx = fmaxf(fmaxf(mx, s[0][r]), s[0][r + 1]);
    mx = fmaxf(fmaxf(mx, s[0][15]), s[1][0]);
#pragma unroll
    for (int r = 1; r < 15; r += 2) mx = fmaxf(fmaxf(mx, s[1][r]), s[1][r + 1]);
    mx = fmaxf(mx, s[1][15]);
    mx = pair_max(mx);
    return fmaxf(m2, c2 * mx);
}

// p = exp(s - m) for registers 4c..4c+3 (c = 0..7), summed in fp32, packed to
// bf16 pairs: registers r..r+3 of block kb are elements e0..e0+3 of k-step
// 2 kb + r/8, e0 = r % 8.
template <bool TAIL>
__device__ __forceinline__ void tile_exp_chunk(const v16f (&s)[2], float c2, float mnew, int nvalid, int hl, int c,
                                               uint32_t (&pw)[16], float &part) {
    const int kb = c >> 2, r = 4 * (c & 3);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        p[i] = fast_exp2(c2 * s[kb][r + i] - mnew);
        if (TAIL && 32 * kb + 8 * (r >> 2) + 4 * hl + i >= nvalid) p[i] = 0.0f;
    }
    const float chunk = (p[0] + p[1]) + (p[2] + p[3]);
    part = c == 0 ? chunk : part + chunk;   // (no add of the initial zero)
    const int ks = 2 * kb + (r >> 3), e0 = r & 7;
    pw[4 * ks + (e0 >> 1)] = pack_bf16(p[0], p[1]);
    pw[4 * ks + (e0 >> 1) + 1] = pack_bf16(p[2], p[3]);
}

struct RowState {
    float m2, lsum;
    uint32_t pw[16];   // bf16 P^T operand of the last processed tile (its P.V pending)
};

// One pipeline step (see the quantised kernel): P.V of tile t-1, max and exp of
// tile t with the 16 QK^T MFMAs of tile t+1 interleaved, then the rescale.
template <bool PV, bool QK, bool TAIL>
__device__ __forceinline__ void step(v16f (&s)[2], v16f (&sn)[2], const v4i *lk_next, const v4i *lv_prev,
                                     const v8bf (&qa)[8], float c2, int nvalid, int lane, int hl, int ql,
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
    if (PV) {
#pragma unroll
        for (int j = 0; j < 6; j++) pv(j);
    }
    const float mnew = tile_max<TAIL>(s, c2, nvalid, hl, st.m2);
    const float alpha = fast_exp2(st.m2 - mnew);
    st.m2 = mnew;
    float part = 0.0f;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < 8; c++) {
        if (QK) {
            qk_mfma(lk_next, qa, hl, ql, sn, 2 * c);
            qk_mfma(lk_next, qa, hl, ql, sn, 2 * c + 1);
        }
        if (PV && c < 5) {
            pv(6 + 2 * c);
            pv(7 + 2 * c);
        }
        tile_exp_chunk<TAIL>(s, c2, mnew, nvalid, hl, c, st.pw, part);
        asm volatile("" ::"v"(part));
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < 16; i++) asm volatile("" ::"v"(st.pw[i]));
    if (QK) asm volatile("" ::"v"(sn[0]), "v"(sn[1]));
    __builtin_amdgcn_sched_barrier(0);
    st.lsum = st.lsum * alpha + part;
    if (PV) rescale(alpha, o);
}

__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(View Q, View K, View V, int N, int H, float c2,
                                                               OutView out, int nqwg) {
    __shared__ v4i lk0[kChunks16], lk1[kChunks16], lv0[kChunks16], lv1[kChunks16];

    const uint32_t id = xcd_remap(blockIdx.x, gridDim.x);
    const int qb = (int)(id % (uint32_t)nqwg);
    const int64_t bh = id / (uint32_t)nqwg;
    const int b = (int)(bh / H), h = (int)(bh % H);
    const int t = threadIdx.x, lane = t & 63, hl = lane >> 5, ql = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform: LDS addresses stay scalar
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
    const uint16_t *kbase = K.data + (int64_t)b * K.sb + (int64_t)h * K.sh;
    const uint16_t *vbase = V.data + (int64_t)b * V.sb + (int64_t)h * V.sh;
    const int64_t krow = K.sn * 2, vrow = V.sn * 2;
    int koff[4], voff[4];
    make_k16_offsets(w, lane, krow, koff);
    make_v16_offsets(w, lane, vrow, voff);
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

    lds_load16(lk0, kbase, rows(0), krow, koff, w);
    if (ntiles > 1) lds_load16(lk1, kbase + (int64_t)kTile * K.sn, rows(1), krow, koff, w);
    wait_lds_loads_and_sync();
    v16f sa[2], sb[2];
#pragma unroll
    for (int i = 0; i < 16; i++) qk_mfma(lk0, qa, hl, ql, sa, i);
    __syncthreads();

    auto prefetch = [&](int tt, v4i *lkw, v4i *lvw) {
        if (tt + 2 < ntiles) lds_load16(lkw, kbase + (int64_t)(tt + 2) * kTile * K.sn, rows(tt + 2), krow, koff, w);
        lds_load16(lvw, vbase + (int64_t)tt * kTile * V.sn, rows(tt), vrow, voff, w);
    };

    prefetch(0, lk0, lv0);
    if (ntiles == 1) {
        if (partial) step<false, false, true>(sa, sb, lk1, lv1, qa, c2, tail_valid, lane, hl, ql, rs, o);
        else step<false, false, false>(sa, sb, lk1, lv1, qa, c2, kTile, lane, hl, ql, rs, o);
    } else {
        step<false, true, false>(sa, sb, lk1, lv1, qa, c2, kTile, lane, hl, ql, rs, o);
    }
    wait_lds_loads_and_sync();
    int tt = 1;
    for (; tt + 2 < ntiles; tt += 2) {
        prefetch(tt, lk1, lv1);
        step<true, true, false>(sb, sa, lk0, lv0, qa, c2, kTile, lane, hl, ql, rs, o);
        wait_lds_loads_and_sync();
        prefetch(tt + 1, lk0, lv0);
        step<true, true, false>(sa, sb, lk1, lv1, qa, c2, kTile, lane, hl, ql, rs, o);
        wait_lds_loads_and_sync();
    }
    if (tt + 1 < ntiles) {
        prefetch(tt, lk1, lv1);
        step<true, true, false>(sb, sa, lk0, lv0, qa, c2, kTile, lane, hl, ql, rs, o);
        wait_lds_loads_and_sync();
        tt++;
    }
    if (tt < ntiles) {
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
    LAUNCH_OR_RETURN(attn_bf16_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, q, k, v, N, H,
                       sm_scale * kLog2E, out, nqwg);
    return hipSuccess;
}

}  // namespace sage
