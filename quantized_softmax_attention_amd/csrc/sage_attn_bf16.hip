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
#include "sage_common.h"

namespace sage {

namespace {

constexpr int kWaves = 4;
constexpr int kQWg = 32 * kWaves;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowBytes = kD * 2;                 // 256 B per key row
constexpr int kTileBytes16 = kTile * kRowBytes;   // 16 KB per K or V tile
constexpr int kChunks16 = kTileBytes16 / 16;      // 1024 16-byte chunks
constexpr float kLog2E = 1.4426950408889634f;

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4s lds_v4s;

// Stored 16-byte chunk of source chunk c (0..15) in key row r.  K: fragment
// reads take one chunk of 16 consecutive rows per 16-lane cycle, so c ^ (r % 16)
// spreads them over all 16 slots of a 256-byte bank line.  V: each 32-lane cycle
// of a transposing read takes 8 bytes from 4 consecutive rows x 8 units, and
// c ^ 4 (r % 4) puts the four rows on different 64-byte quarters.
__device__ __forceinline__ int k_chunk(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int v_chunk(int r, int c) { return c ^ ((r & 3) << 2); }

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

// HBM -> LDS staging of a 64-row tile of a strided view (buffer_load ... lds).
// Wave w issues LDS slots [256 w, 256 w + 256); lane L of instruction i writes
// slot 256 w + 64 i + L.  The descriptor's record limit is the tile's valid
// rows, so rows at or beyond N read as zero.
struct Loader16 {
    int koff[4], voff[4];   // per-lane source byte offsets within a K / V tile
};

__device__ __forceinline__ Loader16 make_loader16(int w, int lane, int64_t krow_bytes, int64_t vrow_bytes) {
    Loader16 L;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int slot = 256 * w + 64 * i + lane;
        const int r = slot >> 4, cs = slot & 15;
        L.koff[i] = (int)(r * krow_bytes) + 16 * k_chunk(r, cs);   // k_chunk is an involution
        L.voff[i] = (int)(r * vrow_bytes) + 16 * v_chunk(r, cs);
    }
    return L;
}

__device__ __forceinline__ void lds_load(v4i *lbuf, const uint16_t *tile, int rows_valid, int64_t row_bytes,
                                         const int (&off)[4], int w) {
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(tile), 0,
                                                      (int)(rows_valid * row_bytes), 0x00020000);
#pragma unroll
    for (int i = 0; i < 4; i++)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(lbuf + 256 * w + 64 * i), 16, off[i], 0, 0, 0);
}

__device__ __forceinline__ void wait_lds_loads_and_sync() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
}

// QK^T MFMA i (0..15): block i%2, 16-channel k-step i/2.
__device__ __forceinline__ void qk_mfma(const v4i *lk, const v8bf (&qa)[8], int hl, int ql, v16f (&s)[2], int i) {
    const int kb = i & 1, st = i >> 1;
    const int r = 32 * kb + ql;
    v8bf ka = __builtin_bit_cast(v8bf, lk[r * 16 + k_chunk(r, 2 * st + hl)]);
    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qa[st], st ? s[kb] : v16f{}, 0, 0, 0);
}

// V^T operand of k-step ks, channel block db: two transposing reads (keys
// 16ks + 4u + 0..3 and 16ks + 8 + 4u + 0..3).  Lane s = 4j + a of each 16-lane
// group reads 4 channels (a quad) of key row 16ks + 4u + j.
__device__ __forceinline__ v8bf v_operand(const v4i *lv, int lane, int ks, int db) {
    const int g = lane >> 4, s = lane & 15, j = s >> 2, a = s & 3;
    const int u = g >> 1, g2 = g & 1;
    const int c = 4 * db + 2 * g2 + (a >> 1);                // source 16-byte chunk of the channel quad
    const char *base = reinterpret_cast<const char *>(lv);
    const int r0 = 16 * ks + 4 * u + j, r1 = r0 + 8;
    lds_v4s *p0 = (lds_v4s *)(base + r0 * kRowBytes + 16 * v_chunk(r0, c) + 8 * (a & 1));
    lds_v4s *p1 = (lds_v4s *)(base + r1 * kRowBytes + 16 * v_chunk(r1, c) + 8 * (a & 1));
    v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p0);
    v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p1);
    typedef short v8s __attribute__((ext_vector_type(8)));
    v8s both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(v8bf, both);
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
    part += (p[0] + p[1]) + (p[2] + p[3]);
    const int ks = 2 * kb + (r >> 3), e0 = r & 7;
    pw[4 * ks + (e0 >> 1)] = pack_bf16(p[0], p[1]);
    pw[4 * ks + (e0 >> 1) + 1] = pack_bf16(p[2], p[3]);
}

__device__ __forceinline__ void pv_tile(const v4i *lv, const uint32_t (&pw)[16], int lane, v16f (&o)[4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
        const v8bf pb = __builtin_bit_cast(v8bf, make_uint4(pw[4 * ks], pw[4 * ks + 1], pw[4 * ks + 2], pw[4 * ks + 3]));
#pragma unroll
        for (int db = 0; db < 4; db++)
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand(lv, lane, ks, db), pb, o[db], 0, 0, 0);
    }
}

__device__ __forceinline__ void rescale(float alpha, v16f (&o)[4]) {
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
        for (int db = 0; db < 4; db++)
#pragma unroll
            for (int r = 0; r < 16; r++) o[db][r] *= alpha;
    }
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
    if (PV) pv_tile(lv_prev, st.pw, lane, o);
    const float mnew = tile_max<TAIL>(s, c2, nvalid, hl, st.m2);
    const float alpha = fast_exp2(st.m2 - mnew);
    st.m2 = mnew;
    float part = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; c++) {
        if (QK) {
            qk_mfma(lk_next, qa, hl, ql, sn, 2 * c);
            qk_mfma(lk_next, qa, hl, ql, sn, 2 * c + 1);
        }
        tile_exp_chunk<TAIL>(s, c2, mnew, nvalid, hl, c, st.pw, part);
    }
    asm volatile("" ::"v"(st.pw[0]), "v"(st.pw[4]), "v"(st.pw[8]), "v"(st.pw[12]), "v"(part));
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
    const uint16_t *kbase = K.data + (int64_t)b * K.sb + (int64_t)h * K.sh;
    const uint16_t *vbase = V.data + (int64_t)b * V.sb + (int64_t)h * V.sh;
    const int64_t krow = K.sn * 2, vrow = V.sn * 2;
    const Loader16 ldr = make_loader16(w, lane, krow, vrow);
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

    lds_load(lk0, kbase, rows(0), krow, ldr.koff, w);
    if (ntiles > 1) lds_load(lk1, kbase + (int64_t)kTile * K.sn, rows(1), krow, ldr.koff, w);
    wait_lds_loads_and_sync();
    v16f sa[2], sb[2];
#pragma unroll
    for (int i = 0; i < 16; i++) qk_mfma(lk0, qa, hl, ql, sa, i);
    __syncthreads();

    auto prefetch = [&](int tt, v4i *lkw, v4i *lvw) {
        if (tt + 2 < ntiles) lds_load(lkw, kbase + (int64_t)(tt + 2) * kTile * K.sn, rows(tt + 2), krow, ldr.koff, w);
        lds_load(lvw, vbase + (int64_t)tt * kTile * V.sn, rows(tt), vrow, ldr.voff, w);
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
    if ((ntiles - 1) & 1) pv_tile(lv1, rs.pw, lane, o);
    else pv_tile(lv0, rs.pw, lane, o);

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
    hipLaunchKernelGGL(attn_bf16_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, q, k, v, N, H,
                       sm_scale * kLog2E, out, nqwg);
    return hipGetLastError();
}

}  // namespace sage
