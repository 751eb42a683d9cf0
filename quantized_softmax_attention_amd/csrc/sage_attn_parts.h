// sage_attn_parts.h -- device pieces shared by the attention kernels of
// libsage_mi355x.so (INT8/FP8, INT8/bf16 and bf16): the wave geometry, the
// half-wave exchanges, HBM -> LDS tile staging, the INT8 K tile (codes written
// by sage_quantize_qk) and the row-major bf16 tile of a strided view.
//
// Common layout: a workgroup is 4 waves of 32 queries; with K as the A operand
// and Q^T as the B operand of a 32x32 MFMA, lane (hl, ql) = (lane / 32,
// lane % 32) holds query ql and, in register r of 32-key block kb, key
// 32 kb + 8 (r / 4) + 4 hl + r % 4.
#pragma once

#include "sage_common.h"

namespace sage {
namespace attn {

constexpr int kWaves = 4;                  // waves per workgroup
constexpr int kQWg = 32 * kWaves;          // queries per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2E = 1.4426950408889634f;

typedef __attribute__((address_space(3))) void lds_void;
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// v_permlane32_swap exchanges the upper half-wave of its first operand with the
// lower half-wave of its second.  With both operands x, one result holds x of
// lanes 0..31 in every lane position l % 32 and the other x of lanes 32..63, so
// combining the two gives every lane the value of its pair (l, l ^ 32).
__device__ __forceinline__ int pair_max(int x) {
    auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return max((int)r[0], (int)r[1]);
}
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// Two fp32 values as a bf16 pair (round to nearest even), a first.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    v2bf r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
}

// Wait for this wave's outstanding HBM -> LDS loads (vmcnt = 0), then the
// barrier.  The scheduling fences keep register-only work of neighbouring steps
// from drifting across it, so each step keeps its MFMA/VALU interleave.
__device__ __forceinline__ void wait_lds_loads_and_sync() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt, lgkmcnt unchanged
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
}

// O = alpha O, skipped (wave-uniformly) when no row's maximum moved.
__device__ __forceinline__ void rescale(float alpha, v16f (&o)[4]) {
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
        for (int db = 0; db < 4; db++)
#pragma unroll
            for (int r = 0; r < 16; r++) o[db][r] *= alpha;
    }
}

// Direct HBM -> LDS staging (buffer_load_dwordx4 ... lds): lane L of a wave's
// load instruction writes LDS bytes [16 L, 16 L + 16) after the instruction's
// LDS base, so each lane fetches the global chunk that belongs at its
// (swizzled) LDS slot.  The tile base lives in a buffer descriptor whose record
// limit bounds every access (reads past it return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void *tile, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(tile), 0, bytes, 0x00020000);
}

// ---- INT8 K tile: 64 key rows of 128 code bytes, contiguous in the code buffer
constexpr int kI8TileBytes = kTile * kD;       // 8 KB
constexpr int kI8Chunks = kI8TileBytes / 16;   // 512 16-byte chunks

// LDS slot of 16-byte chunk c (0..7) of K row r (0..63) (conflict-free for the
// fragment reads: 32 rows x one chunk).
__device__ __forceinline__ int k_slot(int r, int c) { return r * 8 + (c ^ ((r ^ (r >> 3)) & 7)); }

// Wave w fills slots [128 w, 128 w + 128) of a tile: lane L of load i slot
// 128 w + 64 i + L.  Per-lane source offsets within the tile:
struct K8Loader {
    int off[2];
};
__device__ __forceinline__ K8Loader make_k8_loader(int w, int lane) {
    K8Loader L;
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int slot = 128 * w + 64 * i + lane;
        const int r = slot >> 3, rc = slot & 7;   // LDS slot -> row, stored chunk
        L.off[i] = r * 128 + 16 * (rc ^ ((r ^ (r >> 3)) & 7));
    }
    return L;
}
__device__ __forceinline__ void lds_load_k8(v4i *lk, const int8_t *tile, const K8Loader &L, int w) {
    const auto r = tile_rsrc(tile, kI8TileBytes);
#pragma unroll
    for (int i = 0; i < 2; i++)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(lk + 128 * w + 64 * i), 16, L.off[i], 0, 0, 0);
}

// K operand of INT8 MFMA i (0..7): 32-key block i % 2, 32-channel k-step i / 2.
__device__ __forceinline__ v4i k8_operand(const v4i *lk, int i, int hl, int ql) {
    const int kb = i & 1, st = i >> 1;
    return lk[k_slot(32 * kb + ql, 2 * st + hl)];
}

// S^T = K Q^T for one tile (the two accumulation chains alternate).
__device__ __forceinline__ void qk8_tile(const v4i *lk, const v4i (&qa)[4], int hl, int ql, v16i (&s)[2]) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int kb = i & 1, st = i >> 1;
        s[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(k8_operand(lk, i, hl, ql), qa[st], st ? s[kb] : v16i{}, 0, 0,
                                                      0);
    }
}

// Running maximum after one tile, from its int32 scores (log2 units; c2 >= 0 so
// the maximum of c2 * a is c2 * max a).  TAIL first masks keys >= nvalid.
template <bool TAIL>
__device__ __forceinline__ float tile_max_i32(v16i (&s)[2], float c2, int nvalid, int hl, float m2) {
    if (TAIL) {
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                if (32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3) >= nvalid) s[kb][r] = INT32_MIN;
    }
    // a chain of 3-input maxima: 16 v_max3_i32 for 32 values
    int imax = max(max(s[0][0], s[0][1]), s[0][2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) imax = max(max(imax, s[0][r]), s[0][r + 1]);
    imax = max(max(imax, s[0][15]), s[1][0]);
#pragma unroll
    for (int r = 1; r < 15; r += 2) imax = max(max(imax, s[1][r]), s[1][r + 1]);
    imax = max(imax, s[1][15]);
    imax = pair_max(imax);
    return fmaxf(m2, c2 * (float)imax);
}

// ---- bf16 tile of a strided view: 64 key rows x 128 channels, row-major in
// LDS (256 B per row), staged from rows that sit row_bytes apart in HBM
constexpr int kRowBytes16 = kD * 2;                 // 256 B per key row
constexpr int kTileBytes16 = kTile * kRowBytes16;   // 16 KB
constexpr int kChunks16 = kTileBytes16 / 16;        // 1024 16-byte chunks

// Stored 16-byte chunk of source chunk c (0..15) in key row r.  K: fragment
// reads take one chunk of 16 consecutive rows per 16-lane cycle, so c ^ (r % 16)
// spreads them over all 16 slots of a 256-byte bank line.  V: each 32-lane cycle
// of a transposing read takes 8 bytes from 4 consecutive rows x 8 units, and
// c ^ 4 (r % 4) puts the four rows on different 64-byte quarters.  Both are
// involutions, so the same map gives the source chunk of a stored slot.
__device__ __forceinline__ int k_chunk16(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int v_chunk16(int r, int c) { return c ^ ((r & 3) << 2); }

// Wave w fills slots [256 w, 256 w + 256): lane L of load i slot 256 w + 64 i + L.
__device__ __forceinline__ void make_k16_offsets(int w, int lane, int64_t row_bytes, int (&off)[4]) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int slot = 256 * w + 64 * i + lane;
        const int r = slot >> 4, cs = slot & 15;
        off[i] = (int)(r * row_bytes) + 16 * k_chunk16(r, cs);
    }
}
__device__ __forceinline__ void make_v16_offsets(int w, int lane, int64_t row_bytes, int (&off)[4]) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int slot = 256 * w + 64 * i + lane;
        const int r = slot >> 4, cs = slot & 15;
        off[i] = (int)(r * row_bytes) + 16 * v_chunk16(r, cs);
    }
}

// The record limit is the tile's valid rows, so rows at or beyond N read as zero.
__device__ __forceinline__ void lds_load16(v4i *lbuf, const uint16_t *tile, int rows_valid, int64_t row_bytes,
                                           const int (&off)[4], int w) {
    const auto rs = tile_rsrc(tile, (int)(rows_valid * row_bytes));
#pragma unroll
    for (int i = 0; i < 4; i++)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(lbuf + 256 * w + 64 * i), 16, off[i], 0, 0, 0);
}

// V^T operand of k-step ks (16 keys), channel block db: two transposing reads
// (keys 16ks + 4u + 0..3 and 16ks + 8 + 4u + 0..3).  ds_read_b64_tr_b16 hands,
// within each 16-lane group, lane i element i%4 of the 8-byte reads of lanes
// 4j + i/4, j = 0..3; lane s = 4j + a of the group reads 4 channels (a quad) of
// key row 16ks + 4u + j.
__device__ __forceinline__ v8bf v16_operand(const v4i *lv, int lane, int ks, int db) {
    const int g = lane >> 4, s = lane & 15, j = s >> 2, a = s & 3;
    const int u = g >> 1, g2 = g & 1;
    const int c = 4 * db + 2 * g2 + (a >> 1);   // source 16-byte chunk of the channel quad
    const char *base = reinterpret_cast<const char *>(lv);
    const int r0 = 16 * ks + 4 * u + j, r1 = r0 + 8;
    lds_v4s *p0 = (lds_v4s *)(base + r0 * kRowBytes16 + 16 * v_chunk16(r0, c) + 8 * (a & 1));
    lds_v4s *p1 = (lds_v4s *)(base + r1 * kRowBytes16 + 16 * v_chunk16(r1, c) + 8 * (a & 1));
    v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p0);
    v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p1);
    v8s both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(v8bf, both);
}

// O^T += V^T P^T with bf16 P (pw: four k-steps of four bf16 pairs) and a bf16 V tile.
__device__ __forceinline__ void pv16_tile(const v4i *lv, const uint32_t (&pw)[16], int lane, v16f (&o)[4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
        const v8bf pb = __builtin_bit_cast(v8bf, make_uint4(pw[4 * ks], pw[4 * ks + 1], pw[4 * ks + 2], pw[4 * ks + 3]));
#pragma unroll
        for (int db = 0; db < 4; db++)
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v16_operand(lv, lane, ks, db), pb, o[db], 0, 0, 0);
    }
}

}  // namespace attn
}  // namespace sage
