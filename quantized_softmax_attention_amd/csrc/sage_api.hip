// sage_api.hip -- the C ABI of libsage_mi355x.so (declared in sage_mi355x.h):
// host-side argument validation, then asynchronous launches on the caller's
// stream.  No allocation, no synchronisation, no global mutable state.
#include <cmath>
#include <cstdint>
#include <mutex>

#include "sage_common.h"
#include "sage_norm_rope.h"

namespace sage {
hipError_t launch_quantize_qk(View q, View k, int B, int N, int H, int8_t *qc, float *qs, int8_t *kc,
                              float *ks, float *km, void *workspace, hipStream_t stream);
hipError_t launch_quantize_v(View v, int B, int N, int H, uint8_t *vc, float *vs, void *workspace,
                             hipStream_t stream);
hipError_t launch_quantize_qkv(View q, View k, View v, int B, int N, int H, const NormRope *nr, int8_t *qc, float *qs,
                               int8_t *kc, float *ks, float *km, uint8_t *vc, float *vs, void *workspace,
                               hipStream_t stream);
hipError_t launch_norm_rope(OutView q, OutView k, int B, int N, int H, NormRope nr, hipStream_t stream);
hipError_t launch_attn_fwd(const int8_t *qc, const float *qs, const int8_t *kc, const float *ks, const uint8_t *vc,
                           const float *vs, int B, int N, int H, float sm_scale, OutView out, hipStream_t stream);
hipError_t launch_attn_fwd_mx(const int8_t *qc, const float *qs, const int8_t *kc, const float *ks, const uint8_t *vc,
                              const float *vs, int B, int N, int H, float sm_scale, int fmt, uint8_t *codes,
                              uint8_t *scales, hipStream_t stream);
hipError_t launch_mx_quantize(View x, int B, int N, int H, int fmt, uint8_t *codes, uint8_t *scales,
                              hipStream_t stream);
hipError_t launch_attn_fwd_bf16(View q, View k, View v, int B, int N, int H, float sm_scale, OutView out,
                                hipStream_t stream);
hipError_t launch_attn_fwd_int8qk(const int8_t *qc, const float *qs, const int8_t *kc, const float *ks, View v,
                                  int B, int N, int H, float sm_scale, OutView out, hipStream_t stream);
}  // namespace sage

namespace {

using sage::kD;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Upper bound on sizes: every byte offset the kernels form must fit in int64,
// grid.x of the attention launch in 32 bits, and B, H in grid.y / grid.z.
int check_shape(int B, int N, int H, int D) {
    if (B < 1 || N < 1 || H < 1) return SAGE_ERR_SHAPE;
    if (D != kD) return SAGE_ERR_SHAPE;
    if (B > 65535 || H > 65535) return SAGE_ERR_SHAPE;
    const int64_t npad = ((int64_t)N + SAGE_N_ALIGN - 1) / SAGE_N_ALIGN * SAGE_N_ALIGN;
    // Every launch's work-item count (workgroups x threads) must fit the
    // dispatch's 32-bit grid size.  The largest is the fused RoPE quantiser's
    // first pass, 2 B H Npad/64 workgroups of 256 threads = 8 B H Npad work-items
    // (the other quantiser grids are half that, attention B H ceil(N/128) x 256,
    // the MX quantiser B N H D/32); this also bounds every tensor's size.
    if ((double)B * H * (double)npad * 8.0 > 4294967295.0) return SAGE_ERR_SHAPE;
    return SAGE_OK;
}

// An input view: non-null, 16-byte aligned rows, non-negative strides.  Input
// views may alias (they are only read).
int check_in(const sage_bf16_in *v) {
    if (!v || !v->data) return SAGE_ERR_NULL;
    if (v->stride_b < 0 || v->stride_n < 0 || v->stride_h < 0) return SAGE_ERR_STRIDE;
    if (!aligned(v->data, 16)) return SAGE_ERR_ALIGN;
    if (v->stride_b % 8 || v->stride_n % 8 || v->stride_h % 8) return SAGE_ERR_ALIGN;
    return SAGE_OK;
}

// Every (b, n, h) row of D elements must be distinct memory.
bool rows_disjoint(int64_t sb, int64_t sn, int64_t sh, int B, int N, int H) {
    int64_t small = sn, large = sh, cnt_small = N, cnt_large = H;
    if (sh < sn) {
        small = sh; large = sn; cnt_small = H; cnt_large = N;
    }
    if (cnt_small > 1 && small < kD) return false;
    if (cnt_large > 1 && large < (cnt_small > 1 ? small * cnt_small : (int64_t)kD)) return false;
    if (B > 1) {
        int64_t span = (cnt_large > 1 ? large * cnt_large : (cnt_small > 1 ? small * cnt_small : (int64_t)kD));
        if (sb < span) return false;
    }
    return true;
}

int check_out(const sage_bf16_out *o, int B, int N, int H) {
    if (!o || !o->data) return SAGE_ERR_NULL;
    if (o->stride_b < 0 || o->stride_n < 0 || o->stride_h < 0) return SAGE_ERR_STRIDE;
    if (!aligned(o->data, 8)) return SAGE_ERR_ALIGN;
    if (o->stride_b % 4 || o->stride_n % 4 || o->stride_h % 4) return SAGE_ERR_ALIGN;
    if (!rows_disjoint(o->stride_b, o->stride_n, o->stride_h, B, N, H)) return SAGE_ERR_STRIDE;
    return SAGE_OK;
}

sage::View to_view(const sage_bf16_in *v) {
    return sage::View{static_cast<const uint16_t *>(v->data), v->stride_b, v->stride_n, v->stride_h};
}

sage::OutView to_out(const sage_bf16_out *o) {
    return sage::OutView{static_cast<uint16_t *>(o->data), o->stride_b, o->stride_n, o->stride_h};
}

int hip_status(hipError_t e) { return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP; }

// A view transformed in place: rows are read and written whole with 16-byte
// accesses, so as an input view, plus distinct rows.
int check_inplace(const sage_bf16_out *v, int B, int N, int H) {
    if (!v || !v->data) return SAGE_ERR_NULL;
    if (v->stride_b < 0 || v->stride_n < 0 || v->stride_h < 0) return SAGE_ERR_STRIDE;
    if (!aligned(v->data, 16)) return SAGE_ERR_ALIGN;
    if (v->stride_b % 8 || v->stride_n % 8 || v->stride_h % 8) return SAGE_ERR_ALIGN;
    if (!rows_disjoint(v->stride_b, v->stride_n, v->stride_h, B, N, H)) return SAGE_ERR_STRIDE;
    return SAGE_OK;
}

// RMSNorm weights and rotary table: read with 16-byte loads; eps > 0 keeps
// all-zero rows finite.
int check_norm_rope(const float *gamma_q, const float *gamma_k, const float *rope, float eps) {
    if (!gamma_q || !gamma_k || !rope) return SAGE_ERR_NULL;
    if (!aligned(gamma_q, 16) || !aligned(gamma_k, 16) || !aligned(rope, 16)) return SAGE_ERR_ALIGN;
    if (!std::isfinite(eps) || !(eps > 0.0f)) return SAGE_ERR_VALUE;
    return SAGE_OK;
}

// K and V tiles of a strided view are staged as 64 token rows through 32-bit,
// row-bounded buffer offsets: token rows may not overlap and a tile must span
// < 2 GiB.
int check_tile_rows(const sage_bf16_in *x) {
    return (x->stride_n < kD || x->stride_n > (int64_t)1 << 23) ? SAGE_ERR_STRIDE : SAGE_OK;
}

}  // namespace

extern "C" {

int64_t sage_npad(int N) {
    if (N < 1) return 0;
    return ((int64_t)N + SAGE_N_ALIGN - 1) / SAGE_N_ALIGN * SAGE_N_ALIGN;
}

size_t sage_qk_workspace_bytes(int B, int N, int H, int D) {
    if (check_shape(B, N, H, D) != SAGE_OK) return 0;
    return (size_t)((N + sage::kSumChunk - 1) / sage::kSumChunk) * B * H * D * sizeof(double);
}

size_t sage_v_workspace_bytes(int B, int N, int H, int D) {
    if (check_shape(B, N, H, D) != SAGE_OK) return 0;
    size_t nchunk = (size_t)((N + sage::kVChunk - 1) / sage::kVChunk);
    return (nchunk + 1) * (size_t)B * H * D * sizeof(float);
}

size_t sage_qkv_workspace_bytes(int B, int N, int H, int D) {
    if (check_shape(B, N, H, D) != SAGE_OK) return 0;
    const size_t nchunk = (size_t)((N + SAGE_K_BLOCK - 1) / SAGE_K_BLOCK);
    const size_t total = (size_t)B * H * D;
    return nchunk * total * (sizeof(double) + sizeof(float)) + total * sizeof(float);
}

size_t sage_qkv_rope_workspace_bytes(int B, int N, int H, int D) {
    const size_t base = sage_qkv_workspace_bytes(B, N, H, D);
    if (base == 0) return 0;
    const size_t npad = ((size_t)N + SAGE_N_ALIGN - 1) / SAGE_N_ALIGN * SAGE_N_ALIGN;
    return base + (size_t)B * H * npad * sizeof(float);
}

int sage_quantize_qk(const sage_bf16_in *q, const sage_bf16_in *k, int B, int N, int H, int D, int8_t *q_codes,
                     float *q_scale, int8_t *k_codes, float *k_scale, float *k_mean, void *workspace,
                     size_t workspace_bytes, void *stream) {
    int st;
    if ((st = check_in(q)) || (st = check_in(k))) return st;
    if (!q_codes || !q_scale || !k_codes || !k_scale || !k_mean || !workspace) return SAGE_ERR_NULL;
    if ((st = check_shape(B, N, H, D))) return st;
    if (!aligned(q_codes, 16) || !aligned(k_codes, 16) || !aligned(q_scale, 4) || !aligned(k_scale, 4) ||
        !aligned(k_mean, 4) || !aligned(workspace, 8))
        return SAGE_ERR_ALIGN;
    if (workspace_bytes < sage_qk_workspace_bytes(B, N, H, D)) return SAGE_ERR_WORKSPACE;
    return hip_status(sage::launch_quantize_qk(to_view(q), to_view(k), B, N, H, q_codes, q_scale, k_codes, k_scale,
                                               k_mean, workspace, static_cast<hipStream_t>(stream)));
}

int sage_quantize_v(const sage_bf16_in *v, int B, int N, int H, int D, uint8_t *v_codes, float *v_scale,
                    void *workspace, size_t workspace_bytes, void *stream) {
    int st;
    if ((st = check_in(v))) return st;
    if (!v_codes || !v_scale || !workspace) return SAGE_ERR_NULL;
    if ((st = check_shape(B, N, H, D))) return st;
    if (!aligned(v_codes, 16) || !aligned(v_scale, 4) || !aligned(workspace, 4)) return SAGE_ERR_ALIGN;
    if (workspace_bytes < sage_v_workspace_bytes(B, N, H, D)) return SAGE_ERR_WORKSPACE;
    return hip_status(sage::launch_quantize_v(to_view(v), B, N, H, v_codes, v_scale, workspace,
                                              static_cast<hipStream_t>(stream)));
}

int sage_quantize_qkv(const sage_bf16_in *q, const sage_bf16_in *k, const sage_bf16_in *v, int B, int N, int H,
                      int D, int8_t *q_codes, float *q_scale, int8_t *k_codes, float *k_scale, float *k_mean,
                      uint8_t *v_codes, float *v_scale, void *workspace, size_t workspace_bytes, void *stream) {
    int st;
    if ((st = check_in(q)) || (st = check_in(k)) || (st = check_in(v))) return st;
    if (!q_codes || !q_scale || !k_codes || !k_scale || !k_mean || !v_codes || !v_scale || !workspace)
        return SAGE_ERR_NULL;
    if ((st = check_shape(B, N, H, D))) return st;
    if (!aligned(q_codes, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(q_scale, 4) ||
        !aligned(k_scale, 4) || !aligned(k_mean, 4) || !aligned(v_scale, 4) || !aligned(workspace, 8))
        return SAGE_ERR_ALIGN;
    if (workspace_bytes < sage_qkv_workspace_bytes(B, N, H, D)) return SAGE_ERR_WORKSPACE;
    return hip_status(sage::launch_quantize_qkv(to_view(q), to_view(k), to_view(v), B, N, H, nullptr, q_codes,
                                                q_scale, k_codes, k_scale, k_mean, v_codes, v_scale, workspace,
                                                static_cast<hipStream_t>(stream)));
}

// ---- sage_quantize_qkv_noalloc: sage_quantize_qkv with library-owned scratch
}  // extern "C"

namespace {

// The scratch of sage_quantize_qkv_noalloc (the K-mean chunk partials, the V
// channel maxima and their reduction: sage_qkv_workspace_bytes of it per call).
// A device global: every GPU the library runs on holds its own copy from the
// first use until the process ends, and every call on that GPU shares it.  In
// host code `scratch` only names the symbol; its device address on the current
// device comes from hipGetSymbolAddress (noalloc_scratch below).
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];   // per device ordinal: the address of its copy, set on first use

// This device's copy of `scratch`, looked up once per device (with it current).
hipError_t noalloc_scratch(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

size_t sage_qkv_noalloc_max_bytes(void) { return kNoallocScratchBytes; }

int sage_quantize_qkv_noalloc(const sage_bf16_in *q, const sage_bf16_in *k, const sage_bf16_in *v, int B, int N,
                              int H, int D, int8_t *q_codes, float *q_scale, int8_t *k_codes, float *k_scale,
                              float *k_mean, uint8_t *v_codes, float *v_scale, void *stream) {
    int st;
    if ((st = check_in(q)) || (st = check_in(k)) || (st = check_in(v))) return st;
    if (!q_codes || !q_scale || !k_codes || !k_scale || !k_mean || !v_codes || !v_scale) return SAGE_ERR_NULL;
    if ((st = check_shape(B, N, H, D))) return st;
    if (!aligned(q_codes, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(q_scale, 4) ||
        !aligned(k_scale, 4) || !aligned(k_mean, 4) || !aligned(v_scale, 4))
        return SAGE_ERR_ALIGN;
    if (sage_qkv_workspace_bytes(B, N, H, D) > kNoallocScratchBytes) return SAGE_ERR_WORKSPACE;
    void *ws = nullptr;
    if (noalloc_scratch(&ws) != hipSuccess) return SAGE_ERR_HIP;
    return hip_status(sage::launch_quantize_qkv(to_view(q), to_view(k), to_view(v), B, N, H, nullptr, q_codes,
                                                q_scale, k_codes, k_scale, k_mean, v_codes, v_scale, ws,
                                                static_cast<hipStream_t>(stream)));
}

int sage_qk_norm_rope(const sage_bf16_out *q, const sage_bf16_out *k, int B, int N, int H, int D,
                      const float *gamma_q, const float *gamma_k, const float *rope, float eps, void *stream) {
    int st;
    if ((st = check_shape(B, N, H, D))) return st;
    if ((st = check_inplace(q, B, N, H)) || (st = check_inplace(k, B, N, H))) return st;
    if ((st = check_norm_rope(gamma_q, gamma_k, rope, eps))) return st;
    return hip_status(sage::launch_norm_rope(to_out(q), to_out(k), B, N, H,
                                             sage::NormRope{gamma_q, gamma_k, rope, eps},
                                             static_cast<hipStream_t>(stream)));
}

int sage_quantize_qkv_rope(const sage_bf16_in *q, const sage_bf16_in *k, const sage_bf16_in *v, int B, int N, int H,
                           int D, const float *gamma_q, const float *gamma_k, const float *rope, float eps,
                           int8_t *q_codes, float *q_scale, int8_t *k_codes, float *k_scale, float *k_mean,
                           uint8_t *v_codes, float *v_scale, void *workspace, size_t workspace_bytes, void *stream) {
    int st;
    if ((st = check_in(q)) || (st = check_in(k)) || (st = check_in(v))) return st;
    if (!q_codes || !q_scale || !k_codes || !k_scale || !k_mean || !v_codes || !v_scale || !workspace)
        return SAGE_ERR_NULL;
    if ((st = check_shape(B, N, H, D))) return st;
    if ((st = check_norm_rope(gamma_q, gamma_k, rope, eps))) return st;
    if (!aligned(q_codes, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(q_scale, 4) ||
        !aligned(k_scale, 4) || !aligned(k_mean, 4) || !aligned(v_scale, 4) || !aligned(workspace, 8))
        return SAGE_ERR_ALIGN;
    if (workspace_bytes < sage_qkv_rope_workspace_bytes(B, N, H, D)) return SAGE_ERR_WORKSPACE;
    const sage::NormRope nr{gamma_q, gamma_k, rope, eps};
    return hip_status(sage::launch_quantize_qkv(to_view(q), to_view(k), to_view(v), B, N, H, &nr, q_codes, q_scale,
                                                k_codes, k_scale, k_mean, v_codes, v_scale, workspace,
                                                static_cast<hipStream_t>(stream)));
}

int sage_attn_fwd(const int8_t *q_codes, const float *q_scale, const int8_t *k_codes, const float *k_scale,
                  const uint8_t *v_codes, const float *v_scale, int B, int N, int H, int D, float sm_scale,
                  const sage_bf16_out *out, void *stream) {
    int st;
    if (!q_codes || !q_scale || !k_codes || !k_scale || !v_codes || !v_scale) return SAGE_ERR_NULL;
    if ((st = check_shape(B, N, H, D))) return st;
    if ((st = check_out(out, B, N, H))) return st;
    if (!aligned(q_codes, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(q_scale, 4) ||
        !aligned(k_scale, 4) || !aligned(v_scale, 4))
        return SAGE_ERR_ALIGN;
    if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f)) return SAGE_ERR_VALUE;
    return hip_status(sage::launch_attn_fwd(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, B, N, H, sm_scale,
                                            to_out(out), static_cast<hipStream_t>(stream)));
}

int sage_attn_fwd_bf16(const sage_bf16_in *q, const sage_bf16_in *k, const sage_bf16_in *v, int B, int N, int H,
                       int D, float sm_scale, const sage_bf16_out *out, void *stream) {
    int st;
    if ((st = check_in(q)) || (st = check_in(k)) || (st = check_in(v))) return st;
    if ((st = check_tile_rows(k)) || (st = check_tile_rows(v))) return st;
    if ((st = check_shape(B, N, H, D))) return st;
    if ((st = check_out(out, B, N, H))) return st;
    if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f)) return SAGE_ERR_VALUE;
    return hip_status(sage::launch_attn_fwd_bf16(to_view(q), to_view(k), to_view(v), B, N, H, sm_scale, to_out(out),
                                                 static_cast<hipStream_t>(stream)));
}

int sage_attn_fwd_int8qk(const int8_t *q_codes, const float *q_scale, const int8_t *k_codes, const float *k_scale,
                         const sage_bf16_in *v, int B, int N, int H, int D, float sm_scale, const sage_bf16_out *out,
                         void *stream) {
    int st;
    if (!q_codes || !q_scale || !k_codes || !k_scale) return SAGE_ERR_NULL;
    if ((st = check_in(v))) return st;
    if ((st = check_tile_rows(v))) return st;
    if ((st = check_shape(B, N, H, D))) return st;
    if ((st = check_out(out, B, N, H))) return st;
    if (!aligned(q_codes, 16) || !aligned(k_codes, 16) || !aligned(q_scale, 4) || !aligned(k_scale, 4))
        return SAGE_ERR_ALIGN;
    if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f)) return SAGE_ERR_VALUE;
    return hip_status(sage::launch_attn_fwd_int8qk(q_codes, q_scale, k_codes, k_scale, to_view(v), B, N, H, sm_scale,
                                                   to_out(out), static_cast<hipStream_t>(stream)));
}

int sage_mx_quantize(const sage_bf16_in *x, int B, int N, int H, int D, int fmt, uint8_t *codes, uint8_t *scales,
                     void *stream) {
    int st;
    if ((st = check_in(x))) return st;
    if (!codes || !scales) return SAGE_ERR_NULL;
    if ((st = check_shape(B, N, H, D))) return st;
    if (!aligned(codes, 16)) return SAGE_ERR_ALIGN;
    if (fmt != SAGE_MX_E4M3 && fmt != SAGE_MX_E2M1) return SAGE_ERR_VALUE;
    return hip_status(sage::launch_mx_quantize(to_view(x), B, N, H, fmt, codes, scales,
                                               static_cast<hipStream_t>(stream)));
}

int sage_attn_fwd_mx(const int8_t *q_codes, const float *q_scale, const int8_t *k_codes, const float *k_scale,
                     const uint8_t *v_codes, const float *v_scale, int B, int N, int H, int D, float sm_scale, int fmt,
                     uint8_t *codes, uint8_t *scales, void *stream) {
    int st;
    if (!q_codes || !q_scale || !k_codes || !k_scale || !v_codes || !v_scale || !codes || !scales)
        return SAGE_ERR_NULL;
    if ((st = check_shape(B, N, H, D))) return st;
    if (!aligned(q_codes, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(q_scale, 4) ||
        !aligned(k_scale, 4) || !aligned(v_scale, 4) || !aligned(codes, 4))
        return SAGE_ERR_ALIGN;
    if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f)) return SAGE_ERR_VALUE;
    if (fmt != SAGE_MX_E4M3 && fmt != SAGE_MX_E2M1) return SAGE_ERR_VALUE;
    return hip_status(sage::launch_attn_fwd_mx(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, B, N, H,
                                               sm_scale, fmt, codes, scales, static_cast<hipStream_t>(stream)));
}

const char *sage_status_str(int status) {
    switch (status) {
        case SAGE_OK: return "ok";
        case SAGE_ERR_NULL: return "null pointer";
        case SAGE_ERR_SHAPE: return "unsupported shape";
        case SAGE_ERR_STRIDE: return "invalid strides";
        case SAGE_ERR_ALIGN: return "misaligned pointer or stride";
        case SAGE_ERR_WORKSPACE: return "workspace too small";
        case SAGE_ERR_HIP: return "HIP runtime error";
        case SAGE_ERR_VALUE: return "invalid value (sm_scale, eps or format)";
        default: return "unknown status";
    }
}

}  // extern "C"
