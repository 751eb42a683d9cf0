/*
 * c_abi_client.c -- a plain C99 caller of libsage_mi355x.so: HIP runtime C API
 * for device memory, the library's public header for everything else, no torch.
 * tests/test_gpu_c_client.py writes its input and checks its output against the
 * oracle.
 *
 *   c_abi_client IN OUT
 *
 * IN:  int32 B, N, H, then Q, K, V as bf16 bit patterns, each [B, N, H, 128]
 *      contiguous.
 * OUT: int32 status (0 = every call returned SAGE_OK), then q_codes, k_codes
 *      ([B, H, Npad, 128] int8), v_codes ([B, H, Npad/64, 128, 64] uint8),
 *      q_scale [B, H, Npad/32], k_scale [B, H, Npad/64], k_mean [B, H, 128],
 *      v_scale [B, H, 128] (fp32), the quantised forward's output and the bf16
 *      path's output ([B, N, H, 128] bf16 bit patterns).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "sage_mi355x.h"

#define D SAGE_HEAD_DIM

static int fail(const char *what, int code) {
    fprintf(stderr, "c_abi_client: %s failed (%d: %s)\n", what, code,
            code >= 0 && code < 16 ? sage_status_str(code) : "hip error");
    return 1;
}

static void *dev(size_t bytes) {
    void *p = NULL;
    if (hipMalloc(&p, bytes ? bytes : 16) != hipSuccess) return NULL;
    return p;
}

static int fetch(FILE *f, const void *d, size_t bytes) {
    void *h = malloc(bytes ? bytes : 1);
    int ok = h && hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost) == hipSuccess && fwrite(h, 1, bytes, f) == bytes;
    free(h);
    return ok;
}

int main(int argc, char **argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
        return 2;
    }
    FILE *in = fopen(argv[1], "rb");
    int32_t dims[3];
    if (!in || fread(dims, sizeof dims, 1, in) != 1) return fail("reading the input header", -1);
    const int B = dims[0], N = dims[1], H = dims[2];
    const int64_t npad = sage_npad(N);
    if (npad == 0) return fail("sage_npad", SAGE_ERR_SHAPE);
    const size_t elems = (size_t)B * N * H * D, bytes16 = elems * 2;
    uint16_t *host = malloc(3 * bytes16);
    if (!host || fread(host, 1, 3 * bytes16, in) != 3 * bytes16) return fail("reading Q, K, V", -1);
    fclose(in);

    /* inputs: contiguous [B, N, H, D] bf16 */
    uint16_t *qkv = dev(3 * bytes16);
    if (!qkv || hipMemcpy(qkv, host, 3 * bytes16, hipMemcpyHostToDevice) != hipSuccess)
        return fail("copying the inputs", -1);
    const int64_t sn = (int64_t)H * D, sb = (int64_t)N * sn;
    sage_bf16_in q = {qkv, sb, sn, D}, k = {qkv + elems, sb, sn, D}, v = {qkv + 2 * elems, sb, sn, D};

    /* library-layout buffers, sized by the header's rules */
    const size_t ncodes = (size_t)B * H * npad * D;
    int8_t *q_codes = dev(ncodes), *k_codes = dev(ncodes);
    uint8_t *v_codes = dev(ncodes);
    float *q_scale = dev((size_t)B * H * (npad / SAGE_Q_BLOCK) * 4);
    float *k_scale = dev((size_t)B * H * (npad / SAGE_K_BLOCK) * 4);
    float *k_mean = dev((size_t)B * H * D * 4), *v_scale = dev((size_t)B * H * D * 4);
    const size_t ws_bytes = sage_qkv_workspace_bytes(B, N, H, D);
    void *ws = dev(ws_bytes);
    uint16_t *o8 = dev(bytes16), *o16 = dev(bytes16);
    if (!q_codes || !k_codes || !v_codes || !q_scale || !k_scale || !k_mean || !v_scale || !ws || !o8 || !o16)
        return fail("hipMalloc", -1);
    sage_bf16_out out8 = {o8, sb, sn, D}, out16 = {o16, sb, sn, D};

    hipStream_t stream;
    if (hipStreamCreate(&stream) != hipSuccess) return fail("hipStreamCreate", -1);
    const float sm = 0.08838834764831845f; /* 1 / sqrt(128) */
    int st = sage_quantize_qkv(&q, &k, &v, B, N, H, D, q_codes, q_scale, k_codes, k_scale, k_mean, v_codes,
                               v_scale, ws, ws_bytes, stream);
    if (st != SAGE_OK) return fail("sage_quantize_qkv", st);
    st = sage_attn_fwd(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, B, N, H, D, sm, &out8, stream);
    if (st != SAGE_OK) return fail("sage_attn_fwd", st);
    st = sage_attn_fwd_bf16(&q, &k, &v, B, N, H, D, sm, &out16, stream);
    if (st != SAGE_OK) return fail("sage_attn_fwd_bf16", st);
    if (hipStreamSynchronize(stream) != hipSuccess) return fail("hipStreamSynchronize", -1);

    FILE *out = fopen(argv[2], "wb");
    const int32_t ok = 0;
    if (!out || fwrite(&ok, sizeof ok, 1, out) != 1) return fail("writing the output", -1);
    int good = fetch(out, q_codes, ncodes) && fetch(out, k_codes, ncodes) && fetch(out, v_codes, ncodes) &&
               fetch(out, q_scale, (size_t)B * H * (npad / SAGE_Q_BLOCK) * 4) &&
               fetch(out, k_scale, (size_t)B * H * (npad / SAGE_K_BLOCK) * 4) &&
               fetch(out, k_mean, (size_t)B * H * D * 4) && fetch(out, v_scale, (size_t)B * H * D * 4) &&
               fetch(out, o8, bytes16) && fetch(out, o16, bytes16);
    fclose(out);
    if (!good) return fail("copying the results back", -1);

    hipStreamDestroy(stream);
    void *bufs[] = {qkv, q_codes, k_codes, v_codes, q_scale, k_scale, k_mean, v_scale, ws, o8, o16};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; i++) hipFree(bufs[i]);
    free(host);
    printf("c_abi_client: B=%d N=%d H=%d done\n", B, N, H);
    return 0;
}
