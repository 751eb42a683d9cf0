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

extern "C" {

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
