// Probes of gfx950 builtins used by the layer kernels: the lane layouts of
// the bf16 MFMA instructions, the fp4 -> bf16/f32 scaled conversions, the
// OCP E4M3 -> f32 conversion and float -> bf16 rounding. Every kernel reads
// and writes only the element ranges its host wrapper sizes for it.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// One wave. A [32][16] row-major bf16, B [16][32] row-major (k, n), C [32][32].
// Lane l holds A[l%32][(l/32)*8 + i] and B[(l/32)*8 + i][l%32]; the result
// register r of lane l is written to C[(r/4)*8 + (l/32)*4 + r%4][l%32].
__global__ void k_mfma32(const __bf16* A, const __bf16* B, float* C) {
  int l = threadIdx.x;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = A[(l % 32) * 16 + (l / 32) * 8 + i];
    b[i] = B[((l / 32) * 8 + i) * 32 + (l % 32)];
  }
  f32x16 c = {};
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  for (int r = 0; r < 16; ++r) C[((r / 4) * 8 + (l / 32) * 4 + r % 4) * 32 + (l % 32)] = c[r];
}

// One wave. A [16][32], B [32][16], C [16][16]. Lane l holds
// A[l%16][(l/16)*8 + i], B[(l/16)*8 + i][l%16]; register r -> C[(l/16)*4 + r][l%16].
__global__ void k_mfma16(const __bf16* A, const __bf16* B, float* C) {
  int l = threadIdx.x;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = A[(l % 16) * 32 + (l / 16) * 8 + i];
    b[i] = B[((l / 16) * 8 + i) * 16 + (l % 16)];
  }
  f32x4 c = {};
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  for (int r = 0; r < 4; ++r) C[((l / 16) * 4 + r) * 16 + (l % 16)] = c[r];
}

// n dwords of codes (8 fp4 each), one f32 scale per dword -> 8 bf16 / 8 f32 each.
__global__ void k_cvt_fp4(const uint32_t* codes, const float* scales, __bf16* outb,
                          float* outf, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  uint32_t c = codes[i];
  float s = scales[i];
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 3);
  outb[8 * i + 0] = p0[0]; outb[8 * i + 1] = p0[1];
  outb[8 * i + 2] = p1[0]; outb[8 * i + 3] = p1[1];
  outb[8 * i + 4] = p2[0]; outb[8 * i + 5] = p2[1];
  outb[8 * i + 6] = p3[0]; outb[8 * i + 7] = p3[1];
  f32x2 q0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, s, 0);
  f32x2 q1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, s, 1);
  f32x2 q2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, s, 2);
  f32x2 q3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, s, 3);
  outf[8 * i + 0] = q0[0]; outf[8 * i + 1] = q0[1];
  outf[8 * i + 2] = q1[0]; outf[8 * i + 3] = q1[1];
  outf[8 * i + 4] = q2[0]; outf[8 * i + 5] = q2[1];
  outf[8 * i + 6] = q3[0]; outf[8 * i + 7] = q3[1];
}

// 256 bytes (one per lane group) -> f32 via the OCP FP8 conversion.
__global__ void k_cvt_fp8(const uint32_t* packed, float* out) {
  int i = threadIdx.x;  // 0..63: dword i holds bytes 4i..4i+3
  uint32_t v = packed[i];
  out[4 * i + 0] = __builtin_amdgcn_cvt_f32_fp8(v, 0);
  out[4 * i + 1] = __builtin_amdgcn_cvt_f32_fp8(v, 1);
  out[4 * i + 2] = __builtin_amdgcn_cvt_f32_fp8(v, 2);
  out[4 * i + 3] = __builtin_amdgcn_cvt_f32_fp8(v, 3);
}

__global__ void k_f32_to_bf16(const float* in, __bf16* out, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = (__bf16)in[i];
}

extern "C" {
int probe_mfma32(const void* A, const void* B, void* C) {
  hipLaunchKernelGGL(k_mfma32, dim3(1), dim3(64), 0, 0, (const __bf16*)A, (const __bf16*)B, (float*)C);
  return (int)hipGetLastError();
}
int probe_mfma16(const void* A, const void* B, void* C) {
  hipLaunchKernelGGL(k_mfma16, dim3(1), dim3(64), 0, 0, (const __bf16*)A, (const __bf16*)B, (float*)C);
  return (int)hipGetLastError();
}
int probe_cvt_fp4(const void* codes, const void* scales, void* outb, void* outf, int n) {
  hipLaunchKernelGGL(k_cvt_fp4, dim3((n + 63) / 64), dim3(64), 0, 0, (const uint32_t*)codes,
                     (const float*)scales, (__bf16*)outb, (float*)outf, n);
  return (int)hipGetLastError();
}
int probe_cvt_fp8(const void* packed, void* out) {
  hipLaunchKernelGGL(k_cvt_fp8, dim3(1), dim3(64), 0, 0, (const uint32_t*)packed, (float*)out);
  return (int)hipGetLastError();
}
int probe_f32_to_bf16(const void* in, void* out, int n) {
  hipLaunchKernelGGL(k_f32_to_bf16, dim3((n + 255) / 256), dim3(256), 0, 0, (const float*)in,
                     (__bf16*)out, n);
  return (int)hipGetLastError();
}
}
