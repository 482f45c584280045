// Device helpers shared by the latent-MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round to nearest even (the hardware conversion).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// 32x32x16 bf16 matrix-core product, fp32 accumulate. Operand lane layout:
// lane l holds A[l%32][(l/32)*8 + i] and B[(l/32)*8 + i][l%32], i = 0..7;
// result register r of lane l is C[(r/4)*8 + (l/32)*4 + r%4][l%32].
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 bf16: lane l holds A[l%16][(l/16)*8 + i], B[(l/16)*8 + i][l%16];
// result register r of lane l is C[(l/16)*4 + r][l%16].
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// OCP E4M3fn byte -> float (gfx950 converts the OCP encoding natively).
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8(byte, 0);
}

// Eight e2m1 codes (one dword: byte j holds element 2j in its low nibble and
// 2j+1 in its high nibble) times the block scale s -> eight bf16 in element
// order. e2m1 * E4M3 needs at most 6 significant bits, so the products are
// exact in fp32 and in bf16: nothing is rounded here.
//
// The scaled fp4 conversions of gfx950 apply only the exponent of their f32
// scale operand (the MX convention of power-of-two block scales), so they are
// used with scale 1.0 and the E4M3 block scale is applied by an fp32 multiply.
__device__ __forceinline__ bf16x8 dequant8(uint32_t codes, float s) {
  const f32x2 q0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
  const f32x2 q1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
  const f32x2 q2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
  const f32x2 q3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
  bf16x8 r;
  r[0] = (__bf16)(q0[0] * s); r[1] = (__bf16)(q0[1] * s);
  r[2] = (__bf16)(q1[0] * s); r[3] = (__bf16)(q1[1] * s);
  r[4] = (__bf16)(q2[0] * s); r[5] = (__bf16)(q2[1] * s);
  r[6] = (__bf16)(q3[0] * s); r[7] = (__bf16)(q3[1] * s);
  return r;
}

// As dequant8, to fp16: e2m1 (at most 2 significant bits, magnitude <= 6)
// times E4M3 (at most 4 significant bits, 2^-9 <= magnitude <= 448) needs at
// most 6 significant bits and lies in [2^-10, 2688], inside fp16's normal
// range, so these products are exact too. The fp16 conversions produce the
// codes' values as fp16 pairs and one packed fp16 multiply per pair applies
// the scale: 8 vector ops per 8 weights against 16 for the bf16 route (gfx950
// has no packed bf16 multiply). s16 = the block scale as fp16 (exact).
__device__ __forceinline__ f16x8 dequant8_f16(uint32_t codes, _Float16 s16) {
  const f16x2 ss = {s16, s16};
  const f16x2 q0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * ss;
  const f16x2 q1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * ss;
  const f16x2 q2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * ss;
  const f16x2 q3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * ss;
  return f16x8{q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
}

__device__ __forceinline__ f32x4 mfma16x16x32_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Elements 8G .. 8G+7 of a 32-element E1M1 chunk (3-bit codes: sign,
// exponent bit, mantissa bit; magnitudes 0, 0.5, 1, 1.5) as the eight e2m1
// codes of the same values, in dequant8's nibble order. The chunk's words
// w0, w1, w2 hold elements 0..23 as e2m1 nibbles already (an E1M1 value is
// the e2m1 value whose high exponent bit, nibble bit 2, is clear); that
// free bit of nibble p carries element 24 + p: its mantissa in w0, its
// exponent in w1, its sign in w2. So groups 0..2 cost one mask and group 3
// three shifts and masks.
template <int G>
__device__ __forceinline__ uint32_t e1m1_group_to_e2m1(uint32_t w0, uint32_t w1, uint32_t w2) {
  static_assert(G >= 0 && G < 4, "four groups of eight per chunk");
  if constexpr (G == 0) return w0 & 0xBBBBBBBBu;
  else if constexpr (G == 1) return w1 & 0xBBBBBBBBu;
  else if constexpr (G == 2) return w2 & 0xBBBBBBBBu;
  else
    return ((w0 >> 2) & 0x11111111u) | ((w1 >> 1) & 0x22222222u) | ((w2 << 1) & 0x88888888u);
}
__device__ __forceinline__ uint32_t e1m1_group_to_e2m1(uint32_t w0, uint32_t w1, uint32_t w2,
                                                       int g) {
  switch (g) {  // g is a compile-time constant after unrolling
    case 0: return e1m1_group_to_e2m1<0>(w0, w1, w2);
    case 1: return e1m1_group_to_e2m1<1>(w0, w1, w2);
    case 2: return e1m1_group_to_e2m1<2>(w0, w1, w2);
    default: return e1m1_group_to_e2m1<3>(w0, w1, w2);
  }
}

// silu(g) = g / (1 + e^-g), with e^-g = 2^(-g log2 e) on the hardware base-2
// exponential and the reciprocal on the hardware reciprocal (each within about
// one fp32 ulp; the result is rounded to bf16 afterwards). Five instructions
// instead of a correctly rounded exp and an IEEE division (about thirty).
// Limits: g -> -inf gives e^-g = inf, a zero reciprocal and -0; g -> +inf
// gives g.
__device__ __forceinline__ float silu_fast(float g) {
  const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
  return g * __builtin_amdgcn_rcpf(1.0f + e);
}

// Eight e2m1 codes -> their plain values as bf16 (exact; no block scale).
__device__ __forceinline__ bf16x8 e2m1x8_to_bf16(uint32_t codes) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, 3);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Waits until at most n vector-memory loads of this wave are outstanding
// (gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left
// at "no wait"). Loads complete in issue order, so this waits for all but
// the n most recent.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// Direct-to-LDS DMA of 16 or 4 bytes per lane (lane L's bytes land at
// lds_base + L * size; lds_base wave-uniform). In asm, so the compiler does
// not see the LDS write: where it cannot tell LDS stages apart it would
// otherwise wait for every DMA in flight before each LDS read. Callers
// order these loads themselves, with vmcnt waits and barriers. M0 is
// restored afterwards.
__device__ __forceinline__ void dma_lds16(const void* g, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds_base)
      : "memory");
}
__device__ __forceinline__ void dma_lds4(const void* g, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds_base)
      : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Workgroup barrier that orders LDS accesses only: global loads still in
// flight are not waited for (a full __syncthreads() would wait for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <class T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Inclusive prefix sum across the wave (lane order).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int u = __shfl_up(v, d, kWave);
    if (lane >= d) v += u;
  }
  return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (kWave - 1);
  return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}

// ------------------------------------------------------------------ top-k selection

// Order-preserving 32-bit key of an fp32 value (larger value, larger key;
// -0 and +0 share a key, and 0 is below every non-NaN value and marks an
// empty or taken entry).
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_umax(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
  return o > v ? o : v;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_umin(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
  return o < v ? o : v;
}

// Largest / smallest value over the 64 lanes (wave-uniform): DPP steps
// inside each 16-lane row, then the four row results through readlane.
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = dpp_umax<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_umax<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_umax<0x141>(v);  // row_half_mirror: over 8 lanes
  v = dpp_umax<0x140>(v);  // row_mirror: over 16 lanes
  uint32_t m = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)v, r * 16);
    m = o > m ? o : m;
  }
  return m;
}
__device__ __forceinline__ uint32_t wave_umin(uint32_t v) {
  v = dpp_umin<0xB1>(v);
  v = dpp_umin<0x4E>(v);
  v = dpp_umin<0x141>(v);
  v = dpp_umin<0x140>(v);
  uint32_t m = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)v, r * 16);
    m = o < m ? o : m;
  }
  return m;
}

// k rounds of a wave-wide arg-max over the keys of one token, lane l holding
// experts l, l + 64, ... (key 0 = absent). Round r takes the largest key
// left, ties to the lower expert; lane r ends with its key and expert.
// The largest key comes from one DPP reduction. The lanes holding it are
// found by a ballot: when exactly one lane does (the usual case) its lowest
// such expert wins directly; otherwise a second reduction takes the lowest
// expert over those lanes.
template <int EPL>
__device__ __forceinline__ void wave_select_topk(uint32_t (&key)[EPL], int E, int k,
                                                 uint32_t& my_key, int& my_e) {
  const int lane = threadIdx.x & 63;
  my_key = 0u;
  my_e = 0;
  for (int r = 0; r < k; ++r) {
    uint32_t best = key[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) best = key[i] > best ? key[i] : best;
    const uint32_t m = wave_umax(best);
    // this lane's lowest expert holding m (expert = lane + 64 i)
    uint32_t first = 0xFFFFFFFFu;
#pragma unroll
    for (int i = EPL - 1; i >= 0; --i) first = key[i] == m ? (uint32_t)(lane + 64 * i) : first;
    const uint64_t holders = __ballot(best == m);
    uint32_t win;
    if (__popcll(holders) == 1)
      win = (uint32_t)__builtin_amdgcn_readlane((int)first, __ffsll((unsigned long long)holders) - 1);
    else
      win = wave_umin(first);
    const int w = (int)min(win, (uint32_t)(E - 1));  // in range even for NaN
#pragma unroll
    for (int i = 0; i < EPL; ++i) key[i] = lane + 64 * i == w ? 0u : key[i];
    if (lane == r) {
      my_key = m;
      my_e = w;
    }
  }
}

}  // namespace moe
