// Weight-streaming decode path of the latent-MoE layer (T <= 8 tokens).
//
// At a handful of tokens every weight byte feeds only T multiply-adds, so the
// layer is bound by HBM bandwidth and by the fixed latency of each dependent
// step (a kernel boundary costs a launch plus at least one memory round
// trip). Four kernels, each a grid-wide dependency of the next:
//
//   1. dec_front   h = x D^T (RMSNorm fused for the residual block) and, in
//                  the same launch, the router logits straight from x: the
//                  router folded onto the residual width, W = R D (computed
//                  once when the weights are packed, stored as bf16 hi + lo),
//                  gives l = x W^T = (x D^T) R^T. Without a folded router the
//                  logits come from h in a second launch (dec_dproj writes h
//                  as bf16 hi + lo, dec_router reads both halves).
//   2. dec_gateup  at most one workgroup per CU; each takes the top-k of
//                  every token from the logits and builds the active-expert
//                  list (workgroup 0 publishes the routing table); then the
//                  (expert slot, 16 intermediate rows) tasks are split
//                  evenly over the grid, one per wave at a time: the gate
//                  and the up tile over the whole latent width, SiLU * up
//                  in registers. Slot 0 is the shared expert. With one
//                  routing group the products run in fp16 when the front
//                  kernel found every value of bf16(h) exact in fp16.
//   3. dec_down    one workgroup per (16 or 32 latent rows, group of 8
//                  slots), one slot per wave; the weighted products are
//                  summed in slot order and added into z in 64-bit fixed
//                  point with integer atomics (exact, so the arrival order
//                  does not matter)
//   4. dec_uproj   out = bf16(z) U^T (+ x)
//
// Matrix-core tiles are v_mfma_f32_16x16x32_bf16 (or _f16) with weight rows
// as the M operand (16 rows) and tokens as the N operand (16 columns, T
// used; the rest repeat token T - 1 and are never stored, so no operand load
// is conditional). Lane l serves weight row l%16; its lane group g = l/16
// takes every fourth chunk of the wave's K range (chunk c*4 + g at step c),
// so one load instruction reads 64 contiguous bytes of each of 16 rows (1 KB
// of contiguous memory on the decode-packed copies). K order inside a dot
// product is free; the token operand is read with the same chunk mapping.
// The expert weight streams keep the next chunks' loads in flight while one
// is dequantised and multiplied; D, U and the router issue all their weight
// loads before their first product.
#include <limits.h>

#include <map>
#include <mutex>
#include <set>
#include <type_traits>
#include <utility>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kDecThreads = 512;  // 8 waves
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kDownGroup = kDecodeDownGroup;
static_assert(kDownGroup == kDecWaves, "one expert slot per down wave");

#define AGENT __HIP_MEMORY_SCOPE_AGENT

// ------------------------------------------------------------------ weight addressing

// A wave streams a 16-row tile (rows r0 .. r0+15, r0 % 16 == 0) of a weight
// matrix over the K range [kb, ...): lane l serves row r0 + l % 16 and lane
// group g = l / 16 takes chunk 4i + g at step i. Plain row-major weights put
// a lane's successive chunks 64 (fp4) or 32 (bf16) elements apart within its
// row. The decode-packed layout (launch_pack_*_decode) stores each step's
// 64 lane chunks contiguously (1 KB), so that the wave's loads are too.
struct Fp4Lane {
  const uint8_t* c;
  int cstep;
  const uint8_t* s;
  int sstep;
};

// fp4 matrix e of a set [count][N][K]; kb % 128 == 0. bits 4: e2m1 codes,
// 16 bytes per 32 weights; bits 3: E1M1 codes, one 12-byte chunk per 32.
__device__ __forceinline__ Fp4Lane fp4_lane(const Fp4Mat& m, bool packed, int e, int N, int K,
                                            int r0, int kb, int bits = 4) {
  const int lane = threadIdx.x & 63;
  const int cb = bits == 4 ? 16 : 12;  // code bytes of 32 weights
  if (packed) {  // block (e, t, c): 64 lanes x cb code bytes, 128 B scales [row][8]
    const size_t blk = ((size_t)e * (N / 16) + min(r0, N - 16) / 16) * (K / 128) + kb / 128;
    return {m.codes + blk * 64 * cb + lane * cb, 64 * cb, m.scales + blk * 128 + (lane & 15) * 8,
            128};
  }
  const size_t row = (size_t)e * N + min(r0 + (lane & 15), N - 1);
  return {m.codes + row * ((size_t)K / 32 * cb) + (kb / 32 + (lane >> 4)) * cb, 4 * cb,
          m.scales + row * (K / 16) + kb / 16, 8};
}

// Lane base and step (elements) of a bf16 matrix [N][K]; kb % 32 == 0.
__device__ __forceinline__ const uint16_t* bf16_lane(const uint16_t* w, bool packed, int N, int K,
                                                    int r0, int kb, int* step) {
  const int lane = threadIdx.x & 63;
  if (packed) {  // block (t, c): 1 KB [lane][8 elements]
    *step = 512;
    const size_t blk = (size_t)(min(r0, N - 16) / 16) * (K / 32) + kb / 32;
    return w + blk * 512 + lane * 8;
  }
  *step = 32;
  return w + (size_t)min(r0 + (lane & 15), N - 1) * K + kb + (lane >> 4) * 8;
}

// ------------------------------------------------------------------ wave tiles

// Keeps every load above issued before anything below: without it the
// scheduler may sink late weight chunks and the matrix scales under the
// first products, and each such load then adds its own memory round trip to
// the end of the kernel. Only where no staged value is live across it: the
// register allocator spills such values around the barrier.
__device__ __forceinline__ void issue_fence() { __builtin_amdgcn_sched_barrier(0); }

// NCH chunks of 8 bf16 per lane group: the wave's K range is [kb, kb + 32*NCH).
// Chunk c of the lane sits at base + c * step (elements); see bf16_lane.
template <int NCH>
struct Bf16Rows {
  uint4 w[NCH];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ base, int step) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) w[c] = *(const uint4*)(base + c * step);
  }
  // acc += W . act over the range; act = this lane's token row in LDS
  __device__ __forceinline__ void mma(const uint16_t* act, int kb, int g, f32x4& acc) const {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const bf16x8 b = *(const bf16x8*)(act + kb + (c * 4 + g) * 8);
      acc = mfma16x16x32(__builtin_bit_cast(bf16x8, w[c]), b, acc);
    }
  }
  // two token operands: the hi and lo bf16 halves of one fp32 vector
  __device__ __forceinline__ void mma2(const uint16_t* hi, const uint16_t* lo, int kb, int g,
                                       f32x4& acc) const {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const bf16x8 bh = *(const bf16x8*)(hi + kb + (c * 4 + g) * 8);
      const bf16x8 bl = *(const bf16x8*)(lo + kb + (c * 4 + g) * 8);
      const bf16x8 a = __builtin_bit_cast(bf16x8, w[c]);
      acc = mfma16x16x32(a, bh, acc);
      acc = mfma16x16x32(a, bl, acc);
    }
  }
};

// NCH chunks of 32 fp4 weights (16 bytes of codes + 2 E4M3 scales) per lane
// group: the wave's K range is [kb, kb + 128*NCH). The four lane groups of a
// row take chunks 4i .. 4i + 3 at step i, whose eight scale bytes are
// contiguous: every lane of the row loads those eight bytes (16 distinct
// addresses per instruction instead of 64 two-byte ones; measured 12.7 ->
// 11.3 us for the routed gate/up weight stream) and keeps its two.
// BITS = 3: E1M1 codes, a lane's chunk of 32 weights being 12 bytes (three
// words of e2m1-shaped nibbles, see e1m1_group_to_e2m1), widened in mma.
template <int NCH, int BITS = 4>
struct Fp4Rows {
  static constexpr int kW = BITS == 4 ? 4 : 3;  // code words per chunk
  uint32_t c[NCH][kW];
  uint2 s[NCH];
  // chunk i of the lane at l.c + i * l.cstep, its row's 8 scale bytes at
  // l.s + i * l.sstep (see fp4_lane)
  __device__ __forceinline__ void load(const Fp4Lane& l);
  // e2m1 nibbles of elements 8q .. 8q+7 of chunk i
  __device__ __forceinline__ uint32_t codes8(int i, int q) const {
    if constexpr (BITS == 4)
      return c[i][q];
    else
      return e1m1_group_to_e2m1(c[i][0], c[i][1], c[i][2], q);
  }
  // token operand: this lane's token row in LDS
  __device__ __forceinline__ void mma(const uint16_t* act, int kb, int g, f32x4& acc) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const uint32_t sp = ((g & 2) ? s[i].y : s[i].x) >> (16 * (g & 1));
      const float s0 = e4m3_to_f32(sp & 0xFFu), s1 = e4m3_to_f32((sp >> 8) & 0xFFu);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x8 b = *(const bf16x8*)(act + kb + (i * 4 + g) * 32 + q * 8);
        acc = mfma16x16x32(dequant8(codes8(i, q), q < 2 ? s0 : s1), b, acc);
      }
    }
  }
};

template <int NCH, int BITS>
__device__ __forceinline__ void Fp4Rows<NCH, BITS>::load(const Fp4Lane& l) {
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    if constexpr (BITS == 4) {
      const uint4 v = *(const uint4*)(l.c + i * l.cstep);
      c[i][0] = v.x; c[i][1] = v.y; c[i][2] = v.z; c[i][3] = v.w;
    } else {
      const uint3 v = *(const uint3*)(l.c + i * l.cstep);
      c[i][0] = v.x; c[i][1] = v.y; c[i][2] = v.z;
    }
    s[i] = *(const uint2*)(l.s + i * l.sstep);
  }
}

// Sum the per-wave partial tiles through LDS in wave order; lane l of wave 0
// returns the totals of rows (l/16)*4 + r, token l%16.
__device__ __forceinline__ f32x4 reduce_waves(f32x4 acc, float* red /*[8][64][4]*/) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  *(f32x4*)(red + (wave * 64 + lane) * 4) = acc;
  __syncthreads();
  f32x4 tot = {0.f, 0.f, 0.f, 0.f};
  if (wave == 0)
    for (int w = 0; w < kDecWaves; ++w) tot += *(const f32x4*)(red + (w * 64 + lane) * 4);
  return tot;
}

// Up to kDecodeMaxT rows of activations moved to LDS in two steps, so their
// global loads can be issued before a wave's weight loads (memory counters
// drain in order: whatever is loaded first can be used first).
// NV 16-byte vectors per thread hold up to 512 * NV * 8 elements: a kernel
// whose staged rows are `width` wide uses NV = ceil(8 * width / 4096).
template <int NV>
struct RowStage {
  uint4 v[NV];
  // count is a multiple of 8 and >= 8. Out-of-range slots re-read the last
  // vector and store it back to its own place (the same bytes the in-range
  // slot writes there). Both halves stay unconditional: a store under a
  // branch lets the compiler sink its load into the branch, which turns NV
  // loads in flight into NV round trips one after another.
  __device__ __forceinline__ void load(const uint16_t* src, int count) {
#pragma unroll
    for (int j = 0; j < NV; ++j) v[j] = *(const uint4*)(src + slot(j, count));
  }
  // rows of `width` elements (a multiple of 8) taken `stride` apart in src;
  // stored contiguously by store(dst, rows * width)
  __device__ __forceinline__ void load_rows(const uint16_t* src, int rows, int width, int stride) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int i = slot(j, rows * width);
      v[j] = *(const uint4*)(src + (size_t)(i / width) * stride + i % width);
    }
  }
  __device__ __forceinline__ void store(uint16_t* dst, int count) const {
#pragma unroll
    for (int j = 0; j < NV; ++j) *(uint4*)(dst + slot(j, count)) = v[j];
  }
  static __device__ __forceinline__ int slot(int j, int count) {
    return min((int)(threadIdx.x + j * kDecThreads) * 8, count - 8);
  }
};

// count (a multiple of 8) bf16 elements from global src into LDS dst with
// direct-to-LDS loads (global_load_lds_dwordx4: lane l of a wave writes 16
// bytes at the wave's LDS base + 16 l). Thread t moves 16-byte slots t,
// t + 512, ...; a wave whose first slot is past the end issues nothing, and
// the lanes past the end of the last busy wave re-read the last slot and
// write up to 63 slots past count (callers keep that much LDS behind the
// rows). No registers hold the rows, so other loads can be in flight and
// consumed meanwhile; the caller waits (vmcnt) before its barrier.
template <int NV>
__device__ __forceinline__ void stage_dma(const uint16_t* src, int count, uint16_t* dst) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nslots = count / 8;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int first = v * kDecThreads + wave * 64;  // wave-uniform
    if (first < nslots)
      __builtin_amdgcn_global_load_lds((const void*)(src + (size_t)min(first + lane, nslots - 1) * 8),
                                       (__attribute__((address_space(3))) void*)(dst + first * 8),
                                       16, 0, 0);
  }
}


// As stage_dma for `rows` rows of `width` elements (a multiple of 8) taken
// `stride` apart in src, stored contiguously at dst.
template <int NV>
__device__ __forceinline__ void stage_dma_rows(const uint16_t* src, int rows, int width, int stride,
                                               uint16_t* dst) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nslots = rows * width / 8;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int first = v * kDecThreads + wave * 64;  // wave-uniform
    if (first < nslots) {
      const int i = min(first + lane, nslots - 1) * 8;
      __builtin_amdgcn_global_load_lds((const void*)(src + (size_t)(i / width) * stride + i % width),
                                       (__attribute__((address_space(3))) void*)(dst + first * 8),
                                       16, 0, 0);
    }
  }
}

// As stage_dma, by one wave into its own region (no workgroup barrier
// needed before the wave reads it): lane l moves 16-byte slots l, l + 64,
// ...; at most 63 slots past count are written (regions are padded to a
// whole number of 1 KB).
template <int NV>
__device__ __forceinline__ void stage_dma_wave(const uint16_t* src, int count, uint16_t* dst) {
  const int lane = threadIdx.x & 63;
  const int nslots = count / 8;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int first = v * 64;
    if (first < nslots)
      __builtin_amdgcn_global_load_lds((const void*)(src + (size_t)min(first + lane, nslots - 1) * 8),
                                       (__attribute__((address_space(3))) void*)(dst + first * 8),
                                       16, 0, 0);
  }
}

// Dynamic LDS layouts (bytes), sized by the call's T. Regions that
// stage_dma fills keep 1 KB behind them (its overrun).
constexpr size_t kRedBytes = kDecWaves * 64 * 4 * sizeof(float);
constexpr size_t kDmaPad = 1024;
inline size_t front_lds(int T, int H) { return (size_t)T * H * 2 + kRedBytes + kDecodeMaxT * 4; }
inline size_t router_lds(int T, int L) { return (size_t)2 * T * L * 2 + kRedBytes; }
// two regions of token rows: with routing groups a workgroup's tasks read
// the latents of at most two groups
__host__ __device__ inline size_t gateup_region(int T, int L) { return (size_t)T * L + kDmaPad / 2; }
inline size_t gateup_lds(int T, int L) { return 2 * gateup_region(T, L) * 2; }
// a down wave's activation region (elements): T x inter rounded up to 1 KB
__host__ __device__ inline int down_region(int T, int I) { return (T * I + 511) / 512 * 512; }
// rt: latent tiles per wave (the partial sums of each go through LDS)
inline size_t down_lds(int T, int I, int rt) {
  return (size_t)kDownGroup * down_region(T, I) * 2 + rt * kRedBytes;
}
inline size_t uproj_lds(int T, int L) { return (size_t)T * L * 2 + kRedBytes; }

// ------------------------------------------------------------------ 1. D (+ folded router)

// Stages x (T x hidden) into LDS: the loads are issued by load(), the
// caller issues its weight loads, then finish() stores the rows and (for the
// residual block) applies RMSNorm in place: per token, in fp32, rounded to
// bf16 (the layer's input is a bf16 tensor).
template <int NV>
struct XStage {
  RowStage<NV> r;
  __device__ __forceinline__ void load(const DecodeArgs& a) { r.load(a.x, a.T * a.hidden); }
  __device__ __forceinline__ void finish(const DecodeArgs& a, uint16_t* xs, float* rstd) {
    const int H = a.hidden, T = a.T;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    r.store(xs, T * H);
    __syncthreads();
    if (!a.norm_weight) return;
    if (wave < T) {
      const uint16_t* xrow = xs + wave * H;
      float ss = 0.f;
      for (int k = lane * 8; k < H; k += 64 * 8) {
        const uint4 v = *(const uint4*)(xrow + k);
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = bf16_bits_to_f32(d[q] & 0xFFFFu), hi = bf16_bits_to_f32(d[q] >> 16);
          ss = fmaf(lo, lo, ss);
          ss = fmaf(hi, hi, ss);
        }
      }
      ss = wave_sum(ss);
      if (lane == 0) rstd[wave] = 1.0f / sqrtf(ss / (float)H + a.norm_eps);
    }
    __syncthreads();
    for (int i = tid * 8; i < T * H; i += kDecThreads * 8) {
      const int tt = i / H, k = i % H;
      const uint4 v = *(const uint4*)(xs + i);
      const uint32_t d[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = pack_bf16x2(bf16_bits_to_f32(d[q] & 0xFFFFu) * rstd[tt] * a.norm_weight[k + 2 * q],
                           bf16_bits_to_f32(d[q] >> 16) * rstd[tt] * a.norm_weight[k + 2 * q + 1]);
      *(uint4*)(xs + i) = make_uint4(o[0], o[1], o[2], o[3]);
    }
    __syncthreads();
  }
};

// Workgroups [0, G*latent/16) compute h for 16 latent rows each (K split
// over the 8 waves; with routing groups the rows of every group's D_g) and
// write bf16(h), plus the low half h - bf16(h) when hlo is set (the
// unfolded router reads both), and with one routing group bf16(h) as fp16
// with the workgroup's flag (1 when a value is not exact in fp16). With a
// folded router (a.RD), the next n_parts * E/16 workgroups compute logits
// for 16 experts over one of n_parts K parts: l_part = x_part . (W_hi +
// W_lo)_part (the bias with part 0). NCH = hidden / 256, NCHR = NCH /
// n_parts, TM >= T (the x staging's size). The workgroups also zero the
// fixed-point sum the down kernel adds into.
template <int NCH, int NCHR, int TM>
__global__ __launch_bounds__(kDecThreads) void k_dec_front(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int H = a.hidden, L = a.latent, T = a.T, E = a.n_experts;
  const int GL = a.n_groups * L;            // latent rows of all groups' D_g
  uint16_t* xs = lds;                       // [T][H] bf16
  float* red = (float*)(lds + T * H);       // [8][64][4]
  float* rstd = red + kDecWaves * 64 * 4;   // [T]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, t = lane & 15;
  for (int i = blockIdx.x * kDecThreads + tid; i < T * GL; i += gridDim.x * kDecThreads)
    a.zfix[i] = 0ull;  // the down kernel adds into it
  const int nd = GL / 16;
  XStage<(TM * NCH + 15) / 16> xr;  // T x hidden, T <= TM, hidden = 256 NCH
  if ((int)blockIdx.x < nd) {
    const int row0 = blockIdx.x * 16;
    const int kb = wave * (H / kDecWaves);
    xr.load(a);
    Bf16Rows<NCH> wr;
    int step;
    wr.load(bf16_lane(a.D, a.packed, GL, H, row0, kb, &step), step);
    xr.finish(a, xs, rstd);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    wr.mma(xs + min(t, T - 1) * H, kb, g, acc);  // token columns >= T are not stored
    const f32x4 tot = reduce_waves(acc, red);
    if (wave == 0) {
      bool inexact = false;
      if (t < T) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = row0 + g * 4 + r;
          const uint16_t hi = f32_to_bf16_bits(tot[r]);
          const float v = bf16_bits_to_f32(hi);
          a.hhi[(size_t)t * GL + n] = hi;
          if (a.hlo) a.hlo[(size_t)t * GL + n] = f32_to_bf16_bits(tot[r] - v);
          if (a.h16) {
            // bf16(h) as fp16: exact unless out of range, too small for
            // fp16's subnormals, or NaN
            const _Float16 f = (_Float16)v;
            inexact |= !((float)f == v);
            a.h16[(size_t)t * L + n] = __builtin_bit_cast(uint16_t, f);
          }
        }
      }
      if (a.h16) {
        const bool any = __ballot(inexact) != 0ull;
        if (lane == 0) a.hflag[blockIdx.x] = any ? 1 : 0;
      }
    }
    return;
  }
  // folded router: 16 experts, K part `part`
  const int rb = blockIdx.x - nd;
  const int e0 = (rb / a.n_parts) * 16, part = rb % a.n_parts;
  const int kb = part * (H / a.n_parts) + wave * (H / a.n_parts / kDecWaves);
  xr.load(a);
  Bf16Rows<NCHR> wh, wl;
  int step;
  wh.load(bf16_lane(a.RD, true, E, H, e0, kb, &step), step);
  wl.load(bf16_lane(a.RD + (size_t)E * H, true, E, H, e0, kb, &step), step);
  float bias[4] = {0.f, 0.f, 0.f, 0.f};
  if (a.bias && part == 0 && wave == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) bias[r] = a.bias[e0 + g * 4 + r];
  }
  xr.finish(a, xs, rstd);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const uint16_t* xrow = xs + min(t, T - 1) * H;
  wh.mma(xrow, kb, g, acc);
  wl.mma(xrow, kb, g, acc);
  const f32x4 tot = reduce_waves(acc, red);
  if (wave == 0 && t < T) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      a.logits[((size_t)part * T + t) * E + e0 + g * 4 + r] = tot[r] + bias[r];
  }
}

// ------------------------------------------------------------------ 1b. router from h

// logits = (hi + lo) R^T + b for 16 experts per workgroup (the unfolded
// router; K split over the 8 waves). latent = 256 NCH.
template <int NCH>
__global__ __launch_bounds__(kDecThreads) void k_dec_router(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int L = a.latent, T = a.T, E = a.n_experts;
  const int GL = a.n_groups * L;
  uint16_t* hi = lds;           // [T][L]
  uint16_t* lo = lds + T * L;   // [T][L]
  float* red = (float*)(lo + T * L);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, t = lane & 15;
  const int e0 = blockIdx.x * 16;
  const int grp = e0 / (E / a.n_groups);  // the 16 experts' routing group
  const int kb = wave * (L / kDecWaves);
  RowStage<(NCH + 1) / 2> sh_hi, sh_lo;  // T x latent, latent = 256 NCH
  // latent rows staged (and waited for) before the router rows are loaded
  // (measured: 0.6 us less per decode step)
  sh_hi.load_rows(a.hhi + (size_t)grp * L, T, L, GL);
  sh_lo.load_rows(a.hlo + (size_t)grp * L, T, L, GL);
  sh_hi.store(hi, T * L);
  sh_lo.store(lo, T * L);
  __syncthreads();
  (void)tid;
  Bf16Rows<NCH> wr;
  int step;
  wr.load(bf16_lane(a.R, a.packed, E, L, e0, kb, &step), step);
  float bias[4] = {0.f, 0.f, 0.f, 0.f};
  if (a.bias && wave == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) bias[r] = a.bias[min(e0 + g * 4 + r, E - 1)];
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  wr.mma2(hi + min(t, T - 1) * L, lo + min(t, T - 1) * L, kb, g, acc);
  const f32x4 tot = reduce_waves(acc, red);
  if (wave == 0 && t < T) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ee = e0 + g * 4 + r;
      if (ee < E) a.logits[(size_t)t * E + ee] = tot[r] + bias[r];
    }
  }
}

// ------------------------------------------------------------------ top-k

// One token's logits as order-preserving keys, lane l holding experts
// l, l + 64, ... (experts past E: key 0, below every logit's key). A logit
// is the sum of its n_parts parts, in part order. The loads are
// unconditional (clamped index) so that they stay in flight together.
template <int EPL>
__device__ __forceinline__ void wave_load_keys(const float* row, int E, int part_stride,
                                               int n_parts, float (&v)[EPL]) {
  const int lane = threadIdx.x & 63;
  float p1[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = min(lane + 64 * i, E - 1);
    v[i] = row[e];
    p1[i] = row[(n_parts > 1 ? part_stride : 0) + e];
  }
  if (n_parts > 1) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) v[i] += p1[i];
  }
}

// Top-k of one token from its logits (wave_load_keys) by this wave; lane
// j < k ends with choice j (descending value, equal values to the lower
// expert). Renormalised weights: exp(l_j - l_0) / sum over the k chosen.
template <int EPL>
__device__ __forceinline__ void wave_topk(const float (&v)[EPL], int E, int k, int* out_e,
                                          float* out_w) {
  const int lane = threadIdx.x & 63;
  uint32_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) key[i] = lane + 64 * i < E ? order_key(v[i]) : 0u;
  uint32_t my_key;
  int my_e;
  wave_select_topk<EPL>(key, E, k, my_key, my_e);
  const float top = key_value((uint32_t)__builtin_amdgcn_readlane((int)my_key, 0));
  const float ex = lane < k ? expf(key_value(my_key) - top) : 0.0f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    out_e[lane] = my_e;
    out_w[lane] = ex / sum;
  }
}

// ------------------------------------------------------------------ routing table

struct RouteLds {
  int idx[kDecodeMaxT * 16];
  float w[kDecodeMaxT * 16];
  uint32_t flags[kMaxExperts / 32];
  int list[kDecodeMaxT * 16];
  int n_act;
};

// The active experts of the T x k choices in ascending order (rl.list,
// rl.n_act). rl.flags must be zero and rl.idx complete (barrier) on entry.
__device__ __forceinline__ void build_active_list(int E, int P, RouteLds& rl) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int p = tid; p < P; p += kDecThreads)
    atomicOr(&rl.flags[rl.idx[p] >> 5], 1u << (rl.idx[p] & 31));
  __syncthreads();
  if (wave == 0) {  // compact the set bits in ascending order (E <= 1024 bits)
    const int nw = (E + 31) / 32;
    const uint32_t bits = lane < nw ? rl.flags[lane] : 0u;
    const int cnt = __popc(bits);
    const int inc = wave_inclusive_scan(cnt);
    int pos = inc - cnt;
    for (uint32_t b = bits; b; b &= b - 1) rl.list[pos++] = lane * 32 + __ffs(b) - 1;
    if (lane == 63) rl.n_act = inc;
  }
  __syncthreads();
}

// Routing table for the down kernel: the active list, each token's gate
// weight per slot (slot 0 is the shared expert with weight 1, slot s >= 1
// the s-th active expert), and the optional debug copies.
__device__ __forceinline__ void publish_routing(const DecodeArgs& a, const RouteLds& rl) {
  const int E = a.n_experts, T = a.T, k = a.top_k, P = T * k;
  const int tid = threadIdx.x;
  const int n_act = rl.n_act;
  if (tid == 0) a.route_n_act[0] = n_act;
  for (int i = tid; i < n_act; i += kDecThreads) a.route_list[i] = rl.list[i];
  for (int i = tid; i < (n_act + 1) * T; i += kDecThreads) {
    const int slot = i / T, t = i % T;
    float w = 0.0f;
    if (slot == 0) {
      w = a.n_shared ? 1.0f : 0.0f;
    } else {
      const int e = rl.list[slot - 1];
      for (int j = 0; j < k; ++j)
        if (rl.idx[t * k + j] == e) w = rl.w[t * k + j];
    }
    a.route_wtab[i] = w;
  }
  if (a.dbg_idx)
    for (int i = tid; i < P; i += kDecThreads) a.dbg_idx[i] = rl.idx[i];
  if (a.dbg_w)
    for (int i = tid; i < P; i += kDecThreads) a.dbg_w[i] = rl.w[i];
  if (a.dbg_logits)
    for (int i = tid; i < T * E; i += kDecThreads)
      a.dbg_logits[i] = a.n_parts > 1 ? a.logits[i] + a.logits[T * E + i] : a.logits[i];
  // counts, offsets and the stable permutation of the P pairs (pair p of
  // expert e goes after the pairs of smaller experts and the earlier pairs of e)
  if (a.dbg_counts)
    for (int e = tid; e < E; e += kDecThreads) {
      int c = 0;
      for (int p = 0; p < P; ++p) c += rl.idx[p] == e;
      a.dbg_counts[e] = c;
    }
  if (a.dbg_offsets)
    for (int e = tid; e <= E; e += kDecThreads) {
      int o = 0;
      for (int p = 0; p < P; ++p) o += rl.idx[p] < e;
      a.dbg_offsets[e] = o;
    }
  if (a.dbg_perm)
    for (int p = tid; p < P; p += kDecThreads) {
      const int e = rl.idx[p];
      int pos = 0;
      for (int q = 0; q < P; ++q) pos += (rl.idx[q] < e) || (rl.idx[q] == e && q < p);
      a.dbg_perm[pos] = p;
    }
}

// SiLU(gate) * up of a 16-row tile, to act[t][n0 + rows] (bf16, t < T).
__device__ __forceinline__ void store_gateup(const f32x4& g4, const f32x4& u4, float gsg,
                                             float gsu, uint16_t* act, int I, int T, int n0,
                                             int lane) {
  const int t = lane & 15, g = lane >> 4;
  if (t >= T) return;
  float v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float gg = gsg * g4[r], uu = gsu * u4[r];
    v[r] = silu_fast(gg) * uu;
  }
  *(uint2*)(act + (size_t)t * I + n0 + g * 4) =
      make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}


// ------------------------------------------------------------------ 2. top-k + gate/up

// One wave's task: the gate and up tiles of one expert slot, 16 rows
// (n0 .. n0+15) over the whole latent width, SiLU(gate) * up to
// act[slot][t][n0 + rows]. hs = the token rows in LDS. latent = 128 NCH.
// The chunks are software-pipelined: W chunk pairs (gate and up) stay in
// flight and each pair is dequantised and multiplied as soon as it lands,
// so the vector work of the exact dequantisation overlaps the weight
// stream instead of piling up after it (measured at the 145B decode shapes
// with T = 4: 20.1 us with every chunk issued up front, 17.5 us with
// W = 2, 18.6 us with 4 and 20.3 us with 8).
template <int NCH, int BITS, bool F16>
__device__ __forceinline__ void gateup_task(const DecodeArgs& a, const uint16_t* hs, int slot,
                                            int e, int n0) {
  constexpr int W = 2;  // chunk pairs in flight per wave (measured best of 2, 4, 8)
  const int L = a.latent, T = a.T, I = a.inter;
  const int lane = threadIdx.x & 63, t = lane & 15, g = lane >> 4;
  const bool sh = slot == 0;
  const Fp4Mat gm = sh ? a.sh_gate : a.gate;
  const Fp4Mat um = sh ? a.sh_up : a.up;
  const float gsg = gm.gscale[e], gsu = um.gscale[e];
  const Fp4Lane lg = fp4_lane(gm, a.packed, e, I, L, n0, 0, BITS);
  const Fp4Lane lu = fp4_lane(um, a.packed, e, I, L, n0, 0, BITS);
  Fp4Rows<NCH, BITS> wg, wu;
  auto ld = [&](int i) {
    if constexpr (BITS == 4) {
      const uint4 v = *(const uint4*)(lg.c + i * lg.cstep);
      wg.c[i][0] = v.x; wg.c[i][1] = v.y; wg.c[i][2] = v.z; wg.c[i][3] = v.w;
      const uint4 u = *(const uint4*)(lu.c + i * lu.cstep);
      wu.c[i][0] = u.x; wu.c[i][1] = u.y; wu.c[i][2] = u.z; wu.c[i][3] = u.w;
    } else {
      const uint3 v = *(const uint3*)(lg.c + i * lg.cstep);
      wg.c[i][0] = v.x; wg.c[i][1] = v.y; wg.c[i][2] = v.z;
      const uint3 u = *(const uint3*)(lu.c + i * lu.cstep);
      wu.c[i][0] = u.x; wu.c[i][1] = u.y; wu.c[i][2] = u.z;
    }
    wg.s[i] = *(const uint2*)(lg.s + i * lg.sstep);
    wu.s[i] = *(const uint2*)(lu.s + i * lu.sstep);
  };
  f32x4 ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
  const uint16_t* row = hs + min(t, T - 1) * L;
#pragma unroll
  for (int i = 0; i < W && i < NCH; ++i) ld(i);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    if (i + W < NCH) ld(i + W);
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t spg = ((g & 2) ? wg.s[i].y : wg.s[i].x) >> (16 * (g & 1));
    const uint32_t spu = ((g & 2) ? wu.s[i].y : wu.s[i].x) >> (16 * (g & 1));
    const float g0 = e4m3_to_f32(spg & 0xFFu), g1 = e4m3_to_f32((spg >> 8) & 0xFFu);
    const float u0 = e4m3_to_f32(spu & 0xFFu), u1 = e4m3_to_f32((spu >> 8) & 0xFFu);
    if constexpr (F16) {  // hs holds the token rows as fp16 (all exact)
      const _Float16 hg0 = (_Float16)g0, hg1 = (_Float16)g1;
      const _Float16 hu0 = (_Float16)u0, hu1 = (_Float16)u1;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f16x8 b = *(const f16x8*)(row + (i * 4 + g) * 32 + q * 8);
        ag = mfma16x16x32_f16(dequant8_f16(wg.codes8(i, q), q < 2 ? hg0 : hg1), b, ag);
        au = mfma16x16x32_f16(dequant8_f16(wu.codes8(i, q), q < 2 ? hu0 : hu1), b, au);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x8 b = *(const bf16x8*)(row + (i * 4 + g) * 32 + q * 8);
        ag = mfma16x16x32(dequant8(wg.codes8(i, q), q < 2 ? g0 : g1), b, ag);
        au = mfma16x16x32(dequant8(wu.codes8(i, q), q < 2 ? u0 : u1), b, au);
      }
    }
  }
  store_gateup(ag, au, gsg, gsu, a.act + (size_t)slot * T * I, I, T, n0, lane);
}

// Each workgroup takes the top-k of every token (one wave per token) from
// the logits, loaded together with its staged token rows (one round trip),
// and builds the active list (the same in every workgroup); workgroup 0
// publishes the routing table for the down kernel. The (slot, 16-row tile)
// tasks of the live slots (slot 0: the shared expert when there is one;
// slot s >= 1: the s-th active expert) are then split evenly over the grid
// (one workgroup per CU, so the top-k is paid once per CU and every CU
// shares the dequantisation work): workgroup b takes tasks
// [b P / G, (b + 1) P / G) of the P, wave w every eighth of them from w.
// latent = 128 NCH.
template <int NCH, int BITS>
__global__ __launch_bounds__(kDecThreads) void k_dec_gateup(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  __shared__ RouteLds rl;
  const int L = a.latent, T = a.T, I = a.inter, E = a.n_experts;
  const int GL = a.n_groups * L, epg = E / a.n_groups;
  uint16_t* hs = lds;  // two regions of [T][L] (+ the DMA pad)
  const int region = (int)gateup_region(T, L);
  const int tid = threadIdx.x, wave = tid >> 6;
  const int tiles = I / 16;
  constexpr int NV = (NCH + 3) / 4;  // 16-byte slots per thread: T x latent, T <= 8
  for (int i = tid; i < kMaxExperts / 32; i += kDecThreads) rl.flags[i] = 0u;
  const float* lrow = a.logits + (size_t)min(wave, T - 1) * E;
  const bool one_group = a.n_groups == 1;  // the rows are known before the routing
  // with one group the rows come both as bf16 (region 0) and as fp16
  // (region 1), and the front's flags say whether the fp16 copy is exact
  const int nfl = a.h16 ? L / 16 : 0;
  const int fl = nfl > 0 ? a.hflag[min(tid, nfl - 1)] : 0;  // (the flags exist whenever h16 does)
  auto stage_rows = [&]() {
    if (one_group) {
      stage_dma<NV>(a.hhi, T * L, hs);
      if (a.h16) stage_dma<NV>(a.h16, T * L, hs + region);
    }
  };
  if (E <= 512) {
    float v[8];
    wave_load_keys<8>(lrow, E, T * E, a.n_parts, v);
    stage_rows();
    if (wave < T) wave_topk<8>(v, E, a.top_k, rl.idx + wave * a.top_k, rl.w + wave * a.top_k);
  } else {
    float v[16];
    wave_load_keys<16>(lrow, E, T * E, a.n_parts, v);
    stage_rows();
    if (wave < T) wave_topk<16>(v, E, a.top_k, rl.idx + wave * a.top_k, rl.w + wave * a.top_k);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's rows have landed in LDS
  // the barrier every thread passes (not under the && below)
  const int inexact = __syncthreads_or(tid < nfl && fl != 0);
  const bool use16 = nfl > 0 && !inexact;
  build_active_list(E, T * a.top_k, rl);
  if (blockIdx.x == 0) publish_routing(a, rl);
  const int s0 = a.n_shared ? 0 : 1;  // first live slot
  const int P = (rl.n_act + 1 - s0) * tiles;
  const int G = gridDim.x;
  const int p0 = (int)((int64_t)blockIdx.x * P / G);
  const int p1 = (int)((int64_t)(blockIdx.x + 1) * P / G);
  // routing groups: this workgroup's tasks span at most two slots, so at
  // most two groups' latents (region 0: the first task's group)
  auto group_of = [&](int slot) { return slot == 0 ? 0 : rl.list[slot - 1] / epg; };
  int ga = 0;
  if (!one_group && p0 < p1) {
    ga = group_of(s0 + p0 / tiles);
    const int gb = group_of(s0 + (p1 - 1) / tiles);
    stage_dma_rows<NV>(a.hhi + (size_t)ga * L, T, L, GL, hs);
    if (gb != ga) stage_dma_rows<NV>(a.hhi + (size_t)gb * L, T, L, GL, hs + region);
    __builtin_amdgcn_s_waitcnt(0);
  }
  if (!one_group) __syncthreads();
  if (use16) {  // one group: every task reads region 1
    for (int p = p0 + wave; p < p1; p += kDecWaves) {
      const int slot = s0 + p / tiles;
      gateup_task<NCH, BITS, true>(a, hs + region, slot, slot == 0 ? 0 : rl.list[slot - 1],
                                   (p % tiles) * 16);
    }
    return;
  }
  for (int p = p0 + wave; p < p1; p += kDecWaves) {
    const int slot = s0 + p / tiles;
    const uint16_t* rows = hs + (group_of(slot) == ga ? 0 : region);
    gateup_task<NCH, BITS, false>(a, rows, slot, slot == 0 ? 0 : rl.list[slot - 1],
                                  (p % tiles) * 16);
  }
}

// ------------------------------------------------------------------ 3. down + combine

// Workgroup (16 RT latent rows from r0, slot group q): wave w takes slot
// s = 8q + w (slot 0 the shared expert, s >= 1 the s-th active expert;
// slots past the active ones, and slot 0 without a shared expert, have
// nothing to do). The wave stages its slot's activations (the matrix-core
// token operand) into its own LDS region once, streams the 16 rows of each
// of its RT latent tiles of the slot's down matrix chunk by chunk with the
// next chunk in flight (across the tiles too), and scales the products by
// the gate weight and the matrix scale. (Reading the
// token operand straight from L2 instead took four 16-byte loads per lane
// and chunk, three quarters of them repeats at T = 4: 12.4 us for the
// 145B layer at T = 4.) The eight
// slots' products are added in slot order through LDS, and the group sum is
// added into zfix in 64-bit fixed point (units of 2^-32) with integer
// atomics: integer addition is exact, so the result does not depend on the
// order in which the groups arrive. inter = 128 NCH.
// Held to at most 85 registers (six waves per SIMD) so that three
// workgroups share a CU and the grid of (latent/16) x groups workgroups
// runs in one round at T = 4 (672 workgroups, 768 resident); at 94
// registers it took two. Each of the RT tiles has its own LDS sums.
template <int NCH, int RT>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(6, 8))) void k_dec_down(
    DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];  // 8 activation regions, red
  __shared__ int wgrp[kDecWaves];  // each wave's routing group (-1: no slot)
  const int L = a.latent, T = a.T, I = a.inter;
  const int GL = a.n_groups * L, epg = a.n_experts / a.n_groups;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, t = lane & 15;
  const int ntile = L / (16 * RT);
  const int r0 = (blockIdx.x % ntile) * 16 * RT, q = blockIdx.x / ntile;
  const int region = down_region(T, I);
  float* red = (float*)(lds + kDownGroup * region);
  // the routing table, read together (clamped indices; used only when live)
  const int n_act = a.route_n_act[0];
  const int s = kDownGroup * q + wave;
  const int sc = min(s, a.max_active);
  const int e_guess = a.route_list[max(sc - 1, 0)];
  const float w_guess = a.route_wtab[sc * T + min(t, T - 1)];
  if (q >= (n_act + kDownGroup) / kDownGroup) return;  // uniform over the workgroup
  f32x4 y[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) y[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool live = (s > 0 || a.n_shared) && s <= n_act;
  if (lane == 0) wgrp[wave] = live ? (s == 0 ? 0 : e_guess / epg) : -1;
  if (live) {  // uniform over the wave
    const bool sh = s == 0;
    const Fp4Mat dm = sh ? a.sh_down : a.down;
    const int e = sh ? 0 : e_guess;
    const float gs = dm.gscale[e];
    // this slot's activations into the wave's own LDS region, before any
    // weight load: the wave waits for them with a count of its later loads
    uint16_t* act = lds + wave * region;
    stage_dma_wave<2 * NCH>(a.act + (size_t)s * T * I, T * I, act);
    issue_fence();
    Fp4Lane l[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) l[rt] = fp4_lane(dm, a.packed, e, L, I, r0 + 16 * rt, 0);
    Fp4Rows<NCH * RT> wd;  // chunk i: tile i / NCH, chunk i % NCH of its row
    // software-pipelined as in the gate/up kernel: the next chunk is in
    // flight while one is multiplied (across the tiles too)
    auto ld = [&](int i) {
      const Fp4Lane& lt = l[i / NCH];
      const int c = i % NCH;
      const uint4 v = *(const uint4*)(lt.c + c * lt.cstep);
      wd.c[i][0] = v.x; wd.c[i][1] = v.y; wd.c[i][2] = v.z; wd.c[i][3] = v.w;
      wd.s[i] = *(const uint2*)(lt.s + c * lt.sstep);
    };
    ld(0);
    issue_fence();
    wait_vmcnt<2>();  // everything but chunk 0's two loads: the staged rows have landed
    const uint16_t* arow = act + min(t, T - 1) * I;
#pragma unroll
    for (int i = 0; i < NCH * RT; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < NCH * RT) ld(i + 1);
      __builtin_amdgcn_sched_barrier(0);
      const int c = i % NCH;
      const uint32_t sp = ((g & 2) ? wd.s[i].y : wd.s[i].x) >> (16 * (g & 1));
      const float s0 = e4m3_to_f32(sp & 0xFFu), s1 = e4m3_to_f32((sp >> 8) & 0xFFu);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        y[i / NCH] = mfma16x16x32(dequant8(wd.codes8(i, k), k < 2 ? s0 : s1),
                                  *(const bf16x8*)(arow + (c * 4 + g) * 32 + k * 8), y[i / NCH]);
    }
    const float sw = w_guess * gs;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) y[rt][r] *= sw;
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) *(f32x4*)(red + ((rt * kDecWaves + wave) * 64 + lane) * 4) = y[rt];
  __syncthreads();
  if (wave == 0 && t < T) {
    // the slots' products in slot order, one sum per run of slots of one
    // routing group (slots are in ascending expert order, so a group's
    // slots are adjacent), each added into that group's z
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      auto flush = [&](const f32x4& tot, int grp) {
        unsigned long long* zp =
            a.zfix + (size_t)t * GL + (size_t)grp * L + r0 + 16 * rt + g * 4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const long long fx = (long long)__builtin_rintf(tot[r] * 4294967296.0f);
          __hip_atomic_fetch_add(zp + r, (unsigned long long)fx, __ATOMIC_RELAXED, AGENT);
        }
      };
      f32x4 tot = {0.f, 0.f, 0.f, 0.f};
      int cur = -1;
      for (int w = 0; w < kDecWaves; ++w) {
        const int gw = wgrp[w];
        if (gw < 0) continue;
        if (gw != cur) {
          if (cur >= 0) flush(tot, cur);
          tot = f32x4{0.f, 0.f, 0.f, 0.f};
          cur = gw;
        }
        tot += *(const f32x4*)(red + ((rt * kDecWaves + w) * 64 + lane) * 4);
      }
      if (cur >= 0) flush(tot, cur);
    }
  }
}

// ------------------------------------------------------------------ 4. U

template <int NCH, int TM>
__global__ __launch_bounds__(kDecThreads) void k_dec_uproj(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int L = a.latent, H = a.hidden, T = a.T;
  const int GL = a.n_groups * L;
  uint16_t* zs = lds;  // [T][L] bf16
  float* red = (float*)(lds + T * L);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, t = lane & 15;
  const int m0 = blockIdx.x * 16;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // one pass per routing group g: z_g U_g^T (one pass without groups)
  for (int grp = 0; grp < a.n_groups; ++grp) {
    const int kb = grp * L + wave * (L / kDecWaves);
    // z_g = bf16(zfix * 2^-32): thread i converts pairs 2 (i + 512 j) of the
    // T x latent sums (loads issued before the weight loads)
    constexpr int NZ = (TM * 256 * NCH / 2 + kDecThreads - 1) / kDecThreads;  // T <= TM
    ulonglong2 zv[NZ];
#pragma unroll
    for (int j = 0; j < NZ; ++j) {
      const int i = 2 * min(tid + j * kDecThreads, T * L / 2 - 1);
      zv[j] = *(const ulonglong2*)(a.zfix + (size_t)(i / L) * GL + grp * L + i % L);
    }
    Bf16Rows<NCH> wr;
    int step;
    const uint16_t* wb = bf16_lane(a.U, a.packed, H, GL, m0, kb, &step);
    wr.load(wb, step);
    if (grp > 0) __syncthreads();  // the previous group's rows have been read
#pragma unroll
    for (int j = 0; j < NZ; ++j) {
      const int i = min(tid + j * kDecThreads, T * L / 2 - 1);  // the last pair repeats (same value)
      *(uint32_t*)(zs + 2 * i) =
          pack_bf16x2((float)(long long)zv[j].x * 2.3283064365386963e-10f,
                      (float)(long long)zv[j].y * 2.3283064365386963e-10f);
    }
    __syncthreads();
    wr.mma(zs + min(t, T - 1) * L - grp * L, kb, g, acc);
  }
  const f32x4 tot = reduce_waves(acc, red);
  if (wave == 0 && t < T) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = m0 + g * 4 + r;
      if (n < H) {
        float o = tot[r];
        if (a.norm_weight) o += bf16_bits_to_f32(a.x[(size_t)t * H + n]);
        a.out[(size_t)t * H + n] = f32_to_bf16_bits(o);
      }
    }
  }
}

// ------------------------------------------------------------------ launch

// Raises a kernel's dynamic-LDS limit once per device (to what the largest
// supported T needs) instead of on every call.
static hipError_t ensure_lds(const void* fn, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({fn, dev})) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) done.insert({fn, dev});
  return e;
}

// Calls f(std::integral_constant<int, N>) for the chunk counts the kernels
// are instantiated for.
template <class F>
static hipError_t with_nch(int n, F&& f) {
  switch (n) {
    case 1: return f(std::integral_constant<int, 1>{});
    case 2: return f(std::integral_constant<int, 2>{});
    case 4: return f(std::integral_constant<int, 4>{});
    case 5: return f(std::integral_constant<int, 5>{});
    case 7: return f(std::integral_constant<int, 7>{});
    case 8: return f(std::integral_constant<int, 8>{});
    case 10: return f(std::integral_constant<int, 10>{});
    default: return hipErrorInvalidValue;
  }
}

static bool nch_ok(int n) {
  return n == 1 || n == 2 || n == 4 || n == 5 || n == 7 || n == 8 || n == 10;
}

bool decode_supported(int hidden, int latent, int inter, int n_experts, int top_k, int n_groups,
                      int T) {
  if (T < 1 || T > kDecodeMaxT || n_experts > kMaxExperts || top_k > 16) return false;
  // routing groups: a router workgroup's 16 experts share a group
  if (n_groups > 1 && (n_experts / n_groups) % 16) return false;
  // D, U and the router split K over 8 waves x 4 lane groups x 8 bf16;
  // expert rows are consumed in 128-weight chunks by 4 lane groups.
  if (hidden % 256 || latent % 256 || inter % 128) return false;
  if (!nch_ok(hidden / 256) || !nch_ok(latent / 256) || !nch_ok(inter / 128)) return false;
  // register budgets: a gate/up wave holds 2 x latent/128 chunks of
  // weights, a down wave inter/128 chunks and their token operands
  if (latent / 128 > 14 || inter / 128 > 7) return false;
  const size_t lim = 96 * 1024;
  return front_lds(kDecodeMaxT, hidden) <= lim && router_lds(kDecodeMaxT, latent) <= lim &&
         gateup_lds(kDecodeMaxT, latent) + sizeof(RouteLds) <= lim &&
         down_lds(kDecodeMaxT, inter, 2) <= lim && uproj_lds(kDecodeMaxT, latent) <= lim;
}

int decode_front_parts(int hidden) { return (hidden / 256) % 2 == 0 ? 2 : 1; }

// Compute units of the current device (once per device).
static int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  static std::mutex mu;
  static std::map<int, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  const auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  return cache[dev] = n;
}

hipError_t launch_decode(const DecodeArgs& args, hipStream_t st, const StageMarks& mk) {
  DecodeArgs a = args;
  const int H = a.hidden, L = a.latent, I = a.inter, E = a.n_experts, T = a.T;
  const dim3 block(kDecThreads);
  hipError_t err;
  // 1. h = x D^T (+ the router logits from x with a folded router)
  const int nparts = a.RD ? decode_front_parts(H) : 1;
  a.n_parts = nparts;
  err = with_nch(H / 256, [&](auto N) {
    constexpr int n = decltype(N)::value;
    constexpr int nr = n % 2 == 0 ? n / 2 : n;
    // x staged for at most 4 or 8 tokens: at T <= 4 half the loads of the
    // T <= 8 copy would re-read the last slot
    const auto fn = T <= 4 ? k_dec_front<n, nr, 4> : k_dec_front<n, nr, kDecodeMaxT>;
    hipError_t e = ensure_lds((const void*)fn, front_lds(kDecodeMaxT, H));
    const int grid = a.n_groups * L / 16 + (a.RD ? nparts * (E / 16) : 0);
    if (e == hipSuccess) e = mk.launch(kStageDproj, fn, dim3(grid), block, front_lds(T, H), a);
    return e;
  });
  if (err != hipSuccess) return err;
  // 1b. without a folded router: logits = (hi + lo) R^T + b
  if (!a.RD) {
    err = with_nch(L / 256, [&](auto N) {
      constexpr int n = decltype(N)::value;
      hipError_t e = ensure_lds((const void*)k_dec_router<n>, router_lds(kDecodeMaxT, L));
      if (e == hipSuccess)
        e = mk.launch(kStageRouter, k_dec_router<n>, dim3((E + 15) / 16), block, router_lds(T, L),
                      a);
      return e;
    });
    if (err != hipSuccess) return err;
  }
  // 2. top-k + gate/up (slot 0: the shared expert)
  const auto gateup = [&](auto N, auto B) {
    constexpr int n = decltype(N)::value, bits = decltype(B)::value;
    if constexpr (2 * n > 14) {
      return hipErrorInvalidValue;  // excluded by decode_supported
    } else {
      const int tasks = (1 + a.max_active) * (I / 16);
      // at most one workgroup per CU: 8 tasks each (one per wave) when that
      // keeps at least half the CUs busy, else every CU with fewer tasks
      // each (measured at the 145B shapes: T = 2, 105 workgroups of 8
      // tasks, 36.1 us per step; 256 of 3 or 4, 33.5 us; at T = 3 and 4 the
      // 8-task grid is as fast or faster); and at most inter/16 tasks each
      // (so a workgroup's tasks span at most two slots: the two latent
      // regions of the routing-group staging)
      const int cus = cu_count();
      const int full = (tasks + kDecWaves - 1) / kDecWaves;
      const int grid =
          std::max(std::min(cus, full < cus / 2 ? tasks : full), (tasks + I / 16 - 1) / (I / 16));
      const auto fn = k_dec_gateup<2 * n, bits>;
      hipError_t e = ensure_lds((const void*)fn, gateup_lds(kDecodeMaxT, L));
      if (e == hipSuccess)
        e = mk.launch(kStageGateup, fn, dim3(std::max(grid, 1)), block, gateup_lds(T, L), a);
      return e;
    }
  };
  err = with_nch(L / 256, [&](auto N) {
    return a.gateup_bits == 3 ? gateup(N, std::integral_constant<int, 3>{})
                              : gateup(N, std::integral_constant<int, 4>{});
  });
  if (err != hipSuccess) return err;
  // 3. down + combine
  err = with_nch(I / 128, [&](auto N) {
    constexpr int n = decltype(N)::value;
    if constexpr (n > 7) {
      return hipErrorInvalidValue;  // excluded by decode_supported
    } else {
      // from T = 5 a slot's staged activations (T x inter) outweigh the
      // wave's 16 weight rows, so each wave takes two latent tiles of its
      // slot and stages them once (measured at the 145B shapes: T = 5
      // 46.3 -> 45.3 us, T = 8 68.7 -> 65.5 us per step; T <= 4 slower)
      const int rt = (T >= 5 && (L / 16) % 2 == 0) ? 2 : 1;
      const int grid = (L / (16 * rt)) * decode_down_groups(a.max_active);
      const auto fn = rt == 2 ? k_dec_down<n, 2> : k_dec_down<n, 1>;
      hipError_t e = ensure_lds((const void*)fn, down_lds(kDecodeMaxT, I, rt));
      if (e == hipSuccess) e = mk.launch(kStageDown, fn, dim3(grid), block, down_lds(T, I, rt), a);
      return e;
    }
  });
  if (err != hipSuccess) return err;
  // 4. out = z U^T (+ x)
  return with_nch(L / 256, [&](auto N) {
    constexpr int n = decltype(N)::value;
    const auto fn = T <= 4 ? k_dec_uproj<n, 4> : k_dec_uproj<n, kDecodeMaxT>;  // as the front
    hipError_t e = ensure_lds((const void*)fn, uproj_lds(kDecodeMaxT, L));
    if (e == hipSuccess)
      e = mk.launch(kStageUproj, fn, dim3((H + 15) / 16), block, uproj_lds(T, L), a);
    return e;
  });
}

// ------------------------------------------------------------------ decode-packed layouts

// fp4 set [count][N][K] (N % 16 == 0, K % 128 == 0): block (e, t, c) = matrix
// e, rows [16t, 16t + 16), columns [128c, 128c + 128), in (e, t, c) order.
// Codes: 64 lanes x CB bytes (CB = 16 for e2m1, 12 for an E1M1 chunk), lane
// l's at CB l = row 16t + l % 16, columns 128c + 32 (l / 16) .. +32. Scales:
// 128 bytes, row 16t + r's eight block scales of the 128 columns at 8 r. One
// thread moves one lane's code bytes and (lanes 0..15) its row's 8 scale bytes.
template <int BITS>
__global__ __launch_bounds__(256) void k_pack_fp4_decode(const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales,
                                                         int64_t n_lanes, int K,
                                                         uint8_t* __restrict__ pcodes,
                                                         uint8_t* __restrict__ pscales) {
  constexpr int CB = BITS == 4 ? 16 : 12;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_lanes) return;
  const int l = (int)(i & 63);
  const int64_t blk = i >> 6;
  const int c = (int)(blk % (K / 128));
  const int64_t row = (blk / (K / 128)) * 16 + (l & 15);  // e * N + 16 t + l % 16
  const uint8_t* src = codes + row * ((int64_t)K / 32 * CB) + (c * 4 + (l >> 4)) * CB;
  if (BITS == 4)
    *(uint4*)(pcodes + i * CB) = *(const uint4*)src;
  else
    *(uint3*)(pcodes + i * CB) = *(const uint3*)src;
  if (l < 16)
    *(uint2*)(pscales + blk * 128 + l * 8) = *(const uint2*)(scales + row * (K / 16) + c * 8);
}

// bf16 [N][K] (N % 16 == 0, K % 32 == 0): block (t, c) = rows [16t, 16t + 16),
// columns [32c, 32c + 32), in (t, c) order, 1 KB: lane l's 16 bytes at 16 l =
// row 16t + l % 16, columns 32c + 8 (l / 16) .. +8.
__global__ __launch_bounds__(256) void k_pack_bf16_decode(const uint16_t* __restrict__ w,
                                                          int64_t n_lanes, int K,
                                                          uint16_t* __restrict__ pw) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_lanes) return;
  const int l = (int)(i & 63);
  const int64_t blk = i >> 6;
  const int c = (int)(blk % (K / 32));
  const int64_t row = (blk / (K / 32)) * 16 + (l & 15);
  *(uint4*)(pw + i * 8) = *(const uint4*)(w + row * K + c * 32 + (l >> 4) * 8);
}

hipError_t launch_pack_fp4_decode(const uint8_t* codes, const uint8_t* scales, int count, int N,
                                  int K, int bits, uint8_t* pcodes, uint8_t* pscales,
                                  hipStream_t stream) {
  const int64_t n_lanes = (int64_t)count * (N / 16) * (K / 128) * 64;
  if (n_lanes == 0) return hipSuccess;
  const dim3 grid((unsigned)((n_lanes + 255) / 256));
  if (bits == 3)
    hipLaunchKernelGGL(k_pack_fp4_decode<3>, grid, dim3(256), 0, stream, codes, scales, n_lanes,
                       K, pcodes, pscales);
  else
    hipLaunchKernelGGL(k_pack_fp4_decode<4>, grid, dim3(256), 0, stream, codes, scales, n_lanes,
                       K, pcodes, pscales);
  return hipGetLastError();
}

hipError_t launch_pack_bf16_decode(const uint16_t* w, int N, int K, uint16_t* pw,
                                   hipStream_t stream) {
  const int64_t n_lanes = (int64_t)N * K / 8;
  if (n_lanes == 0) return hipSuccess;
  hipLaunchKernelGGL(k_pack_bf16_decode, dim3((unsigned)((n_lanes + 255) / 256)), dim3(256), 0,
                     stream, w, n_lanes, K, pw);
  return hipGetLastError();
}

// The router folded onto the residual width: W[e][i] = sum_j R[e][j] D[j][i]
// (so x W^T = (x D^T) R^T; with routing groups, D is the expert's D_g), accumulated in fp64 in j order, then stored as
// hi = bf16(W) and lo = bf16(W - hi) (together about 16 significant bits)
// at their places in the decode-packed bf16 layout of an [E][hidden]
// matrix: hi in dst[0 .. E*hidden), lo after it. One thread per element;
// the workgroup's 256 threads share e (the R row is read as a broadcast).
__global__ __launch_bounds__(256) void k_router_fold(const uint16_t* __restrict__ R,
                                                     const uint16_t* __restrict__ D, int E,
                                                     int latent, int hidden, int n_groups,
                                                     uint16_t* __restrict__ dst) {
  const int i = blockIdx.x * 256 + threadIdx.x;  // column (hidden)
  const int e = blockIdx.y;                      // row (expert)
  if (i >= hidden) return;
  const uint16_t* rrow = R + (size_t)e * latent;
  D += (size_t)(e / (E / n_groups)) * latent * hidden;  // the expert's group's D_g
  double acc = 0.0;
  for (int j = 0; j < latent; ++j)
    acc = fma((double)bf16_bits_to_f32(rrow[j]), (double)bf16_bits_to_f32(D[(size_t)j * hidden + i]),
              acc);
  const float w = (float)acc;
  const uint16_t hi = f32_to_bf16_bits(w);
  const uint16_t lo = f32_to_bf16_bits(w - bf16_bits_to_f32(hi));
  // decode-packed position: block (e / 16, i / 32), lane (e % 16) + 16 ((i % 32) / 8), element i % 8
  const size_t pos = ((size_t)(e / 16) * (hidden / 32) + i / 32) * 512 +
                     ((e % 16) + 16 * ((i % 32) / 8)) * 8 + i % 8;
  dst[pos] = hi;
  dst[(size_t)E * hidden + pos] = lo;
}

hipError_t launch_router_fold(const uint16_t* R, const uint16_t* D, int E, int latent, int hidden,
                              int n_groups, uint16_t* dst, hipStream_t stream) {
  if (E <= 0 || hidden <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_router_fold, dim3((hidden + 255) / 256, E), dim3(256), 0, stream, R, D, E,
                     latent, hidden, n_groups < 1 ? 1 : n_groups, dst);
  return hipGetLastError();
}

}  // namespace moe
