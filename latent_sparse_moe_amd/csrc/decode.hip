// Weight-streaming decode path of the latent-MoE layer (T <= 8 tokens).
//
// At a handful of tokens every weight byte feeds only T multiply-adds, so the
// layer is bound by HBM bandwidth and by the fixed latency of each dependent
// step. Six kernels; in each, every wave issues its loads before anything
// else (the router and routed gate/up kernels first stage their activations),
// and a kernel boundary is the only grid-wide synchronisation (no workgroup
// ever waits for another one to be scheduled):
//
//   1. dec_dproj   h = x D^T (RMSNorm fused for the residual block); K split
//                  over the 8 waves; h leaves as bf16 hi + lo
//   2. dec_router  logits = (hi + lo) R^T + b, 16 experts per workgroup. The
//                  shared expert's gate/up (routing-independent) runs in the
//                  same launch.
//   3. dec_gateup  every workgroup first takes the top-k of every token and
//                  builds the active list (workgroup 0 also publishes the
//                  routing table); then one wave per (routed expert, 16
//                  intermediate rows, matrix, K half): silu(gate) * up
//   4. dec_down    one workgroup per (expert slot, 128 latent rows): the slot's
//                  activations are staged once in LDS, each wave takes 16 rows;
//                  partial rows, weighted by the gate weights, go to a per-slot
//                  buffer
//   5. dec_combine z = the slots' partial rows summed in slot order (bf16)
//   6. dec_uproj   out = z U^T (+ x)
//
// Matrix-core tiles are v_mfma_f32_16x16x32_bf16 with weight rows as the M
// operand (16 rows) and tokens as the N operand (16 columns, T used; the rest
// repeat token T - 1 and are never stored, so no operand load is
// conditional). Lane l serves weight row l%16; its lane group g = l/16 takes
// every fourth chunk of the wave's K range (chunk c*4 + g at step c), so one
// load instruction reads 64 contiguous bytes of each of 16 rows. K order
// inside a dot product is free; the token operand is read with the same
// chunk mapping.
//
// Every gate/up workgroup repeats the top-k (some hundreds of dependent
// instructions per token, on one wave per token) instead of one workgroup
// of the router launch taking it after an in-launch hand-off (logits
// stores, an arrival count, the last arriver's gather): measured, the
// repeated top-k costs gate/up about what the hand-off and tail cost the
// router at T = 4, and less at T = 1..3 (1.5 to 3.7 us per step).
//
// Data moves between workgroups only across kernel boundaries.
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
constexpr int kDownRows = kDecodeDownRows;
static_assert(kDownRows == kDecWaves * 16, "one 16-row tile per wave");

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

// Dynamic LDS layouts (bytes), sized by the call's T.
constexpr size_t kRedBytes = kDecWaves * 64 * 4 * sizeof(float);
inline size_t dproj_lds(int T, int H) { return (size_t)T * H * 2 + kRedBytes + kDecodeMaxT * 4; }
inline size_t router_lds(int T, int L) { return (size_t)2 * T * L * 2 + kRedBytes; }
inline size_t gateup_lds(int T, int L) { return (size_t)T * L * 2 + kRedBytes; }
inline size_t down_lds(int T, int I) { return (size_t)T * I * 2; }
inline size_t uproj_lds(int T, int L) { return (size_t)T * L * 2 + kRedBytes; }

// ------------------------------------------------------------------ 1. D

template <int NCH>
__global__ __launch_bounds__(kDecThreads) void k_dec_dproj(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int H = a.hidden, L = a.latent, T = a.T;
  uint16_t* xs = lds;                       // [T][H] bf16
  float* red = (float*)(lds + T * H);       // [8][64][4]
  float* rstd = red + kDecWaves * 64 * 4;   // [T]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, t = lane & 15;
  const int row0 = blockIdx.x * 16;
  const int kb = wave * (H / kDecWaves);
  if (a.topk_in_router && blockIdx.x == 0 && tid == 0) *a.route_counter = 0u;
  RowStage<(NCH + 1) / 2> xr;  // T x hidden, hidden = 256 NCH
  xr.load(a.x, T * H);
  Bf16Rows<NCH> wr;
  int step;
  const uint16_t* wb = bf16_lane(a.D, a.packed, L, H, row0, kb, &step);
  wr.load(wb, step);
  xr.store(xs, T * H);
  __syncthreads();
  if (a.norm_weight) {  // residual block: RMSNorm per token in fp32, then bf16, in place
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
  }
  __syncthreads();
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  wr.mma(xs + min(t, T - 1) * H, kb, g, acc);  // token columns >= T are not stored
  const f32x4 tot = reduce_waves(acc, red);
  if (wave == 0 && t < T) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = row0 + g * 4 + r;
      if (n < L) {
        const uint16_t hi = f32_to_bf16_bits(tot[r]);
        a.hhi[(size_t)t * L + n] = hi;
        a.hlo[(size_t)t * L + n] = f32_to_bf16_bits(tot[r] - bf16_bits_to_f32(hi));
      }
    }
  }
}

// ------------------------------------------------------------------ 2. router + shared gate/up

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

// Gate/up of one expert for two 16-row tiles per workgroup: wave w handles
// tile w/4, matrix (w/2)%2 (gate, up), K half w%2. The halves and matrices
// meet in LDS; waves 0 and 4 apply SiLU*mul and store.
template <int NCH_H, int BITS>
struct GateUpTask {
  Fp4Rows<NCH_H, BITS> wr;
  __device__ __forceinline__ void load(const Fp4Mat& gate, const Fp4Mat& up, bool packed, int e,
                                       int I, int L, int n0, int wave, int lane) {
    const int mat = (wave >> 1) & 1, half = wave & 1;
    (void)lane;
    wr.load(fp4_lane(mat ? up : gate, packed, e, I, L, n0, half * (L / 2), BITS));
  }
  __device__ __forceinline__ f32x4 mma(const uint16_t* act, int L, int wave, int lane) const {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    wr.mma(act, (wave & 1) * (L / 2), lane >> 4, acc);
    return acc;
  }
};

// Writes this wave's tile, then (waves 0 and 4) combines the four partial
// tiles of its row tile: gate = half0 + half1, up = half0 + half1.
__device__ __forceinline__ void finish_gateup(f32x4 acc, float* red, bool tile_busy, float gsg,
                                              float gsu, uint16_t* act, int I, int T, int n0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  *(f32x4*)(red + (wave * 64 + lane) * 4) = acc;
  __syncthreads();
  if ((wave & 3) == 0 && tile_busy) {
    const f32x4 g0 = *(const f32x4*)(red + ((wave + 0) * 64 + lane) * 4);
    const f32x4 g1 = *(const f32x4*)(red + ((wave + 1) * 64 + lane) * 4);
    const f32x4 u0 = *(const f32x4*)(red + ((wave + 2) * 64 + lane) * 4);
    const f32x4 u1 = *(const f32x4*)(red + ((wave + 3) * 64 + lane) * 4);
    store_gateup(g0 + g1, u0 + u1, gsg, gsu, act, I, T, n0, lane);
  }
}

// ------------------------------------------------------------------ top-k

// One token's logits as order-preserving keys, lane l holding experts
// l, l + 64, ... (experts past E: key 0, below every logit's key). The loads
// are unconditional (clamped index) so that they stay in flight together.
// in_launch: the logits were written by other workgroups of this launch
// (agent-scope loads); else by an earlier launch.
template <int EPL>
__device__ __forceinline__ void wave_load_keys(const float* row, int E, float (&v)[EPL],
                                               bool in_launch = false) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    v[i] = in_launch ? __hip_atomic_load(row + min(lane + 64 * i, E - 1), __ATOMIC_RELAXED, AGENT)
                     : row[min(lane + 64 * i, E - 1)];
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
      a.dbg_logits[i] = __hip_atomic_load(a.logits + i, __ATOMIC_RELAXED, AGENT);
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

template <int NCH_R, int NCH_H, int BITS>
__global__ __launch_bounds__(kDecThreads) void k_dec_router(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  __shared__ RouteLds rl;
  __shared__ unsigned last_flag;
  const int L = a.latent, T = a.T, E = a.n_experts, I = a.inter;
  uint16_t* hi = lds;           // [T][L]
  uint16_t* lo = lds + T * L;   // [T][L]
  float* red = (float*)(lo + T * L);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, t = lane & 15;
  const int nrb = (E + 15) / 16;

  if ((int)blockIdx.x < nrb) {
    const int e0 = blockIdx.x * 16;
    const int kb = wave * (L / kDecWaves);
    RowStage<(NCH_R + 1) / 2> sh_hi, sh_lo;  // T x latent, latent = 256 NCH_R
    // latent rows staged (and waited for) before the router rows are loaded,
    // as in the routed gate/up kernel (measured: 0.6 us less per decode step)
    sh_hi.load(a.hhi, T * L);
    sh_lo.load(a.hlo, T * L);
    sh_hi.store(hi, T * L);
    sh_lo.store(lo, T * L);
    __syncthreads();
    Bf16Rows<NCH_R> wr;
    int step;
    const uint16_t* wb = bf16_lane(a.R, a.packed, E, L, e0, kb, &step);
    wr.load(wb, step);
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
        if (ee < E)
          __hip_atomic_store(a.logits + (size_t)t * E + ee, tot[r] + bias[r], __ATOMIC_RELAXED,
                             AGENT);
      }
    }
    if (!a.topk_in_router) return;  // the gate/up workgroups take the top-k
    // Hand-off: every thread's logits stores are released at agent scope
    // before the workgroup's arrival is counted (release fence, barrier,
    // acquire-release increment); the last arriver acquires at agent scope
    // before it reads any workgroup's logits.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (tid == 0)
      last_flag = __hip_atomic_fetch_add(a.route_counter, 1u, __ATOMIC_ACQ_REL, AGENT) ==
                  (unsigned)(nrb - 1);
    __syncthreads();
    if (!last_flag) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    // the last router workgroup: top-k of every token, then the routing table
    for (int i = tid; i < kMaxExperts / 32; i += kDecThreads) rl.flags[i] = 0u;
    const float* lrow = a.logits + (size_t)min(wave, T - 1) * E;
    if (E <= 512) {
      float v[8];
      wave_load_keys<8>(lrow, E, v, true);
      if (wave < T) wave_topk<8>(v, E, a.top_k, rl.idx + wave * a.top_k, rl.w + wave * a.top_k);
    } else {
      float v[16];
      wave_load_keys<16>(lrow, E, v, true);
      if (wave < T) wave_topk<16>(v, E, a.top_k, rl.idx + wave * a.top_k, rl.w + wave * a.top_k);
    }
    __syncthreads();
    build_active_list(E, T * a.top_k, rl);
    publish_routing(a, rl);
    return;
  }
  // shared expert gate/up: two 16-row tiles per workgroup (see GateUpTask)
  if (!a.n_shared) return;
  const int tile = (blockIdx.x - nrb) * 2 + (wave >> 2);
  const bool busy = tile * 16 < I;
  const int n0 = busy ? tile * 16 : 0;
  RowStage<(NCH_H + 1) / 2> st;  // T x latent, latent = 256 NCH_H
  st.load(a.hhi, T * L);
  GateUpTask<NCH_H, BITS> task;
  const float gsg = a.sh_gate.gscale[0], gsu = a.sh_up.gscale[0];
  task.load(a.sh_gate, a.sh_up, a.packed, 0, I, L, n0, wave, lane);  // idle tiles: rows 0..15
  st.store(hi, T * L);
  __syncthreads();
  const f32x4 acc = task.mma(hi + min(t, T - 1) * L, L, wave, lane);
  finish_gateup(acc, red, busy, gsg, gsu, a.act, I, T, n0);
}

// ------------------------------------------------------------------ 3. routed gate/up

// The wave's tile of a routed gate/up workgroup: expert e (active slot
// `slot`), rows n0 .. n0+15, with the token rows staged in `hi`. An idle tile
// (busy false) reads expert 0's rows 0..15 (in range) and stores nothing,
// which keeps the loads and their uses in one block.
template <int NCH_H, int BITS>
__device__ __forceinline__ void gateup_tiles(const DecodeArgs& a, const uint16_t* hi, float* red,
                                             bool busy, int e, int slot, int n0) {
  const int L = a.latent, T = a.T, I = a.inter;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, t = lane & 15;
  GateUpTask<NCH_H, BITS> task;
  const float gsg = a.gate.gscale[e], gsu = a.up.gscale[e];
  task.load(a.gate, a.up, a.packed, e, I, L, n0, wave, lane);
  issue_fence();
  const f32x4 acc = task.mma(hi + min(t, T - 1) * L, L, wave, lane);
  finish_gateup(acc, red, busy, gsg, gsu, a.act + (size_t)(1 + slot) * T * I, I, T, n0);
}

// TOPK: this workgroup takes the top-k itself (a.topk_in_router is false);
// else it reads the routing table the router published.
template <int NCH_H, int BITS, bool TOPK>
__global__ __launch_bounds__(kDecThreads) void k_dec_gateup(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  __shared__ RouteLds rl;
  const int L = a.latent, T = a.T, I = a.inter, E = a.n_experts;
  uint16_t* hi = lds;  // [T][L]
  float* red = (float*)(lds + T * L);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = lane & 15;
  const int tiles = I / 16;
  const int tile = blockIdx.x * 2 + (wave >> 2);  // (slot - 1) * tiles + row tile
  // The activations are staged, and waited for, before any weight load is
  // issued. Four workgroups share a CU and all of them stream weights at
  // once, so activations loaded behind the weights arrive only when most of
  // the CU's weights have; every workgroup's compute would then start after
  // the data window instead of riding on it (measured: 60.3 -> 58.2 us per
  // decode step at T = 4). They go straight into LDS, so no registers hold
  // them while the routing is worked out.
  constexpr int NV = (NCH_H + 1) / 2;  // T x latent, latent = 256 NCH_H: up to 8 rows
  if constexpr (!TOPK) {  // the routing table is published: read it
    const int n_act = a.route_n_act[0];
    const int e_guess = a.route_list[min(tile / tiles, a.max_active - 1)];
    if ((int)blockIdx.x * 2 >= n_act * tiles) return;  // both tiles idle (uniform)
    stage_dma<NV>(a.hhi, T * L, hi);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's rows have landed in LDS
    __syncthreads();
    const bool busy = tile < n_act * tiles;
    gateup_tiles<NCH_H, BITS>(a, hi, red, busy, busy ? e_guess : 0, busy ? tile / tiles : 0,
                              busy ? (tile % tiles) * 16 : 0);
  } else {
    // every workgroup takes the top-k of every token from the router's
    // logits, loaded together with the staged rows (one round trip), and
    // builds the active list (the same result in each); workgroup 0
    // publishes the routing table for the down and combine kernels
    for (int i = tid; i < kMaxExperts / 32; i += kDecThreads) rl.flags[i] = 0u;
    const float* lrow = a.logits + (size_t)min(wave, T - 1) * E;
    if (E <= 512) {
      float v[8];
      wave_load_keys<8>(lrow, E, v);
      stage_dma<NV>(a.hhi, T * L, hi);
      if (wave < T) wave_topk<8>(v, E, a.top_k, rl.idx + wave * a.top_k, rl.w + wave * a.top_k);
    } else {
      float v[16];
      wave_load_keys<16>(lrow, E, v);
      stage_dma<NV>(a.hhi, T * L, hi);
      if (wave < T) wave_topk<16>(v, E, a.top_k, rl.idx + wave * a.top_k, rl.w + wave * a.top_k);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's rows have landed in LDS
    __syncthreads();
    build_active_list(E, T * a.top_k, rl);
    if (blockIdx.x == 0) publish_routing(a, rl);
    const int n_act = rl.n_act;
    if ((int)blockIdx.x * 2 >= n_act * tiles) return;  // both tiles idle (uniform)
    const bool busy = tile < n_act * tiles;
    gateup_tiles<NCH_H, BITS>(a, hi, red, busy, busy ? rl.list[tile / tiles] : 0,
                              busy ? tile / tiles : 0, busy ? (tile % tiles) * 16 : 0);
  }
}

// ------------------------------------------------------------------ 4. down + combine

template <int NCH_D>
__global__ __launch_bounds__(kDecThreads) void k_dec_down(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];  // [T][I] activations
  const int L = a.latent, T = a.T, I = a.inter;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, t = lane & 15;
  (void)tid;
  const int nrr = decode_row_ranges(L);
  const int s = blockIdx.x / nrr, rr = blockIdx.x % nrr;
  // the routing table, read together (the guesses are clamped in range)
  const int n_act = a.route_n_act[0];
  const int e_guess = a.route_list[min(max(s - 1, 0), a.max_active - 1)];
  const float w_guess = a.route_wtab[min(s, a.max_active) * T + min(t, T - 1)];
  const bool sh = s == 0;
  if (sh ? a.n_shared == 0 : s > n_act) return;  // uniform over the workgroup
  const int e = sh ? 0 : e_guess;
  const Fp4Mat& dm = sh ? a.sh_down : a.down;
  const float* gscale = dm.gscale;
  RowStage<(NCH_D + 3) / 4> st;  // T x inter, inter = 128 NCH_D
  st.load(a.act + (size_t)s * T * I, T * I);
  const int row0 = rr * kDownRows + wave * 16;
  Fp4Rows<NCH_D> wd;
  const float gs = gscale[e];
  wd.load(fp4_lane(dm, a.packed, e, L, I, row0, 0));
  st.store(lds, T * I);
  __syncthreads();
  f32x4 y = {0.f, 0.f, 0.f, 0.f};
  wd.mma(lds + min(t, T - 1) * I, 0, g, y);
  if (t < T) {
    const float wt = w_guess * gs;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = row0 + g * 4 + r;
      if (n < L) a.zpart[((size_t)s * T + t) * L + n] = wt * y[r];
    }
  }
}

// z[t][n] = bf16(sum over the active slots, in slot order, of the weighted
// partial rows); one thread per output. Its own launch: the kernel boundary
// makes every down workgroup's partial rows visible, which costs less than a
// release, an arrival count and a last-arriver sum inside the down launch
// (measured: 6.5 us of hand-off there against one extra launch here).
// The loads cover every slot of the table's capacity (1 + max_active rows,
// all in range), NB at a time, so none of them waits for the active count,
// which decides only what is summed. Up to 60 rows (T <= 5 at top-10) the
// batch stays below the 64 loads a wave can count in flight; past that one
// batch of 96, which the compiler splits with waits, still measured faster
// than two batches (T = 8: 63.5 -> 63.0 us per step).
template <int NB>
__global__ __launch_bounds__(256) void k_dec_combine(DecodeArgs a) {
  const int T = a.T, L = a.latent;
  const int i = blockIdx.x * 256 + threadIdx.x;  // t * L + n
  if (i >= T * L) return;
  const int n_act = a.route_n_act[0];
  const int s0 = a.n_shared ? 0 : 1;
  const int last = a.max_active;  // highest slot of the table
  const size_t step = (size_t)T * L;
  const float* src = a.zpart + i;
  float v = 0.f;
  for (int ss = s0; ss <= last; ss += NB) {
    float p[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) p[j] = src[min(ss + j, last) * step];
    issue_fence();  // else the first sums are placed between the loads, each a round trip
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (ss + j <= n_act) v += p[j];
  }
  a.z[i] = f32_to_bf16_bits(v);
}

// ------------------------------------------------------------------ 5. U

template <int NCH>
__global__ __launch_bounds__(kDecThreads) void k_dec_uproj(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int L = a.latent, H = a.hidden, T = a.T;
  uint16_t* zs = lds;  // [T][L] bf16
  float* red = (float*)(lds + T * L);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, t = lane & 15;
  const int m0 = blockIdx.x * 16;
  const int kb = wave * (L / kDecWaves);
  RowStage<(NCH + 1) / 2> st;  // T x latent, latent = 256 NCH
  st.load(a.z, T * L);
  Bf16Rows<NCH> wr;
  int step;
  const uint16_t* wb = bf16_lane(a.U, a.packed, H, L, m0, kb, &step);
  wr.load(wb, step);
  st.store(zs, T * L);
  __syncthreads();
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  wr.mma(zs + min(t, T - 1) * L, kb, g, acc);
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

bool decode_supported(int hidden, int latent, int inter, int n_experts, int top_k, int T) {
  if (T < 1 || T > kDecodeMaxT || n_experts > kMaxExperts || top_k > 16) return false;
  // D, U and the router split K over 8 waves x 4 lane groups x 8 bf16;
  // expert rows are consumed in 32-weight chunks by 4 lane groups.
  if (hidden % 256 || latent % 256 || inter % 128) return false;
  if (!nch_ok(hidden / 256) || !nch_ok(latent / 256) || !nch_ok(inter / 128)) return false;
  if (latent / 128 > 14) return false;  // register budget of the gate/up waves
  // (activation staging is sized per kernel from the same chunk counts:
  // RowStage<ceil(width / 512)> holds 8 rows of `width`)
  const size_t lim = 96 * 1024;
  return dproj_lds(kDecodeMaxT, hidden) <= lim && router_lds(kDecodeMaxT, latent) <= lim &&
         router_lds(kDecodeMaxT, latent) + sizeof(RouteLds) <= lim &&
         gateup_lds(kDecodeMaxT, latent) <= lim &&
         down_lds(kDecodeMaxT, inter) <= lim && uproj_lds(kDecodeMaxT, latent) <= lim;
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

// Workgroups of a gate/up instantiation resident on the device at once (its
// occupancy at the largest LDS size times the CU count), once per device.
static int gateup_resident(const void* fn, size_t lds) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  const auto it = cache.find({fn, dev});
  if (it != cache.end()) return it->second;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kDecThreads, lds) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return cache[{fn, dev}] = per_cu * cus;
}

hipError_t launch_decode(const DecodeArgs& args, hipStream_t st, const StageMarks& mk) {
  DecodeArgs a = args;
  const int H = a.hidden, L = a.latent, I = a.inter, E = a.n_experts, T = a.T;
  const dim3 block(kDecThreads);
  hipError_t err;
  // Top-k placement: in every gate/up workgroup when the gate/up grid is
  // resident in one round (then it overlaps the staging and costs each
  // workgroup once), else in the router's last workgroup (a second round
  // of gate/up workgroups would pay it again).
  {
    int resident = 0;
    err = with_nch(L / 256, [&](auto N) {
      constexpr int n = decltype(N)::value;
      const void* fn = a.gateup_bits == 3 ? (const void*)k_dec_gateup<n, 3, true>
                                          : (const void*)k_dec_gateup<n, 4, true>;
      hipError_t e = ensure_lds(fn, gateup_lds(kDecodeMaxT, L));
      if (e == hipSuccess) resident = gateup_resident(fn, gateup_lds(kDecodeMaxT, L));
      return e;
    });
    if (err != hipSuccess) return err;
    a.topk_in_router = (a.max_active * (I / 16) + 1) / 2 > resident;
  }
  // 1. h = x D^T
  err = with_nch(H / 256, [&](auto N) {
    constexpr int n = decltype(N)::value;
    hipError_t e = ensure_lds((const void*)k_dec_dproj<n>, dproj_lds(kDecodeMaxT, H));
    if (e == hipSuccess)
      e = mk.launch(kStageDproj, k_dec_dproj<n>, dim3((L + 15) / 16), block, dproj_lds(T, H), a);
    return e;
  });
  if (err != hipSuccess) return err;
  // 2. router logits + top-k + routing table, shared expert gate/up
  const auto router = [&](auto N, auto B) {
    constexpr int n = decltype(N)::value, bits = decltype(B)::value;
    const int nrb = (E + 15) / 16;
    const int nsh = a.n_shared ? (I / 16 + 1) / 2 : 0;
    const auto fn = k_dec_router<n, n, bits>;
    hipError_t e = ensure_lds((const void*)fn, router_lds(kDecodeMaxT, L));
    if (e == hipSuccess)
      e = mk.launch(kStageRouter, fn, dim3(nrb + nsh), block, router_lds(T, L), a);
    return e;
  };
  err = with_nch(L / 256, [&](auto N) {
    return a.gateup_bits == 3 ? router(N, std::integral_constant<int, 3>{})
                              : router(N, std::integral_constant<int, 4>{});
  });
  if (err != hipSuccess) return err;
  // 3. routed gate/up
  const auto gateup = [&](auto N, auto B) {
    constexpr int n = decltype(N)::value, bits = decltype(B)::value;
    const int nblk = (a.max_active * (I / 16) + 1) / 2;
    const auto fn = a.topk_in_router ? k_dec_gateup<n, bits, false> : k_dec_gateup<n, bits, true>;
    hipError_t e = ensure_lds((const void*)fn, gateup_lds(kDecodeMaxT, L));
    if (e == hipSuccess) e = mk.launch(kStageGateup, fn, dim3(nblk), block, gateup_lds(T, L), a);
    return e;
  };
  err = with_nch(L / 256, [&](auto N) {
    return a.gateup_bits == 3 ? gateup(N, std::integral_constant<int, 3>{})
                              : gateup(N, std::integral_constant<int, 4>{});
  });
  if (err != hipSuccess) return err;
  // 4. down + combine
  err = with_nch(I / 128, [&](auto N) {
    constexpr int n = decltype(N)::value;
    hipError_t e = ensure_lds((const void*)k_dec_down<n>, down_lds(kDecodeMaxT, I));
    if (e == hipSuccess)
      e = mk.launch_first(kStageDown, k_dec_down<n>,
                          dim3((1 + a.max_active) * decode_row_ranges(L)), block, down_lds(T, I), a);
    return e;
  });
  if (err != hipSuccess) return err;
  {
    const int n_rows = a.max_active + (a.n_shared ? 1 : 0);  // slots the combine reads
    const dim3 cg((T * L + 255) / 256), cb(256);
    err = n_rows <= 16   ? mk.launch_last(kStageDown, k_dec_combine<16>, cg, cb, 0, a)
          : n_rows <= 32 ? mk.launch_last(kStageDown, k_dec_combine<32>, cg, cb, 0, a)
          : n_rows <= 48 ? mk.launch_last(kStageDown, k_dec_combine<48>, cg, cb, 0, a)
          : n_rows <= 60 ? mk.launch_last(kStageDown, k_dec_combine<60>, cg, cb, 0, a)
                         : mk.launch_last(kStageDown, k_dec_combine<96>, cg, cb, 0, a);
  }
  if (err != hipSuccess) return err;
  // 5. out = z U^T (+ x)
  return with_nch(L / 256, [&](auto N) {
    constexpr int n = decltype(N)::value;
    hipError_t e = ensure_lds((const void*)k_dec_uproj<n>, uproj_lds(kDecodeMaxT, L));
    if (e == hipSuccess)
      e = mk.launch(kStageUproj, k_dec_uproj<n>, dim3((H + 15) / 16), block, uproj_lds(T, L), a);
    return e;
  });
}

}  // namespace moe
