// Tiled bf16 matrix-core GEMMs of the latent-MoE layer (gfx950).
//
//   dense:   C[M][N] = A[M][K] . B[N][K]^T     (D down-projection, router, U up-projection)
//   grouped: per expert e, rows of A routed to e times dequant(W_e)^T with
//            W_e in e2m1 codes + E4M3 per-16 block scales (gate/up fused with
//            SiLU*mul, then down).
//
// One 256-thread workgroup computes a 128x128 tile; its four waves each own a
// 64x64 sub-tile made of 2x2 v_mfma_f32_32x32x16_bf16 products. A and B
// tiles are staged through LDS (rows padded by 16 bytes so the 16-byte
// fragment reads of a half-wave hit distinct banks), double-buffered with
// register prefetch: the global loads of step k+1 are in flight while the
// matrix cores work on step k. Expert weights arrive as 4-bit codes and are
// dequantised in registers (exactly, to bf16) on their way into LDS, so the
// HBM traffic for weights is the 4.5-bit format, not bf16.
//
// Grids are one-dimensional over (m-tile, n-tile) with n fastest, and the
// block id is permuted so that the workgroups the hardware places on one XCD
// (consecutive ids go to the 8 XCDs in turn) take a contiguous range of
// tiles: the n-tiles of one m-tile then run together on one XCD and share its
// A rows through that XCD's L2 instead of fetching them once per n-tile.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kTile = 128;
constexpr int kThreads = 256;
constexpr int kXcds = 8;

// Logical tile of workgroup b among n: XCD x = b % 8 takes the contiguous
// range [x*q + min(x, r), ...) of q or q+1 tiles (q = n / 8, r = n % 8).
__device__ __forceinline__ int xcd_tile(int b, int n) {
  const int x = b % kXcds, q = n / kXcds, r = n % kXcds;
  return x * q + min(x, r) + b / kXcds;
}

template <int BK>
struct TileShape {
  static constexpr int kStride = BK + 8;              // bf16 per LDS row
  static constexpr int kElems = kTile * kStride;      // bf16 per tile
  static constexpr int kChunksPerRow = BK / 8;        // 16-byte chunks per row
  static constexpr int kChunksPerThread = kTile * kChunksPerRow / kThreads;
};

// 128 rows of bf16, row r starting at ptr_r; column index wraps modulo
// `kwrap` (a multiple of BK) so one physical matrix can stand for two
// concatenated copies along K.
template <int BK>
struct RowLoader {
  static constexpr int CPT = TileShape<BK>::kChunksPerThread;
  const uint16_t* ptr[CPT];
  int lds_off[CPT];
  uint4 reg[CPT];
  int kwrap;

  template <class RowFn>
  __device__ __forceinline__ void init(RowFn rowfn, int kwrap_) {
    kwrap = kwrap_;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = threadIdx.x + kThreads * i;
      const int row = c / TileShape<BK>::kChunksPerRow;
      const int col8 = c % TileShape<BK>::kChunksPerRow;
      ptr[i] = rowfn(row) + col8 * 8;
      lds_off[i] = row * TileShape<BK>::kStride + col8 * 8;
    }
  }
  __device__ __forceinline__ void load(int kt) {
    int kc = kt * BK;
    if (kc >= kwrap) kc -= kwrap;
#pragma unroll
    for (int i = 0; i < CPT; ++i) reg[i] = *(const uint4*)(ptr[i] + kc);
  }
  __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
    for (int i = 0; i < CPT; ++i) *(uint4*)(lds + lds_off[i]) = reg[i];
  }
};

// 128 rows of 4-bit codes + E4M3 block scales; each active thread moves 32
// consecutive weights (16 bytes of codes, 2 scale bytes) per K step.
template <int BK>
struct Fp4Loader {
  static constexpr int kParts = BK / 32;
  static constexpr int kActive = kTile * kParts;
  bool active;
  const uint8_t* cptr;
  const uint8_t* sptr;
  int lds_off;
  uint4 creg;
  uint32_t sreg;

  // rowfn(row, &codes_row, &scales_row)
  template <class RowFn>
  __device__ __forceinline__ void init(RowFn rowfn) {
    const int t = threadIdx.x;
    active = t < kActive;
    const int row = active ? t / kParts : 0;
    const int part = active ? t % kParts : 0;
    const uint8_t* c;
    const uint8_t* s;
    rowfn(row, &c, &s);
    cptr = c + part * 16;
    sptr = s + part * 2;
    lds_off = row * TileShape<BK>::kStride + part * 32;
  }
  __device__ __forceinline__ void load(int kt) {
    if (!active) return;
    creg = *(const uint4*)(cptr + kt * (BK / 2));
    sreg = *(const uint16_t*)(sptr + kt * (BK / 16));
  }
  __device__ __forceinline__ void store(uint16_t* lds) const {
    if (!active) return;
    const float s0 = e4m3_to_f32(sreg & 0xFFu);
    const float s1 = e4m3_to_f32((sreg >> 8) & 0xFFu);
    bf16x8* dst = (bf16x8*)(lds + lds_off);
    dst[0] = dequant8(creg.x, s0);
    dst[1] = dequant8(creg.y, s0);
    dst[2] = dequant8(creg.z, s1);
    dst[3] = dequant8(creg.w, s1);
  }
};

// Wave w of the workgroup owns rows [wm*64, wm*64+64) of the tile, wm = w/2.
// Its two B sub-tiles are tile rows brow(wn, j) .. +32 (wn = w%2): adjacent
// 32-row groups for a plain GEMM; for gate/up the tile holds 64 gate rows
// then 64 up rows, and sub-tile j = 0 (gate) and j = 1 (up) cover the same
// 32 output columns so SiLU*mul can pair them in registers.
template <bool GATEUP>
__device__ __forceinline__ int b_subtile_row(int wn, int j) {
  return GATEUP ? (j * 64 + wn * 32) : (wn * 64 + j * 32);
}

template <int BK, bool GATEUP, class AL, class BL>
__device__ __forceinline__ void mainloop(AL& al, BL& bl, int KT, uint16_t* smem,
                                         f32x16 (&acc)[2][2]) {
  using TS = TileShape<BK>;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  uint16_t* As[2] = {smem, smem + 2 * TS::kElems};
  uint16_t* Bs[2] = {smem + TS::kElems, smem + 3 * TS::kElems};
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  al.load(0);
  bl.load(0);
  al.store(As[0]);
  bl.store(Bs[0]);
  __syncthreads();
  const int arow = wm * 64 + (lane & 31);
  const int kof = (lane >> 5) * 8;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) {
      al.load(kt + 1);
      bl.load(kt + 1);
    }
    const uint16_t* A = As[cur];
    const uint16_t* B = Bs[cur];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *(const bf16x8*)(A + (arow + i * 32) * TS::kStride + ks * 16 + kof);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *(const bf16x8*)(B + (b_subtile_row<GATEUP>(wn, j) + (lane & 31)) * TS::kStride +
                                ks * 16 + kof);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < KT) {
      al.store(As[cur ^ 1]);
      bl.store(Bs[cur ^ 1]);
    }
    __syncthreads();
  }
}

// Output coordinates of accumulator (i, j, r) for this lane, relative to the tile.
__device__ __forceinline__ int acc_row(int wm, int i, int r, int lane) {
  return wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}

template <int BK>
constexpr int smem_elems() {
  return 4 * TileShape<BK>::kElems;
}

// ------------------------------------------------------------------ dense

template <int BK, int EPI>
__global__ __launch_bounds__(kThreads) void k_gemm_dense(const uint16_t* __restrict__ A, int lda,
                                                         const uint16_t* __restrict__ B, int ldb,
                                                         int kwrap, int M, int N, int K,
                                                         DenseEpilogue ep) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[smem_elems<BK>()];
  const int nt = (N + kTile - 1) / kTile;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int m0 = (tile / nt) * kTile, n0 = (tile % nt) * kTile;
  RowLoader<BK> al, bl;
  al.init([&](int r) { return A + (size_t)min(m0 + r, M - 1) * lda; }, K);
  bl.init([&](int r) { return B + (size_t)min(n0 + r, N - 1) * ldb; }, kwrap);
  f32x16 acc[2][2];
  mainloop<BK, false>(al, bl, K / BK, smem, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + j * 32 + (lane & 31);
    if (n >= N) continue;
    float bias = 0.0f;
    if (EPI == kEpiLogits && ep.bias) bias = ep.bias[n];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + acc_row(wm, i, r, lane);
        if (m >= M) continue;
        const float v = acc[i][j][r];
        if (EPI == kEpiSplit) {
          // latent vector as bf16 hi + bf16 lo: hi feeds the experts, hi + lo
          // (about 16 significant bits) feeds the router
          uint16_t* o = (uint16_t*)ep.out + (size_t)m * ep.ldo;
          const uint16_t hi = f32_to_bf16_bits(v);
          const float rest = v - bf16_bits_to_f32(hi);
          o[n] = hi;
          o[ep.lo_off + n] = f32_to_bf16_bits(rest);
        } else if (EPI == kEpiLogits) {
          ((float*)ep.out)[(size_t)m * ep.ldo + n] = v + bias;
        } else {  // kEpiOut
          float o = v;
          if (ep.resid) o += bf16_bits_to_f32(ep.resid[(size_t)m * ep.ldr + n]);
          ((uint16_t*)ep.out)[(size_t)m * ep.ldo + n] = f32_to_bf16_bits(o);
        }
      }
  }
}

// ------------------------------------------------------------------ grouped

// Index of the group whose tile range holds global m-tile `mt`:
// the largest g with tile_off[g] <= mt (tile_off has ngroups + 1 entries).
__device__ __forceinline__ int find_group(const int* tile_off, int ngroups, int mt) {
  int lo = 0, hi = ngroups;  // invariant: tile_off[lo] <= mt < tile_off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_off[mid] <= mt) lo = mid; else hi = mid;
  }
  return lo;
}

struct TileWork {
  int group;   // expert index; n_experts = the shared expert
  int rbeg;    // first permuted row of this tile
  int rend;    // end of the group's rows
};

__device__ __forceinline__ bool tile_work(const RouteView& rv, int mt, TileWork* w) {
  const int ngroups = rv.n_experts + rv.n_shared;
  const int total = rv.tile_off[ngroups];
  if (mt >= total) return false;
  const int g = find_group(rv.tile_off, ngroups, mt);
  w->group = g;
  w->rbeg = rv.off[g] + (mt - rv.tile_off[g]) * kTile;
  w->rend = rv.off[g + 1];
  return true;
}

__device__ __forceinline__ const Fp4Set& pick_set(const ExpertsView& ex, int g, int n_experts,
                                                  int* local) {
  if (g < n_experts) {
    *local = g;
    return ex.routed;
  }
  *local = g - n_experts;
  return ex.shared;
}

template <int BK>
__global__ __launch_bounds__(kThreads) void k_expert_gateup(const uint16_t* __restrict__ hcat,
                                                            int ldh, RouteView rv,
                                                            ExpertsView ex, uint16_t* __restrict__ act,
                                                            int inter, int latent) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[smem_elems<BK>()];
  const int nt = (inter + 63) / 64;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  TileWork tw;
  if (!tile_work(rv, tile / nt, &tw)) return;
  const int n0 = (tile % nt) * 64;
  int le;
  const Fp4Set& set = pick_set(ex, tw.group, rv.n_experts, &le);
  const int P = rv.pairs;
  RowLoader<BK> al;
  al.init([&](int r) {
    const int row = min(tw.rbeg + r, tw.rend - 1);
    const int tok = row < P ? rv.perm[row] / rv.top_k : row - P;
    return hcat + (size_t)tok * ldh;
  }, latent);
  Fp4Loader<BK> bl;
  bl.init([&](int r, const uint8_t** c, const uint8_t** s) {
    const bool up = r >= 64;
    const int n = min(n0 + (r & 63), inter - 1);
    const Fp4Mat& m = up ? set.up : set.gate;
    const size_t row = (size_t)le * inter + n;
    *c = m.codes + row * (latent / 2);
    *s = m.scales + row * (latent / 16);
  });
  f32x16 acc[2][2];
  mainloop<BK, true>(al, bl, latent / BK, smem, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n = n0 + wn * 32 + (lane & 31);
  if (n >= inter) return;
  const float gsg = set.gate.gscale[le], gsu = set.up.gscale[le];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = tw.rbeg + acc_row(wm, i, r, lane);
      if (row >= tw.rend) continue;
      const float g = gsg * acc[i][0][r];
      const float u = gsu * acc[i][1][r];
      const float a = g / (1.0f + expf(-g)) * u;
      act[(size_t)row * inter + n] = f32_to_bf16_bits(a);
    }
}

template <int BK>
__global__ __launch_bounds__(kThreads) void k_expert_down(const uint16_t* __restrict__ act,
                                                          RouteView rv, ExpertsView ex,
                                                          uint16_t* __restrict__ y, int inter,
                                                          int latent) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[smem_elems<BK>()];
  const int nt = (latent + kTile - 1) / kTile;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  TileWork tw;
  if (!tile_work(rv, tile / nt, &tw)) return;
  const int n0 = (tile % nt) * kTile;
  int le;
  const Fp4Set& set = pick_set(ex, tw.group, rv.n_experts, &le);
  RowLoader<BK> al;
  al.init([&](int r) { return act + (size_t)min(tw.rbeg + r, tw.rend - 1) * inter; }, inter);
  Fp4Loader<BK> bl;
  bl.init([&](int r, const uint8_t** c, const uint8_t** s) {
    const size_t row = (size_t)le * latent + min(n0 + r, latent - 1);
    *c = set.down.codes + row * (inter / 2);
    *s = set.down.scales + row * (inter / 16);
  });
  f32x16 acc[2][2];
  mainloop<BK, false>(al, bl, inter / BK, smem, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const float gsd = set.down.gscale[le];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + j * 32 + (lane & 31);
    if (n >= latent) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = tw.rbeg + acc_row(wm, i, r, lane);
        if (row >= tw.rend) continue;
        y[(size_t)row * latent + n] = f32_to_bf16_bits(gsd * acc[i][j][r]);
      }
  }
}

// ------------------------------------------------------------------ launchers

static inline int pick_bk(int K, int kwrap) { return (K % 64 == 0 && kwrap % 64 == 0) ? 64 : 32; }

hipError_t launch_gemm_dense(int epi, const uint16_t* A, int lda, const uint16_t* B, int ldb,
                             int kwrap, int M, int N, int K, const DenseEpilogue& ep,
                             hipStream_t stream) {
  dim3 grid(((N + kTile - 1) / kTile) * ((M + kTile - 1) / kTile)), block(kThreads);
  const int bk = pick_bk(K, kwrap);
#define MOE_LAUNCH_DENSE(BKV, EPIV)                                                           \
  hipLaunchKernelGGL((k_gemm_dense<BKV, EPIV>), grid, block, 0, stream, A, lda, B, ldb, kwrap, \
                     M, N, K, ep)
  if (bk == 64) {
    if (epi == kEpiSplit) MOE_LAUNCH_DENSE(64, kEpiSplit);
    else if (epi == kEpiLogits) MOE_LAUNCH_DENSE(64, kEpiLogits);
    else MOE_LAUNCH_DENSE(64, kEpiOut);
  } else {
    if (epi == kEpiSplit) MOE_LAUNCH_DENSE(32, kEpiSplit);
    else if (epi == kEpiLogits) MOE_LAUNCH_DENSE(32, kEpiLogits);
    else MOE_LAUNCH_DENSE(32, kEpiOut);
  }
#undef MOE_LAUNCH_DENSE
  return hipGetLastError();
}

hipError_t launch_expert_gateup(const uint16_t* hcat, int ldh, const RouteView& rv,
                                const ExpertsView& ex, uint16_t* act, int inter, int latent,
                                int max_mtiles, hipStream_t stream) {
  dim3 grid(max_mtiles * ((inter + 63) / 64)), block(kThreads);
  if (latent % 64 == 0)
    hipLaunchKernelGGL(k_expert_gateup<64>, grid, block, 0, stream, hcat, ldh, rv, ex, act, inter,
                       latent);
  else
    hipLaunchKernelGGL(k_expert_gateup<32>, grid, block, 0, stream, hcat, ldh, rv, ex, act, inter,
                       latent);
  return hipGetLastError();
}

hipError_t launch_expert_down(const uint16_t* act, const RouteView& rv, const ExpertsView& ex,
                              uint16_t* y, int inter, int latent, int max_mtiles,
                              hipStream_t stream) {
  dim3 grid(max_mtiles * ((latent + kTile - 1) / kTile)), block(kThreads);
  if (inter % 64 == 0)
    hipLaunchKernelGGL(k_expert_down<64>, grid, block, 0, stream, act, rv, ex, y, inter, latent);
  else
    hipLaunchKernelGGL(k_expert_down<32>, grid, block, 0, stream, act, rv, ex, y, inter, latent);
  return hipGetLastError();
}

}  // namespace moe
