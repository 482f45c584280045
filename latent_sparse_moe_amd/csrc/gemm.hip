// Tiled bf16 matrix-core GEMMs of the latent-MoE layer (gfx950).
//
//   dense:   C[M][N] = A[M][K] . B[N][K]^T     (D down-projection, router, U up-projection)
//   grouped: per expert e, rows of A routed to e times dequant(W_e)^T with
//            W_e in e2m1 codes + E4M3 per-16 block scales (gate/up fused with
//            SiLU*mul, then down).
//
// One 256-thread workgroup computes a 128 x 256 tile: wave w owns all 128
// rows and columns [64w, 64w + 64), as 4 x 2 v_mfma_f32_32x32x16_bf16
// products. The operands take different routes, chosen from measured LDS
// rates on gfx950 (16-byte reads ~200+ B/clk/CU, writes from registers ~64):
//   - A (activation rows, shared by all four waves) is staged through LDS:
//     loaded two K steps ahead straight from global memory into one of three
//     LDS stages (global_load_lds_dwordx4, no registers in between), read as
//     fragments. Rows are BK elements with their 16-byte chunks XOR-swizzled
//     by row pair (measured: a 16-byte read is served 16 lanes at a time over
//     256 bytes of banks), so that the fragment reads of 16 consecutive rows
//     at one chunk are conflict-free; each lane loads the chunk that the
//     swizzle puts in its slot. (Measured against loading A into registers
//     and writing it to LDS one step later: 16K prefill 2.20 -> 2.14 ms.)
//   - B (weights, used by exactly one wave) never touches LDS: each lane
//     loads its own weight row's slice straight into registers, three K
//     steps deep, and for the experts dequantises the 4-bit codes (exactly,
//     to bf16) right before its matrix-core op. HBM and L2 traffic for expert
//     weights is the 4.5-bit format.
// The workgroup meets once per K step at a barrier, after each wave has
// waited for its own A loads of the next step (an explicit count: the
// compiler does not track direct-to-LDS loads across waves); nothing in the
// steady-state loop is conditional, so the compiler's other load waits are
// exact.
// The expert kernels are held to 256 registers per lane so that two
// workgroups share a CU (two waves per SIMD): one wave's LDS, barrier and
// load waits then overlap the other's matrix-core work (measured on the 16K
// prefill shapes: gate/up 1.51 -> 1.11 ms, down 0.93 -> 0.72 ms).
//
// Grids are one-dimensional over (m-tile, n-tile) with n fastest, and the
// block id is permuted so that the workgroups the hardware places on one XCD
// (consecutive ids go to the 8 XCDs in turn) take a contiguous range of
// tiles: the n-tiles of one m-tile then run together on one XCD and share its
// A rows through that XCD's L2 instead of fetching them once per n-tile.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kBM = 128;       // tile rows (tokens)
constexpr int kBN = 256;       // tile columns (weight rows)
constexpr int kThreads = 256;  // four waves
constexpr int kXcds = 8;

// Logical tile of workgroup b among n: XCD x = b % 8 takes the contiguous
// range [x*q + min(x, r), ...) of q or q+1 tiles (q = n / 8, r = n % 8).
__device__ __forceinline__ int xcd_tile(int b, int n) {
  const int x = b % kXcds, q = n / kXcds, r = n % kXcds;
  return x * q + min(x, r) + b / kXcds;
}

template <int BK>
struct Geo {
  static constexpr int kCpr = BK / 8;     // 16-byte chunks per A row
  static constexpr int kRpl = 16 / kCpr;  // A rows per 256 bytes (all 64 banks)
  static constexpr int kSub = BK / 16;   // K = 16 matrix-core steps per K step
};

// Slot (16-byte unit) of logical chunk c of `row` in a swizzled A tile.
template <int BK>
__device__ __forceinline__ int swz(int row, int c) {
  using G = Geo<BK>;
  return row * G::kCpr + (c ^ ((row / G::kRpl) % G::kCpr));
}

// Order of K inside a step. The 32x32x16 product takes its K = 16 as two
// halves of 8, lane l supplying half l / 32. A K step is split the same way
// at the top level: lane half h covers columns [h*BK/2, (h+1)*BK/2) of the
// step and matrix-core step ks takes its 8-column chunk ks. A lane's B
// operand for a whole step is then BK/2 consecutive weights of one row (one
// 16-byte load of 4-bit codes), and its A fragment for (ks, half h) is
// logical chunk h * kSub + ks of the row. The order of the products within
// an fp32 accumulation differs from plain K order; the set of products
// does not.

// 128 rows of bf16 A into a swizzled [128][BK] LDS tile, straight from
// global memory (global_load_lds_dwordx4: lane L of a wave writes its 16
// bytes at the wave's LDS base + 16 L). Thread t fills the tile's 16-byte
// slots t, t + 256, ...: it loads the logical chunk that the swizzle puts in
// that slot (the XOR permutation is its own inverse). No registers hold A.
template <int BK>
struct ALoader {
  static constexpr int V = kBM * Geo<BK>::kCpr / kThreads;  // DMA loads per thread and step
  const uint16_t* src[V];
  int wbase;  // this wave's first slot (elements), wave-uniform

  // rowfn(r) = address of row r's K = 0 element
  template <class RowFn>
  __device__ __forceinline__ void init(RowFn rowfn) {
    using G = Geo<BK>;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int slot = v * kThreads + (int)threadIdx.x;
      const int row = slot / G::kCpr, pos = slot % G::kCpr;
      const int c = pos ^ ((row / G::kRpl) % G::kCpr);
      src[v] = rowfn(row) + c * 8;
    }
    wbase = __builtin_amdgcn_readfirstlane((int)(threadIdx.x & ~63)) * 8;
  }
  __device__ __forceinline__ void issue(int kt, uint16_t* tile) const {
#pragma unroll
    for (int v = 0; v < V; ++v)
      __builtin_amdgcn_global_load_lds((const void*)(src[v] + kt * BK),
                                       (__attribute__((address_space(3))) void*)(tile + wbase + v * kThreads * 8),
                                       16, 0, 0);
  }
  // the same loads, unseen by the compiler (see dma_lds16)
  __device__ __forceinline__ void issue_asm(int kt, uint16_t* tile) const {
    const uint32_t base = lds_addr(tile) + (uint32_t)wbase * 2;
#pragma unroll
    for (int v = 0; v < V; ++v)
      dma_lds16(src[v] + kt * BK, __builtin_amdgcn_readfirstlane(base + v * kThreads * 16));
  }
};

// Workgroup barrier after this wave's own direct-to-LDS loads are waited
// for (wait_vmcnt) and its LDS reads have been consumed: no memory fence, so
// the compiler adds no wait for the loads still in flight.
__device__ __forceinline__ void dma_barrier() { __builtin_amdgcn_s_barrier(); }

// B operand in registers: expert weights in e2m1 codes + E4M3 block scales.
// Lane (half h) of sub-tile j holds BK/2 codes and BK/32 scale bytes of its
// weight row per step. The weights are either in the plain row-major layout
// (a lane's bytes of one step are 16 of its row's 32; a load instruction
// touches 32 rows) or packed (PK, BK = 64 only; see launch_pack_fp4): the 64
// lanes' bytes of one step are contiguous, 1 KB of codes and 128 bytes of
// scales per load instruction. The values loaded are the same.
//
// BITS = 3 reads 3-bit E1M1 codes (BK = 64): a lane's 32 weights of a step
// are one 12-byte chunk (three words of e2m1-shaped nibbles, see
// e1m1_group_to_e2m1), widened right before the dequantisation.
template <int BK, bool PK, int BITS = 4>
struct Fp4B {
  static_assert(!PK || BK == 64, "the packed layout has 64-wide K steps");
  static_assert(BITS == 4 || (BITS == 3 && BK == 64), "3-bit codes need 64-wide K steps");
  static constexpr bool kInterleave = false;              // see gemm_step
  static constexpr int kValuPerMfma = 0;
  static constexpr int kLoads = 4;  // load instructions per issue
  static constexpr int kWords = BITS == 4 ? BK / 16 : 3;  // code words per lane per step
  static constexpr int kCodeStep =                        // bytes between a lane's steps
      PK ? 64 * 4 * kWords : (BITS == 4 ? BK / 2 : 24);
  static constexpr int kScaleStep = PK ? 128 : BK / 16;
  struct Set {
    uint32_t c[2][kWords];
    uint32_t s[2];
  };
  const uint8_t* cp[2];
  const uint8_t* sp[2];

  // this lane's code and scale bytes of sub-tile j at step 0
  __device__ __forceinline__ void set(int j, const uint8_t* c, const uint8_t* s) {
    cp[j] = c;
    sp[j] = s;
  }
  __device__ __forceinline__ void issue(int kt, Set& st) const {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (BITS == 3) {
        const uint3 v = *(const uint3*)(cp[j] + kt * kCodeStep);
        st.c[j][0] = v.x; st.c[j][1] = v.y; st.c[j][2] = v.z;
        st.s[j] = *(const uint16_t*)(sp[j] + kt * kScaleStep);
      } else if (BK == 64) {
        const uint4 v = *(const uint4*)(cp[j] + kt * kCodeStep);
        st.c[j][0] = v.x; st.c[j][1] = v.y; st.c[j][2] = v.z; st.c[j][3] = v.w;
        st.s[j] = *(const uint16_t*)(sp[j] + kt * kScaleStep);
      } else {
        const uint2 v = *(const uint2*)(cp[j] + kt * kCodeStep);
        st.c[j][0] = v.x; st.c[j][1] = v.y;
        st.s[j] = *(const uint8_t*)(sp[j] + kt * kScaleStep);
      }
    }
  }
  // chunk ks (8 weights) of sub-tile j; scale block ks / 2 of the lane's half
  __device__ __forceinline__ bf16x8 frag(const Set& st, int j, int ks) const {
    const float sc = e4m3_to_f32((st.s[j] >> (8 * (ks >> 1))) & 0xFFu);
    if (BITS == 3)  // elements 8ks .. 8ks+7 of the chunk
      return dequant8(e1m1_group_to_e2m1(st.c[j][0], st.c[j][1], st.c[j][2], ks), sc);
    return dequant8(st.c[j][ks], sc);
  }
};

// B operand in registers: bf16 weights (dense GEMMs). Column index wraps
// modulo kwrap (a multiple of BK), so one physical matrix can stand for two
// copies concatenated along K. Plain row-major weights (a load instruction
// touches 32 rows) or packed (PK, BK = 64 only; see launch_pack_bf16: the
// 64 lanes' 16 bytes of one load are contiguous). The values are the same.
template <int BK, bool PK>
struct Bf16B {
  static_assert(!PK || BK == 64, "the packed layout has 64-wide K steps");
  static constexpr bool kInterleave = true;  // see gemm_step
  static constexpr int kValuPerMfma = 2;
  static constexpr int kLoads = 2 * Geo<BK>::kSub;  // load instructions per issue
  static constexpr int kSub = Geo<BK>::kSub;
  struct Set {
    uint4 c[2][kSub];
  };
  const uint16_t* p[2];
  int kwrap;

  // this lane's first element of sub-tile j (K = 0)
  __device__ __forceinline__ void set(int j, const uint16_t* q) { p[j] = q; }
  __device__ __forceinline__ void issue(int kt, Set& st) const {
    int kc = kt * BK;
    if (kc >= kwrap) kc -= kwrap;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int ks = 0; ks < kSub; ++ks)
        st.c[j][ks] = PK ? *(const uint4*)(p[j] + kc * 32 + ks * 512)
                         : *(const uint4*)(p[j] + kc + ks * 8);
  }
  __device__ __forceinline__ bf16x8 frag(const Set& st, int j, int ks) const {
    return __builtin_bit_cast(bf16x8, st.c[j][ks]);
  }
};

// The three LDS stages of the A tile, each its own array.
struct Pipe {
  uint16_t* a[3];
};

// One K step on stage S = kt % 3: issue the loads of step kt + 2 (A into LDS
// stage (S+2)%3, read last in step kt - 1, B into B set (S+2)%3), run the
// matrix cores on A stage S and B set S, then wait for step kt + 1's loads
// and meet at the barrier. Past the last step the loads repeat step KT - 1
// into a stage nobody reads (and are waited for before the epilogue). Only
// the first NI 32-row blocks of the tile are multiplied (the last tile of an
// expert's rows may hold fewer than 128).
template <int BK, int S, int NI, class BL>
__device__ __forceinline__ void gemm_step(int kt, int KT, ALoader<BK>& al, const BL& bl,
                                          const Pipe& p, typename BL::Set (&bs)[3],
                                          const int (&frag)[Geo<BK>::kSub],
                                          f32x16 (&acc)[NI][2]) {
  using G = Geo<BK>;
  constexpr int N1 = (S + 1) % 3, N2 = (S + 2) % 3;
  const int kl = min(kt + 2, KT - 1);
  al.issue(kl, p.a[N2]);  // stage N2 was read last in step kt - 1
  bl.issue(kl, bs[N2]);
  const uint16_t* ca = p.a[S];
#pragma unroll
  for (int ks = 0; ks < G::kSub; ++ks) {
    bf16x8 a[NI], b[2];
#pragma unroll
    for (int i = 0; i < NI; ++i) a[i] = *(const bf16x8*)(ca + i * 32 * BK + frag[ks]);
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = bl.frag(bs[S], j, ks);
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(b[j], a[i], acc[i][j]);
  }
  if constexpr (BL::kInterleave) {
    // one matrix-core op, two vector ops and one LDS read at a time
    // (measured on the 16K prefill: D 0.237 -> 0.199 ms, U 0.192 -> 0.174 ms).
    // The expert kernels are left to the scheduler: there the same
    // constraint lifts register pressure past the 256-register budget.
#pragma unroll
    for (int m = 0; m < G::kSub * NI * 2; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, BL::kValuPerMfma, 0);  // VALU
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
  }
  // step kt + 1's A (loaded during step kt - 1) complete in every wave
  // before the barrier: only this step's loads may still be in flight
  wait_vmcnt<ALoader<BK>::V + BL::kLoads>();
  dma_barrier();
}

template <int NI>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[NI][2]) {
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
}

// Accumulates the tile's products into acc (zeroed by the caller).
template <int BK, int NI, class BL>
__device__ __forceinline__ void mainloop(ALoader<BK>& al, const BL& bl, int KT, const Pipe& p,
                                         f32x16 (&acc)[NI][2]) {
  using G = Geo<BK>;
  // this lane's A fragment slot (in elements) for each matrix-core step,
  // relative to the first row of its 32-row block
  const int lane = threadIdx.x & 63;
  int frag[G::kSub];
#pragma unroll
  for (int ks = 0; ks < G::kSub; ++ks)
    frag[ks] = swz<BK>(lane & 31, (lane >> 5) * G::kSub + ks) * 8;

  typename BL::Set bs[3];
  // prologue: step 0 in LDS and B set 0, step 1 in flight
  al.issue(0, p.a[0]);
  bl.issue(0, bs[0]);
  al.issue(min(1, KT - 1), p.a[1]);
  bl.issue(min(1, KT - 1), bs[1]);
  wait_vmcnt<ALoader<BK>::V + BL::kLoads>();
  dma_barrier();
  int kt = 0;
  for (; kt + 3 <= KT; kt += 3) {
    gemm_step<BK, 0, NI>(kt, KT, al, bl, p, bs, frag, acc);
    gemm_step<BK, 1, NI>(kt + 1, KT, al, bl, p, bs, frag, acc);
    gemm_step<BK, 2, NI>(kt + 2, KT, al, bl, p, bs, frag, acc);
  }
  if (kt < KT) gemm_step<BK, 0, NI>(kt, KT, al, bl, p, bs, frag, acc);
  if (kt + 1 < KT) gemm_step<BK, 1, NI>(kt + 1, KT, al, bl, p, bs, frag, acc);
  // the repeated tail loads into LDS land before the workgroup can end (its
  // LDS may then go to the next workgroup on this CU)
  wait_vmcnt<0>();
}

// The dense GEMMs' loop: A three stages deep in LDS as above, the bf16
// weights (B) only one step ahead in two register sets (B set kt % 2, A
// stage kt % 3; unrolled over six steps). Two sets instead of three keep a
// wave within 256 registers, so two workgroups share a CU (two waves per
// SIMD) and one wave's waits overlap the other's matrix-core work; with
// three sets the kernels needed about 284 registers and ran one wave per
// SIMD. Step kt issues B of kt + 1 and then A of kt + 2, computes, and
// waits for all but the newest A loads: B of kt + 1 and A of kt + 1 are
// then complete.
template <int BK, int SA, int SB, int NI, class BL>
__device__ __forceinline__ void dense_step(int kt, int KT, ALoader<BK>& al, const BL& bl,
                                           const Pipe& p, typename BL::Set (&bs)[2],
                                           const int (&frag)[Geo<BK>::kSub],
                                           f32x16 (&acc)[NI][2]) {
  using G = Geo<BK>;
  constexpr int A2 = (SA + 2) % 3, B1 = (SB + 1) % 2;
  bl.issue(min(kt + 1, KT - 1), bs[B1]);  // set B1 was used last in step kt - 1
  __builtin_amdgcn_sched_barrier(0);       // B's loads first, then A's
  al.issue(min(kt + 2, KT - 1), p.a[A2]);  // stage A2 was read last in step kt - 1
  __builtin_amdgcn_sched_barrier(0);
  const uint16_t* ca = p.a[SA];
#pragma unroll
  for (int ks = 0; ks < G::kSub; ++ks) {
    bf16x8 a[NI], b[2];
#pragma unroll
    for (int i = 0; i < NI; ++i) a[i] = *(const bf16x8*)(ca + i * 32 * BK + frag[ks]);
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = bl.frag(bs[SB], j, ks);
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(b[j], a[i], acc[i][j]);
  }
#pragma unroll
  for (int m = 0; m < G::kSub * NI * 2; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, BL::kValuPerMfma, 0);  // VALU
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
  }
  wait_vmcnt<ALoader<BK>::V>();
  dma_barrier();
}

template <int BK, int NI, class BL>
__device__ __forceinline__ void mainloop_dense(ALoader<BK>& al, const BL& bl, int KT, const Pipe& p,
                                               f32x16 (&acc)[NI][2]) {
  using G = Geo<BK>;
  const int lane = threadIdx.x & 63;
  int frag[G::kSub];
#pragma unroll
  for (int ks = 0; ks < G::kSub; ++ks)
    frag[ks] = swz<BK>(lane & 31, (lane >> 5) * G::kSub + ks) * 8;
  typename BL::Set bs[2];
  // prologue: A and B of step 0, A of step 1 in flight
  bl.issue(0, bs[0]);
  al.issue(0, p.a[0]);
  al.issue(min(1, KT - 1), p.a[1]);
  wait_vmcnt<ALoader<BK>::V>();
  dma_barrier();
  int kt = 0;
  for (; kt + 6 <= KT; kt += 6) {
    dense_step<BK, 0, 0, NI>(kt, KT, al, bl, p, bs, frag, acc);
    dense_step<BK, 1, 1, NI>(kt + 1, KT, al, bl, p, bs, frag, acc);
    dense_step<BK, 2, 0, NI>(kt + 2, KT, al, bl, p, bs, frag, acc);
    dense_step<BK, 0, 1, NI>(kt + 3, KT, al, bl, p, bs, frag, acc);
    dense_step<BK, 1, 0, NI>(kt + 4, KT, al, bl, p, bs, frag, acc);
    dense_step<BK, 2, 1, NI>(kt + 5, KT, al, bl, p, bs, frag, acc);
  }
  if (kt < KT) dense_step<BK, 0, 0, NI>(kt, KT, al, bl, p, bs, frag, acc);
  if (kt + 1 < KT) dense_step<BK, 1, 1, NI>(kt + 1, KT, al, bl, p, bs, frag, acc);
  if (kt + 2 < KT) dense_step<BK, 2, 0, NI>(kt + 2, KT, al, bl, p, bs, frag, acc);
  if (kt + 3 < KT) dense_step<BK, 0, 1, NI>(kt + 3, KT, al, bl, p, bs, frag, acc);
  if (kt + 4 < KT) dense_step<BK, 1, 0, NI>(kt + 4, KT, al, bl, p, bs, frag, acc);
  // the repeated tail loads into LDS land before the workgroup can end
  wait_vmcnt<0>();
}

// The products are computed transposed (weights as the first matrix-core
// operand): result register r of lane l belongs to matrix-core row
// m = (r/4)*8 + (l/32)*4 + r%4, i.e. to the weight row loaded by lane m of
// the operand. Lanes do not load weight row m of their 32-row block but row
// weight_row(m), chosen so that registers 8q .. 8q+7 of lane l hold the eight
// consecutive output columns starting at acc_col(q, l) = 16q + 8*(l/32). A
// lane then stores eight outputs (16 bytes of bf16) at once, and the two
// lanes of a token row fill 32 contiguous bytes per store instruction.
__device__ __forceinline__ int weight_row(int m) {
  const int r = (m >> 3) * 4 + (m & 3), h = (m >> 2) & 1;
  return (r >> 3) * 16 + h * 8 + (r & 7);
}
__device__ __forceinline__ int acc_col(int q, int lane) { return q * 16 + (lane >> 5) * 8; }

// Registers 8q .. 8q+7 of an accumulator, each times s, as eight bf16.
__device__ __forceinline__ uint4 pack_bf16x8(const f32x16& c, int q, float s) {
  return uint4{pack_bf16x2(s * c[8 * q], s * c[8 * q + 1]), pack_bf16x2(s * c[8 * q + 2], s * c[8 * q + 3]),
               pack_bf16x2(s * c[8 * q + 4], s * c[8 * q + 5]),
               pack_bf16x2(s * c[8 * q + 6], s * c[8 * q + 7])};
}
__device__ __forceinline__ uint4 pack_bf16x8(const float (&v)[8]) {
  return uint4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
               pack_bf16x2(v[6], v[7])};
}

#define MOE_GEMM_LDS(BK)                                                        \
  __shared__ __attribute__((aligned(16))) uint16_t lds_a0[kBM * BK];            \
  __shared__ __attribute__((aligned(16))) uint16_t lds_a1[kBM * BK];            \
  __shared__ __attribute__((aligned(16))) uint16_t lds_a2[kBM * BK];            \
  const Pipe pipe{{lds_a0, lds_a1, lds_a2}}

// ------------------------------------------------------------------ dense

// TWO: the two-set loop at two waves per SIMD (mainloop_dense), for grids of
// at least two workgroups per CU; else the three-set loop at one wave per
// SIMD (about 284 registers), which prefetches the weights a step further
// and wins when there is only one workgroup per CU anyway (the router: 16K
// tokens x 512 experts is 256 tiles; 10% faster there).
// NI: 32-row blocks per tile (4: 128 x 256 tiles; 2: 64 x 256 tiles for
// small grids, whose A loads still fill the 128-row LDS tile and are half
// used: twice the workgroups for twice the A traffic).
template <int BK, int EPI, bool PK, bool TWO, int NI>
__device__ __forceinline__ void dense_tile(const uint16_t* __restrict__ A, int lda,
                                           const uint16_t* __restrict__ B, int ldb, int kwrap,
                                           int M, int N, int K, const DenseEpilogue& ep) {
  MOE_GEMM_LDS(BK);
  const int nt = (N + kBN - 1) / kBN;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int m0 = (tile / nt) * (32 * NI), n0 = (tile % nt) * kBN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  ALoader<BK> al;
  al.init([&](int r) { return A + (size_t)min(m0 + r, M - 1) * lda; });
  Bf16B<BK, PK> bl;
  bl.kwrap = kwrap;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int nb = n0 + wave * 64 + j * 32;  // first weight row of sub-tile j
    if (PK) {  // block (t, 0) of sub-tile t; N % 32 == 0
      const int t = min(nb, N - 32) / 32;
      bl.set(j, B + (size_t)t * 32 * kwrap + lane * 8);
    } else {   // the lane's row (rows past N read the last one; never stored)
      bl.set(j, B + (size_t)min(nb + weight_row(lane & 31), N - 1) * ldb + (lane >> 5) * (BK / 2));
    }
  }
  f32x16 acc[NI][2];
  zero_acc<NI>(acc);
  if (TWO) mainloop_dense<BK, NI>(al, bl, K / BK, pipe, acc);
  else mainloop<BK, NI>(al, bl, K / BK, pipe, acc);

  const int nbase = n0 + wave * 64;
  // 8-wide stores need the row starts 16-byte aligned
  const bool vec = EPI == kEpiLogits
                       ? (ep.ldo & 3) == 0
                       : (ep.ldo & 7) == 0 && (EPI != kEpiSplit || (ep.lo_off & 7) == 0) &&
                             (EPI != kEpiOut || !ep.resid || (ep.ldr & 7) == 0);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int m = m0 + i * 32 + (lane & 31);
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int n = nbase + j * 32 + acc_col(q, lane);
        if (n >= N) continue;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = acc[i][j][8 * q + e];
        const int nv = min(8, N - n);
        if (EPI == kEpiSplit) {
          // latent vector as bf16 hi + bf16 lo: hi feeds the experts, hi + lo
          // (about 16 significant bits) feeds the router; group g's columns
          // (of group_w, a multiple of 8) go to its own hi | lo block
          uint16_t* o = (uint16_t*)ep.out + (size_t)m * ep.ldo + n + (n / ep.group_w) * ep.group_w;
          float lo[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) lo[e] = v[e] - bf16_bits_to_f32(f32_to_bf16_bits(v[e]));
          if (vec && nv == 8) {
            *(uint4*)o = pack_bf16x8(v);
            *(uint4*)(o + ep.lo_off) = pack_bf16x8(lo);
          } else {
            for (int e = 0; e < nv; ++e) {
              o[e] = f32_to_bf16_bits(v[e]);
              o[ep.lo_off + e] = f32_to_bf16_bits(lo[e]);
            }
          }
        } else if (EPI == kEpiLogits) {
          float* o = (float*)ep.out + (size_t)m * ep.ldo + n;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] += ep.bias && e < nv ? ep.bias[n + e] : 0.0f;
          if (vec && nv == 8) {
            *(float4*)o = float4{v[0], v[1], v[2], v[3]};
            *(float4*)(o + 4) = float4{v[4], v[5], v[6], v[7]};
          } else {
            for (int e = 0; e < nv; ++e) o[e] = v[e];
          }
        } else {  // kEpiOut
          uint16_t* o = (uint16_t*)ep.out + (size_t)m * ep.ldo + n;
          if (ep.resid) {
            const uint16_t* rr = ep.resid + (size_t)m * ep.ldr + n;
            if (vec && nv == 8) {
              const uint4 rv = *(const uint4*)rr;
              const uint32_t d[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                v[2 * e] += bf16_bits_to_f32(d[e] & 0xFFFFu);
                v[2 * e + 1] += bf16_bits_to_f32(d[e] >> 16);
              }
            } else {
              for (int e = 0; e < nv; ++e) v[e] += bf16_bits_to_f32(rr[e]);
            }
          }
          if (vec && nv == 8) *(uint4*)o = pack_bf16x8(v);
          else for (int e = 0; e < nv; ++e) o[e] = f32_to_bf16_bits(v[e]);
        }
      }
  }
}

template <int BK, int EPI, bool PK, int NI = 4>
__global__ __launch_bounds__(kThreads) void k_gemm_dense(const uint16_t* __restrict__ A, int lda,
                                                         const uint16_t* __restrict__ B, int ldb,
                                                         int kwrap, int M, int N, int K,
                                                         DenseEpilogue ep) {
  dense_tile<BK, EPI, PK, false, NI>(A, lda, B, ldb, kwrap, M, N, K, ep);
}

template <int BK, int EPI, bool PK, int NI = 4>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm_dense2(
    const uint16_t* __restrict__ A, int lda, const uint16_t* __restrict__ B, int ldb, int kwrap,
    int M, int N, int K, DenseEpilogue ep) {
  dense_tile<BK, EPI, PK, true, NI>(A, lda, B, ldb, kwrap, M, N, K, ep);
}

// ------------------------------------------------------------------ grouped

struct TileWork {
  int group;   // expert index; n_experts = the shared expert
  int rbeg;    // first permuted row of this tile
  int rend;    // end of the group's rows
};

// m-tile mt of the routing's tile list, which has tile_off[groups] entries.
// The entry is loaded alongside the count (one round trip): grids never
// exceed the list's capacity, and entries past the count are not used.
__device__ __forceinline__ bool tile_work(const RouteView& rv, int mt, TileWork* w) {
  const int4 t = rv.ttab[mt];
  const int total = rv.tile_off[rv.n_experts + rv.n_shared];
  if (mt >= total) return false;
  w->group = t.x;
  w->rbeg = t.y;
  w->rend = t.z;
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

// This lane's code and scale bytes at step 0 for the 32-row sub-tile that
// starts at weight row nb of matrix le of the set m ([count][N][K]); the
// lane's row is nb + weight_row(lane % 32). Sub-tiles past N read the last
// one (their results are not stored).
template <int BK, bool PK, int BITS = 4>
__device__ __forceinline__ void fp4_lane_ptrs(const Fp4Mat& m, int le, int nb, int N, int K,
                                              const uint8_t** c, const uint8_t** s) {
  const int lane = threadIdx.x & 63;
  constexpr int kLaneBytes = BITS == 4 ? 16 : 12;  // a lane's codes of one 64-wide step
  if (PK) {
    const int st = min(nb, N - 32) / 32;
    const size_t blk = ((size_t)le * (N / 32) + st) * (K / 64);
    *c = m.codes + blk * 64 * kLaneBytes + lane * kLaneBytes;
    *s = m.scales + blk * 128 + lane * 2;
  } else {
    const size_t row = (size_t)le * N + min(nb + weight_row(lane & 31), N - 1);
    const int h = lane >> 5;
    *c = m.codes + row * ((size_t)K * BITS / 8) + h * (BITS == 4 ? BK / 4 : 12);
    *s = m.scales + row * (K / 16) + h * (BK / 32);
  }
}

// Packs an fp4 matrix set [count][N][K] (N % 32 == 0, K % 64 == 0) into the
// order the grouped kernels load it in. Block (e, t, kt) = matrix e, rows
// [32t, 32t + 32), columns [64kt, 64kt + 64), blocks in that nesting order.
// Its codes are 64 lanes x 16 bytes: lane L holds the 32 codes of row
// 32t + weight_row(L % 32), columns 64kt + 32(L / 32) .. +32, bytes in the
// plain order. Its scales are 64 lanes x 2 bytes: the two block scales of
// the same 32 columns. One thread moves one lane's 16 + 2 bytes.
// With 3-bit E1M1 codes (BITS = 3) a lane's codes are its 12-byte chunk
// (chunk 2s + L / 32 of the row) at 12 L of a 768-byte block.
template <int BITS>
__global__ __launch_bounds__(256) void k_pack_fp4(const uint8_t* __restrict__ codes,
                                                  const uint8_t* __restrict__ scales,
                                                  int64_t n_lanes, int N, int K,
                                                  uint8_t* __restrict__ pcodes,
                                                  uint8_t* __restrict__ pscales) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_lanes) return;
  const int L = (int)(i & 63);
  const int64_t blk = i >> 6;               // (e * (N / 32) + t) * (K / 64) + kt
  const int kt = (int)(blk % (K / 64));
  const int64_t et = blk / (K / 64);        // e * (N / 32) + t
  const int64_t row = et * 32 + weight_row(L & 31);  // e * N + 32 t + ...
  const int h = L >> 5;
  if (BITS == 4)
    *(uint4*)(pcodes + i * 16) = *(const uint4*)(codes + row * (K / 2) + kt * 32 + h * 16);
  else
    *(uint3*)(pcodes + i * 12) =
        *(const uint3*)(codes + row * ((int64_t)K * 3 / 8) + (2 * kt + h) * 12);
  *(uint16_t*)(pscales + i * 2) = *(const uint16_t*)(scales + row * (K / 16) + kt * 4 + h * 2);
}

// Packs a bf16 matrix [N][K] (N % 32 == 0, K % 64 == 0) into the order the
// dense kernels load it in. Block (t, s) = rows [32t, 32t + 32), columns
// [64s, 64s + 64), blocks in that nesting order, 4 KB each: load ks (0..3)
// of lane L is 16 bytes at 1024 ks + 16 L: row 32t + weight_row(L % 32),
// columns 64s + 32(L / 32) + 8ks .. +8. One thread moves 16 bytes.
__global__ __launch_bounds__(256) void k_pack_bf16(const uint16_t* __restrict__ w, int64_t n_chunks,
                                                   int K, uint16_t* __restrict__ pw) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_chunks) return;
  const int L = (int)(i & 63), ks = (int)((i >> 6) & 3);
  const int64_t blk = i >> 8;  // t * (K / 64) + s
  const int s = (int)(blk % (K / 64));
  const int64_t t = blk / (K / 64);
  const int64_t row = t * 32 + weight_row(L & 31);
  *(uint4*)(pw + i * 8) = *(const uint4*)(w + row * K + s * 64 + (L >> 5) * 32 + ks * 8);
}

hipError_t launch_pack_bf16(const uint16_t* w, int N, int K, uint16_t* pw, hipStream_t stream) {
  const int64_t n_chunks = (int64_t)N * K / 8;
  if (n_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_pack_bf16, dim3((unsigned)((n_chunks + 255) / 256)), dim3(256), 0, stream,
                     w, n_chunks, K, pw);
  return hipGetLastError();
}

hipError_t launch_pack_fp4(const uint8_t* codes, const uint8_t* scales, int count, int N, int K,
                           int bits, uint8_t* pcodes, uint8_t* pscales, hipStream_t stream) {
  const int64_t n_lanes = (int64_t)count * (N / 32) * (K / 64) * 64;
  if (n_lanes == 0) return hipSuccess;
  const dim3 grid((unsigned)((n_lanes + 255) / 256));
  if (bits == 3)
    hipLaunchKernelGGL(k_pack_fp4<3>, grid, dim3(256), 0, stream, codes, scales, n_lanes, N, K,
                       pcodes, pscales);
  else
    hipLaunchKernelGGL(k_pack_fp4<4>, grid, dim3(256), 0, stream, codes, scales, n_lanes, N, K,
                       pcodes, pscales);
  return hipGetLastError();
}

// Blocks of 32 rows holding the tile's rows (1..4). The last tile of an
// expert's rows is usually partial; the one-tile kernels run it with 1, 2 or
// 4 blocks of matrix-core work, the persistent ones with 1, 2, 3 or 4 (at
// the 16K-token routing this cuts the padded rows from 15% to 4%; at 4096
// tokens with uniform routing, about 80 rows per expert, three blocks
// instead of four take a quarter of the work off most tiles). Each count
// has its own copy of the tile body, so nothing stays live across the
// dispatch.
__device__ __forceinline__ int row_blocks(const TileWork& tw) {
  return min(4, (tw.rend - tw.rbeg + 31) / 32);
}

// Gate/up: a tile covers 128 output columns of the SwiGLU width; wave w
// takes columns n0 + 32w .. +32 as sub-tile 0 (gate rows) and sub-tile 1 (up
// rows), so SiLU*mul pairs them in registers.
template <int BK, bool PK, int BITS, int NI>
__device__ __forceinline__ void gateup_tile(const uint16_t* __restrict__ hcat, int ldh,
                                            const RouteView& rv, const ExpertsView& ex,
                                            uint16_t* __restrict__ act, int inter, int latent,
                                            const TileWork& tw, int n0, const Pipe& pipe) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nb = n0 + wave * 32;  // first weight row of this wave's sub-tiles
  int le;
  const Fp4Set& set = pick_set(ex, tw.group, rv.n_experts, &le);
  const int P = rv.pairs;
  ALoader<BK> al;
  al.init([&](int r) {
    const int row = min(tw.rbeg + r, tw.rend - 1);
    const int tok = row < P ? rv.perm[row] / rv.top_k : row - P;
    return hcat + (size_t)tok * ldh;
  });
  Fp4B<BK, PK, BITS> bl;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint8_t *c, *s;
    fp4_lane_ptrs<BK, PK, BITS>(j ? set.up : set.gate, le, nb, inter, latent, &c, &s);
    bl.set(j, c, s);
  }
  f32x16 acc[NI][2];
  zero_acc<NI>(acc);
  mainloop<BK, NI>(al, bl, latent / BK, pipe, acc);

  const float gsg = set.gate.gscale[le], gsu = set.up.gscale[le];
  const int nbase = n0 + wave * 32;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = tw.rbeg + i * 32 + (lane & 31);
    if (row >= tw.rend) continue;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int nc = nbase + acc_col(q, lane);
      if (nc >= inter) continue;  // inter is a multiple of 32: all eight or none
      float a[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float g = gsg * acc[i][0][8 * q + e];
        const float u = gsu * acc[i][1][8 * q + e];
        a[e] = silu_fast(g) * u;
      }
      *(uint4*)(act + (size_t)row * inter + nc) = pack_bf16x8(a);
    }
  }
}

template <int BK, bool PK, int BITS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_expert_gateup(
    const uint16_t* __restrict__ hcat, int ldh, RouteView rv, ExpertsView ex,
    uint16_t* __restrict__ act, int inter, int latent) {
  MOE_GEMM_LDS(BK);
  const int nt = (inter + kBN / 2 - 1) / (kBN / 2);
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  TileWork tw;
  if (!tile_work(rv, tile / nt, &tw)) return;
  const int n0 = (tile % nt) * (kBN / 2);
  const int nb = row_blocks(tw);
  // the latent of the expert's routing group (the shared expert: group 0);
  // added here, ahead of the row-block dispatch, it leaves the tile bodies'
  // register allocation as it is without groups (computed inside them it
  // made the K loop spill)
  hcat += (size_t)(tw.group < rv.n_experts ? tw.group / rv.experts_per_group : 0) * rv.group_stride;
  if (nb == 1) gateup_tile<BK, PK, BITS, 1>(hcat, ldh, rv, ex, act, inter, latent, tw, n0, pipe);
  else if (nb == 2) gateup_tile<BK, PK, BITS, 2>(hcat, ldh, rv, ex, act, inter, latent, tw, n0, pipe);
  else gateup_tile<BK, PK, BITS, 4>(hcat, ldh, rv, ex, act, inter, latent, tw, n0, pipe);
}

template <int BK, bool PK, int NI>
__device__ __forceinline__ void down_tile(const uint16_t* __restrict__ act, const RouteView& rv,
                                          const ExpertsView& ex, uint16_t* __restrict__ y,
                                          int inter, int latent, const TileWork& tw, int n0,
                                          const Pipe& pipe) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nb = n0 + wave * 64;  // first weight row of this wave's sub-tiles
  int le;
  const Fp4Set& set = pick_set(ex, tw.group, rv.n_experts, &le);
  ALoader<BK> al;
  al.init([&](int r) { return act + (size_t)min(tw.rbeg + r, tw.rend - 1) * inter; });
  Fp4B<BK, PK> bl;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint8_t *c, *s;
    fp4_lane_ptrs<BK, PK>(set.down, le, nb + j * 32, latent, inter, &c, &s);
    bl.set(j, c, s);
  }
  f32x16 acc[NI][2];
  zero_acc<NI>(acc);
  mainloop<BK, NI>(al, bl, inter / BK, pipe, acc);

  const float gsd = set.down.gscale[le];
  const int nbase = n0 + wave * 64;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = tw.rbeg + i * 32 + (lane & 31);
    if (row >= tw.rend) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int nc = nbase + j * 32 + acc_col(q, lane);
        if (nc >= latent) continue;  // latent is a multiple of 32: all eight or none
        *(uint4*)(y + (size_t)row * latent + nc) = pack_bf16x8(acc[i][j], q, gsd);
      }
  }
}

template <int BK, bool PK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_expert_down(
    const uint16_t* __restrict__ act, RouteView rv, ExpertsView ex, uint16_t* __restrict__ y,
    int inter, int latent) {
  MOE_GEMM_LDS(BK);
  const int nt = (latent + kBN - 1) / kBN;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  TileWork tw;
  if (!tile_work(rv, tile / nt, &tw)) return;
  const int n0 = (tile % nt) * kBN;
  const int nb = row_blocks(tw);
  if (nb == 1) down_tile<BK, PK, 1>(act, rv, ex, y, inter, latent, tw, n0, pipe);
  else if (nb == 2) down_tile<BK, PK, 2>(act, rv, ex, y, inter, latent, tw, n0, pipe);
  else down_tile<BK, PK, 4>(act, rv, ex, y, inter, latent, tw, n0, pipe);
}

// ------------------------------------------------------------------ grouped, persistent

// The expert GEMMs for K of at least two steps run persistent: two
// workgroups per CU, each walking its share of the tile list (the list is
// cut into eight runs of about equal cost, one per XCD, computed with the
// routing; a workgroup takes every 64th tile of its XCD's run, so the
// n-tiles of an m-tile and the m-tiles of an expert run side by side on one
// XCD and share its L2). Measured on the 128-row kernels with every load and
// the dequantisation taken out, a tile's set-up and epilogue cost as much as
// a third of the time (down, ten K steps per tile, ran at 40 % of the
// matrix cores' rate even so). Here the loads run on across tiles: the last
// two K steps of a tile load the first two of the workgroup's next tile,
// and that tile's rows and weight pointers are set up before the epilogue.
// For that the stages are indexed at run time, so both operands go through
// LDS: three stages, each the A tile (as in the kernels above) and each
// wave's weight codes and scales of the step (direct-to-LDS DMA from the
// lane's own addresses; per sub-tile 64 lanes x 16 bytes of e2m1 codes, or
// three planes of 64 dwords of the 3-bit chunks, and the dword holding each
// lane's two scale bytes). A wave reads its step's codes and scales from
// LDS at the start of the step and dequantises from registers as before.
// Every step issues the same loads (after the last tile the last step is
// loaded again into a stage nobody reads), so the waits are exact counts.

constexpr int kPStages = 3;

template <bool PK, int BITS>
struct PWeights {
  using FB = Fp4B<64, PK, BITS>;
  using Set = typename FB::Set;
  static constexpr int kCodeBytes = BITS == 4 ? 1024 : 768;  // per sub-tile and step
  static constexpr int kSubBytes = kCodeBytes + 256;
  static constexpr int kWaveBytes = 2 * kSubBytes;
  static constexpr int kLoads = BITS == 4 ? 4 : 8;  // DMA instructions per step
  const uint8_t* cp[2];  // this lane's codes of sub-tile j at step 0
  const uint8_t* sp[2];  // the aligned dword holding its scale bytes at step 0
  int shift[2];          // where in that dword they start (bits)

  __device__ __forceinline__ void set(int j, const uint8_t* c, const uint8_t* s) {
    cp[j] = c;
    sp[j] = (const uint8_t*)((uintptr_t)s & ~(uintptr_t)3);
    shift[j] = (int)((uintptr_t)s & 3) * 8;
  }
  // step k's codes and scales into this wave's region of a stage
  __device__ __forceinline__ void issue(int k, uint8_t* wreg) const {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(wreg));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t d = base + j * kSubBytes;
      if (BITS == 4) {
        dma_lds16(cp[j] + (size_t)k * FB::kCodeStep, d);
      } else {
#pragma unroll
        for (int w = 0; w < 3; ++w) dma_lds4(cp[j] + (size_t)k * FB::kCodeStep + 4 * w, d + 256 * w);
      }
      dma_lds4(sp[j] + (size_t)k * FB::kScaleStep, d + kCodeBytes);
    }
  }
  __device__ static __forceinline__ bf16x8 frag(const Set& st, int j, int ks) {
    const FB f{};
    return f.frag(st, j, ks);
  }
  // this lane's codes and scale bytes of the step, from the wave's region
  // (shift: that of the tile the step belongs to)
  __device__ static __forceinline__ void read(const uint8_t* wreg, const int (&shift)[2], Set& st) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint8_t* d = wreg + j * kSubBytes;
      if (BITS == 4) {
        const uint4 v = *(const uint4*)(d + lane * 16);
        st.c[j][0] = v.x; st.c[j][1] = v.y; st.c[j][2] = v.z; st.c[j][3] = v.w;
      } else {
#pragma unroll
        for (int w = 0; w < 3; ++w) st.c[j][w] = *(const uint32_t*)(d + 256 * w + lane * 4);
      }
      st.s[j] = *(const uint32_t*)(d + kCodeBytes + lane * 4) >> shift[j];
    }
  }
};

// Where the loads for two steps ahead come from: the tile being run, then
// (from its second-last step on) the workgroup's next tile.
template <class W>
struct PIssue {
  ALoader<64> a;
  W b;
  int k;  // next step to load
};

template <bool PK, int BITS>
struct PGateUp {
  using W = PWeights<PK, BITS>;
  static constexpr int kTileN = kBN / 2;  // SwiGLU columns per tile
  static constexpr int kSplit = 0;
  static constexpr bool kStagedEpi = false;
  const uint16_t* hcat;
  int ldh;
  RouteView rv;
  ExpertsView ex;
  uint16_t* act;
  int inter, latent;

  __device__ __forceinline__ int n_tiles() const { return (inter + kTileN - 1) / kTileN; }
  __device__ __forceinline__ int k_steps() const { return latent / 64; }
  __device__ __forceinline__ void setup(const TileWork& tw, int n0, ALoader<64>& al, W& bl) const {
    const int wave = threadIdx.x >> 6, P = rv.pairs;
    // the latent of the expert's routing group (the shared expert: group 0)
    const uint16_t* h =
        hcat + (size_t)(tw.group < rv.n_experts ? tw.group / rv.experts_per_group : 0) * rv.group_stride;
    al.init([&](int r) {
      const int row = min(tw.rbeg + r, tw.rend - 1);
      const int tok = row < P ? rv.perm[row] / rv.top_k : row - P;
      return h + (size_t)tok * ldh;
    });
    int le;
    const Fp4Set& set = pick_set(ex, tw.group, rv.n_experts, &le);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint8_t *c, *s;
      fp4_lane_ptrs<64, PK, BITS>(j ? set.up : set.gate, le, n0 + wave * 32, inter, latent, &c, &s);
      bl.set(j, c, s);
    }
  }
  template <int NI>
  __device__ __forceinline__ void epilogue(const TileWork& tw, int n0, const f32x16 (&acc)[NI][2],
                                           uint16_t* /*stage*/) const {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int le;
    const Fp4Set& set = pick_set(ex, tw.group, rv.n_experts, &le);
    const float gsg = set.gate.gscale[le], gsu = set.up.gscale[le];
    const int nbase = n0 + wave * 32;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = tw.rbeg + i * 32 + (lane & 31);
      if (row >= tw.rend) continue;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int nc = nbase + acc_col(q, lane);
        if (nc >= inter) continue;  // inter is a multiple of 32: all eight or none
        float a[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          a[e] = silu_fast(gsg * acc[i][0][8 * q + e]) * (gsu * acc[i][1][8 * q + e]);
        *(uint4*)(act + (size_t)row * inter + nc) = pack_bf16x8(a);
      }
    }
  }
};

template <bool PK>
struct PDown {
  using W = PWeights<PK, 4>;
  static constexpr int kTileN = kBN;
  static constexpr int kSplit = 1;
  static constexpr bool kStagedEpi = true;  // the epilogue writes through LDS (below)
  const uint16_t* act;
  RouteView rv;
  ExpertsView ex;
  uint16_t* y;
  int inter, latent;

  __device__ __forceinline__ int n_tiles() const { return (latent + kTileN - 1) / kTileN; }
  __device__ __forceinline__ int k_steps() const { return inter / 64; }
  __device__ __forceinline__ void setup(const TileWork& tw, int n0, ALoader<64>& al, W& bl) const {
    const int wave = threadIdx.x >> 6;
    al.init([&](int r) { return act + (size_t)min(tw.rbeg + r, tw.rend - 1) * inter; });
    int le;
    const Fp4Set& set = pick_set(ex, tw.group, rv.n_experts, &le);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint8_t *c, *s;
      fp4_lane_ptrs<64, PK>(set.down, le, n0 + wave * 64 + j * 32, latent, inter, &c, &s);
      bl.set(j, c, s);
    }
  }
  // The wave's 128 x 64 outputs go out one 32-row block at a time through
  // its own 4 KB of the LDS stage that no load is filling (stage): the
  // accumulators give a lane 8-column pieces of one row (two lanes share a
  // row), so direct stores would touch 32 rows per instruction; read back
  // by rows, eight lanes cover one row's 128 bytes and a store instruction
  // writes eight whole 128-byte lines. The 16-byte chunks of a row are
  // XOR-swizzled by row. One wave's LDS accesses complete in order, so the
  // region needs no barrier between blocks; the caller holds a workgroup
  // barrier before any load may fill the stage again.
  template <int NI>
  __device__ __forceinline__ void epilogue(const TileWork& tw, int n0, const f32x16 (&acc)[NI][2],
                                           uint16_t* stage) const {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int le;
    const Fp4Set& set = pick_set(ex, tw.group, rv.n_experts, &le);
    const float gsd = set.down.gscale[le];
    const int nbase = n0 + wave * 64;
    uint16_t* st = stage + wave * (32 * 64);  // [32 rows][64 columns] bf16
    const int wr = lane & 31;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int c = 4 * j + 2 * q + (lane >> 5);  // the row's 16-byte chunk (acc_col / 8)
          *(uint4*)(st + wr * 64 + (c ^ (wr & 7)) * 8) = pack_bf16x8(acc[i][j], q, gsd);
        }
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int rr = it * 8 + (lane >> 3), c = lane & 7;
        const uint4 v = *(const uint4*)(st + rr * 64 + (c ^ (rr & 7)) * 8);
        const int row = tw.rbeg + i * 32 + rr, nc = nbase + c * 8;
        // latent is a multiple of 32: a chunk is all in or all out
        if (row < tw.rend && nc < latent) *(uint4*)(y + (size_t)row * latent + nc) = v;
      }
    }
  }
};

// Advances the load stream by one step: past the tile's last step it
// continues with the next tile, or (after the last tile) repeats the last
// step into a stage nobody reads. Written without branches: a join in the
// control flow makes the compiler forget which LDS stages the DMA in
// flight writes, and it then waits for all of it before the next LDS read.
template <class W>
__device__ __forceinline__ void padvance(PIssue<W>& is, int KT, bool has_next, const ALoader<64>& aln,
                                         const W& bln) {
  const bool wrap = ++is.k == KT;
  const bool sw = wrap && has_next;
  is.k = wrap ? (has_next ? 0 : KT - 1) : is.k;
#pragma unroll
  for (int v = 0; v < ALoader<64>::V; ++v) is.a.src[v] = sw ? aln.src[v] : is.a.src[v];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    is.b.cp[j] = sw ? bln.cp[j] : is.b.cp[j];
    is.b.sp[j] = sw ? bln.sp[j] : is.b.sp[j];
  }
}

// Pointers to the three stages, each its own LDS array: with a stage
// index known at compile time the compiler sees that the fragment reads of
// one stage do not touch the stages the DMA is filling, and adds no wait
// for those loads (with one array indexed at run time it waits for all of
// them before every LDS read).
struct PStages {
  uint16_t* a[kPStages];  // A tiles
  uint8_t* b[kPStages];   // each wave's weights
};

// One K step of a tile on stage S (see pkernel).
template <int S, int NI, class W>
__device__ __forceinline__ void pstep(int KT, bool has_next, PIssue<W>& is, const ALoader<64>& aln,
                                      const W& bln, const PStages& ps, const int (&shift)[2],
                                      const int (&frag)[4], f32x16 (&acc)[NI][2]) {
  constexpr int S2 = (S + 2) % kPStages;
  const int wave = threadIdx.x >> 6;
  // the loads two steps ahead, into the stage every wave finished with at
  // the last barrier
  is.a.issue_asm(is.k, ps.a[S2]);
  is.b.issue(is.k, ps.b[S2] + wave * W::kWaveBytes);
  padvance(is, KT, has_next, aln, bln);
  typename W::Set bs;
  W::read(ps.b[S] + wave * W::kWaveBytes, shift, bs);
  const uint16_t* ca = ps.a[S];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    bf16x8 a[NI], b[2];
#pragma unroll
    for (int i = 0; i < NI; ++i) a[i] = *(const bf16x8*)(ca + i * 32 * 64 + frag[ks]);
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = W::frag(bs, j, ks);
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(b[j], a[i], acc[i][j]);
  }
  // the next step's loads complete in this wave (those two ahead may be in
  // flight), then in every wave
  wait_vmcnt<ALoader<64>::V + W::kLoads>();
  dma_barrier();
}

// A tile's KT steps with its first step on stage P.
template <int P, int NI, class W>
__device__ __forceinline__ void psteps(int KT, bool has_next, PIssue<W>& is, const ALoader<64>& aln,
                                       const W& bln, const PStages& ps, const int (&shift)[2],
                                       const int (&frag)[4], f32x16 (&acc)[NI][2]) {
  constexpr int P1 = (P + 1) % kPStages, P2 = (P + 2) % kPStages;
  int kt = 0;
  for (; kt + 3 <= KT; kt += 3) {
    pstep<P, NI>(KT, has_next, is, aln, bln, ps, shift, frag, acc);
    pstep<P1, NI>(KT, has_next, is, aln, bln, ps, shift, frag, acc);
    pstep<P2, NI>(KT, has_next, is, aln, bln, ps, shift, frag, acc);
  }
  if (kt < KT) pstep<P, NI>(KT, has_next, is, aln, bln, ps, shift, frag, acc);
  if (kt + 1 < KT) pstep<P1, NI>(KT, has_next, is, aln, bln, ps, shift, frag, acc);
}

// One tile's K steps, starting on stage s (updated to the stage after its
// last step), then between(), then the epilogue. The loads of its first
// two steps are in flight or done, the first complete in every wave; shift:
// where the tile's scale bytes sit in their dwords.
template <int NI, class Op, class F>
__device__ __forceinline__ void ptile_run(const Op& op, const TileWork& tw, int n0, const int (&shift)[2],
                                          bool has_next, PIssue<typename Op::W>& is,
                                          const ALoader<64>& aln, const typename Op::W& bln,
                                          const PStages& ps, int& s, const int (&frag)[4], F between) {
  const int KT = op.k_steps();
  f32x16 acc[NI][2];
  zero_acc<NI>(acc);
  if (s == 0) psteps<0, NI>(KT, has_next, is, aln, bln, ps, shift, frag, acc);
  else if (s == 1) psteps<1, NI>(KT, has_next, is, aln, bln, ps, shift, frag, acc);
  else psteps<2, NI>(KT, has_next, is, aln, bln, ps, shift, frag, acc);
  s = (s + KT) % kPStages;
  between();
  // the stage of the tile's last step: every wave finished reading it at
  // that step's barrier, and no load fills it until the next tile's first
  // step issues its loads (picked by selects: indexing the pointer array at
  // run time made the compiler spill hundreds of registers)
  const int sl = (s + 2) % kPStages;
  op.template epilogue<NI>(tw, n0, acc, sl == 0 ? ps.a[0] : (sl == 1 ? ps.a[1] : ps.a[2]));
  if constexpr (Op::kStagedEpi) dma_barrier();
}

template <class Op>
__device__ __forceinline__ void pkernel(const Op& op) {
  using W = typename Op::W;
  __shared__ __attribute__((aligned(16))) uint16_t lds_a0[kBM * 64];
  __shared__ __attribute__((aligned(16))) uint16_t lds_a1[kBM * 64];
  __shared__ __attribute__((aligned(16))) uint16_t lds_a2[kBM * 64];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b0[4 * W::kWaveBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b1[4 * W::kWaveBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b2[4 * W::kWaveBytes];
  const PStages ps{{lds_a0, lds_a1, lds_a2}, {lds_b0, lds_b1, lds_b2}};
  const int nt = op.n_tiles(), KT = op.k_steps();
  const int x = blockIdx.x % kXcds, nq = gridDim.x / kXcds;
  const int* split = op.rv.split + 9 * Op::kSplit;
  const int hi = split[x + 1];
  int t = split[x] + blockIdx.x / kXcds;
  if (t >= hi) return;
  auto info = [&](int i, TileWork* tw, int* n0) {
    const int mt = i / nt;
    const int4 w = op.rv.ttab[mt];
    *tw = TileWork{w.x, w.y, w.z};
    *n0 = (i - mt * nt) * Op::kTileN;
  };
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int frag[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) frag[ks] = swz<64>(lane & 31, (lane >> 5) * 4 + ks) * 8;
  // this tile and the next one set up, the first two steps' loads issued
  TileWork cur, nxt;
  int n0, n1;
  info(t, &cur, &n0);
  PIssue<W> is;
  op.setup(cur, n0, is.a, is.b);
  int shift[2] = {is.b.shift[0], is.b.shift[1]};
  bool has_next = t + nq < hi;
  nxt = cur;
  n1 = n0;
  ALoader<64> aln = is.a;
  W bln = is.b;
  if (has_next) {
    info(t + nq, &nxt, &n1);
    op.setup(nxt, n1, aln, bln);
  }
  is.k = 0;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    is.a.issue_asm(is.k, ps.a[k]);
    is.b.issue(is.k, ps.b[k] + wave * W::kWaveBytes);
    padvance(is, KT, has_next, aln, bln);
  }
  wait_vmcnt<ALoader<64>::V + W::kLoads>();
  dma_barrier();
  int s = 0;
  for (;;) {
    // the tile after the next one, set up between this tile's steps and its
    // epilogue (its row loads then wait for nothing but the next tile's
    // second step)
    const bool has2 = has_next && t + 2 * nq < hi;
    TileWork nxt2;
    int n2;
    ALoader<64> an2;  // not live during the tile's steps
    W bn2;
    auto between = [&]() {
      if (has2) {
        info(t + 2 * nq, &nxt2, &n2);
        op.setup(nxt2, n2, an2, bn2);
      } else {
        nxt2 = nxt;
        n2 = n1;
        an2 = aln;
        bn2 = bln;
      }
    };
    const int nb = row_blocks(cur);
    if (nb == 1) ptile_run<1>(op, cur, n0, shift, has_next, is, aln, bln, ps, s, frag, between);
    else if (nb == 2) ptile_run<2>(op, cur, n0, shift, has_next, is, aln, bln, ps, s, frag, between);
    else if (nb == 3) ptile_run<3>(op, cur, n0, shift, has_next, is, aln, bln, ps, s, frag, between);
    else ptile_run<4>(op, cur, n0, shift, has_next, is, aln, bln, ps, s, frag, between);
    if (!has_next) break;
    t += nq;
    cur = nxt;
    n0 = n1;
    shift[0] = bln.shift[0];
    shift[1] = bln.shift[1];
    nxt = nxt2;
    n1 = n2;
    aln = an2;
    bln = bn2;
    has_next = has2;
  }
  // the DMA into LDS has landed before the workgroup ends
  wait_vmcnt<0>();
}

template <bool PK, int BITS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_expert_gateup_p(
    const uint16_t* __restrict__ hcat, int ldh, RouteView rv, ExpertsView ex,
    uint16_t* __restrict__ act, int inter, int latent) {
  pkernel(PGateUp<PK, BITS>{hcat, ldh, rv, ex, act, inter, latent});
}

template <bool PK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_expert_down_p(
    const uint16_t* __restrict__ act, RouteView rv, ExpertsView ex, uint16_t* __restrict__ y,
    int inter, int latent) {
  pkernel(PDown<PK>{act, rv, ex, y, inter, latent});
}

// ------------------------------------------------------------------ launchers

static inline int pick_bk(int K, int kwrap) { return (K % 64 == 0 && kwrap % 64 == 0) ? 64 : 32; }

// Two persistent workgroups per CU, a multiple of 8 in all (every XCD the
// same number).
static int persistent_grid() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8)
      n = 256;
    cached[dev] = 2 * (n / kXcds) * kXcds;
  }
  return cached[dev];
}

hipError_t launch_gemm_dense(int epi, const uint16_t* A, int lda, const uint16_t* B, int ldb,
                             int kwrap, int M, int N, int K, const DenseEpilogue& ep,
                             hipStream_t stream, bool packed) {
  const int nt = (N + kBN - 1) / kBN;
  // 64-row tiles when 128-row tiles would fill at most half the CUs
  // (measured on the 4096-token 120B layer: its router, 64 tiles, 42 -> 32
  // us; its D, 160 tiles, 53 -> 59 us, so at 160 the 128-row tiles stay)
  const bool half = nt * ((M + kBM - 1) / kBM) <= persistent_grid() / 4;
  dim3 grid(nt * ((M + (half ? kBM / 2 : kBM) - 1) / (half ? kBM / 2 : kBM))), block(kThreads);
  const int bk = pick_bk(K, kwrap);
  if (packed && (bk != 64 || N % 32)) return hipErrorInvalidValue;
  const bool two = (int)grid.x >= persistent_grid();  // at least two workgroups per CU
#define MOE_LAUNCH_DENSE(BKV, EPIV, PKV)                                                       \
  do {                                                                                         \
    if (half && two)                                                                           \
      hipLaunchKernelGGL((k_gemm_dense2<BKV, EPIV, PKV, 2>), grid, block, 0, stream, A, lda, B, \
                         ldb, kwrap, M, N, K, ep);                                             \
    else if (half)                                                                             \
      hipLaunchKernelGGL((k_gemm_dense<BKV, EPIV, PKV, 2>), grid, block, 0, stream, A, lda, B,  \
                         ldb, kwrap, M, N, K, ep);                                             \
    else if (two)                                                                              \
      hipLaunchKernelGGL((k_gemm_dense2<BKV, EPIV, PKV>), grid, block, 0, stream, A, lda, B,   \
                         ldb, kwrap, M, N, K, ep);                                             \
    else                                                                                       \
      hipLaunchKernelGGL((k_gemm_dense<BKV, EPIV, PKV>), grid, block, 0, stream, A, lda, B,    \
                         ldb, kwrap, M, N, K, ep);                                             \
  } while (0)
  if (packed) {
    if (epi == kEpiSplit) MOE_LAUNCH_DENSE(64, kEpiSplit, true);
    else if (epi == kEpiLogits) MOE_LAUNCH_DENSE(64, kEpiLogits, true);
    else MOE_LAUNCH_DENSE(64, kEpiOut, true);
  } else if (bk == 64) {
    if (epi == kEpiSplit) MOE_LAUNCH_DENSE(64, kEpiSplit, false);
    else if (epi == kEpiLogits) MOE_LAUNCH_DENSE(64, kEpiLogits, false);
    else MOE_LAUNCH_DENSE(64, kEpiOut, false);
  } else {
    if (epi == kEpiSplit) MOE_LAUNCH_DENSE(32, kEpiSplit, false);
    else if (epi == kEpiLogits) MOE_LAUNCH_DENSE(32, kEpiLogits, false);
    else MOE_LAUNCH_DENSE(32, kEpiOut, false);
  }
#undef MOE_LAUNCH_DENSE
  return hipGetLastError();
}


hipError_t launch_expert_gateup(const uint16_t* hcat, int ldh, const RouteView& rv,
                                const ExpertsView& ex, uint16_t* act, int inter, int latent,
                                int max_mtiles, hipStream_t stream) {
  if ((ex.packed || ex.gateup_bits == 3) && latent % 64 != 0) return hipErrorInvalidValue;
  if (latent % 64 == 0 && latent >= 128) {  // persistent: K steps of 64, at least two
    const dim3 grid(persistent_grid()), block(kThreads);
#define MOE_LAUNCH_GUP(PKV, BITSV)                                                                 \
  hipLaunchKernelGGL((k_expert_gateup_p<PKV, BITSV>), grid, block, 0, stream, hcat, ldh, rv, ex,   \
                     act, inter, latent)
    if (ex.gateup_bits == 3) {
      if (ex.packed) MOE_LAUNCH_GUP(true, 3);
      else MOE_LAUNCH_GUP(false, 3);
    } else if (ex.packed) {
      MOE_LAUNCH_GUP(true, 4);
    } else {
      MOE_LAUNCH_GUP(false, 4);
    }
#undef MOE_LAUNCH_GUP
    return hipGetLastError();
  }
  dim3 grid(max_mtiles * ((inter + kBN / 2 - 1) / (kBN / 2))), block(kThreads);
#define MOE_LAUNCH_GU(BKV, PKV, BITSV)                                                           \
  hipLaunchKernelGGL((k_expert_gateup<BKV, PKV, BITSV>), grid, block, 0, stream, hcat, ldh, rv, ex, \
                     act, inter, latent)
  if (ex.gateup_bits == 3) {
    if (ex.packed) MOE_LAUNCH_GU(64, true, 3);
    else MOE_LAUNCH_GU(64, false, 3);
  } else if (ex.packed) {
    MOE_LAUNCH_GU(64, true, 4);
  } else if (latent % 64 == 0) {
    MOE_LAUNCH_GU(64, false, 4);
  } else {
    MOE_LAUNCH_GU(32, false, 4);
  }
#undef MOE_LAUNCH_GU
  return hipGetLastError();
}

hipError_t launch_expert_down(const uint16_t* act, const RouteView& rv, const ExpertsView& ex,
                              uint16_t* y, int inter, int latent, int max_mtiles,
                              hipStream_t stream) {
  if (ex.packed && inter % 64 != 0) return hipErrorInvalidValue;
  if (inter % 64 == 0 && inter >= 128) {  // persistent: K steps of 64, at least two
    const dim3 grid(persistent_grid()), block(kThreads);
    if (ex.packed)
      hipLaunchKernelGGL((k_expert_down_p<true>), grid, block, 0, stream, act, rv, ex, y, inter, latent);
    else
      hipLaunchKernelGGL((k_expert_down_p<false>), grid, block, 0, stream, act, rv, ex, y, inter, latent);
    return hipGetLastError();
  }
  dim3 grid(max_mtiles * ((latent + kBN - 1) / kBN)), block(kThreads);
  if (ex.packed)
    hipLaunchKernelGGL((k_expert_down<64, true>), grid, block, 0, stream, act, rv, ex, y, inter,
                       latent);
  else if (inter % 64 == 0)
    hipLaunchKernelGGL((k_expert_down<64, false>), grid, block, 0, stream, act, rv, ex, y, inter,
                       latent);
  else
    hipLaunchKernelGGL((k_expert_down<32, false>), grid, block, 0, stream, act, rv, ex, y, inter,
                       latent);
  return hipGetLastError();
}

}  // namespace moe
