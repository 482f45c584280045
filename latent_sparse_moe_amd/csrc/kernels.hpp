// Kernel-side views and launcher declarations of the latent-MoE layer.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// One set of quantised matrices [count][N][K] (see include/moe_latent.h).
struct Fp4Mat {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* gscale;
};

struct Fp4Set {
  Fp4Mat gate, up, down;
};

// Routed experts and the shared expert. Grouped kernels number the groups
// 0..n_experts-1 (routed) and n_experts (shared, when present). packed: both
// sets are in the layout written by launch_pack_fp4 (K multiples of 64).
struct ExpertsView {
  Fp4Set routed;
  Fp4Set shared;
  bool packed;
  int gateup_bits;  // 4: e2m1 gate/up codes; 3: E1M1 (down is e2m1 either way)
};

// Routing as the grouped GEMMs consume it. Rows of the permuted activation
// matrices: [0, pairs) are the routed (token, choice) pairs grouped by expert,
// [pairs, pairs + T) the shared expert's rows (token t at pairs + t).
struct RouteView {
  const int* tile_off;  // [n_groups + 1] exclusive prefix of ceil(count_g / 128)
  const int* off;       // [n_groups + 1] first permuted row of each group
  const int* perm;      // [pairs] pair index at each permuted row
  int n_experts;
  int n_shared;
  int pairs;  // T * top_k
  int top_k;
  // routing groups of D/U: expert e reads the latent of group
  // e / experts_per_group, at column (that group) * group_stride of its
  // token's row (the shared expert: group 0)
  int experts_per_group;
  int group_stride;
  // the m-tiles listed ({group, first row, end of the group's rows, 0}),
  // tile_off[n_groups] of them, and each XCD's run of the tile list
  // (m-tile x n-tile, n fastest): gate/up split[0..8], down split[9..17]
  const int4* ttab;
  const int* split;
};

enum { kEpiSplit = 0, kEpiLogits = 1, kEpiOut = 2 };

struct DenseEpilogue {
  void* out;
  int ldo;
  // kEpiSplit: output column n (of group g = n / group_w) goes to column
  // n + g * group_w (hi) and that plus lo_off (lo): per group, group_w hi
  // columns then group_w lo columns when lo_off = group_w
  int lo_off;
  int group_w;
  const float* bias;       // kEpiLogits: [N] or null
  const uint16_t* resid;   // kEpiOut: bf16 [M][ldr] added before rounding, or null
  int ldr;
};

// packed: B is in the layout written by launch_pack_bf16 ([N][kwrap] packed;
// N % 32 == 0, K and kwrap multiples of 64).
hipError_t launch_gemm_dense(int epi, const uint16_t* A, int lda, const uint16_t* B, int ldb,
                             int kwrap, int M, int N, int K, const DenseEpilogue& ep,
                             hipStream_t stream, bool packed = false);
hipError_t launch_expert_gateup(const uint16_t* hcat, int ldh, const RouteView& rv,
                                const ExpertsView& ex, uint16_t* act, int inter, int latent,
                                int max_mtiles, hipStream_t stream);
hipError_t launch_expert_down(const uint16_t* act, const RouteView& rv, const ExpertsView& ex,
                              uint16_t* y, int inter, int latent, int max_mtiles,
                              hipStream_t stream);
// fp4 matrix set [count][N][K] (N % 32 == 0, K % 64 == 0) -> the packed
// layout the grouped kernels load with one 1 KB (codes) and one 128-byte
// (scales) access per wave and K step; same byte counts as the plain layout.
// bits: 4 (e2m1 codes) or 3 (E1M1 codes, 12-byte chunks per 32 elements).
hipError_t launch_pack_fp4(const uint8_t* codes, const uint8_t* scales, int count, int N, int K,
                           int bits, uint8_t* pcodes, uint8_t* pscales, hipStream_t stream);
// bf16 matrix [N][K] (N % 32 == 0, K % 64 == 0) -> the packed layout the
// dense kernels load with one contiguous 1 KB access per wave.
hipError_t launch_pack_bf16(const uint16_t* w, int N, int K, uint16_t* pw, hipStream_t stream);

// Routing bookkeeping (route.hip).
constexpr int kRouteChunk = 2048;  // pairs per histogram / permute chunk
constexpr int kMaxExperts = 1024;

hipError_t launch_rmsnorm(const uint16_t* x, const float* w, float eps, uint16_t* u, int T,
                          int hidden, hipStream_t stream);
hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                       hipStream_t stream);
hipError_t launch_route_hist(const int32_t* idx, int pairs, int E, int32_t* chunk_hist,
                             hipStream_t stream);
hipError_t launch_route_scan(int32_t* chunk_hist, int n_chunks, int E, int pairs, int T,
                             int n_shared, int32_t* counts, int32_t* off, int32_t* tile_off,
                             int4* ttab, int nt_gu, int nt_dn, int32_t* split, hipStream_t stream);
hipError_t launch_route_permute(const int32_t* idx, int pairs, int E,
                                const int32_t* chunk_base, const int32_t* off, int32_t* perm,
                                int32_t* slot, hipStream_t stream);
// z [T][G * latent]: group g's columns hold the token's experts of group g
// (expert e in group e / experts_per_group; the shared expert in group 0).
hipError_t launch_combine(const uint16_t* y, const int32_t* slot, const float* w,
                          const int32_t* idx, int T, int k, int pairs, int latent, int n_shared,
                          int n_groups, int experts_per_group, uint16_t* z, hipStream_t stream);

// ------------------------------------------------------------------ decode path

constexpr int kDecodeMaxT = 8;   // tokens the weight-streaming decode kernels take

// Stage ids for optional timing events (match MOE_LATENT_STAGE_* in the header).
enum { kStageNorm = 0, kStageDproj = 1, kStageRouter = 2, kStageTopk = 3, kStageRoute = 4,
       kStageGateup = 5, kStageDown = 6, kStageCombine = 7, kStageUproj = 8 };

// Records the caller's event pair of a stage on the stream (no-op when absent).
struct StageMarks {
  void* const* ev;
  hipStream_t st;
  hipError_t mark(int stage, int end) const {
    if (!ev) return hipSuccess;
    void* e = ev[2 * stage + end];
    return e ? hipEventRecord((hipEvent_t)e, st) : hipSuccess;
  }
  // Launches `kernel` as the whole of `stage`: the stage's events (when
  // given) are recorded by the dispatch itself, so they time the kernel
  // alone rather than the kernel plus two extra queue packets.
  template <typename K, typename... Args>
  hipError_t launch(int stage, K kernel, dim3 grid, dim3 block, size_t lds, Args... args) const {
    hipEvent_t e0 = ev ? (hipEvent_t)ev[2 * stage] : nullptr;
    hipEvent_t e1 = ev ? (hipEvent_t)ev[2 * stage + 1] : nullptr;
    return launch_ev(e0, e1, kernel, grid, block, lds, args...);
  }
  // A stage of two launches: the first records the start event, the last
  // the end event.
  template <typename K, typename... Args>
  hipError_t launch_first(int stage, K kernel, dim3 grid, dim3 block, size_t lds,
                          Args... args) const {
    return launch_ev(ev ? (hipEvent_t)ev[2 * stage] : nullptr, nullptr, kernel, grid, block, lds,
                     args...);
  }
  template <typename K, typename... Args>
  hipError_t launch_last(int stage, K kernel, dim3 grid, dim3 block, size_t lds,
                         Args... args) const {
    return launch_ev(nullptr, ev ? (hipEvent_t)ev[2 * stage + 1] : nullptr, kernel, grid, block,
                     lds, args...);
  }
  template <typename K, typename... Args>
  hipError_t launch_ev(hipEvent_t e0, hipEvent_t e1, K kernel, dim3 grid, dim3 block, size_t lds,
                       Args... args) const {
    if (e0 || e1)
      hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, st, e0, e1, 0u, args...);
    else
      hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
    return hipGetLastError();
  }
};

struct DecodeArgs {
  // inputs
  const uint16_t* x;
  const uint16_t* D;
  const uint16_t* R;
  const uint16_t* RD;        // folded router [2][E][hidden] (hi, lo; decode-packed), or null
  const uint16_t* U;
  const float* bias;         // or null
  const float* norm_weight;  // residual block when non-null
  float norm_eps;
  Fp4Mat gate, up, down;           // routed experts
  Fp4Mat sh_gate, sh_up, sh_down;  // shared expert (count 1)
  int hidden, latent, inter, n_experts, top_k, n_shared, T;
  int n_groups;  // routing groups: D [G*latent][hidden], U [hidden][G*latent]; h, z [T][G*latent]
  bool packed;  // D, U, R and the expert sets above are in the decode-packed layouts
  int gateup_bits;  // 4: e2m1 gate/up codes (routed and shared); 3: E1M1
  int n_parts;      // the logits are the sum of n_parts [T][E] parts (set by launch_decode)
  // scratch (workspace)
  uint16_t* hhi;       // [T][G*latent] bf16(h)
  uint16_t* hlo;       // [T][G*latent] h - bf16(h) (unfolded router only; else null)
  // one routing group only (else null): bf16(h) as fp16 [T][latent], and
  // one flag per front workgroup of h rows (1: one of its values is not
  // exact in fp16); with no flag set gate/up takes its fp16 route
  uint16_t* h16;
  int* hflag;          // [latent / 16]
  float* logits;       // [n_parts][T][E]
  uint16_t* act;       // [1 + max_active][T][inter]   slot 0: shared expert
  // [T][G*latent] combined expert output in 64-bit fixed point (units of
  // 2^-32), zeroed by the first kernel, summed by the down kernel
  unsigned long long* zfix;
  int max_active;      // min(n_experts, T * top_k): capacity of the routing table
  int gu_grid;         // gate/up workgroups (set by launch_decode)
  int* route_n_act;    // [1]
  int* route_list;     // [max_active]
  float* route_wtab;   // [1 + max_active][T]
  // output
  uint16_t* out;
  // optional routing copies
  int32_t* dbg_idx;
  float* dbg_w;
  int32_t* dbg_counts;
  int32_t* dbg_offsets;
  int32_t* dbg_perm;
  float* dbg_logits;
};

bool decode_supported(int hidden, int latent, int inter, int n_experts, int top_k, int n_groups,
                      int T);
constexpr int kDecodeDownGroup = 8;  // expert slots per down workgroup (one per wave)
// Slot groups of the down kernel for a routing table of max_active experts
// (slots 0 .. max_active, slot 0 the shared expert).
__host__ __device__ inline int decode_down_groups(int max_active) {
  return (max_active + kDecodeDownGroup) / kDecodeDownGroup;
}
// The router folded onto the residual width (moe_router_fold): W = R D in
// fp64, stored as bf16 hi = bf16(W) and lo = bf16(W - hi) in the
// decode-packed bf16 layout ([2][E][hidden]); E % 16 == 0, hidden % 32 == 0.
hipError_t launch_router_fold(const uint16_t* R, const uint16_t* D, int E, int latent, int hidden,
                              int n_groups, uint16_t* dst, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st, const StageMarks& mk);
// Decode-packed layouts (decode.hip): fp4 set [count][N][K] with N % 16 == 0,
// K % 128 == 0; bf16 [N][K] with N % 16 == 0, K % 32 == 0.
hipError_t launch_pack_fp4_decode(const uint8_t* codes, const uint8_t* scales, int count, int N,
                                  int K, int bits, uint8_t* pcodes, uint8_t* pscales,
                                  hipStream_t stream);
hipError_t launch_pack_bf16_decode(const uint16_t* w, int N, int K, uint16_t* pw,
                                   hipStream_t stream);

}  // namespace moe
