// Routing, combine and normalisation kernels of the latent-MoE layer (gfx950).
//
// Routing follows the layer description on the Hugging Face card
// "Edge0-145B . Q3_K" (section "Architecture": the router picks 10 of 512
// experts per token). Gating reading: softmax over all expert logits, the k
// largest (ties to the lower index), weights renormalised over the k. The
// renormalised weight of a chosen expert is exp(l_j - l_max) over the sum of
// the same terms for the chosen k: the full softmax denominator cancels, so
// only the k chosen logits are exponentiated.
//
// Everything here is deterministic: integer counting uses LDS atomics only
// for order-free sums, positions come from wave ballots in lane order, and
// floating-point reductions run in a fixed order.
#include <limits.h>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// ------------------------------------------------------------------ RMSNorm

// u[t] = bf16(x[t] / sqrt(mean(x[t]^2) + eps) * w), one workgroup per token.
__global__ __launch_bounds__(256) void k_rmsnorm(const uint16_t* __restrict__ x,
                                                 const float* __restrict__ w, float eps,
                                                 uint16_t* __restrict__ u, int hidden) {
  __shared__ float part[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const uint16_t* row = x + (size_t)t * hidden;
  const int nch = hidden / 8;
  float ss = 0.0f;
  for (int c = tid; c < nch; c += 256) {
    const uint4 v = *(const uint4*)(row + c * 8);
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float a = bf16_bits_to_f32(d[q] & 0xFFFFu), b = bf16_bits_to_f32(d[q] >> 16);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  const float tot = ((part[0] + part[1]) + part[2]) + part[3];
  const float r = 1.0f / sqrtf(tot / (float)hidden + eps);
  uint16_t* urow = u + (size_t)t * hidden;
  for (int c = tid; c < nch; c += 256) {
    const uint4 v = *(const uint4*)(row + c * 8);
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = c * 8 + 2 * q;
      const float a = bf16_bits_to_f32(d[q] & 0xFFFFu) * r * w[k];
      const float b = bf16_bits_to_f32(d[q] >> 16) * r * w[k + 1];
      o[q] = pack_bf16x2(a, b);
    }
    *(uint4*)(urow + c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

hipError_t launch_rmsnorm(const uint16_t* x, const float* w, float eps, uint16_t* u, int T,
                          int hidden, hipStream_t stream) {
  hipLaunchKernelGGL(k_rmsnorm, dim3(T), dim3(256), 0, stream, x, w, eps, u, hidden);
  return hipGetLastError();
}

// ------------------------------------------------------------------ top-k

// One wave per token; lane l holds the logits of experts l, l+64, ... (EPL
// of them) as order-preserving keys; k rounds of a wave-wide arg-max (larger
// value wins, ties to the lower expert index); lane j keeps the j-th choice.
template <int EPL>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int T, int E,
                                              int k, int32_t* __restrict__ idx,
                                              float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  uint32_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? order_key(row[e]) : 0u;
  }
  uint32_t my_key;
  int my_e;
  wave_select_topk<EPL>(key, E, k, my_key, my_e);
  const float mx = key_value((uint32_t)__builtin_amdgcn_readlane((int)my_key, 0));
  const float ex = lane < k ? expf(key_value(my_key) - mx) : 0.0f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    idx[(size_t)t * k + lane] = my_e;
    w[(size_t)t * k + lane] = ex / sum;
  }
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                       hipStream_t stream) {
  const int epl = (E + 63) / 64;
  dim3 grid((T + 3) / 4), block(256);
  if (epl <= 1) hipLaunchKernelGGL(k_topk<1>, grid, block, 0, stream, logits, T, E, k, idx, w);
  else if (epl <= 2) hipLaunchKernelGGL(k_topk<2>, grid, block, 0, stream, logits, T, E, k, idx, w);
  else if (epl <= 4) hipLaunchKernelGGL(k_topk<4>, grid, block, 0, stream, logits, T, E, k, idx, w);
  else if (epl <= 8) hipLaunchKernelGGL(k_topk<8>, grid, block, 0, stream, logits, T, E, k, idx, w);
  else hipLaunchKernelGGL(k_topk<16>, grid, block, 0, stream, logits, T, E, k, idx, w);
  return hipGetLastError();
}

// ------------------------------------------------------------------ histogram

// chunk_hist[c][e] = pairs of chunk c (pairs [c*CH, (c+1)*CH)) routed to e.
__global__ __launch_bounds__(256) void k_route_hist(const int32_t* __restrict__ idx, int pairs,
                                                    int E, int32_t* __restrict__ chunk_hist) {
  __shared__ int h[kMaxExperts];
  const int tid = threadIdx.x, c = blockIdx.x;
  for (int e = tid; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int p0 = c * kRouteChunk, p1 = min(p0 + kRouteChunk, pairs);
  for (int p = p0 + tid; p < p1; p += 256) atomicAdd(&h[idx[p]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += 256) chunk_hist[(size_t)c * E + e] = h[e];
}

hipError_t launch_route_hist(const int32_t* idx, int pairs, int E, int32_t* chunk_hist,
                             hipStream_t stream) {
  const int nch = (pairs + kRouteChunk - 1) / kRouteChunk;
  hipLaunchKernelGGL(k_route_hist, dim3(nch), dim3(256), 0, stream, idx, pairs, E, chunk_hist);
  return hipGetLastError();
}

// ------------------------------------------------------------------ scan

// Exclusive prefix sum over the 1024 threads of the block; *total gets the sum.
__device__ int block_exclusive_scan_1024(int v, int* total) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int inc = wave_inclusive_scan(v);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int s = lane < 16 ? wsum[lane] : 0;
    const int sinc = wave_inclusive_scan(s);
    if (lane < 16) wsum[lane] = sinc - s;  // exclusive over waves
    if (lane == 15) *total = sinc;
  }
  __syncthreads();
  const int r = wsum[wave] + inc - v;
  __syncthreads();
  return r;
}

// One block of 1024 threads, thread e for expert e:
//   counts[e]; off[e] = exclusive prefix of counts (off[E] = pairs,
//   off[E+1] = pairs + n_shared*T for the shared expert's rows);
//   tile_off likewise over ceil(count/128) (the grouped GEMM m-tiles);
//   chunk_hist[c][e] becomes the pairs of e in chunks before c (the permute
//   adds off[e]). A thread's chunk counts are loaded 32 at a time before
//   any is used, so the walk over the chunks is not one load round trip per
//   chunk.
//   ttab: the m-tiles listed, m-tile i = {group, first row, end of the
//   group's rows, 0} (experts in order, then the shared expert's).
//   split[9k .. 9k+8] (k = 0 for gate/up with nt[0] n-tiles per m-tile,
//   k = 1 for down with nt[1]): the tile list (m-tiles times n-tiles, n
//   fastest) cut into eight runs of about equal cost, one per XCD (run x =
//   tiles [split[9k+x], split[9k+x+1])). An m-tile's cost is tile_cost of
//   its row count, the same for each of its n-tiles.
__device__ __forceinline__ int tile_cost(int rows) {
  const int nb = (rows + 31) / 32;  // blocks of 32 rows the tile runs with: 1 to 4
  return nb <= 1 ? 6 : nb == 2 ? 7 : nb == 3 ? 8 : 10;
}

// Cost of the m-tiles of a group of cnt > 0 rows: 10 per full tile, the
// last one by its rows.
__device__ __forceinline__ int group_cost(int cnt) {
  const int n = (cnt + 127) / 128;
  return 10 * (n - 1) + tile_cost(cnt - 128 * (n - 1));
}

__global__ __launch_bounds__(1024) void k_route_scan(int32_t* __restrict__ chunk_hist,
                                                     int n_chunks, int E, int pairs, int T,
                                                     int n_shared, int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ off,
                                                     int32_t* __restrict__ tile_off,
                                                     int4* __restrict__ ttab, int nt_gu, int nt_dn,
                                                     int32_t* __restrict__ split) {
  __shared__ int totals[3];
  const int e = threadIdx.x;
  int cnt = 0;
  if (e < E) {
    for (int c0 = 0; c0 < n_chunks; c0 += 32) {
      int v[32];
#pragma unroll
      for (int j = 0; j < 32; ++j)
        v[j] = c0 + j < n_chunks ? chunk_hist[(size_t)(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        if (c0 + j < n_chunks) chunk_hist[(size_t)(c0 + j) * E + e] = cnt;
        cnt += v[j];
      }
    }
  }
  const int tiles = (cnt + 127) / 128;
  const int ex_cnt = block_exclusive_scan_1024(cnt, &totals[0]);
  const int ex_tiles = block_exclusive_scan_1024(tiles, &totals[1]);
  const int ex_cost = block_exclusive_scan_1024(cnt > 0 ? group_cost(cnt) : 0, &totals[2]);
  // per group (the shared expert last): first row, first m-tile, cost before it
  __shared__ int g_off[kMaxExperts + 2], g_tile[kMaxExperts + 2], g_cost[kMaxExperts + 2];
  const int shared_tiles = n_shared * ((T + 127) / 128);
  const int G = E + n_shared;  // groups
  if (e < E) {
    counts[e] = cnt;
    off[e] = ex_cnt;
    tile_off[e] = ex_tiles;
    g_off[e] = ex_cnt;
    g_tile[e] = ex_tiles;
    g_cost[e] = ex_cost;
  }
  if (e == 0) {
    off[E] = pairs;
    off[E + 1] = pairs + n_shared * T;
    tile_off[E] = totals[1];
    tile_off[E + 1] = totals[1] + shared_tiles;
    g_off[E] = pairs;
    g_off[E + 1] = pairs + n_shared * T;
    g_tile[E] = totals[1];
    g_tile[E + 1] = totals[1] + shared_tiles;
    g_cost[E] = totals[2];
    g_cost[E + 1] = totals[2] + (n_shared && T > 0 ? group_cost(T) : 0);
  }
  __syncthreads();
  // the group of m-tile i: the largest g with g_tile[g] <= i (LDS search)
  auto group_of_tile = [&](int i) {
    int lo = 0, hi = G;  // g_tile[lo] <= i < g_tile[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (g_tile[mid] <= i) lo = mid; else hi = mid;
    }
    return lo;
  };
  const int n_mt = g_tile[G];
  for (int i = threadIdx.x; i < n_mt; i += 1024) {
    const int g = group_of_tile(i);
    ttab[i] = make_int4(g, g_off[g] + 128 * (i - g_tile[g]), g_off[g + 1], 0);
  }
  // split points: thread 8k + x (x = 1..7) finds the first tile whose cost
  // prefix reaches x/8 of the total (its m-tile by a search over the groups'
  // cost prefixes, then within the group)
  const int64_t C = g_cost[G];
  if (threadIdx.x < 16) {
    const int k = threadIdx.x >> 3, x = threadIdx.x & 7;
    const int64_t q = k ? nt_dn : nt_gu;
    const int n_tiles = n_mt * (int)q;
    int res;
    if (x == 0) {
      res = 0;
    } else {
      const int64_t tau = (x * q * C + 7) / 8;  // in tile-cost units (each m-tile's cost counts q times)
      if (tau >= q * C) {
        res = n_tiles;
      } else {
        int lo = 0, hi = G;  // q * g_cost[lo] <= tau < q * g_cost[hi]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (q * g_cost[mid] <= tau) lo = mid; else hi = mid;
        }
        const int rows = g_off[lo + 1] - g_off[lo], n = (rows + 127) / 128;
        const int clast = tile_cost(rows - 128 * (n - 1));
        const int64_t o = tau - q * g_cost[lo];
        int64_t m = o / (10 * q);
        if (m > n - 1) m = n - 1;
        const int64_t r = o - m * 10 * q;
        const int c = m < n - 1 ? 10 : clast;
        res = (int)((g_tile[lo] + m) * q + (r + c - 1) / c);
      }
    }
    split[9 * k + x] = res;
    if (x == 7) split[9 * k + 8] = n_tiles;
  }
}

hipError_t launch_route_scan(int32_t* chunk_hist, int n_chunks, int E, int pairs, int T,
                             int n_shared, int32_t* counts, int32_t* off, int32_t* tile_off,
                             int4* ttab, int nt_gu, int nt_dn, int32_t* split, hipStream_t stream) {
  hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(1024), 0, stream, chunk_hist, n_chunks, E, pairs,
                     T, n_shared, counts, off, tile_off, ttab, nt_gu, nt_dn, split);
  return hipGetLastError();
}

// ------------------------------------------------------------------ permute

// One 4-wave workgroup per chunk walks its pairs in order, 256 at a time
// (wave w takes pairs base + 64w .. +64). Lanes of a wave holding the same
// expert find each other with one ballot per bit of the expert id, and a
// lane's rank among them (lanes below it) orders them. The waves then meet
// in LDS: each wave's count per expert, summed over the earlier waves, comes
// before it. Position = the chunk's cursor for the expert + earlier waves +
// rank, so the result is the stable counting sort: ascending pair index
// within each expert. A lane's expert ids for the whole chunk are loaded
// before the walk.
constexpr int kPermThreads = 256;
constexpr int kPermWaves = kPermThreads / 64;
constexpr int kPermIter = kRouteChunk / kPermThreads;

__global__ __launch_bounds__(kPermThreads) void k_route_permute(
    const int32_t* __restrict__ idx, int pairs, int E, const int32_t* __restrict__ chunk_base,
    const int32_t* __restrict__ off, int32_t* __restrict__ perm, int32_t* __restrict__ slot) {
  __shared__ int cursor[kMaxExperts + 1];
  __shared__ int wcnt[kPermWaves][kMaxExperts + 1];  // per-wave counts of this step
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = blockIdx.x;
  for (int e = tid; e <= E; e += kPermThreads) {
    cursor[e] = e < E ? off[e] + chunk_base[(size_t)c * E + e] : 0;
#pragma unroll
    for (int w = 0; w < kPermWaves; ++w) wcnt[w][e] = 0;
  }
  const int nbits = 32 - __clz(E);  // enough bits for the sentinel value E
  const uint64_t below = lanemask_lt();
  const int p0 = c * kRouteChunk, p1 = min(p0 + kRouteChunk, pairs);
  int ev[kPermIter];
#pragma unroll
  for (int i = 0; i < kPermIter; ++i) {
    const int p = p0 + i * kPermThreads + tid;
    ev[i] = p < p1 ? idx[p] : E;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPermIter; ++i) {
    const int p = p0 + i * kPermThreads + tid;
    const bool valid = p < p1;
    const int e = ev[i];
    uint64_t peers = ~0ull;
    for (int b = 0; b < nbits; ++b) {
      const int bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & below);
    const int cnt = __popcll(peers);
    if (valid && rank == 0) wcnt[wave][e] = cnt;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wcnt[w][e];
    if (valid) {
      const int pos = cursor[e] + before + rank;
      perm[pos] = p;
      slot[p] = pos;
    }
    __syncthreads();  // every lane has read this step's cursors and counts
    if (valid && rank == 0) {
      atomicAdd(&cursor[e], cnt);  // order-free sum over the waves
      wcnt[wave][e] = 0;
    }
    __syncthreads();
  }
}

hipError_t launch_route_permute(const int32_t* idx, int pairs, int E, const int32_t* chunk_base,
                                const int32_t* off, int32_t* perm, int32_t* slot,
                                hipStream_t stream) {
  const int nch = (pairs + kRouteChunk - 1) / kRouteChunk;
  hipLaunchKernelGGL(k_route_permute, dim3(nch), dim3(kPermThreads), 0, stream, idx, pairs, E,
                     chunk_base, off, perm, slot);
  return hipGetLastError();
}

// ------------------------------------------------------------------ combine

// z[t] = sum_j w[t][j] * y[slot(t, j)] (+ y[pairs + t], the shared expert),
// summed in the fixed order j = 0..k-1 then shared, fp32, one bf16 rounding.
// With G routing groups, z[t] has G blocks of latent columns and choice j
// adds into the block of its expert's group idx[t][j] / experts_per_group
// (the shared expert into block 0); each block is summed in the same order.
// A thread owns 8 columns of one token. It reads the token's K slots and
// weights first, then issues all K + 1 row loads before summing, so that
// each thread has K + 1 loads in flight rather than one at a time.
template <int K>
__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ y,
                                                 const int32_t* __restrict__ slot,
                                                 const float* __restrict__ w,
                                                 const int32_t* __restrict__ idx, int T, int pairs,
                                                 int latent, int n_shared, int G, int epg,
                                                 uint16_t* __restrict__ z) {
  const int cpt = latent / 8;
  const int gid = blockIdx.x * 256 + threadIdx.x;
  const int t = gid / cpt, c8 = gid % cpt;
  if (t >= T) return;
  int r[K], grp[K];
  float wt[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    r[j] = slot[(size_t)t * K + j];
    wt[j] = w[(size_t)t * K + j];
    grp[j] = G > 1 ? idx[(size_t)t * K + j] / epg : 0;
  }
  uint4 v[K];
#pragma unroll
  for (int j = 0; j < K; ++j) v[j] = *(const uint4*)(y + (size_t)r[j] * latent + c8 * 8);
  uint4 vs = make_uint4(0u, 0u, 0u, 0u);
  if (n_shared) vs = *(const uint4*)(y + (size_t)(pairs + t) * latent + c8 * 8);
  for (int g = 0; g < G; ++g) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      if (grp[j] != g) continue;
      const uint32_t d[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(wt[j], bf16_bits_to_f32(d[q] & 0xFFFFu), acc[2 * q]);
        acc[2 * q + 1] = fmaf(wt[j], bf16_bits_to_f32(d[q] >> 16), acc[2 * q + 1]);
      }
    }
    if (n_shared && g == 0) {
      const uint32_t d[4] = {vs.x, vs.y, vs.z, vs.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf16_bits_to_f32(d[q] & 0xFFFFu);
        acc[2 * q + 1] += bf16_bits_to_f32(d[q] >> 16);
      }
    }
    *(uint4*)(z + ((size_t)t * G + g) * latent + c8 * 8) =
        make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                   pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
  }
}

template <int K>
static void launch_combine_k(dim3 grid, hipStream_t stream, const uint16_t* y, const int32_t* slot,
                             const float* w, const int32_t* idx, int T, int pairs, int latent,
                             int n_shared, int G, int epg, uint16_t* z) {
  hipLaunchKernelGGL(k_combine<K>, grid, dim3(256), 0, stream, y, slot, w, idx, T, pairs, latent,
                     n_shared, G, epg, z);
}

hipError_t launch_combine(const uint16_t* y, const int32_t* slot, const float* w,
                          const int32_t* idx, int T, int k, int pairs, int latent, int n_shared,
                          int n_groups, int experts_per_group, uint16_t* z, hipStream_t stream) {
  const long total = (long)T * (latent / 8);
  const dim3 grid((unsigned)((total + 255) / 256));
  const int G = n_groups < 1 ? 1 : n_groups;
  switch (k) {
#define MOE_COMBINE_CASE(KV)                                                                  \
    case KV:                                                                                  \
      launch_combine_k<KV>(grid, stream, y, slot, w, idx, T, pairs, latent, n_shared, G,     \
                           experts_per_group, z);                                             \
      break;
    MOE_COMBINE_CASE(1) MOE_COMBINE_CASE(2) MOE_COMBINE_CASE(3) MOE_COMBINE_CASE(4)
    MOE_COMBINE_CASE(5) MOE_COMBINE_CASE(6) MOE_COMBINE_CASE(7) MOE_COMBINE_CASE(8)
    MOE_COMBINE_CASE(9) MOE_COMBINE_CASE(10) MOE_COMBINE_CASE(11) MOE_COMBINE_CASE(12)
    MOE_COMBINE_CASE(13) MOE_COMBINE_CASE(14) MOE_COMBINE_CASE(15) MOE_COMBINE_CASE(16)
#undef MOE_COMBINE_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
