// Host side of the latent-MoE layer library: argument validation, workspace
// layout and the launch sequence (see include/moe_latent.h for the contract).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <mutex>
#include <string>

#include "kernels.hpp"
#include "moe_latent.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Routing groups of D/U (dims.n_groups, 0 meaning 1).
int groups_of(const moe_latent_dims& d) { return d.n_groups > 1 ? d.n_groups : 1; }

// Upper bound on the grouped path's 128-row m-tiles: full tiles of all
// pairs, one partial tile per expert that has pairs, the shared expert's.
int64_t max_mtiles(const moe_latent_dims& d, int64_t T) {
  const int64_t P = T * d.top_k;
  return (P + 127) / 128 + (d.n_experts < P ? d.n_experts : P) + d.n_shared * ((T + 127) / 128);
}

// Byte offsets of the scratch buffers inside the workspace.
struct Layout {
  size_t u;         // bf16 [T][hidden]       RMSNorm output (residual block)
  size_t hcat;      // bf16 [T][G][2*latent]  latent vector per group: hi | lo halves
  size_t logits;    // fp32 [T][E]
  size_t idx;       // int32 [T][k]
  size_t w;         // fp32 [T][k]
  size_t chunk;     // int32 [n_chunks][E]    per-chunk histogram, then chunk bases
  size_t counts;    // int32 [E]
  size_t off;       // int32 [E + 2]
  size_t tile_off;  // int32 [E + 2]
  size_t ttab;      // int4 [max m-tiles]     the m-tiles listed
  size_t split;     // int32 [2][9]           each XCD's run of the tile list
  size_t perm;      // int32 [P]
  size_t slot;      // int32 [P]
  size_t act;       // bf16 [P + T*n_shared][inter]
  size_t y;         // bf16 [P + T*n_shared][latent]
  size_t z;         // bf16 [T][G*latent]
  // decode path (T <= kDecodeMaxT)
  size_t d_hhi, d_hlo;   // bf16 [T][G*latent]
  size_t d_h16, d_hflag; // fp16 [T][G*latent], int32 [G*latent/16]
  size_t d_logits;       // fp32 [2][T][E]
  size_t d_act;          // bf16 [1 + max_active][T][inter]
  size_t d_zfix;         // int64 [T][G*latent] (fixed point)
  size_t d_n_act, d_list, d_wtab;
  size_t total;
};

Layout layout_of(const moe_latent_dims& d, int64_t T) {
  const int64_t P = T * d.top_k;
  const int64_t nch = (P + moe::kRouteChunk - 1) / moe::kRouteChunk;
  const int64_t rows = P + T * d.n_shared;
  const int64_t GL = (int64_t)groups_of(d) * d.latent;  // latent columns over all groups
  Layout L;
  size_t at = 0;
  auto take = [&](int64_t bytes) {
    const size_t o = at;
    at = align256(at + (size_t)bytes);
    return o;
  };
  L.u = take(T * d.hidden * 2);
  L.hcat = take(T * 2 * GL * 2);
  L.logits = take(T * d.n_experts * 4);
  L.idx = take(P * 4);
  L.w = take(P * 4);
  L.chunk = take(nch * d.n_experts * 4);
  L.counts = take(d.n_experts * 4);
  L.off = take((d.n_experts + 2) * 4);
  L.tile_off = take((d.n_experts + 2) * 4);
  L.ttab = take(max_mtiles(d, T) * 16);
  L.split = take(2 * 9 * 4);
  L.perm = take(P * 4);
  L.slot = take(P * 4);
  L.act = take(rows * d.inter * 2);
  L.y = take(rows * d.latent * 2);
  L.z = take(T * GL * 2);
  if (T <= moe::kDecodeMaxT) {
    const int64_t max_act = d.n_experts < T * d.top_k ? d.n_experts : T * d.top_k;
    L.d_hhi = take(T * GL * 2);
    L.d_hlo = take(T * GL * 2);
    L.d_h16 = take(T * GL * 2);
    L.d_hflag = take(GL / 16 * 4 + 4);
    L.d_logits = take(2 * T * d.n_experts * 4);
    L.d_act = take((1 + max_act) * T * d.inter * 2);
    L.d_zfix = take(T * GL * 8);
    L.d_n_act = take(4);
    L.d_list = take(max_act * 4);
    L.d_wtab = take((1 + max_act) * T * 4);
  } else {
    L.d_hhi = L.d_hlo = L.d_h16 = L.d_hflag = L.d_logits = L.d_act = L.d_zfix = L.d_n_act =
        L.d_list = L.d_wtab = 0;
  }
  L.total = at;
  return L;
}

int check_dims(const moe_latent_dims* d) {
  if (!d) return fail(MOE_LATENT_EINVAL, "dims is NULL");
  if (d->hidden <= 0 || d->latent <= 0 || d->inter <= 0 || d->n_experts <= 0 || d->top_k <= 0)
    return fail(MOE_LATENT_EINVAL, "dims must be positive (hidden %d latent %d inter %d experts %d top_k %d)",
                d->hidden, d->latent, d->inter, d->n_experts, d->top_k);
  if (d->hidden % 32 || d->latent % 32 || d->inter % 32)
    return fail(MOE_LATENT_EUNSUPPORTED, "hidden, latent and inter must be multiples of 32 (%d, %d, %d)",
                d->hidden, d->latent, d->inter);
  if (d->n_experts > moe::kMaxExperts)
    return fail(MOE_LATENT_EUNSUPPORTED, "n_experts %d > %d", d->n_experts, moe::kMaxExperts);
  if (d->top_k > 16 || d->top_k > d->n_experts)
    return fail(MOE_LATENT_EUNSUPPORTED, "top_k %d must be <= 16 and <= n_experts %d", d->top_k,
                d->n_experts);
  if (d->n_shared != 0 && d->n_shared != 1)
    return fail(MOE_LATENT_EUNSUPPORTED, "n_shared must be 0 or 1 (got %d)", d->n_shared);
  if (d->n_groups < 0) return fail(MOE_LATENT_EINVAL, "n_groups must be >= 0 (got %d)", d->n_groups);
  if (d->n_groups > 1 && d->n_experts % d->n_groups)
    return fail(MOE_LATENT_EUNSUPPORTED, "n_groups %d must divide n_experts %d", d->n_groups,
                d->n_experts);
  return 0;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_set(const moe_fp4_experts* s, const char* name, int count) {
  if (!s) return fail(MOE_LATENT_EINVAL, "%s is NULL", name);
  if (s->count != count)
    return fail(MOE_LATENT_EINVAL, "%s->count is %d, expected %d", name, s->count, count);
  const moe_fp4_matrix* m[3] = {&s->gate, &s->up, &s->down};
  const char* mn[3] = {"gate", "up", "down"};
  for (int i = 0; i < 3; ++i) {
    if (!m[i]->codes || !m[i]->scales || !m[i]->gscale)
      return fail(MOE_LATENT_EINVAL, "%s->%s has a NULL pointer", name, mn[i]);
    if (!aligned(m[i]->codes, 16) || !aligned(m[i]->scales, 16) || !aligned(m[i]->gscale, 4))
      return fail(MOE_LATENT_EINVAL, "%s->%s: codes and scales must be 16-byte aligned", name, mn[i]);
  }
  return 0;
}

// Element format of a matrix: 4 (e2m1; 0 means 4) or 3 (E1M1); -1 otherwise.
int fmt_bits(const moe_fp4_matrix& m) {
  const int b = m.bits == 0 ? 4 : m.bits;
  return b == 3 || b == 4 ? b : -1;
}

// The gate/up format of an expert set (gate and up alike, down e2m1), or an
// error return.
int set_bits(const moe_fp4_experts* s, const char* name, int* bits) {
  const int g = fmt_bits(s->gate), u = fmt_bits(s->up), dn = fmt_bits(s->down);
  if (g < 0 || u < 0 || dn < 0)
    return fail(MOE_LATENT_EUNSUPPORTED, "%s: bits must be 0, 3 or 4 (gate %d, up %d, down %d)",
                name, s->gate.bits, s->up.bits, s->down.bits);
  if (g != u || dn != 4)
    return fail(MOE_LATENT_EUNSUPPORTED, "%s: gate and up need one format and down e2m1 "
                                         "(gate %d, up %d, down %d bits)", name, g, u, dn);
  *bits = g;
  return 0;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return pa < pb + nb && pb < pa + na;
}

moe::Fp4Set to_set(const moe_fp4_experts* s) {
  moe::Fp4Set r;
  r.gate = {s->gate.codes, s->gate.scales, s->gate.gscale};
  r.up = {s->up.codes, s->up.scales, s->up.gscale};
  r.down = {s->down.codes, s->down.scales, s->down.gscale};
  return r;
}

#define HIP_TRY(expr)                                                                 \
  do {                                                                                \
    hipError_t e_ = (expr);                                                           \
    if (e_ != hipSuccess)                                                             \
      return fail(MOE_LATENT_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_));    \
  } while (0)

int run_grouped(const moe_latent_dims& d, int T, const uint16_t* x, const uint16_t* D,
                const uint16_t* U, const moe_router* router, const moe_fp4_experts* experts,
                const moe_fp4_experts* shared, int gu_bits, uint16_t* out, char* ws, const Layout& L,
                moe_route_debug* dbg, const moe_latent_opts& o, hipStream_t st) {
  const int H = d.hidden, Lat = d.latent, E = d.n_experts, I = d.inter, k = d.top_k;
  const int P = T * k;
  const int nch = (P + moe::kRouteChunk - 1) / moe::kRouteChunk;
  uint16_t* u = (uint16_t*)(ws + L.u);
  uint16_t* hcat = (uint16_t*)(ws + L.hcat);
  float* logits = (float*)(ws + L.logits);
  int32_t* idx = (int32_t*)(ws + L.idx);
  float* w = (float*)(ws + L.w);
  int32_t* chunk = (int32_t*)(ws + L.chunk);
  int32_t* counts = (int32_t*)(ws + L.counts);
  int32_t* off = (int32_t*)(ws + L.off);
  int32_t* tile_off = (int32_t*)(ws + L.tile_off);
  int4* ttab = (int4*)(ws + L.ttab);
  int32_t* split = (int32_t*)(ws + L.split);
  int32_t* perm = (int32_t*)(ws + L.perm);
  int32_t* slot = (int32_t*)(ws + L.slot);
  uint16_t* act = (uint16_t*)(ws + L.act);
  uint16_t* y = (uint16_t*)(ws + L.y);
  uint16_t* z = (uint16_t*)(ws + L.z);

  const int G = groups_of(d), epg = E / G;
  const moe::StageMarks sm{o.stage_events, st};
  // S0 (residual block only): pre-norm.
  const uint16_t* a_in = x;
  if (o.residual) {
    HIP_TRY(sm.mark(moe::kStageNorm, 0));
    HIP_TRY(moe::launch_rmsnorm(x, o.norm_weight, o.norm_eps, u, T, H, st));
    HIP_TRY(sm.mark(moe::kStageNorm, 1));
    a_in = u;
  }
  // S1: h = x D^T (every group's D_g), stored per group as bf16 hi | lo.
  moe::DenseEpilogue ep{};
  ep.out = hcat;
  ep.ldo = 2 * G * Lat;
  ep.lo_off = Lat;
  ep.group_w = Lat;
  HIP_TRY(sm.mark(moe::kStageDproj, 0));
  const moe_packed_weights* gp = o.grouped_packed;
  const uint16_t* pD = gp ? (const uint16_t*)gp->D : nullptr;
  const uint16_t* pU = gp ? (const uint16_t*)gp->U : nullptr;
  const uint16_t* pR = gp ? (const uint16_t*)gp->R : nullptr;
  HIP_TRY(moe::launch_gemm_dense(moe::kEpiSplit, a_in, H, pD ? pD : D, H, H, T, G * Lat, H, ep,
                                 st, pD != nullptr));
  HIP_TRY(sm.mark(moe::kStageDproj, 1));
  // S2: logits = (hi + lo) R^T + b, as a GEMM over K = 2*latent with R read
  // twice; one per routing group (its experts read its latent).
  HIP_TRY(sm.mark(moe::kStageRouter, 0));
  const uint16_t* Rw = pR ? pR : router->w;
  for (int g = 0; g < G; ++g) {
    ep = moe::DenseEpilogue{};
    ep.out = logits + (size_t)g * epg;
    ep.ldo = E;
    ep.bias = router->bias ? router->bias + (size_t)g * epg : nullptr;
    HIP_TRY(moe::launch_gemm_dense(moe::kEpiLogits, hcat + (size_t)g * 2 * Lat, 2 * G * Lat,
                                   Rw + (size_t)g * epg * Lat, Lat, Lat, T, epg, 2 * Lat, ep, st,
                                   pR != nullptr));
  }
  HIP_TRY(sm.mark(moe::kStageRouter, 1));
  // S3: top-k + renormalised softmax weights.
  HIP_TRY(sm.mark(moe::kStageTopk, 0));
  HIP_TRY(moe::launch_topk(logits, T, E, k, idx, w, st));
  HIP_TRY(sm.mark(moe::kStageTopk, 1));
  // S4-S6: histogram, prefix sums, stable permutation.
  HIP_TRY(sm.mark(moe::kStageRoute, 0));
  HIP_TRY(moe::launch_route_hist(idx, P, E, chunk, st));
  HIP_TRY(moe::launch_route_scan(chunk, nch, E, P, T, d.n_shared, counts, off, tile_off, ttab,
                                 (I + 127) / 128, (Lat + 255) / 256, split, st));
  HIP_TRY(moe::launch_route_permute(idx, P, E, chunk, off, perm, slot, st));
  HIP_TRY(sm.mark(moe::kStageRoute, 1));
  // S7-S9: grouped expert GEMMs (routed groups, then the shared expert).
  moe::RouteView rv{tile_off, off, perm, E, d.n_shared, P, k, epg, 2 * Lat, ttab, split};
  moe::ExpertsView ex{};
  ex.packed = gp && gp->experts;
  ex.gateup_bits = gu_bits;
  ex.routed = to_set(ex.packed ? gp->experts : experts);
  if (d.n_shared) ex.shared = to_set(ex.packed ? gp->shared : shared);
  const int n_mtiles = (int)max_mtiles(d, T);
  HIP_TRY(sm.mark(moe::kStageGateup, 0));
  HIP_TRY(moe::launch_expert_gateup(hcat, 2 * G * Lat, rv, ex, act, I, Lat, n_mtiles, st));
  HIP_TRY(sm.mark(moe::kStageGateup, 1));
  HIP_TRY(sm.mark(moe::kStageDown, 0));
  HIP_TRY(moe::launch_expert_down(act, rv, ex, y, I, Lat, n_mtiles, st));
  HIP_TRY(sm.mark(moe::kStageDown, 1));
  // S10: weighted combine in fixed order.
  HIP_TRY(sm.mark(moe::kStageCombine, 0));
  HIP_TRY(moe::launch_combine(y, slot, w, idx, T, k, P, Lat, d.n_shared, G, epg, z, st));
  HIP_TRY(sm.mark(moe::kStageCombine, 1));
  // S11: out = z U^T (+ x for the residual block).
  ep = moe::DenseEpilogue{};
  ep.out = out;
  ep.ldo = H;
  if (o.residual) {
    ep.resid = x;
    ep.ldr = H;
  }
  HIP_TRY(sm.mark(moe::kStageUproj, 0));
  HIP_TRY(moe::launch_gemm_dense(moe::kEpiOut, z, G * Lat, pU ? pU : U, G * Lat, G * Lat, T, H,
                                 G * Lat, ep, st, pU != nullptr));
  HIP_TRY(sm.mark(moe::kStageUproj, 1));

  if (dbg) {
    if (dbg->topk_idx) HIP_TRY(hipMemcpyAsync(dbg->topk_idx, idx, (size_t)P * 4, hipMemcpyDeviceToDevice, st));
    if (dbg->topk_w) HIP_TRY(hipMemcpyAsync(dbg->topk_w, w, (size_t)P * 4, hipMemcpyDeviceToDevice, st));
    if (dbg->counts) HIP_TRY(hipMemcpyAsync(dbg->counts, counts, (size_t)E * 4, hipMemcpyDeviceToDevice, st));
    if (dbg->offsets) HIP_TRY(hipMemcpyAsync(dbg->offsets, off, (size_t)(E + 1) * 4, hipMemcpyDeviceToDevice, st));
    if (dbg->perm) HIP_TRY(hipMemcpyAsync(dbg->perm, perm, (size_t)P * 4, hipMemcpyDeviceToDevice, st));
    if (dbg->logits) HIP_TRY(hipMemcpyAsync(dbg->logits, logits, (size_t)T * E * 4, hipMemcpyDeviceToDevice, st));
  }
  return 0;
}

int run_decode(const moe_latent_dims& d, int T, const uint16_t* x, const uint16_t* D,
               const uint16_t* U, const moe_router* router, const moe_fp4_experts* experts,
               const moe_fp4_experts* shared, int gu_bits, uint16_t* out, char* ws, const Layout& L,
               moe_route_debug* dbg, const moe_latent_opts& o, hipStream_t st) {
  moe::DecodeArgs a{};
  const moe_packed_weights* dp = o.decode_packed;
  a.packed = dp != nullptr;
  a.gateup_bits = gu_bits;
  if (dp) {  // all members present (validated)
    D = (const uint16_t*)dp->D;
    U = (const uint16_t*)dp->U;
    experts = dp->experts;
    shared = dp->shared;
  }
  a.x = x;
  a.D = D;
  a.R = dp ? (const uint16_t*)dp->R : router->w;
  a.RD = dp ? (const uint16_t*)dp->RD : nullptr;
  a.U = U;
  a.bias = router->bias;
  a.norm_weight = o.residual ? o.norm_weight : nullptr;
  a.norm_eps = o.norm_eps;
  const moe::Fp4Set rs = to_set(experts);
  a.gate = rs.gate;
  a.up = rs.up;
  a.down = rs.down;
  if (d.n_shared) {
    const moe::Fp4Set ss = to_set(shared);
    a.sh_gate = ss.gate;
    a.sh_up = ss.up;
    a.sh_down = ss.down;
  }
  a.hidden = d.hidden;
  a.latent = d.latent;
  a.inter = d.inter;
  a.n_experts = d.n_experts;
  a.top_k = d.top_k;
  a.n_shared = d.n_shared;
  a.n_groups = groups_of(d);
  a.T = T;
  a.hhi = (uint16_t*)(ws + L.d_hhi);
  a.hlo = a.RD ? nullptr : (uint16_t*)(ws + L.d_hlo);
  a.h16 = a.n_groups == 1 ? (uint16_t*)(ws + L.d_h16) : nullptr;
  a.hflag = a.n_groups == 1 ? (int*)(ws + L.d_hflag) : nullptr;
  a.logits = (float*)(ws + L.d_logits);
  a.act = (uint16_t*)(ws + L.d_act);
  a.zfix = (unsigned long long*)(ws + L.d_zfix);
  a.route_n_act = (int*)(ws + L.d_n_act);
  a.route_list = (int*)(ws + L.d_list);
  a.route_wtab = (float*)(ws + L.d_wtab);
  a.max_active = d.n_experts < T * d.top_k ? d.n_experts : T * d.top_k;
  a.out = out;
  if (dbg) {
    a.dbg_idx = dbg->topk_idx;
    a.dbg_w = dbg->topk_w;
    a.dbg_counts = dbg->counts;
    a.dbg_offsets = dbg->offsets;
    a.dbg_perm = dbg->perm;
    a.dbg_logits = dbg->logits;
  }
  HIP_TRY(moe::launch_decode(a, st, moe::StageMarks{o.stage_events, st}));
  return 0;
}

}  // namespace

extern "C" {

int moe_latent_version(void) { return MOE_LATENT_ABI_VERSION; }

int moe_bf16_pack(const void* src, int32_t N, int32_t K, int32_t layout, void* dst, void* stream) {
  g_err.clear();
  if (layout != MOE_LATENT_PACK_GROUPED && layout != MOE_LATENT_PACK_DECODE)
    return fail(MOE_LATENT_EINVAL, "unknown packing layout %d", layout);
  if (!src || !dst) return fail(MOE_LATENT_EINVAL, "src and dst must be non-NULL");
  if (N <= 0 || K <= 0) return fail(MOE_LATENT_EINVAL, "N and K must be positive (%d, %d)", N, K);
  const int nm = layout == MOE_LATENT_PACK_GROUPED ? 32 : 16;
  const int km = layout == MOE_LATENT_PACK_GROUPED ? 64 : 32;
  if (N % nm || K % km)
    return fail(MOE_LATENT_EUNSUPPORTED, "this layout needs N a multiple of %d and K of %d (%d, %d)",
                nm, km, N, K);
  if (!aligned(src, 16) || !aligned(dst, 16))
    return fail(MOE_LATENT_EINVAL, "src and dst must be 16-byte aligned");
  const size_t n = (size_t)N * K * 2;
  if (overlaps(src, n, dst, n)) return fail(MOE_LATENT_EINVAL, "dst overlaps src");
  if (layout == MOE_LATENT_PACK_GROUPED)
    HIP_TRY(moe::launch_pack_bf16((const uint16_t*)src, N, K, (uint16_t*)dst, (hipStream_t)stream));
  else
    HIP_TRY(moe::launch_pack_bf16_decode((const uint16_t*)src, N, K, (uint16_t*)dst,
                                         (hipStream_t)stream));
  return 0;
}

int moe_fp4_pack(const moe_fp4_matrix* src, int32_t count, int32_t N, int32_t K, int32_t layout,
                 uint8_t* dst_codes, uint8_t* dst_scales, void* stream) {
  g_err.clear();
  if (layout != MOE_LATENT_PACK_GROUPED && layout != MOE_LATENT_PACK_DECODE)
    return fail(MOE_LATENT_EINVAL, "unknown packing layout %d", layout);
  if (!src || !src->codes || !src->scales || !dst_codes || !dst_scales)
    return fail(MOE_LATENT_EINVAL, "src, its codes and scales, and the destinations must be non-NULL");
  if (count < 0 || N <= 0 || K <= 0)
    return fail(MOE_LATENT_EINVAL, "count must be >= 0 and N, K positive (%d, %d, %d)", count, N, K);
  const int bits = fmt_bits(*src);
  if (bits < 0) return fail(MOE_LATENT_EUNSUPPORTED, "src->bits must be 0, 3 or 4 (%d)", src->bits);
  const int nm = layout == MOE_LATENT_PACK_GROUPED ? 32 : 16;
  const int km = layout == MOE_LATENT_PACK_GROUPED ? 64 : 128;
  if (N % nm || K % km)
    return fail(MOE_LATENT_EUNSUPPORTED, "this layout needs N a multiple of %d and K of %d (%d, %d)",
                nm, km, N, K);
  if (!aligned(src->codes, 16) || !aligned(src->scales, 16) || !aligned(dst_codes, 16) ||
      !aligned(dst_scales, 16))
    return fail(MOE_LATENT_EINVAL, "codes and scales must be 16-byte aligned");
  const size_t nc = (size_t)count * N * (K / 32) * (bits == 4 ? 16 : 12);
  const size_t ns = (size_t)count * N * (K / 16);
  if (overlaps(dst_codes, nc, src->codes, nc) || overlaps(dst_codes, nc, src->scales, ns) ||
      overlaps(dst_scales, ns, src->codes, nc) || overlaps(dst_scales, ns, src->scales, ns) ||
      overlaps(dst_codes, nc, dst_scales, ns))
    return fail(MOE_LATENT_EINVAL, "packed buffers overlap the source or each other");
  if (count == 0) return 0;
  if (layout == MOE_LATENT_PACK_GROUPED)
    HIP_TRY(moe::launch_pack_fp4(src->codes, src->scales, count, N, K, bits, dst_codes,
                                 dst_scales, (hipStream_t)stream));
  else
    HIP_TRY(moe::launch_pack_fp4_decode(src->codes, src->scales, count, N, K, bits, dst_codes,
                                        dst_scales, (hipStream_t)stream));
  return 0;
}

int moe_router_fold(const moe_latent_dims* dims, const void* D, const void* R, void* dst,
                    void* stream) {
  g_err.clear();
  int rc = check_dims(dims);
  if (rc) return rc;
  const moe_latent_dims& d = *dims;
  if (!D || !R || !dst) return fail(MOE_LATENT_EINVAL, "D, R and dst must be non-NULL");
  if (d.n_experts % 16 || d.hidden % 32)
    return fail(MOE_LATENT_EUNSUPPORTED, "the folded router needs n_experts a multiple of 16 and "
                                         "hidden of 32 (%d, %d)", d.n_experts, d.hidden);
  if (!aligned(D, 16) || !aligned(R, 16) || !aligned(dst, 16))
    return fail(MOE_LATENT_EINVAL, "D, R and dst must be 16-byte aligned");
  const size_t nd = (size_t)2 * d.n_experts * d.hidden * 2;
  if (overlaps(dst, nd, D, (size_t)groups_of(d) * d.latent * d.hidden * 2) ||
      overlaps(dst, nd, R, (size_t)d.n_experts * d.latent * 2))
    return fail(MOE_LATENT_EINVAL, "dst overlaps D or R");
  HIP_TRY(moe::launch_router_fold((const uint16_t*)R, (const uint16_t*)D, d.n_experts, d.latent,
                                  d.hidden, groups_of(d), (uint16_t*)dst, (hipStream_t)stream));
  return 0;
}

const char* moe_latent_last_error(void) { return g_err.c_str(); }

size_t moe_latent_workspace_bytes(const moe_latent_dims* dims, int64_t T) {
  if (check_dims(dims) != 0 || T <= 0) return 0;
  if (T * dims->top_k >= ((int64_t)1 << 31)) return 0;
  return layout_of(*dims, T).total;
}

}  // extern "C"

namespace {

// Scratch of the allocation-free entry point: one array per device (each
// device that loads the library's code object holds its own copy until the
// process ends). Host code never names it as an address: its device
// address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = MOE_LATENT_NOALLOC_MAX_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The scratch array's device address on the calling thread's current device
// (looked up on the first call on that device), or nullptr with the error
// set.
void* scratch_address() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    fail(MOE_LATENT_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    return nullptr;
  }
  static std::mutex mu;
  static std::map<int, void*> by_device;
  std::lock_guard<std::mutex> lock(mu);
  const auto it = by_device.find(dev);
  if (it != by_device.end()) return it->second;
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr) {
    fail(MOE_LATENT_EHIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
         hipGetErrorString(e));
    return nullptr;
  }
  by_device[dev] = ptr;
  return ptr;
}

// Validation and dispatch shared by the entry points. noalloc: the
// workspace arguments are ignored and the device's scratch array is used.
int forward_impl(const moe_latent_dims* dims, int64_t T, const void* x, const void* D,
                 const void* U, const moe_router* router, const moe_fp4_experts* experts,
                 const moe_fp4_experts* shared, void* out, void* workspace,
                 size_t workspace_bytes, moe_route_debug* debug, const moe_latent_opts* opts,
                 void* stream, bool noalloc) {
  g_err.clear();
  int rc = check_dims(dims);
  if (rc) return rc;
  const moe_latent_dims& d = *dims;
  if (T < 0) return fail(MOE_LATENT_EINVAL, "T must be >= 0 (got %lld)", (long long)T);
  if (T * d.top_k >= ((int64_t)1 << 31))
    return fail(MOE_LATENT_EUNSUPPORTED, "T * top_k must be < 2^31");
  moe_latent_opts o{};
  if (opts) o = *opts;
  if (o.path < MOE_LATENT_PATH_AUTO || o.path > MOE_LATENT_PATH_DECODE)
    return fail(MOE_LATENT_EINVAL, "unknown path %d", o.path);
  if (o.path == MOE_LATENT_PATH_DECODE && T > MOE_LATENT_DECODE_MAX_T)
    return fail(MOE_LATENT_EUNSUPPORTED, "the decode path takes T <= %d (got %lld)",
                MOE_LATENT_DECODE_MAX_T, (long long)T);
  if (T == 0) return 0;  // nothing to do; buffers may be empty (NULL)
  const bool dec_ok = moe::decode_supported(d.hidden, d.latent, d.inter, d.n_experts, d.top_k,
                                            groups_of(d), (int)T);
  if (o.path == MOE_LATENT_PATH_DECODE && !dec_ok)
    return fail(MOE_LATENT_EUNSUPPORTED, "the decode path does not take these dims / T");
  const bool use_decode =
      o.path == MOE_LATENT_PATH_DECODE || (o.path == MOE_LATENT_PATH_AUTO && dec_ok);
  // plain weights the chosen path reads (the rest may be NULL: packed copies
  // stand in for them)
  const moe_packed_weights* gpk = use_decode ? nullptr : o.grouped_packed;
  const bool all_packed = use_decode && o.decode_packed;
  const bool need_D = !all_packed && !(gpk && gpk->D);
  const bool need_U = !all_packed && !(gpk && gpk->U);
  const bool need_R = !all_packed && !(gpk && gpk->R);
  const bool need_ex = !all_packed && !(gpk && gpk->experts);
  if (!x || !out) return fail(MOE_LATENT_EINVAL, "x and out must be non-NULL");
  if ((need_D && !D) || (need_U && !U))
    return fail(MOE_LATENT_EINVAL, "D and U must be non-NULL (no packed copy for this path)");
  if (!aligned(x, 16) || !aligned(out, 16) || (D && !aligned(D, 16)) || (U && !aligned(U, 16)))
    return fail(MOE_LATENT_EINVAL, "x, D, U and out must be 16-byte aligned");
  if (!router) return fail(MOE_LATENT_EINVAL, "router must be non-NULL");
  if (need_R && !router->w)
    return fail(MOE_LATENT_EINVAL, "router->w must be non-NULL (no packed copy for this path)");
  if ((router->w && !aligned(router->w, 16)) || (router->bias && !aligned(router->bias, 4)))
    return fail(MOE_LATENT_EINVAL, "router->w must be 16-byte aligned");
  if (need_ex || experts) {
    if ((rc = check_set(experts, "experts", d.n_experts))) return rc;
    if (d.n_shared && (rc = check_set(shared, "shared", d.n_shared))) return rc;
  }
  if (const moe_packed_weights* gp = o.grouped_packed) {
    if (gp->experts || gp->shared) {
      if (!gp->experts || (d.n_shared && !gp->shared))
        return fail(MOE_LATENT_EINVAL, "grouped_packed: experts and (with a shared expert) shared "
                                       "come together");
      if (d.latent % 64 || d.inter % 64)
        return fail(MOE_LATENT_EUNSUPPORTED, "grouped-packed experts need latent and inter "
                                             "multiples of 64 (%d, %d)", d.latent, d.inter);
      if ((rc = check_set(gp->experts, "grouped_packed->experts", d.n_experts))) return rc;
      if (d.n_shared && (rc = check_set(gp->shared, "grouped_packed->shared", d.n_shared)))
        return rc;
    }
    if ((gp->D && !aligned(gp->D, 16)) || (gp->U && !aligned(gp->U, 16)) ||
        (gp->R && !aligned(gp->R, 16)))
      return fail(MOE_LATENT_EINVAL, "grouped-packed D, U and R must be 16-byte aligned");
    if (gp->D && d.hidden % 64)
      return fail(MOE_LATENT_EUNSUPPORTED, "grouped-packed D needs hidden a multiple of 64 (%d)",
                  d.hidden);
    if ((gp->U || gp->R) && d.latent % 64)
      return fail(MOE_LATENT_EUNSUPPORTED, "grouped-packed U and R need latent a multiple of 64 "
                                           "(%d)", d.latent);
    if (gp->R && (d.n_experts / groups_of(d)) % 32)
      return fail(MOE_LATENT_EUNSUPPORTED, "grouped-packed R needs n_experts / n_groups a "
                                           "multiple of 32 (%d)", d.n_experts / groups_of(d));
  }
  if (const moe_packed_weights* dp = o.decode_packed) {
    if (!dp->experts || (d.n_shared && !dp->shared) || !dp->D || !dp->U || (!dp->R && !dp->RD))
      return fail(MOE_LATENT_EINVAL, "decode_packed needs experts, shared (n_shared = 1), D, U "
                                     "and R or RD");
    if (d.n_experts % 16)
      return fail(MOE_LATENT_EUNSUPPORTED, "decode-packed weights need n_experts a multiple of 16 "
                                           "(%d)", d.n_experts);
    if (!aligned(dp->D, 16) || !aligned(dp->U, 16) || (dp->R && !aligned(dp->R, 16)) ||
        (dp->RD && !aligned(dp->RD, 16)))
      return fail(MOE_LATENT_EINVAL, "decode-packed D, U, R and RD must be 16-byte aligned");
    if ((rc = check_set(dp->experts, "decode_packed->experts", d.n_experts))) return rc;
    if (d.n_shared && (rc = check_set(dp->shared, "decode_packed->shared", d.n_shared))) return rc;
  }
  // one gate/up format over every expert set given (routed, shared, copies)
  int gu_bits = 0;
  {
    const moe_fp4_experts* sets[6] = {experts, d.n_shared ? shared : nullptr};
    const char* names[6] = {"experts", "shared", "grouped_packed->experts",
                            "grouped_packed->shared", "decode_packed->experts",
                            "decode_packed->shared"};
    if (const moe_packed_weights* gp = o.grouped_packed) {
      sets[2] = gp->experts;
      sets[3] = d.n_shared ? gp->shared : nullptr;
    }
    if (const moe_packed_weights* dp = o.decode_packed) {
      sets[4] = dp->experts;
      sets[5] = d.n_shared ? dp->shared : nullptr;
    }
    for (int i = 0; i < 6; ++i) {
      if (!sets[i]) continue;
      int b = 0;
      if ((rc = set_bits(sets[i], names[i], &b))) return rc;
      if (gu_bits && b != gu_bits)
        return fail(MOE_LATENT_EUNSUPPORTED, "%s has %d-bit gate/up, an earlier set %d-bit",
                    names[i], b, gu_bits);
      gu_bits = b;
    }
    if (gu_bits == 3 && d.latent % 64)
      return fail(MOE_LATENT_EUNSUPPORTED, "E1M1 gate/up need latent a multiple of 64 (%d)",
                  d.latent);
  }
  if (o.residual) {
    if (!o.norm_weight) return fail(MOE_LATENT_EINVAL, "residual block needs norm_weight");
    if (!(o.norm_eps >= 0.0f)) return fail(MOE_LATENT_EINVAL, "norm_eps must be >= 0");
  }
  const size_t xbytes = (size_t)T * d.hidden * 2;
  if (overlaps(x, xbytes, out, xbytes)) return fail(MOE_LATENT_EINVAL, "out overlaps x");
  const Layout L = layout_of(d, T);
  if (noalloc) {
    if (L.total > kScratchBytes)
      return fail(MOE_LATENT_EWORKSPACE,
                  "this call needs %zu bytes of scratch; the allocation-free entry point "
                  "holds %zu (use moe_latent_forward_ex with a workspace)",
                  L.total, kScratchBytes);
    // every argument is valid: the first HIP call of this entry point
    workspace = scratch_address();
    if (!workspace) return MOE_LATENT_EHIP;
    workspace_bytes = kScratchBytes;
  }
  if (!workspace) return fail(MOE_LATENT_EINVAL, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(MOE_LATENT_EINVAL, "workspace must be 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(MOE_LATENT_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, L.total);
  if (overlaps(workspace, L.total, out, xbytes) || overlaps(workspace, L.total, x, xbytes))
    return fail(MOE_LATENT_EINVAL, "workspace overlaps x or out");

  if (use_decode)
    return run_decode(d, (int)T, (const uint16_t*)x, (const uint16_t*)D, (const uint16_t*)U,
                      router, experts, shared, gu_bits, (uint16_t*)out, (char*)workspace, L,
                      debug, o, (hipStream_t)stream);
  return run_grouped(d, (int)T, (const uint16_t*)x, (const uint16_t*)D, (const uint16_t*)U,
                     router, experts, shared, gu_bits, (uint16_t*)out, (char*)workspace, L, debug,
                     o, (hipStream_t)stream);
}

}  // namespace

extern "C" {

int moe_latent_forward_ex(const moe_latent_dims* dims, int64_t T, const void* x, const void* D,
                          const void* U, const moe_router* router,
                          const moe_fp4_experts* experts, const moe_fp4_experts* shared,
                          void* out, void* workspace, size_t workspace_bytes,
                          moe_route_debug* debug, const moe_latent_opts* opts, void* stream) {
  return forward_impl(dims, T, x, D, U, router, experts, shared, out, workspace, workspace_bytes,
                      debug, opts, stream, false);
}

int moe_latent_forward_noalloc(const moe_latent_dims* dims, int64_t T, const void* x,
                               const void* D, const void* U, const moe_router* router,
                               const moe_fp4_experts* experts, const moe_fp4_experts* shared,
                               void* out, moe_route_debug* debug, const moe_latent_opts* opts,
                               void* stream) {
  return forward_impl(dims, T, x, D, U, router, experts, shared, out, nullptr, 0, debug, opts,
                      stream, true);
}

int moe_latent_forward(const moe_latent_dims* dims, int64_t T, const void* x, const void* D,
                       const void* U, const moe_router* router,
                       const moe_fp4_experts* experts, const moe_fp4_experts* shared,
                       void* out, void* workspace, size_t workspace_bytes,
                       moe_route_debug* debug, void* stream) {
  return moe_latent_forward_ex(dims, T, x, D, U, router, experts, shared, out, workspace,
                               workspace_bytes, debug, nullptr, stream);
}

}  // extern "C"
