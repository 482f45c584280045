"""The latent-MoE layer forward, written from its definition (oracle; test
infrastructure only -- see the package docstring for who may call it).

Layer recipe (Hugging Face card "Edge0-145B . Q3_K", section "Architecture",
paragraph under the table; agentspulse tutorial, section "latent MoE
architecture"):

    h      = x D^T                                  D: [latent][hidden]
    l      = h R^T + b                              R: [E][latent]
    S, w   = top-k of softmax(l), renormalised      (reading: see gate_topk)
    y_t    = sum_j w_j SwiGLU_{S_j}(h_t) + SwiGLU_shared(h_t)
    out    = y U^T                                  U: [hidden][latent]

SwiGLU_e(v) = W_down (silu(W_gate v) * (W_up v)), each W dequantised from its
e2m1 codes, E4M3 block scales and fp32 matrix scale; silu(v) = v/(1+e^-v).

Routing groups (agentspulse tutorial, section "latent MoE architecture": a
layer holds eight D/U pairs, and a label on each expert names the pair it
uses; card, "Architecture" paragraph: the down projection is done per routing
group). With G groups, expert e belongs to group g(e) = e // (E/G) (any
labelling is this one after renumbering the experts), and

    h_g  = x D_g^T                                  for every group g
    l_e  = h_{g(e)} R_e^T + b_e
    z_g  = sum over the token's choices j in group g of w_j SwiGLU_{S_j}(h_g)
           (+ SwiGLU_shared(h_0) for g = 0: the shared expert belongs to group 0)
    out  = sum_g z_g U_g^T

G = 1 is the layer above.

Everything is float64. ``x``, ``D``, ``U`` and ``R`` are bf16 inputs,
widened exactly.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

from .formats import bf16_value, dequant_e1m1, dequant_fp4


def silu(v: np.ndarray) -> np.ndarray:
    """silu(v) = v * sigmoid(v) = v / (1 + exp(-v)) (the SwiGLU activation named
    by the card's architecture table, "SwiGLU width 640")."""
    return v / (1.0 + np.exp(-v))


def _bank_matrix(bank, proj: str, e: int) -> np.ndarray:
    m = getattr(bank, proj)
    dq = dequant_e1m1 if getattr(m, "bits", 4) == 3 else dequant_fp4
    return dq(m.codes[e], m.scales[e], m.gscale[e])


def swiglu_expert(v: np.ndarray, bank, e: int) -> np.ndarray:
    """One expert, latent -> inter -> latent, on rows v [n][latent].

    Card "Edge0-145B . Q3_K", section "Architecture": each expert runs
    latent -> 640 -> latent; table: "SwiGLU width 640". Reading: silu applies
    to the gate projection, no biases.
    """
    wg = _bank_matrix(bank, "gate", e)   # [inter][latent]
    wu = _bank_matrix(bank, "up", e)     # [inter][latent]
    wd = _bank_matrix(bank, "down", e)   # [latent][inter]
    a = silu(v @ wg.T) * (v @ wu.T)
    return a @ wd.T


# The shared expert's routing group (reading: the pages give the shared
# expert no group label; it runs on group 0's latent and adds into it).
SHARED_GROUP = 0


def group_latent(h: np.ndarray, g: int, latent: int) -> np.ndarray:
    """Group g's latent vectors: columns g*latent .. (g+1)*latent of h."""
    return h[..., g * latent:(g + 1) * latent]


def router_logits(h: np.ndarray, R: np.ndarray, b: np.ndarray, n_groups: int,
                  latent: int) -> np.ndarray:
    """l_e = h_{g(e)} R_e^T + b_e: each expert scored from its own group's
    latent, expert e in group e // (E / n_groups) (card, "Architecture": the
    router scores the experts from the latent; one group is the plain layer)."""
    E = R.shape[0]
    epg = E // n_groups
    logits = np.empty((h.shape[0], E))
    for g in range(n_groups):
        ex = slice(g * epg, (g + 1) * epg)
        logits[:, ex] = group_latent(h, g, latent) @ R[ex].T + b[ex]
    return logits


def gate_topk(logits32: np.ndarray, k: int):
    """Softmax over all E logits, the k largest, renormalised.

    The card ("Architecture" paragraph) says only that the router picks 10 of
    512 experts. Reading: S = the k largest logits in descending order, exact
    ties going to the lower expert index; p = softmax(l) over all E;
    w_j = p[S_j] / sum_{i in S} p[i]. No scaling factor, noise or capacity.

    ``logits32`` are float32 (the precision in which the choice is made);
    the softmax is evaluated in float64 from them.

    Returns idx int32 [T][k], w float64 [T][k], gap float64 [T] (the k-th
    largest logit minus the (k+1)-th; +inf when k == E).
    """
    l32 = np.asarray(logits32, dtype=np.float32)
    T, E = l32.shape
    order_index = np.broadcast_to(np.arange(E), (T, E))
    # sort by descending logit, then ascending expert index (stable lexsort:
    # the last key is primary)
    order = np.lexsort((order_index, -l32.astype(np.float64)), axis=-1)
    idx = order[:, :k].astype(np.int32)
    l64 = l32.astype(np.float64)
    m = l64.max(axis=1, keepdims=True)
    p = np.exp(l64 - m)
    p = p / p.sum(axis=1, keepdims=True)
    p_sel = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    w = p_sel / p_sel.sum(axis=1, keepdims=True)
    if k < E:
        sorted_l = np.take_along_axis(l64, order, axis=1)
        gap = sorted_l[:, k - 1] - sorted_l[:, k]
    else:
        gap = np.full((T,), np.inf)
    return idx, w, gap


def route_bookkeeping(idx: np.ndarray, n_experts: int):
    """Token-to-expert histogram, exclusive prefix sum and stable permutation.

    Pair p = t*k + j is the j-th choice of token t. counts[e] = number of pairs
    routed to e (sums to T*k); offsets = [0, cumsum(counts)] (E+1 entries);
    perm lists the pairs grouped by expert, ascending p within an expert
    (a counting sort written out), so perm[offsets[e]:offsets[e+1]] are e's
    pairs.
    """
    flat = np.asarray(idx, dtype=np.int64).ravel()
    counts = np.zeros(n_experts, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    cursor = offsets[:-1].copy()
    perm = np.empty(flat.size, dtype=np.int64)
    for p, e in enumerate(flat):
        perm[cursor[e]] = p
        cursor[e] += 1
    return counts.astype(np.int32), offsets.astype(np.int32), perm.astype(np.int32)


@dataclass
class OracleResult:
    h: np.ndarray            # float64 [T][G*latent] (G routing groups; G = 1: [T][latent])
    logits: np.ndarray       # float64 [T][E]
    logits32: np.ndarray     # float32 [T][E] (the values the choice is made on)
    idx: np.ndarray          # int32 [T][k]
    w: np.ndarray            # float64 [T][k]
    gap: np.ndarray          # float64 [T]
    counts: np.ndarray       # int32 [E]
    offsets: np.ndarray      # int32 [E+1]
    perm: np.ndarray         # int32 [T*k]
    tokens: np.ndarray       # int64 [Ts]: tokens whose outputs were computed
    z: np.ndarray            # float64 [Ts][G*latent]: combined expert output
    out: np.ndarray          # float64 [Ts][hidden]


def forward(layer, x_bits: Optional[np.ndarray] = None, tokens: Optional[Sequence[int]] = None,
            x_values: Optional[np.ndarray] = None) -> OracleResult:
    """Forward of one latent-MoE layer.

    ``x_bits``: bf16 bit patterns [T][hidden] (default: none; pass x_values
    for float64 inputs). Routing is computed for every token; the expert
    part and the output only for ``tokens`` (default: all).
    """
    d = layer.dims
    if x_values is None:
        x = bf16_value(x_bits)
    else:
        x = np.asarray(x_values, dtype=np.float64)
    T = x.shape[0]
    L = d.latent
    G = getattr(d, "n_groups", 1)
    epg = d.n_experts // G           # experts per routing group
    D = bf16_value(layer.D)          # [G*latent][hidden]: D_g = rows g*latent ..
    U = bf16_value(layer.U)          # [hidden][G*latent]: U_g = columns g*latent ..
    R = bf16_value(layer.R)
    b = (np.zeros(d.n_experts) if layer.bias is None
         else np.asarray(layer.bias, dtype=np.float32).astype(np.float64))

    # D projects each token down to the latent width (card, "Architecture");
    # with routing groups, through every group's D_g (the card's per-group
    # down projection), group g's latent in columns g*latent .. of h.
    h = x @ D.T
    # The router scores every expert from the latent vector (of the expert's
    # group: expert e belongs to group e // (n_experts / G)).
    logits = router_logits(h, R, b, G, L)
    logits32 = logits.astype(np.float32)
    idx, w, gap = gate_topk(logits32, d.top_k)
    counts, offsets, perm = route_bookkeeping(idx, d.n_experts)

    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    hs = h[tok]
    # Combined expert output: weighted routed experts plus the shared expert,
    # which the card places beside the routed ones, with weight 1. Each expert
    # reads and adds into its own group's latent; the shared expert belongs
    # to group 0.
    z = np.zeros((tok.size, G * L))
    sel_idx = idx[tok]
    for e in np.unique(sel_idx):
        rows, js = np.nonzero(sel_idx == e)
        g = int(e) // epg
        ye = swiglu_expert(group_latent(hs[rows], g, L), layer.experts, int(e))
        group_latent(z, g, L)[rows] += w[tok[rows], js][:, None] * ye
    if d.n_shared:
        group_latent(z, SHARED_GROUP, L)[:] += swiglu_expert(group_latent(hs, SHARED_GROUP, L),
                                                             layer.shared, 0)
    # U projects the combined result back to the hidden width (summed over
    # the groups' U_g).
    out = z @ U.T
    return OracleResult(h=h, logits=logits, logits32=logits32, idx=idx, w=w, gap=gap,
                        counts=counts, offsets=offsets, perm=perm, tokens=tok, z=z, out=out)


def rmsnorm(x: np.ndarray, weight: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * weight, per row. The pages name a final
    norm in the model stack (card, "Architecture": token embedding, 48 layers,
    final norm, lm_head) but no norm inside the MoE block; the residual block
    here is a reading for the stacked workload."""
    x = np.asarray(x, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    return x * r * np.asarray(weight, dtype=np.float64)


def block_forward(layer, x_bits: np.ndarray, eps: float = 1e-6,
                  tokens: Optional[Sequence[int]] = None):
    """Residual block: x + MoE(u), u = rmsnorm(x) * g. The layer's input is a
    bf16 tensor (its interface type), so u enters the layer rounded to bf16
    (nearest even). Returns (float64 output rows for ``tokens``, the
    OracleResult of the MoE)."""
    x = bf16_value(x_bits)
    u_bits = _to_bf16_bits(rmsnorm(x, layer.norm_w, eps))
    res = forward(layer, u_bits, tokens=tokens)
    return x[res.tokens] + res.out, res


def _to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns, round to nearest even: bf16 keeps 8
    significant bits, so the quantum at v = f * 2^e (f in [0.5, 1)) is
    2^(e-8); np.rint rounds halves to even."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    quantum = np.ldexp(1.0, e - 8)
    q = np.rint(v / quantum) * quantum          # exactly representable in bf16
    return (q.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def stack_forward(layers: List, x_bits: np.ndarray, eps: float = 1e-6):
    """Stacked residual blocks. The residual stream between blocks is a bf16
    tensor (the layer interface's activation type), so each block's output is
    rounded to bf16 before it feeds the next. Returns the list of bf16 block
    inputs x_0..x_n (x_n is the stack output) and the per-block results."""
    xs = [np.asarray(x_bits, dtype=np.uint16)]
    results = []
    for layer in layers:
        y, res = block_forward(layer, xs[-1], eps)
        xs.append(_to_bf16_bits(y))
        results.append(res)
    return xs, results


def expert_record_bytes(latent: int, inter: int, block: int = 16,
                        with_matrix_scales: bool = False, gateup_bits: int = 4) -> int:
    """Bytes of one expert (gate, up, down): gate and up codes of
    ``gateup_bits`` (4: e2m1, 3: E1M1) and 4-bit down codes, plus one E4M3
    byte per ``block`` weights; optionally the three fp32 matrix scales."""
    n = 3 * latent * inter
    code_bits = 2 * latent * inter * gateup_bits + latent * inter * 4
    return code_bits // 8 + n // block + (12 if with_matrix_scales else 0)


def param_counts(n_layers: int, n_experts: int, top_k: int, latent: int, inter: int):
    """(expert pool parameters, active routed-expert parameters per token):
    each expert holds gate and up [inter][latent] and down [latent][inter]."""
    per_expert = 3 * latent * inter
    return n_layers * n_experts * per_expert, n_layers * top_k * per_expert
