"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare it with the oracle.

Bars (the layer's stated acceptance criteria):
* routing: expert sets, per-expert counts, offsets and the token order inside
  every expert's segment of the permutation are exact, excluding tokens whose
  oracle gap between the k-th and (k+1)-th largest logit is below 1e-4
  (their pairs are removed from both sides before counting); the GPU's own
  permutation must be exactly the stable counting sort of its own choices;
* gate weights: within 1e-5 absolute, matched by (token, expert);
* output: relative L2 error at most 2e-2 against the float64 oracle, over
  all compared rows and for every row on its own.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import latent_sparse_moe_amd as lsm
import oracle

NEAR_TIE = 1e-4
REL_L2 = 2e-2
W_ATOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device():
    return torch.device("cuda:0")


def to_dev_x(x_bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).to(dev)


def run_gpu(dlayer: lsm.DeviceLayer, x_bits: np.ndarray, path: int = lsm.PATH_AUTO,
            residual: bool = False, debug: bool = True):
    dev = device()
    x = to_dev_x(x_bits, dev)
    T = x.shape[0]
    dbg = lsm.RouteDebug.alloc(dlayer.dims, T, dev) if debug and T > 0 else None
    out = lsm.forward(x, dlayer, debug=dbg, path=path, residual=residual)
    torch.cuda.synchronize()
    res = {"out": out.float().cpu().numpy(), "out_bits": out.view(torch.int16).cpu().numpy()}
    if dbg is not None:
        for f in ("topk_idx", "topk_w", "counts", "offsets", "perm", "logits"):
            res[f] = getattr(dbg, f).cpu().numpy()
    return res


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def check_routing(ref: oracle.OracleResult, gpu: dict, k: int, E: int):
    T = ref.idx.shape[0]
    near = ref.gap < NEAR_TIE
    ok = ~near
    gi, gw = gpu["topk_idx"], gpu["topk_w"]
    # expert sets
    for t in np.nonzero(ok)[0]:
        assert set(gi[t].tolist()) == set(ref.idx[t].tolist()), (t, gi[t], ref.idx[t], ref.gap[t])
    # weights matched by expert
    for t in np.nonzero(ok)[0]:
        ow = dict(zip(ref.idx[t].tolist(), ref.w[t].tolist()))
        for e, w in zip(gi[t].tolist(), gw[t].tolist()):
            assert abs(w - ow[e]) <= W_ATOL, (t, e, w, ow[e])
    # the GPU's bookkeeping is exactly the stable counting sort of its own choices
    flat = gi.ravel().astype(np.int64)
    assert np.array_equal(gpu["counts"], np.bincount(flat, minlength=E))
    assert gpu["offsets"][0] == 0 and np.array_equal(np.diff(gpu["offsets"]), gpu["counts"])
    assert np.array_equal(gpu["perm"], np.argsort(flat, kind="stable"))
    # counts and segment contents against the oracle, near-tie tokens removed
    near_tok = np.nonzero(near)[0]
    adj_g = gpu["counts"] - np.bincount(gi[near_tok].ravel(), minlength=E)
    adj_o = ref.counts - np.bincount(ref.idx[near_tok].ravel(), minlength=E)
    assert np.array_equal(adj_g, adj_o), np.nonzero(adj_g != adj_o)
    for e in range(E):
        seg_g = gpu["perm"][gpu["offsets"][e]:gpu["offsets"][e + 1]] // k
        seg_o = ref.perm[ref.offsets[e]:ref.offsets[e + 1]] // k
        seg_g = seg_g[~near[seg_g]]
        seg_o = seg_o[~near[seg_o]]
        assert np.array_equal(seg_g, seg_o), (e, seg_g[:8], seg_o[:8])
    return int(near.sum())


def row_rel_l2(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Relative L2 error of each row of a against the same row of b."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b, axis=-1) / np.maximum(np.linalg.norm(b, axis=-1), 1e-300)


def check_output(ref: oracle.OracleResult, gpu_out: np.ndarray, tol: float = REL_L2):
    """Output rows for ref.tokens at the layer bar: the rows together, and
    every row on its own (so that one wrong row, such as the last row of a
    partial tile, cannot hide in the aggregate), near-tie tokens left out."""
    tok = ref.tokens
    got = gpu_out[tok]
    near = ref.gap[tok] < NEAR_TIE
    err_all = rel_l2(got, ref.out)
    err_ok = rel_l2(got[~near], ref.out[~near]) if (~near).any() else 0.0
    assert np.isfinite(got).all()
    assert err_ok <= tol, (err_ok, err_all)
    if (~near).any():
        rows = row_rel_l2(got[~near], ref.out[~near])
        worst = int(np.argmax(rows))
        assert rows[worst] <= tol, ("row", int(tok[~near][worst]), float(rows[worst]))
    return err_ok, err_all
