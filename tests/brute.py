"""Independent brute-force evaluation of the latent-MoE layer, used to pin the
oracle. It shares no code with ``oracle/``: the number formats are decoded a
different way (e2m1 by lookup in the OCP table of magnitudes, E4M3 through
torch's float8_e4m3fn dtype, bf16 through torch's bfloat16 dtype) and the
layer runs token by token, expert by expert, with Python loops over rows and
torch float64 dot products. With routing groups, each expert's logit and
output use its own group's latent (label e * G // E), the shared expert
group 0's, and the output is the sum of the per-group up projections. Only
for small shapes."""
from __future__ import annotations

import math

import numpy as np
import torch

# OCP Microscaling Formats v1.0, FP4 E2M1: magnitudes of codes 0..7 (bit 3 is
# the sign).
E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
_E2M1_SIGNED = torch.tensor(E2M1_MAGNITUDES + [-v for v in E2M1_MAGNITUDES],
                            dtype=torch.float64)


def bf16_to_f64(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64)


def e4m3_to_f64(b: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64)


def fp4_matrix(codes: np.ndarray, scales: np.ndarray, gscale: float) -> torch.Tensor:
    """[n][k/2] packed codes (low nibble = even column) -> float64 [n][k]."""
    c = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).to(torch.int64)
    n, half = c.shape
    nib = torch.stack([c & 0xF, c >> 4], dim=-1).reshape(n, 2 * half)
    vals = _E2M1_SIGNED[nib]
    sc = e4m3_to_f64(scales).repeat_interleave(16, dim=1)
    return vals * sc * float(gscale)


E1M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5]


def e1m1_matrix(codes: np.ndarray, scales: np.ndarray, gscale: float) -> torch.Tensor:
    """[n][3k/8] 12-byte chunks (three little-endian 32-bit words; elements
    0..23 as e2m1 nibbles with bit 2 clear, element 24 + p spread over bit
    4p + 2 of the three words: mantissa, exponent, sign) -> float64 [n][k],
    decoded element by element with Python integers."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    n, nb = c.shape
    k = nb // 12 * 32
    vals = torch.empty((n, k), dtype=torch.float64)
    for r in range(n):
        row = bytes(c[r])
        for ch in range(nb // 12):
            w = [int.from_bytes(row[12 * ch + 4 * j:12 * ch + 4 * j + 4], "little") for j in range(3)]
            for i in range(32):
                if i < 24:
                    nib = (w[i // 8] >> (4 * (i % 8))) & 0xF   # bit 2: element 24 + i % 8
                    neg, idx = nib >> 3, nib & 3
                else:
                    sh = 4 * (i - 24) + 2
                    neg = (w[2] >> sh) & 1
                    idx = (((w[1] >> sh) & 1) << 1) | ((w[0] >> sh) & 1)
                v = E1M1_MAGNITUDES[idx]
                vals[r, 32 * ch + i] = -v if neg else v
    sc = e4m3_to_f64(scales).repeat_interleave(16, dim=1)
    return vals * sc * float(gscale)


def quant_matrix(m, e: int) -> torch.Tensor:
    """Matrix e of a quantised set, in whichever element format it holds."""
    f = e1m1_matrix if getattr(m, "bits", 4) == 3 else fp4_matrix
    return f(m.codes[e], m.scales[e], float(m.gscale[e]))


class BruteLayer:
    def __init__(self, layer):
        self.layer = layer
        self._cache = {}

    def expert(self, bank_name: str, e: int):
        key = (bank_name, e)
        if key not in self._cache:
            bank = getattr(self.layer, bank_name)
            mats = []
            for proj in ("gate", "up", "down"):
                mats.append(quant_matrix(getattr(bank, proj), e))
            self._cache[key] = mats
        return self._cache[key]


def silu(v: float) -> float:
    return v / (1.0 + math.exp(-v))


def run_expert(bl: BruteLayer, bank_name: str, e: int, h: torch.Tensor) -> torch.Tensor:
    wg, wu, wd = bl.expert(bank_name, e)
    inter = wg.shape[0]
    a = torch.empty(inter, dtype=torch.float64)
    for i in range(inter):
        g = float(torch.dot(wg[i], h))
        u = float(torch.dot(wu[i], h))
        a[i] = silu(g) * u
    return torch.mv(wd, a)


def brute_forward(layer, x_bits: np.ndarray = None, x_values=None):
    """Returns (out [T][hidden] float64, idx [T][k], w [T][k], logits32 [T][E])."""
    d = layer.dims
    x = bf16_to_f64(x_bits) if x_values is None else torch.as_tensor(x_values, dtype=torch.float64)
    D = bf16_to_f64(layer.D)
    U = bf16_to_f64(layer.U)
    R = bf16_to_f64(layer.R)
    b = (torch.zeros(d.n_experts, dtype=torch.float64) if layer.bias is None
         else torch.from_numpy(np.asarray(layer.bias, dtype=np.float32)).to(torch.float64))
    bl = BruteLayer(layer)
    T = x.shape[0]
    L = d.latent
    G = getattr(d, "n_groups", 1)
    group = [e * G // d.n_experts for e in range(d.n_experts)]   # the expert's label
    Dg = [D[g * L:(g + 1) * L] for g in range(G)]                 # D_g [latent][hidden]
    Ug = [U[:, g * L:(g + 1) * L] for g in range(G)]              # U_g [hidden][latent]
    outs, idxs, ws, logits_all = [], [], [], []
    for t in range(T):
        hg = [torch.mv(Dg[g], x[t]) for g in range(G)]
        logits = torch.tensor([float(torch.dot(R[e], hg[group[e]])) for e in range(d.n_experts)],
                              dtype=torch.float64) + b
        l32 = logits.to(torch.float32).to(torch.float64).tolist()
        logits_all.append(l32)
        order = sorted(range(d.n_experts), key=lambda e: (-l32[e], e))
        sel = order[: d.top_k]
        mx = max(l32)
        ex = [math.exp(v - mx) for v in l32]
        tot = sum(ex)
        p = [v / tot for v in ex]
        ps = sum(p[e] for e in sel)
        w = [p[e] / ps for e in sel]
        zg = [torch.zeros(L, dtype=torch.float64) for _ in range(G)]
        for j, e in enumerate(sel):
            zg[group[e]] += w[j] * run_expert(bl, "experts", e, hg[group[e]])
        if d.n_shared:
            zg[0] += run_expert(bl, "shared", 0, hg[0])
        out_t = torch.zeros(U.shape[0], dtype=torch.float64)
        for g in range(G):
            out_t += torch.mv(Ug[g], zg[g])
        outs.append(out_t)
        idxs.append(sel)
        ws.append(w)
    return (torch.stack(outs).numpy(), np.array(idxs, dtype=np.int32), np.array(ws),
            np.array(logits_all))
