"""Seeded synthetic inputs for the latent-MoE layer.

This module is shared by the CPU oracle and the HIP path. It draws weights
and activations and quantises expert weights to the NVFP4-style format
(e2m1 codes, E4M3 per-16 block scales, one fp32 scale per matrix); it holds
none of the layer's arithmetic and decodes nothing.

Recipe (every stream is independent, so any tensor can be drawn alone):

* Philox4x32-10 counter-based generator, Box-Muller normals; element ``i`` of
  stream ``(seed, tag, sub)`` uses counter ``(i // 4, tag, sub)``.
* ``x`` ~ N(0, 1) rounded to bf16; ``D`` ~ N(0, 1/hidden), ``U`` ~ N(0, 1/latent),
  router ``R`` ~ N(0, 1/latent), all bf16.
* Expert gate/up ~ N(0, 1/latent), down ~ N(0, 1/inter), fp32, then quantised:
  ``gscale = amax / (6 * 448)``, block scale ``s = E4M3_rne(amax_b / (6 gscale))``,
  code ``= e2m1_rne(w / (s gscale))``.
* With ``Dims.gateup_bits = 3`` (the mixed 3/4-bit record) gate and up use
  3-bit E1M1 codes instead (magnitudes 0, 0.5, 1, 1.5; 6 replaced by 1.5 in
  the recipe above); down stays e2m1. Codes are stored per row as K/32
  chunks of 12 bytes, three little-endian 32-bit words w0, w1, w2: for
  g < 3, nibble p of w_g is element 8g + p as an e2m1 code (sign bit 3,
  exponent bit 1, mantissa bit 0) whose bit 2 carries one bit of element
  24 + p (mantissa in w0, exponent in w1, sign in w2).
* Router bias: zero, or the log of an unnormalised Zipf(s) prior,
  ``b_e = -s * ln(e + 1)`` ("hot experts").
* Routing groups (``Dims.n_groups`` = G): D [G*latent][hidden] and U
  [hidden][G*latent] drawn as one matrix each from the same streams.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_lib", "libsynth.so")
_SRC = os.path.join(_HERE, "csrc", "synth.c")

# Stream tags (one per tensor kind); ``sub`` is the expert index.
TAG_X, TAG_D, TAG_U, TAG_R = 1, 2, 3, 4
TAG_GATE, TAG_UP, TAG_DOWN = 5, 6, 7
TAG_SH_GATE, TAG_SH_UP, TAG_SH_DOWN = 8, 9, 10


def build_library(force: bool = False) -> str:
    """Compile the generator with gcc into ``synth/_lib/libsynth.so``."""
    if os.path.exists(_LIB_PATH) and not force:
        return _LIB_PATH
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    tmp = _LIB_PATH + f".tmp{os.getpid()}"
    subprocess.check_call(
        ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-D_GNU_SOURCE",
         _SRC, "-o", tmp, "-lm", "-lpthread"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_library()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, u32, i64, f32, ci = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                  ctypes.c_float, ctypes.c_int)
        vp = ctypes.c_void_p
        lib.synth_normal_f32.argtypes = [u64, u32, u32, f32, vp, i64, ci]
        lib.synth_normal_bf16.argtypes = [u64, u32, u32, f32, vp, i64, ci]
        lib.synth_fp4_bank.argtypes = [u64, u32, ctypes.c_int32, i64, i64, f32,
                                       vp, vp, vp, ci]
        lib.synth_quantize_fp4.argtypes = [vp, i64, i64, vp, vp, vp]
        lib.synth_e1m1_bank.argtypes = [u64, u32, ctypes.c_int32, i64, i64, f32,
                                        vp, vp, vp, ci]
        lib.synth_quantize_e1m1.argtypes = [vp, i64, i64, vp, vp, vp]
        lib.synth_f32_to_bf16.argtypes = [vp, vp, i64]
        lib.synth_philox4x32_10.argtypes = [vp, vp, vp]
        _lib = lib
    return _lib


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ------------------------------------------------------------------ primitives

def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.zeros(4, dtype=np.uint32)
    _load().synth_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def normal_f32(seed: int, tag: int, sub: int, shape, std: float = 1.0) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _load().synth_normal_f32(seed, tag, sub, std, _ptr(out), out.size, _threads())
    return out


def normal_bf16(seed: int, tag: int, sub: int, shape, std: float = 1.0) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(0, std^2) draws rounded to nearest even."""
    out = np.empty(shape, dtype=np.uint16)
    _load().synth_normal_bf16(seed, tag, sub, std, _ptr(out), out.size, _threads())
    return out


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().synth_f32_to_bf16(_ptr(a), _ptr(out), a.size)
    return out


# ------------------------------------------------------------------ containers

@dataclass
class Fp4Mat:
    """``count`` quantised matrices of shape [n][k].

    codes  uint8 [count][n][k/2] (bits 4: element 2j low nibble, 2j+1 high
           nibble) or [count][n][3k/8] (bits 3: E1M1, 12-byte chunks of 32
           elements, see the module docstring)
    scales uint8 [count][n][k/16] (E4M3fn bits, one per 16 consecutive k)
    gscale fp32  [count]
    """
    codes: np.ndarray
    scales: np.ndarray
    gscale: np.ndarray
    bits: int = 4

    @property
    def count(self) -> int:
        return self.codes.shape[0]


@dataclass
class Fp4Bank:
    gate: Fp4Mat  # [count][inter][latent]
    up: Fp4Mat    # [count][inter][latent]
    down: Fp4Mat  # [count][latent][inter]

    @property
    def count(self) -> int:
        return self.gate.count


@dataclass(frozen=True)
class Dims:
    hidden: int
    latent: int
    n_experts: int
    inter: int
    top_k: int
    n_shared: int = 1
    gateup_bits: int = 4   # 4: e2m1 gate/up; 3: E1M1 gate/up (down is e2m1 either way)
    n_groups: int = 1      # routing groups: one (D_g, U_g) pair per n_experts / n_groups experts


@dataclass
class Layer:
    """One latent-MoE layer's weights (host numpy).

    D uint16 [latent][hidden] bf16 bits, U uint16 [hidden][latent],
    R uint16 [n_experts][latent], bias fp32 [n_experts] or None,
    norm_w fp32 [hidden] (pre-norm weight, used by the residual block).
    With n_groups = G > 1: D is [G*latent][hidden] (group g's D_g = rows
    g*latent ..) and U is [hidden][G*latent] (U_g = columns g*latent ..).
    """
    dims: Dims
    D: np.ndarray
    U: np.ndarray
    R: np.ndarray
    bias: Optional[np.ndarray]
    experts: Fp4Bank
    shared: Optional[Fp4Bank]
    norm_w: Optional[np.ndarray] = None
    seed: int = 0


@dataclass(frozen=True)
class Config:
    name: str
    dims: Dims
    T: int
    seed: int = 0
    bias: str = "none"       # "none" | "zipf"
    zipf_s: float = 1.1
    n_layers: int = 1        # > 1: residual stack, layer l drawn with seed + l
    description: str = ""


def fp4_bank(seed: int, tags, count: int, latent: int, inter: int,
             gateup_bits: int = 4) -> Fp4Bank:
    tg, tu, td = tags
    lib = _load()

    def one(tag, n, k, std, bits=4):
        scales = np.empty((count, n, k // 16), dtype=np.uint8)
        gs = np.empty((count,), dtype=np.float32)
        if bits == 4:
            codes = np.empty((count, n, k // 2), dtype=np.uint8)
            lib.synth_fp4_bank(seed, tag, count, n, k, std, _ptr(codes), _ptr(scales),
                               _ptr(gs), _threads())
        else:
            assert bits == 3 and k % 32 == 0
            codes = np.empty((count, n, k // 32 * 12), dtype=np.uint8)
            lib.synth_e1m1_bank(seed, tag, count, n, k, std, _ptr(codes), _ptr(scales),
                                _ptr(gs), _threads())
        return Fp4Mat(codes, scales, gs, bits)

    return Fp4Bank(gate=one(tg, inter, latent, latent ** -0.5, gateup_bits),
                   up=one(tu, inter, latent, latent ** -0.5, gateup_bits),
                   down=one(td, latent, inter, inter ** -0.5))


def quantize_fp4(w: np.ndarray) -> Fp4Mat:
    """Quantise fp32 matrices [count][n][k] (or one [n][k]) with the recipe above."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    single = w.ndim == 2
    if single:
        w = w[None]
    count, n, k = w.shape
    assert k % 16 == 0
    codes = np.empty((count, n, k // 2), dtype=np.uint8)
    scales = np.empty((count, n, k // 16), dtype=np.uint8)
    gs = np.empty((count,), dtype=np.float32)
    lib = _load()
    for m in range(count):
        lib.synth_quantize_fp4(_ptr(w[m]), n, k, _ptr(codes[m]), _ptr(scales[m]),
                               gs[m:].ctypes.data)
    return Fp4Mat(codes, scales, gs)


def quantize_e1m1(w: np.ndarray) -> Fp4Mat:
    """Quantise fp32 matrices [count][n][k] (or one [n][k]) to E1M1 codes."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    single = w.ndim == 2
    if single:
        w = w[None]
    count, n, k = w.shape
    assert k % 32 == 0
    codes = np.empty((count, n, k // 32 * 12), dtype=np.uint8)
    scales = np.empty((count, n, k // 16), dtype=np.uint8)
    gs = np.empty((count,), dtype=np.float32)
    lib = _load()
    for m in range(count):
        lib.synth_quantize_e1m1(_ptr(w[m]), n, k, _ptr(codes[m]), _ptr(scales[m]),
                                gs[m:].ctypes.data)
    return Fp4Mat(codes, scales, gs, 3)


def zipf_bias(n_experts: int, s: float) -> np.ndarray:
    return (-s * np.log(np.arange(1, n_experts + 1, dtype=np.float64))).astype(np.float32)


def make_layer(dims: Dims, seed: int = 0, bias: str = "none", zipf_s: float = 1.1) -> Layer:
    H, L, E, I = dims.hidden, dims.latent, dims.n_experts, dims.inter
    G = dims.n_groups
    assert H % 32 == 0 and L % 32 == 0 and I % 32 == 0 and E % G == 0
    D = normal_bf16(seed, TAG_D, 0, (G * L, H), H ** -0.5)
    U = normal_bf16(seed, TAG_U, 0, (H, G * L), L ** -0.5)
    R = normal_bf16(seed, TAG_R, 0, (E, L), L ** -0.5)
    b = zipf_bias(E, zipf_s) if bias == "zipf" else None
    gb = dims.gateup_bits
    experts = fp4_bank(seed, (TAG_GATE, TAG_UP, TAG_DOWN), E, L, I, gb)
    shared = (fp4_bank(seed, (TAG_SH_GATE, TAG_SH_UP, TAG_SH_DOWN), 1, L, I, gb)
              if dims.n_shared else None)
    return Layer(dims=dims, D=D, U=U, R=R, bias=b, experts=experts, shared=shared,
                 norm_w=np.ones((H,), dtype=np.float32), seed=seed)


def make_x(T: int, hidden: int, seed: int = 0) -> np.ndarray:
    return normal_bf16(seed, TAG_X, 0, (T, hidden), 1.0)


# ------------------------------------------------------------------ workloads

E145 = Dims(hidden=2560, latent=1792, n_experts=512, inter=640, top_k=10, n_shared=1)
E120 = Dims(hidden=2560, latent=1280, n_experts=512, inter=640, top_k=10, n_shared=1)
TINY = Dims(hidden=256, latent=64, n_experts=16, inter=32, top_k=2, n_shared=1)

CONFIGS = {
    "tiny": Config("tiny", TINY, T=8, seed=0,
                   description="tiny layer T=8 H=256 l=64 E=16 I=32 top-2 + shared"),
    "decode145": Config("decode145", E145, T=4, seed=0,
                        description="145B-shaped layer, decode / verify window T=4"),
    "prefill145": Config("prefill145", E145, T=16384, seed=0, bias="zipf",
                         description="145B-shaped layer, 16K-token prefill, Zipf(1.1) router bias"),
    "prefill120": Config("prefill120", E120, T=4096, seed=0,
                         description="120B-shaped layer (l=1280), T=4096 prefill"),
    "stack145": Config("stack145", E145, T=8, seed=0, bias="zipf", n_layers=48,
                       description="48 residual blocks (RMSNorm + latent MoE), T=8, Zipf bias"),
    "grouped145": Config("grouped145", replace(E145, n_groups=8), T=4, seed=0,
                         description="145B-shaped layer with 8 routing groups of 64 experts, "
                                     "each with its own (D_g, U_g), decode T=4"),
    "grouped_tiny": Config("grouped_tiny", replace(TINY, n_groups=4), T=8, seed=0,
                           description="tiny layer with 4 routing groups of 4 experts"),
}


def make_config(name_or_cfg, T: Optional[int] = None):
    """Returns (layers, x) for a workload: ``layers`` is a list (one per block)."""
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    T = cfg.T if T is None else T
    layers = [make_layer(cfg.dims, cfg.seed + l, cfg.bias, cfg.zipf_s)
              for l in range(cfg.n_layers)]
    x = make_x(T, cfg.dims.hidden, cfg.seed)
    return layers, x


__all__ = [
    "Dims", "Config", "Layer", "Fp4Mat", "Fp4Bank", "CONFIGS", "E145", "E120", "TINY",
    "make_layer", "make_x", "make_config", "quantize_fp4", "quantize_e1m1", "normal_f32", "normal_bf16",
    "f32_to_bf16", "philox4x32_10", "zipf_bias", "fp4_bank", "build_library", "replace",
]
