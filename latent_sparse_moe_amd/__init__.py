"""Python binding of the latent-MoE layer library (``include/moe_latent.h``).

Argument marshalling only: every step of the layer runs in the HIP kernels of
``_lib/libmoe_latent.so``. PyTorch provides device memory and the stream.
There is no fallback: if the library is missing, loading raises.

    layer = DeviceLayer.from_host(host_layer, device)     # weights to HBM
    out = forward(x, layer)                                # x: bf16 [T][hidden] on device
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LATENT_LIB names another build of the same library (the host-sanitizer copy)
LIB_PATH = os.environ.get("MOE_LATENT_LIB") or os.path.join(_HERE, "_lib", "libmoe_latent.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, -1, -2, -3, -4
PATH_AUTO, PATH_GROUPED, PATH_DECODE = 0, 1, 2
DECODE_MAX_T = 8

c_i32, c_i64, c_size, c_vp, c_f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float


class CDims(ctypes.Structure):
    _fields_ = [("hidden", c_i32), ("latent", c_i32), ("n_experts", c_i32), ("inter", c_i32),
                ("top_k", c_i32), ("n_shared", c_i32), ("n_groups", c_i32)]


class CFp4Matrix(ctypes.Structure):
    _fields_ = [("codes", c_vp), ("scales", c_vp), ("gscale", c_vp), ("bits", c_i32)]


class CFp4Experts(ctypes.Structure):
    _fields_ = [("gate", CFp4Matrix), ("up", CFp4Matrix), ("down", CFp4Matrix), ("count", c_i32)]


class CRouter(ctypes.Structure):
    _fields_ = [("w", c_vp), ("bias", c_vp)]


class CRouteDebug(ctypes.Structure):
    _fields_ = [("topk_idx", c_vp), ("topk_w", c_vp), ("counts", c_vp), ("offsets", c_vp),
                ("perm", c_vp), ("logits", c_vp)]


class CPackedWeights(ctypes.Structure):
    _fields_ = [("experts", ctypes.POINTER(CFp4Experts)), ("shared", ctypes.POINTER(CFp4Experts)),
                ("D", c_vp), ("U", c_vp), ("R", c_vp), ("RD", c_vp)]


class COpts(ctypes.Structure):
    _fields_ = [("path", c_i32), ("residual", c_i32), ("norm_weight", c_vp), ("norm_eps", c_f32),
                ("stage_events", ctypes.POINTER(c_vp)),
                ("grouped_packed", ctypes.POINTER(CPackedWeights)),
                ("decode_packed", ctypes.POINTER(CPackedWeights))]


PACK_GROUPED, PACK_DECODE = 1, 2


STAGES = ("norm", "dproj", "router", "topk", "route", "gateup", "down", "combine", "uproj")
N_STAGES = len(STAGES)


EXPORTS = ("moe_latent_forward", "moe_latent_forward_ex", "moe_latent_forward_noalloc",
           "moe_latent_workspace_bytes", "moe_latent_last_error", "moe_latent_version",
           "moe_fp4_pack", "moe_bf16_pack", "moe_router_fold")

_lib = None


def load_library(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with latent_sparse_moe_amd/build.py "
                           "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    fwd_args = [P(CDims), c_i64, c_vp, c_vp, c_vp, P(CRouter), P(CFp4Experts), P(CFp4Experts),
                c_vp, c_vp, c_size, P(CRouteDebug)]
    lib.moe_latent_forward.argtypes = fwd_args + [c_vp]
    lib.moe_latent_forward.restype = ctypes.c_int
    lib.moe_latent_forward_ex.argtypes = fwd_args + [P(COpts), c_vp]
    lib.moe_latent_forward_ex.restype = ctypes.c_int
    lib.moe_latent_forward_noalloc.argtypes = fwd_args[:9] + [P(CRouteDebug), P(COpts), c_vp]
    lib.moe_latent_forward_noalloc.restype = ctypes.c_int
    lib.moe_latent_workspace_bytes.argtypes = [P(CDims), c_i64]
    lib.moe_latent_workspace_bytes.restype = c_size
    lib.moe_latent_last_error.argtypes = []
    lib.moe_latent_last_error.restype = ctypes.c_char_p
    lib.moe_latent_version.argtypes = []
    lib.moe_latent_version.restype = ctypes.c_int
    lib.moe_fp4_pack.argtypes = [P(CFp4Matrix), c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp]
    lib.moe_fp4_pack.restype = ctypes.c_int
    lib.moe_bf16_pack.argtypes = [c_vp, c_i32, c_i32, c_i32, c_vp, c_vp]
    lib.moe_bf16_pack.restype = ctypes.c_int
    lib.moe_router_fold.argtypes = [P(CDims), c_vp, c_vp, c_vp, c_vp]
    lib.moe_router_fold.restype = ctypes.c_int
    _lib = lib
    return lib


class MoeLatentError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"moe_latent error {code}: {msg}")
        self.code = code


def _dims(d) -> CDims:
    return CDims(d.hidden, d.latent, d.n_experts, d.inter, d.top_k, d.n_shared,
                 getattr(d, "n_groups", 1))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


@dataclass
class DeviceFp4:
    codes: torch.Tensor   # uint8 [count][N][K/2] (E1M1: [count][N][3K/8])
    scales: torch.Tensor  # uint8 [count][N][K/16]
    gscale: torch.Tensor  # float32 [count]
    bits: int = 4         # 4: e2m1 codes, 3: E1M1

    def c(self) -> CFp4Matrix:
        return CFp4Matrix(self.codes.data_ptr(), self.scales.data_ptr(), self.gscale.data_ptr(),
                          self.bits)


@dataclass
class DeviceExperts:
    gate: DeviceFp4
    up: DeviceFp4
    down: DeviceFp4

    @property
    def count(self) -> int:
        return self.gate.codes.shape[0]

    def c(self) -> CFp4Experts:
        return CFp4Experts(self.gate.c(), self.up.c(), self.down.c(), self.count)


@dataclass
class DeviceLayer:
    """One layer's weights in device memory, laid out as moe_latent.h describes."""
    dims: object
    D: torch.Tensor                 # bf16 [G*latent][hidden] (G routing groups, default 1)
    U: torch.Tensor                 # bf16 [hidden][G*latent]
    R: torch.Tensor                 # bf16 [n_experts][latent]
    bias: Optional[torch.Tensor]    # float32 [n_experts]
    experts: DeviceExperts
    shared: Optional[DeviceExperts]
    norm_w: Optional[torch.Tensor] = None  # float32 [hidden]
    # packed copies of the weights for each path (moe_fp4_pack / moe_bf16_pack);
    # see pack()
    grouped_packed: Optional["PackedWeights"] = None
    decode_packed: Optional["PackedWeights"] = None

    def pack(self, grouped: bool = True, decode: bool = True,
             stream: Optional[torch.cuda.Stream] = None,
             fold_router: bool = True) -> "DeviceLayer":
        """Adds packed copies of the weights (same bytes, reordered so each
        wave's loads are contiguous). Grouped: each matrix whose dims allow
        it (experts: latent and inter % 64; D: hidden % 64; U: latent % 64;
        router rows: also n_experts % 32). Decode: every matrix, when the
        decode kernels take these dims and n_experts % 16 == 0, and (with
        fold_router) the router folded onto the residual width
        (moe_router_fold), which lets the decode path compute the logits
        from x beside h = x D^T."""
        d = self.dims
        if grouped:
            g = PackedWeights()
            if d.latent % 64 == 0 and d.inter % 64 == 0:
                g.experts = pack_experts(self.experts, d, PACK_GROUPED, stream)
                g.shared = (pack_experts(self.shared, d, PACK_GROUPED, stream)
                            if self.shared is not None else None)
            if d.hidden % 64 == 0:
                g.D = pack_bf16(self.D, PACK_GROUPED, stream)
            if d.latent % 64 == 0:
                g.U = pack_bf16(self.U, PACK_GROUPED, stream)
                if (d.n_experts // getattr(d, "n_groups", 1)) % 32 == 0:
                    g.R = pack_bf16(self.R, PACK_GROUPED, stream)
            self.grouped_packed = g
        if decode and d.hidden % 256 == 0 and d.latent % 256 == 0 and d.inter % 128 == 0 \
                and d.n_experts % 16 == 0:
            self.decode_packed = PackedWeights(
                pack_experts(self.experts, d, PACK_DECODE, stream),
                pack_experts(self.shared, d, PACK_DECODE, stream) if self.shared is not None else None,
                pack_bf16(self.D, PACK_DECODE, stream), pack_bf16(self.U, PACK_DECODE, stream),
                pack_bf16(self.R, PACK_DECODE, stream),
                fold_router_weights(d, self.D, self.R, stream) if fold_router else None)
        return self

    def drop_plain(self) -> "DeviceLayer":
        """Frees the plain weights once packed copies cover every path that
        will run (calls on a path without such copies then fail with
        EINVAL). The router bias and norm weight stay."""
        self.D = self.U = self.R = None
        self.experts = self.shared = None
        return self

    @staticmethod
    def from_host(h, device) -> "DeviceLayer":
        """Copy a host layer (numpy: bf16 as uint16 bits, fp4 codes/scales as
        uint8, scales fp32) to ``device``."""
        def bf16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

        def u8(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(device)

        def f32(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

        def bank(b):
            if b is None:
                return None
            return DeviceExperts(*[DeviceFp4(u8(getattr(b, p).codes), u8(getattr(b, p).scales),
                                             f32(getattr(b, p).gscale), getattr(b, p).bits)
                                   for p in ("gate", "up", "down")])

        return DeviceLayer(dims=h.dims, D=bf16(h.D), U=bf16(h.U), R=bf16(h.R),
                           bias=None if h.bias is None else f32(h.bias),
                           experts=bank(h.experts), shared=bank(h.shared),
                           norm_w=None if getattr(h, "norm_w", None) is None else f32(h.norm_w))


@dataclass
class PackedWeights:
    """Packed copies for one path (members None when not packed)."""
    experts: Optional[DeviceExperts] = None
    shared: Optional[DeviceExperts] = None
    D: Optional[torch.Tensor] = None
    U: Optional[torch.Tensor] = None
    R: Optional[torch.Tensor] = None
    RD: Optional[torch.Tensor] = None   # decode only: folded router (moe_router_fold)

    def c(self):
        """(CPackedWeights, objects to keep alive while it is used)."""
        ex = self.experts.c() if self.experts is not None else None
        sh = self.shared.c() if self.shared is not None else None
        cp = CPackedWeights(ctypes.pointer(ex) if ex is not None else None,
                            ctypes.pointer(sh) if sh is not None else None,
                            _ptr(self.D), _ptr(self.U), _ptr(self.R), _ptr(self.RD))
        return cp, (ex, sh)


def pack_fp4(m: DeviceFp4, N: int, K: int, layout: int = PACK_GROUPED,
             stream: Optional[torch.cuda.Stream] = None) -> DeviceFp4:
    """A packed copy of one fp4 matrix set [count][N][K] (moe_fp4_pack)."""
    lib = load_library()
    if stream is None:
        stream = torch.cuda.current_stream(m.codes.device)
    with torch.cuda.stream(stream):  # allocated on the stream the copy runs on
        codes = torch.empty_like(m.codes)
        scales = torch.empty_like(m.scales)
    src = m.c()
    rc = lib.moe_fp4_pack(ctypes.byref(src), m.codes.shape[0], N, K, layout, codes.data_ptr(),
                          scales.data_ptr(), stream.cuda_stream)
    if rc != 0:
        raise MoeLatentError(rc, lib.moe_latent_last_error().decode())
    return DeviceFp4(codes, scales, m.gscale, m.bits)


def pack_bf16(w: torch.Tensor, layout: int = PACK_GROUPED,
              stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """A packed copy of a bf16 matrix [N][K] (moe_bf16_pack)."""
    lib = load_library()
    if stream is None:
        stream = torch.cuda.current_stream(w.device)
    with torch.cuda.stream(stream):  # allocated on the stream the copy runs on
        out = torch.empty_like(w)
    rc = lib.moe_bf16_pack(w.data_ptr(), w.shape[0], w.shape[1], layout, out.data_ptr(),
                           stream.cuda_stream)
    if rc != 0:
        raise MoeLatentError(rc, lib.moe_latent_last_error().decode())
    return out


def fold_router_weights(dims, D: torch.Tensor, R: torch.Tensor,
                        stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """The router folded onto the residual width, W = R D, as bf16 hi and lo
    matrices in the decode-packed layout (moe_router_fold): bf16
    [2][n_experts][hidden]."""
    lib = load_library()
    if stream is None:
        stream = torch.cuda.current_stream(D.device)
    with torch.cuda.stream(stream):
        out = torch.empty((2, dims.n_experts, dims.hidden), dtype=torch.bfloat16, device=D.device)
    rc = lib.moe_router_fold(ctypes.byref(_dims(dims)), D.data_ptr(), R.data_ptr(), out.data_ptr(),
                             stream.cuda_stream)
    if rc != 0:
        raise MoeLatentError(rc, lib.moe_latent_last_error().decode())
    return out


def pack_experts(b: DeviceExperts, dims, layout: int = PACK_GROUPED, stream=None) -> DeviceExperts:
    L, I = dims.latent, dims.inter
    return DeviceExperts(pack_fp4(b.gate, I, L, layout, stream), pack_fp4(b.up, I, L, layout, stream),
                         pack_fp4(b.down, L, I, layout, stream))


def workspace_bytes(dims, T: int) -> int:
    return int(load_library().moe_latent_workspace_bytes(ctypes.byref(_dims(dims)), int(T)))


def alloc_workspace(dims, T: int, device) -> torch.Tensor:
    n = workspace_bytes(dims, T)
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


@dataclass
class RouteDebug:
    topk_idx: torch.Tensor
    topk_w: torch.Tensor
    counts: torch.Tensor
    offsets: torch.Tensor
    perm: torch.Tensor
    logits: torch.Tensor

    @staticmethod
    def alloc(dims, T: int, device) -> "RouteDebug":
        k, E = dims.top_k, dims.n_experts
        i32 = dict(dtype=torch.int32, device=device)
        return RouteDebug(torch.empty((T, k), **i32), torch.empty((T, k), dtype=torch.float32, device=device),
                          torch.empty((E,), **i32), torch.empty((E + 1,), **i32),
                          torch.empty((T * k,), **i32),
                          torch.empty((T, E), dtype=torch.float32, device=device))

    def c(self) -> CRouteDebug:
        return CRouteDebug(*[getattr(self, f).data_ptr() for f, _ in CRouteDebug._fields_])


def _check_rows(name: str, t, hidden: int) -> None:
    """t must be a contiguous 2-D bf16 CUDA tensor [T][hidden] (the layout the
    library reads and writes as row-major bf16)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor (got {type(t).__name__})")
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16 (got {t.dtype})")
    if t.dim() != 2 or t.shape[1] != hidden:
        raise ValueError(f"{name} must have shape [T][{hidden}] (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")


def _check_layer_device(layer: "DeviceLayer", dev: torch.device) -> None:
    for name in ("D", "U", "R", "bias", "norm_w"):
        t = getattr(layer, name)
        if t is not None and t.device != dev:
            raise ValueError(f"layer.{name} is on {t.device}, x on {dev}")
    for bank_name in ("experts", "shared"):
        b = getattr(layer, bank_name)
        if b is not None and b.gate.codes.device != dev:
            raise ValueError(f"layer.{bank_name} is on {b.gate.codes.device}, x on {dev}")


def _check_call(x, layer, out, workspace):
    d = layer.dims
    _check_rows("x", x, d.hidden)
    if out is not None:
        _check_rows("out", out, d.hidden)
        if out.shape != x.shape or out.device != x.device:
            raise ValueError(f"out must match x: shape {tuple(x.shape)} on {x.device} "
                             f"(got {tuple(out.shape)} on {out.device})")
    if workspace is not None:
        if workspace.dtype != torch.uint8 or not workspace.is_contiguous() \
                or workspace.device != x.device:
            raise ValueError("workspace must be a contiguous uint8 tensor on x's device")
    # devices last, so the layout checks above also run on host tensors
    if x.device.type != "cuda":
        raise ValueError(f"x must be on a CUDA (HIP) device (got {x.device})")
    _check_layer_device(layer, x.device)


def _call_args(x, layer, out, debug, path, residual, norm_eps, stage_events):
    """ctypes arguments shared by the forward entry points (up to and
    excluding out / workspace), plus the objects they point into."""
    d = layer.dims
    router = CRouter(_ptr(layer.R), _ptr(layer.bias))
    ex = layer.experts.c() if layer.experts is not None else None
    sh = layer.shared.c() if layer.shared is not None else None
    ev_arr = None
    if stage_events:
        ev_arr = (c_vp * (2 * N_STAGES))()
        for name, (a, b) in stage_events.items():
            i = STAGES.index(name)
            ev_arr[2 * i] = a.cuda_event
            ev_arr[2 * i + 1] = b.cuda_event
    gp = layer.grouped_packed.c() if layer.grouped_packed is not None else None
    dp = layer.decode_packed.c() if layer.decode_packed is not None else None
    opts = COpts(path, 1 if residual else 0, _ptr(layer.norm_w) if residual else None, norm_eps,
                 ev_arr, ctypes.pointer(gp[0]) if gp is not None else None,
                 ctypes.pointer(dp[0]) if dp is not None else None)
    dbg = debug.c() if debug is not None else None
    head = (ctypes.byref(_dims(d)), x.shape[0], x.data_ptr(), _ptr(layer.D), _ptr(layer.U),
            ctypes.byref(router), ctypes.byref(ex) if ex is not None else None,
            ctypes.byref(sh) if sh is not None else None)
    keep = (router, ex, sh, ev_arr, gp, dp, opts, dbg)
    return head, (ctypes.byref(dbg) if dbg is not None else None), ctypes.byref(opts), keep


def forward(x: torch.Tensor, layer: DeviceLayer, *, out: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None, debug: Optional[RouteDebug] = None,
            path: int = PATH_AUTO, residual: bool = False, norm_eps: float = 1e-6,
            stream: Optional[torch.cuda.Stream] = None, stage_events=None) -> torch.Tensor:
    """out = MoE(x) (or x + MoE(rmsnorm(x) * norm_w) with residual=True),
    enqueued on ``stream`` (default: torch's current stream)
    (moe_latent_forward_ex).

    x (and ``out`` when given) must be contiguous bf16 [T][hidden] tensors on
    one CUDA device; ``workspace`` a contiguous uint8 tensor on that device.
    Buffers this call allocates (``out``, the workspace) come from torch's
    allocator on ``stream``, so the allocator does not hand them to other
    work before the kernels enqueued on ``stream`` are done with them.

    ``stage_events``: optional dict {stage name: (start, end)} of
    torch.cuda.Event(enable_timing=True), recorded around that stage's
    kernels on ``stream``."""
    lib = load_library()
    _check_call(x, layer, out, workspace)
    T = x.shape[0]
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    with torch.cuda.stream(stream):
        if out is None:
            out = torch.empty_like(x)
        if workspace is None and T > 0:
            workspace = alloc_workspace(layer.dims, T, x.device)
    head, dbg, opts, keep = _call_args(x, layer, out, debug, path, residual, norm_eps,
                                       stage_events)
    rc = lib.moe_latent_forward_ex(
        *head, out.data_ptr(), workspace.data_ptr() if workspace is not None else None,
        workspace.numel() if workspace is not None else 0, dbg, opts, stream.cuda_stream)
    del keep
    if rc != 0:
        raise MoeLatentError(rc, lib.moe_latent_last_error().decode())
    return out


def forward_noalloc(x: torch.Tensor, layer: DeviceLayer, out: torch.Tensor, *,
                    debug: Optional[RouteDebug] = None, path: int = PATH_AUTO,
                    residual: bool = False, norm_eps: float = 1e-6,
                    stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """As forward(), through moe_latent_forward_noalloc: no workspace, the
    library's per-device scratch array instead, and ``out`` supplied by the
    caller (nothing is allocated). Raises MoeLatentError (EWORKSPACE) when
    the call needs more than NOALLOC_MAX_BYTES of scratch."""
    lib = load_library()
    _check_call(x, layer, out, None)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    head, dbg, opts, keep = _call_args(x, layer, out, debug, path, residual, norm_eps, None)
    rc = lib.moe_latent_forward_noalloc(*head, out.data_ptr(), dbg, opts, stream.cuda_stream)
    del keep
    if rc != 0:
        raise MoeLatentError(rc, lib.moe_latent_last_error().decode())
    return out


NOALLOC_MAX_BYTES = 32 << 20   # MOE_LATENT_NOALLOC_MAX_BYTES


__all__ = ["load_library", "DeviceLayer", "DeviceExperts", "DeviceFp4", "RouteDebug", "forward",
           "forward_noalloc", "NOALLOC_MAX_BYTES",
           "pack_fp4", "pack_experts", "pack_bf16", "PackedWeights", "PACK_GROUPED", "PACK_DECODE",
           "fold_router_weights",
           "workspace_bytes", "alloc_workspace", "MoeLatentError", "EXPORTS",
           "PATH_AUTO", "PATH_GROUPED", "PATH_DECODE", "DECODE_MAX_T", "STAGES"]
