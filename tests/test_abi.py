"""The C-ABI library on the host (no GPU needed): it loads, exports every
function the public header declares, and rejects bad arguments before any
HIP call (so these error paths never touch a device)."""
import ctypes
import glob
import os
import re

import pytest
import torch  # noqa: F401  (loads the HIP runtime the library binds to)

import latent_sparse_moe_amd as lsm
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b(moe_\w+)\s*\(", text):
            names.add(m.group(1))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    return lsm.load_library()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert "moe_latent_forward" in names and len(names) >= 5
    for n in names:
        assert hasattr(lib, n), n
    assert set(lsm.EXPORTS) == set(names)


def test_version(lib):
    assert lib.moe_latent_version() == 4


def _dims(**kw):
    d = dict(hidden=2560, latent=1792, n_experts=512, inter=640, top_k=10, n_shared=1)
    d.update(kw)
    return lsm.CDims(**d)


def test_workspace_bytes(lib):
    d = _dims()
    b4 = lib.moe_latent_workspace_bytes(ctypes.byref(d), 4)
    b16k = lib.moe_latent_workspace_bytes(ctypes.byref(d), 16384)
    assert 0 < b4 < b16k
    assert b16k > 16384 * 11 * (1792 + 640) * 2  # expert activations dominate
    assert lib.moe_latent_workspace_bytes(ctypes.byref(d), 0) == 0
    assert lib.moe_latent_workspace_bytes(ctypes.byref(_dims(latent=100)), 4) == 0
    assert lib.moe_latent_workspace_bytes(None, 4) == 0


# Fake, never dereferenced device addresses (every validation precedes use).
A = 1 << 20


def _call(lib, dims, T=4, x=A, D=2 * A, U=3 * A, router=True, experts=True, shared=True,
          out=5 * A, ws=64 * A, ws_bytes=1 << 40, opts=None, bias=None, count=None,
          bits=(0, 0, 0), sh_bits=(0, 0, 0)):
    r = lsm.CRouter(7 * A, bias) if router else None

    def mats(b):
        return [lsm.CFp4Matrix(8 * A, 9 * A, 10 * A, x) for x in b]
    ex = (lsm.CFp4Experts(*mats(bits), dims.n_experts if count is None else count)
          if experts else None)
    sh = lsm.CFp4Experts(*mats(sh_bits), dims.n_shared) if shared else None
    rc = lib.moe_latent_forward_ex(ctypes.byref(dims), T, x, D, U,
                                   ctypes.byref(r) if r else None,
                                   ctypes.byref(ex) if ex else None,
                                   ctypes.byref(sh) if sh else None, out, ws, ws_bytes, None,
                                   ctypes.byref(opts) if opts else None, None)
    return rc, lib.moe_latent_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(hidden=0), lsm.EINVAL),
    (dict(latent=100), lsm.EUNSUPPORTED),
    (dict(inter=48), lsm.EUNSUPPORTED),
    (dict(top_k=17, n_experts=32), lsm.EUNSUPPORTED),
    (dict(top_k=11, n_experts=10), lsm.EUNSUPPORTED),
    (dict(n_experts=2048), lsm.EUNSUPPORTED),
    (dict(n_shared=2), lsm.EUNSUPPORTED),
    (dict(n_groups=-1), lsm.EINVAL),
    (dict(n_groups=3), lsm.EUNSUPPORTED),      # does not divide 512 experts
])
def test_bad_dims(lib, kw, code):
    rc, msg = _call(lib, _dims(**kw))
    assert rc == code and msg


def test_error_paths(lib):
    d = _dims()
    assert _call(lib, d, T=-1)[0] == lsm.EINVAL
    assert _call(lib, d, x=0)[0] == lsm.EINVAL
    assert _call(lib, d, x=A + 8)[0] == lsm.EINVAL            # misaligned
    assert _call(lib, d, router=False)[0] == lsm.EINVAL
    assert _call(lib, d, experts=False)[0] == lsm.EINVAL
    assert _call(lib, d, shared=False)[0] == lsm.EINVAL       # n_shared = 1 needs it
    assert _call(lib, d, count=511)[0] == lsm.EINVAL
    assert _call(lib, d, out=A)[0] == lsm.EINVAL              # out aliases x
    assert _call(lib, d, ws=0)[0] == lsm.EINVAL
    assert _call(lib, d, ws=64 * A + 16)[0] == lsm.EINVAL     # workspace alignment
    rc, msg = _call(lib, d, ws_bytes=1000)
    assert rc == lsm.EWORKSPACE and "needed" in msg
    assert _call(lib, d, opts=lsm.COpts(7, 0, None, 0.0, None))[0] == lsm.EINVAL
    assert _call(lib, d, T=17, opts=lsm.COpts(lsm.PATH_DECODE, 0, None, 0.0, None))[0] == lsm.EUNSUPPORTED
    assert _call(lib, d, opts=lsm.COpts(0, 1, None, 1e-6, None))[0] == lsm.EINVAL  # residual w/o weight
    assert _call(lib, d, T=2 ** 31 // 10 + 1)[0] == lsm.EUNSUPPORTED
    # T = 0 is a valid no-op; shared may be NULL when n_shared = 0
    assert _call(lib, d, T=0)[0] == 0
    assert _call(lib, _dims(n_shared=0), T=0, shared=False)[0] == 0
    assert _call(lib, d, T=0, x=0, out=0, ws=0, ws_bytes=0)[0] == 0


def test_last_error_cleared(lib):
    _call(lib, _dims(hidden=0))
    assert lib.moe_latent_last_error()
    assert _call(lib, _dims(), T=0)[0] == 0
    assert lib.moe_latent_last_error() == b""


def test_binding_fails_loudly_without_library(tmp_path):
    saved = lsm._lib
    try:
        lsm._lib = None
        with pytest.raises(RuntimeError, match="no fallback"):
            lsm.load_library(str(tmp_path / "missing.so"))
    finally:
        lsm._lib = saved


def _opts_with(grouped=None, decode=None):
    return lsm.COpts(lsm.PATH_AUTO, 0, None, 0.0, None,
                     ctypes.pointer(grouped) if grouped is not None else None,
                     ctypes.pointer(decode) if decode is not None else None)


_M = lsm.CFp4Matrix(11 * A, 12 * A, 10 * A)
_PEX = lsm.CFp4Experts(_M, _M, _M, 512)
_PSH = lsm.CFp4Experts(_M, _M, _M, 1)


def _pw(experts=True, shared=True, D=None, U=None, R=None):
    return lsm.CPackedWeights(ctypes.pointer(_PEX) if experts else None,
                              ctypes.pointer(_PSH) if shared else None, D, U, R)


def test_grouped_packed_validation(lib):
    rc, msg = _call(lib, _dims(), opts=_opts_with(_pw(shared=False)))  # shared copy missing
    assert rc == lsm.EINVAL and "shared" in msg
    rc, msg = _call(lib, _dims(latent=1760), opts=_opts_with(_pw()))  # latent % 64 != 0
    assert rc == lsm.EUNSUPPORTED and "64" in msg
    assert _call(lib, _dims(inter=608), opts=_opts_with(_pw()))[0] == lsm.EUNSUPPORTED
    bad = lsm.CFp4Experts(lsm.CFp4Matrix(11 * A + 8, 12 * A, 10 * A), _M, _M, 512)
    g = lsm.CPackedWeights(ctypes.pointer(bad), ctypes.pointer(_PSH), None, None, None)
    assert _call(lib, _dims(), opts=_opts_with(g))[0] == lsm.EINVAL    # misaligned codes
    dense = _pw(experts=False, shared=False, R=30 * A)
    assert _call(lib, _dims(n_experts=24, top_k=4), opts=_opts_with(dense))[0] == lsm.EUNSUPPORTED
    dense = _pw(experts=False, shared=False, D=30 * A)
    assert _call(lib, _dims(hidden=2528), opts=_opts_with(dense))[0] == lsm.EUNSUPPORTED
    dense = _pw(experts=False, shared=False, U=30 * A)
    assert _call(lib, _dims(latent=1760), opts=_opts_with(dense))[0] == lsm.EUNSUPPORTED
    dense = _pw(experts=False, shared=False, U=30 * A + 8)
    assert _call(lib, _dims(), opts=_opts_with(dense))[0] == lsm.EINVAL
    full = _pw(D=30 * A, U=31 * A, R=32 * A)
    assert _call(lib, _dims(), T=0, opts=_opts_with(full))[0] == 0


def test_decode_packed_validation(lib):
    full = _pw(D=30 * A, U=31 * A, R=32 * A)
    assert _call(lib, _dims(), T=0, opts=_opts_with(decode=full))[0] == 0
    for missing in (dict(D=None), dict(U=None), dict(R=None)):
        kw = dict(D=30 * A, U=31 * A, R=32 * A)
        kw.update(missing)
        rc, msg = _call(lib, _dims(), opts=_opts_with(decode=_pw(**kw)))
        assert rc == lsm.EINVAL and "decode_packed" in msg
    assert _call(lib, _dims(), opts=_opts_with(decode=_pw(experts=False, D=30 * A, U=31 * A,
                                                              R=32 * A)))[0] == lsm.EINVAL
    rc, msg = _call(lib, _dims(n_experts=24, top_k=4), opts=_opts_with(decode=full))
    assert rc == lsm.EUNSUPPORTED and "16" in msg
    assert _call(lib, _dims(), opts=_opts_with(decode=_pw(D=30 * A + 2, U=31 * A,
                                                          R=32 * A)))[0] == lsm.EINVAL


def _pack(lib, src=True, count=4, N=64, K=128, layout=1, dc=20 * A, ds=21 * A, codes=8 * A,
          scales=9 * A, bits=0):
    m = lsm.CFp4Matrix(codes, scales, 10 * A, bits)
    rc = lib.moe_fp4_pack(ctypes.byref(m) if src else None, count, N, K, layout, dc, ds, None)
    return rc, lib.moe_latent_last_error().decode()


def test_pack_validation(lib):
    assert _pack(lib, src=False)[0] == lsm.EINVAL
    assert _pack(lib, dc=0)[0] == lsm.EINVAL
    assert _pack(lib, layout=3)[0] == lsm.EINVAL
    assert _pack(lib, N=48)[0] == lsm.EUNSUPPORTED                 # grouped: N % 32
    assert _pack(lib, K=96)[0] == lsm.EUNSUPPORTED                 # grouped: K % 64
    assert _pack(lib, K=192, layout=2)[0] == lsm.EUNSUPPORTED      # decode: K % 128
    assert _pack(lib, K=0)[0] == lsm.EINVAL
    assert _pack(lib, count=-1)[0] == lsm.EINVAL
    assert _pack(lib, dc=20 * A + 4)[0] == lsm.EINVAL              # misaligned
    assert _pack(lib, dc=8 * A)[0] == lsm.EINVAL                   # over the source codes
    assert _pack(lib, ds=20 * A + 64)[0] == lsm.EINVAL             # scales inside packed codes
    assert _pack(lib, count=0) == (0, "")                          # nothing to do
    assert _pack(lib, count=0, layout=2) == (0, "")
    assert _pack(lib, bits=5)[0] == lsm.EUNSUPPORTED               # unknown element format
    assert _pack(lib, bits=3, K=96)[0] == lsm.EUNSUPPORTED         # E1M1, grouped: K % 64
    # E1M1 codes are 3/8 of a byte per element: 4 x 64 x 128 x 3/8 = 12 KiB
    assert _pack(lib, bits=3, dc=8 * A + 12288 - 16)[0] == lsm.EINVAL  # overlaps by 16 bytes
    assert _pack(lib, bits=3, count=0) == (0, "")


def test_format_validation(lib):
    """Expert element formats: gate and up alike (e2m1 or E1M1), down e2m1,
    one gate/up format per layer, E1M1 with latent a multiple of 64. Only
    combinations that fail are called (a valid one would launch kernels on
    these fake addresses)."""
    d = _dims()
    for bits in ((5, 5, 0), (3, 4, 0), (4, 3, 4), (0, 0, 3), (3, 3, 3), (3, 0, 0)):
        rc, msg = _call(lib, d, bits=bits, sh_bits=bits)
        assert rc == lsm.EUNSUPPORTED and "bits" in msg, (bits, msg)
    rc, msg = _call(lib, d, bits=(3, 3, 4), sh_bits=(0, 0, 0))   # routed E1M1, shared e2m1
    assert rc == lsm.EUNSUPPORTED and "shared" in msg
    rc, msg = _call(lib, _dims(latent=1760), bits=(3, 3, 4), sh_bits=(3, 3, 4))
    assert rc == lsm.EUNSUPPORTED and "64" in msg
    # a packed copy in another format than the plain sets
    o = _opts_with(_pw())                                         # e2m1 copies
    rc, msg = _call(lib, d, bits=(3, 3, 0), sh_bits=(3, 3, 0), opts=o)
    assert rc == lsm.EUNSUPPORTED and "grouped_packed" in msg
    assert _call(lib, d, T=0, bits=(3, 3, 4), sh_bits=(3, 3, 4))[0] == 0


def test_bf16_pack_validation(lib):
    def pk(src=8 * A, N=64, K=128, layout=1, dst=20 * A):
        return lib.moe_bf16_pack(src, N, K, layout, dst, None)
    assert pk(src=0) == lsm.EINVAL
    assert pk(dst=0) == lsm.EINVAL
    assert pk(layout=0) == lsm.EINVAL
    assert pk(N=48) == lsm.EUNSUPPORTED
    assert pk(N=40, layout=2) == lsm.EUNSUPPORTED      # decode: N % 16
    assert pk(K=96) == lsm.EUNSUPPORTED
    assert pk(K=80, layout=2) == lsm.EUNSUPPORTED      # decode: K % 32
    assert pk(N=-32) == lsm.EINVAL
    assert pk(dst=20 * A + 2) == lsm.EINVAL
    assert pk(dst=8 * A + 4096) == lsm.EINVAL          # overlaps the source


def test_binding_api_present():
    """The binding's public entry points exist (the GPU tests depend on them)."""
    for name in ("load_library", "forward", "pack_fp4", "pack_bf16", "pack_experts",
                 "workspace_bytes", "alloc_workspace"):
        assert callable(getattr(lsm, name)), name
    assert callable(lsm.DeviceLayer.from_host) and callable(lsm.DeviceLayer.pack)
    assert callable(lsm.RouteDebug.alloc)
    assert {f for f, _ in lsm.COpts._fields_} >= {"grouped_packed", "decode_packed"}


def test_plain_weights_needed_without_packed_copies(lib):
    d = _dims()
    g = lsm.COpts(lsm.PATH_GROUPED, 0, None, 0.0, None, None, None)
    rc, msg = _call(lib, d, D=0, opts=g)
    assert rc == lsm.EINVAL and "packed" in msg
    assert _call(lib, d, U=0, opts=g)[0] == lsm.EINVAL
    assert _call(lib, d, experts=False, opts=g)[0] == lsm.EINVAL
    # a grouped-packed D does not stand in for the experts
    dense = _pw(experts=False, shared=False, D=30 * A)
    o = lsm.COpts(lsm.PATH_GROUPED, 0, None, 0.0, None, ctypes.pointer(dense), None)
    assert _call(lib, d, experts=False, opts=o)[0] == lsm.EINVAL
    # decode-packed copies do not serve the grouped path (T = 64 runs grouped)
    full = _pw(D=30 * A, U=31 * A, R=32 * A)
    o = lsm.COpts(lsm.PATH_AUTO, 0, None, 0.0, None, None, ctypes.pointer(full))
    assert _call(lib, d, T=64, D=0, opts=o)[0] == lsm.EINVAL


def test_bench_helpers_on_host_layers():
    """bench.py's layer copy and byte counts work on a layer held in host
    memory (no kernel runs): the copy keeps every field, including each
    matrix's element format, and the mixed record's expert is smaller."""
    import sys
    sys.path.insert(0, ROOT)
    import bench
    d = synth.replace(synth.TINY, gateup_bits=3)
    dl = lsm.DeviceLayer.from_host(synth.make_layer(d, 1), "cpu")
    cp = bench.clone_layer(lsm, dl)
    assert cp.experts.gate.bits == 3 and cp.experts.down.bits == 4
    assert cp.experts.gate.codes.data_ptr() != dl.experts.gate.codes.data_ptr()
    assert torch.equal(cp.experts.gate.codes, dl.experts.gate.codes)
    # 145B expert: 3 x 1792 x 640 weights; codes + one E4M3 byte per 16
    assert bench.rec_bytes(1792, 640, 4) == 3 * 1792 * 640 * 4 // 8 + 3 * 1792 * 640 // 16
    assert bench.rec_bytes(1792, 640, 3) == 1648640   # 2 x 3-bit + 1 x 4-bit matrices


# ------------------------------------------------------------------ Python binding argument checks
# The binding checks tensor dtypes, shapes, contiguity and devices before it
# hands raw pointers to the library; host tensors are enough to exercise each
# rejection (nothing reaches the library or a device).

def _host_layer():
    return lsm.DeviceLayer(dims=synth.TINY, D=None, U=None, R=None, bias=None, experts=None,
                           shared=None)


@pytest.mark.parametrize("case", ["dtype", "rank", "width", "strided", "device"])
def test_binding_rejects_bad_x(case):
    H = synth.TINY.hidden
    x = torch.zeros((4, H), dtype=torch.bfloat16)
    if case == "dtype":
        x = x.float()
    elif case == "rank":
        x = x.reshape(-1)
    elif case == "width":
        x = torch.zeros((4, H + 32), dtype=torch.bfloat16)
    elif case == "strided":
        x = torch.zeros((H, 4), dtype=torch.bfloat16).t()   # [4][H] view, column-major
    with pytest.raises((ValueError, TypeError)):
        lsm.forward(x, _host_layer())


@pytest.mark.parametrize("case", ["dtype", "shape", "strided"])
def test_binding_rejects_bad_out(case):
    H = synth.TINY.hidden
    x = torch.zeros((4, H), dtype=torch.bfloat16)
    out = torch.zeros((4, H), dtype=torch.bfloat16)
    if case == "dtype":
        out = out.float()
    elif case == "shape":
        out = torch.zeros((3, H), dtype=torch.bfloat16)
    elif case == "strided":
        out = torch.zeros((H, 4), dtype=torch.bfloat16).t()
    with pytest.raises(ValueError, match="out"):
        lsm.forward(x, _host_layer(), out=out)


def test_binding_rejects_bad_workspace():
    x = torch.zeros((4, synth.TINY.hidden), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="workspace"):
        lsm.forward(x, _host_layer(), workspace=torch.zeros(1024, dtype=torch.int32))


def _call_noalloc(lib, dims, T=4, x=A, out=1 << 36):
    r = lsm.CRouter(7 * A, None)
    mats = [lsm.CFp4Matrix(8 * A, 9 * A, 10 * A, 0) for _ in range(3)]
    ex = lsm.CFp4Experts(*mats, dims.n_experts)
    sh = lsm.CFp4Experts(*mats, dims.n_shared)
    rc = lib.moe_latent_forward_noalloc(ctypes.byref(dims), T, x, 2 * A, 3 * A, ctypes.byref(r),
                                        ctypes.byref(ex), ctypes.byref(sh), out, None, None,
                                        None)
    return rc, lib.moe_latent_last_error().decode()


def test_noalloc_rejects_oversized_calls_before_any_hip_call(lib):
    d = _dims()
    need = lib.moe_latent_workspace_bytes(ctypes.byref(d), 4096)
    assert need > lsm.NOALLOC_MAX_BYTES
    rc, msg = _call_noalloc(lib, d, T=4096)
    assert rc == lsm.EWORKSPACE and "allocation-free" in msg
    # invalid arguments are still reported as such, and T = 0 is a no-op
    assert _call_noalloc(lib, d, x=0)[0] == lsm.EINVAL
    assert _call_noalloc(lib, d, T=0, x=0, out=0)[0] == 0
    # every decode-path call of the 145B and 120B layers fits the scratch array
    for lat in (1792, 1280):
        assert lib.moe_latent_workspace_bytes(ctypes.byref(_dims(latent=lat)), 8) \
            <= lsm.NOALLOC_MAX_BYTES


def test_grouped_workspace_grows_with_groups(lib):
    """Routing groups: the latent vector and the combined output hold every
    group's columns (G * latent)."""
    one = lib.moe_latent_workspace_bytes(ctypes.byref(_dims()), 300)
    eight = lib.moe_latent_workspace_bytes(ctypes.byref(_dims(n_groups=8)), 300)
    assert eight >= one + 300 * 7 * 1792 * (4 + 2)
    assert lib.moe_latent_workspace_bytes(ctypes.byref(_dims(n_groups=1)), 300) == one
