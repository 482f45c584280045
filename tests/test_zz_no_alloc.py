"""The allocation-free entry point (moe_latent_forward_noalloc, through the
C ABI) against the workspace entry point (moe_latent_forward_ex) on the same
inputs: outputs and routing bit for bit. Two calls in a row per path, the
second with fewer tokens, so the second call runs on scratch that still
holds the first call's contents."""
import numpy as np
import pytest
import torch

import latent_sparse_moe_amd as lsm
import synth
from gpu_helpers import device, say, to_dev_x

pytestmark = pytest.mark.gpu

_layer = {}


def _decode145():
    if "l" not in _layer:
        cfg = synth.CONFIGS["decode145"]
        say(f"[gen] decode145 dims={cfg.dims}")
        host = synth.make_layer(cfg.dims, cfg.seed)
        _layer["l"] = (host, lsm.DeviceLayer.from_host(host, device()))
    return _layer["l"]


@pytest.mark.parametrize("path,Ts", [(lsm.PATH_DECODE, (8, 3)), (lsm.PATH_GROUPED, (300, 37))])
def test_noalloc_matches_workspace_entry(path, Ts):
    host, dl = _decode145()
    d = host.dims
    dev = device()
    for T in Ts:
        assert lsm.workspace_bytes(d, T) <= lsm.NOALLOC_MAX_BYTES
        x = to_dev_x(synth.make_x(T, d.hidden, 70 + T), dev)
        say(f"[case] noalloc vs workspace entry, path={path} T={T}")
        dbg_a = lsm.RouteDebug.alloc(d, T, dev)
        want = lsm.forward(x, dl, workspace=lsm.alloc_workspace(d, T, dev), debug=dbg_a,
                           path=path)
        out = torch.empty_like(x)
        dbg_b = lsm.RouteDebug.alloc(d, T, dev)
        got = lsm.forward_noalloc(x, dl, out, debug=dbg_b, path=path)
        torch.cuda.synchronize()
        assert got is out
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))
        for f in ("topk_idx", "topk_w", "counts", "offsets", "perm", "logits"):
            assert torch.equal(getattr(dbg_a, f), getattr(dbg_b, f)), f
        say(f"[ok] path={path} T={T}: bit-identical")


def test_noalloc_rejects_oversized_call():
    host, dl = _decode145()
    T = 4096
    x = torch.zeros((T, host.dims.hidden), dtype=torch.bfloat16, device=device())
    say(f"[case] noalloc T={T} needs {lsm.workspace_bytes(host.dims, T)} bytes: rejected")
    with pytest.raises(lsm.MoeLatentError) as ei:
        lsm.forward_noalloc(x, dl, torch.empty_like(x))
    assert ei.value.code == lsm.EWORKSPACE
