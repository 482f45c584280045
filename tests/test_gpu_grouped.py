"""Routing groups of D/U on the GPU: G (D_g, U_g) pairs, expert e in group
e / (E/G), every token projected by every D_g, the shared expert in group 0
(the reading the oracle documents), on both paths against the oracle (needs
an MI355X). Every case prints what it runs before touching the GPU."""
import numpy as np
import pytest
import torch

import latent_sparse_moe_amd as lsm
import oracle
import synth
from gpu_helpers import check_output, check_routing, run_gpu, say, device

pytestmark = pytest.mark.gpu

_cache = {}

# 64 experts in 4 groups of 16: small enough for quick oracle runs, and the
# decode path takes it (16 experts per group)
DEC_SMALL_G = synth.Dims(hidden=512, latent=256, n_experts=64, inter=128, top_k=4, n_shared=1,
                         n_groups=4)


def grouped_layer(name):
    if name not in _cache:
        if name == "small":
            dims, seed, bias, zs = DEC_SMALL_G, 31, "zipf", 0.5
        elif name == "tiny":
            cfg = synth.CONFIGS["grouped_tiny"]
            dims, seed, bias, zs = cfg.dims, cfg.seed, "zipf", 0.5
        else:
            cfg = synth.CONFIGS[name]
            dims, seed, bias, zs = cfg.dims, cfg.seed, cfg.bias, cfg.zipf_s
        say(f"[gen] grouped {name} dims={dims} bias={bias}")
        host = synth.make_layer(dims, seed, bias, zs)
        _cache[name] = (host, lsm.DeviceLayer.from_host(host, device()))
    return _cache[name]


def run_case(name, host, dl, x, path):
    d = host.dims
    say(f"[case] grouped {name} T={x.shape[0]} path={path}")
    gpu = run_gpu(dl, x, path=path)
    ref = oracle.forward(host, x)
    n_near = check_routing(ref, gpu, d.top_k, d.n_experts)
    err, _ = check_output(ref, gpu["out"])
    say(f"[ok] grouped {name}: rel_l2={err:.3e} near_ties={n_near}")
    return gpu


@pytest.mark.parametrize("T", [1, 8, 37, 300])
def test_grouped_tiny_grouped_path(T):
    host, dl = grouped_layer("tiny")
    run_case(f"tiny T={T}", host, dl, synth.make_x(T, host.dims.hidden, 50 + T), lsm.PATH_GROUPED)


@pytest.mark.parametrize("path,T", [(lsm.PATH_DECODE, 1), (lsm.PATH_DECODE, 5),
                                    (lsm.PATH_DECODE, 8), (lsm.PATH_GROUPED, 8),
                                    (lsm.PATH_GROUPED, 257)])
def test_grouped_small(path, T):
    host, dl = grouped_layer("small")
    run_case(f"small T={T}", host, dl, synth.make_x(T, host.dims.hidden, 60 + T), path)


@pytest.mark.parametrize("path,T", [(lsm.PATH_DECODE, 1), (lsm.PATH_DECODE, 4),
                                    (lsm.PATH_DECODE, 8), (lsm.PATH_GROUPED, 4),
                                    (lsm.PATH_GROUPED, 300)])
def test_grouped145(path, T):
    host, dl = grouped_layer("grouped145")
    run_case(f"145b T={T}", host, dl, synth.make_x(T, host.dims.hidden, 70 + T), path)


@pytest.mark.parametrize("T", [1, 4, 8])
def test_grouped145_packed_folded_router(T):
    """Decode-packed weights with the folded router (each expert's row folded
    with its group's D_g), plain weights dropped: the bench's configuration."""
    host, dl = grouped_layer("grouped145")
    if "pk145" not in _cache:
        _cache["pk145"] = lsm.DeviceLayer(**{**dl.__dict__}).pack().drop_plain()
    run_case(f"145b packed T={T}", host, _cache["pk145"], synth.make_x(T, host.dims.hidden, 80 + T),
             lsm.PATH_AUTO)


def test_grouped145_packed_grouped_path_bit_exact():
    """The grouped path on grouped-packed copies equals the plain layout bit
    for bit (same bytes per lane)."""
    host, dl = grouped_layer("grouped145")
    x = synth.make_x(300, host.dims.hidden, 90)
    say("[case] grouped145 packed vs plain, grouped path T=300")
    a = run_gpu(dl, x, path=lsm.PATH_GROUPED)
    pk = lsm.DeviceLayer(**{**dl.__dict__}).pack(decode=False)
    b = run_gpu(pk, x, path=lsm.PATH_GROUPED)
    assert np.array_equal(a["out_bits"], b["out_bits"])
    assert np.array_equal(a["topk_idx"], b["topk_idx"])


@pytest.mark.parametrize("path,T", [(lsm.PATH_DECODE, 4), (lsm.PATH_GROUPED, 300)])
def test_grouped_deterministic(path, T):
    host, dl = grouped_layer("small")
    x = synth.make_x(T, host.dims.hidden, 99)
    say(f"[case] grouped determinism path={path} T={T}")
    a = run_gpu(dl, x, path=path)
    b = run_gpu(dl, x, path=path)
    for f in ("out_bits", "topk_idx", "topk_w", "perm", "counts", "logits"):
        assert np.array_equal(a[f], b[f]), f
