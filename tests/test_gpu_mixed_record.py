"""The mixed 3/4-bit expert record on the GPU: E1M1 gate/up and e2m1 down,
on both paths, against the oracle (needs an MI355X).

The packed copies of an E1M1 set are checked byte for byte against the
layout the public header defines, and runs on them bit for bit against runs
on the plain layout. Every case prints what it runs before touching the GPU."""
import numpy as np
import pytest
import torch

import latent_sparse_moe_amd as lsm
import oracle
import synth
from gpu_helpers import check_output, check_routing, run_gpu, say, device

pytestmark = pytest.mark.gpu

DEC_SMALL = synth.Dims(hidden=512, latent=256, n_experts=64, inter=128, top_k=4, n_shared=1,
                       gateup_bits=3)
_cache = {}


def mixed_layer(name):
    if name not in _cache:
        if name == "tiny":
            dims, seed, bias, zs = synth.replace(synth.TINY, gateup_bits=3), 5, "none", 1.1
        elif name == "dec_small":
            dims, seed, bias, zs = DEC_SMALL, 23, "zipf", 1.1
        else:
            cfg = synth.CONFIGS[name]
            dims, seed, bias, zs = synth.replace(cfg.dims, gateup_bits=3), cfg.seed, cfg.bias, cfg.zipf_s
        say(f"[gen] mixed {name} dims={dims} bias={bias} seed={seed}")
        host = synth.make_layer(dims, seed, bias, zs)
        assert host.experts.gate.bits == 3 and host.experts.down.bits == 4
        _cache[name] = (host, lsm.DeviceLayer.from_host(host, device()))
    return _cache[name]


def run_case(name, host, dl, x, path, tokens=None):
    d = host.dims
    say(f"[case] mixed {name} T={x.shape[0]} path={path}")
    gpu = run_gpu(dl, x, path=path)
    ref = oracle.forward(host, x, tokens=tokens)
    n_near = check_routing(ref, gpu, d.top_k, d.n_experts)
    err_ok, err_all = check_output(ref, gpu["out"])
    say(f"[ok] mixed {name}: rel_l2={err_ok:.3e} (all {err_all:.3e}) near_ties={n_near}")
    return gpu


@pytest.mark.parametrize("T", [1, 37, 300])
def test_mixed_tiny_grouped(T):
    host, dl = mixed_layer("tiny")
    run_case(f"tiny T={T}", host, dl, synth.make_x(T, host.dims.hidden, 70 + T), lsm.PATH_GROUPED)


@pytest.mark.parametrize("path,T", [(lsm.PATH_GROUPED, 257), (lsm.PATH_DECODE, 1),
                                    (lsm.PATH_DECODE, 4), (lsm.PATH_DECODE, 8)])
def test_mixed_dec_small(path, T):
    host, dl = mixed_layer("dec_small")
    run_case(f"dec_small T={T}", host, dl, synth.make_x(T, host.dims.hidden, 80 + T), path)


@pytest.mark.parametrize("path,T", [(lsm.PATH_DECODE, 4), (lsm.PATH_DECODE, 8),
                                    (lsm.PATH_GROUPED, 4)])
def test_mixed_decode145(path, T):
    host, dl = mixed_layer("decode145")
    run_case(f"decode145 T={T}", host, dl, synth.make_x(T, host.dims.hidden, 90 + T), path)


@pytest.mark.timeout(900)
def test_mixed_prefill145_full():
    host, dl = mixed_layer("decode145")  # same 145B layer; a 4096-token batch, every row
    T = 4096
    run_case(f"145b T={T} (every row)", host, dl, synth.make_x(T, host.dims.hidden, 91),
             lsm.PATH_GROUPED)


@pytest.mark.parametrize("name,T", [("dec_small", 300), ("decode145", 513)])
def test_mixed_packed_bit_exact(name, T):
    """Runs on the packed copies of a mixed layer equal runs on its plain
    layout bit for bit, on both paths."""
    host, dl = mixed_layer(name)
    x = synth.make_x(T, host.dims.hidden, 95)
    say(f"[case] mixed packed vs plain {name} T={T}")
    plain = run_gpu(dl, x, path=lsm.PATH_GROUPED)
    pk = lsm.DeviceLayer(**{**dl.__dict__})
    pk.pack(fold_router=False)   # the same logits as the plain path: bit for bit
    assert pk.grouped_packed.experts.gate.bits == 3 and pk.decode_packed.experts.up.bits == 3
    got = run_gpu(pk, x, path=lsm.PATH_GROUPED)
    assert np.array_equal(got["out_bits"], plain["out_bits"])
    assert np.array_equal(got["topk_idx"], plain["topk_idx"])
    for Td in (1, 4, 8):
        xd = synth.make_x(Td, host.dims.hidden, 96 + Td)
        say(f"[case] mixed decode packed vs plain {name} T={Td}")
        a = run_gpu(dl, xd, path=lsm.PATH_DECODE)
        b = run_gpu(pk, xd, path=lsm.PATH_DECODE)
        assert np.array_equal(a["out_bits"], b["out_bits"])
        assert np.array_equal(a["topk_idx"], b["topk_idx"])


def _chunks(codes, N, K):
    """E1M1 codes [count][N][3K/8] as [count][N][K/32][12] chunks."""
    return codes.reshape(codes.shape[0], N, K // 32, 12)


def _e1m1_dev(codes, scales):
    dev = device()
    return lsm.DeviceFp4(torch.from_numpy(codes).to(dev), torch.from_numpy(scales).to(dev),
                         torch.ones(codes.shape[0], dtype=torch.float32, device=dev), 3)


@pytest.mark.parametrize("count,N,K", [(1, 32, 64), (3, 96, 192), (2, 640, 1792)])
def test_pack_e1m1_grouped_layout(count, N, K):
    """Grouped-packed E1M1: block (e, t, s) of 768 code bytes, lane L's
    12-byte chunk at 12 L = row 32t + r(L % 32), chunk 2s + L // 32."""
    say(f"[case] E1M1 grouped pack layout count={count} N={N} K={K}")
    rng = np.random.default_rng(N + 5 * K)
    codes = rng.integers(0, 256, (count, N, K * 3 // 8), dtype=np.uint8)
    scales = rng.integers(0, 256, (count, N, K // 16), dtype=np.uint8)
    p = lsm.pack_fp4(_e1m1_dev(codes, scales), N, K, lsm.PACK_GROUPED)
    torch.cuda.synchronize()
    assert p.bits == 3
    ch = _chunks(codes, N, K)
    m = np.arange(32)
    q = 4 * (m // 8) + m % 4
    r = 16 * (q // 8) + 8 * ((m // 4) % 2) + q % 8
    pc = np.empty((count, N // 32, K // 64, 64, 12), np.uint8)
    ps = np.empty((count, N // 32, K // 64, 64, 2), np.uint8)
    rows = np.arange(N // 32) * 32
    for L in range(64):
        for s in range(K // 64):
            pc[:, :, s, L, :] = ch[:, rows + r[L % 32], 2 * s + L // 32, :]
            c0 = 64 * s + 32 * (L // 32)
            ps[:, :, s, L, :] = scales[:, rows + r[L % 32], c0 // 16:c0 // 16 + 2]
    assert np.array_equal(p.codes.cpu().numpy().reshape(count, -1), pc.reshape(count, -1))
    assert np.array_equal(p.scales.cpu().numpy().reshape(count, -1), ps.reshape(count, -1))


@pytest.mark.parametrize("count,N,K", [(1, 16, 128), (3, 48, 384), (2, 640, 1792)])
def test_pack_e1m1_decode_layout(count, N, K):
    """Decode-packed E1M1: block (e, t, c) of 768 code bytes, lane l's
    12-byte chunk at 12 l = row 16t + l % 16, chunk 4c + l // 16."""
    say(f"[case] E1M1 decode pack layout count={count} N={N} K={K}")
    rng = np.random.default_rng(7 * N + K)
    codes = rng.integers(0, 256, (count, N, K * 3 // 8), dtype=np.uint8)
    scales = rng.integers(0, 256, (count, N, K // 16), dtype=np.uint8)
    p = lsm.pack_fp4(_e1m1_dev(codes, scales), N, K, lsm.PACK_DECODE)
    torch.cuda.synchronize()
    ch = _chunks(codes, N, K)
    pc = np.empty((count, N // 16, K // 128, 64, 12), np.uint8)
    ps = np.empty((count, N // 16, K // 128, 16, 8), np.uint8)
    rows = np.arange(N // 16) * 16
    for l in range(64):
        for c in range(K // 128):
            pc[:, :, c, l, :] = ch[:, rows + l % 16, 4 * c + l // 16, :]
    for i in range(16):
        for c in range(K // 128):
            ps[:, :, c, i, :] = scales[:, rows + i, 8 * c:8 * c + 8]
    assert np.array_equal(p.codes.cpu().numpy().reshape(count, -1), pc.reshape(count, -1))
    assert np.array_equal(p.scales.cpu().numpy().reshape(count, -1), ps.reshape(count, -1))


@pytest.mark.parametrize("T", [1, 4, 8])
def test_mixed_decode145_folded_router(T):
    """The mixed record on the decode path with decode-packed weights and the
    folded router (the bench's configuration) against the oracle."""
    host, dl = mixed_layer("decode145")
    pk = lsm.DeviceLayer(**{**dl.__dict__}).pack(grouped=False)
    assert pk.decode_packed.RD is not None
    run_case(f"decode145 folded T={T}", host, pk, synth.make_x(T, host.dims.hidden, 97 + T),
             lsm.PATH_DECODE)
