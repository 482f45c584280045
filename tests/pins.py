"""Checks that pin the oracle to facts outside itself: the OCP format tables,
torch's float8/bfloat16 dtypes, the pages' printed dimensions and totals,
closed forms worked out by hand, an independent brute-force evaluation, and
invariants of the routing bookkeeping.

Each check is a plain function that raises AssertionError on failure, so the
same checks run both against the real oracle (test_oracle_pins.py) and
against deliberately broken copies of it (test_oracle_mutations.py)."""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle
import synth
from brute import E2M1_MAGNITUDES, brute_forward, e1m1_matrix, fp4_matrix

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def page_pins():
    with open(os.path.join(GOLDEN, "page_pins.json")) as f:
        return json.load(f)


def sig_round(v: float, sig: int) -> float:
    if v == 0:
        return 0.0
    return round(v, sig - 1 - int(math.floor(math.log10(abs(v)))))


# --------------------------------------------------------------- formats

def check_e2m1_table():
    """OCP MX v1.0 FP4 E2M1: codes 0..7 are 0, .5, 1, 1.5, 2, 3, 4, 6; bit 3 negates."""
    got = oracle.e2m1_value(np.arange(16))
    want = np.array(E2M1_MAGNITUDES + [-v for v in E2M1_MAGNITUDES])
    assert np.array_equal(got, want), (got, want)


def check_e4m3_vs_torch():
    """All 256 E4M3fn bytes against torch.float8_e4m3fn (library decode)."""
    b = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3fn_value(b)
    want = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok]), np.nonzero(got[ok] != want[ok])


def check_bf16_vs_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint16)
    exp_field = (bits >> 7) & 0xFF
    bits = bits[exp_field != 0xFF]  # finite only
    got = oracle.bf16_value(bits)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, want)


def check_nibble_order():
    """Byte 0x21 holds element 2j = code 1 (0.5) in the low nibble and element
    2j+1 = code 2 (1.0) in the high nibble; scale byte 0x38 is 1.0."""
    codes = np.full((1, 8), 0x21, dtype=np.uint8)
    scales = np.full((1, 1), 0x38, dtype=np.uint8)
    w = oracle.dequant_fp4(codes, scales, 1.0)
    assert np.array_equal(w[0], np.tile([0.5, 1.0], 8)), w


def check_dequant_vs_brute(seed=3):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(5, 24), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, size=(5, 3), dtype=np.uint8)  # no NaN bytes
    g = np.float32(0.37)
    got = oracle.dequant_fp4(codes, scales, g)
    want = fp4_matrix(codes, scales, float(g)).numpy()
    assert np.array_equal(got, want)


# --------------------------------------------------------------- page dims

def check_e1m1_table():
    """E1M1 (this repository's 3-bit format): sign, exponent bit (bias 1),
    mantissa bit -> 0, .5, 1, 1.5 and their negatives; each value equals the
    OCP e2m1 value with the same sign and mantissa and the top exponent bit
    clear."""
    got = oracle.e1m1_value(np.arange(8))
    want = np.array([0.0, 0.5, 1.0, 1.5, -0.0, -0.5, -1.0, -1.5])
    assert np.array_equal(got, want), got
    widened = [((c >> 2) << 3) | (c & 3) for c in range(8)]
    assert np.array_equal(got, oracle.e2m1_value(np.array(widened)))


def check_e1m1_chunk_layout():
    """A chunk worked out by hand. Codes (sign, exponent, mantissa):
    elements 0..7 are 001 (+0.5), 8..15 are 110 (-1), 16..23 are 0..7 in
    order, 24..31 are 101 (-0.5). As e2m1 nibbles: w0 = 0x11111111, w1 =
    0xAAAAAAAA, w2 = 0xBA983210; then element 24 + p adds its mantissa (1)
    at bit 4p+2 of w0 and its sign (1) there in w2, its exponent (0) leaves
    w1 alone: w0 = 0x55555555, w1 = 0xAAAAAAAA, w2 = 0xFEDC7654."""
    words = [0x55555555, 0xAAAAAAAA, 0xFEDC7654]
    chunk = np.frombuffer(b"".join(v.to_bytes(4, "little") for v in words), dtype=np.uint8)
    codes = oracle.unpack_e1m1(chunk[None])[0]
    want = [1] * 8 + [6] * 8 + list(range(8)) + [5] * 8
    assert codes.tolist() == want, codes
    vals = oracle.e1m1_value(codes)
    assert vals[0] == 0.5 and vals[8] == -1.0 and vals[23] == -1.5 and vals[31] == -0.5
    # a second chunk in the same row decodes independently (byte-swapped words)
    two = oracle.unpack_e1m1(np.concatenate([chunk, chunk[::-1]])[None])[0]
    assert two[:32].tolist() == want
    rev = [int.from_bytes(bytes(chunk[::-1][4 * j:4 * j + 4]), "little") for j in range(3)]
    assert rev == [0x5476DCFE, 0xAAAAAAAA, 0x55555555]
    # element 0 of the second chunk: nibble 0 of w0 = 0xE -> sign 1, exp 1, mant 0
    # (bit 2 set: that bit is element 24's mantissa); element 24: bit 2 of the
    # three words' nibble 0 = (1, 0, 1) -> mantissa 1, exponent 0, sign 1
    assert two[32] == 0b110 and two[56] == 0b101


def check_e1m1_dequant_vs_brute(seed=4):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(3, 24), dtype=np.uint8)   # k = 64
    scales = rng.integers(0, 0x7F, size=(3, 4), dtype=np.uint8)
    g = np.float32(0.0123)
    got = oracle.dequant_e1m1(codes, scales, g)
    want = e1m1_matrix(codes, scales, float(g)).numpy()
    assert np.array_equal(got, want)


def check_e1m1_quantiser_error(seed=9):
    """The input generator's E1M1 quantiser, decoded by the oracle, is within
    half a step (0.25 s g) of the fp32 weights wherever the block maximum fits
    under 1.5 s g, and within the clamp elsewhere."""
    w = synth.normal_f32(seed, 77, 0, (8, 256), 1.0)
    m = synth.quantize_e1m1(w)
    dq = oracle.dequant_e1m1(m.codes[0], m.scales[0], m.gscale[0])
    step = np.repeat(oracle.e4m3fn_value(m.scales[0]), 16, axis=-1) * float(m.gscale[0]) * 0.5
    over = np.maximum(np.abs(w) - 3.0 * step, 0.0)
    assert np.all(np.abs(dq - w) <= 0.5 * step * (1 + 1e-6) + over)
    assert np.mean(np.abs(dq - w) / step) < 0.35


def check_page_dimensions():
    p = page_pins()
    for dims, lat in ((synth.E145, p["latent_145b"]["value"]), (synth.E120, p["latent_120b"]["value"])):
        assert dims.hidden == p["hidden"]["value"]
        assert dims.latent == lat
        assert dims.n_experts == p["n_experts"]["value"]
        assert dims.top_k == p["top_k"]["value"]
        assert dims.n_shared == p["n_shared"]["value"]
        assert dims.inter == p["inter"]["value"]
    L = p["n_layers"]["value"]
    for key_pool, key_act, lat in (("expert_pool_params_145b", "active_expert_params_145b", 1792),
                                   ("expert_pool_params_120b", "active_expert_params_120b", 1280),
                                   ("expert_pool_params_base", "active_expert_params_base", 2560)):
        pool, act = oracle.param_counts(L, 512, 10, lat, 640)
        assert sig_round(pool, p[key_pool]["sig"]) == p[key_pool]["value"], (key_pool, pool)
        assert sig_round(act, p[key_act]["sig"]) == p[key_act]["value"], (key_act, act)


def check_record_bytes():
    """NVFP4 experts.bin (47.6 GB) = 48 layers x 512 experts x our e2m1+E4M3/16
    record; the Q3_K records scale with the latent width (1792 : 1280)."""
    p = page_pins()
    rec = oracle.expert_record_bytes(1792, 640)
    assert rec == 1_935_360
    total = 48 * 512 * rec
    assert sig_round(total / 1e9, p["nvfp4_experts_bin_gb"]["sig"]) == p["nvfp4_experts_bin_gb"]["value"]
    q145 = p["q3k_record_bytes_145b"]["value"]
    q120 = p["q3k_record_bytes_120b"]["value"]
    assert q145 * 1280 == q120 * 1792
    assert sig_round(48 * 512 * q145 / 1e9, 3) == p["q3k_experts_bin_gb"]["value"]
    assert oracle.expert_record_bytes(1280, 640) * 1792 == rec * 1280
    # the mixed 3/4-bit record (3-bit gate/up, 4-bit down): within 1.2% of the
    # pages' Q3_K record for both latent widths
    m145 = oracle.expert_record_bytes(1792, 640, gateup_bits=3)
    m120 = oracle.expert_record_bytes(1280, 640, gateup_bits=3)
    assert m145 == 2 * 1792 * 640 * 3 // 8 + 1792 * 640 // 2 + 3 * 1792 * 640 // 16 == 1_648_640
    assert m120 == 1_177_600
    assert abs(m145 / q145 - 1) < 0.012 and abs(m120 / q120 - 1) < 0.012


# --------------------------------------------------------------- gating

def check_gate_vs_torch_topk(seed=5, T=64, E=48, k=7):
    rng = np.random.default_rng(seed)
    l32 = rng.standard_normal((T, E)).astype(np.float32)
    idx, w, gap = oracle.gate_topk(l32, k)
    tv, ti = torch.topk(torch.from_numpy(l32), k, dim=1, sorted=True)
    assert np.array_equal(idx, ti.numpy().astype(np.int32))
    want_w = torch.softmax(tv.to(torch.float64), dim=1).numpy()
    assert np.allclose(w, want_w, rtol=1e-13, atol=0)
    srt = np.sort(l32.astype(np.float64), axis=1)[:, ::-1]
    assert np.array_equal(gap, srt[:, k - 1] - srt[:, k])


def check_gate_ties_lower_index():
    l32 = np.array([[1.0, 3.0, 3.0, 2.0, 3.0, 0.0]], dtype=np.float32)
    idx, w, gap = oracle.gate_topk(l32, 4)
    assert idx.tolist() == [[1, 2, 4, 3]]
    assert np.allclose(w[0, :3], w[0, 0]) and gap[0] == 1.0


def check_gate_invariants(seed=6):
    rng = np.random.default_rng(seed)
    l32 = (3 * rng.standard_normal((200, 512))).astype(np.float32)
    idx, w, _ = oracle.gate_topk(l32, 10)
    assert np.allclose(w.sum(1), 1.0, atol=1e-12)
    assert (w > 0).all() and (np.diff(w, axis=1) <= 0).all()
    for t in range(200):
        assert len(set(idx[t].tolist())) == 10


def check_dense_softmax_when_k_equals_E(seed=7):
    """k = E: renormalising over every expert leaves the plain softmax."""
    rng = np.random.default_rng(seed)
    l32 = rng.standard_normal((9, 12)).astype(np.float32)
    idx, w, gap = oracle.gate_topk(l32, 12)
    dense = np.zeros_like(w)
    np.put_along_axis(dense, idx.astype(np.int64), w, axis=1)
    want = torch.softmax(torch.from_numpy(l32).to(torch.float64), dim=1).numpy()
    assert np.allclose(dense, want, rtol=1e-13, atol=0)
    assert np.isinf(gap).all()


# --------------------------------------------------------------- bookkeeping

def check_bookkeeping(seed=8, T=300, E=37, k=5):
    rng = np.random.default_rng(seed)
    # random choices (distinct per token), some experts empty
    idx = np.stack([rng.choice(E - 4, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm = oracle.route_bookkeeping(idx, E)
    flat = idx.ravel()
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert counts.sum() == T * k and offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(np.sort(perm), np.arange(T * k))
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    assert (np.diff(flat[perm]) >= 0).all()
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert (flat[seg] == e).all() and (np.diff(seg) > 0).all()


# --------------------------------------------------------------- closed forms

def _const_layer(dims, gate_code=0x22, up_code=0x22, down_code=0x22, down_scales=None,
                 shared_down_scale=0x38, R_rows=None):
    """Hand-built layer: D = U = identity (hidden == latent), expert codes all
    one byte, block scales 1.0 (0x38) unless given, matrix scales 1."""
    H, L, E, I = dims.hidden, dims.latent, dims.n_experts, dims.inter
    assert H == L
    one = np.uint16(0x3F80)
    eye = np.where(np.eye(L, dtype=bool), one, np.uint16(0)).astype(np.uint16)

    def mat(count, n, k, code, scale_bytes):
        codes = np.full((count, n, k // 2), code, dtype=np.uint8)
        scales = np.empty((count, n, k // 16), dtype=np.uint8)
        for c in range(count):
            scales[c] = scale_bytes[c]
        return synth.Fp4Mat(codes, scales, np.ones((count,), dtype=np.float32))

    ds = down_scales if down_scales is not None else [0x38] * E
    experts = synth.Fp4Bank(mat(E, I, L, gate_code, [0x38] * E), mat(E, I, L, up_code, [0x38] * E),
                            mat(E, L, I, down_code, ds))
    shared = synth.Fp4Bank(mat(1, I, L, gate_code, [0x38]), mat(1, I, L, up_code, [0x38]),
                           mat(1, L, I, down_code, [shared_down_scale]))
    if R_rows is None:
        R = np.full((E, L), 0x3F80, dtype=np.uint16)
    else:
        R = np.stack([np.full((L,), r, dtype=np.uint16) for r in R_rows])
    return synth.Layer(dims=dims, D=eye, U=eye.copy(), R=R, bias=None, experts=experts,
                       shared=shared, norm_w=np.ones((H,), np.float32))


def check_closed_form_all_ones():
    """All expert weights 1, D = U = I, x = c: h = c, gate = up = L c,
    a = silu(L c) L c, every routed and the shared expert give I a, the routed
    weights sum to 1, so out = 2 I (L c) silu(L c). With L = I = 32,
    c = 1/32: out = 64 silu(1) in every entry."""
    dims = synth.Dims(hidden=32, latent=32, n_experts=4, inter=32, top_k=2, n_shared=1)
    layer = _const_layer(dims)
    x = np.full((3, 32), 0x3D00, dtype=np.uint16)  # 1/32
    res = oracle.forward(layer, x)
    want = 64.0 / (1.0 + math.exp(-1.0))
    assert np.allclose(res.out, want, rtol=1e-14, atol=0), res.out[0, :4]


def check_closed_form_routing():
    """Router rows constant r_e, so logit_e = L c r_e = r_e for c = 1/L:
    r = (0.5, 2, 1, 1.5) selects experts 1 then 3 with weights
    softmax(2, 1.5). Down block scales 2 (0x40) for expert 1, 4 (0x48) for
    expert 3, 0.5 (0x30) for the shared one: out = (2 w0 + 4 w1 + 0.5) 32 silu(1)."""
    dims = synth.Dims(hidden=32, latent=32, n_experts=4, inter=32, top_k=2, n_shared=1)
    r_bits = [0x3F00, 0x4000, 0x3F80, 0x3FC0]  # 0.5, 2, 1, 1.5
    layer = _const_layer(dims, down_scales=[0x38, 0x40, 0x44, 0x48], shared_down_scale=0x30,
                         R_rows=r_bits)
    x = np.full((2, 32), 0x3D00, dtype=np.uint16)
    res = oracle.forward(layer, x)
    assert res.idx.tolist() == [[1, 3], [1, 3]]
    w0 = 1.0 / (1.0 + math.exp(-0.5))
    w1 = 1.0 - w0
    assert np.allclose(res.w, [[w0, w1]] * 2, rtol=1e-14)
    want = (2.0 * w0 + 4.0 * w1 + 0.5) * 32.0 / (1.0 + math.exp(-1.0))
    assert np.allclose(res.out, want, rtol=1e-14, atol=0), (res.out[0, 0], want)
    assert res.counts.tolist() == [0, 2, 0, 2]
    assert res.perm.tolist() == [0, 2, 1, 3]


def check_closed_form_signs_and_subnormal():
    """Gate codes 0xAA (every weight -1), up codes 0x22 (+1), down block scale
    0x01 (2^-9, the smallest E4M3 subnormal), x = 1/32: gate = -1, up = 1,
    a = silu(-1), each expert gives I 2^-9 silu(-1), the routed weights sum
    to 1 and the shared expert adds the same, so out = 2 * 32 * 2^-9 * silu(-1)."""
    dims = synth.Dims(hidden=32, latent=32, n_experts=2, inter=32, top_k=1, n_shared=1)
    layer = _const_layer(dims, gate_code=0xAA, down_scales=[0x01, 0x01], shared_down_scale=0x01)
    x = np.full((1, 32), 0x3D00, dtype=np.uint16)
    res = oracle.forward(layer, x)
    silu_m1 = -1.0 / (1.0 + math.exp(1.0))
    want = 2 * 32 * 2.0 ** -9 * silu_m1
    assert np.allclose(res.out, want, rtol=1e-14, atol=0), (res.out[0, 0], want)


def check_identical_experts_routing_free(seed=11):
    """Every expert (and the shared one) identical: the routed weights sum to
    1, so out = U (2 SwiGLU(h)) whatever the routing."""
    dims = synth.Dims(hidden=64, latent=32, n_experts=6, inter=32, top_k=3, n_shared=1)
    base = synth.make_layer(dims, seed)
    one = synth.Fp4Bank(*[synth.Fp4Mat(np.repeat(getattr(base.experts, p).codes[:1], 6, 0),
                                       np.repeat(getattr(base.experts, p).scales[:1], 6, 0),
                                       np.repeat(getattr(base.experts, p).gscale[:1], 6, 0))
                          for p in ("gate", "up", "down")])
    sh = synth.Fp4Bank(*[synth.Fp4Mat(getattr(base.experts, p).codes[:1].copy(),
                                      getattr(base.experts, p).scales[:1].copy(),
                                      getattr(base.experts, p).gscale[:1].copy())
                         for p in ("gate", "up", "down")])
    layer = synth.replace(base, experts=one, shared=sh)
    x = synth.make_x(5, 64, seed)
    res = oracle.forward(layer, x)
    xb = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    Dm = torch.from_numpy(layer.D.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    Um = torch.from_numpy(layer.U.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    wg = fp4_matrix(sh.gate.codes[0], sh.gate.scales[0], float(sh.gate.gscale[0]))
    wu = fp4_matrix(sh.up.codes[0], sh.up.scales[0], float(sh.up.gscale[0]))
    wd = fp4_matrix(sh.down.codes[0], sh.down.scales[0], float(sh.down.gscale[0]))
    h = xb @ Dm.T
    g = h @ wg.T
    a = torch.nn.functional.silu(g) * (h @ wu.T)
    want = (2.0 * (a @ wd.T)) @ Um.T
    assert np.allclose(res.out, want.numpy(), rtol=1e-12, atol=1e-12)


def check_single_expert_no_shared(seed=12):
    """E = 1, k = 1, no shared expert: out = U SwiGLU(D x) (torch float64)."""
    dims = synth.Dims(hidden=64, latent=32, n_experts=1, inter=64, top_k=1, n_shared=0)
    layer = synth.make_layer(dims, seed)
    x = synth.make_x(4, 64, seed)
    res = oracle.forward(layer, x)
    xb = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    Dm = torch.from_numpy(layer.D.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    Um = torch.from_numpy(layer.U.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    b = layer.experts
    wg = fp4_matrix(b.gate.codes[0], b.gate.scales[0], float(b.gate.gscale[0]))
    wu = fp4_matrix(b.up.codes[0], b.up.scales[0], float(b.up.gscale[0]))
    wd = fp4_matrix(b.down.codes[0], b.down.scales[0], float(b.down.gscale[0]))
    h = xb @ Dm.T
    want = ((torch.nn.functional.silu(h @ wg.T) * (h @ wu.T)) @ wd.T) @ Um.T
    assert np.allclose(res.out, want.numpy(), rtol=1e-12, atol=1e-12)
    assert np.all(res.w == 1.0) and np.all(res.idx == 0)


# --------------------------------------------------------------- brute force

def check_vs_brute(layer, x, rtol=1e-10):
    res = oracle.forward(layer, x)
    out_b, idx_b, w_b, l_b = brute_forward(layer, x)
    assert np.array_equal(res.idx, idx_b)
    assert np.allclose(res.w, w_b, rtol=1e-12, atol=0)
    assert np.array_equal(res.logits32.astype(np.float64), l_b)
    scale = np.abs(out_b).max()
    assert np.allclose(res.out, out_b, rtol=rtol, atol=rtol * scale), np.abs(res.out - out_b).max()


def check_dense_all_experts(layer, x):
    """out = U (sum_e wfull[t, e] E_e(h_t) + S(h_t)), wfull scattering the
    routed weights into a dense [T][E] matrix (zero for unrouted experts)."""
    res = oracle.forward(layer, x)
    d = layer.dims
    xb = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    Dm = torch.from_numpy(layer.D.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    Um = torch.from_numpy(layer.U.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    h = xb @ Dm.T
    wfull = torch.zeros((x.shape[0], d.n_experts), dtype=torch.float64)
    wfull.scatter_(1, torch.from_numpy(res.idx.astype(np.int64)), torch.from_numpy(res.w))

    def ex(bank, e):
        wg = fp4_matrix(bank.gate.codes[e], bank.gate.scales[e], float(bank.gate.gscale[e]))
        wu = fp4_matrix(bank.up.codes[e], bank.up.scales[e], float(bank.up.gscale[e]))
        wd = fp4_matrix(bank.down.codes[e], bank.down.scales[e], float(bank.down.gscale[e]))
        return (torch.nn.functional.silu(h @ wg.T) * (h @ wu.T)) @ wd.T

    z = sum(wfull[:, e:e + 1] * ex(layer.experts, e) for e in range(d.n_experts))
    if d.n_shared:
        z = z + ex(layer.shared, 0)
    want = (z @ Um.T).numpy()
    assert np.allclose(res.out, want, rtol=1e-10, atol=1e-10 * np.abs(want).max())


# --------------------------------------------------------------- block / stack

def check_rmsnorm_vs_torch(seed=13):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((7, 96))
    g = rng.standard_normal(96)
    got = oracle.rmsnorm(x, g, 1e-6)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), 1e-6).numpy()
    assert np.allclose(got, want, rtol=1e-13, atol=1e-13)


def check_block_residual(seed=14):
    """x + brute(bf16(rms_norm(x) * g)), with torch's rms_norm and bfloat16 cast."""
    dims = synth.Dims(hidden=64, latent=32, n_experts=8, inter=32, top_k=2, n_shared=1)
    layer = synth.make_layer(dims, seed)
    x = synth.make_x(3, 64, seed)
    got, _ = oracle.block_forward(layer, x, 1e-6)
    xb = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    u = torch.nn.functional.rms_norm(xb, (64,), torch.from_numpy(layer.norm_w).to(torch.float64), 1e-6)
    u_bits = u.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    out_b, _, _, _ = brute_forward(layer, u_bits)
    assert np.allclose(got, xb.numpy() + out_b, rtol=1e-10, atol=1e-10)


def check_bf16_rounding_vs_torch(seed=15):
    from oracle.latent_moe import _to_bf16_bits
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(2.0 + 2.0 ** -7)])
    v = np.concatenate([v, ties])
    got = _to_bf16_bits(v)
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def _torch_block_bits(layer, x_bits, H):
    """One residual block by the independent route: torch rms_norm, the
    per-token brute-force layer, torch's bfloat16 rounding of the sum."""
    xb = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    u = torch.nn.functional.rms_norm(xb, (H,), torch.from_numpy(layer.norm_w).to(torch.float64), 1e-6)
    u_bits = u.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    out_b, _, _, _ = brute_forward(layer, u_bits)
    y = xb.numpy() + out_b
    return torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def check_stack_zero_up_projection_is_identity(seed=16):
    """U = 0 in every block makes each block's MoE output exactly zero, so the
    residual stream passes through unchanged: every x_l equals x bit for bit."""
    dims = synth.Dims(hidden=64, latent=32, n_experts=8, inter=32, top_k=2, n_shared=1)
    layers = [synth.make_layer(dims, seed + l, "zipf") for l in range(3)]
    for layer in layers:
        layer.U = np.zeros_like(layer.U)
    x = synth.make_x(5, 64, seed)
    xs, _ = oracle.stack_forward(layers, x, 1e-6)
    for xl in xs:
        assert np.array_equal(xl, x)


def check_stack_vs_torch_chain(seed=17):
    """Three blocks chained by the independent route (torch rms_norm + brute
    layer + torch bf16 rounding between blocks) equal the oracle's stack bit
    for bit, including a middle block whose U = 0 (it must return its input)."""
    dims = synth.Dims(hidden=64, latent=32, n_experts=8, inter=32, top_k=2, n_shared=1)
    layers = [synth.make_layer(dims, seed + l, "zipf") for l in range(3)]
    layers[1].U = np.zeros_like(layers[1].U)
    x = synth.make_x(6, 64, seed)
    xs, _ = oracle.stack_forward(layers, x, 1e-6)
    cur = x
    for l, layer in enumerate(layers):
        cur = _torch_block_bits(layer, cur, 64)
        assert np.array_equal(xs[l + 1], cur), l
    assert np.array_equal(xs[2], xs[1])


# --------------------------------------------------------------- routing groups

def _grouped_tiny(seed=21, bias="zipf", zs=0.7):
    d = synth.replace(synth.TINY, n_groups=4)
    return synth.make_layer(d, seed, bias, zs)


def check_grouped_vs_brute(seed=21):
    """The grouped layer (4 groups of 4 experts, each with its own D_g and
    U_g) against the independent per-token evaluation."""
    layer = _grouped_tiny(seed)
    x = synth.make_x(6, layer.dims.hidden, seed)
    check_vs_brute(layer, x)


def check_grouped_repeated_pairs_equal_one_pair(seed=22):
    """With every (D_g, U_g) equal to (D_0, U_0), the grouped layer equals the
    layer with one pair: every group's latent is the same h, the router sees
    the same logits, and sum_g z_g U_0^T = (sum_g z_g) U_0^T."""
    layer = _grouped_tiny(seed)
    d = layer.dims
    L, G = d.latent, d.n_groups
    one = synth.make_layer(synth.replace(d, n_groups=1), seed, "zipf", 0.7)
    layer.D = np.tile(one.D, (G, 1))
    layer.U = np.tile(one.U, (1, G))
    x = synth.make_x(9, d.hidden, seed)
    a = oracle.forward(layer, x)
    b = oracle.forward(one, x)
    assert np.array_equal(a.idx, b.idx)
    assert np.allclose(a.out, b.out, rtol=1e-12, atol=1e-12), np.abs(a.out - b.out).max()
    assert np.allclose(a.h[:, :L], b.h, rtol=0, atol=0)


def check_grouped_up_projection_per_group(seed=23):
    """Only group g's U_g nonzero: the output is z_g U_g^T, i.e. exactly the
    contribution of the token's choices in group g (and of the shared
    expert for g = 0); the other groups' terms vanish."""
    layer = _grouped_tiny(seed)
    d = layer.dims
    L, G, epg = d.latent, d.n_groups, d.n_experts // d.n_groups
    x = synth.make_x(7, d.hidden, seed)
    full = oracle.forward(layer, x)
    total = np.zeros_like(full.out)
    for g in range(G):
        lg = synth.make_layer(d, seed, "zipf", 0.7)
        U = lg.U.copy()
        keep = np.zeros_like(U)
        keep[:, g * L:(g + 1) * L] = U[:, g * L:(g + 1) * L]
        lg.U = keep
        r = oracle.forward(lg, x)
        # tokens with no choice in group g (and g != 0) get exactly zero
        for t in range(x.shape[0]):
            if g != 0 and not any(int(e) // epg == g for e in full.idx[t]):
                assert np.all(r.out[t] == 0.0), (g, t)
        total += r.out
    assert np.allclose(total, full.out, rtol=1e-12, atol=1e-12)
