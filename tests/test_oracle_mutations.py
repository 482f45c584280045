"""Each test plants one plausible mistake in the oracle (CPU only, through
monkeypatch) and asserts that at least one pin then fails. This shows the pins
are sharp enough to catch a dropped term, a wrong sign, a wrong index or a
transposed operand."""
import numpy as np
import pytest

import oracle
import oracle.formats as F
import oracle.latent_moe as M
import pins
import synth


def _fails(*checks):
    for chk in checks:
        try:
            chk()
        except Exception:
            return True
    return False


def _tiny_vs_brute():
    layers, x = synth.make_config("tiny")
    pins.check_vs_brute(layers[0], x)


def test_swapped_nibbles_caught(monkeypatch):
    def bad_unpack(codes):
        codes = np.asarray(codes, dtype=np.uint8)
        out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.uint8)
        out[..., 0::2] = codes >> 4
        out[..., 1::2] = codes & 0xF
        return out
    monkeypatch.setattr(F, "unpack_codes", bad_unpack)
    assert _fails(pins.check_nibble_order)
    assert _fails(_tiny_vs_brute)


def test_e2m1_exponent_bias_caught(monkeypatch):
    orig = F.e2m1_value
    monkeypatch.setattr(F, "e2m1_value", lambda c: orig(c) * np.where((np.asarray(c) >> 1) & 3, 2.0, 1.0))
    monkeypatch.setattr(oracle, "e2m1_value", F.e2m1_value)
    assert _fails(pins.check_e2m1_table)
    assert _fails(_tiny_vs_brute)


def test_e4m3_subnormal_caught(monkeypatch):
    orig = F.e4m3fn_value
    def bad(b):
        v = orig(b)
        e = (np.asarray(b).astype(np.int64) >> 3) & 0xF
        return np.where(e == 0, v * 2.0, v)
    monkeypatch.setattr(F, "e4m3fn_value", bad)
    monkeypatch.setattr(oracle, "e4m3fn_value", bad)
    assert _fails(pins.check_e4m3_vs_torch)
    assert _fails(pins.check_closed_form_signs_and_subnormal)


def test_scale_block_index_caught(monkeypatch):
    def bad_dequant(codes, scales, gscale):
        q = F.e2m1_value(F.unpack_codes(codes))
        s = F.e4m3fn_value(scales)
        s_full = np.roll(np.repeat(s, 16, axis=-1), 8, axis=-1)  # blocks off by 8
        return q * s_full * np.float64(np.float32(gscale))
    monkeypatch.setattr(F, "dequant_fp4", bad_dequant)
    monkeypatch.setattr(M, "dequant_fp4", bad_dequant)
    monkeypatch.setattr(oracle, "dequant_fp4", bad_dequant)
    assert _fails(pins.check_dequant_vs_brute)
    assert _fails(_tiny_vs_brute)


def test_matrix_scale_dropped_caught(monkeypatch):
    orig = F.dequant_fp4
    bad = lambda c, s, g: orig(c, s, 1.0)
    monkeypatch.setattr(M, "dequant_fp4", bad)
    assert _fails(_tiny_vs_brute)


def test_silu_sign_caught(monkeypatch):
    monkeypatch.setattr(M, "silu", lambda v: v / (1.0 + np.exp(v)))
    assert _fails(pins.check_closed_form_all_ones)
    assert _fails(_tiny_vs_brute)


def test_silu_on_up_instead_of_gate_caught(monkeypatch):
    def bad(v, bank, e):
        wg = M._bank_matrix(bank, "gate", e)
        wu = M._bank_matrix(bank, "up", e)
        wd = M._bank_matrix(bank, "down", e)
        return ((v @ wg.T) * M.silu(v @ wu.T)) @ wd.T
    monkeypatch.setattr(M, "swiglu_expert", bad)
    assert _fails(pins.check_closed_form_signs_and_subnormal, _tiny_vs_brute)


def test_shared_expert_dropped_caught(monkeypatch):
    orig = M.forward
    def bad(layer, *a, **k):
        d = layer.dims
        layer2 = synth.replace(layer, dims=synth.replace(d, n_shared=0))
        return orig(layer2, *a, **k)
    monkeypatch.setattr(oracle, "forward", bad)
    assert _fails(pins.check_closed_form_all_ones)


def test_no_renormalisation_caught(monkeypatch):
    orig = M.gate_topk
    def bad(l32, k):
        idx, w, gap = orig(l32, k)
        l64 = np.asarray(l32, np.float64)
        p = np.exp(l64 - l64.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        return idx, np.take_along_axis(p, idx.astype(np.int64), 1), gap
    monkeypatch.setattr(M, "gate_topk", bad)
    monkeypatch.setattr(oracle, "gate_topk", bad)
    assert _fails(pins.check_gate_vs_torch_topk)
    assert _fails(pins.check_closed_form_routing)


def test_ties_to_higher_index_caught(monkeypatch):
    def bad(l32, k):
        l32 = np.asarray(l32, np.float32)
        T, E = l32.shape
        order = np.lexsort((-np.broadcast_to(np.arange(E), (T, E)), -l32.astype(np.float64)), axis=-1)
        idx = order[:, :k].astype(np.int32)
        l64 = l32.astype(np.float64)
        p = np.exp(l64 - l64.max(1, keepdims=True))
        ps = np.take_along_axis(p, idx.astype(np.int64), 1)
        srt = np.take_along_axis(l64, order, 1)
        return idx, ps / ps.sum(1, keepdims=True), srt[:, k - 1] - srt[:, k]
    monkeypatch.setattr(oracle, "gate_topk", bad)
    assert _fails(pins.check_gate_ties_lower_index)


def test_unstable_permutation_caught(monkeypatch):
    orig = M.route_bookkeeping
    def bad(idx, E):
        counts, offsets, perm = orig(idx, E)
        perm = perm.copy()
        for e in range(E):
            perm[offsets[e]:offsets[e + 1]] = perm[offsets[e]:offsets[e + 1]][::-1]
        return counts, offsets, perm
    monkeypatch.setattr(oracle, "route_bookkeeping", bad)
    assert _fails(pins.check_bookkeeping)


def test_transposed_projection_caught(monkeypatch):
    """U applied transposed (only expressible when hidden == latent)."""
    orig = M.forward
    monkeypatch.setattr(oracle, "forward",
                        lambda layer, *a, **k: orig(synth.replace(layer, U=np.ascontiguousarray(layer.U.T)), *a, **k))

    def check():
        dims = synth.Dims(hidden=64, latent=64, n_experts=8, inter=32, top_k=3, n_shared=1)
        layer = synth.make_layer(dims, 9)
        pins.check_vs_brute(layer, synth.make_x(4, 64, 9))
    assert _fails(check)


def test_stack_without_residual_caught(monkeypatch):
    """Blocks that return the MoE output alone (residual add dropped)."""
    orig = M.block_forward
    def bad(layer, x_bits, eps=1e-6, tokens=None):
        y, res = orig(layer, x_bits, eps, tokens)
        return y - oracle.bf16_value(x_bits)[res.tokens], res
    monkeypatch.setattr(M, "block_forward", bad)
    assert _fails(pins.check_stack_zero_up_projection_is_identity)
    assert _fails(pins.check_stack_vs_torch_chain)


def test_stack_truncating_residual_caught(monkeypatch):
    """Residual stream rounded toward zero between blocks instead of to nearest."""
    orig = M.block_forward
    def bad(layer, x_bits, eps=1e-6, tokens=None):
        y, res = orig(layer, x_bits, eps, tokens)
        t = (np.asarray(y, np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)
        return t.astype(np.float64), res
    monkeypatch.setattr(M, "block_forward", bad)
    assert _fails(pins.check_stack_vs_torch_chain)


def _tiny_mixed_vs_brute():
    d = synth.replace(synth.TINY, gateup_bits=3)
    layer = synth.make_layer(d, 21)
    pins.check_vs_brute(layer, synth.make_x(4, d.hidden, 21))


def test_e1m1_planes_swapped_caught(monkeypatch):
    orig = F.unpack_e1m1
    def bad(codes):   # reads the chunk's three words in the wrong order
        c = np.asarray(codes, dtype=np.uint8)
        lead, nb = c.shape[:-1], c.shape[-1]
        ch = c.reshape(lead + (nb // 12, 12))
        ch = np.concatenate([ch[..., 4:12], ch[..., 0:4]], axis=-1)
        return orig(ch.reshape(lead + (nb,)))
    monkeypatch.setattr(F, "unpack_e1m1", bad)
    monkeypatch.setattr(oracle, "unpack_e1m1", bad)
    assert _fails(pins.check_e1m1_chunk_layout)
    assert _fails(pins.check_e1m1_dequant_vs_brute)
    assert _fails(_tiny_mixed_vs_brute)


def test_e1m1_subnormal_caught(monkeypatch):
    orig = F.e1m1_value
    def bad(c):   # the exponent-0 codes read as normal
        c = np.asarray(c).astype(np.int64)
        v = orig(c)
        return np.where(((c >> 1) & 1) == 0, np.sign(v) * (1.0 + (c & 1) * 0.5) * ((c & 1) > 0), v)
    monkeypatch.setattr(F, "e1m1_value", bad)
    monkeypatch.setattr(oracle, "e1m1_value", bad)
    assert _fails(pins.check_e1m1_table)
    assert _fails(pins.check_e1m1_dequant_vs_brute)


def test_mixed_record_gateup_read_as_fp4_caught(monkeypatch):
    def bad_bank_matrix(bank, proj, e):
        m = getattr(bank, proj)
        return F.dequant_fp4(m.codes[e][..., : m.scales.shape[-1] * 8], m.scales[e], m.gscale[e])
    monkeypatch.setattr(M, "_bank_matrix", bad_bank_matrix)
    assert _fails(_tiny_mixed_vs_brute)


# ---- routing groups: each planted mistake must fail a grouped pin

def _grouped_fails():
    return _fails(pins.check_grouped_vs_brute, pins.check_grouped_repeated_pairs_equal_one_pair,
                  pins.check_grouped_up_projection_per_group)


def test_router_reads_group0_latent_caught(monkeypatch):
    """Every expert's logit read from group 0's latent."""
    def bad(h, R, b, n_groups, latent):
        return h[:, :latent] @ R.T + b
    monkeypatch.setattr(M, "router_logits", bad)
    assert _grouped_fails()


def test_experts_read_group0_latent_caught(monkeypatch):
    """Every expert run on group 0's latent (and added into group 0)."""
    monkeypatch.setattr(M, "group_latent", lambda h, g, latent: h[..., :latent])
    assert _grouped_fails()


def test_shared_expert_in_group1_caught(monkeypatch):
    """The shared expert run on, and added into, group 1."""
    monkeypatch.setattr(M, "SHARED_GROUP", 1)
    assert _grouped_fails()


def test_groups_up_projections_swapped_caught(monkeypatch):
    """z_0 projected with U_1 and z_1 with U_0."""
    src = M.forward

    def fwd(layer, x_bits=None, tokens=None, x_values=None):
        r = src(layer, x_bits, tokens, x_values)
        if getattr(layer.dims, "n_groups", 1) > 1:
            L = layer.dims.latent
            U = oracle.bf16_value(layer.U).copy()
            U[:, :L], U[:, L:2 * L] = U[:, L:2 * L].copy(), U[:, :L].copy()
            r.out = r.z @ U.T
        return r
    monkeypatch.setattr(M, "forward", fwd)
    monkeypatch.setattr(oracle, "forward", fwd)
    assert _grouped_fails()
