"""The seeded input generator: determinism, distributions, and the fp4
quantiser checked against the oracle's (independent) decoders."""
import numpy as np
import torch

import oracle
import synth


def test_philox_known_answers():
    # Known-answer vectors published with Random123 for philox4x32_10.
    assert synth.philox4x32_10([0, 0, 0, 0], [0, 0]).tolist() == [
        0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]
    assert synth.philox4x32_10([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2).tolist() == [
        0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]
    assert synth.philox4x32_10([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344],
                               [0xA4093822, 0x299F31D0]).tolist() == [
        0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]


def test_normals_deterministic_and_standard():
    a = synth.normal_f32(7, 1, 0, (1 << 18,))
    b = synth.normal_f32(7, 1, 0, (1 << 18,))
    c = synth.normal_f32(7, 1, 1, (1 << 18,))
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert abs(a.mean()) < 0.01 and abs(a.std() - 1) < 0.01
    # any prefix of a stream is the same draws (counter-based)
    assert np.array_equal(synth.normal_f32(7, 1, 0, (1001,)), a[:1001])


def test_bf16_rounding_matches_torch():
    v = synth.normal_f32(3, 2, 0, (50000,), 5.0)
    got = synth.f32_to_bf16(v)
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_zipf_bias():
    b = synth.zipf_bias(512, 1.1)
    assert b[0] == 0.0 and np.allclose(b, -1.1 * np.log(np.arange(1, 513)), rtol=1e-6)


def _all_e4m3():
    vals = oracle.e4m3fn_value(np.arange(0x7F))  # non-negative, finite
    return vals


def test_quantizer_against_decoders():
    w = synth.normal_f32(11, 5, 0, (3, 48, 96), 0.05)
    w[1, 3, 16:32] = 0.0          # an all-zero block
    w[2, 5, 7] = 10.0             # an outlier sets the matrix scale
    q = synth.quantize_fp4(w)
    e4 = _all_e4m3()
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    for m in range(3):
        g = np.float32(q.gscale[m])
        amax = np.abs(w[m]).max()
        assert g == np.float32(amax / np.float32(6 * 448))
        deq = oracle.dequant_fp4(q.codes[m], q.scales[m], g)
        blocks = np.abs(w[m]).reshape(48, 6, 16).max(-1)
        s = oracle.e4m3fn_value(q.scales[m])
        # each block scale is a nearest E4M3 value to amax_b / (6 g)
        target = (blocks.astype(np.float32) / (np.float32(6.0) * g)).astype(np.float64)
        best = np.abs(e4[None, None, :] - target[..., None]).min(-1)
        assert np.allclose(np.abs(s - target), best, rtol=0, atol=1e-12)
        # each code is a nearest e2m1 value to w / (s g) (saturating at 6)
        sg = np.repeat(s, 16, axis=1) * np.float64(g)
        ratio = np.where(sg > 0, w[m] / np.where(sg > 0, sg, 1), 0.0)
        qv = deq / np.where(sg > 0, sg, 1)
        nearest = np.abs(np.abs(ratio)[..., None] - grid).min(-1)
        assert np.all(np.abs(np.abs(qv) - np.minimum(np.abs(ratio), 6.0)) <= nearest + 1e-6)
        assert np.all((np.sign(qv) == np.sign(ratio)) | (qv == 0))
        # zero block -> zero scale and zero codes
        if m == 1:
            assert q.scales[1, 3, 1] == 0 and np.all(deq[3, 16:32] == 0)
    # the outlier itself is reproduced to within one e2m1 step at the top
    assert abs(oracle.dequant_fp4(q.codes[2], q.scales[2], q.gscale[2])[5, 7] - 10.0) < 10.0 / 6


def test_quantized_weights_track_normals():
    """N(0, 1/fan_in) weights through the quantiser keep their scale: the
    relative RMS error of 4-bit weights is about 10%."""
    layer = synth.make_layer(synth.Dims(256, 64, 4, 32, 2, 1), 1)
    w = synth.normal_f32(1, synth.TAG_GATE, 0, (32, 64), 64 ** -0.5)
    deq = oracle.dequant_fp4(layer.experts.gate.codes[0], layer.experts.gate.scales[0],
                             layer.experts.gate.gscale[0])
    rel = np.sqrt(((deq - w) ** 2).mean() / (w ** 2).mean())
    assert 0.02 < rel < 0.2, rel


def test_layer_shapes_and_determinism():
    d = synth.TINY
    a = synth.make_layer(d, 5)
    b = synth.make_layer(d, 5)
    assert a.D.shape == (d.latent, d.hidden) and a.U.shape == (d.hidden, d.latent)
    assert a.R.shape == (d.n_experts, d.latent)
    assert a.experts.gate.codes.shape == (d.n_experts, d.inter, d.latent // 2)
    assert a.experts.down.scales.shape == (d.n_experts, d.latent, d.inter // 16)
    assert a.shared.count == 1
    for p in ("gate", "up", "down"):
        assert np.array_equal(getattr(a.experts, p).codes, getattr(b.experts, p).codes)
    assert not np.array_equal(a.experts.gate.codes[0], a.experts.gate.codes[1])
