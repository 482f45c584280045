"""The oracle against facts outside itself (CPU only)."""
import numpy as np
import pytest

import pins
import synth


def test_e2m1_table():
    pins.check_e2m1_table()


def test_e4m3_vs_torch():
    pins.check_e4m3_vs_torch()


def test_bf16_vs_torch():
    pins.check_bf16_vs_torch()


def test_nibble_order():
    pins.check_nibble_order()


def test_dequant_vs_brute():
    pins.check_dequant_vs_brute()


def test_page_dimensions():
    pins.check_page_dimensions()


def test_record_bytes():
    pins.check_record_bytes()


def test_gate_vs_torch_topk():
    pins.check_gate_vs_torch_topk()


def test_gate_ties_lower_index():
    pins.check_gate_ties_lower_index()


def test_gate_invariants():
    pins.check_gate_invariants()


def test_dense_softmax_when_k_equals_E():
    pins.check_dense_softmax_when_k_equals_E()


def test_bookkeeping():
    pins.check_bookkeeping()


def test_closed_form_all_ones():
    pins.check_closed_form_all_ones()


def test_closed_form_routing():
    pins.check_closed_form_routing()


def test_closed_form_signs_and_subnormal():
    pins.check_closed_form_signs_and_subnormal()


def test_identical_experts_routing_free():
    pins.check_identical_experts_routing_free()


def test_single_expert_no_shared():
    pins.check_single_expert_no_shared()


def test_vs_brute_tiny():
    layers, x = synth.make_config("tiny")
    pins.check_vs_brute(layers[0], x)


def test_vs_brute_tiny_zipf_bias():
    cfg = synth.replace(synth.CONFIGS["tiny"], bias="zipf", seed=4)
    layers, x = synth.make_config(cfg)
    pins.check_vs_brute(layers[0], x)


def test_vs_brute_145b_expert_shapes():
    """Full 145B expert and projection shapes (2560 / 1792 / 640, top-10 +
    shared) with fewer experts so the brute force stays quick."""
    dims = synth.replace(synth.E145, n_experts=24)
    layer = synth.make_layer(dims, 2)
    x = synth.make_x(2, dims.hidden, 2)
    pins.check_vs_brute(layer, x)


def test_standard_moe_when_identity_projections():
    """hidden == latent with D = U = I: the layer is a plain top-k MoE plus a
    shared expert, evaluated by the brute force directly on x."""
    dims = synth.Dims(hidden=64, latent=64, n_experts=8, inter=32, top_k=3, n_shared=1)
    layer = synth.make_layer(dims, 9)
    eye = np.where(np.eye(64, dtype=bool), np.uint16(0x3F80), np.uint16(0)).astype(np.uint16)
    layer = synth.replace(layer, D=eye, U=eye.copy())
    x = synth.make_x(6, 64, 9)
    pins.check_vs_brute(layer, x)


def test_dense_all_experts_tiny():
    layers, x = synth.make_config("tiny")
    pins.check_dense_all_experts(layers[0], x)


def test_rmsnorm_vs_torch():
    pins.check_rmsnorm_vs_torch()


def test_block_residual():
    pins.check_block_residual()


def test_bf16_rounding_vs_torch():
    pins.check_bf16_rounding_vs_torch()


def test_stack_zero_up_projection_is_identity():
    pins.check_stack_zero_up_projection_is_identity()


def test_stack_vs_torch_chain():
    pins.check_stack_vs_torch_chain()


def test_e1m1_table():
    pins.check_e1m1_table()


def test_e1m1_chunk_layout():
    pins.check_e1m1_chunk_layout()


def test_e1m1_dequant_vs_brute():
    pins.check_e1m1_dequant_vs_brute()


def test_e1m1_quantiser_error():
    pins.check_e1m1_quantiser_error()


def test_vs_brute_tiny_mixed_record():
    """A tiny layer with 3-bit E1M1 gate/up experts (and e2m1 down)."""
    d = synth.replace(synth.TINY, gateup_bits=3)
    layer = synth.make_layer(d, 21)
    x = synth.make_x(6, d.hidden, 21)
    pins.check_vs_brute(layer, x)


def test_grouped_vs_brute():
    pins.check_grouped_vs_brute()


def test_grouped_repeated_pairs_equal_one_pair():
    pins.check_grouped_repeated_pairs_equal_one_pair()


def test_grouped_up_projection_per_group():
    pins.check_grouped_up_projection_per_group()
