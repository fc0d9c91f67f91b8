"""The benchmark's FLOP counter is the appendix G closed-form model; pin it to
the values appendix G.7 prints (tests/golden/g7_flops.json)."""
import json
import os

from sketch_attention_flashsa_amd import flops

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "g7_flops.json")))


def test_g7_values_reproduced():
    got = flops.g7_numbers()
    for key, digits in GOLD["printed_digits"].items():
        assert round(got[key], digits) == GOLD[key], (key, got[key], GOLD[key])


def test_sa_layer_closed_form_terms():
    # G.3: 2Ld^2 + 14 L_s d^2 + 4 L_s L d, with the SwiGLU FFN (inner 2d) = 12 L_s d^2
    L, Ls, d = 100_000, 1024, 128
    assert flops.swiglu(Ls, d, 2 * d) == 12 * Ls * d * d
    assert flops.sa_layer(L, Ls, d) == 2 * L * d * d + 14 * Ls * d * d + 4 * Ls * L * d
    # G.2: 12LD^2 + 4LDh + 20D^2
    D, h = 1024, 16
    assert flops.stca_layer(L, D, h) == 12 * L * D * D + 4 * L * D * h + 20 * D * D


def test_on_path_counter_is_the_affinity_aggregation_term():
    # one head of the G.3 layer at d = dh, L_s = m: 4 L_s L d
    assert flops.sa_forward_flops(1000, 1, 64, 32) == 4 * 64 * 1000 * 32
    assert flops.sa_forward_flops(1000, 8, 64, 32) == 8 * flops.sa_forward_flops(1000, 1, 64, 32)
