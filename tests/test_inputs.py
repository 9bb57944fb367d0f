"""Seeded input generator: bf16 rounding, determinism, page-table structure (CPU)."""

import numpy as np
import torch

from io_aware_exact_fa_amd.inputs import (bf16_round, decode_inputs,
                                          decode_lengths_and_table, grad_output,
                                          prefill_inputs)


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100_000, dtype=np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, -3.5e-20,
                                  65504.0, 1e30], dtype=np.float32)])
    vals, bits = bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(bits, ref.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(vals, ref.to(torch.float32).numpy())


def test_prefill_deterministic_and_scaled():
    a = prefill_inputs(1, 2, 1, 33, 8, seed=4)
    b = prefill_inputs(1, 2, 1, 33, 8, seed=4)
    for name in ("q", "k", "v"):
        assert np.array_equal(a[name + "_bits"], b[name + "_bits"])
    half = prefill_inputs(1, 2, 1, 33, 8, seed=4, draw_scale=0.5)
    # x0.5 is exact before rounding, so the rounded values halve exactly
    assert np.array_equal(half["q"], a["q"] * np.float32(0.5))
    f = prefill_inputs(1, 1, 1, 5, 4, seed=1, dtype="f32")
    assert f["q"].dtype == np.float32 and "q_bits" not in f


def test_grad_output_independent_of_qkv():
    a, abits = grad_output(1, 2, 33, 8, seed=4)
    b, bbits = grad_output(1, 2, 33, 8, seed=4)
    assert np.array_equal(abits, bbits) and a.shape == (1, 2, 33, 8)
    assert np.array_equal(bf16_round(a)[1], abits)  # bf16-exact values
    qkv = prefill_inputs(1, 2, 2, 33, 8, seed=4)
    assert not np.array_equal(a, qkv["q"])  # its own stream, not a copy of Q
    h, _ = grad_output(1, 2, 33, 8, seed=4, draw_scale=0.5)
    assert np.array_equal(h, a * np.float32(0.5))


def test_decode_table_is_a_permutation():
    meta = decode_lengths_and_table(8, 4, 16, 16, 1, 200, seed=5)
    t = meta["page_table"]
    used = t[t >= 0]
    assert sorted(used.tolist()) == list(range(meta["num_pages"]))
    for b in range(8):
        pb = int(meta["pages"][b])
        assert pb == (int(meta["seqlens"][b]) + 15) // 16
        assert np.all(t[b, :pb] >= 0) and np.all(t[b, pb:] == -1)
    assert meta["seqlens"].min() >= 1 and meta["seqlens"].max() <= 200


def test_decode_cache_places_sequence_pages():
    meta = decode_inputs(3, 4, 2, 8, 16, 5, 40, seed=6)
    from io_aware_exact_fa_amd.inputs import decode_sequence_kv
    for b in range(3):
        pb = int(meta["pages"][b])
        kv, kb, vv, vb = decode_sequence_kv(6, b, pb, 2, 16, 8)
        phys = meta["page_table"][b, :pb]
        assert np.array_equal(meta["kcache_bits"][phys], kb)
        assert np.array_equal(meta["vcache"][phys], vv)


def test_stress_inputs_shapes_and_rounding():
    from io_aware_exact_fa_amd.inputs import STRESS_KINDS, bf16_bits_to_f32, stress_inputs
    for kind in STRESS_KINDS:
        a = stress_inputs(kind, 1, 2, 1, 200, 64, seed=5)
        b = stress_inputs(kind, 1, 2, 1, 200, 64, seed=5)
        for name in ("q", "k", "v"):
            assert np.array_equal(a[name + "_bits"], b[name + "_bits"])
            assert np.array_equal(bf16_bits_to_f32(a[name + "_bits"]), a[name])
    r = stress_inputs("rising", 1, 2, 1, 200, 64, seed=5)
    assert np.all(r["q"][..., 0] == 4.0)
    # the ramp dominates dim 0 of the keys: increasing along the sequence
    assert np.all(np.diff(r["k"][0, 0, ::20, 0]) > 0)
    f = stress_inputs("flat", 1, 2, 1, 200, 64, seed=5)
    assert np.all(f["q"] == 0.0)


def test_decode_stress_ramps_by_position():
    from io_aware_exact_fa_amd.inputs import decode_inputs, decode_stress
    m = decode_inputs(2, 4, 2, 32, 16, 1, 100, seed=3, seqlens=[50, 100])
    s = decode_stress(m, "rising", 100)
    t = m["page_table"]
    for b, L in enumerate([50, 100]):
        for tok in (0, L // 2, L - 1):
            pg, sl = t[b, tok // 16], tok % 16
            delta = s["kcache"][pg, :, sl, 0] - m["kcache"][pg, :, sl, 0]
            assert np.allclose(delta, 849.0 * tok / 100, rtol=0, atol=4.0)
    assert np.all(s["q"][..., 0] == 4.0)
    # values other than dim 0 of K are untouched
    assert np.array_equal(s["kcache"][..., 1:], m["kcache"][..., 1:])
    assert np.array_equal(s["vcache_bits"], m["vcache_bits"])
