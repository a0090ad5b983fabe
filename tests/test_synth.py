"""Seeded generators: determinism, shapes, and the bf16 storage cast."""
import numpy as np
import torch

import synth


def test_bf16_cast_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 37,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.0078125, 65504.0, -3.3e38, 1e-40],
                                 np.float32)])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()
    back = synth.bf16_bits_to_f32(ours)
    assert (torch.from_numpy(back) == torch.from_numpy(x).to(torch.bfloat16).float()).all()


def test_attention_inputs_deterministic_and_shaped():
    w = synth.WORKLOADS["bf16_b64_ragged1k_8k"].with_(B=5, ctx_lo=10, ctx_hi=40)
    a = synth.make_attention_inputs(w, 7)
    b = synth.make_attention_inputs(w, 7)
    for k in ("q", "k_blk", "v_blk", "k_ctx", "v_ctx", "offsets"):
        assert (a[k] == b[k]).all()
    assert a["q"].shape == (5, 16, 32, 128) and a["q"].dtype == np.uint16
    assert a["k_ctx"].shape == (a["total_ctx"], 2, 128)
    assert a["offsets"][0] == 0 and (np.diff(a["offsets"]) == a["lengths"]).all()
    assert ((a["lengths"] >= 10) & (a["lengths"] <= 40)).all()
    c = synth.make_attention_inputs(w, 8)
    assert not (a["q"] == c["q"]).all()


def test_explicit_lengths_and_empty_context():
    w = synth.WORKLOADS["tiny_f32_b1_ctx64"].with_(B=3)
    a = synth.make_attention_inputs(w, 1, lengths=[0, 5, 0])
    assert a["total_ctx"] == 5 and a["max_ctx"] == 5
    assert a["q"].dtype == np.float32


def test_peak_logit_model():
    w = synth.WORKLOADS["bf16_b8_ctx4k"].with_(B=2, V=4096)
    c = synth.make_commit_inputs(w, 3)
    x = synth.bf16_bits_to_f32(c["logits"]).reshape(-1, w.V)
    r = np.arange(x.shape[0])
    assert (x[r, c["peak"]] == x.max(axis=1)).all()


def test_loop_logits_peak_grows():
    w = synth.WORKLOADS["bf16_b32_ctx2k_loop"].with_(B=2, V=512)
    base, peak, stored = synth.loop_peak_values(w, 5, 4)
    v = synth.bf16_bits_to_f32(stored)
    assert (np.diff(v, axis=0) >= 0).all()
    x2 = synth.loop_step_logits(base, peak, stored, 2)
    assert (x2[np.arange(x2.shape[0]), peak] == stored[2]).all()
    x0 = synth.loop_step_logits(base, peak, stored, 0)
    assert (x0 == base).all()


def test_lmhead_inputs_deterministic_and_shaped():
    w = synth.LMHEAD_WORKLOADS["lmhead_bf16_b4_h256_v5000"]
    a = synth.make_lmhead_inputs(w, 11)
    b = synth.make_lmhead_inputs(w, 11)
    assert a["hidden"].shape == (4, 16, 256) and a["hidden"].dtype == np.uint16
    assert a["w_head"].shape == (5000, 256) and a["w_head"].dtype == np.uint16
    assert np.array_equal(a["hidden"], b["hidden"]) and np.array_equal(a["w_head"], b["w_head"])
    c = synth.make_lmhead_inputs(w, 12)
    assert not np.array_equal(a["w_head"], c["w_head"])
    # the head's spread: sw = logit_std / sqrt(H)
    sw = synth.bf16_bits_to_f64(a["w_head"]).std()
    assert abs(sw - 2.0 / 16.0) < 0.005


def test_mamba_inputs_deterministic_and_ranged():
    w = synth.MAMBA_WORKLOADS["mamba_b4_s16_h8"]
    a = synth.make_mamba_inputs(w, 3)
    b = synth.make_mamba_inputs(w, 3)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    assert a["x"].shape == (4, 16, 8, 64) and a["x"].dtype == np.uint16
    assert a["Bm"].shape == (4, 16, 2, 128) and a["h0"].shape == (4, 8, 64, 128)
    assert a["h0"].dtype == np.float32 and a["dt"].dtype == np.float32
    assert (a["dt"] >= 1e-3 * 0.999).all() and (a["dt"] <= 0.1 * 1.001).all()
    assert (a["A"] <= -1.0 + 1e-6).all() and (a["A"] >= -16.0 - 1e-4).all()


def test_adaln_inputs_deterministic_and_exact_grid():
    w = synth.ADALN_WORKLOADS["adaln_exact_b4_s16_h256"]
    a = synth.make_adaln_inputs(w, 3)
    b = synth.make_adaln_inputs(w, 3)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    assert a["x"].shape == (4, 16, 256) and a["x"].dtype == np.uint16
    assert a["t_mod"].shape == (4, 3, 256) and a["t_mod"].dtype == np.float32
    x = synth.bf16_bits_to_f64(a["x"])
    f = synth.bf16_bits_to_f64(a["f"])
    assert np.array_equal(x * 64, np.round(x * 64)) and np.abs(x).max() < 4
    assert np.array_equal(f * 64, np.round(f * 64))
    g = a["t_mod"][:, 2, :].astype(np.float64)[:, None, :] + a["tab_gate"].astype(np.float64)
    r = x + g * f
    # the gated sum is exact in fp32: fp32 arithmetic reproduces it
    r32 = np.float32(x) + (np.float32(a["t_mod"][:, 2, :])[:, None, :] + a["tab_gate"]) * np.float32(f)
    assert np.array_equal(r32.astype(np.float64), r)
    c = synth.make_adaln_inputs(synth.ADALN_WORKLOADS["adaln_b4_s16_h256"], 3)
    assert abs(synth.bf16_bits_to_f64(c["x"]).std() - 2.0) < 0.1
