"""GPU parity of the adaLN-single modulation (td_adaln_modulate, through the
C ABI) against the oracle's adaln_modulate.

Bounds.  The kernel forms r = x + gate * f with one fp32 fma and rounds it to
bf16, so |r - r_ref| <= 2^-8 |r_ref| + 1e-6 (half a bf16 ulp is at most 2^-8
of the value).  h is computed from the rounded r: each element moves by at
most 2^-8 relative, so the row's rms moves by at most 2^-8 relative too and
the normalised value n = r / rms by at most 2^-7 relative; h = n * a + shift is
then rounded to bf16.  Hence |h - h_ref| <= 2^-8 |h_ref| + 2^-7 |h_ref - shift|
+ 1e-5, shift being the sequence's shift vector.  On the exact-grid inputs the
gated sum is exact in fp32, so r must equal the oracle's r rounded to bf16 bit
for bit.  Shapes cover hidden sizes of one 8-wide chunk to 8192 (one or two
passes, ragged last passes), one to eight tokens per workgroup with a ragged
last run, no residual, missing tables, and the in-place forms."""
import numpy as np
import pytest
import torch

import block_diffusion_lm_td_amd as td
import oracle
import synth
from gpu_util import log

pytestmark = pytest.mark.gpu
AW = synth.ADALN_WORKLOADS


def _bf(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def _f(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _run(d, use_f=True, tables=True, eps=1e-5, inplace=None):
    B, S, H = d["x"].shape
    x = _bf(d["x"])
    f = _bf(d["f"]) if use_f else None
    nan = torch.full((B, S, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    r_out = nan.clone() if use_f else None
    h = nan.clone()
    if inplace == "r_is_x":
        r_out = x
    elif inplace == "h_is_f":
        h = f
    elif inplace == "h_is_x":
        h = x
    tb = {k: (_f(d[k]) if tables else None) for k in ("tab_gate", "tab_shift", "tab_scale", "w_norm")}
    td.td_adaln_modulate(x, f, _f(d["t_mod"]), h, r_out, eps=eps, **tb)
    torch.cuda.synchronize()
    return (None if r_out is None else r_out), h


def _ref(d, use_f=True, tables=True, eps=1e-5):
    f64 = synth.bf16_bits_to_f64
    tb = {k: (d[k] if tables else None) for k in ("tab_gate", "tab_shift", "tab_scale", "w_norm")}
    r, h = oracle.adaln_modulate(f64(d["x"]), f64(d["f"]) if use_f else None, d["t_mod"],
                                 tb["tab_gate"], tb["tab_shift"], tb["tab_scale"], tb["w_norm"], eps)
    shift = d["t_mod"][:, 0, :].astype(np.float64)
    if tables:
        shift = shift + d["tab_shift"]
    return r, h, shift


def _check(r_got, h_got, d, label, use_f=True, tables=True, eps=1e-5, exact=False):
    r_ref, h_ref, shift = _ref(d, use_f, tables, eps)
    h = h_got.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(h).all(), label
    hb = 2.0 ** -8 * np.abs(h_ref) + 2.0 ** -7 * np.abs(h_ref - shift[:, None, :]) + 1e-5
    hw = float((np.abs(h - h_ref) / hb).max())
    rw = 0.0
    if use_f:
        r = r_got.float().cpu().numpy().astype(np.float64)
        if exact:
            want = synth.f32_to_bf16_bits(r_ref.astype(np.float32))
            assert np.array_equal(_bits(r_got), want), f"{label}: r not bit-exact"
        rb = 2.0 ** -8 * np.abs(r_ref) + 1e-6
        rw = float((np.abs(r - r_ref) / rb).max())
    log(f"[adaln] {label}: max err/bound r {rw:.3f}, h {hw:.3f}")
    assert rw <= 1.0 and hw <= 1.0, label


def test_adaln_exact_small():
    w = AW["adaln_exact_b4_s16_h256"]
    d = synth.make_adaln_inputs(w, 81)
    log(f"case adaln {w.name}")
    r, h = _run(d)
    _check(r, h, d, w.name, exact=True)


def test_adaln_realistic_small():
    w = AW["adaln_b4_s16_h256"]
    d = synth.make_adaln_inputs(w, 82)
    log(f"case adaln {w.name}")
    r, h = _run(d)
    _check(r, h, d, w.name)


@pytest.mark.parametrize("B,S,H", [
    (1, 1, 8),          # one 8-wide chunk, 1 token per workgroup
    (3, 5, 136),        # 17 chunks, most threads idle
    (2, 16, 4096),      # exactly one pass of 512 x 8
    (7, 3, 4104),       # two passes, one chunk in the second
    (5, 16, 6144),      # a pass and a half
    (4, 2, 8192),       # the widest: two full passes
    (40, 16, 512),      # 2 tokens per workgroup
    (64, 16, 4096),     # 4 tokens per workgroup (the batched shape)
    (150, 5, 256),      # 4 per workgroup, a ragged last run of 1
    (200, 16, 512),     # 8 per workgroup
    (600, 5, 64),       # 8 per workgroup, each run cut to the sequence's 5
])
def test_adaln_shapes(B, S, H):
    w = AW["adaln_exact_b4_s16_h256"].with_(B=B, S=S, H=H)
    d = synth.make_adaln_inputs(w, 83 + B + H)
    log(f"case adaln exact B{B} S{S} H{H}")
    r, h = _run(d)
    _check(r, h, d, f"exact B{B} S{S} H{H}", exact=True)


@pytest.mark.parametrize("use_f,tables", [(False, True), (True, False), (False, False)])
def test_adaln_optional_inputs(use_f, tables):
    """No residual (r_out untouched: still NaN), missing tables and weight."""
    w = AW["adaln_b4_s16_h256"].with_(B=6, S=7, H=1032)
    d = synth.make_adaln_inputs(w, 84)
    log(f"case adaln optional f={use_f} tables={tables}")
    r, h = _run(d, use_f=use_f, tables=tables, eps=1e-3)
    _check(r, h, d, f"f={use_f} tables={tables}", use_f=use_f, tables=tables, eps=1e-3)


@pytest.mark.parametrize("B,S,H", [
    (64, 16, 1024),     # 4 tokens per workgroup, whole runs
    (150, 5, 256),      # 4 per workgroup, a ragged last run of 1 (its spare loads re-read the row it writes)
])
@pytest.mark.parametrize("mode", ["r_is_x", "h_is_f", "h_is_x"])
def test_adaln_in_place(mode, B, S, H):
    w = AW["adaln_exact_b4_s16_h256"].with_(B=B, S=S, H=H)
    d = synth.make_adaln_inputs(w, 85)
    log(f"case adaln in place {mode} B{B} S{S} H{H}")
    r, h = _run(d, inplace=mode)
    _check(r, h, d, f"in place {mode} B{B} S{S} H{H}", exact=True)


def test_adaln_batched_and_deterministic():
    w = AW["adaln_b64_s16_h4096"]
    d = synth.make_adaln_inputs(w, 86)
    log(f"case adaln {w.name}")
    r, h = _run(d)
    _check(r, h, d, w.name)
    r2, h2 = _run(d)
    assert torch.equal(r.view(torch.int16), r2.view(torch.int16))
    assert torch.equal(h.view(torch.int16), h2.view(torch.int16))
