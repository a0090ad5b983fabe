"""GPU parity of the denoiser Mamba-2 block scan (td_mamba_block_scan, through
the C ABI) against the oracle's mamba_block_scan.

The kernel computes in fp32 and rounds y to bf16, so the bound per element is
|got - ref| <= 2^-8 |ref| + 1e-3: bf16 rounding moves a value by at most half
an ulp, which is 2^-8 of it just above a power of two, and 1e-3 covers the
fp32 sums (a 128-term dot product of magnitude ~100 carries an fp32 error
near 1e-5).  Cases span every supported head dim, state sizes and
token counts, (sequence, head) counts that do not fill the last workgroup,
and the batched shape (64 x 128 heads, sampled sequences)."""
import numpy as np
import pytest
import torch

import block_diffusion_lm_td_amd as td
import oracle
import synth
from gpu_util import log

pytestmark = pytest.mark.gpu
MW = synth.MAMBA_WORKLOADS


def _bf(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda")


def _f(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def _run(d):
    B, S, H, P = d["x"].shape
    y = torch.full((B, S, H, P), float("nan"), dtype=torch.bfloat16, device="cuda")
    td.td_mamba_block_scan(_bf(d["x"]), _f(d["dt"]), _f(d["A"]), _bf(d["Bm"]), _bf(d["Cm"]),
                           _f(d["D"]), _f(d["h0"]), y)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def _ref(d, seqs=None):
    f64 = synth.bf16_bits_to_f64
    sl = slice(None) if seqs is None else list(seqs)
    y, _ = oracle.mamba_block_scan(f64(d["x"][sl]), d["dt"][sl], d["A"], f64(d["Bm"][sl]),
                                   f64(d["Cm"][sl]), d["D"], d["h0"][sl])
    return y


def _check(got, ref, label):
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-3
    worst = float((err / bound).max())
    log(f"[mamba] {label}: max abs {float(err.max()):.3e}, max err/bound {worst:.3f}, "
        f"|ref| max {float(np.abs(ref).max()):.2f}")
    assert np.isfinite(got).all(), label
    assert worst <= 1.0, label


def test_mamba_small_full():
    w = MW["mamba_b4_s16_h8"]
    d = synth.make_mamba_inputs(w, 71)
    log("case mamba", w)
    _check(_run(d), _ref(d), w.name)


@pytest.mark.parametrize("S,H,P,N,G", [(16, 3, 16, 32, 1), (5, 8, 32, 64, 4), (1, 6, 64, 128, 3),
                                       (16, 10, 128, 256, 5), (13, 4, 64, 32, 2), (16, 7, 64, 1024, 7)])
def test_mamba_shapes(S, H, P, N, G):
    w = MW["mamba_b4_s16_h8"].with_(B=3, S=S, H=H, P=P, N=N, G=G)
    d = synth.make_mamba_inputs(w, 72 + S + H)
    log(f"case mamba S={S} H={H} P={P} N={N} G={G}")
    _check(_run(d), _ref(d), f"S={S} H={H} P={P} N={N} G={G}")


def test_mamba_batched_sampled_and_deterministic():
    w = MW["mamba_b64_s16_h128"]
    d = synth.make_mamba_inputs(w, 73)
    log("case mamba b64 h128 sampled")
    got = _run(d)
    seqs = [0, 31, 63]
    _check(got[seqs], _ref(d, seqs), "b64 h128 (3 sequences)")
    again = _run(d)
    assert np.array_equal(got, again), "not deterministic"
