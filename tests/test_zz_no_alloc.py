"""td_denoise_step_noalloc: the denoise step on the library's own per-GPU
scratch array instead of a caller workspace.

Checked through the C ABI against td_denoise_step with a workspace on the
same inputs: two calls in a row, the second on a smaller input than the
first (the array keeps the first call's contents), each bit for bit equal to
the workspace route in every output (attention out, commit, token, maxprob,
n_commit, masked_out, tokens, n_masked_left).  Both routes run the same
deterministic kernels, so equality is exact, stricter than the oracle
tolerances the workspace route is held to elsewhere.
"""
import ctypes

import numpy as np
import pytest
import torch

import block_diffusion_lm_td_amd as td
from block_diffusion_lm_td_amd import _td
import synth
from gpu_util import dev, log, upload_attn

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _no_plan_override(monkeypatch):
    monkeypatch.delenv("TD_ATTN_GRID", raising=False)
    monkeypatch.delenv("TD_COMMIT_SPLIT", raising=False)


def _inputs(w, seed, lengths, frac):
    a = synth.make_attention_inputs(w, seed, lengths=lengths)
    c = synth.make_commit_inputs(w, seed)
    el = synth.make_eligible(w, seed, frac)
    return a, c, el


def _outs(B, S, q):
    z = lambda shape, dt: torch.zeros(shape, dtype=dt, device="cuda")
    return dict(out=torch.full_like(q, 7.0), commit=z((B, S), torch.uint8),
                token=z((B, S), torch.int32), maxprob=z((B, S), torch.float32),
                n_commit=z((B,), torch.int32), masked_out=z((B, S), torch.uint8),
                tokens=torch.full((B, S), -1, dtype=torch.int32, device="cuda"),
                n_left=torch.full((1,), -3, dtype=torch.int32, device="cuda"))


def _structs(w, a, d, logits, masked_in, o):
    aa = td.attn_args(d["q"], d["k_blk"], d["v_blk"], d["k_ctx"], d["v_ctx"], d["offsets"], o["out"],
                      a["total_ctx"], a["max_ctx"])
    cc = td.commit_args(logits, o["commit"], o["token"], w.gamma, masked_in, o["maxprob"],
                        o["n_commit"], o["masked_out"], o["tokens"], o["n_left"])
    return aa, cc


def _compare(label, x, y):
    for k in x:
        assert torch.equal(x[k], y[k]), f"{label}: {k} differs"


CASES = [
    # (workload, seed, context lengths, eligible fraction)
    ("bf16_b8_ctx4k", 8101, [4096, 3000, 17, 0, 2500, 4096, 1, 777], 0.7),
    ("bf16_b8_ctx4k", 8102, [300, 0, 65], 1.0),
]


def test_noalloc_matches_workspace_route_two_calls_second_smaller():
    L = td.lib()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    for i, (name, seed, lengths, frac) in enumerate(CASES):
        w = synth.WORKLOADS[name].with_(B=len(lengths), V=131072 if i == 0 else 5000)
        a, c, el = _inputs(w, seed, lengths, frac)
        log(f"case noalloc call {i}: B={w.B} lengths={lengths} V={w.V}")
        d = upload_attn(a)
        logits = dev(c["logits"], w.dtype)
        masked_in = torch.from_numpy(el).to("cuda")
        ref, got = _outs(w.B, w.S, d["q"]), _outs(w.B, w.S, d["q"])
        ra, rc = _structs(w, a, d, logits, masked_in, ref)
        ga, gc = _structs(w, a, d, logits, masked_in, got)
        need = L.td_denoise_workspace_bytes(ctypes.byref(ra), ctypes.byref(rc))
        assert 0 < need <= _td.TD_NOALLOC_SCRATCH_BYTES
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        rr = L.td_denoise_step(ctypes.byref(ra), ctypes.byref(rc), ctypes.c_void_p(ws.data_ptr()), need, sp)
        assert rr == _td.TD_OK, _td.status_str(rr)
        rg = L.td_denoise_step_noalloc(ctypes.byref(ga), ctypes.byref(gc), sp)
        assert rg == _td.TD_OK, _td.status_str(rg)
        torch.cuda.synchronize()
        _compare(f"call {i}", got, ref)
        assert int(got["n_left"].item()) == int(got["masked_out"].sum().item())
        assert not bool((got["out"] == 7.0).all())
        log(f"[noalloc] call {i}: identical to td_denoise_step ({int(got['commit'].sum())} commits)")
