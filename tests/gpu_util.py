"""Helpers of the GPU parity tests: upload seeded inputs, run the C ABI
through the binding, compare with the oracle.

Gates (also stated in the tests' docstrings):
  attention, bf16 inputs: max abs err <= 2e-2, mean abs err <= 2e-3 versus
    float64, plus relative L2 error <= 1e-2 (the absolute gates are loose
    for inputs scaled by 1/sqrt(128), whose outputs are ~1e-3);
  attention, fp32 inputs: max abs err <= 1e-4;
  commit: token ids bit-exact at every position; commit mask, n_commit,
    masked_out and committed ids bit-exact, except positions whose oracle
    max-probability lies within 1e-4 of gamma (and sequences whose
    force-one choice is within 1e-4 of a tie, or whose force-one trigger
    depends on such a position), which are excluded and counted; maxprob
    within 2e-5 absolute.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import block_diffusion_lm_td_amd as td
import oracle
import synth

BAND = 1e-4


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(arr: np.ndarray, dtype: str):
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to("cuda")


def f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    return synth.bf16_bits_to_f64(arr) if dtype == "bf16" else np.asarray(arr, np.float64)


def upload_attn(a: dict):
    dt = a["dtype"]
    d = {k: dev(a[k], dt) for k in ("q", "k_blk", "v_blk", "k_ctx", "v_ctx")}
    d["offsets"] = torch.from_numpy(a["offsets"]).to("cuda")
    d["out"] = torch.empty_like(d["q"])
    return d


def run_attn(d: dict, a: dict, scale=0.0):
    td.td_block_attn(d["q"], d["k_blk"], d["v_blk"], d["k_ctx"], d["v_ctx"], d["offsets"], d["out"],
                     total_ctx=a["total_ctx"], max_ctx=a["max_ctx"], scale=scale)
    torch.cuda.synchronize()
    return d["out"].float().cpu().numpy().astype(np.float64)


def oracle_attn(a: dict, seqs=None, scale=None):
    """Oracle output for the sequences ``seqs`` (default: all)."""
    dt = a["dtype"]
    B = a["q"].shape[0]
    seqs = range(B) if seqs is None else seqs
    outs = []
    for b in seqs:
        lo, hi = int(a["offsets"][b]), int(a["offsets"][b + 1])
        o = oracle.block_attention(
            f64(a["q"][b:b + 1], dt), f64(a["k_blk"][b:b + 1], dt), f64(a["v_blk"][b:b + 1], dt),
            f64(a["k_ctx"][lo:hi], dt), f64(a["v_ctx"][lo:hi], dt), np.array([0, hi - lo]), scale)
        outs.append(o[0])
    return np.stack(outs)


def check_attn(got: np.ndarray, ref: np.ndarray, label: str, fp32: bool = False):
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    log(f"[attn] {label}: max_abs={mx:.3e} mean_abs={mean:.3e} rel_l2={rel:.3e}")
    assert np.isfinite(got).all(), label
    if fp32:
        assert mx <= 1e-4, label
    else:
        assert mx <= 2e-2 and mean <= 2e-3 and rel <= 1e-2, label
    return mx, mean, rel


def upload_commit(logits_bits: np.ndarray, dtype: str, masked_in=None):
    B, S, V = logits_bits.shape
    d = dict(logits=dev(logits_bits, dtype),
             commit=torch.empty((B, S), dtype=torch.uint8, device="cuda"),
             token=torch.empty((B, S), dtype=torch.int32, device="cuda"),
             maxprob=torch.empty((B, S), dtype=torch.float32, device="cuda"),
             n_commit=torch.empty((B,), dtype=torch.int32, device="cuda"),
             masked_out=torch.empty((B, S), dtype=torch.uint8, device="cuda"),
             tokens=torch.full((B, S), -1, dtype=torch.int32, device="cuda"),
             n_masked_left=torch.full((1,), -7, dtype=torch.int32, device="cuda"))
    d["masked_in"] = None if masked_in is None else torch.from_numpy(
        np.ascontiguousarray(masked_in, dtype=np.uint8)).to("cuda")
    return d


def run_commit(d: dict, gamma: float):
    td.td_commit(d["logits"], d["commit"], d["token"], gamma=gamma, masked_in=d["masked_in"],
                 maxprob=d["maxprob"], n_commit=d["n_commit"], masked_out=d["masked_out"],
                 tokens=d["tokens"], n_masked_left=d["n_masked_left"])
    torch.cuda.synchronize()
    return {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in d.items()
            if k in ("commit", "token", "maxprob", "n_commit", "masked_out", "tokens", "n_masked_left")}


def compare_commit(g: dict, ref: dict, masked_in, gamma: float, tokens_in, label: str,
                   seqs=None):
    """Bit-exact comparison with the near-gamma exclusions; returns counts."""
    p = np.asarray(ref["maxprob"])
    B, S = p.shape
    seqs = list(range(B)) if seqs is None else list(seqs)
    elig_all = np.ones((B, S), bool) if masked_in is None else np.asarray(masked_in).astype(bool)
    g32 = float(np.float32(gamma))
    # every position: argmax id exact, maxprob close
    gt = g["token"][seqs]
    assert (gt == ref["token"]).all(), f"{label}: argmax ids differ at " \
        f"{np.argwhere(gt != ref['token'])[:5].tolist()}"
    dp = float(np.abs(g["maxprob"][seqs] - p).max())
    assert dp <= 2e-5, f"{label}: maxprob differs by {dp:.3e}"
    excluded_pos = excluded_seq = 0
    for k, b in enumerate(seqs):
        el = elig_all[b]
        pb = p[k]
        near = el & (np.abs(pb - g32) < BAND)
        sure_pass = el & (pb >= g32 + BAND)
        gc = g["commit"][b].astype(bool)
        rc = np.asarray(ref["commit"][k]).astype(bool)
        # internal consistency of the GPU's own outputs
        assert not (gc & ~el).any(), f"{label}: committed an ineligible position (b={b})"
        assert (g["masked_out"][b].astype(bool) == (el & ~gc)).all(), f"{label}: masked_out (b={b})"
        assert g["n_commit"][b] == gc.sum(), f"{label}: n_commit (b={b})"
        exp_tok = np.where(gc, g["token"][b], tokens_in[b])
        assert (g["tokens"][b] == exp_tok).all(), f"{label}: tokens (b={b})"
        if sure_pass.any():
            keep = ~near
            excluded_pos += int(near.sum())
            assert (gc[keep] == rc[keep]).all(), f"{label}: commit mask differs (b={b}) " \
                f"gpu={gc.astype(int).tolist()} ref={rc.astype(int).tolist()} p={pb.tolist()}"
        elif near.any():
            excluded_seq += 1          # whether force-one fires depends on a near-gamma position
        elif el.any():
            pe = np.sort(pb[el])[::-1]
            if len(pe) > 1 and pe[0] - pe[1] < BAND:
                excluded_seq += 1      # force-one choice within the band of a tie
            else:
                assert (gc == rc).all(), f"{label}: force-one differs (b={b})"
        else:
            assert not gc.any()
    if len(seqs) == B:
        assert int(g["n_masked_left"][0]) == int(g["masked_out"].astype(bool).sum()), label
    log(f"[commit] {label}: seqs={len(seqs)} committed={int(g['commit'][seqs].sum())} "
        f"excluded_positions={excluded_pos} excluded_sequences={excluded_seq}")
    return excluded_pos, excluded_seq


def oracle_commit(logits_bits, dtype, masked_in, gamma, seqs=None):
    x = logits_bits if seqs is None else logits_bits[list(seqs)]
    el = None if masked_in is None else (masked_in if seqs is None else masked_in[list(seqs)])
    return oracle.confidence_commit(f64(x, dtype), el, gamma)
