"""GPU parity of the decode-shaped attention path (at most 16 query rows per
KV head: G heads x S positions, G*S <= 16, bf16, D = 128), which
td_block_attn takes by itself, against the fp64 oracle.  Gates as for the
block path (tests/gpu_util.py): max abs <= 2e-2, mean abs <= 2e-3, relative
L2 <= 1e-2 for bf16 inputs.  Cases span splits of the 32-key blocks over
1 to 4000 waves (units whole in one wave, or cut into pieces), empty and
one-key contexts, the batched cache at S = 1 (sampled), 64K contexts, every
G*S <= 16 split, and the gated step."""
import numpy as np
import pytest
import torch

import block_diffusion_lm_td_amd as td
import synth
from gpu_util import check_attn, dev, log, oracle_attn, run_attn, upload_attn

pytestmark = pytest.mark.gpu
W = synth.WORKLOADS


def test_decode_b64_ragged_sampled_and_deterministic():
    w = W["bf16_b64_ragged1k_8k_s1"]
    a = synth.make_attention_inputs(w, 2001)
    d = upload_attn(a)
    log("case decode b64 ragged S=1")
    got = run_attn(d, a)
    seqs = [0, 9, int(np.argmax(a["lengths"])), int(np.argmin(a["lengths"])), 63]
    check_attn(got[seqs], oracle_attn(a, seqs), f"decode b64 ragged sampled seqs={seqs}")
    first = d["out"].clone()
    run_attn(d, a)
    assert torch.equal(first.view(torch.int16), d["out"].view(torch.int16)), "not deterministic"


def test_decode_short_and_empty_contexts():
    """Contexts of 0 .. 600 keys: units of one to 19 blocks, empty caches (the
    one block key only), ragged last blocks."""
    rng = np.random.default_rng(2002)
    lengths = rng.integers(0, 600, 50)
    lengths[:6] = [0, 1, 255, 256, 257, 511]
    w = W["bf16_b64_ragged1k_8k_s1"].with_(B=50)
    a = synth.make_attention_inputs(w, 2003, lengths=lengths)
    log("case decode short/empty contexts", lengths[:10])
    check_attn(run_attn(upload_attn(a), a), oracle_attn(a), "decode short and empty contexts")


def test_decode_b4_ctx64k_sampled():
    w = W["bf16_b4_ctx64k"].with_(S=1)
    a = synth.make_attention_inputs(w, 2004)
    log("case decode b4 64K S=1")
    got = run_attn(upload_attn(a), a)
    check_attn(got[[0, 3]], oracle_attn(a, [0, 3]), "decode b4 ctx64k sampled")


@pytest.mark.parametrize("S,Hq,Hkv", [(1, 32, 2), (2, 16, 2), (4, 8, 2), (8, 4, 2), (16, 8, 8),
                                      (1, 8, 8), (1, 24, 2), (3, 15, 3), (1, 4, 1)])
def test_decode_row_splits(S, Hq, Hkv):
    """Every way of filling at most 16 rows per KV head (G = Hq / Hkv heads
    x S positions), including G = 1, G = 12 and G*S = 15."""
    rng = np.random.default_rng(2005 + S * 100 + Hq)
    w = W["bf16_b8_ctx4k"].with_(B=5, S=S, Hq=Hq, Hkv=Hkv)
    lengths = rng.integers(0, 1500, 5)
    a = synth.make_attention_inputs(w, 2006 + S + Hq, lengths=lengths)
    log(f"case decode S={S} Hq={Hq} Hkv={Hkv} lengths={lengths.tolist()}")
    check_attn(run_attn(upload_attn(a), a), oracle_attn(a), f"decode S={S} Hq={Hq} Hkv={Hkv}")


def test_decode_grid_override_has_no_effect(monkeypatch):
    """The block path's grid override leaves the decode path alone."""
    w = W["bf16_b8_ctx4k"].with_(B=3, S=1)
    a = synth.make_attention_inputs(w, 2007, lengths=[700, 0, 3000])
    d = upload_attn(a)
    monkeypatch.delenv("TD_ATTN_GRID", raising=False)
    first = run_attn(d, a)
    monkeypatch.setenv("TD_ATTN_GRID", "3")
    second = run_attn(d, a)
    assert np.array_equal(first, second)
    check_attn(first, oracle_attn(a), "decode, grid override set")


@pytest.mark.parametrize("grid", [1, 3, 37, 512, 1000])
def test_decode_grids(grid, monkeypatch):
    """The decode split over waves: every wave streams an even run of 32-key
    blocks, a unit cut between waves is merged from its pieces.  From one
    workgroup (each unit whole or cut across few waves) to more waves than
    blocks (capped: one block per wave, every unit cut into single-block
    pieces), against the oracle."""
    rng = np.random.default_rng(2010 + grid)
    lengths = rng.integers(0, 3000, 5)
    lengths[0] = 0
    w = W["bf16_b8_ctx4k"].with_(B=5, S=1)
    a = synth.make_attention_inputs(w, 2011 + grid, lengths=lengths)
    monkeypatch.setenv("TD_DECODE_GRID", str(grid))
    log(f"case decode grid={grid} lengths={lengths.tolist()}")
    check_attn(run_attn(upload_attn(a), a), oracle_attn(a), f"decode grid {grid}")


def test_decode_gated_step():
    """The decode kernels honour td_denoise_step_if's gate: gate 0 leaves the
    output untouched, gate 1 computes it."""
    w = W["bf16_b8_ctx4k"].with_(B=4, S=1, V=1000)
    a = synth.make_attention_inputs(w, 2008, lengths=[300, 1000, 0, 77])
    c = synth.make_commit_inputs(w, 2008)
    d = upload_attn(a)
    B, S = w.B, w.S
    logits = dev(c["logits"], "bf16")
    commit = torch.empty((B, S), dtype=torch.uint8, device="cuda")
    token = torch.empty((B, S), dtype=torch.int32, device="cuda")
    n_left = torch.empty((1,), dtype=torch.int32, device="cuda")
    aa = td.attn_args(d["q"], d["k_blk"], d["v_blk"], d["k_ctx"], d["v_ctx"], d["offsets"], d["out"],
                      a["total_ctx"], a["max_ctx"])
    cc = td.commit_args(logits, commit, token, 0.8, n_masked_left=n_left)
    gate = torch.zeros((1,), dtype=torch.int32, device="cuda")
    d["out"].view(torch.int16).fill_(1234)
    log("case decode gated step")
    td.td_denoise_step_if(aa, cc, gate, device=d["out"].device)
    torch.cuda.synchronize()
    assert (d["out"].view(torch.int16) == 1234).all(), "a gated-off step wrote the output"
    gate.fill_(1)
    td.td_denoise_step_if(aa, cc, gate, device=d["out"].device)
    torch.cuda.synchronize()
    check_attn(d["out"].float().cpu().numpy().astype(np.float64), oracle_attn(a), "decode gated on")
