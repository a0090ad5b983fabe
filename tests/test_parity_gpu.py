"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Sizes span several key tiles, several context chunks and ragged tails; the
full-size workloads are checked on every sequence where the oracle finishes
in seconds (the headline batch, the uniform 8K batch, the 64K batch) and on
sampled sequences elsewhere.  Gates: see tests/gpu_util.py.
"""
import os

import numpy as np
import pytest
import torch

import block_diffusion_lm_td_amd as td
import oracle
import synth
from gpu_util import (check_attn, compare_commit, dev, f64, log, oracle_attn, oracle_commit,
                      run_attn, run_commit, upload_attn, upload_commit)

pytestmark = pytest.mark.gpu
W = synth.WORKLOADS


@pytest.fixture(autouse=True)
def _no_chunk_override(monkeypatch):
    monkeypatch.delenv("TD_ATTN_GRID", raising=False)
    monkeypatch.delenv("TD_COMMIT_SPLIT", raising=False)


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------
def test_attn_tiny_f32():
    w = W["tiny_f32_b1_ctx64"]
    a = synth.make_attention_inputs(w, 1001)
    log("case attn tiny_f32", w)
    got = run_attn(upload_attn(a), a)
    check_attn(got, oracle_attn(a), "tiny_f32", fp32=True)


@pytest.mark.parametrize("D,dtype", [(128, "f32"), (64, "f32")])
def test_attn_valu_path_other_shapes(D, dtype):
    w = W["tiny_f32_b1_ctx64"].with_(B=3, D=D, dtype=dtype, Hq=6, Hkv=3, S=5)
    a = synth.make_attention_inputs(w, 7, lengths=[0, 45, 70])
    log("case attn valu", D, dtype)
    got = run_attn(upload_attn(a), a)
    check_attn(got, oracle_attn(a), f"valu D={D} {dtype}", fp32=(dtype == "f32"))


@pytest.mark.parametrize("grid", [None, "1", "3", "37", "1000"])
def test_attn_bf16_ragged_small(grid, monkeypatch):
    """Empty context, a context shorter than a tile, ragged tails; the
    persistent grid size varies from one workgroup (no split unit) to more
    workgroups than key tiles (every unit split many ways)."""
    if grid:
        monkeypatch.setenv("TD_ATTN_GRID", grid)
    w = W["bf16_b8_ctx4k"].with_(B=5)
    a = synth.make_attention_inputs(w, 17, lengths=[0, 37, 1000, 513, 2])
    log("case attn ragged small grid", grid)
    d = upload_attn(a)
    got = run_attn(d, a)
    check_attn(got, oracle_attn(a), f"ragged small grid={grid}")
    # the merge folds its piece groups in a fixed order: a rerun is bitwise equal
    first = d["out"].clone()
    run_attn(d, a)
    assert torch.equal(first.view(torch.int16), d["out"].view(torch.int16)), "not deterministic"


@pytest.mark.parametrize("S,Hq,Hkv", [(1, 32, 2), (16, 32, 2), (32, 32, 2), (64, 32, 2),
                                      (16, 8, 8), (16, 64, 1), (7, 12, 3), (3, 4, 1)])
def test_attn_bf16_shapes(S, Hq, Hkv):
    """Decode (S=1), S=32/64 (several row groups), MHA (G=1), G=64, odd sizes."""
    w = W["bf16_b8_ctx4k"].with_(B=3, S=S, Hq=Hq, Hkv=Hkv)
    a = synth.make_attention_inputs(w, 100 + S + Hq, lengths=[300, 0, 777])
    log("case attn shape", S, Hq, Hkv)
    got = run_attn(upload_attn(a), a)
    check_attn(got, oracle_attn(a), f"S={S} Hq={Hq} Hkv={Hkv}")


@pytest.mark.parametrize("S,Hq,Hkv", [(16, 64, 8), (4, 32, 8), (1, 8, 1)])
def test_attn_gqa_long_ragged(S, Hq, Hkv):
    """Other GQA groupings over long ragged contexts, every sequence: G = 8
    with 128 live rows of each 256-row group (block path), and G*S = 16 and 8
    (decode path) with contexts from 3 to 20K keys."""
    w = W["bf16_b8_ctx4k"].with_(B=6, S=S, Hq=Hq, Hkv=Hkv)
    a = synth.make_attention_inputs(w, 300 + S + Hq, lengths=[16000, 3, 9000, 20000, 64, 4097])
    log("case attn gqa long ragged", S, Hq, Hkv)
    d = upload_attn(a)
    got = run_attn(d, a)
    check_attn(got, oracle_attn(a), f"gqa long S={S} Hq={Hq} Hkv={Hkv}")
    first = d["out"].clone()
    run_attn(d, a)
    assert torch.equal(first.view(torch.int16), d["out"].view(torch.int16)), "not deterministic"


def _random_attn_cases(n=24, seed=4242):
    """Seeded random valid shapes: ragged lengths with empty and sub-tile
    contexts and tile-edge lengths, S from 1 to 64, several GQA groupings,
    and persistent grids from 1 workgroup to more than there are tiles."""
    rng = np.random.default_rng(seed)
    heads = [(2, 1), (4, 2), (8, 1), (12, 3), (32, 2), (16, 16), (64, 4), (24, 1)]
    grids = [None, None, "1", "2", "5", "16", "64", "333"]
    cases = []
    for i in range(n):
        S = int(rng.choice([1, 2, 5, 16, 17, 33, 64]))
        Hq, Hkv = heads[int(rng.integers(len(heads)))]
        B = int(rng.integers(1, 9))
        while B * Hq * S > 4096 and B > 1:
            B -= 1
        kinds = rng.integers(0, 4, size=B)
        lengths = [0 if k == 0 else int(rng.integers(1, 64)) if k == 1 else
                   int(64 * rng.integers(1, 8) - S) if k == 2 else int(rng.integers(64, 500))
                   for k in kinds]
        lengths = [max(0, x) for x in lengths]
        cases.append((i, B, S, Hq, Hkv, lengths, grids[int(rng.integers(len(grids)))]))
    return cases


@pytest.mark.parametrize("case", _random_attn_cases(), ids=lambda c: f"r{c[0]}")
def test_attn_random_shapes(case, monkeypatch):
    i, B, S, Hq, Hkv, lengths, grid = case
    if grid:
        monkeypatch.setenv("TD_ATTN_GRID", grid)
    w = W["bf16_b8_ctx4k"].with_(B=B, S=S, Hq=Hq, Hkv=Hkv)
    a = synth.make_attention_inputs(w, 5000 + i, lengths=lengths)
    log("case attn random", i, "B", B, "S", S, "Hq", Hq, "Hkv", Hkv, "lengths", lengths, "grid", grid)
    got = run_attn(upload_attn(a), a)
    check_attn(got, oracle_attn(a), f"random case {i}")


def test_attn_unit_variance_and_scale():
    w = W["bf16_b4_ctx64k"].with_(B=2)
    a = synth.make_attention_inputs(w, 23, lengths=[1500, 2100])
    d = upload_attn(a)
    log("case attn unit variance + explicit scale")
    check_attn(run_attn(d, a), oracle_attn(a), "unit variance")
    check_attn(run_attn(d, a, scale=0.05), oracle_attn(a, scale=0.05), "scale=0.05")


def test_attn_bf16_b8_ctx4k_full():
    w = W["bf16_b8_ctx4k"]
    a = synth.make_attention_inputs(w, 1002)
    log("case attn bf16_b8_ctx4k full")
    d = upload_attn(a)
    got = run_attn(d, a)
    check_attn(got, oracle_attn(a), "bf16_b8_ctx4k (all sequences)")
    first = d["out"].clone()      # ~11 pieces per unit: the grouped merge, rerun bitwise equal
    run_attn(d, a)
    assert torch.equal(first.view(torch.int16), d["out"].view(torch.int16)), "not deterministic"


def test_attn_b64_ragged_all_and_deterministic():
    """The headline batch, every sequence against the oracle."""
    w = W["bf16_b64_ragged1k_8k"]
    a = synth.make_attention_inputs(w, 1003)
    d = upload_attn(a)
    log("case attn b64 ragged all sequences, lengths", a["lengths"][:8])
    got = run_attn(d, a)
    check_attn(got, oracle_attn(a), "b64 ragged (all 64 sequences)")
    first = d["out"].clone()
    run_attn(d, a)
    assert torch.equal(first.view(torch.int16), d["out"].view(torch.int16)), "not deterministic"


def test_attn_many_sequences_sampled():
    """More sequences than the workgroup has threads: the prologue scans the
    ragged lengths in several passes; many short (and empty) contexts."""
    w = W["bf16_b8_ctx4k"].with_(B=600)
    lengths = np.random.default_rng(31).integers(0, 120, size=600)
    lengths[[5, 77, 599]] = 0
    a = synth.make_attention_inputs(w, 31, lengths=lengths)
    log("case attn B=600 short contexts")
    got = run_attn(upload_attn(a), a)
    seqs = [0, 5, 77, 255, 511, 512, 513, 598, 599]
    check_attn(got[seqs], oracle_attn(a, seqs), f"B=600 sampled seqs={seqs}")


def test_attn_b64_ctx8k_all():
    w = W["bf16_b64_ctx8k"]
    a = synth.make_attention_inputs(w, 1006)
    log("case attn b64 ctx8k all sequences")
    got = run_attn(upload_attn(a), a)
    check_attn(got, oracle_attn(a), "b64 ctx8k (all 64 sequences)")


def test_attn_b4_ctx64k_all():
    w = W["bf16_b4_ctx64k"]
    a = synth.make_attention_inputs(w, 1004)
    log("case attn b4 ctx64k all sequences")
    got = run_attn(upload_attn(a), a)
    check_attn(got, oracle_attn(a), "b4 ctx64k (all 4 sequences)")


@pytest.mark.parametrize("S", [16, 32, 64])
def test_attn_loop_shapes_sampled(S):
    w = W["bf16_b32_ctx2k_loop"].with_(S=S)
    a = synth.make_attention_inputs(w, 1005 + S)
    log("case attn loop shape S", S)
    got = run_attn(upload_attn(a), a)
    check_attn(got[[0, 31]], oracle_attn(a, [0, 31]), f"b32 ctx2k S={S} seqs 0,31")


# ----------------------------------------------------------------------------
# commit
# ----------------------------------------------------------------------------
def _commit_case(w, seed, gamma, frac=1.0, seqs=None, label=""):
    c = synth.make_commit_inputs(w, seed)
    el = synth.make_eligible(w, seed, frac)
    d = upload_commit(c["logits"], w.dtype, el)
    g = run_commit(d, gamma)
    ref = oracle_commit(c["logits"], w.dtype, el, gamma, seqs)
    tok_in = np.full((w.B, w.S), -1)
    return compare_commit(g, ref, el, gamma, tok_in, label or w.name, seqs)


def test_commit_tiny_f32():
    w = W["tiny_f32_b1_ctx64"]
    log("case commit tiny f32")
    _commit_case(w, 2001, w.gamma, label="tiny f32")


@pytest.mark.parametrize("gamma", [0.5, 0.8, 0.95])
def test_commit_b8_v131072(gamma):
    w = W["bf16_b8_ctx4k"]
    log("case commit b8 V131072 gamma", gamma)
    _commit_case(w, 2002, gamma, frac=0.75, label=f"b8 gamma={gamma}")


def test_commit_b64_all():
    w = W["bf16_b64_ragged1k_8k"]
    log("case commit b64 all sequences")
    _commit_case(w, 2003, 0.8, label="b64 (all 64 sequences)")


def test_commit_b4_row_split():
    """64 rows: each row is split over several workgroups."""
    w = W["bf16_b4_ctx64k"]
    log("case commit b4 (row split)")
    _commit_case(w, 2004, 0.8, frac=0.9, label="b4 split rows")


@pytest.mark.parametrize("V,dtype", [(1001, "bf16"), (1003, "f32"), (8, "bf16"), (1, "f32"),
                                     (40000, "f32")])
def test_commit_odd_vocab(V, dtype):
    w = W["bf16_b8_ctx4k"].with_(B=3, S=9, V=V, dtype=dtype, logit_model="boost",
                                 logit_std=1.0, margin_hi=6.0)
    log("case commit odd vocab", V, dtype)
    _commit_case(w, 2005 + V, 0.6, frac=0.8, label=f"V={V} {dtype}")


def test_commit_ties_across_parts(monkeypatch):
    """Equal maxima in different lanes / row parts: the lowest id wins."""
    monkeypatch.setenv("TD_COMMIT_SPLIT", "4")
    B, S, V = 2, 5, 131072
    rng = np.random.default_rng(7)
    x = rng.standard_normal((B, S, V)).astype(np.float32)
    spots = [(0, 0, [5, 70000]), (0, 1, [131071, 65536, 40000]), (0, 2, [0, 1]),
             (1, 3, [9, 17, 33000, 100000]), (1, 4, [32768, 32767])]
    for b, i, ids in spots:
        x[b, i, ids] = 9.0
    bits = synth.f32_to_bf16_bits(x)
    d = upload_commit(bits, "bf16", None)
    g = run_commit(d, 0.5)
    for b, i, ids in spots:
        assert g["token"][b, i] == min(ids), (b, i, g["token"][b, i])
    ref = oracle_commit(bits, "bf16", None, 0.5)
    compare_commit(g, ref, None, 0.5, np.full((B, S), -1), "ties")


@pytest.mark.parametrize("gamma", [1.5, 1e-6])
def test_commit_extreme_gamma(gamma):
    w = W["bf16_b8_ctx4k"].with_(V=4096)
    log("case commit gamma", gamma)
    c = synth.make_commit_inputs(w, 2010)
    el = synth.make_eligible(w, 2010, 0.6)
    el[3] = 0
    d = upload_commit(c["logits"], "bf16", el)
    g = run_commit(d, gamma)
    n = g["commit"].sum(axis=1)
    if gamma > 1:
        assert (n == el.any(axis=1)).all()
    else:
        assert (g["commit"].astype(bool) == el.astype(bool)).all()
    compare_commit(g, oracle_commit(c["logits"], "bf16", el, gamma), el, gamma,
                   np.full((w.B, w.S), -1), f"gamma={gamma}")


def test_commit_masked_inplace_and_tokens():
    """masked_out aliasing masked_in; tokens keeps ids where nothing commits."""
    w = W["bf16_b8_ctx4k"].with_(V=8192)
    c = synth.make_commit_inputs(w, 2011)
    el = synth.make_eligible(w, 2011, 0.7)
    d = upload_commit(c["logits"], "bf16", el)
    tok_in = np.arange(w.B * w.S, dtype=np.int32).reshape(w.B, w.S) + 1000000
    d["tokens"].copy_(torch.from_numpy(tok_in))
    d["masked_out"] = d["masked_in"]
    g = run_commit(d, 0.8)
    ref = oracle_commit(c["logits"], "bf16", el, 0.8)
    compare_commit(g, ref, el, 0.8, tok_in, "in-place masks")


# ----------------------------------------------------------------------------
# denoise step and the block loop
# ----------------------------------------------------------------------------
def _step_inputs(w, seed, frac):
    a = synth.make_attention_inputs(w, seed)
    c = synth.make_commit_inputs(w, seed)
    el = synth.make_eligible(w, seed, frac)
    da = upload_attn(a)
    dc = upload_commit(c["logits"], w.dtype, el)
    return a, c, el, da, dc


def _run_step(w, da, dc, a, gamma):
    aa = td.attn_args(da["q"], da["k_blk"], da["v_blk"], da["k_ctx"], da["v_ctx"], da["offsets"],
                      da["out"], a["total_ctx"], a["max_ctx"])
    cc = td.commit_args(dc["logits"], dc["commit"], dc["token"], gamma, dc["masked_in"],
                        dc["maxprob"], dc["n_commit"], dc["masked_out"], dc["tokens"],
                        dc["n_masked_left"])
    td.td_denoise_step(aa, cc, device=da["q"].device)
    torch.cuda.synchronize()


def _decode_step_workload():
    # G*S = 16 with S = 4: the decode attention path with several positions
    return W["bf16_b8_ctx4k"].with_(B=5, S=4, Hq=8, Hkv=2, V=5000)


@pytest.mark.parametrize("name", ["tiny_f32_b1_ctx64", "bf16_b8_ctx4k", "bf16_b64_ragged1k_8k",
                                  "bf16_b64_ragged1k_8k_s1", "decode_b5_s4"])
def test_denoise_step(name):
    """td_denoise_step against oracle.denoise_step, every sequence and every
    position, including the headline batch.  On the MFMA path: attention main
    kernel, commit row pass, then the tail launch that merges the attention
    and takes the commit decision; at S = 1 (and G*S <= 16) the decode path:
    the streaming kernel, the row pass, then one launch for the decode merge
    and the decision."""
    w = _decode_step_workload() if name == "decode_b5_s4" else W[name]
    a, c, el, da, dc = _step_inputs(w, 3001, 0.8)
    log("case denoise step", name)
    _run_step(w, da, dc, a, w.gamma)
    got = da["out"].float().cpu().numpy().astype(np.float64)
    ref = oracle.denoise_step({k: f64(a[k], w.dtype) if k in ("q", "k_blk", "v_blk", "k_ctx", "v_ctx")
                               else a[k] for k in a}, f64(c["logits"], w.dtype), el,
                              np.full((w.B, w.S), -1), w.gamma)
    check_attn(got, ref["out"], f"step {name}", fp32=(w.dtype == "f32"))
    g = {k: dc[k].cpu().numpy() for k in ("commit", "token", "maxprob", "n_commit", "masked_out",
                                          "tokens", "n_masked_left")}
    compare_commit(g, ref, el, w.gamma, np.full((w.B, w.S), -1), f"step {name}")


@pytest.mark.parametrize("S,gamma", [(16, 0.5), (16, 0.8), (16, 0.95), (32, 0.5), (32, 0.8),
                                     (32, 0.95), (64, 0.5), (64, 0.8), (64, 0.95)])
def test_block_loop_teacher_forced(S, gamma):
    """Whole-block loop: each step's commit is compared with the oracle's
    commit from the same masked state; the loop ends within S steps."""
    w = W["bf16_b32_ctx2k_loop"].with_(B=8, S=S, V=16384, gamma=gamma)
    base, peak, stored = synth.loop_peak_values(w, 4000 + S, S + 1)
    log("case loop S gamma", S, gamma)
    logits = dev(base, "bf16").view(w.B, w.S, w.V)
    rows = torch.arange(w.B * w.S, device="cuda")
    peak_d = torch.from_numpy(peak).to("cuda")
    masked = np.ones((w.B, w.S), np.uint8)
    dc = upload_commit(base.reshape(w.B, w.S, w.V), "bf16", masked)
    dc["logits"] = logits
    tokens = np.full((w.B, w.S), -1)
    steps = 0
    while masked.any():
        assert steps < S, "block did not finish within S steps"
        logits.view(-1, w.V)[rows, peak_d] = dev(stored[steps], "bf16")
        dc["masked_in"].copy_(torch.from_numpy(masked))
        g = run_commit(dc, gamma)
        x = synth.loop_step_logits(base, peak, stored, steps).reshape(w.B, w.S, w.V)
        ref = oracle_commit(x, "bf16", masked, gamma)
        compare_commit(g, ref, masked, gamma, tokens, f"loop S={S} g={gamma} step={steps}")
        tokens = g["tokens"].astype(np.int64)
        masked = g["masked_out"].copy()
        assert int(g["n_masked_left"][0]) == int(masked.sum())
        steps += 1
    assert (tokens >= 0).all()
    log(f"[loop] S={S} gamma={gamma}: steps={steps}")


# ----------------------------------------------------------------------------
# gated step: a block's whole loop enqueued with no host synchronisation
# ----------------------------------------------------------------------------
def _loop_setup(S, gamma, seed):
    w = W["bf16_b32_ctx2k_loop"].with_(B=8, S=S, V=16384, gamma=gamma)
    a = synth.make_attention_inputs(w, seed, lengths=[300, 0, 700, 64, 129, 1000, 5, 450])
    base, peak, stored = synth.loop_peak_values(w, seed + 1, S + 1)
    d = upload_attn(a)
    logits = dev(base, "bf16").view(w.B, w.S, w.V)
    return w, a, d, logits, torch.from_numpy(peak).to("cuda"), dev(stored, "bf16")


def _commit_bufs(B, S):
    z = lambda shape, dt: torch.zeros(shape, dtype=dt, device="cuda")
    return dict(commit=z((B, S), torch.uint8), token=z((B, S), torch.int32),
                maxprob=z((B, S), torch.float32), n_commit=z((B,), torch.int32),
                masked=torch.ones((B, S), dtype=torch.uint8, device="cuda"),
                tokens=torch.full((B, S), -1, dtype=torch.int32, device="cuda"))


def _cargs(logits, c, gamma, n_left):
    return td.commit_args(logits, c["commit"], c["token"], gamma, c["masked"], c["maxprob"],
                          c["n_commit"], c["masked"], c["tokens"], n_left)


def test_denoise_step_if_gate_zero_and_one():
    """gate = 0: nothing is written except n_masked_left = 0; gate = 1: the
    same outputs as td_denoise_step."""
    w, a, d, logits, peak, stored = _loop_setup(16, 0.8, 6100)
    B, S = w.B, w.S
    L = td.lib()
    out = torch.full_like(d["q"], 3.0)
    aa = td.attn_args(d["q"], d["k_blk"], d["v_blk"], d["k_ctx"], d["v_ctx"], d["offsets"], out,
                      a["total_ctx"], a["max_ctx"])
    c = _commit_bufs(B, S)
    for k in ("commit", "token", "n_commit"):
        c[k].fill_(7)
    c["maxprob"].fill_(-1.0)
    n_left = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    cc = _cargs(logits, c, w.gamma, n_left)
    gate = torch.zeros((1,), dtype=torch.int32, device="cuda")
    log("case gated step, gate 0")
    td.td_denoise_step_if(aa, cc, gate)
    torch.cuda.synchronize()
    assert int(n_left.item()) == 0
    assert bool((out == 3.0).all()), "attention wrote with gate 0"
    assert bool((c["commit"] == 7).all()) and bool((c["token"] == 7).all())
    assert bool((c["n_commit"] == 7).all()) and bool((c["maxprob"] == -1.0).all())
    assert bool((c["masked"] == 1).all()) and bool((c["tokens"] == -1).all())

    log("case gated step, gate 1 vs td_denoise_step")
    gate.fill_(1)
    td.td_denoise_step_if(aa, cc, gate)
    ref = _commit_bufs(B, S)
    out_ref = torch.empty_like(d["q"])
    n_ref = torch.zeros((1,), dtype=torch.int32, device="cuda")
    aa_ref = td.attn_args(d["q"], d["k_blk"], d["v_blk"], d["k_ctx"], d["v_ctx"], d["offsets"],
                          out_ref, a["total_ctx"], a["max_ctx"])
    td.td_denoise_step(aa_ref, _cargs(logits, ref, w.gamma, n_ref))
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref)
    for k in ("commit", "token", "maxprob", "n_commit", "masked", "tokens"):
        assert torch.equal(c[k], ref[k]), k
    assert int(n_left.item()) == int(n_ref.item())


@pytest.mark.parametrize("S", [16, 64])
def test_block_loop_device_resident(S):
    """S gated steps enqueued back to back, the gate of each step being the
    previous step's n_masked_left (two counters used alternately), with one
    synchronisation at the end, give exactly the host-driven loop's result.
    The gated loop itself is compared step by step with the oracle at the
    loop workload's full shape in test_loop_gpu.py."""
    gamma = 0.8
    w, a, d, logits, peak, stored = _loop_setup(S, gamma, 6200 + S)
    B = w.B
    rows = torch.arange(B * S, device="cuda")
    aa = td.attn_args(d["q"], d["k_blk"], d["v_blk"], d["k_ctx"], d["v_ctx"], d["offsets"],
                      torch.empty_like(d["q"]), a["total_ctx"], a["max_ctx"])

    # host-driven: a synchronisation after every step
    log("case device-resident loop S", S, "host-driven reference")
    h = _commit_bufs(B, S)
    n_h = torch.zeros((1,), dtype=torch.int32, device="cuda")
    ch = _cargs(logits, h, gamma, n_h)
    left_h = []
    while True:
        logits.view(-1, w.V)[rows, peak] = stored[len(left_h)]
        td.td_denoise_step(aa, ch)
        left_h.append(int(n_h.item()))
        if left_h[-1] == 0:
            break
        assert len(left_h) < S, "block did not finish within S steps"
    tokens_h, masked_h = h["tokens"].clone(), h["masked"].clone()

    # device-resident: S gated steps, no synchronisation until the end
    log("case device-resident loop S", S, "gated")
    g = _commit_bufs(B, S)
    cnt = torch.zeros((2,), dtype=torch.int32, device="cuda")
    cnt[1] = 1                                        # opens step 0
    cg = [_cargs(logits, g, gamma, cnt[k:k + 1]) for k in range(2)]
    hist = torch.full((S,), -1, dtype=torch.int32, device="cuda")
    for k in range(S):
        logits.view(-1, w.V)[rows, peak] = stored[k]
        td.td_denoise_step_if(aa, cg[k % 2], cnt[(k + 1) % 2:(k + 1) % 2 + 1])
        hist[k:k + 1].copy_(cnt[k % 2:k % 2 + 1])
    torch.cuda.synchronize()
    hist = hist.cpu().numpy().tolist()
    n = len(left_h)
    assert hist[:n] == left_h, (hist, left_h)
    assert all(x == 0 for x in hist[n:]), hist
    assert torch.equal(g["tokens"], tokens_h) and torch.equal(g["masked"], masked_h)
    assert bool((g["tokens"] >= 0).all())
    log(f"[device loop] S={S}: {n} steps of {S} enqueued")


def test_block_loop_graph_replay():
    """The device-resident loop (S gated steps, no host round trip) captured
    once in a graph and replayed three times, with eager resets and
    synchronisations between the replays: every replay gives exactly the
    host-driven loop's counts, tokens and masks.  The library records kernel
    launches only (no memset nodes).  test_loop_gpu.py compares graph-replayed
    loops with the oracle step by step at the loop workload's full shape."""
    S, gamma = 16, 0.8
    w, a, d, logits, peak, stored = _loop_setup(S, gamma, 6300)
    B = w.B
    rows = torch.arange(B * S, device="cuda")
    aa = td.attn_args(d["q"], d["k_blk"], d["v_blk"], d["k_ctx"], d["v_ctx"], d["offsets"],
                      torch.empty_like(d["q"]), a["total_ctx"], a["max_ctx"])
    log("case graph-replayed loop: host-driven reference")
    h = _commit_bufs(B, S)
    n_h = torch.zeros((1,), dtype=torch.int32, device="cuda")
    ch = _cargs(logits, h, gamma, n_h)
    left_h = []
    while True:
        logits.view(-1, w.V)[rows, peak] = stored[len(left_h)]
        td.td_denoise_step(aa, ch)
        left_h.append(int(n_h.item()))
        if left_h[-1] == 0:
            break
        assert len(left_h) < S, "block did not finish within S steps"
    n = len(left_h)

    g = _commit_bufs(B, S)
    cnt = torch.zeros((2,), dtype=torch.int32, device="cuda")
    cg = [_cargs(logits, g, gamma, cnt[k:k + 1]) for k in range(2)]
    hist = torch.full((S,), -1, dtype=torch.int32, device="cuda")
    ws = td.Workspace(torch.device("cuda"))

    def reset():
        for k in ("commit", "token", "maxprob", "n_commit"):
            g[k].zero_()
        g["masked"].fill_(1)
        g["tokens"].fill_(-1)
        cnt.zero_()
        cnt[1] = 1                                    # opens step 0
        hist.fill_(-1)

    def loop():
        for k in range(S):
            logits.view(-1, w.V)[rows, peak] = stored[k]
            td.td_denoise_step_if(aa, cg[k % 2], cnt[(k + 1) % 2:(k + 1) % 2 + 1], workspace=ws)
            hist[k:k + 1].copy_(cnt[k % 2:k % 2 + 1])

    def check(label):
        got = hist.cpu().numpy().tolist()
        assert got[:n] == left_h and all(x == 0 for x in got[n:]), (label, got, left_h)
        assert torch.equal(g["tokens"], h["tokens"]) and torch.equal(g["masked"], h["masked"]), label

    log("case graph-replayed loop: eager warm-up")
    reset()
    loop()                                            # allocates the workspace outside the capture
    torch.cuda.synchronize()
    check("eager")
    graph = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    log("case graph-replayed loop: capture")
    with torch.cuda.graph(graph):
        loop()
    for rep in range(3):
        reset()                                       # eager work between replays
        torch.cuda.synchronize()
        log(f"case graph-replayed loop: replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        check(f"replay {rep}")
    log(f"[graph loop] {n} steps of {S}, 3 replays identical to the host-driven loop")
