"""Independent pins of the fp64 oracle.

Each ``pin_*`` takes the implementation under test (so the mutation test can
hand it a deliberately broken copy of the oracle) and raises AssertionError on
a mismatch.  None of them re-types the oracle's formula: they compare against
a different library routine (torch SDPA, torch softmax), closed forms,
invariants the pages fix, or pure-Python brute force.

Page references: [chathome] is news.chathome.org, "NVIDIA releases
Nemotron-Labs-TwoTower ..." (inference, block-generation and evaluation
paragraphs); [aiboss] is aiboss88.com, technical-principle section.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

TOL = 1e-12
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------
def rand_attn(rng, B, S, Hq, Hkv, D, lengths, std=1.0):
    lengths = np.asarray(lengths, dtype=np.int64)
    off = np.zeros(B + 1, dtype=np.int64)
    off[1:] = np.cumsum(lengths)
    T = int(off[-1])
    return dict(
        q=rng.standard_normal((B, S, Hq, D)) * std,
        k_blk=rng.standard_normal((B, S, Hkv, D)) * std,
        v_blk=rng.standard_normal((B, S, Hkv, D)),
        k_ctx=rng.standard_normal((T, Hkv, D)) * std,
        v_ctx=rng.standard_normal((T, Hkv, D)),
        offsets=off,
    )


def call_attn(attn, a, scale=None):
    return attn(a["q"], a["k_blk"], a["v_blk"], a["k_ctx"], a["v_ctx"], a["offsets"], scale)


def sdpa_seq(a, b, scale=None, causal=False, q_override=None):
    """torch SDPA (CPU, float64, GQA) for sequence b over [context ; block]."""
    lo, hi = int(a["offsets"][b]), int(a["offsets"][b + 1])
    K = np.concatenate([a["k_ctx"][lo:hi], a["k_blk"][b]], axis=0)   # [N, Hkv, D]
    V = np.concatenate([a["v_ctx"][lo:hi], a["v_blk"][b]], axis=0)
    Q = a["q"][b] if q_override is None else q_override              # [M, Hq, D]
    tq = torch.from_numpy(np.ascontiguousarray(Q.transpose(1, 0, 2)))[None]
    tk = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None]
    tv = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None]
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, scale=scale, is_causal=causal, enable_gqa=True)
    return o[0].numpy().transpose(1, 0, 2)                           # [M, Hq, D]


def _close(x, y, tol=TOL, what=""):
    err = float(np.max(np.abs(np.asarray(x) - np.asarray(y)))) if np.size(x) else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# ----------------------------------------------------------------------------
# attention pins ([chathome] inference paragraph, [aiboss] technical principle)
# ----------------------------------------------------------------------------
def pin_attn_sdpa_general(attn):
    """General ragged GQA case == torch SDPA on each sequence's [context ; block]."""
    rng = np.random.default_rng(11)
    for (B, S, Hq, Hkv, D, lens, scale) in [
        (3, 5, 4, 2, 8, [0, 3, 7], None),
        (2, 4, 6, 3, 16, [5, 1], 0.37),
        (1, 3, 8, 1, 4, [9], None),
        (2, 2, 4, 4, 8, [2, 0], None),
    ]:
        a = rand_attn(rng, B, S, Hq, Hkv, D, lens)
        out = call_attn(attn, a, scale)
        for b in range(B):
            _close(out[b], sdpa_seq(a, b, scale), what=f"sdpa b={b} shape={(B, S, Hq, Hkv, D)}")


def pin_attn_empty_context(attn):
    """L_b = 0: plain bidirectional attention inside the block."""
    rng = np.random.default_rng(12)
    a = rand_attn(rng, 2, 6, 4, 2, 8, [0, 0])
    out = call_attn(attn, a)
    for b in range(2):
        tq = torch.from_numpy(a["q"][b].transpose(1, 0, 2).copy())[None]
        tk = torch.from_numpy(a["k_blk"][b].transpose(1, 0, 2).copy())[None]
        tv = torch.from_numpy(a["v_blk"][b].transpose(1, 0, 2).copy())[None]
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, enable_gqa=True)
        _close(out[b], ref[0].numpy().transpose(1, 0, 2), what="empty context")


def pin_attn_single_token_decode(attn):
    """S = 1: the last row of causal attention over [context ; new token],
    i.e. one autoregressive decode step over the cache ([chathome]
    block-generation paragraph: AR commits one token per step)."""
    rng = np.random.default_rng(13)
    Hq, Hkv, D = 4, 2, 8
    lens = [6, 0, 3]
    a = rand_attn(rng, 3, 1, Hq, Hkv, D, lens)
    out = call_attn(attn, a)
    for b, L in enumerate(lens):
        qfull = np.concatenate([rng.standard_normal((L, Hq, D)), a["q"][b]], axis=0)
        ref = sdpa_seq(a, b, causal=True, q_override=qfull)
        _close(out[b, 0], ref[-1], what=f"decode b={b}")


def pin_attn_gqa_is_repeated_mha(attn):
    """GQA equals multi-head attention on K/V heads repeated G times in order."""
    rng = np.random.default_rng(14)
    a = rand_attn(rng, 2, 3, 6, 2, 8, [4, 2])
    G = 3
    m = dict(a)
    for k in ("k_blk", "v_blk"):
        m[k] = np.repeat(a[k], G, axis=2)
    for k in ("k_ctx", "v_ctx"):
        m[k] = np.repeat(a[k], G, axis=1)
    _close(call_attn(attn, a), call_attn(attn, m), what="gqa vs repeated mha")


def pin_attn_uniform_keys(attn):
    """All keys equal: every weight is 1/(L+S), output = mean of V."""
    rng = np.random.default_rng(15)
    a = rand_attn(rng, 2, 4, 4, 2, 8, [5, 3])
    kvec = rng.standard_normal(8)
    a["k_blk"][:] = kvec
    a["k_ctx"][:] = kvec
    out = call_attn(attn, a)
    for b in range(2):
        lo, hi = a["offsets"][b], a["offsets"][b + 1]
        for h in range(4):
            g = h // 2
            V = np.concatenate([a["v_ctx"][lo:hi, g], a["v_blk"][b, :, g]], axis=0)
            _close(out[b, :, h], np.broadcast_to(V.mean(axis=0), (4, 8)), what="uniform keys")


def pin_attn_dominant_key(attn):
    """One key scores >= 60 above all others: output = that key's V row."""
    rng = np.random.default_rng(16)
    B, S, Hq, Hkv, D = 1, 3, 2, 1, 4
    a = rand_attn(rng, B, S, Hq, Hkv, D, [5], std=0.1)
    a["q"][:] = 1.0
    a["k_ctx"][3, 0, :] = 60.0          # score = 60*4/sqrt(4) = 120 vs |others| < 2
    out = call_attn(attn, a)
    _close(out[0], np.broadcast_to(a["v_ctx"][3, 0], (S, Hq, D)), tol=1e-12, what="dominant key")
    a2 = rand_attn(rng, B, S, Hq, Hkv, D, [5], std=0.1)
    a2["q"][:] = 1.0
    a2["k_blk"][0, 2, 0, :] = 60.0      # a block key dominates
    out2 = call_attn(attn, a2)
    _close(out2[0], np.broadcast_to(a2["v_blk"][0, 2, 0], (S, Hq, D)), what="dominant block key")


def pin_attn_permutation(attn):
    """Permuting the block's tokens (Q, K, V together) permutes the outputs."""
    rng = np.random.default_rng(17)
    a = rand_attn(rng, 2, 6, 4, 2, 8, [3, 5])
    perm = rng.permutation(6)
    p = dict(a)
    for k in ("q", "k_blk", "v_blk"):
        p[k] = a[k][:, perm]
    _close(call_attn(attn, p), call_attn(attn, a)[:, perm], what="permutation")


def pin_attn_batch_independence(attn):
    """Sequence b's output does not change when it is run alone."""
    rng = np.random.default_rng(18)
    a = rand_attn(rng, 3, 4, 4, 2, 8, [2, 0, 5])
    out = call_attn(attn, a)
    for b in range(3):
        lo, hi = int(a["offsets"][b]), int(a["offsets"][b + 1])
        one = dict(q=a["q"][b:b + 1], k_blk=a["k_blk"][b:b + 1], v_blk=a["v_blk"][b:b + 1],
                   k_ctx=a["k_ctx"][lo:hi], v_ctx=a["v_ctx"][lo:hi],
                   offsets=np.array([0, hi - lo]))
        _close(call_attn(attn, one)[0], out[b], what=f"batch independence b={b}")


def pin_attn_key_shift(attn):
    """Adding one vector to every key of a KV head leaves the output unchanged."""
    rng = np.random.default_rng(19)
    a = rand_attn(rng, 2, 4, 4, 2, 8, [3, 6])
    s = dict(a)
    c = rng.standard_normal((2, 8))
    s["k_blk"] = a["k_blk"] + c[None, None]
    s["k_ctx"] = a["k_ctx"] + c[None]
    _close(call_attn(attn, s), call_attn(attn, a), tol=1e-11, what="key shift")


def pin_attn_linear_in_v(attn):
    """O(alpha V1 + V2) = alpha O(V1) + O(V2)."""
    rng = np.random.default_rng(20)
    a1 = rand_attn(rng, 2, 3, 4, 2, 8, [4, 1])
    a2 = dict(a1)
    a2["v_blk"] = rng.standard_normal(a1["v_blk"].shape)
    a2["v_ctx"] = rng.standard_normal(a1["v_ctx"].shape)
    al = 2.5
    a3 = dict(a1)
    a3["v_blk"] = al * a1["v_blk"] + a2["v_blk"]
    a3["v_ctx"] = al * a1["v_ctx"] + a2["v_ctx"]
    _close(call_attn(attn, a3), al * call_attn(attn, a1) + call_attn(attn, a2), tol=1e-11,
           what="linearity")


def brute_attention(a, scale=None):
    """Pure-Python loops, no numpy arithmetic."""
    q, kb, vb, kc, vc, off = (a[k] for k in ("q", "k_blk", "v_blk", "k_ctx", "v_ctx", "offsets"))
    B, S, Hq, D = q.shape
    Hkv = kb.shape[2]
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(D) if scale is None else scale
    out = [[[[0.0] * D for _ in range(Hq)] for _ in range(S)] for _ in range(B)]
    for b in range(B):
        keys, vals = [], []
        for t in range(int(off[b]), int(off[b + 1])):
            keys.append(t)
        for h in range(Hq):
            g = h // G
            K = [[float(kc[t, g, d]) for d in range(D)] for t in keys] + \
                [[float(kb[b, j, g, d]) for d in range(D)] for j in range(S)]
            Vv = [[float(vc[t, g, d]) for d in range(D)] for t in keys] + \
                 [[float(vb[b, j, g, d]) for d in range(D)] for j in range(S)]
            for i in range(S):
                sc_list = [sc * sum(float(q[b, i, h, d]) * k[d] for d in range(D)) for k in K]
                mx = max(sc_list)
                w = [math.exp(x - mx) for x in sc_list]
                tot = sum(w)
                for d in range(D):
                    out[b][i][h][d] = sum(w[n] * Vv[n][d] for n in range(len(K))) / tot
    return np.array(out)


def pin_attn_brute_force(attn):
    rng = np.random.default_rng(21)
    for (B, S, Hq, Hkv, D, lens) in [(2, 3, 4, 2, 4, [2, 0]), (1, 2, 2, 1, 3, [4])]:
        a = rand_attn(rng, B, S, Hq, Hkv, D, lens)
        _close(call_attn(attn, a), brute_attention(a), what="brute force")
        _close(call_attn(attn, a, 0.21), brute_attention(a, 0.21), what="brute force scaled")


ATTN_PINS = [pin_attn_sdpa_general, pin_attn_empty_context, pin_attn_single_token_decode,
             pin_attn_gqa_is_repeated_mha, pin_attn_uniform_keys, pin_attn_dominant_key,
             pin_attn_permutation, pin_attn_batch_independence, pin_attn_key_shift,
             pin_attn_linear_in_v, pin_attn_brute_force]


# ----------------------------------------------------------------------------
# commit pins ([chathome] block-generation and evaluation paragraphs)
# ----------------------------------------------------------------------------
def pin_conf_vs_torch(row_conf):
    """p = max of torch.softmax (float64); token = torch.argmax (documented to
    return the first maximal index)."""
    rng = np.random.default_rng(31)
    x = rng.standard_normal((3, 5, 50)) * 3
    x[0, 1, 7] = x[0, 1, 30] = x[0, 1].max() + 1.0     # a tie: first index wins
    p, tok = row_conf(x)
    t = torch.from_numpy(x)
    _close(p, torch.softmax(t, dim=-1).max(dim=-1).values.numpy(), what="p vs torch")
    assert (np.asarray(tok) == torch.argmax(t, dim=-1).numpy()).all(), "token vs torch"
    assert int(tok[0, 1]) == 7


def pin_conf_closed_forms(row_conf):
    V = 37
    p, tok = row_conf(np.zeros((1, 1, V)))
    _close(p, [[1.0 / V]], what="uniform row")
    assert int(tok[0, 0]) == 0
    for c, j in [(2.0, 5), (-1.5, 36), (9.0, 0)]:
        x = np.zeros((1, 1, V))
        x[0, 0, j] = c
        p, tok = row_conf(x)
        want = math.exp(c) / (math.exp(c) + V - 1) if c > 0 else 1.0 / (math.exp(c) + V - 1)
        _close(p, [[want]], what=f"one-hot logit c={c}")
        assert int(tok[0, 0]) == (j if c > 0 else (0 if j != 0 else 1))


def pin_conf_large_logits(row_conf):
    """Logits near 1e3 (exp overflows without the max shift) stay exact."""
    x = np.full((1, 1, 4), 1000.0)
    x[0, 0, 2] = 1000.0 + math.log(6.0)
    p, tok = row_conf(x)
    _close(p, [[6.0 / 9.0]], what="large logits")
    assert int(tok[0, 0]) == 2


def pin_commit_golden(commit):
    """Hand-derived fixture (tests/golden/commit_closed_form.json)."""
    with open(os.path.join(GOLDEN, "commit_closed_form.json")) as f:
        g = json.load(f)
    x = np.array(g["logits"], dtype=np.float64)
    for case in g["cases"]:
        r = commit(x, np.array(case["eligible"], dtype=np.uint8), case["gamma"])
        assert np.asarray(r["commit"]).astype(int).tolist() == case["commit"], case["name"]
        assert np.asarray(r["token"]).tolist() == g["token"], case["name"]
        assert np.asarray(r["n_commit"]).tolist() == case["n_commit"], case["name"]
        _close(r["maxprob"], np.array(g["maxprob"]), tol=1e-15, what=case["name"])


def pin_commit_gamma_above_one(commit):
    """gamma > 1: only the force-one rule commits -- exactly one eligible
    position per sequence that has one, none otherwise."""
    rng = np.random.default_rng(32)
    x = rng.standard_normal((4, 6, 20)) * 2
    el = (rng.random((4, 6)) < 0.6).astype(np.uint8)
    el[3] = 0
    r = commit(x, el, 1.5)
    c = np.asarray(r["commit"]).astype(bool)
    for b in range(4):
        assert c[b].sum() == (1 if el[b].any() else 0)
        assert not (c[b] & ~el[b].astype(bool)).any()
    # AR-like loop: each step commits exactly one token (force-one only)


def pin_commit_gamma_tiny(commit):
    rng = np.random.default_rng(33)
    x = rng.standard_normal((3, 5, 20))
    el = (rng.random((3, 5)) < 0.7).astype(np.uint8)
    r = commit(x, el, 1e-6)
    assert (np.asarray(r["commit"]).astype(bool) == el.astype(bool)).all()


def pin_commit_monotone(commit):
    """Commit count is non-increasing as gamma rises, >= 1 when any position
    is eligible, and ineligible positions never commit ([chathome]
    evaluation paragraph: a lower gamma commits more tokens per step)."""
    rng = np.random.default_rng(34)
    x = rng.standard_normal((5, 8, 30)) * 2.5
    el = (rng.random((5, 8)) < 0.8).astype(np.uint8)
    el[0] = 1
    prev = None
    for gam in np.linspace(0.02, 1.2, 40):
        r = commit(x, el, float(gam))
        c = np.asarray(r["commit"]).astype(bool)
        n = c.sum(axis=1)
        assert not (c & ~el.astype(bool)).any()
        assert ((n >= 1) | ~el.astype(bool).any(axis=1)).all()
        if prev is not None:
            assert (n <= prev).all()
        prev = n


def pin_commit_inclusive_threshold(commit):
    """p == gamma exactly commits (V = 2, equal logits: p = 0.5 = gamma)."""
    x = np.zeros((1, 2, 2))
    x[0, 1] = [3.0, 0.0]         # p = 1/(1+e^-3) = 0.9526 also commits
    r = commit(x, np.ones((1, 2), np.uint8), 0.5)
    assert np.asarray(r["commit"]).astype(int).tolist() == [[1, 1]]
    r = commit(x, np.ones((1, 2), np.uint8), 0.6)
    assert np.asarray(r["commit"]).astype(int).tolist() == [[0, 1]]


def pin_commit_float32_gamma(commit):
    """gamma is the float32 value the kernel sees: float32(0.8) = 0.80000001192...,
    so p = 0.8 + 5e-9 does not reach it, while p = 0.8 + 5e-8 does."""
    def row(p):
        return [math.log(p / (1.0 - p)), 0.0]
    x = np.array([[row(0.9), row(0.8 + 5e-9), row(0.8 + 5e-8)]])
    r = commit(x, np.ones((1, 3), np.uint8), 0.8)
    assert np.asarray(r["commit"]).astype(int).tolist() == [[1, 0, 1]]


def pin_commit_force_one_ties(commit):
    """Force-one: largest p among ELIGIBLE positions, lowest position on ties."""
    V = 10
    x = np.zeros((2, 5, V))
    # sequence 0: positions 1 and 3 tie at the eligible max; 4 is higher but ineligible
    for i, c in [(0, 0.5), (1, 1.0), (2, 0.2), (3, 1.0), (4, 3.0)]:
        x[0, i, 2] = c
    el = np.array([[1, 1, 1, 1, 0], [0, 0, 1, 1, 1]], np.uint8)
    x[1, 2, 0] = 0.7
    x[1, 4, 0] = 0.7
    r = commit(x, el, 0.99)
    assert np.asarray(r["commit"]).astype(int).tolist() == [[0, 1, 0, 0, 0], [0, 0, 1, 0, 0]]


COMMIT_PINS = [pin_commit_golden, pin_commit_gamma_above_one, pin_commit_gamma_tiny,
               pin_commit_monotone, pin_commit_inclusive_threshold, pin_commit_float32_gamma,
               pin_commit_force_one_ties]
CONF_PINS = [pin_conf_vs_torch, pin_conf_closed_forms, pin_conf_large_logits]


# ----------------------------------------------------------------------------
# step / loop pins ([chathome] block-generation paragraph)
# ----------------------------------------------------------------------------
def _loop_logits(seed, B, S, V):
    rng = np.random.default_rng(seed)
    xs = [rng.standard_normal((B, S, V)) * 2 for _ in range(S + 2)]
    return lambda t: xs[t]


def pin_loop_force_one_is_ar(loop):
    """With gamma > 1 only force-one commits: exactly one token per step and
    exactly S steps per block -- the autoregressive one-token-per-step case."""
    B, S = 3, 5
    r = loop(_loop_logits(41, B, S, 12), B, S, 1.01)
    assert r["steps"] == S and r["done"]
    assert (np.asarray(r["commits_per_step"]) == 1).all()
    assert (np.asarray(r["tokens"]) >= 0).all()


def pin_loop_low_gamma_one_step(loop):
    B, S = 2, 6
    r = loop(_loop_logits(42, B, S, 12), B, S, 1e-9)
    assert r["steps"] == 1 and r["done"]


def pin_loop_steps_monotone(loop):
    """Steps per block never rise as gamma falls, and every block finishes
    within S steps."""
    B, S = 4, 8
    f = _loop_logits(43, B, S, 6)
    prev = None
    for gam in [0.1, 0.3, 0.5, 0.8, 0.95, 1.2]:
        r = loop(f, B, S, gam)
        assert r["done"] and r["steps"] <= S
        st = np.asarray(r["steps_per_seq"])
        if prev is not None:
            assert (st >= prev).all()
        prev = st


def pin_step_masks(step):
    """A step never re-masks a committed position, and changes the stored
    token only where it commits."""
    rng = np.random.default_rng(44)
    a = rand_attn(rng, 2, 4, 4, 2, 8, [3, 2])
    x = rng.standard_normal((2, 4, 9)) * 3
    m_in = np.array([[1, 0, 1, 1], [0, 0, 1, 0]], np.uint8)
    tok_in = np.array([[-1, 5, -1, -1], [2, 3, -1, 4]])
    r = step(a, x, m_in, tok_in, 0.6)
    mo = np.asarray(r["masked_out"]).astype(bool)
    c = np.asarray(r["commit"]).astype(bool)
    assert not (mo & ~m_in.astype(bool)).any()
    assert (mo | c == m_in.astype(bool)).all() and not (mo & c).any()
    t = np.asarray(r["tokens"])
    assert (t[~c] == tok_in[~c]).all()
    assert (t[c] == np.argmax(x, axis=-1)[c]).all()
    assert r["n_masked_left"] == int(mo.sum())


def pin_step_attention_sdpa(step):
    """The step's attention output is the layer's block attention: per
    sequence, torch SDPA (float64, GQA) over [context ; block] keys, with the
    default scale and with an explicit one ([chathome] inference paragraph).
    Block and context K/V are all distinct draws, so a swapped or dropped
    operand in the step's wiring changes the output."""
    rng = np.random.default_rng(45)
    a = rand_attn(rng, 3, 4, 4, 2, 8, [5, 0, 3])
    x = rng.standard_normal((3, 4, 7)) * 2
    m_in = np.ones((3, 4), np.uint8)
    tok_in = np.full((3, 4), -1)
    for scale in (None, 0.3):
        r = step(a, x, m_in, tok_in, 0.8, scale)
        out = np.asarray(r["out"])
        for b in range(3):
            _close(out[b], sdpa_seq(a, b, scale=scale), what=f"step out b={b} scale={scale}")


LOOP_PINS = [pin_loop_force_one_is_ar, pin_loop_low_gamma_one_step, pin_loop_steps_monotone]
STEP_PINS = [pin_step_masks, pin_step_attention_sdpa]


# ----------------------------------------------------------------------------
# cache-append pins ([chathome] block-generation paragraph)
# ----------------------------------------------------------------------------
def _labelled_cache(lengths, S, Hkv=2, D=3):
    """Rows whose values name (sequence, time index, tensor): old row t of
    sequence b is (b, t), new row s is (b, L_b + s); K and V differ in sign."""
    lengths = np.asarray(lengths, dtype=np.int64)
    B = len(lengths)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(off[-1])
    k_ctx = np.zeros((T, Hkv, D))
    k_new = np.zeros((B, S, Hkv, D))
    for b in range(B):
        for t in range(int(lengths[b])):
            k_ctx[off[b] + t] = 1000.0 * (b + 1) + t
        for s in range(S):
            k_new[b, s] = 1000.0 * (b + 1) + lengths[b] + s
    k_ctx[..., 1:] += 0.5                  # the head / lane index stays visible
    k_new[..., 1:] += 0.5
    return k_ctx, -k_ctx, off, k_new, -k_new


def pin_append_time_order(append):
    """Reading the new cache row by row gives every sequence's keys in time
    order, sequence after sequence: a stable sort of all rows by (sequence,
    time) -- a different route to the same layout."""
    lengths, S = [3, 0, 5, 1], 2
    k_ctx, v_ctx, off, k_new, v_new = _labelled_cache(lengths, S)
    k_out, v_out, off_out = append(k_ctx, v_ctx, off, k_new, v_new)
    rows = np.concatenate([k_ctx, k_new.reshape(-1, *k_ctx.shape[1:])], axis=0)
    key = rows[:, 0, 0]
    want = rows[np.lexsort((key % 1000.0, key // 1000.0))]
    assert np.array_equal(np.asarray(k_out), want)
    assert np.array_equal(np.asarray(v_out), -want)
    assert np.array_equal(np.asarray(off_out), np.searchsorted(want[:, 0, 0] // 1000.0,
                                                               np.arange(1, len(lengths) + 2)))


def pin_append_offsets_closed_form(append):
    """Sequence b moves down by b*S rows and grows by S."""
    rng = np.random.default_rng(45)
    lengths, S = np.array([0, 7, 2, 0, 11]), 3
    off = np.concatenate([[0], np.cumsum(lengths)])
    T, B = int(off[-1]), len(lengths)
    k_ctx = rng.standard_normal((T, 2, 4))
    k_new = rng.standard_normal((B, S, 2, 4))
    _, _, off_out = append(k_ctx, k_ctx, off, k_new, k_new)
    off_out = np.asarray(off_out)
    assert np.array_equal(off_out, off + S * np.arange(B + 1))
    assert np.array_equal(np.diff(off_out), lengths + S)


def pin_append_identities(append):
    """S = 0 leaves the cache as it was; an empty cache becomes the new rows."""
    rng = np.random.default_rng(46)
    lengths = [4, 0, 2]
    off = np.concatenate([[0], np.cumsum(lengths)])
    k_ctx = rng.standard_normal((6, 1, 5))
    v_ctx = rng.standard_normal((6, 1, 5))
    k_out, v_out, off_out = append(k_ctx, v_ctx, off, np.zeros((3, 0, 1, 5)),
                                   np.zeros((3, 0, 1, 5)))
    assert np.array_equal(np.asarray(k_out), k_ctx) and np.array_equal(np.asarray(v_out), v_ctx)
    assert np.array_equal(np.asarray(off_out), off)
    k_new = rng.standard_normal((3, 4, 1, 5))
    v_new = rng.standard_normal((3, 4, 1, 5))
    k_out, v_out, off_out = append(np.zeros((0, 1, 5)), np.zeros((0, 1, 5)),
                                   np.zeros(4, np.int64), k_new, v_new)
    assert np.array_equal(np.asarray(k_out), k_new.reshape(12, 1, 5))
    assert np.array_equal(np.asarray(v_out), v_new.reshape(12, 1, 5))
    assert np.array_equal(np.asarray(off_out), [0, 4, 8, 12])


def pin_append_two_blocks_at_once(append):
    """Appending S1 rows and then S2 rows equals appending the S1 + S2 rows
    in one call."""
    rng = np.random.default_rng(47)
    lengths = [2, 5, 0]
    off = np.concatenate([[0], np.cumsum(lengths)])
    k_ctx, v_ctx = rng.standard_normal((7, 2, 3)), rng.standard_normal((7, 2, 3))
    k1, v1 = rng.standard_normal((3, 2, 2, 3)), rng.standard_normal((3, 2, 2, 3))
    k2, v2 = rng.standard_normal((3, 3, 2, 3)), rng.standard_normal((3, 3, 2, 3))
    ka, va, oa = append(k_ctx, v_ctx, off, k1, v1)
    ka, va, oa = append(ka, va, oa, k2, v2)
    kb, vb, ob = append(k_ctx, v_ctx, off, np.concatenate([k1, k2], axis=1),
                        np.concatenate([v1, v2], axis=1))
    assert np.array_equal(np.asarray(ka), np.asarray(kb))
    assert np.array_equal(np.asarray(va), np.asarray(vb))
    assert np.array_equal(np.asarray(oa), np.asarray(ob))


def pin_append_then_attend(append):
    """Attention over the grown cache (torch SDPA, keys read from the new
    rows of sequence b) equals attention over the keys [old cache ; block]
    with the block's rows moved into the cache -- the next block then sees
    the committed tokens as context."""
    rng = np.random.default_rng(48)
    B, S, Hq, Hkv, D = 3, 4, 4, 2, 8
    a = rand_attn(rng, B, S, Hq, Hkv, D, [5, 0, 3])
    k_out, v_out, off_out = append(a["k_ctx"], a["v_ctx"], a["offsets"], a["k_blk"], a["v_blk"])
    q_next = rng.standard_normal((B, S, Hq, D))
    kb_next = rng.standard_normal((B, S, Hkv, D))
    vb_next = rng.standard_normal((B, S, Hkv, D))
    grown = dict(q=q_next, k_blk=kb_next, v_blk=vb_next, k_ctx=np.asarray(k_out),
                 v_ctx=np.asarray(v_out), offsets=np.asarray(off_out))
    for b in range(B):
        want_keys = np.concatenate([a["k_ctx"][a["offsets"][b]:a["offsets"][b + 1]],
                                    a["k_blk"][b], kb_next[b]], axis=0)
        want_vals = np.concatenate([a["v_ctx"][a["offsets"][b]:a["offsets"][b + 1]],
                                    a["v_blk"][b], vb_next[b]], axis=0)
        tq = torch.from_numpy(np.ascontiguousarray(q_next[b].transpose(1, 0, 2)))[None]
        tk = torch.from_numpy(np.ascontiguousarray(want_keys.transpose(1, 0, 2)))[None]
        tv = torch.from_numpy(np.ascontiguousarray(want_vals.transpose(1, 0, 2)))[None]
        want = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, enable_gqa=True)[0].numpy().transpose(1, 0, 2)
        _close(sdpa_seq(grown, b), want, what=f"sequence {b}")


APPEND_PINS = [pin_append_time_order, pin_append_offsets_closed_form, pin_append_identities,
               pin_append_two_blocks_at_once, pin_append_then_attend]


# ----------------------------------------------------------------------------
# LM-head pins ([chathome] block-generation and evaluation paragraphs)
# ----------------------------------------------------------------------------
def pin_lmhead_logits_torch(logits_fn):
    """Against torch's float64 linear layer (a different library routine)."""
    rng = np.random.default_rng(51)
    h = rng.standard_normal((2, 3, 40))
    w = rng.standard_normal((50, 40))
    want = torch.nn.functional.linear(torch.from_numpy(h), torch.from_numpy(w)).numpy()
    _close(logits_fn(h, w), want, tol=1e-12, what="logits vs torch linear")


def pin_lmhead_logits_brute(logits_fn):
    """Pure-Python sums on a tiny case, token j's logit = sum_k h_k w[j]_k."""
    rng = np.random.default_rng(52)
    h = rng.integers(-3, 4, (1, 2, 5)).astype(np.float64)
    w = rng.integers(-3, 4, (4, 5)).astype(np.float64)
    got = np.asarray(logits_fn(h, w))
    assert got.shape == (1, 2, 4)
    for i in range(2):
        for j in range(4):
            assert got[0, i, j] == sum(h[0, i, k] * w[j, k] for k in range(5)), (i, j)


def pin_lmhead_identity_head(lmc):
    """With H = V and the identity as LM head, the hidden state is the logit
    row: the hand-derived commit fixture must come out."""
    with open(os.path.join(GOLDEN, "commit_closed_form.json")) as f:
        g = json.load(f)
    x = np.array(g["logits"], dtype=np.float64)
    eye = np.eye(x.shape[-1])
    for case in g["cases"]:
        r = lmc(x, eye, np.array(case["eligible"], dtype=np.uint8), case["gamma"])
        assert np.asarray(r["commit"]).astype(int).tolist() == case["commit"], case["name"]
        assert np.asarray(r["token"]).tolist() == g["token"], case["name"]
        assert np.asarray(r["n_commit"]).tolist() == case["n_commit"], case["name"]
        _close(r["maxprob"], np.array(g["maxprob"]), tol=1e-15, what=case["name"])


def _int_head(seed, B=2, S=4, H=6, V=9):
    rng = np.random.default_rng(seed)
    h = rng.integers(-2, 3, (B, S, H)).astype(np.float64)
    w = rng.integers(-2, 3, (V, H)).astype(np.float64)
    m = rng.integers(0, 2, (B, S)).astype(np.uint8)
    m[:, 0] = 1
    return h, w, m


def pin_lmhead_shift_invariance(lmc):
    """Adding one vector c to every row of the head adds h.c to all logits of
    a position: softmax, argmax and so every decision stay the same (integer
    data keeps this exact)."""
    h, w, m = _int_head(53)
    c = np.array([1.0, -2.0, 0.0, 3.0, 1.0, -1.0])
    for gamma in (0.3, 0.6):
        a = lmc(h, w, m, gamma)
        b = lmc(h, w + c, m, gamma)
        for k in ("commit", "token", "n_commit"):
            assert np.array_equal(np.asarray(a[k]), np.asarray(b[k])), k
        _close(a["maxprob"], b["maxprob"], tol=1e-15, what="maxprob under a shift")


def pin_lmhead_vocab_permutation(lmc):
    """Renumbering the vocabulary (rows of the head) renumbers the argmax and
    leaves the probabilities and the commit decisions unchanged."""
    rng = np.random.default_rng(54)
    h = rng.standard_normal((2, 4, 8))
    w = rng.standard_normal((11, 8))
    m = np.array([[1, 1, 0, 1], [0, 1, 1, 1]], np.uint8)
    perm = rng.permutation(11)                  # new id k is old token perm[k]
    a = lmc(h, w, m, 0.35)
    b = lmc(h, w[perm], m, 0.35)
    assert np.array_equal(perm[np.asarray(b["token"])], np.asarray(a["token"]))
    assert np.array_equal(np.asarray(a["commit"]), np.asarray(b["commit"]))
    _close(a["maxprob"], b["maxprob"], tol=1e-14, what="maxprob under renumbering")


def pin_lmhead_eligibility(lmc):
    """Ineligible positions never commit, and a sequence with no eligible
    position commits nothing; the force-one rule still applies per
    sequence."""
    h, w, _ = _int_head(55)
    m = np.array([[0, 0, 0, 0], [0, 0, 1, 0]], np.uint8)
    r = lmc(h, w, m, 2.0)                          # gamma > 1: force-one only
    c = np.asarray(r["commit"]).astype(bool)
    assert not c[0].any() and c[1].tolist() == [False, False, True, False]
    assert np.asarray(r["n_commit"]).tolist() == [0, 1]


LMHEAD_LOGIT_PINS = [pin_lmhead_logits_torch, pin_lmhead_logits_brute]
LMHEAD_PINS = [pin_lmhead_identity_head, pin_lmhead_shift_invariance, pin_lmhead_vocab_permutation,
               pin_lmhead_eligibility]


# ----------------------------------------------------------------------------
# Mamba-2 block-scan pins ([chathome] inference paragraph: the denoiser's
# Mamba-2 state is seeded from the context tower)
# ----------------------------------------------------------------------------
def _ssm_inputs(seed, B=2, S=5, H=4, P=3, N=6, G=2, A_zero=False, dt_zero=False):
    rng = np.random.default_rng(seed)
    return dict(
        x=rng.standard_normal((B, S, H, P)),
        dt=np.zeros((B, S, H)) if dt_zero else rng.uniform(0.01, 0.3, (B, S, H)),
        A=np.zeros(H) if A_zero else -rng.uniform(0.5, 4.0, H),
        Bm=rng.standard_normal((B, S, G, N)),
        Cm=rng.standard_normal((B, S, G, N)),
        D=rng.uniform(0.5, 1.5, H),
        h0=rng.standard_normal((B, H, P, N)))


def _call_ssm(scan, a):
    return scan(a["x"], a["dt"], a["A"], a["Bm"], a["Cm"], a["D"], a["h0"])


def pin_mamba_closed_form(scan):
    """The block as one sum (the quadratic form of the same recurrence): with
    c_t = sum_{r<=t} dt_r A,
      y_t = e^{c_t} h0 C_t + sum_{s<=t} e^{c_t - c_s} dt_s (C_t . B_s) x_s + D x_t
      h_S = e^{c_S} h0 + sum_s e^{c_S - c_s} dt_s x_s (outer) B_s."""
    a = _ssm_inputs(61)
    y, hS = _call_ssm(scan, a)
    nb, S, H, P = a["x"].shape
    G = a["Bm"].shape[2]
    for b in range(nb):
        for h in range(H):
            g = h // (H // G)
            c = np.cumsum(a["dt"][b, :, h] * a["A"][h])
            for t in range(S):
                want = np.exp(c[t]) * (a["h0"][b, h] @ a["Cm"][b, t, g]) + a["D"][h] * a["x"][b, t, h]
                for s_ in range(t + 1):
                    want = want + (np.exp(c[t] - c[s_]) * a["dt"][b, s_, h]
                                   * (a["Cm"][b, t, g] @ a["Bm"][b, s_, g]) * a["x"][b, s_, h])
                _close(y[b, t, h], want, tol=1e-10, what=f"y b={b} h={h} t={t}")
            wantS = np.exp(c[-1]) * a["h0"][b, h]
            for s_ in range(S):
                wantS = wantS + (np.exp(c[-1] - c[s_]) * a["dt"][b, s_, h]
                                 * np.outer(a["x"][b, s_, h], a["Bm"][b, s_, g]))
            _close(hS[b, h], wantS, tol=1e-10, what=f"h_S b={b} h={h}")


def pin_mamba_zero_step(scan):
    """dt = 0: the state stays the seed, y_t = h0 C_t + D x_t."""
    a = _ssm_inputs(62, dt_zero=True)
    y, hS = _call_ssm(scan, a)
    H, G = a["x"].shape[2], a["Bm"].shape[2]
    grp = np.arange(H) // (H // G)
    want = np.einsum("bhpn,bthn->bthp", a["h0"], a["Cm"][:, :, grp]) + a["D"][None, None, :, None] * a["x"]
    _close(y, want, tol=1e-12, what="dt = 0")
    _close(hS, a["h0"], tol=0.0, what="state unchanged")


def pin_mamba_no_decay(scan):
    """A = 0: no decay, the state is the seed plus running sums of
    dt_s x_s (outer) B_s (cumulative sums along the block)."""
    a = _ssm_inputs(63, A_zero=True)
    y, hS = _call_ssm(scan, a)
    H, G = a["x"].shape[2], a["Bm"].shape[2]
    grp = np.arange(H) // (H // G)
    upd = np.einsum("bth,bthp,bthn->bthpn", a["dt"], a["x"], a["Bm"][:, :, grp])
    states = a["h0"][:, None] + np.cumsum(upd, axis=1)
    want = np.einsum("bthpn,bthn->bthp", states, a["Cm"][:, :, grp]) + a["D"][None, None, :, None] * a["x"]
    _close(y, want, tol=1e-10, what="A = 0")
    _close(hS, states[:, -1], tol=1e-10, what="A = 0 final state")


def pin_mamba_state_passing(scan):
    """Scanning the first 3 tokens, then the last 4 from the state they
    leave, is scanning all 7 at once: the seed is exactly the state the
    earlier tokens produce (what seeding from the context tower means)."""
    a = _ssm_inputs(64, S=7)
    y, hS = _call_ssm(scan, a)
    first = {k: (v[:, :3] if k in ("x", "dt", "Bm", "Cm") else v) for k, v in a.items()}
    y1, h1 = _call_ssm(scan, first)
    second = {k: (v[:, 3:] if k in ("x", "dt", "Bm", "Cm") else v) for k, v in a.items()}
    second["h0"] = np.asarray(h1)
    y2, h2 = _call_ssm(scan, second)
    _close(np.concatenate([np.asarray(y1), np.asarray(y2)], axis=1), y, tol=1e-10, what="split scan")
    _close(h2, hS, tol=1e-10, what="split final state")


def pin_mamba_brute(scan):
    """Pure-Python loops on a tiny case (one group, scalars only)."""
    a = _ssm_inputs(65, B=1, S=3, H=2, P=2, N=2, G=1)
    y, hS = _call_ssm(scan, a)
    for h in range(2):
        st = [[float(a["h0"][0, h, p, n]) for n in range(2)] for p in range(2)]
        for t in range(3):
            dec = math.exp(float(a["dt"][0, t, h]) * float(a["A"][h]))
            for p in range(2):
                for n in range(2):
                    st[p][n] = dec * st[p][n] + float(a["dt"][0, t, h]) * float(a["x"][0, t, h, p]) * float(a["Bm"][0, t, 0, n])
            for p in range(2):
                yt = sum(st[p][n] * float(a["Cm"][0, t, 0, n]) for n in range(2)) + float(a["D"][h]) * float(a["x"][0, t, h, p])
                assert abs(y[0, t, h, p] - yt) < 1e-12, (h, t, p)
        for p in range(2):
            for n in range(2):
                assert abs(hS[0, h, p, n] - st[p][n]) < 1e-12


def pin_mamba_groups(scan):
    """Heads read their group's projections: with one group per head and each
    head's projections copied from its group, the result is unchanged."""
    a = _ssm_inputs(66, H=6, G=2)
    y, hS = _call_ssm(scan, a)
    b = dict(a)
    grp = np.arange(6) // 3
    b["Bm"], b["Cm"] = a["Bm"][:, :, grp], a["Cm"][:, :, grp]
    y2, hS2 = _call_ssm(scan, b)
    _close(y2, y, tol=1e-12, what="groups vs per-head copies")
    _close(hS2, hS, tol=1e-12, what="groups vs per-head copies (state)")


MAMBA_PINS = [pin_mamba_closed_form, pin_mamba_zero_step, pin_mamba_no_decay, pin_mamba_state_passing,
              pin_mamba_brute, pin_mamba_groups]


# ----------------------------------------------------------------------------
# adaLN-single modulation between layers ([chathome] inference paragraph)
# ----------------------------------------------------------------------------
def _ada_inputs(seed, B=3, S=4, H=8, with_f=True, tables=True, eps=1e-5):
    rng = np.random.default_rng(seed)
    return dict(
        x=rng.standard_normal((B, S, H)) * 2.0,
        f=rng.standard_normal((B, S, H)) if with_f else None,
        t_mod=rng.standard_normal((B, 3, H)) * 0.5,
        tab_gate=rng.standard_normal(H) * 0.3 if tables else None,
        tab_shift=rng.standard_normal(H) * 0.3 if tables else None,
        tab_scale=rng.standard_normal(H) * 0.3 if tables else None,
        w_norm=rng.uniform(0.5, 1.5, H) if tables else None,
        eps=eps)


def _call_ada(fn, a):
    return fn(a["x"], a["f"], a["t_mod"], a["tab_gate"], a["tab_shift"], a["tab_scale"],
              a["w_norm"], a["eps"])


def pin_adaln_rmsnorm_library(fn):
    """No residual and no modulation: h is torch's own RMSNorm (float64)."""
    a = _ada_inputs(71, with_f=False)
    a["t_mod"] = np.zeros_like(a["t_mod"])
    a["tab_gate"] = a["tab_shift"] = a["tab_scale"] = None
    r, h = _call_ada(fn, a)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(a["x"]), (a["x"].shape[-1],),
                                       weight=torch.from_numpy(a["w_norm"]), eps=a["eps"]).numpy()
    assert np.allclose(h, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(r, a["x"])


def pin_adaln_closed_form(fn):
    """Rows of +-c (every |r_j| = c, eps = 0) normalise to +-1, so
    h_j = sign_j w_j (1 + scale_j) + shift_j exactly, for any c > 0."""
    B, S, H = 2, 3, 6
    rng = np.random.default_rng(72)
    sign = rng.choice([-1.0, 1.0], (B, S, H))
    c = np.array([0.25, 3.0, 40.0])[None, :, None]
    x = sign * c
    t_mod = rng.standard_normal((B, 3, H))
    w = rng.uniform(0.5, 2.0, H)
    r, h = fn(x, None, t_mod, None, None, None, w, 0.0)
    ref = sign * w * (1.0 + t_mod[:, 1][:, None, :]) + t_mod[:, 0][:, None, :]
    assert np.allclose(h, ref, rtol=1e-13, atol=1e-13)


def pin_adaln_gate_cases(fn):
    """Gate 0 leaves the stream alone (r = x, h as with no residual); gate 1
    with f = -x empties the row, whose normalised value is then 0 and h is the
    shift alone; a gate of g with f = x scales the row by 1 + g, which the
    norm removes (g > -1, eps = 0)."""
    a = _ada_inputs(73)
    a["t_mod"][:, 2, :] = 0.0
    a["tab_gate"] = np.zeros_like(a["tab_gate"])
    r0, h0 = _call_ada(fn, a)
    b = dict(a, f=None)
    r1, h1 = _call_ada(fn, b)
    assert np.array_equal(r0, a["x"]) and np.allclose(h0, h1, rtol=1e-13, atol=1e-13)
    c = dict(a, f=-a["x"])
    c["t_mod"] = a["t_mod"].copy()
    c["t_mod"][:, 2, :] = 1.0
    r2, h2 = _call_ada(fn, c)
    shift = a["t_mod"][:, 0, :] + a["tab_shift"]
    assert np.allclose(r2, 0.0, atol=1e-15)
    assert np.allclose(h2, np.broadcast_to(shift[:, None, :], h2.shape), rtol=1e-13, atol=1e-13)
    d = dict(c, f=a["x"], eps=0.0)
    d["t_mod"] = c["t_mod"].copy()
    d["t_mod"][:, 2, :] = 0.75
    r3, h3 = _call_ada(fn, d)
    r4, h4 = _call_ada(fn, dict(d, f=None))
    assert np.allclose(r3, 1.75 * a["x"], rtol=1e-14, atol=1e-14)
    assert np.allclose(h3, h4, rtol=1e-12, atol=1e-12)


def pin_adaln_scale_invariance(fn):
    """RMSNorm with eps = 0 ignores the row's scale: x and c x (c > 0) give
    the same h; -x gives -h when the shift is zero."""
    a = _ada_inputs(74, with_f=False, eps=0.0)
    _, h = _call_ada(fn, a)
    _, hc = _call_ada(fn, dict(a, x=a["x"] * 7.5))
    assert np.allclose(h, hc, rtol=1e-12, atol=1e-12)
    z = dict(a, tab_shift=None)
    z["t_mod"] = a["t_mod"].copy()
    z["t_mod"][:, 0, :] = 0.0
    _, hp = _call_ada(fn, z)
    _, hn = _call_ada(fn, dict(z, x=-a["x"]))
    assert np.allclose(hn, -hp, rtol=1e-13, atol=1e-13)


def pin_adaln_only_sum_matters(fn):
    """A layer's modulation is the shared vector plus the layer's table: moving
    any amount between the two changes nothing."""
    a = _ada_inputs(75)
    r, h = _call_ada(fn, a)
    rng = np.random.default_rng(76)
    delta = rng.standard_normal((3, a["x"].shape[-1]))
    b = dict(a, t_mod=a["t_mod"] + delta[None], tab_shift=a["tab_shift"] - delta[0],
             tab_scale=a["tab_scale"] - delta[1], tab_gate=a["tab_gate"] - delta[2])
    r2, h2 = _call_ada(fn, b)
    assert np.allclose(r, r2, rtol=1e-12, atol=1e-12) and np.allclose(h, h2, rtol=1e-12, atol=1e-12)


def pin_adaln_per_sequence(fn):
    """Each sequence reads its own timestep vectors: permuting the sequences
    (inputs and t_mod together) permutes the outputs; the positions of one
    sequence do not interact (changing one position leaves the others)."""
    a = _ada_inputs(77, B=4)
    r, h = _call_ada(fn, a)
    perm = np.array([2, 0, 3, 1])
    b = dict(a, x=a["x"][perm], f=a["f"][perm], t_mod=a["t_mod"][perm])
    r2, h2 = _call_ada(fn, b)
    assert np.allclose(r2, r[perm], rtol=1e-14, atol=1e-14)
    assert np.allclose(h2, h[perm], rtol=1e-14, atol=1e-14)
    c = dict(a, x=a["x"].copy())
    c["x"][1, 2] += 5.0
    r3, h3 = _call_ada(fn, c)
    keep = np.ones(a["x"].shape[:2], bool)
    keep[1, 2] = False
    assert np.array_equal(h3[keep], h[keep]) and not np.allclose(h3[1, 2], h[1, 2])


def pin_adaln_brute(fn):
    """Pure-Python loops on a tiny case."""
    a = _ada_inputs(78, B=2, S=2, H=3)
    r, h = _call_ada(fn, a)
    for b in range(2):
        for s in range(2):
            rr = []
            for j in range(3):
                g = float(a["t_mod"][b, 2, j]) + float(a["tab_gate"][j])
                rr.append(float(a["x"][b, s, j]) + g * float(a["f"][b, s, j]))
            ms = sum(v * v for v in rr) / 3.0
            inv = 1.0 / math.sqrt(ms + a["eps"])
            for j in range(3):
                sc = 1.0 + float(a["t_mod"][b, 1, j]) + float(a["tab_scale"][j])
                sh = float(a["t_mod"][b, 0, j]) + float(a["tab_shift"][j])
                want = rr[j] * inv * float(a["w_norm"][j]) * sc + sh
                assert abs(r[b, s, j] - rr[j]) <= 1e-12
                assert abs(h[b, s, j] - want) <= 1e-12 * max(1.0, abs(want))


ADALN_PINS = [pin_adaln_rmsnorm_library, pin_adaln_closed_form, pin_adaln_gate_cases,
              pin_adaln_scale_invariance, pin_adaln_only_sum_matters, pin_adaln_per_sequence,
              pin_adaln_brute]

