"""GPU parity of the context-cache append (td_cache_append, through the C
ABI) against the oracle's cache_append: a copy, so every output byte and every
offset must match exactly.  Inputs are the seeded attention inputs (the block
K/V play the committed tokens' rows); cases span several 64-row workgroups,
ragged tails, empty sequences, S = 0, an empty cache, rows that are not a
power-of-two number of 16-byte vectors, and the full batched workload."""
import numpy as np
import pytest
import torch

import block_diffusion_lm_td_amd as td
import oracle
import synth
from gpu_util import check_attn, dev, f64, log, oracle_attn, run_attn

pytestmark = pytest.mark.gpu
W = synth.WORKLOADS
SENTINEL = -21846        # 0xAAAA: what the outputs hold before the call


def _inputs(B, S, Hkv, D, dtype, lengths, seed):
    w = W["tiny_f32_b1_ctx64"].with_(B=B, S=S, Hq=Hkv, Hkv=Hkv, D=D, dtype=dtype)
    return synth.make_attention_inputs(w, seed, lengths=lengths)


def _run_append(a, k_ctx=None, v_ctx=None, off=None):
    """Upload (unless device tensors are given), append the block rows, return
    the device outputs."""
    dt = a["dtype"]
    k_new, v_new = dev(a["k_blk"], dt), dev(a["v_blk"], dt)
    if k_ctx is None:
        k_ctx, v_ctx = dev(a["k_ctx"], dt), dev(a["v_ctx"], dt)
        off = torch.from_numpy(a["offsets"]).to("cuda")
    B, S, Hkv, D = k_new.shape
    T = k_ctx.shape[0]
    N = T + B * S
    k_out = torch.empty((N, Hkv, D), dtype=k_new.dtype, device="cuda")
    v_out = torch.empty_like(k_out)
    for t in (k_out, v_out):
        t.view(torch.int16).fill_(SENTINEL)
    off_out = torch.full((B + 1,), -5, dtype=torch.int64, device="cuda")
    td.td_cache_append(k_ctx, v_ctx, off, k_new, v_new, k_out, v_out, off_out, total_ctx=T)
    torch.cuda.synchronize()
    return k_out, v_out, off_out


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _want(a):
    """The oracle on the raw element bits: a copy is the same for any dtype."""
    return oracle.cache_append(a["k_ctx"], a["v_ctx"], a["offsets"], a["k_blk"], a["v_blk"])


def _check(got, want, label):
    k_out, v_out, off_out = got
    wk, wv, wo = want
    log(f"[append] {label}: rows={wk.shape[0]}")
    assert np.array_equal(off_out.cpu().numpy(), wo), label
    view = np.int16 if wk.dtype == np.uint16 else np.int32
    assert np.array_equal(_bits(k_out), np.ascontiguousarray(wk).view(view)), label
    assert np.array_equal(_bits(v_out), np.ascontiguousarray(wv).view(view)), label


def _cases(n=20, seed=777):
    rng = np.random.default_rng(seed)
    shapes = [(2, 128, "bf16"), (1, 64, "f32"), (3, 64, "bf16"), (4, 8, "f32"), (1, 8, "bf16"),
              (8, 128, "f32")]
    out = []
    for i in range(n):
        B = int(rng.integers(1, 12))
        S = int(rng.choice([0, 1, 3, 16, 64]))
        Hkv, D, dt = shapes[i % len(shapes)]
        lengths = rng.integers(0, 300, B) * (rng.random(B) > 0.25)
        out.append((i, B, S, Hkv, D, dt, [int(x) for x in lengths]))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"r{c[0]}")
def test_append_random_shapes(case):
    i, B, S, Hkv, D, dt, lengths = case
    log(f"case append random r{i}: B={B} S={S} Hkv={Hkv} D={D} {dt} lengths={lengths}")
    a = _inputs(B, S, Hkv, D, dt, lengths, 9000 + i)
    _check(_run_append(a), _want(a), f"r{i}")


@pytest.mark.parametrize("lengths,S", [([0, 0, 0], 16), ([0], 1), ([64, 0, 63, 65], 0),
                                       ([1], 0), ([0, 5000, 0], 7)])
def test_append_edges(lengths, S):
    """Empty cache, a single row, S = 0 (a plain repack), one-row cache,
    empty neighbours of a long sequence."""
    log(f"case append edges lengths={lengths} S={S}")
    a = _inputs(len(lengths), S, 2, 128, "bf16", lengths, 9100)
    _check(_run_append(a), _want(a), f"lengths={lengths} S={S}")


def test_append_b64_ragged_full():
    """The batched workload's cache (64 sequences, 1K..8K rows, 2 KV heads of
    128 bf16) grows by the 16 rows of the block: every byte checked."""
    w = W["bf16_b64_ragged1k_8k"]
    a = synth.make_attention_inputs(w, 1003)
    log(f"case append b64 ragged full, total_ctx={a['total_ctx']}")
    _check(_run_append(a), _want(a), "b64 ragged1k_8k")


def test_append_twice_alternating_buffers():
    """Two blocks in a row: the first append's outputs are the second's
    inputs (two caches used alternately)."""
    a = _inputs(5, 16, 2, 128, "bf16", [100, 0, 257, 64, 1], 9200)
    b = _inputs(5, 16, 2, 128, "bf16", [0, 0, 0, 0, 0], 9201)     # only its block rows are used
    log("case append twice")
    k1, v1, o1 = _run_append(a)
    b2 = dict(b, k_ctx=None, v_ctx=None)
    got = _run_append(b2, k1, v1, o1)
    wk, wv, wo = _want(a)
    want = oracle.cache_append(wk, wv, wo, b["k_blk"], b["v_blk"])
    _check(got, want, "second append")


def test_append_then_next_block_attention():
    """The next block's attention over the grown cache (td_block_attn on the
    appended cache) against the oracle's attention over the oracle's appended
    cache."""
    w = W["bf16_b8_ctx4k"].with_(B=6)
    a = synth.make_attention_inputs(w, 9300, lengths=[4096, 0, 1000, 77, 4095, 2048])
    k_out, v_out, off_out = _run_append(a)
    nxt = synth.make_attention_inputs(w, 9301, lengths=[0] * 6)
    wk, wv, wo = _want(a)
    grown = dict(nxt, k_ctx=wk, v_ctx=wv, offsets=wo, total_ctx=int(wo[-1]),
                 max_ctx=int(np.diff(wo).max()), lengths=np.diff(wo))
    log("case append then attention, lengths", np.diff(wo))
    d = {k: dev(nxt[k], "bf16") for k in ("q", "k_blk", "v_blk")}
    d.update(k_ctx=k_out, v_ctx=v_out, offsets=off_out, out=torch.empty_like(d["q"]))
    got = run_attn(d, grown)
    check_attn(got, oracle_attn(grown), "attention over the appended cache")
