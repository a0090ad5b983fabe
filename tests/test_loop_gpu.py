"""The block's step loop on the device at the loop workload's full shape,
checked step by step against the fp64 oracle.

A block of S [MASK] positions is refined step by step, several positions
committing per step, until every position has committed (news.chathome.org,
"NVIDIA releases Nemotron-Labs-TwoTower ...", block-generation paragraph;
the threshold gamma from its evaluation paragraph).  Here the loop runs as
td_denoise_step_if steps, each gated by the previous step's n_masked_left, at
32 sequences of 2048 cached tokens, 32 query / 2 KV heads, head dim 128 and a
131072-entry vocabulary, S in {16, 32, 64} and gamma in {0.5, 0.8, 0.95}:

  * chunked: steps enqueued 8 at a time with one host synchronisation per
    chunk (the loop stops once a chunk's last step reports nothing left);
  * graph: all S gated steps captured once in a HIP graph and replayed twice,
    with eager resets and synchronisations between the replays.

Every step's inputs and outputs are copied aside on the device as the loop
runs (masked state before the step, commit, argmax ids, maxprob, n_commit,
tokens, masked state after it, n_masked_left, and the attention output of
two sequences).  Afterwards each active step is compared teacher-forced with
the oracle: oracle.commit_decision over oracle.row_confidence of that step's
logits, from the GPU's own masked state before the step, bit-exact except
positions whose oracle maxprob lies within 1e-4 of gamma (excluded and
counted, see gpu_util.compare_commit); the attention output of the two
sequences against oracle.block_attention (max abs <= 2e-2, mean abs <= 2e-3,
relative L2 <= 1e-2).  Steps after the block has finished must leave every
state untouched and report n_masked_left = 0.
"""
import numpy as np
import pytest
import torch

import block_diffusion_lm_td_amd as td
import oracle
import synth
from gpu_util import check_attn, compare_commit, dev, f64, log, oracle_attn, upload_attn

pytestmark = pytest.mark.gpu
CHUNK = 8
GAMMAS = (0.5, 0.8, 0.95)
SEQS = (0, 31)                       # sequences whose attention output is checked each step


@pytest.fixture(autouse=True)
def _no_plan_override(monkeypatch):
    monkeypatch.delenv("TD_ATTN_GRID", raising=False)
    monkeypatch.delenv("TD_COMMIT_SPLIT", raising=False)


class _Hist:
    """Device copies of every step's state, indexed by step."""

    def __init__(self, B, S, Hq, D):
        z = lambda shape, dt: torch.zeros(shape, dtype=dt, device="cuda")
        self.masked_before = z((S, B, S), torch.uint8)
        self.masked_after = z((S, B, S), torch.uint8)
        self.commit = z((S, B, S), torch.uint8)
        self.token = z((S, B, S), torch.int32)
        self.maxprob = z((S, B, S), torch.float32)
        self.n_commit = z((S, B), torch.int32)
        self.tokens = z((S, B, S), torch.int32)
        self.left = torch.full((S,), -1, dtype=torch.int32, device="cuda")
        self.out = torch.zeros((S, len(SEQS), S, Hq, D), dtype=torch.bfloat16, device="cuda")

    def host(self):
        return {k: getattr(self, k).cpu().numpy() if k != "out" else
                getattr(self, k).float().cpu().numpy().astype(np.float64)
                for k in ("masked_before", "masked_after", "commit", "token", "maxprob",
                          "n_commit", "tokens", "left", "out")}


def _check_history(h, conf_at, ref_attn, gamma, S, label):
    """Teacher-forced comparison of every active step with the oracle."""
    left = h["left"].tolist()
    assert 0 in left, f"{label}: the block did not finish within S={S} steps: {left}"
    n = left.index(0) + 1
    B = h["commit"].shape[1]
    tokens_in = np.full((B, S), -1, np.int64)
    exc_pos = exc_seq = 0
    for k in range(n):
        p, tok = conf_at(k)
        masked = h["masked_before"][k]
        ref = oracle.commit_decision(p, tok, masked, gamma)
        g = dict(commit=h["commit"][k], token=h["token"][k], maxprob=h["maxprob"][k],
                 n_commit=h["n_commit"][k], masked_out=h["masked_after"][k],
                 tokens=h["tokens"][k], n_masked_left=np.array([left[k]]))
        ep, es = compare_commit(g, ref, masked, gamma, tokens_in, f"{label} step {k}")
        exc_pos += ep
        exc_seq += es
        assert left[k] == int(h["masked_after"][k].astype(bool).sum()), f"{label} step {k}"
        if k + 1 < S:
            assert (h["masked_before"][k + 1] == h["masked_after"][k]).all(), f"{label} step {k}"
        tokens_in = h["tokens"][k].astype(np.int64)
        check_attn(h["out"][k], ref_attn, f"{label} step {k} seqs {SEQS}")
    for k in range(n, S):                         # gated off: nothing moves
        assert left[k] == 0, f"{label}: step {k} after the end reports {left[k]}"
        assert not h["masked_after"][k].any(), f"{label}: step {k}"
        assert (h["tokens"][k] == h["tokens"][n - 1]).all(), f"{label}: step {k} changed tokens"
    assert (h["tokens"][n - 1] >= 0).all(), f"{label}: a position never committed"
    log(f"[loop {label}] {n} active steps of {S}; excluded positions={exc_pos} sequences={exc_seq}")
    return n


@pytest.mark.parametrize("S", [16, 32, 64])
def test_gated_loop_full_shape_vs_oracle(S):
    w0 = synth.WORKLOADS["bf16_b32_ctx2k_loop"].with_(S=S)
    B, V = w0.B, w0.V
    log(f"case gated loop B={B} ctx={w0.ctx_lo} V={V} S={S}: generating inputs")
    a = synth.make_attention_inputs(w0, 7000 + S)
    base, peak, stored = synth.loop_peak_values(w0, 7100 + S, S + 1)
    d = upload_attn(a)
    logits = dev(base, "bf16").view(B, S, V)
    rows = torch.arange(B * S, device="cuda")
    peak_d = torch.from_numpy(peak).to("cuda")
    stored_d = dev(stored, "bf16")
    ref_attn = oracle_attn(a, SEQS)
    seq_idx = torch.tensor(SEQS, device="cuda")

    conf = {}

    def conf_at(t):
        """Oracle confidence and argmax of every position at step t."""
        if t not in conf:
            x = f64(synth.loop_step_logits(base, peak, stored, t), "bf16")
            p, tok = oracle.row_confidence(x)
            conf[t] = (p.reshape(B, S), tok.reshape(B, S))
        return conf[t]

    out = torch.empty_like(d["q"])
    aa = td.attn_args(d["q"], d["k_blk"], d["v_blk"], d["k_ctx"], d["v_ctx"], d["offsets"], out,
                      a["total_ctx"], a["max_ctx"])
    z = lambda shape, dt: torch.zeros(shape, dtype=dt, device="cuda")
    st = dict(commit=z((B, S), torch.uint8), token=z((B, S), torch.int32),
              maxprob=z((B, S), torch.float32), n_commit=z((B,), torch.int32),
              masked=z((B, S), torch.uint8), tokens=z((B, S), torch.int32))
    cnt = torch.zeros((2,), dtype=torch.int32, device="cuda")
    ws = td.Workspace(torch.device("cuda"))

    def reset(hist):
        for k in ("commit", "token", "maxprob", "n_commit"):
            st[k].zero_()
        st["masked"].fill_(1)
        st["tokens"].fill_(-1)
        cnt.zero_()
        cnt[1] = 1                                   # opens step 0
        hist.left.fill_(-1)

    def one_step(k, cargs, hist):
        logits.view(-1, V)[rows, peak_d] = stored_d[k]
        hist.masked_before[k].copy_(st["masked"])
        td.td_denoise_step_if(aa, cargs[k % 2], cnt[(k + 1) % 2:(k + 1) % 2 + 1], workspace=ws)
        hist.commit[k].copy_(st["commit"])
        hist.token[k].copy_(st["token"])
        hist.maxprob[k].copy_(st["maxprob"])
        hist.n_commit[k].copy_(st["n_commit"])
        hist.tokens[k].copy_(st["tokens"])
        hist.masked_after[k].copy_(st["masked"])
        hist.left[k:k + 1].copy_(cnt[k % 2:k % 2 + 1])
        hist.out[k].copy_(out.index_select(0, seq_idx))

    for gamma in GAMMAS:
        cargs = [td.commit_args(logits, st["commit"], st["token"], gamma, st["masked"],
                                st["maxprob"], st["n_commit"], st["masked"], st["tokens"],
                                cnt[k:k + 1]) for k in range(2)]
        # ---- chunked: CHUNK gated steps per host synchronisation
        log(f"case gated loop S={S} gamma={gamma}: chunked")
        hist = _Hist(B, S, w0.Hq, w0.D)
        reset(hist)
        k = 0
        while k < S:
            for _ in range(min(CHUNK, S - k)):
                one_step(k, cargs, hist)
                k += 1
            torch.cuda.synchronize()
            if int(cnt[(k + 1) % 2].item()) == 0:      # the last step's n_masked_left
                break
        for j in range(k, S):                          # steps never enqueued: nothing left
            hist.left[j] = 0
            hist.masked_before[j].copy_(st["masked"])
            hist.masked_after[j].copy_(st["masked"])
            hist.tokens[j].copy_(st["tokens"])
        torch.cuda.synchronize()
        n_chunked = _check_history(hist.host(), conf_at, ref_attn, gamma, S,
                                   f"S={S} gamma={gamma} chunked")

        # ---- graph: all S gated steps captured once, replayed twice
        log(f"case gated loop S={S} gamma={gamma}: graph capture")
        hist = _Hist(B, S, w0.Hq, w0.D)
        reset(hist)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for k in range(S):
                one_step(k, cargs, hist)
        for rep in range(2):
            reset(hist)                                # eager work between replays
            torch.cuda.synchronize()
            log(f"case gated loop S={S} gamma={gamma}: graph replay {rep}")
            graph.replay()
            torch.cuda.synchronize()
            n = _check_history(hist.host(), conf_at, ref_attn, gamma, S,
                               f"S={S} gamma={gamma} graph replay {rep}")
            assert n == n_chunked
        del graph
