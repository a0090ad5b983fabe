"""fp64 CPU oracle of one denoising step of the TwoTower diffusion denoiser.

TEST INFRASTRUCTURE.  Only tests/, ``__graft_entry__.smoke()`` and the bench's
``cpu_baseline`` leg may import or run this module; the HIP product path never
does, and this module imports nothing from it.  Everything is plain numpy in
float64; inputs arrive as the exact float32 / bf16 values the GPU consumes,
upcast without loss.

Sources (the pages are news articles on NVIDIA's Nemotron-Labs-TwoTower):
  [chathome]  news.chathome.org, "NVIDIA releases Nemotron-Labs-TwoTower: an
              open-weight diffusion language model built on a frozen
              autoregressive backbone" (Japanese).  Its inference paragraph
              (5th) describes the two towers' attention; the block-generation
              paragraph (6th) the step loop; the evaluation paragraph (7th)
              the confidence threshold gamma = 0.8 and block size S = 16.
  [aiboss]    aiboss88.com, "Nemotron-Labs-TwoTower - NVIDIA's open-source
              dual-tower diffusion language model", technical-principle
              section: bidirectional block attention plus cross-attention.
  [aikraft]   aikraft.ru, architecture section: the denoiser cross-attends to
              the context tower's layers; results section: gamma, S.

Readings where the pages are silent:
  * block attention and the layer-aligned cross-attention are ONE softmax over
    the keys [context ; block] -- the only reading under which an empty
    context gives plain bidirectional block attention and S = 1 gives causal
    decode over the cache;
  * the context keys/values are the context tower's layer cache used as-is;
    all of a sequence's cached keys are visible (the cache only holds the
    prompt and committed tokens, which is what "causal w.r.t. past clean
    blocks" asks);
  * grouped-query attention with contiguous groups: KV head = h // (Hq/Hkv);
  * scale 1/sqrt(D); no mask, positional term, bias, softcap or window;
  * commit: greedy (argmax token, lowest id on ties), confidence = the
    largest softmax probability, commit when p >= gamma with gamma taken as
    the float32 value the GPU sees; if no eligible position reaches gamma,
    the eligible position of largest p (lowest position on ties) commits;
    committed positions are never re-masked.
Every function below has independent pins in tests/ (library routines,
closed forms, invariants, brute force).
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------
# Attention: S block queries over [context cache ; block], one softmax
# ([chathome] inference paragraph; [aiboss] technical principle)
# ----------------------------------------------------------------------------
def block_attention(q, k_blk, v_blk, k_ctx, v_ctx, offsets, scale=None):
    """Denoiser attention of one layer for a batch of blocks.

    q      [B, S, Hq, D]   block queries (the denoiser's projections)
    k_blk  [B, S, Hkv, D]  block keys;    v_blk the same shape
    k_ctx  [T, Hkv, D]     context tower's cached keys of this layer, packed
                           per sequence: sequence b owns rows
                           offsets[b] .. offsets[b+1]; v_ctx the same shape
    offsets int [B+1]      offsets[0] = 0, non-decreasing; L_b may be 0
    Returns O [B, S, Hq, D] in float64.

    For sequence b and query head h (KV head g = h // (Hq/Hkv)):
        K = [k_ctx[offsets[b]:offsets[b+1], g] ; k_blk[b, :, g]]
        V = [v_ctx[offsets[b]:offsets[b+1], g] ; v_blk[b, :, g]]
        O[b, :, h] = softmax(scale * q[b, :, h] K^T, over keys) V
    """
    q = np.asarray(q, dtype=np.float64)
    k_blk = np.asarray(k_blk, dtype=np.float64)
    v_blk = np.asarray(v_blk, dtype=np.float64)
    k_ctx = np.asarray(k_ctx, dtype=np.float64)
    v_ctx = np.asarray(v_ctx, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    B, S, Hq, D = q.shape
    Hkv = k_blk.shape[2]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((B, S, Hq, D), dtype=np.float64)
    for b in range(B):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        for h in range(Hq):
            g = h // G
            K = np.concatenate([k_ctx[lo:hi, g, :], k_blk[b, :, g, :]], axis=0)
            V = np.concatenate([v_ctx[lo:hi, g, :], v_blk[b, :, g, :]], axis=0)
            s = scale * (q[b, :, h, :] @ K.T)                  # [S, L_b + S]
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[b, :, h, :] = p @ V
    return out


# ----------------------------------------------------------------------------
# Confidence of every block position ([chathome] evaluation paragraph:
# confidence masking with threshold gamma)
# ----------------------------------------------------------------------------
def row_confidence(logits):
    """Per row of ``logits`` [..., V]: (p, token) where token is the first
    index of the row maximum and p = max_j softmax(x)_j = 1 / sum_j exp(x_j - max x).
    """
    x = np.asarray(logits, dtype=np.float64)
    m = x.max(axis=-1)
    token = x.argmax(axis=-1).astype(np.int64)        # numpy: first occurrence
    z = np.exp(x - m[..., None]).sum(axis=-1)
    return 1.0 / z, token


def confidence_commit(logits, eligible, gamma):
    """One commit decision per sequence.

    logits   [B, S, V]; eligible uint8/bool [B, S] (1 = still [MASK]) or None
    gamma    threshold; compared as float64(float32(gamma)).
    Returns dict(commit bool [B,S], token int64 [B,S], maxprob float64 [B,S],
                 n_commit int64 [B]).

    The confidence of every position (row_confidence), then the decision
    (commit_decision).
    """
    p, token = row_confidence(logits)
    return commit_decision(p, token, eligible, gamma)


def commit_decision(p, token, eligible, gamma):
    """The block decision of one step from every position's confidence p
    [B, S] and argmax token [B, S] (as row_confidence returns them).

    C_b = {i eligible : p_i >= gamma}; if C_b is empty while some position is
    eligible, C_b = {the eligible i of largest p_i, lowest i on ties}.
    ([chathome] block-generation paragraph: several tokens may commit per
    step, and every block finishes; evaluation paragraph: threshold gamma.)
    Returns the same dict as confidence_commit.
    """
    p = np.asarray(p, dtype=np.float64)
    token = np.asarray(token, dtype=np.int64)
    B, S = p.shape
    elig = np.ones((B, S), dtype=bool) if eligible is None else np.asarray(eligible).astype(bool)
    g = float(np.float32(gamma))
    commit = elig & (p >= g)
    for b in range(B):
        if not commit[b].any() and elig[b].any():
            cand = np.where(elig[b], p[b], -np.inf)
            commit[b, int(np.argmax(cand))] = True
    return dict(commit=commit, token=token, maxprob=p, n_commit=commit.sum(axis=1))


# ----------------------------------------------------------------------------
# One denoise step, and the block loop ([chathome] block-generation paragraph)
# ----------------------------------------------------------------------------
def denoise_step(attn_inputs, logits, masked_in, tokens_in, gamma, scale=None):
    """Attention of the block (the layer's output) plus the commit of the
    block's logits.  Returns dict(out, commit, token, maxprob, n_commit,
    masked_out, tokens, n_masked_left)."""
    a = attn_inputs
    out = block_attention(a["q"], a["k_blk"], a["v_blk"], a["k_ctx"], a["v_ctx"],
                          a["offsets"], scale)
    c = confidence_commit(logits, masked_in, gamma)
    masked_out = np.asarray(masked_in).astype(bool) & ~c["commit"]
    tokens = np.array(tokens_in, dtype=np.int64, copy=True)
    tokens[c["commit"]] = c["token"][c["commit"]]
    return dict(out=out, masked_out=masked_out, tokens=tokens,
                n_masked_left=int(masked_out.sum()), **c)


def denoise_loop(step_logits, B, S, gamma, max_steps=None):
    """Commit loop of one block: start with every position [MASK] and commit
    until none is left.  ``step_logits(t)`` returns the logits [B, S, V] of
    step t.  Returns dict(steps, tokens, commits_per_step [steps, B],
    steps_per_seq [B])."""
    masked = np.ones((B, S), dtype=bool)
    tokens = np.full((B, S), -1, dtype=np.int64)
    per_step = []
    steps_per_seq = np.zeros(B, dtype=np.int64)
    t = 0
    limit = S if max_steps is None else max_steps
    while masked.any() and t < limit:
        c = confidence_commit(step_logits(t), masked, gamma)
        tokens[c["commit"]] = c["token"][c["commit"]]
        steps_per_seq += masked.any(axis=1)
        masked &= ~c["commit"]
        per_step.append(c["n_commit"])
        t += 1
    return dict(steps=t, tokens=tokens, commits_per_step=np.array(per_step),
                steps_per_seq=steps_per_seq, done=not masked.any())


# ----------------------------------------------------------------------------
# LM head of the block's positions, then the commit ([chathome] block-
# generation and evaluation paragraphs: every step scores the vocabulary at
# each block position and commits by confidence)
# ----------------------------------------------------------------------------
def lmhead_logits(hidden, w_head):
    """Vocabulary logits of every block position: the final hidden state
    hidden [B, S, H] against the LM-head weight w_head [V, H], one row per
    token id.  Returns logits [B, S, V] in float64."""
    h = np.asarray(hidden, dtype=np.float64)
    w = np.asarray(w_head, dtype=np.float64)
    B, S, H = h.shape
    return (h.reshape(B * S, H) @ w.T).reshape(B, S, w.shape[0])


def lmhead_commit(hidden, w_head, masked_in, gamma):
    """The commit of one step taken straight from the hidden states: the
    confidence commit over lmhead_logits(hidden, w_head).  Returns the
    confidence_commit dict."""
    return confidence_commit(lmhead_logits(hidden, w_head), masked_in, gamma)


# ----------------------------------------------------------------------------
# Context-cache append after a block has committed
# ([chathome] block-generation paragraph)
# ----------------------------------------------------------------------------
def cache_append(k_ctx, v_ctx, offsets, k_new, v_new):
    """Context-cache update after a block has committed: every sequence's
    cached keys/values are followed by the block's S rows, in a new packed
    cache ([chathome] block-generation paragraph: once a block is done, the
    context tower takes in the committed tokens and its per-layer KV cache
    grows by them).

    k_ctx, v_ctx [T, Hkv, D] packed by ``offsets`` [B+1]; k_new, v_new
    [B, S, Hkv, D].  Returns (k_out, v_out, offsets_out) with sequence b at
    rows offsets_out[b] .. offsets_out[b+1] of k_out / v_out: its L_b old rows,
    then its S new ones."""
    offsets = np.asarray(offsets, dtype=np.int64)
    B, S = k_new.shape[0], k_new.shape[1]
    ks, vs = [], []
    offsets_out = np.zeros(B + 1, dtype=np.int64)
    for b in range(B):
        start, stop = int(offsets[b]), int(offsets[b + 1])
        ks.append(np.concatenate([k_ctx[start:stop], k_new[b]], axis=0))
        vs.append(np.concatenate([v_ctx[start:stop], v_new[b]], axis=0))
        offsets_out[b + 1] = offsets_out[b] + (stop - start) + S
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0), offsets_out


# ----------------------------------------------------------------------------
# Denoiser Mamba-2 layer over the block, its state seeded from the context
# tower ([chathome] inference paragraph: the denoiser's Mamba-2 layers start
# from the context tower's state; the layer itself is Mamba-2's selective
# state-space recurrence with one decay rate per head)
# ----------------------------------------------------------------------------
def mamba_block_scan(x, dt, A, Bm, Cm, D, h0):
    """The state-space core of one Mamba-2 layer over the block's S tokens,
    started from the context tower's final state.

    x  [B, S, H, P]   per-head inputs          dt [B, S, H]  step sizes (> 0)
    A  [H]            decay rates (< 0)        D  [H]        skip weights
    Bm, Cm [B, S, G, N]  input / output projections; head h reads group
                      h // (H / G)
    h0 [B, H, P, N]   seed state (the context tower's state after its tokens)
    For every sequence and head, token by token:
        h <- exp(dt_t * A) * h + dt_t * x_t (outer) B_t
        y_t = h C_t + D * x_t
    Returns (y [B, S, H, P], h_S [B, H, P, N]) in float64."""
    x = np.asarray(x, dtype=np.float64)
    dt = np.asarray(dt, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    Bm = np.asarray(Bm, dtype=np.float64)
    Cm = np.asarray(Cm, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    nb, S, H, P = x.shape
    G = Bm.shape[2]
    hs = np.array(h0, dtype=np.float64, copy=True)
    y = np.zeros((nb, S, H, P))
    for b in range(nb):
        for h in range(H):
            grp = h // (H // G)
            st = hs[b, h]
            for t in range(S):
                st = np.exp(dt[b, t, h] * A[h]) * st + dt[b, t, h] * np.outer(x[b, t, h], Bm[b, t, grp])
                y[b, t, h] = st @ Cm[b, t, grp] + D[h] * x[b, t, h]
            hs[b, h] = st
    return y, hs


def adaln_modulate(x, f, t_mod, tab_gate, tab_shift, tab_scale, w_norm, eps):
    """adaLN-single time conditioning between two denoiser layers ([chathome]
    inference paragraph: the diffusion timestep modulates every layer through
    adaLN-single, a module of about 1.5M parameters).

    Reading (the pages name the scheme only; this is adaLN-single as
    PixArt-alpha defines it): one shared projection of the timestep gives
    every sequence three vectors, shift / scale / gate (t_mod rows 0, 1, 2),
    and each layer adds its own learned [3, H] table to them.  Layer l's
    output f joins the residual stream through its gate; layer l + 1 then
    reads the RMS-normalised stream, scaled by (1 + its scale) and moved by
    its shift:
        r = x + (t_mod[b, 2] + tab_gate) * f              (f given)
        r = x                                             (f None)
        h = r / sqrt(mean_j r_j^2 + eps) * w_norm * (1 + t_mod[b, 1] + tab_scale)
              + (t_mod[b, 0] + tab_shift)
    x, f [B, S, H]; t_mod [B, 3, H]; tab_* and w_norm [H] (None: zero tables,
    unit weight).  Returns (r, h) in float64, unrounded."""
    x = np.asarray(x, dtype=np.float64)
    nb, S, H = x.shape
    t_mod = np.asarray(t_mod, dtype=np.float64)

    def row(v, fill):
        return np.full(H, fill) if v is None else np.asarray(v, dtype=np.float64)

    shift = t_mod[:, 0, :] + row(tab_shift, 0.0)         # [B, H]
    scale = t_mod[:, 1, :] + row(tab_scale, 0.0)
    gate = t_mod[:, 2, :] + row(tab_gate, 0.0)
    w = row(w_norm, 1.0)
    if f is None:
        r = x.copy()
    else:
        r = x + gate[:, None, :] * np.asarray(f, dtype=np.float64)
    rms = np.sqrt(np.mean(r * r, axis=2, keepdims=True) + eps)
    h = r / rms * w * (1.0 + scale[:, None, :]) + shift[:, None, :]
    return r, h

