"""Workload shapes and seeded input generators for the denoise step.

Shapes follow the pages' operating point where they give one: block size
S = 16 and confidence threshold gamma = 0.8 (news.chathome.org, "NVIDIA
releases Nemotron-Labs-TwoTower ...", evaluation paragraph; aikraft.ru,
benchmark-results section).  Batch sizes, head counts, head dim, context
lengths and vocabulary size are not on the pages; the values below are
assumed workloads of realistic shape (32 query heads over 2 KV heads, head
dim 128, a 131072-entry vocabulary).

Draw order inside one generator call is fixed (lengths, Q, block K, block V,
context K, context V, logit noise, peak ids, margins), so a (workload, seed)
pair names one exact input set.  Floating values are drawn in float32; bf16
workloads are stored as uint16 bit patterns obtained with round-to-nearest-
even.  Nothing here computes attention or a commit.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S: int
    Hq: int
    Hkv: int
    D: int
    ctx_lo: int          # context length range, inclusive; lo == hi = uniform
    ctx_hi: int
    dtype: str           # "f32" or "bf16": storage dtype of Q/K/V and logits
    qkv_std: float       # std of Q and of the block's K/V
    ctx_std: float       # std of the context K/V cache
    V: int               # vocabulary size
    logit_model: str     # "boost": N(0, logit_std) + U(0, margin_hi) on one id
                         # "peak":  one id = max(others) + U(0, margin_hi)
    logit_std: float
    margin_hi: float
    gamma: float
    step_margin_hi: float = 0.0   # per-step margin growth of the block loop

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


_INV_SQRT128 = float(1.0 / np.sqrt(128.0))

WORKLOADS: dict[str, Workload] = {
    # Tiny fp32 step that the oracle finishes instantly.
    "tiny_f32_b1_ctx64": Workload(
        "tiny_f32_b1_ctx64", B=1, S=16, Hq=4, Hkv=1, D=64, ctx_lo=64, ctx_hi=64,
        dtype="f32", qkv_std=1.0, ctx_std=1.0, V=1000, logit_model="boost",
        logit_std=1.0, margin_hi=8.0, gamma=0.8),
    # One realistic attention layer, 8 sequences of 4K context.
    "bf16_b8_ctx4k": Workload(
        "bf16_b8_ctx4k", B=8, S=16, Hq=32, Hkv=2, D=128, ctx_lo=4096, ctx_hi=4096,
        dtype="bf16", qkv_std=_INV_SQRT128, ctx_std=_INV_SQRT128, V=131072,
        logit_model="peak", logit_std=2.0, margin_hi=12.0, gamma=0.8),
    # Batched step: 64 sequences, ragged context lengths uniform in [1K, 8K].
    "bf16_b64_ragged1k_8k": Workload(
        "bf16_b64_ragged1k_8k", B=64, S=16, Hq=32, Hkv=2, D=128, ctx_lo=1024,
        ctx_hi=8192, dtype="bf16", qkv_std=_INV_SQRT128, ctx_std=_INV_SQRT128,
        V=131072, logit_model="peak", logit_std=2.0, margin_hi=12.0, gamma=0.8),
    # Same batch, every context exactly 8K.
    "bf16_b64_ctx8k": Workload(
        "bf16_b64_ctx8k", B=64, S=16, Hq=32, Hkv=2, D=128, ctx_lo=8192,
        ctx_hi=8192, dtype="bf16", qkv_std=_INV_SQRT128, ctx_std=_INV_SQRT128,
        V=131072, logit_model="peak", logit_std=2.0, margin_hi=12.0, gamma=0.8),
    # Long context: 4 sequences of 64K context, unit-variance K/V.
    "bf16_b4_ctx64k": Workload(
        "bf16_b4_ctx64k", B=4, S=16, Hq=32, Hkv=2, D=128, ctx_lo=65536,
        ctx_hi=65536, dtype="bf16", qkv_std=1.0, ctx_std=1.0, V=131072,
        logit_model="peak", logit_std=2.0, margin_hi=12.0, gamma=0.8),
    # One-token decode (S = 1, the AR / mock-AR modes) on the batched cache.
    "bf16_b64_ragged1k_8k_s1": Workload(
        "bf16_b64_ragged1k_8k_s1", B=64, S=1, Hq=32, Hkv=2, D=128, ctx_lo=1024,
        ctx_hi=8192, dtype="bf16", qkv_std=_INV_SQRT128, ctx_std=_INV_SQRT128,
        V=131072, logit_model="peak", logit_std=2.0, margin_hi=12.0, gamma=0.8),
    # Whole-block loop: 32 sequences of 2K context; S and gamma are swept.
    "bf16_b32_ctx2k_loop": Workload(
        "bf16_b32_ctx2k_loop", B=32, S=16, Hq=32, Hkv=2, D=128, ctx_lo=2048,
        ctx_hi=2048, dtype="bf16", qkv_std=_INV_SQRT128, ctx_std=_INV_SQRT128,
        V=131072, logit_model="peak", logit_std=2.0, margin_hi=12.0, gamma=0.8,
        step_margin_hi=3.0),
}


# ----------------------------------------------------------------------------
# bf16 storage cast (round to nearest even) and exact upcasts
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round-to-nearest-even. Finite inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(h: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(h).astype(np.float64)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


def _normal(rng, shape, std) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


# ----------------------------------------------------------------------------
# Attention inputs
# ----------------------------------------------------------------------------
def make_attention_inputs(w: Workload, seed: int, lengths=None) -> dict:
    """Q [B,S,Hq,D], block K/V [B,S,Hkv,D], packed context K/V [T,Hkv,D],
    offsets int64 [B+1].  Storage dtype per ``w.dtype`` (bf16 as uint16 bits).

    ``lengths`` overrides the drawn context lengths (edge cases: zeros, ragged).
    """
    rng = np.random.default_rng(seed)
    if lengths is None:
        if w.ctx_lo == w.ctx_hi:
            lengths = np.full(w.B, w.ctx_lo, dtype=np.int64)
        else:
            lengths = rng.integers(w.ctx_lo, w.ctx_hi, endpoint=True, size=w.B).astype(np.int64)
    lengths = np.asarray(lengths, dtype=np.int64)
    assert lengths.shape == (w.B,) and (lengths >= 0).all()
    offsets = np.zeros(w.B + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(lengths)
    T = int(offsets[-1])
    q = _normal(rng, (w.B, w.S, w.Hq, w.D), w.qkv_std)
    kb = _normal(rng, (w.B, w.S, w.Hkv, w.D), w.qkv_std)
    vb = _normal(rng, (w.B, w.S, w.Hkv, w.D), w.qkv_std)
    kc = _normal(rng, (T, w.Hkv, w.D), w.ctx_std)
    vc = _normal(rng, (T, w.Hkv, w.D), w.ctx_std)
    return dict(
        q=_store(q, w.dtype), k_blk=_store(kb, w.dtype), v_blk=_store(vb, w.dtype),
        k_ctx=_store(kc, w.dtype), v_ctx=_store(vc, w.dtype),
        offsets=offsets, lengths=lengths, total_ctx=T,
        max_ctx=int(lengths.max()) if w.B else 0, dtype=w.dtype,
    )


# ----------------------------------------------------------------------------
# Commit inputs (vocabulary logits of the block)
# ----------------------------------------------------------------------------
def _logit_noise(rng, w: Workload, rows: int):
    x = _normal(rng, (rows, w.V), w.logit_std)
    peak = rng.integers(0, w.V, size=rows)
    margin = rng.uniform(0.0, w.margin_hi, size=rows).astype(np.float32)
    return x, peak, margin


def _place_peaks(x: np.ndarray, peak: np.ndarray, margin: np.ndarray, model: str) -> None:
    r = np.arange(x.shape[0])
    if model == "boost":
        x[r, peak] += margin
    elif model == "peak":
        x[r, peak] = -np.inf
        others = x.max(axis=1)
        x[r, peak] = others + margin
    else:
        raise ValueError(model)


def make_commit_inputs(w: Workload, seed: int, rows_only: int | None = None) -> dict:
    """logits [B,S,V] (storage dtype per ``w.dtype``), plus the peak ids and
    margins used to build them.  ``seed`` is offset from the attention seed so
    both draws stay independent."""
    rng = np.random.default_rng([seed, 1])
    rows = w.B * w.S if rows_only is None else rows_only
    x, peak, margin = _logit_noise(rng, w, rows)
    _place_peaks(x, peak, margin, w.logit_model)
    shape = (w.B, w.S, w.V) if rows_only is None else (rows, w.V)
    return dict(logits=_store(x, w.dtype).reshape(shape), peak=peak, margin=margin,
                dtype=w.dtype)


def make_eligible(w: Workload, seed: int, frac: float = 1.0) -> np.ndarray:
    """uint8 [B,S]: 1 = position still [MASK].  ``frac`` < 1 masks a random subset."""
    if frac >= 1.0:
        return np.ones((w.B, w.S), dtype=np.uint8)
    rng = np.random.default_rng([seed, 2])
    return (rng.random((w.B, w.S)) < frac).astype(np.uint8)


# ----------------------------------------------------------------------------
# Block loop: per-step logits whose peak margin grows by U(0, step_margin_hi)
# ----------------------------------------------------------------------------
def loop_peak_values(w: Workload, seed: int, steps: int):
    """Base logits (bf16 bits or f32, [B*S, V]) at step 0, the peak ids, and a
    [steps, B*S] array with the stored value of each peak logit at each step.

    Only the peak logit changes from step to step: its margin above the other
    logits of its row starts at U(0, margin_hi) and grows by a fresh
    U(0, step_margin_hi) draw every step.
    """
    rng = np.random.default_rng([seed, 1])
    rows = w.B * w.S
    x, peak, margin0 = _logit_noise(rng, w, rows)
    r = np.arange(rows)
    x[r, peak] = -np.inf
    others = x.max(axis=1)
    vals = np.empty((steps, rows), dtype=np.float32)
    margin = margin0.copy()
    for t in range(steps):
        if t > 0:
            inc = np.random.default_rng([seed, 3, t]).uniform(0.0, w.step_margin_hi, size=rows)
            margin = margin + inc.astype(np.float32)
        vals[t] = others + margin
    x[r, peak] = vals[0]
    base = _store(x, w.dtype)
    stored = _store(vals, w.dtype)
    return base, peak, stored


def loop_step_logits(base: np.ndarray, peak: np.ndarray, stored: np.ndarray, t: int) -> np.ndarray:
    """Logits of step ``t`` as stored values [B*S, V] (a copy of ``base`` with
    the peak entries of step ``t``)."""
    x = base.copy()
    x[np.arange(x.shape[0]), peak] = stored[t]
    return x


# ----------------------------------------------------------------------------
# LM head of the block positions: hidden states and head weights
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class LMHeadWorkload:
    name: str
    B: int
    S: int
    H: int               # hidden size (not on the pages: assumed)
    V: int               # vocabulary size
    logit_std: float     # std of the background logits h . w_j (hidden part ~ N(0, 1))
    margin_hi: float     # planted peak: expected background max + U(0, margin_hi)
    gamma: float
    exact: bool = False  # values on grids that make every fp32 partial sum exact

    def with_(self, **kw) -> "LMHeadWorkload":
        return dataclasses.replace(self, **kw)


LMHEAD_WORKLOADS: dict[str, LMHeadWorkload] = {
    # Small enough for the oracle on every row: ragged vocabulary and rows.
    "lmhead_bf16_b4_h256_v5000": LMHeadWorkload(
        "lmhead_bf16_b4_h256_v5000", B=4, S=16, H=256, V=5000, logit_std=2.0,
        margin_hi=12.0, gamma=0.8),
    # The same with exactly representable sums (see make_lmhead_inputs).
    "lmhead_exact_b4_h256_v5000": LMHeadWorkload(
        "lmhead_exact_b4_h256_v5000", B=4, S=16, H=256, V=5000, logit_std=2.0,
        margin_hi=12.0, gamma=0.8, exact=True),
    # The batched step's positions (64 blocks of 16) through a 4096-wide head
    # over the 131072-entry vocabulary.
    "lmhead_bf16_b64_h4096_v131072": LMHeadWorkload(
        "lmhead_bf16_b64_h4096_v131072", B=64, S=16, H=4096, V=131072, logit_std=2.0,
        margin_hi=12.0, gamma=0.8),
}


def _expected_max_normal(n: int) -> float:
    """E[max of n standard normals] (the usual asymptotic expansion; 0 for n < 2)."""
    if n < 2:
        return 0.0
    a = np.sqrt(2.0 * np.log(n))
    return float(a - (np.log(np.log(n)) + np.log(4.0 * np.pi)) / (2.0 * a))


def make_lmhead_inputs(w: LMHeadWorkload, seed: int) -> dict:
    """hidden [B,S,H] and w_head [V,H] as bf16 bits (uint16).

    w_head ~ N(0, sw^2) with sw = logit_std / sqrt(H), so a random hidden
    state h ~ N(0, 1) has background logits of std ~logit_std.  Each position
    gets a planted peak: h = g + c * w_head[t] with a uniform token t and
    c = (E[max background] + U(0, margin_hi)) / (H sw^2), which lifts token t's
    logit by about that much above the expected maximum of the others
    (|w_head[t]|^2 is H sw^2 on average).  Draw order: head, noise, peak ids,
    margins.

    ``exact``: hidden values are rounded to multiples of 1/4 in [-8, 8] and
    head values to multiples of 1/256 in [-1/8, 1/8].  Every product is then a
    multiple of 2^-10 of magnitude <= 1, so every partial sum of up to 4096
    products is a multiple of 2^-10 below 2^12 in magnitude: 22 significant
    bits, exact in float32 in any summation order.
    """
    rng = np.random.default_rng([seed, 7])
    sw = w.logit_std / np.sqrt(w.H)
    head = _normal(rng, (w.V, w.H), sw)
    rows = w.B * w.S
    g = _normal(rng, (rows, w.H), 1.0)
    peak = rng.integers(0, w.V, size=rows)
    margin = rng.uniform(0.0, w.margin_hi, size=rows).astype(np.float32)
    lift = np.float32(w.logit_std * _expected_max_normal(w.V)) + margin
    c = (lift / np.float32(w.H * sw * sw)).astype(np.float32)
    g += c[:, None] * head[peak]
    if w.exact:
        assert w.H <= 4096
        head = np.clip(np.rint(head * 256.0), -32.0, 32.0).astype(np.float32) / np.float32(256.0)
        g = np.clip(np.rint(g * 4.0), -32.0, 32.0).astype(np.float32) / np.float32(4.0)
    return dict(hidden=f32_to_bf16_bits(g).reshape(w.B, w.S, w.H),
                w_head=f32_to_bf16_bits(head), peak=peak, margin=margin, dtype="bf16")


# ----------------------------------------------------------------------------
# Denoiser Mamba-2 layer: the block's SSM inputs and the seed state
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class MambaWorkload:
    name: str
    B: int
    S: int
    H: int               # SSM heads
    P: int               # head dim
    N: int               # state size
    G: int               # groups of B / C projections

    def with_(self, **kw) -> "MambaWorkload":
        return dataclasses.replace(self, **kw)


# The pages give no Mamba-2 dimensions; these follow Mamba-2 layers of that
# model size (128 heads of 64 with a 128-wide state in 8 groups).
MAMBA_WORKLOADS: dict[str, MambaWorkload] = {
    "mamba_b4_s16_h8": MambaWorkload("mamba_b4_s16_h8", B=4, S=16, H=8, P=64, N=128, G=2),
    "mamba_b64_s16_h128": MambaWorkload("mamba_b64_s16_h128", B=64, S=16, H=128, P=64, N=128, G=8),
}


def make_mamba_inputs(w: MambaWorkload, seed: int) -> dict:
    """x [B,S,H,P], Bm / Cm [B,S,G,N] as bf16 bits; dt [B,S,H], A [H], D [H]
    and the seed state h0 [B,H,P,N] in float32.  Ranges follow Mamba-2's
    usual initialisation: dt log-uniform in [1e-3, 1e-1], A = -exp(U(0,
    ln 16)), D near 1; x, B, C, h0 standard normal.  Draw order: x, dt, A,
    B, C, D, h0."""
    rng = np.random.default_rng([seed, 13])
    x = _normal(rng, (w.B, w.S, w.H, w.P), 1.0)
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), (w.B, w.S, w.H))).astype(np.float32)
    A = (-np.exp(rng.uniform(0.0, np.log(16.0), w.H))).astype(np.float32)
    Bm = _normal(rng, (w.B, w.S, w.G, w.N), 1.0)
    Cm = _normal(rng, (w.B, w.S, w.G, w.N), 1.0)
    D = rng.uniform(0.5, 1.5, w.H).astype(np.float32)
    h0 = _normal(rng, (w.B, w.H, w.P, w.N), 1.0)
    return dict(x=f32_to_bf16_bits(x), dt=dt, A=A, Bm=f32_to_bf16_bits(Bm), Cm=f32_to_bf16_bits(Cm),
                D=D, h0=h0)



# ----------------------------------------------------------------------------
# adaLN-single modulation inputs
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class AdalnWorkload:
    name: str
    B: int
    S: int
    H: int               # hidden size
    exact: bool = False  # grid values: the gated sum is exact in fp32

    def with_(self, **kw) -> "AdalnWorkload":
        return dataclasses.replace(self, **kw)


# Hidden size 4096 is assumed (the pages give none), as for the LM head.
ADALN_WORKLOADS: dict[str, AdalnWorkload] = {
    "adaln_b4_s16_h256": AdalnWorkload("adaln_b4_s16_h256", B=4, S=16, H=256),
    "adaln_exact_b4_s16_h256": AdalnWorkload("adaln_exact_b4_s16_h256", B=4, S=16, H=256, exact=True),
    "adaln_b64_s16_h4096": AdalnWorkload("adaln_b64_s16_h4096", B=64, S=16, H=4096),
}


def make_adaln_inputs(w: AdalnWorkload, seed: int) -> dict:
    """x, f [B,S,H] as bf16 bits; t_mod [B,3,H] (shift, scale, gate),
    tab_gate / tab_shift / tab_scale and w_norm [H] in float32.  Realistic
    draws: x N(0, 2^2) (the residual stream), f N(0,1), t_mod N(0, 0.3^2),
    tables N(0, 0.1^2), w_norm U(0.5, 1.5).  Exact draws: x and f on the 1/64
    grid in (-4, 4), the gate rows of t_mod and the table on the 1/32 grid in
    [-1, 1], so that x + gate * f is exact in fp32.  Draw order: x, f, t_mod,
    tab_gate, tab_shift, tab_scale, w_norm."""
    rng = np.random.default_rng([seed, 17])
    B, S, H = w.B, w.S, w.H
    if w.exact:
        x = rng.integers(-255, 256, (B, S, H)).astype(np.float32) / 64
        f = rng.integers(-255, 256, (B, S, H)).astype(np.float32) / 64
        t_mod = _normal(rng, (B, 3, H), 0.3)
        t_mod[:, 2, :] = rng.integers(-32, 33, (B, H)).astype(np.float32) / 32
        tab_gate = rng.integers(-32, 33, H).astype(np.float32) / 32
    else:
        x = _normal(rng, (B, S, H), 2.0)
        f = _normal(rng, (B, S, H), 1.0)
        t_mod = _normal(rng, (B, 3, H), 0.3)
        tab_gate = _normal(rng, H, 0.1)
    tab_shift = _normal(rng, H, 0.1)
    tab_scale = _normal(rng, H, 0.1)
    w_norm = rng.uniform(0.5, 1.5, H).astype(np.float32)
    return dict(x=f32_to_bf16_bits(x), f=f32_to_bf16_bits(f), t_mod=t_mod, tab_gate=tab_gate,
                tab_shift=tab_shift, tab_scale=tab_scale, w_norm=w_norm)
