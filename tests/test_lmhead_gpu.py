"""GPU parity of the fused LM head + commit (td_lmhead_commit, through the C
ABI) against the oracle's lmhead_commit.

The strict cases use the exact-arithmetic inputs of synth (hidden values on a
1/4 grid, head values on a 1/256 grid): every partial sum of the logits is
exactly representable in fp32, so the kernel's logits equal the oracle's
whatever the summation order, and the comparison is the commit's own (tokens
bit-exact; commit masks bit-exact except positions whose oracle maxprob lies
within 1e-4 of gamma, excluded and counted).  Shapes span several 256-row and
256-token tiles with ragged tails, hidden sizes of one to 64 pipeline
stages, and the full batched step (sampled sequences).  The realistic
(non-grid) inputs are checked with a band derived from fp32 accumulation:
see test_lmhead_realistic_sampled."""
import numpy as np
import pytest
import torch

import block_diffusion_lm_td_amd as td
import oracle
import synth
from gpu_util import compare_commit, dev, log

pytestmark = pytest.mark.gpu
LW = synth.LMHEAD_WORKLOADS


def _run(d, masked, gamma, tokens_in, packed=False):
    B, S, H = d["hidden"].shape
    hid = dev(d["hidden"], "bf16")
    wh = dev(d["w_head"], "bf16")
    if packed:
        wh = td.td_lmhead_pack_head(wh)
    o = dict(commit=torch.empty((B, S), dtype=torch.uint8, device="cuda"),
             token=torch.empty((B, S), dtype=torch.int32, device="cuda"),
             maxprob=torch.empty((B, S), dtype=torch.float32, device="cuda"),
             n_commit=torch.empty((B,), dtype=torch.int32, device="cuda"),
             masked_out=torch.empty((B, S), dtype=torch.uint8, device="cuda"),
             tokens=torch.from_numpy(np.ascontiguousarray(tokens_in, dtype=np.int32)).to("cuda"),
             n_masked_left=torch.full((1,), -7, dtype=torch.int32, device="cuda"))
    mi = None if masked is None else torch.from_numpy(np.ascontiguousarray(masked, np.uint8)).to("cuda")
    td.td_lmhead_commit(hid, wh, o["commit"], o["token"], gamma=gamma, masked_in=mi,
                        maxprob=o["maxprob"], n_commit=o["n_commit"], masked_out=o["masked_out"],
                        tokens=o["tokens"], n_masked_left=o["n_masked_left"])
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in o.items()}


def _ref(d, masked, gamma, seqs):
    h = synth.bf16_bits_to_f64(d["hidden"][list(seqs)])
    w = synth.bf16_bits_to_f64(d["w_head"])
    m = None if masked is None else masked[list(seqs)]
    return oracle.lmhead_commit(h, w, m, gamma)


def _case(w, seed, gamma, frac=1.0, seqs=None, label="", packed=False):
    d = synth.make_lmhead_inputs(w, seed)
    B, S = w.B, w.S
    if frac >= 1.0:
        masked = np.ones((B, S), np.uint8)
    else:
        masked = (np.random.default_rng([seed, 9]).random((B, S)) < frac).astype(np.uint8)
    tokens_in = np.where(masked.astype(bool), -1, 7)
    log(f"case lmhead {label or w.name}: B={B} S={S} H={w.H} V={w.V} gamma={gamma} frac={frac}")
    g = _run(d, masked, gamma, tokens_in, packed)
    seqs = list(range(B)) if seqs is None else list(seqs)
    ref = _ref(d, masked, gamma, seqs)
    # positions already committed are not scored: token -1, maxprob 0; the
    # oracle's values stand in for them in the commit comparison
    idle = ~masked.astype(bool)
    assert (g["token"][idle] == -1).all() and (g["maxprob"][idle] == 0).all(), "unscored positions"
    ri = idle[seqs]
    g["token"][seqs] = np.where(ri, ref["token"], g["token"][seqs])
    g["maxprob"][seqs] = np.where(ri, ref["maxprob"], g["maxprob"][seqs])
    return compare_commit(g, ref, masked, gamma, tokens_in, label or w.name, seqs)


@pytest.mark.parametrize("gamma,frac", [(0.8, 1.0), (0.5, 0.6), (1.5, 0.8), (1e-6, 1.0)])
def test_lmhead_exact_b4(gamma, frac):
    _case(LW["lmhead_exact_b4_h256_v5000"], 61, gamma, frac)


@pytest.mark.parametrize("B,S,H,V", [
    (20, 16, 192, 300),      # 320 rows: two position tiles, ragged; 3 stages
    (1, 16, 64, 256),        # one stage, exactly one token tile
    (3, 64, 128, 1),         # a one-token vocabulary
    (2, 1, 64, 7),           # S = 1, tiny vocabulary
    (9, 32, 512, 2049),      # 288 rows, 9 token tiles (one token in the last)
    (16, 16, 4096, 1000),    # the widest exact hidden size
    (24, 16, 256, 3000),     # ~288 rows: three 128-position tiles, ragged
])
def test_lmhead_exact_shapes(B, S, H, V):
    w = LW["lmhead_exact_b4_h256_v5000"].with_(B=B, S=S, H=H, V=V)
    _case(w, 62 + B + H, 0.8, 0.75, label=f"exact B{B} S{S} H{H} V{V}")


@pytest.mark.parametrize("frac", [0.0, 0.02, 0.3])
def test_lmhead_exact_few_positions_left(frac):
    """Late steps of a block: few positions still masked (none, one or two
    per sequence, about a third), so only a part of the first position tile
    or none of it is scored."""
    w = LW["lmhead_exact_b4_h256_v5000"].with_(B=24)
    _case(w, 66, 0.8, max(frac, 1e-9), label=f"exact few left frac={frac}")


def test_lmhead_exact_full_step_sampled():
    """The batched step's 64 x 16 positions through a 4096 x 131072 head, on
    the exact grids; whole sequences sampled for the oracle."""
    w = LW["lmhead_bf16_b64_h4096_v131072"].with_(exact=True)
    _case(w, 63, 0.8, 1.0, seqs=[0, 17, 40, 63], label="exact b64 h4096 v131072 (4 sequences)")


def test_lmhead_deterministic():
    w = LW["lmhead_exact_b4_h256_v5000"].with_(B=8, V=20000, H=1024)
    d = synth.make_lmhead_inputs(w, 64)
    log("case lmhead deterministic")
    a = _run(d, None, 0.8, np.full((8, 16), -1))
    b = _run(d, None, 0.8, np.full((8, 16), -1))
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_lmhead_realistic_sampled():
    """Realistic (off-grid) bf16 inputs of the full step.  The kernel's fp32
    logits then differ from the oracle's fp64 ones by at most
    E_m = (H + H/16) * 2^-24 * max_j sum_k |h_mk w_jk| (one rounding per
    product-sum step of the accumulation chain, products exact).  So the
    argmax must match wherever the oracle's top two logits are more than 2 E_m
    apart, and maxprob, whose logit differences move by at most 2 E_m, must
    agree within p (e^(2 E_m) - 1) + 2e-5.  Positions closer than that to a
    tie are counted, not compared."""
    w = LW["lmhead_bf16_b64_h4096_v131072"]
    d = synth.make_lmhead_inputs(w, 65)
    log("case lmhead realistic b64 h4096 v131072, 3 sequences")
    g = _run(d, None, 0.8, np.full((w.B, w.S), -1))
    seqs = [1, 30, 62]
    h = synth.bf16_bits_to_f64(d["hidden"][seqs]).reshape(-1, w.H)
    wf = synth.bf16_bits_to_f64(d["w_head"])
    logits = h @ wf.T
    E = (w.H + w.H / 16) * 2.0 ** -24 * (np.abs(h) @ np.abs(wf).T).max(axis=1)
    ref = oracle.confidence_commit(logits.reshape(len(seqs), w.S, w.V), None, 0.8)
    top2 = np.sort(logits, axis=1)[:, -2:]
    gap = top2[:, 1] - top2[:, 0]
    sure = gap > 2 * E
    gt = g["token"][seqs].reshape(-1)
    rt = ref["token"].reshape(-1)
    assert (gt[sure] == rt[sure]).all(), "argmax differs away from a tie"
    p = ref["maxprob"].reshape(-1)
    tol = p * np.expm1(2 * E) + 2e-5
    assert (np.abs(g["maxprob"][seqs].reshape(-1) - p) <= tol).all(), "maxprob outside the bound"
    log(f"[lmhead] realistic: E_m median {np.median(E):.2e}, max {E.max():.2e}; "
        f"positions near a tie {int((~sure).sum())} of {len(sure)}")


def _packed_ref(w, V, H):
    """The packed order written with plain reshapes: rows padded with zeros to
    a multiple of 256, then [V/256][256][H/64][64] -> [V/256][H/64][256][64]."""
    nt = (V + 255) // 256
    p = torch.zeros((nt * 256, H), dtype=w.dtype, device=w.device)
    p[:V] = w
    return p.reshape(nt, 256, H // 64, 64).permute(0, 2, 1, 3).contiguous().reshape(-1)


@pytest.mark.parametrize("V,H", [(1, 64), (255, 128), (256, 64), (257, 64), (2049, 512), (5000, 256),
                                 (131072, 4096)])
def test_lmhead_pack_head_layout(V, H):
    """Every bit of the packed copy, for arbitrary bit patterns (NaN and
    infinity payloads included)."""
    log(f"case lmhead pack V={V} H={H}")
    g = torch.Generator(device="cuda").manual_seed(V + H)
    bits = torch.randint(-32768, 32768, (V, H), dtype=torch.int32, device="cuda", generator=g)
    w = bits.to(torch.int16).view(torch.bfloat16)
    p = td.td_lmhead_pack_head(w)
    assert (p.V, p.H) == (V, H)
    assert torch.equal(p.data.view(torch.int16), _packed_ref(w, V, H).view(torch.int16))


@pytest.mark.parametrize("B,S,H,V", [
    (20, 16, 192, 300), (1, 16, 64, 256), (3, 64, 128, 1), (2, 1, 64, 7), (9, 32, 512, 2049),
])
def test_lmhead_packed_exact_shapes(B, S, H, V):
    """The packed head against the oracle on the exact grids."""
    w = LW["lmhead_exact_b4_h256_v5000"].with_(B=B, S=S, H=H, V=V)
    _case(w, 62 + B + H, 0.8, 0.75, label=f"packed exact B{B} S{S} H{H} V{V}", packed=True)


@pytest.mark.parametrize("frac", [1.0, 0.3, 0.1])
def test_lmhead_packed_equals_row_major_full_step(frac):
    """The batched step's 4096 x 131072 head, realistic values: the packed
    head gives the row-major head's outputs bit for bit (same products, same
    order).  At 0.1 about 100 positions are left: the late-step tiles."""
    w = LW["lmhead_bf16_b64_h4096_v131072"]
    d = synth.make_lmhead_inputs(w, 67)
    masked = (np.random.default_rng(68).random((w.B, w.S)) < frac).astype(np.uint8)
    tokens_in = np.where(masked.astype(bool), -1, 7)
    log(f"case lmhead packed vs row-major b64 h4096 v131072 frac={frac}")
    a = _run(d, masked, 0.8, tokens_in)
    b = _run(d, masked, 0.8, tokens_in, packed=True)
    for k in a:
        assert np.array_equal(a[k], b[k]), k

