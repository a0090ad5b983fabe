"""Mutation check of the pins: each plausible one-token mistake planted in a
copy of the oracle's source (on the CPU, never in the GPU path) must make at
least one pin fail.  The real oracle passes all of them (test_oracle.py)."""
import inspect
import types

import pytest

import oracle.td_oracle as real
import pins

SRC = inspect.getsource(real)

MUTANTS = [
    ("gqa_modulo", "g = h // G", "g = h % Hkv"),
    ("drop_block_keys", "k_blk[b, :, g, :]], axis=0)", "k_blk[b, :0, g, :]], axis=0)"),
    ("drop_block_values", "v_blk[b, :, g, :]], axis=0)", "v_blk[b, :0, g, :]], axis=0)"),
    ("drop_context", "k_ctx[lo:hi, g, :]", "k_ctx[lo:lo, g, :]"),
    ("offset_off_by_one", "lo, hi = int(offsets[b]), int(offsets[b + 1])",
     "lo, hi = int(offsets[b]) + 1, int(offsets[b + 1])"),
    ("scale_1_over_D", "scale = 1.0 / np.sqrt(D)", "scale = 1.0 / D"),
    ("softmax_wrong_axis", "s = s - s.max(axis=1, keepdims=True)", "s = s - s.max(axis=0, keepdims=True)"),
    ("normalise_wrong_axis", "p /= p.sum(axis=1, keepdims=True)", "p /= p.sum(axis=0, keepdims=True)"),
    ("pv_uses_keys", "out[b, :, h, :] = p @ V", "out[b, :, h, :] = p @ K"),
    ("no_scale_applied", "s = scale * (q[b, :, h, :] @ K.T)", "s = (q[b, :, h, :] @ K.T)"),
    ("argmax_last", "token = x.argmax(axis=-1).astype(np.int64)",
     "token = (x.shape[-1] - 1 - x[..., ::-1].argmax(axis=-1)).astype(np.int64)"),
    ("no_max_shift", "z = np.exp(x - m[..., None]).sum(axis=-1)\n    return 1.0 / z, token",
     "z = np.exp(x).sum(axis=-1)\n    return np.exp(m) / z, token"),
    ("strict_threshold", "commit = elig & (p >= g)", "commit = elig & (p > g)"),
    ("gamma_f64", "g = float(np.float32(gamma))", "g = float(gamma)"),
    ("no_force_one", "if not commit[b].any() and elig[b].any():", "if False:"),
    ("force_one_ignores_eligibility", "cand = np.where(elig[b], p[b], -np.inf)", "cand = p[b]"),
    ("force_one_last_tie", "commit[b, int(np.argmax(cand))] = True",
     "commit[b, len(cand) - 1 - int(np.argmax(cand[::-1]))] = True"),
    ("threshold_ignores_eligibility", "commit = elig & (p >= g)", "commit = (p >= g)"),
    ("step_remasks", "masked_out = np.asarray(masked_in).astype(bool) & ~c[\"commit\"]",
     "masked_out = ~c[\"commit\"]"),
    ("step_writes_all_tokens", "tokens[c[\"commit\"]] = c[\"token\"][c[\"commit\"]]\n    return dict(out=out",
     "tokens[:] = c[\"token\"]\n    return dict(out=out"),
    ("loop_remasks", "masked &= ~c[\"commit\"]", "masked = ~c[\"commit\"]"),
    ("append_new_rows_first", "np.concatenate([k_ctx[start:stop], k_new[b]], axis=0)",
     "np.concatenate([k_new[b], k_ctx[start:stop]], axis=0)"),
    ("append_values_from_keys", "np.concatenate([v_ctx[start:stop], v_new[b]], axis=0)",
     "np.concatenate([v_ctx[start:stop], k_new[b]], axis=0)"),
    ("append_offsets_without_block", "offsets_out[b] + (stop - start) + S",
     "offsets_out[b] + (stop - start)"),
    ("append_drops_last_old_row", "k_ctx[start:stop], k_new[b]", "k_ctx[start:stop - 1], k_new[b]"),
    ("append_neighbours_rows", "k_ctx[start:stop], k_new[b]]", "k_ctx[start:stop], k_new[b - 1]]"),
    ("lmhead_vocab_reversed", "(h.reshape(B * S, H) @ w.T)", "(h.reshape(B * S, H) @ w[::-1].T)"),
    ("lmhead_negated", "(h.reshape(B * S, H) @ w.T)", "(h.reshape(B * S, H) @ -w.T)"),
    ("lmhead_rows_transposed", "(h.reshape(B * S, H) @ w.T)",
     "(h.transpose(1, 0, 2).reshape(B * S, H) @ w.T)"),
    ("lmhead_drops_eligibility", "confidence_commit(lmhead_logits(hidden, w_head), masked_in, gamma)",
     "confidence_commit(lmhead_logits(hidden, w_head), None, gamma)"),
    ("lmhead_last_hidden_unit_dropped", "(h.reshape(B * S, H) @ w.T)",
     "(h[..., :-1].reshape(B * S, H - 1) @ w[:, :-1].T)"),
    ("mamba_decay_after_update", "st = np.exp(dt[b, t, h] * A[h]) * st + dt[b, t, h] * np.outer(x[b, t, h], Bm[b, t, grp])",
     "st = np.exp(dt[b, t, h] * A[h]) * (st + dt[b, t, h] * np.outer(x[b, t, h], Bm[b, t, grp]))"),
    ("mamba_input_without_step", "+ dt[b, t, h] * np.outer(x[b, t, h], Bm[b, t, grp])",
     "+ np.outer(x[b, t, h], Bm[b, t, grp])"),
    ("mamba_group_modulo", "grp = h // (H // G)", "grp = h % G"),
    ("mamba_output_from_seed", "y[b, t, h] = st @ Cm[b, t, grp]", "y[b, t, h] = hs[b, h] @ Cm[b, t, grp]"),
    ("mamba_no_skip", "y[b, t, h] = st @ Cm[b, t, grp] + D[h] * x[b, t, h]", "y[b, t, h] = st @ Cm[b, t, grp]"),
    ("mamba_b_for_c", "np.outer(x[b, t, h], Bm[b, t, grp])", "np.outer(x[b, t, h], Cm[b, t, grp])"),
    ("adaln_layernorm", "rms = np.sqrt(np.mean(r * r, axis=2, keepdims=True) + eps)",
     "rms = np.sqrt(np.var(r, axis=2, keepdims=True) + eps)"),
    ("adaln_scale_without_one", "* w * (1.0 + scale[:, None, :])", "* w * scale[:, None, :]"),
    ("adaln_eps_outside_sqrt", "np.sqrt(np.mean(r * r, axis=2, keepdims=True) + eps)",
     "np.sqrt(np.mean(r * r, axis=2, keepdims=True)) + eps"),
    ("adaln_gate_from_scale_row", "gate = t_mod[:, 2, :]", "gate = t_mod[:, 1, :]"),
    ("adaln_table_ignored", "shift = t_mod[:, 0, :] + row(tab_shift, 0.0)", "shift = t_mod[:, 0, :]"),
    ("adaln_norm_of_x", "rms = np.sqrt(np.mean(r * r, axis=2", "rms = np.sqrt(np.mean(x * x, axis=2"),
    ("adaln_norm_over_tokens", "np.mean(r * r, axis=2, keepdims=True)", "np.mean(r * r, axis=(1, 2), keepdims=True)"),
    ("step_swaps_block_kv", 'out = block_attention(a["q"], a["k_blk"], a["v_blk"], a["k_ctx"], a["v_ctx"],',
     'out = block_attention(a["q"], a["v_blk"], a["k_blk"], a["k_ctx"], a["v_ctx"],'),
    ("step_swaps_context_kv", 'out = block_attention(a["q"], a["k_blk"], a["v_blk"], a["k_ctx"], a["v_ctx"],',
     'out = block_attention(a["q"], a["k_blk"], a["v_blk"], a["v_ctx"], a["k_ctx"],'),
    ("step_drops_scale", '                          a["offsets"], scale)\n    c = confidence_commit',
     '                          a["offsets"], None)\n    c = confidence_commit'),
    ("append_new_rows_truncated", "k_ctx[start:stop], k_new[b]]", "k_ctx[start:stop], k_new[b, 1:]]"),
]


def _load_mutant(old, new):
    assert SRC.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = SRC.replace(old, new, 1)
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__["__name__"] = "oracle_mutant"
    exec(compile(src, "<oracle_mutant>", "exec"), mod.__dict__)
    return mod


def _all_pins(mod):
    yield from ((p, mod.block_attention) for p in pins.ATTN_PINS)
    yield from ((p, mod.row_confidence) for p in pins.CONF_PINS)
    yield from ((p, mod.confidence_commit) for p in pins.COMMIT_PINS)
    yield from ((p, mod.denoise_loop) for p in pins.LOOP_PINS)
    yield from ((p, mod.denoise_step) for p in pins.STEP_PINS)
    yield from ((p, mod.cache_append) for p in pins.APPEND_PINS)
    yield from ((p, mod.lmhead_logits) for p in pins.LMHEAD_LOGIT_PINS)
    yield from ((p, mod.lmhead_commit) for p in pins.LMHEAD_PINS)
    yield from ((p, mod.mamba_block_scan) for p in pins.MAMBA_PINS)
    yield from ((p, mod.adaln_modulate) for p in pins.ADALN_PINS)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    mod = _load_mutant(old, new)
    caught = []
    import warnings
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        for pin, fn in _all_pins(mod):
            try:
                pin(fn)
            except Exception as e:          # AssertionError, or a crash the mistake causes
                caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutant {name} passed every pin"
