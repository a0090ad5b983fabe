"""C-ABI checks that need no GPU: libtd.so loads, exports every function
include/td.h declares, its structs match the binding, and invalid arguments
are rejected on the host before anything is enqueued (no compute calls)."""
import ctypes
import os

import pytest

import block_diffusion_lm_td_amd as td
from block_diffusion_lm_td_amd import _td

INVALID, UNSUPPORTED, WORKSPACE = _td.TD_ERR_INVALID, _td.TD_ERR_UNSUPPORTED, _td.TD_ERR_WORKSPACE
OK = _td.TD_OK
FAKE = 0x10000          # a non-null pointer value; never dereferenced on these paths


@pytest.fixture(scope="module")
def L():
    return td.lib()


def test_exports_every_declared_function(L):
    names = _td.header_functions()
    assert len(names) >= 10
    raw = ctypes.CDLL(_td.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), f"libtd.so does not export {n}"


def test_struct_layout_and_version(L):
    assert L.td_abi_version() == 2
    assert L.td_sizeof_attn_args() == ctypes.sizeof(_td.TdAttnArgs)
    assert L.td_sizeof_commit_args() == ctypes.sizeof(_td.TdCommitArgs)
    assert L.td_sizeof_append_args() == ctypes.sizeof(_td.TdAppendArgs)
    assert L.td_sizeof_lmhead_args() == ctypes.sizeof(_td.TdLmheadArgs)
    assert L.td_sizeof_mamba_args() == ctypes.sizeof(_td.TdMambaArgs)
    assert L.td_sizeof_adaln_args() == ctypes.sizeof(_td.TdAdalnArgs)
    for rc in (0, -1, -2, -3, -4, 7):
        assert isinstance(td.status_str(rc), str)


def attn(**kw):
    a = _td.TdAttnArgs()
    a.B, a.S, a.Hq, a.Hkv, a.D = 2, 16, 32, 2, 128
    a.dtype, a.scale = _td.TD_BF16, 0.0
    a.q = a.k_blk = a.v_blk = a.k_ctx = a.v_ctx = a.ctx_offsets = a.out = FAKE
    a.total_ctx, a.max_ctx = 3000, 2000
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def commit(**kw):
    c = _td.TdCommitArgs()
    c.B, c.S, c.V, c.dtype, c.gamma = 2, 16, 131072, _td.TD_BF16, 0.8
    c.logits = c.commit = c.token = FAKE
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("kw,rc", [
    (dict(B=0), INVALID), (dict(S=0), INVALID), (dict(S=65), INVALID),
    (dict(Hq=30, Hkv=4), INVALID), (dict(Hq=0), INVALID), (dict(Hkv=0), INVALID),
    (dict(D=96), UNSUPPORTED), (dict(D=64), UNSUPPORTED), (dict(dtype=7), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(total_ctx=-1), INVALID), (dict(max_ctx=4000), INVALID),
    (dict(total_ctx=5000, max_ctx=2000), INVALID),
    (dict(q=None), INVALID), (dict(out=None), INVALID), (dict(ctx_offsets=None), INVALID),
    (dict(k_ctx=None), INVALID), (dict(B=70000), UNSUPPORTED), (dict(Hq=256, Hkv=2), UNSUPPORTED),
])
def test_attn_validation(L, kw, rc):
    a = attn(**kw)
    assert L.td_block_attn(ctypes.byref(a), ctypes.c_void_p(FAKE), 1 << 40, None) == rc


def test_noalloc_limit_and_validation(L, monkeypatch):
    """td_denoise_step_noalloc: the header's scratch size matches the
    binding's; invalid arguments and calls whose workspace would exceed the
    library-held scratch are rejected on the host, before the scratch array
    is looked up (these run without a GPU)."""
    import re
    txt = open(_td.HEADER).read()
    m = re.search(r"#define TD_NOALLOC_SCRATCH_BYTES \((\d+)u \* (\d+)u \* (\d+)u\)", txt)
    assert m and int(m.group(1)) * int(m.group(2)) * int(m.group(3)) == _td.TD_NOALLOC_SCRATCH_BYTES
    a, c = attn(), commit()
    assert L.td_denoise_step_noalloc(ctypes.byref(attn(B=0)), ctypes.byref(c), None) == INVALID
    assert L.td_denoise_step_noalloc(ctypes.byref(a), ctypes.byref(commit(B=3)), None) == INVALID
    assert L.td_denoise_step_noalloc(ctypes.byref(attn(D=64)), ctypes.byref(c), None) == UNSUPPORTED
    # a persistent grid of 4096 workgroups needs 2 x 4096 partial slots of 64 KiB
    monkeypatch.setenv("TD_ATTN_GRID", "4096")
    assert L.td_denoise_workspace_bytes(ctypes.byref(a), ctypes.byref(c)) > _td.TD_NOALLOC_SCRATCH_BYTES
    assert L.td_denoise_step_noalloc(ctypes.byref(a), ctypes.byref(c), None) == WORKSPACE
    monkeypatch.delenv("TD_ATTN_GRID")
    # decode-shaped blocks: two partial slots per wave, a size set by the
    # grid alone; the default fits whatever the cache, 4096 workgroups do not
    d = attn(S=1, total_ctx=1 << 27, max_ctx=1 << 26)
    c1 = commit(S=1)
    assert L.td_denoise_workspace_bytes(ctypes.byref(d), ctypes.byref(c1)) <= _td.TD_NOALLOC_SCRATCH_BYTES
    monkeypatch.setenv("TD_DECODE_GRID", "4096")
    assert L.td_denoise_workspace_bytes(ctypes.byref(d), ctypes.byref(c1)) > _td.TD_NOALLOC_SCRATCH_BYTES
    assert L.td_denoise_step_noalloc(ctypes.byref(d), ctypes.byref(c1), None) == WORKSPACE
    monkeypatch.delenv("TD_DECODE_GRID")


def test_attn_empty_context_needs_no_context_pointers(L):
    """total_ctx = 0: null context pointers pass validation (only the
    workspace check then stops the call, before any launch)."""
    a = attn(k_ctx=None, v_ctx=None, total_ctx=0, max_ctx=0)
    need = L.td_attn_workspace_bytes(ctypes.byref(a))
    assert need > 0
    assert L.td_block_attn(ctypes.byref(a), ctypes.c_void_p(FAKE), need - 1, None) == WORKSPACE


def test_attn_workspace_bytes(L):
    """bf16 / D=128 (MFMA path): a persistent grid of 256 workgroups, each
    with two partial slots (256 x 128 bf16 O / l values + 256 fp32 (m, l) pairs),
    plus per-sequence, per-workgroup and per-unit tables.  The size depends
    on the batch shape only, never on the context lengths."""
    slot = 256 * 128 * 2 + 256 * 8
    for B, Lmax, S, Hq in [(64, 8192, 16, 32), (4, 65536, 16, 32), (8, 4096, 16, 32),
                           (32, 2048, 64, 32), (3, 1000, 2, 32)]:
        a = attn(B=B, S=S, Hq=Hq, total_ctx=B * Lmax, max_ctx=Lmax)
        ws = L.td_attn_workspace_bytes(ctypes.byref(a))
        assert 2 * 256 * slot <= ws <= 2 * 256 * slot + 64 * 1024 + B * 64
        a2 = attn(B=B, S=S, Hq=Hq, total_ctx=B * 7, max_ctx=7)
        assert L.td_attn_workspace_bytes(ctypes.byref(a2)) == ws
    f = attn(dtype=_td.TD_F32, D=64)
    assert L.td_attn_workspace_bytes(ctypes.byref(f)) == 0   # VALU path needs none


def test_attn_decode_workspace_bytes(L):
    """At most 16 query rows per KV head (here S = 1, 16 query heads per KV
    head) take the decode path: waves of 4 per workgroup, as many workgroups
    as give each wave about 8 blocks of 32 keys (estimated as (total + B*S)
    / 32 + B blocks per KV head), at most 256; two partial slots per wave
    (16 x 128 bf16 O / l + 16 fp32 (m, l)), plus the per-sequence block
    table."""
    def a256(x):
        return (x + 255) // 256 * 256
    for B, total, S, Hq, Hkv in [(64, 296372, 1, 32, 2), (3, 1000, 1, 32, 2), (1, 0, 1, 4, 1),
                                 (7, 5000, 2, 16, 2), (4, 1 << 20, 1, 32, 2)]:
        a = attn(B=B, S=S, Hq=Hq, Hkv=Hkv, total_ctx=total, max_ctx=total)
        blocks = Hkv * ((total + B * S) // 32 + B)
        wgs = max(1, min(256, -(-blocks // 32)))
        P = 2 * 4 * wgs
        want = a256((B + 1) * 8) + a256(P * 16 * 8) + a256(P * 16 * 128 * 2)
        assert L.td_attn_workspace_bytes(ctypes.byref(a)) == want, (B, total, S)


@pytest.mark.parametrize("kw,rc", [
    (dict(B=0), INVALID), (dict(S=0), INVALID), (dict(S=65), INVALID), (dict(V=0), INVALID),
    (dict(dtype=3), INVALID), (dict(gamma=float("inf")), INVALID),
    (dict(gamma=float("nan")), INVALID), (dict(logits=None), INVALID),
    (dict(commit=None), INVALID), (dict(token=None), INVALID),
])
def test_commit_validation(L, kw, rc):
    c = commit(**kw)
    assert L.td_commit(ctypes.byref(c), ctypes.c_void_p(FAKE), 1 << 40, None) == rc


def test_commit_workspace_checks(L):
    c = commit()
    need = L.td_commit_workspace_bytes(ctypes.byref(c))
    assert need >= 2 * 16 * 16 and need % 256 == 0
    assert L.td_commit(ctypes.byref(c), None, need, None) == WORKSPACE
    assert L.td_commit(ctypes.byref(c), ctypes.c_void_p(FAKE), need - 1, None) == WORKSPACE


def test_denoise_step_checks(L):
    a, c = attn(), commit()
    need = L.td_denoise_workspace_bytes(ctypes.byref(a), ctypes.byref(c))
    assert need >= L.td_attn_workspace_bytes(ctypes.byref(a)) + L.td_commit_workspace_bytes(ctypes.byref(c))
    c2 = commit(S=8)
    assert L.td_denoise_step(ctypes.byref(a), ctypes.byref(c2), ctypes.c_void_p(FAKE), need, None) == INVALID
    assert L.td_denoise_step(ctypes.byref(a), ctypes.byref(c), None, need, None) == WORKSPACE
    a_bad = attn(D=96)
    assert L.td_denoise_step(ctypes.byref(a_bad), ctypes.byref(c), ctypes.c_void_p(FAKE), need, None) == UNSUPPORTED


def test_denoise_step_if_gate_checks(L):
    """The gate must be given and must not be the step's own n_masked_left
    (which the commit clears); otherwise the checks are td_denoise_step's."""
    a = attn()
    c = commit(n_masked_left=FAKE + 4096)
    need = L.td_denoise_workspace_bytes(ctypes.byref(a), ctypes.byref(c))
    ws = ctypes.c_void_p(FAKE)
    step_if = L.td_denoise_step_if
    assert step_if(ctypes.byref(a), ctypes.byref(c), None, ws, need, None) == INVALID
    assert step_if(ctypes.byref(a), ctypes.byref(c), ctypes.c_void_p(FAKE + 4096), ws, need, None) == INVALID
    assert step_if(ctypes.byref(a), ctypes.byref(c), ctypes.c_void_p(FAKE + 8192), None, need, None) == WORKSPACE
    c2 = commit(S=8)
    assert step_if(ctypes.byref(a), ctypes.byref(c2), ctypes.c_void_p(FAKE + 8192), ws, need, None) == INVALID


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 16, 4, 64)
    with pytest.raises(ValueError):
        _td.attn_args(x, x, x, x, x, torch.zeros(2, dtype=torch.int64), x, 0, 0)


GB = 1 << 32            # distinct fake buffers, far apart: no overlap unless a case makes one


def append(**kw):
    p = _td.TdAppendArgs()
    p.B, p.S, p.Hkv, p.D, p.dtype = 2, 16, 2, 128, _td.TD_BF16
    p.total_ctx = 3000
    p.k_ctx, p.v_ctx, p.k_new, p.v_new = 1 * GB, 2 * GB, 3 * GB, 4 * GB
    p.k_out, p.v_out = 5 * GB, 6 * GB
    p.ctx_offsets, p.offsets_out = 7 * GB, 8 * GB
    for k, v in kw.items():
        setattr(p, k, v)
    return p


ROW = 2 * 128 * 2       # bytes per cache row of the default case


@pytest.mark.parametrize("kw,rc", [
    (dict(B=0), INVALID), (dict(S=-1), INVALID), (dict(S=65537), INVALID),
    (dict(Hkv=0), INVALID), (dict(D=0), INVALID), (dict(dtype=7), INVALID),
    (dict(total_ctx=-1), INVALID),
    (dict(Hkv=1, D=3), UNSUPPORTED),                          # 6-byte rows
    (dict(Hkv=256, D=128, dtype=_td.TD_F32), UNSUPPORTED),    # 128 KiB rows
    (dict(total_ctx=1 << 34, Hkv=1, D=8), UNSUPPORTED),       # more than 2^34 output rows
    (dict(ctx_offsets=None), INVALID), (dict(offsets_out=None), INVALID),
    (dict(k_ctx=None), INVALID), (dict(v_new=None), INVALID), (dict(k_out=None), INVALID),
    (dict(k_ctx=1 * GB + 8), INVALID), (dict(v_out=6 * GB + 4), INVALID),
    (dict(offsets_out=8 * GB + 4), INVALID),
    (dict(k_out=1 * GB), INVALID),                            # output on top of its input
    (dict(v_out=5 * GB + 3031 * ROW), INVALID),               # last row of k_out
    (dict(k_out=4 * GB + 16 * ROW), INVALID),                 # k_out starts inside v_new
    (dict(offsets_out=7 * GB + 16), INVALID),                 # offsets_out over ctx_offsets
    (dict(offsets_out=5 * GB + 64), INVALID),                 # offsets_out inside k_out
])
def test_append_validation(L, kw, rc):
    p = append(**kw)
    assert L.td_cache_append(ctypes.byref(p), None) == rc


def test_append_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(2, 4, 2, 64)
    with pytest.raises(ValueError):
        _td.append_args(torch.zeros(0, 2, 64), torch.zeros(0, 2, 64), torch.zeros(3, dtype=torch.int64),
                        0, x, x, torch.zeros(8, 2, 64), torch.zeros(8, 2, 64),
                        torch.zeros(3, dtype=torch.int64))


def lmhead(**kw):
    a = _td.TdLmheadArgs()
    a.B, a.S, a.H, a.V, a.dtype, a.gamma = 64, 16, 4096, 131072, _td.TD_BF16, 0.8
    a.hidden, a.w_head, a.commit, a.token = 1 * GB, 2 * GB, 3 * GB, 4 * GB
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,rc", [
    (dict(B=0), INVALID), (dict(S=0), INVALID), (dict(S=65), INVALID), (dict(V=0), INVALID),
    (dict(H=0), INVALID), (dict(dtype=7), INVALID), (dict(gamma=float("inf")), INVALID),
    (dict(dtype=_td.TD_F32), UNSUPPORTED), (dict(H=100), UNSUPPORTED), (dict(H=96), UNSUPPORTED),
    (dict(H=65600), UNSUPPORTED), (dict(B=4096, H=65536), UNSUPPORTED),
    (dict(hidden=None), INVALID), (dict(w_head=None), INVALID), (dict(commit=None), INVALID),
    (dict(token=None), INVALID), (dict(hidden=1 * GB + 2), INVALID), (dict(w_head=2 * GB + 8), INVALID),
])
def test_lmhead_validation(L, kw, rc):
    a = lmhead(**kw)
    assert L.td_lmhead_commit(ctypes.byref(a), ctypes.c_void_p(FAKE), 1 << 40, None) == rc


def test_lmhead_workspace_bytes(L):
    """16 bytes per (position, 256-token slice), 16 per position, then the
    eligible-position list and its count (each piece 256-byte aligned)."""
    a = lmhead()
    parts = 64 * 16 * 512 * 16
    assert L.td_lmhead_commit_workspace_bytes(ctypes.byref(a)) == parts + 1024 * 16 + 1025 * 4
    b = lmhead(V=257, B=1, S=3)
    assert L.td_lmhead_commit_workspace_bytes(ctypes.byref(b)) == 256 + 256 + 4 * 4
    assert L.td_lmhead_commit_workspace_bytes(ctypes.byref(lmhead(H=100))) == 0
    need = L.td_lmhead_commit_workspace_bytes(ctypes.byref(a))
    assert L.td_lmhead_commit(ctypes.byref(a), ctypes.c_void_p(FAKE), need - 1, None) == WORKSPACE


def mamba(**kw):
    a = _td.TdMambaArgs()
    a.B, a.S, a.H, a.P, a.N, a.G = 64, 16, 128, 64, 128, 8
    a.x, a.dt, a.A, a.Bm, a.Cm, a.D, a.h0, a.y = (k * GB for k in range(1, 9))
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,rc", [
    (dict(B=0), INVALID), (dict(S=0), INVALID), (dict(H=0), INVALID), (dict(G=0), INVALID),
    (dict(H=12, G=8), INVALID), (dict(S=17), UNSUPPORTED), (dict(P=48), UNSUPPORTED),
    (dict(P=256), UNSUPPORTED), (dict(N=100), UNSUPPORTED), (dict(N=48), UNSUPPORTED),
    (dict(N=2048), UNSUPPORTED),
    (dict(x=None), INVALID), (dict(h0=None), INVALID), (dict(y=None), INVALID), (dict(dt=None), INVALID),
    (dict(Bm=2 * GB + 8), INVALID), (dict(h0=7 * GB + 4), INVALID), (dict(y=8 * GB + 2), INVALID),
    (dict(x=1 * GB + 8), INVALID),
])
def test_mamba_validation(L, kw, rc):
    a = mamba(**kw)
    assert L.td_mamba_block_scan(ctypes.byref(a), None) == rc


def adaln(**kw):
    a = _td.TdAdalnArgs()
    a.B, a.S, a.H, a.eps = 64, 16, 4096, 1e-5
    (a.x, a.f, a.t_mod, a.tab_gate, a.tab_shift, a.tab_scale, a.w_norm, a.r_out,
     a.h) = (k * GB for k in range(1, 10))
    for k, v in kw.items():
        setattr(a, k, v)
    return a


ACT = 64 * 16 * 4096 * 2


@pytest.mark.parametrize("kw,rc", [
    (dict(B=-1), INVALID), (dict(S=-1), INVALID), (dict(H=0), INVALID),
    (dict(eps=-1.0), INVALID), (dict(eps=float("nan")), INVALID), (dict(eps=float("inf")), INVALID),
    (dict(H=12), UNSUPPORTED), (dict(H=8200), UNSUPPORTED),
    (dict(x=None), INVALID), (dict(t_mod=None), INVALID), (dict(h=None), INVALID),
    (dict(r_out=None), INVALID),
    (dict(x=1 * GB + 8), INVALID), (dict(f=2 * GB + 2), INVALID), (dict(w_norm=7 * GB + 4), INVALID),
    (dict(tab_gate=4 * GB + 8), INVALID), (dict(h=9 * GB + 8), INVALID), (dict(r_out=8 * GB + 2), INVALID),
    # overlaps: only r_out == x, h == x and h == f are allowed
    (dict(r_out=1 * GB + 16), INVALID), (dict(r_out=2 * GB), INVALID), (dict(h=8 * GB), INVALID),
    (dict(h=8 * GB + ACT - 16), INVALID), (dict(h=3 * GB), INVALID), (dict(h=7 * GB - ACT + 16), INVALID),
    (dict(r_out=1 * GB, h=1 * GB), INVALID), (dict(h=2 * GB + 16), INVALID),
    # nothing to do: valid, nothing enqueued
    (dict(B=0), OK), (dict(S=0), OK), (dict(B=0, x=None, h=None, t_mod=None), OK),
])
def test_adaln_validation(L, kw, rc):
    a = adaln(**kw)
    assert L.td_adaln_modulate(ctypes.byref(a), None) == rc


def test_lmhead_packed_layout_validation(L):
    assert L.td_lmhead_commit(ctypes.byref(lmhead(w_head_packed=2)), ctypes.c_void_p(FAKE),
                              1 << 30, None) == INVALID
    assert L.td_lmhead_packed_bytes(131072, 4096) == 131072 * 4096 * 2
    assert L.td_lmhead_packed_bytes(257, 64) == 512 * 64 * 2
    assert L.td_lmhead_packed_bytes(1, 128) == 256 * 128 * 2
    for V, H in ((0, 64), (5, 100), (5, 0), (5, 32), (5, 65600), ((1 << 30) + 1, 64)):
        assert L.td_lmhead_packed_bytes(V, H) == 0


@pytest.mark.parametrize("w,V,H,p,rc", [
    (GB, 0, 64, 2 * GB, INVALID), (GB, 5, 0, 2 * GB, INVALID), (GB, 5, 100, 2 * GB, UNSUPPORTED),
    (GB, 5, 131072, 2 * GB, UNSUPPORTED), (None, 5, 64, 2 * GB, INVALID), (GB, 5, 64, None, INVALID),
    (GB + 8, 5, 64, 2 * GB, INVALID), (GB, 5, 64, 2 * GB + 4, INVALID),
    (GB, 300, 64, GB + 300 * 64 * 2 - 16, INVALID),       # packed copy overlaps the weight
    (2 * GB, 300, 64, 2 * GB - 512 * 64 * 2 + 16, INVALID),
])
def test_lmhead_pack_validation(L, w, V, H, p, rc):
    assert L.td_lmhead_pack_head(w, V, H, p, None) == rc



def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    """No CPU fallback: with libtd.so absent every entry raises before doing
    anything."""
    monkeypatch.setattr(_td, "LIB_PATH", str(tmp_path / "libtd.so"))
    monkeypatch.setattr(_td, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        _td.lib()
    for call in (lambda: td.td_adaln_modulate(None, None, None, None),
                 lambda: td.td_mamba_block_scan(*([None] * 8)),
                 lambda: td.td_cache_append(*([None] * 8), total_ctx=0)):
        with pytest.raises(RuntimeError, match="not built"):
            call()


def test_product_package_never_imports_the_oracle():
    """The oracle is test infrastructure: nothing under the package imports
    it (or the input generators)."""
    import re
    pkg = os.path.dirname(_td.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                txt = open(os.path.join(root, f), errors="replace").read()
                assert not re.search(r"^\s*(import|from)\s+(oracle|synth)\b", txt, re.M), f
