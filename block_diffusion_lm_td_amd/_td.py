"""ctypes binding of libtd.so (include/td.h).

Argument marshalling only: torch tensors supply device pointers and the HIP
stream, every step of the computation runs in the library's kernels.  There
is no fallback: if libtd.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import c_float, c_int, c_int32, c_int64, c_size_t, c_uint32, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtd.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "td.h")

TD_OK, TD_ERR_INVALID, TD_ERR_UNSUPPORTED, TD_ERR_WORKSPACE, TD_ERR_HIP = 0, -1, -2, -3, -4
TD_F32, TD_BF16 = 0, 1
TD_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024     # td.h's TD_NOALLOC_SCRATCH_BYTES


class TdAttnArgs(ctypes.Structure):
    _fields_ = [("B", c_int32), ("S", c_int32), ("Hq", c_int32), ("Hkv", c_int32),
                ("D", c_int32), ("dtype", c_int), ("scale", c_float),
                ("q", c_void_p), ("k_blk", c_void_p), ("v_blk", c_void_p),
                ("k_ctx", c_void_p), ("v_ctx", c_void_p), ("ctx_offsets", c_void_p),
                ("total_ctx", c_int64), ("max_ctx", c_int64), ("out", c_void_p)]


class TdCommitArgs(ctypes.Structure):
    _fields_ = [("B", c_int32), ("S", c_int32), ("V", c_int32), ("dtype", c_int),
                ("gamma", c_float), ("logits", c_void_p), ("masked_in", c_void_p),
                ("commit", c_void_p), ("token", c_void_p), ("maxprob", c_void_p),
                ("n_commit", c_void_p), ("masked_out", c_void_p), ("tokens", c_void_p),
                ("n_masked_left", c_void_p)]


class TdAppendArgs(ctypes.Structure):
    _fields_ = [("B", c_int32), ("S", c_int32), ("Hkv", c_int32), ("D", c_int32),
                ("dtype", c_int), ("k_ctx", c_void_p), ("v_ctx", c_void_p),
                ("ctx_offsets", c_void_p), ("total_ctx", c_int64), ("k_new", c_void_p),
                ("v_new", c_void_p), ("k_out", c_void_p), ("v_out", c_void_p),
                ("offsets_out", c_void_p)]


class TdLmheadArgs(ctypes.Structure):
    _fields_ = [("B", c_int32), ("S", c_int32), ("H", c_int32), ("V", c_int32),
                ("dtype", c_int), ("gamma", c_float), ("hidden", c_void_p), ("w_head", c_void_p),
                ("masked_in", c_void_p), ("commit", c_void_p), ("token", c_void_p),
                ("maxprob", c_void_p), ("n_commit", c_void_p), ("masked_out", c_void_p),
                ("tokens", c_void_p), ("n_masked_left", c_void_p), ("w_head_packed", c_int32)]


class TdMambaArgs(ctypes.Structure):
    _fields_ = [("B", c_int32), ("S", c_int32), ("H", c_int32), ("P", c_int32), ("N", c_int32),
                ("G", c_int32), ("x", c_void_p), ("dt", c_void_p), ("A", c_void_p), ("Bm", c_void_p),
                ("Cm", c_void_p), ("D", c_void_p), ("h0", c_void_p), ("y", c_void_p)]


class TdAdalnArgs(ctypes.Structure):
    _fields_ = [("B", c_int32), ("S", c_int32), ("H", c_int32), ("eps", ctypes.c_float),
                ("x", c_void_p), ("f", c_void_p), ("t_mod", c_void_p), ("tab_gate", c_void_p),
                ("tab_shift", c_void_p), ("tab_scale", c_void_p), ("w_norm", c_void_p),
                ("r_out", c_void_p), ("h", c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libtd.so once; raise if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m block_diffusion_lm_td_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        A, C = ctypes.POINTER(TdAttnArgs), ctypes.POINTER(TdCommitArgs)
        P = ctypes.POINTER(TdAppendArgs)
        LH = ctypes.POINTER(TdLmheadArgs)
        MB = ctypes.POINTER(TdMambaArgs)
        AD = ctypes.POINTER(TdAdalnArgs)
        sig = {
            "td_abi_version": (c_uint32, []),
            "td_sizeof_attn_args": (c_size_t, []),
            "td_sizeof_commit_args": (c_size_t, []),
            "td_sizeof_append_args": (c_size_t, []),
            "td_sizeof_lmhead_args": (c_size_t, []),
            "td_sizeof_mamba_args": (c_size_t, []),
            "td_sizeof_adaln_args": (c_size_t, []),
            "td_status_str": (ctypes.c_char_p, [c_int]),
            "td_attn_workspace_bytes": (c_size_t, [A]),
            "td_commit_workspace_bytes": (c_size_t, [C]),
            "td_denoise_workspace_bytes": (c_size_t, [A, C]),
            "td_block_attn": (c_int, [A, c_void_p, c_size_t, c_void_p]),
            "td_commit": (c_int, [C, c_void_p, c_size_t, c_void_p]),
            "td_denoise_step": (c_int, [A, C, c_void_p, c_size_t, c_void_p]),
            "td_denoise_step_if": (c_int, [A, C, c_void_p, c_void_p, c_size_t, c_void_p]),
            "td_denoise_step_noalloc": (c_int, [A, C, c_void_p]),
            "td_cache_append": (c_int, [P, c_void_p]),
            "td_lmhead_commit_workspace_bytes": (c_size_t, [LH]),
            "td_lmhead_commit": (c_int, [LH, c_void_p, c_size_t, c_void_p]),
            "td_lmhead_packed_bytes": (c_size_t, [c_int32, c_int32]),
            "td_lmhead_pack_head": (c_int, [c_void_p, c_int32, c_int32, c_void_p, c_void_p]),
            "td_mamba_block_scan": (c_int, [MB, c_void_p]),
            "td_adaln_modulate": (c_int, [AD, c_void_p]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        if L.td_sizeof_attn_args() != ctypes.sizeof(TdAttnArgs) or \
                L.td_sizeof_commit_args() != ctypes.sizeof(TdCommitArgs) or \
                L.td_sizeof_append_args() != ctypes.sizeof(TdAppendArgs) or \
                L.td_sizeof_lmhead_args() != ctypes.sizeof(TdLmheadArgs) or \
                L.td_sizeof_mamba_args() != ctypes.sizeof(TdMambaArgs) or \
                L.td_sizeof_adaln_args() != ctypes.sizeof(TdAdalnArgs):
            raise RuntimeError("libtd.so struct layout does not match the binding")
        _lib = L
    return _lib


def header_functions(path: str = HEADER) -> list[str]:
    """Names of the functions include/td.h declares."""
    txt = open(path).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(td_\w+)\s*\(", txt)))


def status_str(rc: int) -> str:
    return lib().td_status_str(rc).decode()


def check(rc: int, what: str) -> None:
    if rc != TD_OK:
        raise RuntimeError(f"{what}: {status_str(rc)}")


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return TD_BF16
    if t.dtype == torch.float32:
        return TD_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t, name, dtype=None, shape=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _torch_stream(stream, device=None):
    torch = _torch()
    return torch.cuda.current_stream(device) if stream is None else stream


def _stream(stream):
    return c_void_p(_torch_stream(stream).cuda_stream)


def attn_args(q, k_blk, v_blk, k_ctx, v_ctx, ctx_offsets, out, total_ctx, max_ctx,
              scale=0.0) -> TdAttnArgs:
    torch = _torch()
    B, S, Hq, D = q.shape
    Hkv = k_blk.shape[2]
    dt = q.dtype
    a = TdAttnArgs()
    a.B, a.S, a.Hq, a.Hkv, a.D = B, S, Hq, Hkv, D
    a.dtype = _dtype_code(q)
    a.scale = float(scale)
    a.q = _ptr(q, "q", dt)
    a.k_blk = _ptr(k_blk, "k_blk", dt, (B, S, Hkv, D))
    a.v_blk = _ptr(v_blk, "v_blk", dt, (B, S, Hkv, D))
    a.k_ctx = _ptr(k_ctx, "k_ctx", dt, (total_ctx, Hkv, D))
    a.v_ctx = _ptr(v_ctx, "v_ctx", dt, (total_ctx, Hkv, D))
    a.ctx_offsets = _ptr(ctx_offsets, "ctx_offsets", torch.int64, (B + 1,))
    a.total_ctx, a.max_ctx = int(total_ctx), int(max_ctx)
    a.out = _ptr(out, "out", dt, (B, S, Hq, D))
    return a


def commit_args(logits, commit, token, gamma, masked_in=None, maxprob=None, n_commit=None,
                masked_out=None, tokens=None, n_masked_left=None) -> TdCommitArgs:
    torch = _torch()
    B, S, V = logits.shape
    c = TdCommitArgs()
    c.B, c.S, c.V = B, S, V
    c.dtype = _dtype_code(logits)
    c.gamma = float(gamma)
    c.logits = _ptr(logits, "logits")
    c.masked_in = _ptr(masked_in, "masked_in", torch.uint8, (B, S))
    c.commit = _ptr(commit, "commit", torch.uint8, (B, S))
    c.token = _ptr(token, "token", torch.int32, (B, S))
    c.maxprob = _ptr(maxprob, "maxprob", torch.float32, (B, S))
    c.n_commit = _ptr(n_commit, "n_commit", torch.int32, (B,))
    c.masked_out = _ptr(masked_out, "masked_out", torch.uint8, (B, S))
    c.tokens = _ptr(tokens, "tokens", torch.int32, (B, S))
    c.n_masked_left = _ptr(n_masked_left, "n_masked_left", torch.int32, (1,))
    return c


def append_args(k_ctx, v_ctx, ctx_offsets, total_ctx, k_new, v_new, k_out, v_out,
                offsets_out) -> TdAppendArgs:
    torch = _torch()
    B, S, Hkv, D = k_new.shape
    dt = k_new.dtype
    N = int(total_ctx) + B * S
    p = TdAppendArgs()
    p.B, p.S, p.Hkv, p.D = B, S, Hkv, D
    p.dtype = _dtype_code(k_new)
    p.k_ctx = _ptr(k_ctx, "k_ctx", dt, (total_ctx, Hkv, D))
    p.v_ctx = _ptr(v_ctx, "v_ctx", dt, (total_ctx, Hkv, D))
    p.ctx_offsets = _ptr(ctx_offsets, "ctx_offsets", torch.int64, (B + 1,))
    p.total_ctx = int(total_ctx)
    p.k_new = _ptr(k_new, "k_new", dt)
    p.v_new = _ptr(v_new, "v_new", dt, (B, S, Hkv, D))
    p.k_out = _ptr(k_out, "k_out", dt, (N, Hkv, D))
    p.v_out = _ptr(v_out, "v_out", dt, (N, Hkv, D))
    p.offsets_out = _ptr(offsets_out, "offsets_out", torch.int64, (B + 1,))
    return p


class PackedHead:
    """An LM-head weight in the packed order td_lmhead_pack_head writes
    (a flat bf16 device tensor) with its vocabulary and hidden sizes."""

    def __init__(self, data, V: int, H: int):
        self.data, self.V, self.H = data, int(V), int(H)


def lmhead_args(hidden, w_head, commit, token, gamma, masked_in=None, maxprob=None,
                n_commit=None, masked_out=None, tokens=None, n_masked_left=None) -> TdLmheadArgs:
    """w_head: the [V, H] weight, or a PackedHead."""
    torch = _torch()
    B, S, H = hidden.shape
    a = TdLmheadArgs()
    if isinstance(w_head, PackedHead):
        if w_head.H != H:
            raise ValueError(f"packed head has H={w_head.H}, hidden has H={H}")
        V = w_head.V
        a.w_head = _ptr(w_head.data, "w_head", hidden.dtype, (lib().td_lmhead_packed_bytes(V, H) // 2,))
        a.w_head_packed = 1
    else:
        V = w_head.shape[0]
        a.w_head = _ptr(w_head, "w_head", hidden.dtype, (V, H))
        a.w_head_packed = 0
    a.B, a.S, a.H, a.V = B, S, H, V
    a.dtype = _dtype_code(hidden)
    a.gamma = float(gamma)
    a.hidden = _ptr(hidden, "hidden")
    a.masked_in = _ptr(masked_in, "masked_in", torch.uint8, (B, S))
    a.commit = _ptr(commit, "commit", torch.uint8, (B, S))
    a.token = _ptr(token, "token", torch.int32, (B, S))
    a.maxprob = _ptr(maxprob, "maxprob", torch.float32, (B, S))
    a.n_commit = _ptr(n_commit, "n_commit", torch.int32, (B,))
    a.masked_out = _ptr(masked_out, "masked_out", torch.uint8, (B, S))
    a.tokens = _ptr(tokens, "tokens", torch.int32, (B, S))
    a.n_masked_left = _ptr(n_masked_left, "n_masked_left", torch.int32, (1,))
    return a


def mamba_args(x, dt, A, Bm, Cm, D, h0, y) -> TdMambaArgs:
    torch = _torch()
    B, S, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    a = TdMambaArgs()
    a.B, a.S, a.H, a.P, a.N, a.G = B, S, H, P, N, G
    a.x = _ptr(x, "x", torch.bfloat16)
    a.dt = _ptr(dt, "dt", torch.float32, (B, S, H))
    a.A = _ptr(A, "A", torch.float32, (H,))
    a.Bm = _ptr(Bm, "Bm", torch.bfloat16, (B, S, G, N))
    a.Cm = _ptr(Cm, "Cm", torch.bfloat16, (B, S, G, N))
    a.D = _ptr(D, "D", torch.float32, (H,))
    a.h0 = _ptr(h0, "h0", torch.float32, (B, H, P, N))
    a.y = _ptr(y, "y", torch.bfloat16, (B, S, H, P))
    return a


def adaln_args(x, f, t_mod, h, r_out=None, *, tab_gate=None, tab_shift=None, tab_scale=None,
               w_norm=None, eps=1e-5) -> TdAdalnArgs:
    torch = _torch()
    B, S, H = x.shape
    a = TdAdalnArgs()
    a.B, a.S, a.H, a.eps = B, S, H, float(eps)
    a.x = _ptr(x, "x", torch.bfloat16)
    a.f = _ptr(f, "f", torch.bfloat16, (B, S, H))
    a.t_mod = _ptr(t_mod, "t_mod", torch.float32, (B, 3, H))
    a.tab_gate = _ptr(tab_gate, "tab_gate", torch.float32, (H,))
    a.tab_shift = _ptr(tab_shift, "tab_shift", torch.float32, (H,))
    a.tab_scale = _ptr(tab_scale, "tab_scale", torch.float32, (H,))
    a.w_norm = _ptr(w_norm, "w_norm", torch.float32, (H,))
    a.r_out = _ptr(r_out, "r_out", torch.bfloat16, (B, S, H))
    a.h = _ptr(h, "h", torch.bfloat16, (B, S, H))
    return a


class Workspace:
    """Caller-owned device scratch for the td_* calls (a torch byte tensor,
    grown on demand; torch's allocator returns 256-byte aligned blocks).

    A call's kernels use the buffer until they finish on the call's stream.
    One Workspace must therefore not serve two calls that may run at the same
    time on different streams (their partials would race); calls in order on
    one stream may share it.  Every use records its stream on the buffer, so
    that a buffer replaced when it grows is not handed out again by torch's
    allocator before the kernels already enqueued on those streams are done."""

    def __init__(self, device=None):
        self.device = device
        self.buf = None

    def get(self, nbytes: int, stream=None):
        torch = _torch()
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device or "cuda")
        if stream is not None and not torch.cuda.is_current_stream_capturing():
            self.buf.record_stream(stream)
        return c_void_p(self.buf.data_ptr()), self.buf.numel()


_default_ws = {}


def _ws(workspace, device, stream):
    """The caller's workspace, else a default one per (device, stream): calls
    on different streams never share a default workspace."""
    if workspace is not None:
        return workspace
    key = (str(device), int(stream.cuda_stream))
    if key not in _default_ws:
        _default_ws[key] = Workspace(device)
    return _default_ws[key]


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def td_block_attn(q, k_blk, v_blk, k_ctx, v_ctx, ctx_offsets, out, *, total_ctx, max_ctx,
                  scale=0.0, workspace=None, stream=None):
    L = lib()
    a = attn_args(q, k_blk, v_blk, k_ctx, v_ctx, ctx_offsets, out, total_ctx, max_ctx, scale)
    need = L.td_attn_workspace_bytes(ctypes.byref(a))
    ts = _torch_stream(stream, q.device)
    ptr, n = _ws(workspace, q.device, ts).get(need, ts)
    check(L.td_block_attn(ctypes.byref(a), ptr, n, c_void_p(ts.cuda_stream)), "td_block_attn")
    return out


def td_commit(logits, commit, token, *, gamma, masked_in=None, maxprob=None, n_commit=None,
              masked_out=None, tokens=None, n_masked_left=None, workspace=None, stream=None):
    L = lib()
    c = commit_args(logits, commit, token, gamma, masked_in, maxprob, n_commit, masked_out,
                    tokens, n_masked_left)
    need = L.td_commit_workspace_bytes(ctypes.byref(c))
    ts = _torch_stream(stream, logits.device)
    ptr, n = _ws(workspace, logits.device, ts).get(need, ts)
    check(L.td_commit(ctypes.byref(c), ptr, n, c_void_p(ts.cuda_stream)), "td_commit")


def td_denoise_step(attn: TdAttnArgs, commit: TdCommitArgs, *, workspace=None, device=None,
                    stream=None):
    """One denoise step from prepared argument structs (see attn_args /
    commit_args): block attention, then the commit, on one stream."""
    L = lib()
    need = L.td_denoise_workspace_bytes(ctypes.byref(attn), ctypes.byref(commit))
    ts = _torch_stream(stream, device)
    ptr, n = _ws(workspace, device, ts).get(need, ts)
    check(L.td_denoise_step(ctypes.byref(attn), ctypes.byref(commit), ptr, n,
                            c_void_p(ts.cuda_stream)), "td_denoise_step")


def td_denoise_step_noalloc(attn: TdAttnArgs, commit: TdCommitArgs, *, stream=None):
    """td_denoise_step on the library's own per-GPU scratch array: no
    workspace, nothing allocated.  Calls that may overlap on one GPU race on
    that array and must not be made."""
    L = lib()
    check(L.td_denoise_step_noalloc(ctypes.byref(attn), ctypes.byref(commit), _stream(stream)),
          "td_denoise_step_noalloc")


def td_denoise_step_if(attn: TdAttnArgs, commit: TdCommitArgs, gate, *, workspace=None,
                       device=None, stream=None):
    """td_denoise_step gated by the device int32 tensor ``gate`` (shape (1,)):
    the step runs when it holds a nonzero value when the step starts on the
    device, and otherwise only clears the commit's n_masked_left."""
    torch = _torch()
    L = lib()
    g = _ptr(gate, "gate", torch.int32, (1,))
    need = L.td_denoise_workspace_bytes(ctypes.byref(attn), ctypes.byref(commit))
    ts = _torch_stream(stream, device)
    ptr, n = _ws(workspace, device, ts).get(need, ts)
    check(L.td_denoise_step_if(ctypes.byref(attn), ctypes.byref(commit), c_void_p(g), ptr, n,
                               c_void_p(ts.cuda_stream)), "td_denoise_step_if")


def td_cache_append(k_ctx, v_ctx, ctx_offsets, k_new, v_new, k_out, v_out, offsets_out, *,
                    total_ctx, stream=None):
    """Append the block's rows k_new / v_new [B, S, Hkv, D] to every
    sequence's packed cache: k_out / v_out [total_ctx + B*S, Hkv, D] and
    offsets_out [B+1] become the next block's context cache."""
    L = lib()
    p = append_args(k_ctx, v_ctx, ctx_offsets, total_ctx, k_new, v_new, k_out, v_out, offsets_out)
    check(L.td_cache_append(ctypes.byref(p), _stream(stream)), "td_cache_append")
    return k_out, v_out, offsets_out


def td_lmhead_pack_head(w_head, *, stream=None) -> PackedHead:
    """The [V, H] bf16 LM-head weight rearranged once for td_lmhead_commit
    (each pipeline stage's 256 x 64 block contiguous); same results."""
    torch = _torch()
    L = lib()
    V, H = w_head.shape
    n = L.td_lmhead_packed_bytes(V, H)
    if n == 0:
        raise ValueError(f"td_lmhead_pack_head: unsupported V={V}, H={H}")
    out = torch.empty(n // 2, dtype=w_head.dtype, device=w_head.device)
    check(L.td_lmhead_pack_head(_ptr(w_head, "w_head", torch.bfloat16, (V, H)), V, H,
                                _ptr(out, "w_packed"), _stream(stream)), "td_lmhead_pack_head")
    return PackedHead(out, V, H)


def td_lmhead_commit(hidden, w_head, commit, token, *, gamma, masked_in=None, maxprob=None,
                     n_commit=None, masked_out=None, tokens=None, n_masked_left=None,
                     workspace=None, stream=None):
    """Commit of one step straight from the block's hidden states [B, S, H]
    and the LM-head weight [V, H] (or its PackedHead): the logits stay on
    chip."""
    L = lib()
    a = lmhead_args(hidden, w_head, commit, token, gamma, masked_in, maxprob, n_commit,
                    masked_out, tokens, n_masked_left)
    need = L.td_lmhead_commit_workspace_bytes(ctypes.byref(a))
    ts = _torch_stream(stream, hidden.device)
    ptr, n = _ws(workspace, hidden.device, ts).get(need, ts)
    check(L.td_lmhead_commit(ctypes.byref(a), ptr, n, c_void_p(ts.cuda_stream)), "td_lmhead_commit")


def td_mamba_block_scan(x, dt, A, Bm, Cm, D, h0, y, *, stream=None):
    """The state-space core of a denoiser Mamba-2 layer over the block,
    started from the context tower's state h0 [B, H, P, N]; writes y."""
    L = lib()
    a = mamba_args(x, dt, A, Bm, Cm, D, h0, y)
    check(L.td_mamba_block_scan(ctypes.byref(a), _stream(stream)), "td_mamba_block_scan")
    return y


def td_adaln_modulate(x, f, t_mod, h, r_out=None, *, tab_gate=None, tab_shift=None,
                      tab_scale=None, w_norm=None, eps=1e-5, stream=None):
    """adaLN-single between two layers: r = x + gate * f (written to r_out
    when f is given), h = RMSNorm(r) * w_norm * (1 + scale) + shift, with
    shift / scale / gate = t_mod [B, 3, H] rows plus the layer tables."""
    L = lib()
    a = adaln_args(x, f, t_mod, h, r_out, tab_gate=tab_gate, tab_shift=tab_shift,
                   tab_scale=tab_scale, w_norm=w_norm, eps=eps)
    check(L.td_adaln_modulate(ctypes.byref(a), _stream(stream)), "td_adaln_modulate")
    return h

