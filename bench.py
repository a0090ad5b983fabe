"""Denoise-step throughput on one MI355X.

A step is one td_denoise_step: the block attention of one denoiser attention
layer (64 blocks of S = 16 [MASK] positions over ragged cached contexts of
1K..8K tokens, 32 query / 2 KV heads, head dim 128, bf16) plus the
confidence-masked commit of the block's 131072-way logits at gamma = 0.8.
Inputs are seeded synthetic data of that shape, resident in HBM before the
timed region; several input sets rotate so that the 256 MB last-level cache
cannot serve a step from the previous use of its data.

Prints one JSON line (see the "metric" and "config" keys).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "denoise steps/sec (S=16, ctx 8K, B=64) and % of HBM/MFMA roofline, 1 GPU"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2516.6
ATTN_SRC = os.path.join(ROOT, "block_diffusion_lm_td_amd", "csrc", "td_attn.hip")
DECODE_SRC = os.path.join(ROOT, "block_diffusion_lm_td_amd", "csrc", "td_decode.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic_bf16_b64_ragged1k_8k.json")
APPEND_SRC = os.path.join(ROOT, "block_diffusion_lm_td_amd", "csrc", "td_append.hip")
APPEND_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "append_traffic_bf16_b64_ragged1k_8k.json")
PART_WARMUP = 10        # untimed launches of one part before it is timed on its own
PART_LAUNCHES = 100     # at least this many launches of one part are timed back to back


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(w, lengths):
    """Bytes and flops the method itself must move / compute per step."""
    e = 2 if w.dtype == "bf16" else 4
    sum_l = int(lengths.sum())
    attn_bytes = (sum_l * w.Hkv * w.D * 2 * e                       # context K and V
                  + w.B * w.S * (w.Hq + 2 * w.Hkv) * w.D * e         # Q, block K and V
                  + w.B * w.S * w.Hq * w.D * e)                      # out
    attn_flops = 4 * w.Hq * w.S * w.D * (sum_l + w.B * w.S)
    commit_bytes = w.B * w.S * w.V * e + w.B * w.S * 10
    return attn_bytes, attn_flops, commit_bytes


def source_sha(path):
    """sha256 (first 16 hex digits) of a C++/HIP source's code: comments and
    whitespace removed, so that editing a comment keeps a measurement valid
    while any change to the code voids it."""
    import re
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    code = " ".join(text.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def measured_traffic(workload, src=None, path=None):
    """HBM bytes per launch of a kernel (default: the attention kernels) from
    committed rocprofv3 counter runs on this workload, valid only while the
    kernel source is unchanged."""
    src = ATTN_SRC if src is None else src
    path = TRAFFIC_FILE if path is None else path
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha") != source_sha(src) or t.get("workload") != workload:
        return None
    return t.get("bytes_per_launch")


def append_algorithmic(w, total_ctx):
    """Bytes one context-cache append must move: every old and new row of K
    and V read once and written once, plus the offsets read and written."""
    e = 2 if w.dtype == "bf16" else 4
    rows = total_ctx + w.B * w.S
    return 4 * rows * w.Hkv * w.D * e + 16 * (w.B + 1)


def cpu_baseline(w, a, c, el, budget_s):
    """The fp64 oracle on a bounded sample of the same step: whole sequences
    (attention of all heads + commit of all positions) until ``budget_s`` of
    CPU time is spent, scaled to the full batch by context length (attention)
    and by sequence count (commit)."""
    import numpy as np
    import oracle
    import synth
    threads = blas_threads()
    f64 = synth.bf16_bits_to_f64
    t_attn = t_commit = 0.0
    keys = 0
    n = 0
    order = np.random.default_rng(0).permutation(w.B)
    for b in order:
        lo, hi = int(a["offsets"][b]), int(a["offsets"][b + 1])
        t0 = time.perf_counter()
        oracle.block_attention(f64(a["q"][b:b + 1]), f64(a["k_blk"][b:b + 1]), f64(a["v_blk"][b:b + 1]),
                               f64(a["k_ctx"][lo:hi]), f64(a["v_ctx"][lo:hi]), np.array([0, hi - lo]))
        t1 = time.perf_counter()
        oracle.confidence_commit(f64(c["logits"][b:b + 1]), el[b:b + 1], w.gamma)
        t2 = time.perf_counter()
        t_attn += t1 - t0
        t_commit += t2 - t1
        keys += hi - lo + w.S
        n += 1
        if t_attn + t_commit >= budget_s:
            break
    total_keys = int(a["lengths"].sum()) + w.B * w.S
    step_s = t_attn * total_keys / keys + t_commit * w.B / n
    return {"value": 1.0 / step_s, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} of {w.B} sequences (attention of all 32 heads + commit of all "
                      f"{w.S} positions), {t_attn + t_commit:.1f} s of fp64 numpy; scaled to the "
                      f"batch by context keys (attention) and sequence count (commit)",
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": cpu_model()}


def blas_threads():
    """Threads the oracle's numpy BLAS calls use on this host."""
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def block_loop(args, L):
    """The full block-denoising loop on the loop workload: for each (S, gamma),
    td_denoise_step repeats until no position is masked.  Per-step logits come
    from the seeded loop generator (only each row's peak logit changes between
    steps; the update runs between the timed steps).  Reports steps per block
    and committed tokens/s over the timed steps."""
    import numpy as np
    import torch
    import block_diffusion_lm_td_amd as td
    from block_diffusion_lm_td_amd import _td
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    CHUNK = 8
    for S in (16, 32, 64):
        w0 = synth.WORKLOADS["bf16_b32_ctx2k_loop"].with_(S=S)
        a = synth.make_attention_inputs(w0, args.seed + S)
        att = {k: up(a[k]) for k in ("q", "k_blk", "v_blk", "k_ctx", "v_ctx")}
        off = torch.from_numpy(a["offsets"]).to(dev)
        out = torch.empty_like(att["q"])
        for gamma in (0.5, 0.8, 0.95):
            w = w0.with_(gamma=gamma)
            log(f"[loop] S={S} gamma={gamma}: generating logits")
            base, peak, stored = synth.loop_peak_values(w, args.seed + 100 * S, S + 1)
            logits = up(base).view(w.B, w.S, w.V)
            rows = torch.arange(w.B * w.S, device=dev)
            peak_d = torch.from_numpy(peak).to(dev)
            stored_d = up(stored)
            B = w.B
            o = dict(commit=torch.empty((B, S), dtype=torch.uint8, device=dev),
                     token=torch.empty((B, S), dtype=torch.int32, device=dev),
                     maxprob=torch.empty((B, S), dtype=torch.float32, device=dev),
                     n_commit=torch.empty((B,), dtype=torch.int32, device=dev),
                     masked_in=torch.ones((B, S), dtype=torch.uint8, device=dev),
                     masked_out=torch.empty((B, S), dtype=torch.uint8, device=dev),
                     tokens=torch.full((B, S), -1, dtype=torch.int32, device=dev),
                     n_left=torch.empty((1,), dtype=torch.int32, device=dev))
            aa = td.attn_args(att["q"], att["k_blk"], att["v_blk"], att["k_ctx"], att["v_ctx"], off, out,
                              a["total_ctx"], a["max_ctx"])
            cc = td.commit_args(logits, o["commit"], o["token"], gamma, o["masked_in"], o["maxprob"],
                                o["n_commit"], o["masked_out"], o["tokens"], o["n_left"])
            need = L.td_denoise_workspace_bytes(ctypes.byref(aa), ctypes.byref(cc))
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
            wsp = ctypes.c_void_p(ws.data_ptr())

            def run_block(timed):
                o["masked_in"].fill_(1)
                o["tokens"].fill_(-1)
                done_at = np.zeros(B, np.int64)
                ms = 0.0
                steps = 0
                torch.cuda.synchronize()
                t_wall = time.perf_counter()
                while True:
                    logits.view(-1, w.V)[rows, peak_d] = stored_d[steps]
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    r = L.td_denoise_step(ctypes.byref(aa), ctypes.byref(cc), wsp, ws.numel(), sp)
                    e1.record(stream)
                    if r != 0:
                        raise RuntimeError(_td.status_str(r))
                    torch.cuda.synchronize()
                    ms += e0.elapsed_time(e1)
                    steps += 1
                    left = o["masked_out"].view(B, S).sum(dim=1).cpu().numpy()
                    done_at[(left == 0) & (done_at == 0)] = steps
                    if int(o["n_left"].item()) == 0:
                        break
                    if steps >= S:
                        raise RuntimeError("a block did not finish within S steps")
                    o["masked_in"].copy_(o["masked_out"])
                return steps, done_at, ms, (time.perf_counter() - t_wall) * 1e3

            # the same loop resident on the device: steps of td_denoise_step_if, each
            # gated by the previous step's n_masked_left (two counters used
            # alternately), masks updated in place.  Steps go out in chunks of
            # CHUNK with one synchronisation per chunk: a gated-off step still
            # costs the dispatch of its kernels, so enqueueing all S at once would
            # pay for up to S - 1 of them.
            cnt = torch.zeros((2,), dtype=torch.int32, device=dev)
            cd = [td.commit_args(logits, o["commit"], o["token"], gamma, o["masked_in"],
                                 o["maxprob"], o["n_commit"], o["masked_in"], o["tokens"],
                                 cnt[k:k + 1]) for k in range(2)]
            gates = [ctypes.c_void_p(cnt[k:k + 1].data_ptr()) for k in range(2)]

            def run_block_device():
                o["masked_in"].fill_(1)
                o["tokens"].fill_(-1)
                cnt.fill_(0)
                cnt[1] = 1
                torch.cuda.synchronize()
                t_wall = time.perf_counter()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                k = 0
                while k < S:
                    for _ in range(min(CHUNK, S - k)):
                        logits.view(-1, w.V)[rows, peak_d] = stored_d[k]
                        r = L.td_denoise_step_if(ctypes.byref(aa), ctypes.byref(cd[k % 2]),
                                                 gates[(k + 1) % 2], wsp, ws.numel(), sp)
                        if r != 0:
                            raise RuntimeError(_td.status_str(r))
                        k += 1
                    if int(cnt[(k + 1) % 2].item()) == 0:     # the last step's n_masked_left
                        break
                e1.record(stream)
                torch.cuda.synchronize()
                wall = (time.perf_counter() - t_wall) * 1e3
                if int(o["masked_in"].sum().item()) != 0:
                    raise RuntimeError("the device-resident loop left positions masked")
                return e0.elapsed_time(e1), wall

            run_block(False)                       # warm-up pass
            steps, done_at, ms, wall_host = run_block(True)
            tokens_host = o["tokens"].clone()
            run_block_device()                     # warm-up pass
            dev_ms, dev_wall = run_block_device()
            if not torch.equal(o["tokens"], tokens_host):
                raise RuntimeError("device-resident loop committed different tokens")
            committed = B * S
            print(json.dumps({
                "metric": "block loop: steps per block and committed tokens/s",
                "workload": w.name, "B": B, "S": S, "gamma": gamma, "ctx_len": w.ctx_lo, "V": w.V,
                "dtype": w.dtype, "data": "synthetic",
                "loop_steps": steps, "steps_per_block_mean": round(float(done_at.mean()), 3),
                "steps_per_block_max": int(done_at.max()),
                "ms_total": round(ms, 4), "ms_per_step": round(ms / steps, 5),
                "committed_tokens_per_s": round(committed / (ms * 1e-3), 1),
                "host_driven_wall_ms": round(wall_host, 4),
                "device_resident": {"chunk": CHUNK, "gpu_ms": round(dev_ms, 4),
                                    "wall_ms": round(dev_wall, 4),
                                    "committed_tokens_per_s": round(committed / (dev_wall * 1e-3), 1)}}),
                  flush=True)
            del logits, stored_d, ws


def cache_append_bench(args, L):
    """td_cache_append on the batched workload's cache: the 64 sequences'
    1K..8K cached rows (2 KV heads x 128 bf16, K and V) grow by the block's 16
    rows into a second cache.  Rotating input/output sets keep the 256 MB
    last-level cache from serving a launch out of the previous one.  Prints
    one JSON line: appends/s, the roofline of the copy kernel and the oracle's
    rate on the host."""
    import numpy as np
    import torch
    import block_diffusion_lm_td_amd as td
    from block_diffusion_lm_td_amd import _td
    import synth

    w = synth.WORKLOADS[args.workload]
    if args.block_size:
        w = w.with_(S=args.block_size, name=f"{w.name}_s{args.block_size}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[append] generating {w.name}")
    a = synth.make_attention_inputs(w, args.seed)
    T, B, S = int(a["total_ctx"]), w.B, w.S
    N = T + B * S

    def up(x):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    base = {k: up(a[k]) for k in ("k_ctx", "v_ctx", "k_blk", "v_blk")}
    off = torch.from_numpy(a["offsets"]).to(dev)
    alg = append_algorithmic(w, T)
    nsets = args.sets or max(2, int(np.ceil(1.5e9 / alg)))
    sets = []
    for i in range(nsets):
        st = base if i == 0 else {k: v.clone() for k, v in base.items()}
        k_out = torch.empty((N, w.Hkv, w.D), dtype=st["k_ctx"].dtype, device=dev)
        o = dict(k_out=k_out, v_out=torch.empty_like(k_out),
                 off_out=torch.empty((B + 1,), dtype=torch.int64, device=dev))
        p = td.append_args(st["k_ctx"], st["v_ctx"], off, T, st["k_blk"], st["v_blk"],
                           o["k_out"], o["v_out"], o["off_out"])
        sets.append((st, o, p))
    refs = [ctypes.byref(p) for _, _, p in sets]
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    log(f"[append] {nsets} sets, {alg / 1e6:.1f} MB moved per append")

    def run(i):
        r = L.td_cache_append(refs[i % nsets], sp)
        if r != 0:
            raise RuntimeError(_td.status_str(r))

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        run(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_back_to_back = t0.elapsed_time(t1) / args.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps)]
    for i in range(args.steps):
        ev[2 * i].record(stream)
        run(i)
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    launch_ms = float(np.mean([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(args.steps)]))
    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    want_off = a["offsets"] + S * np.arange(B + 1)
    if not np.array_equal(sets[0][1]["off_out"].cpu().numpy(), want_off):
        raise RuntimeError("td_cache_append wrote unexpected offsets")
    achieved = alg / (launch_ms * 1e-3) / 1e9
    res = {
        "metric": "context-cache append: appends/s and % of HBM roofline, 1 GPU",
        "value": round(1e3 / ms_back_to_back, 2), "unit": "appends/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_append": round(ms_back_to_back, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name + "_append", "B": B, "S_appended": S, "Hkv": w.Hkv, "D": w.D,
                   "ctx_len": f"uniform integer in [{w.ctx_lo}, {w.ctx_hi}]", "total_ctx": T,
                   "rows_out": N, "sets": nsets},
        "roofline": {"bound": "hbm", "kernel": "td_cache_append (cache_append_rows)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(w.name, APPEND_SRC, APPEND_TRAFFIC_FILE),
                     "algorithmic_bytes": alg, "avg_launch_us": round(launch_ms * 1e3, 2)},
    }
    if not args.no_cpu_baseline:
        import oracle
        n, spent = 0, 0.0
        while spent < args.cpu_budget:
            c0 = time.perf_counter()
            oracle.cache_append(a["k_ctx"], a["v_ctx"], a["offsets"], a["k_blk"], a["v_blk"])
            spent += time.perf_counter() - c0
            n += 1
        res["cpu_baseline"] = {"value": round(n / spent, 3), "unit": "appends/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{n} whole appends of the same cache (numpy "
                                         f"concatenation, {spent:.1f} s)",
                               "cpu_model": cpu_model()}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


LMHEAD_SRC = os.path.join(ROOT, "block_diffusion_lm_td_amd", "csrc", "td_lmhead.hip")
LMHEAD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lmhead_traffic_lmhead_bf16_b64_h4096_v131072.json")
LMHEAD_PACKED_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lmhead_traffic_lmhead_bf16_b64_h4096_v131072_packed.json")


def lmhead_bench(args, L):
    """td_lmhead_commit on the batched step's 64 x 16 positions with a 4096 x
    131072 bf16 head: one JSON line.  value = fused steps/s with every
    position still masked (a block's first step); the same call with 50 / 25 /
    10 % of the positions still masked (later steps) is reported beside it,
    and so is the unfused route timed in the same run (the library GEMM of
    torch writing bf16 logits, then td_commit) for reference."""
    import numpy as np
    import torch
    import block_diffusion_lm_td_amd as td
    from block_diffusion_lm_td_amd import _td
    import synth

    w = synth.LMHEAD_WORKLOADS["lmhead_bf16_b64_h4096_v131072"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[lmhead] generating {w.name}")
    d = synth.make_lmhead_inputs(w, args.seed)
    B, S, H, V = w.B, w.S, w.H, w.V
    hid = torch.from_numpy(d["hidden"].view(np.int16)).view(torch.bfloat16).to(dev)
    wh = torch.from_numpy(d["w_head"].view(np.int16)).view(torch.bfloat16).to(dev)
    pack_us = None
    if args.packed:
        # the one-time rearrangement at load time, timed on its own
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        wh_packed = td.td_lmhead_pack_head(wh)
        e1.record()
        torch.cuda.synchronize()
        pack_us = round(e0.elapsed_time(e1) * 1e3, 1)
        wh_row_major, wh = wh, wh_packed
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    o = dict(commit=torch.empty((B, S), dtype=torch.uint8, device=dev),
             token=torch.empty((B, S), dtype=torch.int32, device=dev),
             maxprob=torch.empty((B, S), dtype=torch.float32, device=dev),
             n_commit=torch.empty((B,), dtype=torch.int32, device=dev),
             masked_out=torch.empty((B, S), dtype=torch.uint8, device=dev),
             n_left=torch.empty((1,), dtype=torch.int32, device=dev))
    rng = np.random.default_rng([args.seed, 11])
    flops_per_row = 2.0 * H * V

    def timed(call, n):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
        for i in range(n):
            ev[2 * i].record(stream)
            call()
            ev[2 * i + 1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n)]))

    rows = {}
    for frac in [float(x) for x in args.fracs.split(",")]:
        m = (rng.random((B, S)) < frac).astype(np.uint8) if frac < 1.0 else np.ones((B, S), np.uint8)
        mi = torch.from_numpy(m).to(dev)
        a = td.lmhead_args(hid, wh, o["commit"], o["token"], w.gamma, mi, o["maxprob"], o["n_commit"],
                           o["masked_out"], None, o["n_left"])
        need = L.td_lmhead_commit_workspace_bytes(ctypes.byref(a))
        ws = torch.empty(need, dtype=torch.uint8, device=dev)

        def call():
            r = L.td_lmhead_commit(ctypes.byref(a), ctypes.c_void_p(ws.data_ptr()), need, sp)
            if r != 0:
                raise RuntimeError(_td.status_str(r))
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(args.steps):
            call()
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        launch_ms = timed(call, args.steps)
        n_rows = int(m.sum())
        rows[frac] = dict(eligible_positions=n_rows, ms_per_step=round(ms, 5),
                          avg_launch_us=round(launch_ms * 1e3, 2),
                          tflops=round(n_rows * flops_per_row / (launch_ms * 1e-3) / 1e12, 1),
                          committed=int(o["n_commit"].sum().item()))
        log(f"[lmhead] eligible {n_rows}: {ms * 1e3:.1f} us/step")

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # the unfused route, for reference: bf16 logits from the library GEMM, then td_commit
    logits = torch.empty((B, S, V), dtype=torch.bfloat16, device=dev)
    c = td.commit_args(logits, o["commit"], o["token"], w.gamma, None, o["maxprob"])
    cneed = max(L.td_commit_workspace_bytes(ctypes.byref(c)), 256)
    cws = torch.empty(cneed, dtype=torch.uint8, device=dev)
    wht = (wh_row_major if args.packed else wh).t()

    def unfused():
        torch.matmul(hid.view(B * S, H), wht, out=logits.view(B * S, V))
        r = L.td_commit(ctypes.byref(c), ctypes.c_void_p(cws.data_ptr()), cneed, sp)
        if r != 0:
            raise RuntimeError(_td.status_str(r))
    for _ in range(args.warmup):
        unfused()
    unfused_ms = timed(unfused, args.steps)
    del logits

    full = rows[max(rows)]
    achieved = full["tflops"]
    res = {
        "metric": "fused LM head + commit: steps/s (64 x 16 positions, H 4096, V 131072) and % of "
                  "bf16 MFMA roofline, 1 GPU",
        "value": round(1e3 / full["ms_per_step"], 2), "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": full["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "S": S, "H": H, "V": V, "gamma": w.gamma,
                   "w_head": "packed (td_lmhead_pack_head, once: %s us)" % pack_us if args.packed
                   else "row-major [V, H]",
                   "hidden_size": "assumed (not on the pages)"},
        "roofline": {"bound": "mfma", "kernel": "td_lmhead_commit (lmhead_tiles + merge + finalize)",
                     "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": (measured_traffic(w.name + "_packed", LMHEAD_SRC, LMHEAD_PACKED_TRAFFIC_FILE)
                                 if args.packed else measured_traffic(w.name, LMHEAD_SRC, LMHEAD_TRAFFIC_FILE)),
                     "algorithmic_flops": B * S * flops_per_row,
                     "avg_launch_us": full["avg_launch_us"]},
        "by_eligible_fraction": {str(k): v for k, v in rows.items()},
        "unfused_reference_us": round(unfused_ms * 1e3, 2),
    }
    if not args.no_cpu_baseline:
        import oracle
        f64 = synth.bf16_bits_to_f64
        c0 = time.perf_counter()
        wf = f64(d["w_head"])
        n, spent = 0, time.perf_counter() - c0
        while spent < args.cpu_budget and n < B:
            c0 = time.perf_counter()
            oracle.lmhead_commit(f64(d["hidden"][n:n + 1]), wf, None, w.gamma)
            spent += time.perf_counter() - c0
            n += 1
        res["cpu_baseline"] = {"value": round(n / (B * spent), 5), "unit": "steps/s",
                               "cores": blas_threads(), "kind": "oracle",
                               "sample": f"{n} of {B} sequences (all {S} positions over the full "
                                         f"vocabulary, fp64 numpy), {spent:.1f} s including the "
                                         f"head's conversion; scaled to the batch by sequence count",
                               "cpu_model": cpu_model()}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


MAMBA_SRC = os.path.join(ROOT, "block_diffusion_lm_td_amd", "csrc", "td_mamba.hip")
MAMBA_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mamba_traffic_mamba_b64_s16_h128.json")


def mamba_algorithmic(w):
    """Bytes one block scan must move: the fp32 seed state, x and y (bf16),
    Bm and Cm (bf16), dt (fp32) and the per-head A and D."""
    return (w.B * w.H * w.P * w.N * 4 + 2 * w.B * w.S * w.H * w.P * 2
            + 2 * w.B * w.S * w.G * w.N * 2 + w.B * w.S * w.H * 4 + 2 * w.H * 4)


def mamba_bench(args, L):
    """td_mamba_block_scan on the batched block: 64 sequences x 128 heads of
    64 with a 128-wide state (8 groups), S = 16, seeded from fp32 states.
    One JSON line; rotating input sets keep the 256 MB last-level cache from
    serving the seed states of the previous launch."""
    import numpy as np
    import torch
    import block_diffusion_lm_td_amd as td
    from block_diffusion_lm_td_amd import _td
    import synth

    w = synth.MAMBA_WORKLOADS["mamba_b64_s16_h128"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[mamba] generating {w.name}")
    d = synth.make_mamba_inputs(w, args.seed)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    alg = mamba_algorithmic(w)
    nsets = args.sets or max(2, int(np.ceil(1.5e9 / alg)))
    base = dict(x=bf(d["x"]), dt=f32(d["dt"]), A=f32(d["A"]), Bm=bf(d["Bm"]), Cm=bf(d["Cm"]),
                D=f32(d["D"]), h0=f32(d["h0"]))
    structs = []
    keep = []
    for i in range(nsets):
        st = base if i == 0 else {k: v.clone() for k, v in base.items()}
        y = torch.empty((w.B, w.S, w.H, w.P), dtype=torch.bfloat16, device=dev)
        keep.append((st, y))
        structs.append(td.mamba_args(st["x"], st["dt"], st["A"], st["Bm"], st["Cm"], st["D"], st["h0"], y))
    refs = [ctypes.byref(a) for a in structs]
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)

    def run(i):
        r = L.td_mamba_block_scan(refs[i % nsets], sp)
        if r != 0:
            raise RuntimeError(_td.status_str(r))

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        run(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps)]
    for i in range(args.steps):
        ev[2 * i].record(stream)
        run(i)
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    launch_ms = float(np.mean([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(args.steps)]))
    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    achieved = alg / (launch_ms * 1e-3) / 1e9
    res = {
        "metric": "Mamba-2 block scans/s (64 x 128 heads, S 16, seeded state) and % of HBM "
                  "roofline, 1 GPU",
        "value": round(1e3 / ms, 2), "unit": "scans/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_scan": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "S": w.S, "H": w.H, "P": w.P, "N": w.N, "G": w.G,
                   "dims": "assumed (not on the pages)", "sets": nsets},
        "roofline": {"bound": "hbm", "kernel": "td_mamba_block_scan (mamba_block)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(w.name, MAMBA_SRC, MAMBA_TRAFFIC_FILE),
                     "algorithmic_bytes": alg, "avg_launch_us": round(launch_ms * 1e3, 2)},
    }
    if not args.no_cpu_baseline:
        import oracle
        f64 = synth.bf16_bits_to_f64
        n, spent = 0, 0.0
        while spent < args.cpu_budget and n < w.B:
            c0 = time.perf_counter()
            oracle.mamba_block_scan(f64(d["x"][n:n + 1]), d["dt"][n:n + 1], d["A"], f64(d["Bm"][n:n + 1]),
                                    f64(d["Cm"][n:n + 1]), d["D"], d["h0"][n:n + 1])
            spent += time.perf_counter() - c0
            n += 1
        res["cpu_baseline"] = {"value": round(n / (w.B * spent), 4), "unit": "scans/s",
                               "cores": blas_threads(), "kind": "oracle",
                               "sample": f"{n} of {w.B} sequences (all 128 heads, token by token, "
                                         f"fp64 numpy), {spent:.1f} s; scaled to the batch by "
                                         f"sequence count", "cpu_model": cpu_model()}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


ADALN_SRC = os.path.join(ROOT, "block_diffusion_lm_td_amd", "csrc", "td_adaln.hip")
ADALN_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "adaln_traffic_adaln_b64_s16_h4096.json")


def adaln_algorithmic(w):
    """Bytes one modulation call must move: x and f read, r and h written
    (bf16), each sequence's three timestep vectors and the four [H] rows
    (fp32)."""
    return 4 * w.B * w.S * w.H * 2 + 3 * w.B * w.H * 4 + 4 * w.H * 4


def adaln_bench(args, L):
    """td_adaln_modulate between two layers of the batched block: 64
    sequences x 16 tokens, hidden 4096, with the gated residual.  One JSON
    line; rotating input sets keep the last-level cache from serving the
    previous call's rows."""
    import numpy as np
    import torch
    import block_diffusion_lm_td_amd as td
    from block_diffusion_lm_td_amd import _td
    import synth

    w = synth.ADALN_WORKLOADS["adaln_b64_s16_h4096"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[adaln] generating {w.name}")
    d = synth.make_adaln_inputs(w, args.seed)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    alg = adaln_algorithmic(w)
    nsets = args.sets or max(2, int(np.ceil(1.5e9 / alg)))
    base = dict(x=bf(d["x"]), f=bf(d["f"]), t_mod=f32(d["t_mod"]), tab_gate=f32(d["tab_gate"]),
                tab_shift=f32(d["tab_shift"]), tab_scale=f32(d["tab_scale"]), w_norm=f32(d["w_norm"]))
    keep, structs = [], []
    for i in range(nsets):
        st = base if i == 0 else {k: v.clone() for k, v in base.items()}
        r_out = torch.empty_like(st["x"])
        h = torch.empty_like(st["x"])
        keep.append((st, r_out, h))
        structs.append(td.adaln_args(st["x"], st["f"], st["t_mod"], h, r_out, tab_gate=st["tab_gate"],
                                     tab_shift=st["tab_shift"], tab_scale=st["tab_scale"],
                                     w_norm=st["w_norm"], eps=1e-5))
    refs = [ctypes.byref(a) for a in structs]
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)

    def run(i):
        r = L.td_adaln_modulate(refs[i % nsets], sp)
        if r != 0:
            raise RuntimeError(_td.status_str(r))

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        run(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps)]
    for i in range(args.steps):
        ev[2 * i].record(stream)
        run(i)
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    launch_ms = float(np.mean([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(args.steps)]))
    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # one kernel per call, ~11 us: a pair of events around each launch adds
    # about 2 us, so the launch duration is the back-to-back average over the
    # timed region (the one-by-one figure is reported beside it)
    achieved = alg / (ms * 1e-3) / 1e9
    res = {
        "metric": "adaLN-single modulations/s (64 x 16 tokens, hidden 4096, gated residual + "
                  "modulated RMSNorm) and % of HBM roofline, 1 GPU",
        "value": round(1e3 / ms, 2), "unit": "calls/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_call": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "S": w.S, "H": w.H,
                   "dims": "assumed (not on the pages)", "sets": nsets},
        "roofline": {"bound": "hbm", "kernel": "td_adaln_modulate (adaln_rows)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(w.name, ADALN_SRC, ADALN_TRAFFIC_FILE),
                     "algorithmic_bytes": alg, "avg_launch_us": round(ms * 1e3, 2),
                     "avg_launch_us_one_by_one": round(launch_ms * 1e3, 2)},
    }
    if not args.no_cpu_baseline:
        import oracle
        f64 = synth.bf16_bits_to_f64
        n, spent = 0, 0.0
        while spent < args.cpu_budget and n < 50:
            c0 = time.perf_counter()
            oracle.adaln_modulate(f64(d["x"]), f64(d["f"]), d["t_mod"], d["tab_gate"], d["tab_shift"],
                                  d["tab_scale"], d["w_norm"], 1e-5)
            spent += time.perf_counter() - c0
            n += 1
        res["cpu_baseline"] = {"value": round(n / spent, 4), "unit": "calls/s",
                               "cores": blas_threads(), "kind": "oracle",
                               "sample": f"the whole batch {n} times (fp64 numpy), {spent:.1f} s",
                               "cpu_model": cpu_model()}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="bf16_b64_ragged1k_8k")
    ap.add_argument("--block-size", type=int, default=0,
                    help="override the workload's block size S (e.g. 32 or 64 on the loop "
                         "workload, where the attention is bound by the matrix cores)")
    ap.add_argument("--sets", type=int, default=0, help="rotating input sets (0: >= 1.5 GB total)")
    ap.add_argument("--seed", type=int, default=1003)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one 1 GiB device copy (counter calibration)")
    ap.add_argument("--loop", action="store_true",
                    help="block loop: S in {16,32,64} x gamma in {0.5,0.8,0.95}, steps until every "
                         "position is committed (one JSON line per case)")
    ap.add_argument("--hold", type=float, default=0.0,
                    help="run --hold-part back-to-back for this many seconds (for sampling board "
                         "power and clocks from outside), print one JSON line and exit")
    ap.add_argument("--hold-part", choices=("step", "attn", "commit"), default="attn")
    ap.add_argument("--lmhead", action="store_true",
                    help="time td_lmhead_commit (fused LM head + commit) instead of the step "
                         "(one JSON line)")
    ap.add_argument("--packed", action="store_true",
                    help="--lmhead: pass the head as td_lmhead_pack_head's packed copy")
    ap.add_argument("--fracs", default="1,0.5,0.25,0.1",
                    help="--lmhead: fractions of positions still masked to time (the first "
                         "is the headline)")
    ap.add_argument("--adaln", action="store_true",
                    help="time td_adaln_modulate instead of the step (one JSON line)")
    ap.add_argument("--mamba", action="store_true",
                    help="time td_mamba_block_scan instead of the step (one JSON line)")
    ap.add_argument("--append", action="store_true",
                    help="time td_cache_append on the workload's cache instead of the step "
                         "(one JSON line)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the denoise step of one attention layer is one "
              "GPU's share (sequences shard over GPUs with no exchange); --gpus above 1 is not "
              "supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_diffusion_lm_td_amd as td
    from block_diffusion_lm_td_amd import _td
    import synth

    L = td.lib()
    if args.loop:
        block_loop(args, L)
        return
    if args.append:
        cache_append_bench(args, L)
        return
    if args.lmhead:
        lmhead_bench(args, L)
        return
    if args.mamba:
        mamba_bench(args, L)
        return
    if args.adaln:
        adaln_bench(args, L)
        return
    w = synth.WORKLOADS[args.workload]
    if args.block_size:
        w = w.with_(S=args.block_size, name=f"{w.name}_s{args.block_size}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] generating {w.name}")
    a = synth.make_attention_inputs(w, args.seed)
    c = synth.make_commit_inputs(w, args.seed)
    el = np.ones((w.B, w.S), np.uint8)             # a fresh block: every position [MASK]

    def up(x):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    base = {k: up(a[k]) for k in ("q", "k_blk", "v_blk", "k_ctx", "v_ctx")}
    base["logits"] = up(c["logits"])
    off = torch.from_numpy(a["offsets"]).to(dev)
    set_bytes = sum(t.numel() * t.element_size() for t in base.values())
    nsets = args.sets or max(2, int(np.ceil(1.5e9 / set_bytes)))
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(nsets - 1)]
    B, S = w.B, w.S
    outs = []
    structs = []
    for st in sets:
        o = dict(out=torch.empty_like(st["q"]),
                 commit=torch.empty((B, S), dtype=torch.uint8, device=dev),
                 token=torch.empty((B, S), dtype=torch.int32, device=dev),
                 maxprob=torch.empty((B, S), dtype=torch.float32, device=dev),
                 n_commit=torch.empty((B,), dtype=torch.int32, device=dev),
                 masked_in=torch.from_numpy(el).to(dev),
                 masked_out=torch.empty((B, S), dtype=torch.uint8, device=dev),
                 tokens=torch.full((B, S), -1, dtype=torch.int32, device=dev),
                 n_left=torch.empty((1,), dtype=torch.int32, device=dev))
        aa = td.attn_args(st["q"], st["k_blk"], st["v_blk"], st["k_ctx"], st["v_ctx"], off, o["out"],
                          a["total_ctx"], a["max_ctx"])
        cc = td.commit_args(st["logits"], o["commit"], o["token"], w.gamma, o["masked_in"],
                            o["maxprob"], o["n_commit"], o["masked_out"], o["tokens"], o["n_left"])
        outs.append(o)
        structs.append((aa, cc))
    ws_bytes = max(L.td_denoise_workspace_bytes(ctypes.byref(aa), ctypes.byref(cc)) for aa, cc in structs)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    ws_ptr = ctypes.c_void_p(ws.data_ptr())
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    refs = [(ctypes.byref(aa), ctypes.byref(cc)) for aa, cc in structs]
    log(f"[bench] {nsets} input sets x {set_bytes / 1e6:.0f} MB, workspace {ws_bytes / 1e6:.1f} MB")

    def step(i):
        ra, rc = refs[i % nsets]
        r = L.td_denoise_step(ra, rc, ws_ptr, ws.numel(), sp)
        if r != 0:
            raise RuntimeError(_td.status_str(r))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    if args.hold > 0:
        call = {"step": lambda r: L.td_denoise_step(r[0], r[1], ws_ptr, ws.numel(), sp),
                "attn": lambda r: L.td_block_attn(r[0], ws_ptr, ws.numel(), sp),
                "commit": lambda r: L.td_commit(r[1], ws_ptr, ws.numel(), sp)}[args.hold_part]
        n, t0 = 0, time.time()
        while time.time() - t0 < args.hold:
            for i in range(500):
                r = call(refs[(n + i) % nsets])
                if r != 0:
                    raise RuntimeError(_td.status_str(r))
            torch.cuda.synchronize()
            n += 500
        dt = time.time() - t0
        print(json.dumps({"hold_part": args.hold_part, "workload": w.name, "launches": n,
                          "seconds": round(dt, 3), "us_per_launch": round(dt / n * 1e6, 2)}), flush=True)
        return

    # ---- timed region: K whole steps
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    log(f"[bench] {args.steps} steps in {total_ms:.3f} ms -> {ms_per_step * 1e3:.1f} us/step")

    # ---- per-part durations: each part on its own, after its own warm-up,
    # PART_LAUNCHES launches back to back between one pair of HIP events on
    # the launch stream (the average launch duration, as a kernel trace
    # reports it, plus the small gap between consecutive launches)
    def part_ms(call):
        for i in range(PART_WARMUP):
            call(refs[i % nsets])
        n = max(PART_LAUNCHES, args.steps)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            r = call(refs[i % nsets])
            if r != 0:
                raise RuntimeError(_td.status_str(r))
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    attn_ms = part_ms(lambda r: L.td_block_attn(r[0], ws_ptr, ws.numel(), sp))
    commit_ms = part_ms(lambda r: L.td_commit(r[1], ws_ptr, ws.numel(), sp))
    log(f"[bench] td_block_attn {attn_ms * 1e3:.1f} us, td_commit {commit_ms * 1e3:.1f} us "
        f"(back to back, after {PART_WARMUP} warm-up launches each)")

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- committed tokens per step (every set holds the same data)
    step(0)
    torch.cuda.synchronize()
    committed = int(outs[0]["n_commit"].sum().item())

    attn_bytes, attn_flops, commit_bytes = algorithmic(w, a["lengths"])
    achieved = attn_bytes / (attn_ms * 1e-3) / 1e9
    # the attention's bound by the roofline: matrix cores when its algorithmic
    # intensity exceeds the ridge of the bf16 MFMA and HBM peaks
    mfma_bound = attn_flops / attn_bytes > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    mfma_tfs = attn_flops / (attn_ms * 1e-3) / 1e12
    # decode-shaped blocks run attn_decode (the same rule as the library's plan)
    decode = w.dtype == "bf16" and w.D == 128 and w.G * w.S <= 16 and w.B <= 4096
    traffic = measured_traffic(w.name, DECODE_SRC if decode else ATTN_SRC,
                               os.path.join(ROOT, "profiles", f"attn_traffic_{w.name}.json"))
    steps_per_s = 1e3 / ms_per_step
    res = {
        "metric": METRIC,
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "S": S, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
                   "ctx_len": f"uniform integer in [{w.ctx_lo}, {w.ctx_hi}]" if w.ctx_lo != w.ctx_hi
                   else w.ctx_lo, "total_ctx": int(a["total_ctx"]), "V": w.V, "gamma": w.gamma,
                   "input_sets": nsets},
        "tokens_per_s": round(committed * steps_per_s, 1),
        "committed_per_step": committed,
        "roofline": {"bound": "mfma" if mfma_bound else "hbm",
                     "kernel": "td_block_attn (attn_decode + decode_merge)"
                     if decode else "td_block_attn (attn_bf16_mfma + attn_merge)",
                     "achieved": round(mfma_tfs if mfma_bound else achieved, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBS,
                     "unit": "TFLOP/s" if mfma_bound else "GB/s",
                     "frac": round(mfma_tfs / MFMA_BF16_PEAK_TFLOPS if mfma_bound
                                   else achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes": attn_bytes, "algorithmic_flops": attn_flops,
                     "avg_launch_us": round(attn_ms * 1e3, 2),
                     "hbm_GBs": round(achieved, 1), "hbm_frac": round(achieved / HBM_PEAK_GBS, 4),
                     "mfma_tflops": round(mfma_tfs, 1),
                     "mfma_frac": round(mfma_tfs / MFMA_BF16_PEAK_TFLOPS, 4)},
        "commit": {"avg_launch_us": round(commit_ms * 1e3, 2), "algorithmic_bytes": commit_bytes,
                   "achieved_GBs": round(commit_bytes / (commit_ms * 1e-3) / 1e9, 1)},
        "step_roofline_frac": round((attn_bytes + commit_bytes) / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host")
        res["cpu_baseline"] = cpu_baseline(w, a, c, el, args.cpu_budget)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
