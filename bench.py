#!/usr/bin/env python3
"""Decode throughput of the batched single-token decode step on one MI355X.

Default workload: the Llama-3-8B-shaped Q4 decoder (32 layers, hidden 4096,
32 Q / 8 KV heads, head_dim 128, intermediate 14336, vocab 128256), M = 32
sequences at positions drawn uniformly from [2048, 4096] over a synthetic
fp32 KV context, greedy decoding with the whole step -- embedding gather, every
layer, LM head, argmax, position advance -- replayed as one captured HIP graph.
A step is one decode token for all 32 sequences; tok/s = M * steps / time.

Also reported: the M = 1 line (Qwen2.5-0.5B-shaped Q8 decoder after a
512-token teacher-forced context, 256 greedy steps), the HBM roofline of the
dominant kernel (split-K flash decoding, timed alone with HIP events on the
stream it runs on), the FP8 and Q6K block formats on the GEMV at the LM-head
shape, prompt ingestion, an M sweep of the 1.5B-shaped decoder, the standalone
attention workload at every split size, a practical HBM ceiling, and the CPU
oracle's speed on a bounded sample.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-m1", action="store_true", help="skip the M=1 line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fd-reps", type=int, default=20)
    ap.add_argument("--only-m1", action="store_true", help="run only the M=1 line")
    ap.add_argument("--only-attention", action="store_true",
                    help="run only the standalone flash-decode line and the HBM ceiling")
    ap.add_argument("--m1-steps", type=int, default=256)
    ap.add_argument("--m1-ctx", type=int, default=512, help="context tokens of the M=1 line")
    ap.add_argument("--no-sweep", action="store_true", help="skip the 1.5B-shaped M sweep")
    ap.add_argument("--fixed-plans", action="store_true",
                    help="flash decode at the library's default split rule instead of autotuned "
                         "plans (deterministic launch shapes, for counter runs)")
    ap.add_argument("--only-gemv-ab", action="store_true",
                    help="run only the matrix-core vs vector-ALU GEMV comparison")
    ap.add_argument("--only-prefill", action="store_true",
                    help="run only the 8B-shaped 512-token prefill line, for profiling")
    ap.add_argument("--only-sweep", default="",
                    help="run only the 1.5B-shaped M sweep at these batch sizes (e.g. 1,8,32), "
                         "for profiling")
    ap.add_argument("--main-only", action="store_true",
                    help="only the M=32 step and the flash-decode roofline (no M=1, FP8, "
                         "prefill or sweep lines), for profiling")
    ap.add_argument("--gemv-only", action="store_true",
                    help="only the gate/up-shaped Q4 GEMV (28672 x 4096) at M=32 and M=1, "
                         "for counter runs")
    ap.add_argument("--fd-only", action="store_true",
                    help="run only the flash-decode launches (layer-sized synthetic cache at the "
                         "workload's lengths) and a plain copy of known size, for counter runs")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def timed_greedy(dd, S, m, first_tok, start_pos, steps, warmup):
    """Warm up (first call captures the graph), rewind, then time `steps`
    graph replays.  Returns (seconds, final positions)."""
    import quantized_gemv_flash_amd as rra
    dev = "cuda"
    x = torch.empty((m, S.hidden), device=dev)
    pos = torch.empty(m, dtype=torch.int32, device=dev)
    tok = torch.empty(m, dtype=torch.int32, device=dev)
    logits = torch.empty((m, S.vocab), device=dev)
    flags = rra.RRA_GRAPH | rra.RRA_STEP_GATHER | rra.RRA_STEP_ADVANCE
    start_pos_t = torch.as_tensor(start_pos, dtype=torch.int32, device=dev)
    first_t = torch.as_tensor(first_tok, dtype=torch.int32, device=dev)
    pos.copy_(start_pos_t)
    tok.copy_(first_t)
    for _ in range(max(1, warmup)):
        dd.model.rra_decode_step(x, pos, tok, m, flags=flags, logits=logits)
    # rewind: the timed steps overwrite the cache rows the warm-up wrote
    pos.copy_(start_pos_t)
    tok.copy_(first_t)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        dd.model.rra_decode_step(x, pos, tok, m, flags=flags, logits=logits)
    ev1.record()
    torch.cuda.synchronize()
    dd.model.rra_model_check()
    return ev0.elapsed_time(ev1) / 1e3, pos.tolist(), tok.tolist()


def host_handoff_line(dd, S, m, first_tok, start_pos, steps):
    """Host-visible tok/s of the same greedy steps when the host receives every
    step's ids (wall clock from the first enqueue to the last ids in host
    memory): blocking (rra_decode_step with tok_host: one stream sync per step)
    against pipelined (rra_decode_step_async into two pinned buffers with a
    completion event each, the host reading step t's ids while step t+1 runs)."""
    import quantized_gemv_flash_amd as rra
    dev = "cuda"
    x = torch.empty((m, S.hidden), device=dev)
    pos = torch.empty(m, dtype=torch.int32, device=dev)
    tok = torch.empty(m, dtype=torch.int32, device=dev)
    logits = torch.empty((m, S.vocab), device=dev)
    flags = rra.RRA_GRAPH | rra.RRA_STEP_GATHER | rra.RRA_STEP_ADVANCE
    start_t = torch.as_tensor(start_pos, dtype=torch.int32, device=dev)
    first_t = torch.as_tensor(first_tok, dtype=torch.int32, device=dev)

    def rewind():
        pos.copy_(start_t)
        tok.copy_(first_t)
        torch.cuda.synchronize()

    rewind()
    dd.model.rra_decode_step(x, pos, tok, m, flags=flags, logits=logits)  # capture
    rewind()
    t0 = time.perf_counter()
    blocking = [dd.model.rra_decode_step(x, pos, tok, m, flags=flags, logits=logits, tok_host=True)
                for _ in range(steps)]
    t_block = time.perf_counter() - t0
    bufs = [torch.empty(m, dtype=torch.int32, pin_memory=True) for _ in range(2)]
    evs = [torch.cuda.Event() for _ in range(2)]
    for e in evs:
        e.record()
    rewind()
    piped = []
    t0 = time.perf_counter()
    for t in range(steps + 1):
        if t < steps:
            dd.model.rra_decode_step_async(x, pos, tok, bufs[t % 2], evs[t % 2], m, flags=flags,
                                           logits=logits)
        if t >= 1:
            evs[(t - 1) % 2].synchronize()
            piped.append(bufs[(t - 1) % 2].tolist())
    t_pipe = time.perf_counter() - t0
    assert piped == blocking, "pipelined ids differ from the blocking path's"
    return dict(steps=steps, blocking_tok_s=m * steps / t_block,
                pipelined_tok_s=m * steps / t_pipe, ids_equal=True)


def build_decoder(S, m, max_len, seed=0):
    import synth
    from quantized_gemv_flash_amd.loader import load_decoder
    W = synth.decoder_weights(S, seed=seed, device="cuda")
    dd = load_decoder(S, W, m_max=m, max_len=max_len)
    return W, dd


def fill_kv_context(S, dd, lengths, seed=0):
    import synth
    for l in range(S.n_layers):
        for s, L in enumerate(lengths):
            k, v = synth.kv_context_rows(S, l, s, L, seed=seed, device="cuda")
            dd.k_caches[l][s, :, :L] = k
            dd.v_caches[l][s, :, :L] = v
            del k, v


def graph_time(fn, reps):
    """Seconds per call of fn (enqueue-only, on the current stream), timed as
    one replay of a HIP graph holding `reps` calls, so that the time is the
    kernels' own and not the gaps between eager launches."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    g.replay()
    ev1.record()
    torch.cuda.synchronize()
    del g
    return ev0.elapsed_time(ev1) / 1e3 / reps


def flash_decode_roofline(S, dd, lens, reps, plan=None):
    """Times rra_flash_decode (split-K chunk kernel + its reduce) alone on
    layer 0's cache at the step's sequence lengths, with the step's plan
    (chunk, head split) when given, else the default rule."""
    import quantized_gemv_flash_amd as rra
    m, nq, nkv, hd = len(lens), S.n_heads, S.n_kv_heads, S.head_dim
    max_len = dd.k_caches[0].shape[2]
    q = torch.randn((m, nq, hd), device="cuda")
    out = torch.empty_like(q)
    seq = torch.as_tensor(lens, dtype=torch.int32, device="cuda")
    chunk = plan[0] if plan else rra.rra_flash_decode_chunk(m, nkv, max_len, 0)
    ws = torch.empty(rra.rra_flash_decode_workspace_bytes(m, nq, nkv, hd, max_len, 0),
                     dtype=torch.uint8, device="cuda")
    if plan and plan[1] > 0:
        args = (q, dd.k_caches[0], dd.v_caches[0], seq, out, m, nq, nkv, hd, max_len, plan[0],
                plan[1], ws)
        sec = graph_time(lambda: rra.rra_flash_decode_ex(*args), reps)
    else:
        args = (q, dd.k_caches[0], dd.v_caches[0], seq, out, m, nq, nkv, hd, max_len, chunk, ws)
        sec = graph_time(lambda: rra.rra_flash_decode(*args), reps)
    kv_bytes = sum(2 * nkv * L * hd * 4 for L in lens)  # K and V rows read once
    return sec, kv_bytes, chunk


def flash_decode_in_step(S, dd, m, first_tok, start_pos, steps):
    """Flash decode's chunk kernel timed inside the decode step: the same
    greedy steps from the same start, run eagerly, with a pair of HIP events
    per layer that the runtime stamps at the start and end of that layer's
    split-K chunk kernel on the step's stream (rra_model_set_attention_events,
    hipExtLaunchKernel).  Returns (seconds and algorithmic K/V
    bytes summed over every layer of every step, the final positions)."""
    import quantized_gemv_flash_amd as rra
    dev = "cuda"
    cur = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * S.n_layers)]
    for e in evs:
        e.record(cur)  # creates the event
    x = torch.empty((m, S.hidden), device=dev)
    pos = torch.as_tensor(start_pos, dtype=torch.int32, device=dev)
    tok = torch.as_tensor(first_tok, dtype=torch.int32, device=dev)
    logits = torch.empty((m, S.vocab), device=dev)
    flags = rra.RRA_STEP_GATHER | rra.RRA_STEP_ADVANCE
    dd.model.rra_model_set_attention_events(evs)
    sec = nbytes = 0.0
    try:
        for i in range(steps):
            dd.model.rra_decode_step(x, pos, tok, m, flags=flags, logits=logits)
            torch.cuda.synchronize()
            sec += sum(evs[2 * l].elapsed_time(evs[2 * l + 1]) for l in range(S.n_layers)) / 1e3
            # rows read this step: every cached row up to and including position start + i
            nbytes += S.n_layers * sum(2 * S.n_kv_heads * (L + i + 1) * S.head_dim * 4
                                       for L in start_pos)
    finally:
        dd.model.rra_model_set_attention_events(None)
    dd.model.rra_model_check()
    return sec, nbytes, pos.tolist()


def phase_line(S, dd, m, first_tok, start_pos, steps=4):
    """The decode step split into its kernel groups ([reduces]
    forward_graphed_replay_to_token_id: a step's time in sub-phases on
    request): `steps` eager steps from the same start, with
    rra_model_set_phase_events recording a HIP event between the groups on
    the step's stream.  Returns ms per step of each group summed over the
    layers (launch gaps included: eager, not graph-replayed)."""
    import quantized_gemv_flash_amd as rra
    dev = "cuda"
    cur = torch.cuda.current_stream()
    n = 4 * S.n_layers + 3
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record(cur)
    x = torch.empty((m, S.hidden), device=dev)
    pos = torch.as_tensor(start_pos, dtype=torch.int32, device=dev)
    tok = torch.as_tensor(first_tok, dtype=torch.int32, device=dev)
    logits = torch.empty((m, S.vocab), device=dev)
    flags = rra.RRA_STEP_GATHER | rra.RRA_STEP_ADVANCE
    names = ("qkv", "attention", "o_proj", "ffn")
    tot = dict(input=0.0, head=0.0, step=0.0, **{k: 0.0 for k in names})
    dd.model.rra_model_set_phase_events(evs)
    try:
        for _ in range(steps):
            dd.model.rra_decode_step(x, pos, tok, m, flags=flags, logits=logits)
            torch.cuda.synchronize()
            tot["input"] += evs[0].elapsed_time(evs[1])
            for l in range(S.n_layers):
                for j, k in enumerate(names):
                    tot[k] += evs[1 + 4 * l + j].elapsed_time(evs[2 + 4 * l + j])
            tot["head"] += evs[n - 2].elapsed_time(evs[n - 1])
            tot["step"] += evs[0].elapsed_time(evs[n - 1])
    finally:
        dd.model.rra_model_set_phase_events(None)
    dd.model.rra_model_check()
    out = {f"{k}_ms": v / steps for k, v in tot.items()}
    out["groups"] = ("qkv: QKV GEMV (+ qkv_post); attention: flash decode + combine; o_proj: O "
                     "GEMV; ffn: residual/norm, gate/up, SwiGLU, down, residual; head: LM head + "
                     "argmax; eager steps, summed over the layers")
    out["steps"] = steps
    return out


def flash_decode_line(reps=20):
    """The standalone attention workload (32 sequences, 32 Q / 8 KV heads, hd
    128, lengths uniform in [1, 8192], an 8192-row cache): rra_flash_decode at
    each fixed chunk size and at the library's own choice, timed with HIP
    events, against the K+V bytes read once."""
    import synth
    import quantized_gemv_flash_amd as rra
    a = synth.FLASH_DECODE_M32
    q, kc, vc, _, _, lens = synth.attention_inputs(a, seed=0, device="cuda")
    L = lens.tolist()
    seq = lens.to(device="cuda", dtype=torch.int32)
    out = torch.empty_like(q)
    kv_bytes = sum(2 * a.n_kv_heads * l * a.head_dim * 4 for l in L)
    res = dict(workload=f"{a.name}: M={a.m}, {a.n_heads}/{a.n_kv_heads} heads, hd {a.head_dim}, "
                        f"lengths U[1,{a.max_len}], max_len {a.max_len}",
               algorithmic_bytes=kv_bytes, chunks={})
    tuned = None
    for chunk in list(a.chunks) + [0]:
        ws = torch.empty(rra.rra_flash_decode_workspace_bytes(a.m, a.n_heads, a.n_kv_heads,
                                                              a.head_dim, a.max_len, chunk),
                         dtype=torch.uint8, device="cuda")
        args = (q, kc, vc, seq, out, a.m, a.n_heads, a.n_kv_heads, a.head_dim, a.max_len, chunk, ws)
        if chunk == 0:  # the autotuner's pick, cached for this shape, used by chunk = 0
            tuned = rra.rra_flash_decode_tune(*args[:10], ws)
        sec = graph_time(lambda: rra.rra_flash_decode(*args), reps)
        key = str(chunk) if chunk else f"tuned (chunk {tuned[0]}, head split {tuned[1]})"
        res["chunks"][key] = dict(us=sec * 1e6, gbs=kv_bytes / sec / 1e9,
                                  hbm_frac=kv_bytes / sec / 1e9 / HBM_PEAK_GBS)
        del ws
    del q, kc, vc, out
    torch.cuda.empty_cache()
    return res


def hbm_ceiling_line(nbytes=1 << 32, reps=10):
    """Practical HBM ceilings on the same GPU: the library's plain streaming
    read (rra_hbm_read, 128-bit loads; the best of a few grid sizes) and, for
    comparison, PyTorch's device-to-device copy (read + write counted)."""
    import quantized_gemv_flash_amd as rra
    src = torch.empty(nbytes // 4, device="cuda").uniform_()
    dst = torch.empty_like(src)
    sums = torch.empty(32768, device="cuda")

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(reps):
            fn()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / 1e3 / reps

    by_grid = {b: nbytes / timed(lambda: rra.rra_hbm_read(src, sums, b)) / 1e9
               for b in (2048, 8192, 16384, 32768)}
    best = max(by_grid, key=by_grid.get)
    res = dict(read_gbs=by_grid[best], read_hbm_frac=by_grid[best] / HBM_PEAK_GBS,
               read_workgroups=best, read_gbs_by_workgroups=by_grid,
               torch_copy_gbs=2 * nbytes / timed(lambda: dst.copy_(src)) / 1e9, bytes=nbytes)
    del src, dst, sums
    torch.cuda.empty_cache()
    return res


def fd_only(S, steps, reps):
    """Flash decoding alone on one layer-sized synthetic cache at the lengths
    the timed steps end at, then a plain device copy of known size (the
    reference for scaling the HBM byte counters)."""
    import synth
    m, nkv, hd = S.m, S.n_kv_heads, S.head_dim
    max_len = max(S.max_len, 4096 + steps)
    lens = [L + steps for L in synth.context_lengths(S, m)]
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    kc = torch.randn((m, nkv, max_len, hd), device="cuda", generator=g)
    vc = torch.randn((m, nkv, max_len, hd), device="cuda", generator=g)

    class _Caches:
        k_caches, v_caches = [kc], [vc]
    sec, nbytes, chunk = flash_decode_roofline(S, _Caches, lens, reps)
    del kc, vc
    src = torch.randn(COPY_BYTES // 4, device="cuda", generator=g)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    return dict(fd_us=sec * 1e6, fd_bytes=nbytes, chunk=chunk, copy_bytes=COPY_BYTES)


def gemv_only(n=28672, k=4096, reps=5):
    """The 8B-shaped gate/up GEMV (Q4, 28672 x 4096) alone: rra_batched_gemv at
    M = 32, then M = 1, `reps` eager calls each (for counter runs)."""
    import synth
    import quantized_gemv_flash_amd as rra
    data, scale = synth.weight(n, k, "q4", 0.02, 0, "bench_gemv_gu", "cuda")
    w = rra.device_weight(data, scale, "q4")
    del data, scale
    res = {}
    for m in (32, 1):
        x = torch.randn((m, k), device="cuda")
        y = torch.empty((m, n), device="cuda")
        ws = torch.empty(max(4, rra.rra_batched_gemv_workspace_bytes(w, m)), dtype=torch.uint8,
                         device="cuda")
        for _ in range(reps):
            rra.rra_batched_gemv(w, x, y, m, ws)
        torch.cuda.synchronize()
        res[f"m{m}_us"] = graph_time(lambda: rra.rra_batched_gemv(w, x, y, m, ws), 20) * 1e6
    return dict(shape=f"{n}x{k} q4", weight_bytes=n * k * 18 // 32, **res)


def gemv_ab_line(ms=(1, 4, 8), reps=20):
    """The matrix-core GEMV (rra_batched_gemv) against the vector-ALU one
    (rra_batched_gemv_valu) on the same tiled weights: the 0.5B-shaped Q8
    layer and LM-head matrices and the 8B-shaped Q4 ones, at small M, each
    timed as graph replays (the activation-image conversion and the split-K
    sum included on both sides)."""
    import synth
    import quantized_gemv_flash_amd as rra
    shapes = [("q8", "qkv", 1152, 896), ("q8", "gate_up", 9728, 896), ("q8", "down", 896, 4864),
              ("q8", "lm_head", 151936, 896), ("q4", "qkv", 6144, 4096),
              ("q4", "gate_up", 28672, 4096), ("q4", "down", 4096, 14336),
              ("q4", "lm_head", 128256, 4096)]
    res = {}
    for fmt, name, n, k in shapes:
        data, scale = synth.weight(n, k, fmt, 0.02, 0, f"ab_{name}_{n}", "cuda")
        w = rra.device_weight(data, scale, fmt)
        del data, scale
        wbytes = n * k * (18 if fmt == "q4" else 34) // 32
        row = {}
        for m in ms:
            x = torch.randn((m, k), device="cuda")
            y = torch.empty((m, n), device="cuda")
            ws = torch.empty(max(4, rra.rra_batched_gemv_workspace_bytes(w, m)), dtype=torch.uint8,
                             device="cuda")
            t_mfma = sorted(graph_time(lambda: rra.rra_batched_gemv(w, x, y, m, ws), reps)
                            for _ in range(3))[1]
            try:  # the VALU kernel stages a K split of x in LDS: too large a split is refused
                t_valu = sorted(graph_time(lambda: rra.rra_batched_gemv_valu(w, x, y, m, ws), reps)
                                for _ in range(3))[1]
            except rra.RraError:
                t_valu = None
            row[f"m{m}"] = dict(mfma_us=t_mfma * 1e6, valu_us=t_valu and t_valu * 1e6,
                                mfma_gbs=wbytes / t_mfma / 1e9,
                                valu_gbs=t_valu and wbytes / t_valu / 1e9)
        res[f"{fmt}_{name}_{n}x{k}"] = row
        del w
    torch.cuda.empty_cache()
    return res


COPY_BYTES = 1 << 30
COUNTERS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        "flash_decode_llama3_8b_m32.md")
ATTENTION_SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "quantized_gemv_flash_amd",
                             "csrc", "attention.hip")


def counter_traffic():
    """HBM bytes per chunk-kernel launch from the committed counter runs
    (FETCH_SIZE and WRITE_SIZE scaled by a plain copy's readings) and the
    algorithmic bytes of that launch, or (None, None) once the attention
    source has changed since they were taken."""
    import hashlib
    try:
        with open(COUNTERS) as f:
            line = [l for l in f.read().splitlines() if l.startswith("traffic_json: ")][0]
        rec = json.loads(line[len("traffic_json: "):])
        with open(ATTENTION_SRC, "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != rec["attention_hip_sha256"]:
                return None, None
        return float(rec["traffic_bytes_per_launch"]), float(rec["algorithmic_bytes"])
    except (OSError, IndexError, ValueError, KeyError):
        return None, None


PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")


def kernel_sources_sha256():
    """sha256 over the library's kernel and host sources (csrc/*.hip, *.h,
    *.cpp in name order, then include/rra.h): the key under which the step
    profiles record their counter traffic."""
    import glob
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    csrc = os.path.join(root, "quantized_gemv_flash_amd", "csrc")
    files = sorted(f for f in glob.glob(os.path.join(csrc, "*"))
                   if f.endswith((".hip", ".h", ".cpp")))
    h = hashlib.sha256()
    for f in files + [os.path.join(root, "include", "rra.h")]:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def step_counter_traffic(profile, sec_per_step, what):
    """Whole-step HBM traffic from a committed decode-step profile (every
    kernel's FETCH_SIZE and WRITE_SIZE per launch, copy-scaled, times its
    launches per step) over this run's step time, or None once the kernel
    sources have changed since the counters were taken."""
    try:
        with open(os.path.join(PROFILES, profile)) as f:
            line = [l for l in f.read().splitlines() if l.startswith("step_traffic_json: ")][0]
        rec = json.loads(line[len("step_traffic_json: "):])
        if rec["sources_sha256"] != kernel_sources_sha256():
            return None
    except (OSError, IndexError, ValueError, KeyError):
        return None
    b = float(rec["counter_bytes_per_step"])
    return {"bytes_per_step": b, "gbs": b / sec_per_step / 1e9,
            "hbm_frac": b / sec_per_step / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes_per_step": float(rec["algorithmic_bytes_per_step"]),
            "source": f"profiles/{profile}: rocprofv3 FETCH_SIZE x {rec['read_factor']} + "
                      f"WRITE_SIZE x {rec['write_factor']} per launch (factors from a plain "
                      f"copy), times launches per step, {what}; over this run's step time"}


def cpu_baseline(S, W, dd, lengths, first_tok, nseq, steps, of_m=32):
    """The oracle, as it stands, on `steps` greedy decode steps of the first
    `nseq` sequences of the same workload (its own tokens fed back), from the
    same cache contents (the GPU's, copied once; setup not timed)."""
    import oracle
    t_setup = time.time()
    orc = oracle.DecoderOracle(S, W, nseq, max(lengths[:nseq]) + steps)
    for l in range(S.n_layers):
        for s in range(nseq):
            L = lengths[s]
            orc.set_context(l, s, dd.k_caches[l][s, :, :L], dd.v_caches[l][s, :, :L])
    emb = W.embed
    tok = list(first_tok[:nseq])
    log(f"oracle setup {time.time() - t_setup:.1f}s")
    t0 = time.time()
    for i in range(steps):
        x = emb[torch.as_tensor(tok, device=emb.device)].cpu().numpy()
        tok = [int(t) for t in orc.step(x, [L + i for L in lengths[:nseq]])["tok"]]
    sec = time.time() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    return dict(value=nseq * steps / sec, unit="tok/s", cores=threads, kind="oracle",
                sample=f"{steps} greedy decode steps of {nseq} of the {of_m} sequences of the "
                       f"same workload ({sec:.1f} s; fp64, {threads} OpenMP threads)")


def m_sweep_line(steps=32, ms=(1, 4, 8, 16, 32), prefill=True, cpu=False, tune=True):
    """The 1.5B-shaped Q4 decoder over a synthetic 1024-row KV context per
    sequence: greedy decode tok/s at each batch size M (one graph per M)."""
    import synth
    S = synth.QWEN25_15B_Q4
    m_max = max(ms)
    W, dd = build_decoder(S, m_max, S.max_len)
    lengths = synth.context_lengths(S, m_max)
    fill_kv_context(S, dd, lengths)
    first = synth.first_tokens(S, m_max).tolist()
    wbytes = dd.weight_bytes()
    out = dict(workload=f"{S.name}: 1024-row context, {steps} greedy steps per M, one graph per step",
               weight_bytes=wbytes)
    if tune:
        plans = dd.model.rra_model_tune_attention(list(ms), [L + steps // 2 for L in lengths])
    else:
        plans = {m: dd.model.rra_model_attention_plan(m) for m in ms}
    out["attention_plans"] = {f"m{m}": dict(chunk=plans[m][0], head_split=plans[m][1]) for m in ms}
    for m in ms:
        sec, _, _ = timed_greedy(dd, S, m, first[:m], lengths[:m], steps, 2)
        kv = sum(S.n_layers * 2 * S.n_kv_heads * (L + i + 1) * S.head_dim * 4
                 for L in lengths[:m] for i in range(steps)) / steps
        out[f"m{m}"] = dict(tok_s=m * steps / sec, ms_per_step=1e3 * sec / steps,
                            hbm_frac=(wbytes + kv) * steps / sec / 1e9 / HBM_PEAK_GBS)
    if cpu:  # the oracle at both ends of the sweep (M=32: a sample of 8 sequences)
        out["cpu_baseline"] = {
            "m1": cpu_baseline(S, W, dd, lengths, first, 1, 4, of_m=1),
            "m32": cpu_baseline(S, W, dd, lengths, first, 8, 4, of_m=32)}
        log(f"sweep cpu baselines {out['cpu_baseline']}")
    if prefill:
        out["prefill"] = prefill_line(S, dd, 1024)
    del dd, W
    torch.cuda.empty_cache()
    return out


def prefill_line(S, dd, n_tokens, reps=3):
    """Prompt ingestion (rra_prefill) of n_tokens seeded token ids into cache
    slot 0 from position 0, in chunks of the model's prefill rows: per chunk
    and layer, GEMMs that read the weights once for the chunk's rows and a
    matrix-core causal attention."""
    import synth
    toks = synth.uniform_int((n_tokens,), 0, S.vocab - 1, 0, "bench_prompt").to("cuda", torch.int32)
    nt = torch.zeros(1, dtype=torch.int32, device="cuda")
    dd.model.rra_prefill(toks, n_tokens, 0, 0, next_tok=nt)  # warm-up
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        dd.model.rra_prefill(toks, n_tokens, 0, 0, next_tok=nt)
    ev1.record()
    torch.cuda.synchronize()
    sec = ev0.elapsed_time(ev1) / 1e3 / reps
    return dict(tokens=n_tokens, rows_per_chunk=dd.model.prefill_rows, ms=1e3 * sec,
                tok_s=n_tokens / sec)


LM_HEAD_FORMATS = {
    # format: (description, weight bytes per value)
    "fp8": ("fp8 (E4M3 + fp16 scale per 32)", 34 / 32),
    "q6k": ("q6k (6-bit codes, int8 scale per 16, fp16 scale per 256)", 210 / 256),
}


def lm_head_gemv_line(fmt, reps=20):
    """A further block format on the weights-once GEMV at the LM-head shape of
    the 8B-shaped decoder (128256 x 4096): rra_batched_gemv (activation image +
    GEMV) timed with HIP events around graph replays at M = 1 and 32."""
    import synth
    import quantized_gemv_flash_amd as rra
    n, k = 128256, 4096
    data, scale = synth.weight(n, k, fmt, 0.02, 0, f"bench_{fmt}_lm", "cuda")
    w = rra.device_weight(data, scale, fmt)
    del data, scale
    desc, per_value = LM_HEAD_FORMATS[fmt]
    wbytes = n * k * per_value
    res = dict(shape=f"{n}x{k} {desc}", weight_bytes=wbytes)
    for m in (1, 32):
        x = torch.randn((m, k), device="cuda")
        y = torch.empty((m, n), device="cuda")
        ws = torch.empty(max(4, rra.rra_batched_gemv_workspace_bytes(w, m)), dtype=torch.uint8,
                         device="cuda")
        # median of three graph replays of `reps` calls (eager launches let
        # host-side gaps into the event time)
        sec = sorted(graph_time(lambda: rra.rra_batched_gemv(w, x, y, m, ws), reps)
                     for _ in range(3))[1]
        res[f"m{m}_us"] = sec * 1e6
        res[f"m{m}_gbs"] = wbytes / sec / 1e9
        res[f"m{m}_hbm_frac"] = wbytes / sec / 1e9 / HBM_PEAK_GBS
    del w
    torch.cuda.empty_cache()
    return res


def m1_line(steps_m1=256, ctx=512, cpu=False, tune=True):
    import synth
    S = synth.QWEN25_05B_Q8
    W, dd = build_decoder(S, 1, S.max_len)
    ctx_tok = synth.context_tokens(S, 1, ctx).tolist()[0]
    # teacher-forced context: one eager step per context token, run as graph
    # replays of a plain (non-gather) step
    import quantized_gemv_flash_amd as rra
    x = torch.empty((1, S.hidden), device="cuda")
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    lg = torch.empty((1, S.vocab), device="cuda")
    emb = W.embed
    for p in range(ctx):
        x.copy_(emb[ctx_tok[p]].unsqueeze(0))
        pos.fill_(p)
        dd.model.rra_decode_step(x, pos, tok, 1, flags=rra.RRA_GRAPH, logits=lg)
    torch.cuda.synchronize()
    first = synth.first_tokens(S, 1).tolist()
    plan = (dd.model.rra_model_tune_attention([1], [ctx + steps_m1 // 2])[1] if tune
            else dd.model.rra_model_attention_plan(1))
    sec, _, _ = timed_greedy(dd, S, 1, first, [ctx], steps_m1, 3)
    wbytes = dd.weight_bytes()
    kv_read = sum(S.n_layers * 2 * S.n_kv_heads * (ctx + i + 1) * S.head_dim * 4
                  for i in range(steps_m1)) / steps_m1
    res = dict(workload=f"{S.name} M=1, {ctx}-token context then {steps_m1} greedy steps, one graph",
               attention_plan=dict(chunk=plan[0], head_split=plan[1]),
               tok_s=steps_m1 / sec, ms_per_step=1e3 * sec / steps_m1,
               weight_kv_gbs=(wbytes + kv_read) * steps_m1 / sec / 1e9)
    res["hbm_frac"] = res["weight_kv_gbs"] / HBM_PEAK_GBS
    res["counter_traffic"] = step_counter_traffic(
        "decode_step_qwen05b_q8_m1.md", sec / steps_m1,
        "at the counter runs' 32-token context")
    res["host_handoff"] = host_handoff_line(dd, S, 1, first, [ctx], steps_m1)
    if cpu:  # the oracle on 8 steps after the same 512-row context (the GPU's cache rows)
        res["cpu_baseline"] = cpu_baseline(S, W, dd, [ctx], first, 1, 8, of_m=1)
        log(f"m1 cpu baseline {res['cpu_baseline']}")
    del dd, W
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (got --gpus {args.gpus}); the decode "
              "step is not sharded across GPUs", file=sys.stderr)
        sys.exit(2)
    import synth
    import quantized_gemv_flash_amd as rra  # noqa: F401  (fails loudly if not built)
    if args.only_gemv_ab:
        print(json.dumps({"gemv_valu_vs_mfma": gemv_ab_line()}), flush=True)
        return
    if args.only_prefill:
        S = synth.LLAMA3_8B_Q4
        W, dd = build_decoder(S, 1, 1024)
        print(json.dumps({"prefill": prefill_line(S, dd, 512)}), flush=True)
        return
    if args.only_sweep:
        ms = tuple(int(v) for v in args.only_sweep.split(","))
        print(json.dumps({"m_sweep": m_sweep_line(steps=args.steps, ms=ms, prefill=False,
                                                  tune=not args.fixed_plans)}),
              flush=True)
        return
    if args.only_m1:
        print(json.dumps({"m1": m1_line(args.m1_steps, args.m1_ctx, tune=not args.fixed_plans)}),
              flush=True)
        return
    if args.only_attention:
        print(json.dumps({"flash_decode": flash_decode_line(), "hbm_ceiling": hbm_ceiling_line()}),
              flush=True)
        return
    if args.gemv_only:
        print(json.dumps({"gemv_only": gemv_only()}), flush=True)
        return
    if args.fd_only:
        print(json.dumps({"fd_only": fd_only(synth.LLAMA3_8B_Q4, args.steps, args.fd_reps)}),
              flush=True)
        return

    S = synth.LLAMA3_8B_Q4
    m, steps = S.m, args.steps
    max_len = max(S.max_len, 4096 + steps)
    t0 = time.time()
    W, dd = build_decoder(S, m, max_len)
    lengths = synth.context_lengths(S, m)
    fill_kv_context(S, dd, lengths)
    torch.cuda.synchronize()
    log(f"setup {time.time() - t0:.1f}s; weights {dd.weight_bytes() / 1e9:.3f} GB")
    t0 = time.time()
    if args.fixed_plans:
        plan = dd.model.rra_model_attention_plan(m)
    else:
        plan = dd.model.rra_model_tune_attention([m], [L + steps // 2 for L in lengths])[m]
    log(f"flash-decode plan for M={m}: chunk {plan[0]}, head split {plan[1]} "
        f"(tuned in {time.time() - t0:.1f}s)")
    first = synth.first_tokens(S, m).tolist()
    sec, final_pos, _ = timed_greedy(dd, S, m, first, lengths, steps, args.warmup)
    tok_s = m * steps / sec
    ms = 1e3 * sec / steps
    gstats = dd.model.rra_graph_stats()
    log(f"{tok_s:.1f} tok/s, {ms:.3f} ms/step, graph {gstats}")

    wbytes = dd.weight_bytes()
    # KV bytes per step: every cached row read (K and V), averaged over the steps
    kv_read = sum(S.n_layers * 2 * S.n_kv_heads * (L + i + 1) * S.head_dim * 4
                  for L in lengths for i in range(steps)) / steps
    step_gbs = (wbytes + kv_read) / (sec / steps) / 1e9

    # the dominant kernel, timed inside the same steps (rerun eagerly, its
    # launches carrying an event pair), and rra_flash_decode alone on layer 0's cache
    fd_total, fd_total_bytes, pos_ev = flash_decode_in_step(S, dd, m, first, lengths, steps)
    assert pos_ev == final_pos
    launches = S.n_layers * steps
    fd_sec, fd_bytes = fd_total / launches, fd_total_bytes / launches  # per launch
    fd_gbs = fd_bytes / fd_sec / 1e9
    fd_alone, alone_bytes, chunk = flash_decode_roofline(S, dd, [p for p in final_pos],
                                                         args.fd_reps, plan)
    log(f"flash decode in the step: {fd_sec * 1e6:.1f} us, {fd_gbs:.0f} GB/s (chunk {plan[0]}, "
        f"head split {plan[1]}); alone {fd_alone * 1e6:.1f} us")

    phases = phase_line(S, dd, m, first, lengths)
    log(f"step phases {phases}")
    handoff = host_handoff_line(dd, S, m, first, lengths, steps)
    log(f"host hand-off {handoff}")
    m1 = None
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(S, W, dd, lengths, first, 8, 4)
        log(f"cpu baseline {cpu}")
    prefill = None if args.main_only else prefill_line(S, dd, 512)  # overwrites slot 0's cache
    log(f"prefill {prefill}")
    del dd, W
    torch.cuda.empty_cache()
    if not (args.no_m1 or args.main_only):
        m1 = m1_line(args.m1_steps, args.m1_ctx, cpu=not args.no_cpu_baseline)
        log(f"m1 {m1}")
    fp8 = None if args.main_only else lm_head_gemv_line("fp8")
    log(f"fp8 gemv {fp8}")
    q6k = None if args.main_only else lm_head_gemv_line("q6k")
    log(f"q6k gemv {q6k}")
    sweep = None if (args.no_sweep or args.main_only) else m_sweep_line(
        cpu=not args.no_cpu_baseline)
    log(f"m sweep {sweep}")
    gemv_ab = None if args.main_only else gemv_ab_line()
    log(f"gemv valu vs mfma {gemv_ab}")
    fd_c = None if args.main_only else flash_decode_line()
    log(f"flash decode chunks {fd_c}")
    ceil = None if args.main_only else hbm_ceiling_line()
    log(f"hbm ceiling {ceil}")

    traffic, traffic_alg = counter_traffic()
    out = {
        "metric": "decode tok/s at M=1 and M=32; weight+KV stream HBM GB/s as % of peak",
        "value": tok_s,
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{S.name}: M={m}, positions U[2048,4096] over a synthetic fp32 KV "
                        f"context, {steps} greedy steps, one captured HIP graph per step",
            "m": m, "weights": "q4 (32 x 4-bit + fp16 scale per block)", "kv_cache": "f32",
            "max_len": max_len,
        },
        "per_sequence_tok_s": tok_s / m,
        "host_handoff": handoff,
        "step_phases": phases,
        "weight_kv_gbs": step_gbs,
        "weight_kv_hbm_frac": step_gbs / HBM_PEAK_GBS,
        "counter_traffic": step_counter_traffic(
            "decode_step_llama3_8b_q4_m32.md", sec / steps,
            "at the counter runs' context lengths (their first steps)"),
        "roofline": {
            "kernel": "fd_chunk_kernel (flash-decode split-K chunks), every layer of the "
                      f"{steps} timed steps, M={m}, chunk {plan[0]}, head split {plan[1]} "
                      "(autotuned)",
            "bound": "hbm", "achieved": fd_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": fd_gbs / HBM_PEAK_GBS, "traffic": traffic,
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE/WRITE_SIZE, copy-scaled) "
                            "at the final lengths, whose algorithmic bytes are "
                            "traffic_algorithmic_bytes",
            "traffic_algorithmic_bytes": traffic_alg,
            "avg_us": fd_sec * 1e6, "algorithmic_bytes": fd_bytes,
            "timing": "HIP events on the step's stream around each layer's chunk kernel, the "
                      "same steps rerun eagerly; bytes and time summed over layers and steps",
            "alone_us": fd_alone * 1e6,
            "alone_gbs": alone_bytes / fd_alone / 1e9,
            "alone": "rra_flash_decode (chunk kernel + combine) on layer 0's cache at the final "
                     "lengths, 20 launches in one graph replay",
        },
        "m1": m1,
        "fp8_gemv": fp8,
        "q6k_gemv": q6k,
        "prefill": prefill and dict(workload=f"{S.name}: 512 prompt tokens into one slot", **prefill),
        "m_sweep": sweep,
        "gemv_valu_vs_mfma": gemv_ab,
        "flash_decode": fd_c,
        "hbm_ceiling": ceil,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    if torch.cuda.is_available():
        _stream = torch.cuda.Stream()  # graph capture needs a non-null stream
        with torch.cuda.stream(_stream):
            main()
        _stream.synchronize()
    else:
        main()
