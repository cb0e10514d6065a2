"""Parity of the decode step with the CPU oracle at the workloads' own shapes
and in the launch configurations the benchmark times.

* the 0.5B-shaped Q8 decoder at M=1 with its 768-row cache, a 512-token
  context and greedy steps after it (flash decode runs 12 splits with every
  query head of a KV head dealt to its own workgroup, taking the QKV partials
  itself: the benchmark's M=1 launch);
* the 1.5B-shaped Q4 decoder at every batch size of its sweep after a
  1024-row context;
* the 8B-shaped Q4 decoder at M=32, one captured graph, eight steps, the
  shortest and longest contexts among the sampled sequences;
* the device-resident greedy loop (gather and position advance inside the
  graph) against the oracle's own greedy stream;
* the QKV-fused flash decode with many score rounds per split.

Every step is compared: the residual stream after the last layer, the logits
and the greedy ids ([batched_forward] forward_batched_to_token_ids: M
embeddings and positions in, M greedy token ids out).  Where greedy ids could
differ (oracle top-2 gap < 1e-3) the GPU is teacher-forced with the oracle's
ids, so no value computed on the GPU enters the oracle.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import quantized_gemv_flash_amd as rra
import synth
from gpu_common import (DEV, LOGIT_ATOL, TIE_GAP, Run, assert_close, assert_tokens, banner,
                        compare_step, elementwise_violations, host)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def side_stream():
    """Every test runs on its own (default-priority) stream: graph capture
    needs a stream other than the legacy null stream."""
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        yield s
    s.synchronize()


def embed_rows(W, toks):
    return host(W.embed[torch.as_tensor(list(toks), device=DEV)])


def teacher(ids, o, sample, m):
    """Next step's ids: the oracle's on the sampled slots, the GPU's elsewhere."""
    new = list(ids)
    for j, i in enumerate(sample):
        new[i] = int(o["tok"][j])
    return new[:m]


# ---------------------------------------------------------------- 0.5B Q8, M=1
def test_qwen05b_q8_512_context_then_greedy():
    # The benchmark's M=1 workload: 512 teacher-forced context steps at
    # positions 0..511 on random token ids (each a graph replay of the step),
    # then greedy steps from position 512, max_len 768.  The oracle ingests the
    # context as one causal prefill (the same result by definition).
    S = synth.QWEN25_05B_Q8
    ctx_n, greedy = 512, 16
    banner("decode", S.name, "context", ctx_n, "greedy", greedy)
    assert rra.rra_flash_decode_chunk(1, S.n_kv_heads, S.max_len, 0) == 64  # 12 splits
    W = synth.decoder_weights(S, seed=0, device=DEV)
    run = Run(S, W, 1, S.max_len)
    orc = oracle.DecoderOracle(S, W, 1, S.max_len)
    ctx = synth.context_tokens(S, 1, ctx_n).tolist()[0]
    for p in range(ctx_n):
        ids, hid, logits = run.step([ctx[p]], [p], flags=rra.RRA_GRAPH)
    o = orc.prefill(0, embed_rows(W, ctx), 0, head="last")
    compare_step((ids, hid, logits), dict(hidden=o["hidden"][-1:], logits=o["logits"],
                                          tok=o["tok"], gap=o["gap"]), "context end")
    for l in (0, S.n_layers // 2, S.n_layers - 1):
        for name, dc, oc in (("K", run.dd.k_caches, orc.kc), ("V", run.dd.v_caches, orc.vc)):
            assert_close(dc[l][0, :, :ctx_n], oc[l][0, :, :ctx_n], what=f"layer {l} {name}")
    tok = [int(o["tok"][-1])]
    for step in range(greedy):
        pos = [ctx_n + step]
        gpu = run.step(tok, pos, flags=rra.RRA_GRAPH)
        od = orc.step(embed_rows(W, tok), pos)
        compare_step(gpu, od, f"greedy step {step}")
        tok = od["tok"].tolist()
    st = run.dd.model.rra_graph_stats()
    assert st["captures"] == 1 and st["replays"] == ctx_n + greedy - 1
    run.dd.model.rra_model_check()


# ---------------------------------------------------------------- 1.5B Q4 sweep
@pytest.fixture(scope="module")
def qwen15b():
    S = synth.QWEN25_15B_Q4
    return S, synth.decoder_weights(S, seed=0, device=DEV)


@pytest.mark.parametrize("m", [1, 4, 8, 16, 32])
def test_qwen15b_q4_sweep(qwen15b, m):
    # Every batch size of the sweep, 1024-row synthetic contexts, one captured
    # graph, four steps; the oracle follows the first and the last sequence.
    S, W = qwen15b
    steps = 4
    banner("decode", S.name, "m", m, "steps", steps)
    run = Run(S, W, m, S.max_len)
    sample = sorted({0, m - 1})
    orc = oracle.DecoderOracle(S, W, len(sample), S.max_len)
    lens = synth.context_lengths(S, m)
    run.fill_context(lens, orc, sample)
    tok = synth.first_tokens(S, m).tolist()
    for step in range(steps):
        pos = [L + step for L in lens]
        ids, hid, logits = run.step(tok, pos, flags=rra.RRA_GRAPH)
        o = orc.step(embed_rows(W, [tok[i] for i in sample]), [pos[i] for i in sample])
        compare_step(([ids[i] for i in sample], hid[sample], logits[sample]), o,
                     f"m={m} step {step}")
        tok = teacher(ids, o, sample, m)
    assert run.dd.model.rra_graph_stats()["replays"] == steps - 1
    run.dd.model.rra_model_check()


# ---------------------------------------------------------------- 8B Q4, M=32
def test_llama8b_q4_m32_eight_steps():
    # The benchmark's M=32 workload: positions U[2048, 4096] over synthetic
    # contexts, one captured graph, eight steps; the oracle follows four
    # sequences, among them the shortest and the longest context.
    S = synth.LLAMA3_8B_Q4
    m, steps = S.m, 8
    banner("decode", S.name, "m", m, "steps", steps)
    W = synth.decoder_weights(S, seed=0, device=DEV)
    run = Run(S, W, m, S.max_len)
    lens = synth.context_lengths(S, m)
    sample = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, 17})
    orc = oracle.DecoderOracle(S, W, len(sample), S.max_len)
    run.fill_context(lens, orc, sample)
    tok = synth.first_tokens(S, m).tolist()
    for step in range(steps):
        pos = [L + step for L in lens]
        ids, hid, logits = run.step(tok, pos, flags=rra.RRA_GRAPH)
        o = orc.step(embed_rows(W, [tok[i] for i in sample]), [pos[i] for i in sample])
        # the residual stream after 32 layers: row-scaled (tests/test_tolerance_pins.py)
        compare_step(([ids[i] for i in sample], hid[sample], logits[sample]), o,
                     f"step {step} seqs {sample}", row_scale=True)
        tok = teacher(ids, o, sample, m)
    assert run.dd.model.rra_graph_stats()["replays"] == steps - 1
    run.dd.model.rra_model_check()


# ---------------------------------------------------------------- device greedy loop
SMALL_Q4 = dataclasses.replace(synth.SMALL_LLAMA_FP8, name="small-llama-q4", fmt="q4",
                               max_len=32)


@pytest.mark.parametrize("S", [synth.TINY_LLAMA_F32, SMALL_Q4], ids=lambda S: S.name)
def test_device_greedy_loop_matches_oracle_stream(S):
    # RRA_STEP_GATHER | RRA_STEP_ADVANCE inside the captured graph: the device
    # feeds each step's ids back itself.  The oracle runs its own greedy
    # stream; every step's ids, logits and residual stream must match until
    # the oracle's first near-tie (top-2 gap < 1e-3), after which the two
    # streams may legitimately part.
    banner("device loop", S.name)
    m, steps = 2, S.max_len - 4
    W = synth.decoder_weights(S, seed=8, device=DEV, gamma="random")
    run = Run(S, W, m, S.max_len)
    orc = oracle.DecoderOracle(S, W, m, S.max_len)
    first = synth.first_tokens(S, m, seed=8).tolist()
    start = [0, 3]
    run.tok.copy_(torch.as_tensor(first, dtype=torch.int32))
    run.pos.copy_(torch.as_tensor(start, dtype=torch.int32))
    flags = rra.RRA_GRAPH | rra.RRA_STEP_GATHER | rra.RRA_STEP_ADVANCE
    tok, compared = list(first), 0
    for step in range(steps):
        run.dd.model.rra_decode_step(run.x, run.pos, run.tok, m, flags=flags, logits=run.logits)
        o = orc.step(embed_rows(W, tok), [p + step for p in start])
        torch.cuda.current_stream().synchronize()
        ids = host(run.tok).tolist()
        assert host(run.pos).tolist() == [p + step + 1 for p in start]
        compare_step((ids, run.x, run.logits), o, f"loop step {step}")
        compared += 1
        if (o["gap"] < TIE_GAP).any():
            break
        assert ids == o["tok"].tolist()
        tok = ids
    assert compared >= 4
    st = run.dd.model.rra_graph_stats()
    assert st["captures"] == 1 and st["replays"] == compared - 1


# ---------------------------------------------------------------- fused flash decode, long splits
def test_fused_qkv_flash_decode_many_rounds():
    # At M <= 8 flash decode takes the QKV partials itself.  With 256-row
    # splits over a ~1.9k-row context each split runs four score rounds of 64
    # rows, the new row landing in a late round of one split.
    S = dataclasses.replace(SMALL_Q4, name="small-llama-q4-long", max_len=2048)
    banner("decode", S.name, "chunk 256")
    m = 2
    W = synth.decoder_weights(S, seed=9, device=DEV, gamma="random")
    run = Run(S, W, m, S.max_len, attn_chunk=256)
    orc = oracle.DecoderOracle(S, W, m, S.max_len)
    lens = [1901, 1530]
    run.fill_context(lens, orc, [0, 1])
    tok = synth.first_tokens(S, m, seed=9).tolist()
    for step in range(4):
        pos = [L + step for L in lens]
        gpu = run.step(tok, pos, flags=rra.RRA_GRAPH)
        o = orc.step(embed_rows(W, tok), pos)
        compare_step(gpu, o, f"step {step}")
        for l in range(S.n_layers):
            for i in range(m):
                assert_close(run.dd.k_caches[l][i, :, pos[i]], orc.kc[l][i, :, pos[i]],
                             what=f"layer {l} seq {i} new K row")
        tok = o["tok"].tolist()


# ---------------------------------------------------------------- non-blocking hand-off
def test_async_handoff_double_buffered_matches_blocking_and_oracle():
    # rra_decode_step_async: the device loop (gather + advance in the graph)
    # with each step's ids copied to one of two pinned host buffers and a
    # completion event per buffer; the host reads step t's ids while step t+1
    # runs.  The ids equal the blocking path's (tok_host: one sync per step)
    # bit for bit, and follow the oracle's greedy stream until its first
    # near-tie.
    S = SMALL_Q4
    banner("async hand-off", S.name)
    m, steps = 2, S.max_len - 4
    W = synth.decoder_weights(S, seed=10, device=DEV, gamma="random")
    first = synth.first_tokens(S, m, seed=10).tolist()
    start = [0, 3]
    flags = rra.RRA_GRAPH | rra.RRA_STEP_GATHER | rra.RRA_STEP_ADVANCE
    blocking, piped = Run(S, W, m, S.max_len), Run(S, W, m, S.max_len)
    for r in (blocking, piped):
        r.tok.copy_(torch.as_tensor(first, dtype=torch.int32))
        r.pos.copy_(torch.as_tensor(start, dtype=torch.int32))
    want = [blocking.dd.model.rra_decode_step(blocking.x, blocking.pos, blocking.tok, m,
                                              flags=flags, logits=blocking.logits, tok_host=True)
            for _ in range(steps)]
    bufs = [torch.full((m,), -1, dtype=torch.int32, pin_memory=True) for _ in range(2)]
    evs = [torch.cuda.Event() for _ in range(2)]
    for e in evs:
        e.record()  # creates the event
    got = []
    for t in range(steps + 1):
        if t < steps:
            piped.dd.model.rra_decode_step_async(piped.x, piped.pos, piped.tok, bufs[t % 2],
                                                 evs[t % 2], m, flags=flags, logits=piped.logits)
        if t >= 1:  # step t-1's ids, read while step t runs
            evs[(t - 1) % 2].synchronize()
            got.append(bufs[(t - 1) % 2].tolist())
    assert got == want
    orc = oracle.DecoderOracle(S, W, m, S.max_len)
    tok = list(first)
    for step in range(steps):
        o = orc.step(embed_rows(W, tok), [p + step for p in start])
        if (o["gap"] < TIE_GAP).any():
            break
        assert got[step] == o["tok"].tolist(), f"step {step}"
        tok = got[step]
    assert step >= 4
    with pytest.raises(rra.RraError, match="page-locked"):
        piped.dd.model.rra_decode_step_async(piped.x, piped.pos, piped.tok,
                                             torch.zeros(m, dtype=torch.int32), evs[0], m,
                                             flags=flags, logits=piped.logits)
