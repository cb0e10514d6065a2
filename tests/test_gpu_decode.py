"""Parity of the whole decode step (rra_decode_step) with the CPU oracle.

The oracle runs on the same seeded bytes.  Where greedy ids could differ
(oracle top-2 gap < 1e-3) the GPU is teacher-forced with the oracle's ids, so
no value computed on the GPU ever enters the oracle.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import quantized_gemv_flash_amd as rra
import synth
from gpu_common import DEV, LOGIT_ATOL, Run, assert_close, assert_tokens, banner, compare_step, host, u32
from quantized_gemv_flash_amd.loader import load_decoder

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


# ---------------------------------------------------------------- tiny fp32
def test_tiny_f32_sixteen_greedy_steps():
    S = synth.TINY_LLAMA_F32
    banner("decode", S.name)
    W = synth.decoder_weights(S, seed=0, device=DEV, gamma="random")
    run = Run(S, W, 1, S.max_len)
    orc = oracle.DecoderOracle(S, W, 1, S.max_len)
    tok = synth.first_tokens(S, 1).tolist()
    for step in range(S.steps):
        gpu = run.step(tok, [step])
        o = orc.step(host(W.embed[torch.as_tensor(tok, device=DEV)]), [step])
        compare_step(gpu, o, f"step {step}")
        tok = o["tok"].tolist()


SMALL_DECODERS = [synth.TINY_LLAMA_F32,
                  dataclasses.replace(synth.SMALL_LLAMA_FP8, name="small-llama-q8", fmt="q8"),
                  dataclasses.replace(synth.SMALL_LLAMA_FP8, name="small-llama-q4", fmt="q4"),
                  synth.SMALL_LLAMA_FP8]


@pytest.mark.parametrize("m", [3, 6])
@pytest.mark.parametrize("S", SMALL_DECODERS, ids=lambda S: S.name)
def test_batched_equals_separate_bitwise(S, m):
    # M-batched == M separate M=1 runs, bit for bit, in every weight format.
    # At m <= 4 the O and down GEMVs form their inputs in a prologue; m = 6
    # takes the separate epilogue kernels against M=1's prologues.
    W = synth.decoder_weights(S, seed=3, device=DEV, gamma="random")
    both = Run(S, W, m, 16)
    ones = [Run(S, W, 1, 16) for _ in range(m)]
    toks = synth.first_tokens(S, m, seed=3).tolist()
    starts = [0, 2, 5, 1, 3, 4][:m]
    for step in range(6):
        pos = [s + step for s in starts]
        ids_b, hid_b, lg_b = both.step(toks, pos)
        for i in range(m):
            ids_1, hid_1, lg_1 = ones[i].step([toks[i]], [pos[i]])
            assert ids_1[0] == ids_b[i]
            assert torch.equal(hid_1[0], hid_b[i]) and torch.equal(lg_1[0], lg_b[i])
        toks = ids_b


@pytest.mark.parametrize("S", SMALL_DECODERS, ids=lambda S: S.name)
def test_graph_replay_equals_eager_bitwise(S):
    W = synth.decoder_weights(S, seed=1, device=DEV, gamma="random")
    eager, graph = Run(S, W, 2, 16), Run(S, W, 2, 16)
    toks = synth.first_tokens(S, 2, seed=1).tolist()
    steps = 10
    for step in range(steps):
        a = eager.step(toks, [step, step + 1])
        b = graph.step(toks, [step, step + 1], flags=rra.RRA_GRAPH)
        assert a[0] == b[0]
        assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
        toks = a[0]
    st = graph.dd.model.rra_graph_stats()
    assert st["captures"] == 1 and st["replays"] == steps - 1 and st["kernels"] > 0
    for l in range(S.n_layers):
        assert torch.equal(eager.dd.k_caches[l], graph.dd.k_caches[l])
        assert torch.equal(eager.dd.v_caches[l], graph.dd.v_caches[l])


@pytest.mark.parametrize("m", [2, 10])  # flash decode taking the QKV partials (m <= 8) or not
def test_attention_events_time_each_layer_and_change_nothing(m):
    # rra_model_set_attention_events: eager steps with the per-layer event
    # records give the same ids, logits, hidden state and caches bitwise as
    # steps without them, and every layer's interval is a positive time; a
    # graph step records nothing and still matches.
    S = SMALL_DECODERS[2]  # quantised (Q4): the GEMV prologues and split planes are in play
    W = synth.decoder_weights(S, seed=3, device=DEV, gamma="random")
    plain, timed = Run(S, W, m, 16), Run(S, W, m, 16)
    cur = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * S.n_layers)]
    for e in evs:
        e.record(cur)
    timed.dd.model.rra_model_set_attention_events(evs)
    toks = synth.first_tokens(S, m, seed=3).tolist()
    for step in range(4):
        pos = [step + i for i in range(m)]
        a = plain.step(toks, pos)
        b = timed.step(toks, pos)
        assert a[0] == b[0] and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
        toks = a[0]
        torch.cuda.synchronize()
        ms = [evs[2 * l].elapsed_time(evs[2 * l + 1]) for l in range(S.n_layers)]
        assert all(0.0 < t < 1000.0 for t in ms), ms
    pos = [4 + i for i in range(m)]
    a = plain.step(toks, pos)
    b = timed.step(toks, pos, flags=rra.RRA_GRAPH)
    assert a[0] == b[0] and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    for l in range(S.n_layers):
        assert torch.equal(plain.dd.k_caches[l], timed.dd.k_caches[l])
        assert torch.equal(plain.dd.v_caches[l], timed.dd.v_caches[l])
    timed.dd.model.rra_model_set_attention_events(None)
    with pytest.raises(rra.RraError) as e:
        timed.dd.model.rra_model_set_attention_events(evs[:-1])
    assert e.value.status == rra.RRA_EINVAL


@pytest.mark.parametrize("m", [2, 6])  # the fused small-batch path and the separate kernels
def test_phase_events_split_the_step_and_change_nothing(m):
    # rra_model_set_phase_events: eager steps that record the 4 x n_layers + 3
    # sub-phase boundaries give bitwise the same ids, logits, hidden state and
    # caches as steps without them; every group's interval is a time >= 0, and
    # the groups add up to the step's span; a graph step records nothing.
    S = SMALL_DECODERS[2]
    W = synth.decoder_weights(S, seed=4, device=DEV, gamma="random")
    plain, timed = Run(S, W, m, 16), Run(S, W, m, 16)
    cur = torch.cuda.current_stream()
    n = 4 * S.n_layers + 3
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record(cur)
    timed.dd.model.rra_model_set_phase_events(evs)
    toks = synth.first_tokens(S, m, seed=4).tolist()
    for step in range(3):
        pos = [step + i for i in range(m)]
        a = plain.step(toks, pos)
        b = timed.step(toks, pos)
        assert a[0] == b[0] and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
        toks = a[0]
        torch.cuda.synchronize()
        ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(n - 1)]
        assert all(0.0 <= t < 1000.0 for t in ms), ms
        assert abs(sum(ms) - evs[0].elapsed_time(evs[-1])) < 1e-2
    span = evs[0].elapsed_time(evs[-1])  # the last eager step's
    pos = [3 + i for i in range(m)]
    a = plain.step(toks, pos)
    b = timed.step(toks, pos, flags=rra.RRA_GRAPH)
    assert a[0] == b[0] and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    torch.cuda.synchronize()
    assert evs[0].elapsed_time(evs[-1]) == span  # not recorded again by the graph step
    for l in range(S.n_layers):
        assert torch.equal(plain.dd.k_caches[l], timed.dd.k_caches[l])
        assert torch.equal(plain.dd.v_caches[l], timed.dd.v_caches[l])
    timed.dd.model.rra_model_set_phase_events(None)
    with pytest.raises(rra.RraError) as e:
        timed.dd.model.rra_model_set_phase_events(evs[:-1])
    assert e.value.status == rra.RRA_EINVAL


def test_capture_failure_discarded_and_step_runs_eagerly(monkeypatch):
    # A failed capture ([reduces] try_graph_capture): the graph is discarded,
    # the stream leaves capture mode, the step runs eagerly with the same
    # results; once captures succeed again the graph is built and replayed.
    S = synth.TINY_LLAMA_F32
    W = synth.decoder_weights(S, seed=2, device=DEV, gamma="random")
    eager, graph = Run(S, W, 2, S.max_len), Run(S, W, 2, S.max_len)
    toks = synth.first_tokens(S, 2, seed=2).tolist()
    for step in range(4):
        if step == 0:
            monkeypatch.setenv("RRA_FAIL_CAPTURE", "1")
        if step == 2:
            monkeypatch.delenv("RRA_FAIL_CAPTURE")
        a = eager.step(toks, [step, step + 1])
        b = graph.step(toks, [step, step + 1], flags=rra.RRA_GRAPH)
        assert torch.cuda.current_stream().query() in (True, False)  # usable, not capturing
        assert a[0] == b[0] and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
        st = graph.dd.model.rra_graph_stats()
        assert st["captures"] == (0 if step < 2 else 1)
        assert st["replays"] == (1 if step == 3 else 0)
        toks = a[0]


def test_device_greedy_loop_gather_advance_in_graph():
    # The step reads the previous ids, gathers their embeddings and advances
    # the positions on the device; graph replays equal the eager loop.
    S = synth.TINY_LLAMA_F32
    W = synth.decoder_weights(S, seed=2, device=DEV)
    flags = rra.RRA_STEP_GATHER | rra.RRA_STEP_ADVANCE
    runs = [Run(S, W, 2, S.max_len), Run(S, W, 2, S.max_len)]
    first = synth.first_tokens(S, 2, seed=2).tolist()
    seqs = []
    for r, extra in zip(runs, (0, rra.RRA_GRAPH)):
        r.tok.copy_(torch.as_tensor(first, dtype=torch.int32))
        r.pos.zero_()
        ids = []
        for _ in range(12):
            r.dd.model.rra_decode_step(r.x, r.pos, r.tok, 2, flags=flags | extra, logits=r.logits)
            ids.append(host(r.tok).tolist())
        torch.cuda.synchronize()
        assert host(r.pos).tolist() == [12, 12]
        seqs.append(ids)
    assert seqs[0] == seqs[1]
    assert runs[1].dd.model.rra_graph_stats()["replays"] == 11


def test_position_past_cache_is_reported_not_written():
    S = synth.TINY_LLAMA_F32
    W = synth.decoder_weights(S, seed=4, device=DEV)
    run = Run(S, W, 1, 8)
    run.step([3], [2])
    run.dd.model.rra_model_check()
    before = [c.clone() for c in run.dd.k_caches]
    run.step([3], [8])  # == max_len
    with pytest.raises(rra.RraError, match="max_len"):
        run.dd.model.rra_model_check()
    run.dd.model.rra_model_check()  # cleared
    for a, b in zip(before, run.dd.k_caches):
        assert torch.equal(a, b)


def test_graph_recaptures_on_new_buffers():
    S = synth.TINY_LLAMA_F32
    W = synth.decoder_weights(S, seed=5, device=DEV)
    run = Run(S, W, 1, S.max_len)
    run.step([1], [0], flags=rra.RRA_GRAPH)
    run.step([2], [1], flags=rra.RRA_GRAPH)
    run.logits = torch.empty_like(run.logits)  # new logits buffer -> new key
    run.step([3], [2], flags=rra.RRA_GRAPH)
    st = run.dd.model.rra_graph_stats()
    assert st["captures"] == 2 and st["replays"] == 1


def test_continuous_batching_slots_join_and_leave():
    # Four cache slots, one captured graph: slot 0 runs throughout, slot 1 is
    # empty and joins with a new sequence at step 4, slot 2 leaves at step 6
    # and takes a new sequence at step 8, slot 3 stays empty.  Every active
    # slot matches its own single-sequence oracle; empty slots keep their
    # cache rows, token and position.
    S = synth.TINY_LLAMA_F32
    banner("continuous batching", S.name)
    W = synth.decoder_weights(S, seed=6, device=DEV, gamma="random")
    m, steps = 4, 10
    run = Run(S, W, m, S.max_len)
    first = synth.first_tokens(S, 8, seed=6).tolist()
    # (slot, first step, last step, first token) per sequence
    seqs = [(0, 0, 9, first[0]), (1, 4, 9, first[1]), (2, 0, 5, first[2]), (2, 8, 9, first[3])]
    orcs = [oracle.DecoderOracle(S, W, 1, S.max_len) for _ in seqs]
    cur = [t for (_, _, _, t) in seqs]
    none = rra.POS_NONE_I32
    for step in range(steps):
        owner = {}
        for i, (slot, a, b, _) in enumerate(seqs):
            if a <= step <= b:
                owner[slot] = i
        toks = [cur[owner[s]] if s in owner else 0 for s in range(m)]
        pos = [step - seqs[owner[s]][1] if s in owner else none for s in range(m)]
        tok_before = host(run.tok).tolist()
        empty = [s for s in range(m) if s not in owner]
        caches_before = [(run.dd.k_caches[l][empty].clone(), run.dd.v_caches[l][empty].clone())
                         for l in range(S.n_layers)]
        ids, hid, logits = run.step(toks, pos, flags=rra.RRA_GRAPH)
        for s, i in owner.items():
            o = orcs[i].step(host(W.embed[torch.as_tensor([cur[i]], device=DEV)]), [pos[s]])
            compare_step(([ids[s]], hid[s:s + 1], logits[s:s + 1]), o, f"step {step} slot {s}")
            cur[i] = int(o["tok"][0])
        for s in empty:
            assert ids[s] == tok_before[s], f"empty slot {s} token changed"
        for l, (kb, vb) in enumerate(caches_before):
            assert torch.equal(kb, run.dd.k_caches[l][empty]) and torch.equal(vb, run.dd.v_caches[l][empty])
        run.dd.model.rra_model_check()  # an empty slot is not an error
    st = run.dd.model.rra_graph_stats()
    assert st["captures"] == 1 and st["replays"] == steps - 1


def test_empty_slots_in_device_greedy_loop():
    # Under RRA_STEP_GATHER | RRA_STEP_ADVANCE an empty slot keeps its token
    # and is not advanced; the active slots equal a batch without the empty
    # slots, bit for bit.
    S = synth.TINY_LLAMA_F32
    W = synth.decoder_weights(S, seed=7, device=DEV)
    flags = rra.RRA_GRAPH | rra.RRA_STEP_GATHER | rra.RRA_STEP_ADVANCE
    first = synth.first_tokens(S, 2, seed=7).tolist()
    full = Run(S, W, 4, S.max_len)
    full.tok.copy_(torch.as_tensor([first[0], 11, first[1], 12], dtype=torch.int32))
    full.pos.copy_(torch.as_tensor([0, rra.POS_NONE_I32, 3, rra.POS_NONE_I32], dtype=torch.int32))
    pair = Run(S, W, 2, S.max_len)
    pair.tok.copy_(torch.as_tensor(first, dtype=torch.int32))
    pair.pos.copy_(torch.as_tensor([0, 3], dtype=torch.int32))
    for _ in range(6):
        full.dd.model.rra_decode_step(full.x, full.pos, full.tok, 4, flags=flags, logits=full.logits)
        pair.dd.model.rra_decode_step(pair.x, pair.pos, pair.tok, 2, flags=flags, logits=pair.logits)
        torch.cuda.synchronize()
        t4, t2 = host(full.tok).tolist(), host(pair.tok).tolist()
        assert [t4[0], t4[2]] == t2 and t4[1] == 11 and t4[3] == 12
        assert torch.equal(full.logits[[0, 2]], pair.logits)
    p4 = host(full.pos).tolist()
    assert p4 == [6, rra.POS_NONE_I32, 9, rra.POS_NONE_I32]


# ---------------------------------------------------------------- quantised decoders
@pytest.mark.parametrize("S", [synth.SMALL_LLAMA_FP8, synth.SMALL_LLAMA_Q4_FP8_HEAD],
                         ids=lambda S: S.name)
def test_fp8_weights_small_decoder(S):
    # FP8 (E4M3) blocks for every matrix, and a Q4 decoder with an FP8 LM head:
    # two sequences, greedy steps in one graph, against the oracle.
    banner("decode", S.name)
    W = synth.decoder_weights(S, seed=0, device=DEV, gamma="random")
    run = Run(S, W, S.m, S.max_len)
    orc = oracle.DecoderOracle(S, W, S.m, S.max_len)
    tok = synth.first_tokens(S, S.m).tolist()
    for step in range(S.steps):
        pos = [step, step + 3]
        gpu = run.step(tok, pos, flags=rra.RRA_GRAPH)
        o = orc.step(host(W.embed[torch.as_tensor(tok, device=DEV)]), pos)
        compare_step(gpu, o, f"step {step}")
        tok = o["tok"].tolist()


# ---------------------------------------------------------------- error word
def test_token_id_past_vocab_is_reported():
    # Under RRA_STEP_GATHER an id >= vocab gathers a zero row (no read outside
    # the table) and is reported by rra_model_check; the other sequence's
    # results are those of a batch without it.
    S = SMALL_DECODERS[2]
    W = synth.decoder_weights(S, seed=3, device=DEV, gamma="random")
    flags = rra.RRA_STEP_GATHER
    both, one = Run(S, W, 2, 16), Run(S, W, 1, 16)
    both.tok.copy_(torch.as_tensor([7, S.vocab + 5], dtype=torch.int32))
    both.pos.copy_(torch.as_tensor([2, 2], dtype=torch.int32))
    one.tok.copy_(torch.as_tensor([7], dtype=torch.int32))
    one.pos.copy_(torch.as_tensor([2], dtype=torch.int32))
    both.dd.model.rra_decode_step(both.x, both.pos, both.tok, 2, flags=flags, logits=both.logits)
    one.dd.model.rra_decode_step(one.x, one.pos, one.tok, 1, flags=flags, logits=one.logits)
    with pytest.raises(rra.RraError, match="token id >= vocab"):
        both.dd.model.rra_model_check()
    both.dd.model.rra_model_check()  # cleared
    one.dd.model.rra_model_check()
    assert torch.equal(both.logits[0], one.logits[0])


@pytest.mark.parametrize("bad", [1.0e5, float("nan")])
def test_activation_outside_fp16_range_is_reported(bad):
    # The quantised GEMV takes its input as fp16 high + low parts: an input
    # element with |x| >= 65504 (or NaN) is reported by rra_model_check.
    S = SMALL_DECODERS[2]
    W = synth.decoder_weights(S, seed=3, device=DEV, gamma="random")
    run = Run(S, W, 1, 16)
    run.step([5], [0])
    run.dd.model.rra_model_check()
    run.x.copy_(W.embed[5:6])
    run.x[0, 17] = bad
    run.pos.fill_(1)
    run.dd.model.rra_decode_step(run.x, run.pos, run.tok, 1, logits=run.logits)
    with pytest.raises(rra.RraError, match="65504"):
        run.dd.model.rra_model_check()
    for c in run.dd.k_caches + run.dd.v_caches:  # the bad step wrote row 1
        c.zero_()
    run.step([5], [0])
    run.dd.model.rra_model_check()  # cleared, and a normal step reports nothing


@pytest.mark.parametrize("m", [1, 3, 20])
def test_greedy_ids_are_the_lowest_index_of_the_largest_logit(m):
    # The LM head reduces the logits each of its workgroups stores to a
    # (value, lowest index) partial per row, and the ids come from those.
    # Here its rows are zero except r1 < r2 (one random row) and r3 < r4 (its
    # negation), the rows of each pair at the same place in 16-row tiles far
    # apart (different workgroups): the largest logit is an exact tie, and the
    # id must be the lowest index holding it, as the argmax of the step's own
    # logits gives.
    S = dataclasses.replace(synth.SMALL_LLAMA_FP8, name="wide-vocab-q8", fmt="q8", hidden=384,
                            n_heads=6, n_kv_heads=2, head_dim=64, intermediate=1024,
                            vocab=131072, max_len=16)
    banner("lm-head ties", S.name, "m", m)
    W = synth.decoder_weights(S, seed=21, device=DEV, gamma="random")
    q, sc = (torch.zeros_like(t) for t in W.lm_head)
    src_q, src_s = synth.weight(1, S.hidden, "q8", 0.02, 21, "tie-row", DEV)
    r1, r2, r3, r4 = 777, 100_009, 5_001, 120_009
    for r, sign in ((r1, 1), (r2, 1), (r3, -1), (r4, -1)):
        q[r] = sign * src_q[0]
        sc[r] = src_s[0]
    W.lm_head = (q, sc)
    run = Run(S, W, m, S.max_len)
    tok = synth.first_tokens(S, m, seed=21).tolist()
    for step in range(3):
        ids, _, logits = run.step(tok, [step] * m, flags=rra.RRA_GRAPH)
        assert torch.equal(logits[:, r1], logits[:, r2]) and torch.equal(logits[:, r3], logits[:, r4])
        for i in range(m):
            mx = logits[i].max()
            want = int((logits[i] == mx).nonzero()[0])
            assert int(ids[i]) == want, (step, i, int(ids[i]), want)
            assert want in (0, r1, r3)
        tok = [int(v) for v in ids]
