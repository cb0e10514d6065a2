"""The flash-decode split autotuner ([head_dim] flash_decoding_attention_into
takes its chunk size from a fixed constant; here the (rows per split, head
split) pair is chosen by timing on the GPU).

Every candidate the tuner may pick is checked against unsplit softmax
attention from the oracle, at the standalone workload's shapes and at the
decode step's attention shapes; in the decode step every candidate of a small
decoder is checked against the oracle's whole step, on both attention paths
(QKV-fused at M <= 8, separate epilogue above); tuning keeps its choice fixed,
recaptures graphs that held the old grid and leaves the caches untouched.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import quantized_gemv_flash_amd as rra
import synth
from gpu_common import DEV, Run, assert_close, banner, compare_step, host, u32

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def side_stream():
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        yield s
    s.synchronize()


def _inputs(m, nq, nkv, hd, max_len, seed, edge=()):
    a = synth.Attention("t", m, nq, nkv, hd, max_len, 1, max_len, ())
    q, kc, vc, _, _, lens = synth.attention_inputs(a, seed=seed, device=DEV)
    L = list(edge)[:m] + [int(v) for v in lens.tolist()[len(edge):]]
    hq = host(q)
    ref = np.stack([oracle.attention(hq[s], host(kc[s, :, :L[s]]), host(vc[s, :, :L[s]]), L[s])
                    for s in range(m)])
    return q, kc, vc, L, ref


# (m, nq, nkv, hd, max_len): the 8B step (M=32), the 1.5B sweep's ends, the
# 0.5B step (M=1), and a small-group shape
SHAPES = [(32, 32, 8, 128, 4160), (32, 12, 2, 128, 1152), (1, 12, 2, 128, 1152),
          (1, 14, 2, 64, 768), (4, 4, 2, 64, 700)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_every_candidate_equals_unsplit_attention(shape):
    m, nq, nkv, hd, max_len = shape
    cands = rra.rra_flash_decode_candidates(m, nq, nkv, max_len)
    banner("fd candidates", shape, len(cands))
    assert cands
    edge = [1, 2, 31, 32, 33, max_len - 1, max_len]
    q, kc, vc, L, ref = _inputs(m, nq, nkv, hd, max_len, 21, edge if m >= len(edge) else [max_len])
    seq = torch.as_tensor(L, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    for chunk, hs in cands:
        ws = torch.empty(rra.rra_flash_decode_workspace_bytes(m, nq, nkv, hd, max_len, chunk),
                         dtype=torch.uint8, device=DEV)
        out.fill_(float("nan"))
        rra.rra_flash_decode_ex(q, kc, vc, seq, out, m, nq, nkv, hd, max_len, chunk, hs, ws)
        torch.cuda.current_stream().synchronize()
        assert_close(out, ref, what=f"{shape} chunk={chunk} hs={hs}")


def test_tuned_choice_is_cached_and_used_by_chunk_zero():
    # The standalone workload's own shape at a quarter of its sequences.
    m, nq, nkv, hd, max_len = 8, 32, 8, 128, 8192
    q, kc, vc, L, ref = _inputs(m, nq, nkv, hd, max_len, 22)
    seq = torch.as_tensor(L, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    ws = torch.empty(rra.rra_flash_decode_workspace_bytes(m, nq, nkv, hd, max_len, 0),
                     dtype=torch.uint8, device=DEV)
    chunk, hs = rra.rra_flash_decode_tune(q, kc, vc, seq, out, m, nq, nkv, hd, max_len, ws)
    assert (chunk, hs) in rra.rra_flash_decode_candidates(m, nq, nkv, max_len)
    rra.rra_flash_decode(q, kc, vc, seq, out, m, nq, nkv, hd, max_len, 0, ws)
    want = torch.empty_like(q)
    rra.rra_flash_decode_ex(q, kc, vc, seq, want, m, nq, nkv, hd, max_len, chunk, hs, ws)
    torch.cuda.current_stream().synchronize()
    assert torch.equal(out, want)
    assert_close(out, ref, what="tuned")


def test_tuning_rejects_a_capturing_stream():
    m, nq, nkv, hd, max_len = 2, 4, 2, 64, 256
    q, kc, vc, L, _ = _inputs(m, nq, nkv, hd, max_len, 23)
    seq = torch.as_tensor(L, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    ws = torch.empty(rra.rra_flash_decode_workspace_bytes(m, nq, nkv, hd, max_len, 0),
                     dtype=torch.uint8, device=DEV)
    g = torch.cuda.CUDAGraph()
    with pytest.raises(rra.RraError, match="capturing"):
        with torch.cuda.graph(g):
            rra.rra_flash_decode_tune(q, kc, vc, seq, out, m, nq, nkv, hd, max_len, ws)


SMALL_Q4 = dataclasses.replace(synth.SMALL_LLAMA_FP8, name="small-llama-q4-ctx", fmt="q4",
                               max_len=512)


# QKV-fused flash decode (m <= 8; at m = 2 with the first K/V rows requested
# before the position), separate epilogue
@pytest.mark.parametrize("m", [2, 6, 10])
def test_every_candidate_in_the_decode_step(m):
    S = SMALL_Q4
    cands = rra.rra_flash_decode_candidates(m, S.n_heads, S.n_kv_heads, S.max_len)
    banner("step candidates", S.name, "m", m, len(cands))
    W = synth.decoder_weights(S, seed=12, device=DEV, gamma="random")
    run = Run(S, W, m, S.max_len)
    orc = oracle.DecoderOracle(S, W, m, S.max_len)
    lens = [500, 37, 256, 1, 300, 129, 64, 411, 2, 200][:m]
    run.fill_context(lens, orc, range(m))
    tok = synth.first_tokens(S, m, seed=12).tolist()
    x = host(W.embed[torch.as_tensor(tok, device=DEV)])
    pos = list(lens)  # every candidate runs the same step (the same cache row is rewritten)
    o = orc.step(x, pos)
    for chunk, hs in cands:
        run.dd.model.rra_model_set_attention_plan(m, chunk, hs)
        assert run.dd.model.rra_model_attention_plan(m) == (chunk, hs)
        compare_step(run.step(tok, pos, flags=rra.RRA_GRAPH), o, f"chunk={chunk} hs={hs}")
    st = run.dd.model.rra_graph_stats()
    assert st["captures"] == len(cands)  # every plan change recaptured


def test_model_tuning_picks_a_candidate_and_keeps_it():
    S = SMALL_Q4
    m = 3
    W = synth.decoder_weights(S, seed=13, device=DEV, gamma="random")
    run = Run(S, W, m, S.max_len)
    orc = oracle.DecoderOracle(S, W, m, S.max_len)
    lens = [400, 411, 390]
    run.fill_context(lens, orc, range(m))
    tok = synth.first_tokens(S, m, seed=13).tolist()
    run.step(tok, lens, flags=rra.RRA_GRAPH)  # a graph with the default plan
    plan = run.dd.model.rra_model_tune_attention([m], lens)
    cands = rra.rra_flash_decode_candidates(m, S.n_heads, S.n_kv_heads, S.max_len)
    assert plan[m] in cands
    for step in range(3):
        pos = [L + step for L in lens]
        o = orc.step(host(W.embed[torch.as_tensor(tok, device=DEV)]), pos)
        compare_step(run.step(tok, pos, flags=rra.RRA_GRAPH), o, f"tuned step {step}")
        assert run.dd.model.rra_model_attention_plan(m) == plan[m]
        tok = o["tok"].tolist()
    st = run.dd.model.rra_graph_stats()
    # the default-plan graph, then (unless the tuner kept the default plan)
    # one capture for the tuned plan, replayed after
    assert st["captures"] in (1, 2) and st["replays"] >= 2
    with pytest.raises(rra.RraError, match="head_split"):
        run.dd.model.rra_model_set_attention_plan(m, 64, 3)
    with pytest.raises(rra.RraError, match="chunk"):
        run.dd.model.rra_model_set_attention_plan(m, 48, 1)


def test_model_tuning_leaves_the_caches_untouched():
    # At batch sizes where the step fuses the QKV epilogue the tuner times
    # the fused kernel, which forms a new K/V row at each sequence's position:
    # it must attend to it without writing it, and every other launch of the
    # tuner only reads the caches.
    S = SMALL_Q4
    m = 8
    W = synth.decoder_weights(S, seed=14, device=DEV, gamma="random")
    run = Run(S, W, m, S.max_len)
    lens = [400, 37, 256, 1, 300, 129, 64, 510]
    run.fill_context(lens)
    before = [(k.clone(), v.clone()) for k, v in zip(run.dd.k_caches, run.dd.v_caches)]
    plan = run.dd.model.rra_model_tune_attention([1, 4, 8], lens)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int32)  # bitwise, whatever the unused rows hold
    for l, (k, v) in enumerate(before):
        assert torch.equal(bits(run.dd.k_caches[l]), bits(k)), f"layer {l} K cache changed"
        assert torch.equal(bits(run.dd.v_caches[l]), bits(v)), f"layer {l} V cache changed"
    for mm in (1, 4, 8):
        assert plan[mm] in rra.rra_flash_decode_candidates(mm, S.n_heads, S.n_kv_heads, S.max_len)
