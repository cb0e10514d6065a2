"""Parity of prompt ingestion (rra_prefill) with the CPU oracle's prefill.

Prefill runs a sequence's prompt tokens through the model in chunks of
`prefill_rows` tokens, every chunk one pass of the decode step whose rows all
map to the sequence's cache slot.  Checked: every layer's K/V cache rows of
the slot, the last token's logits and greedy id, the other slots untouched,
ragged last chunks, a second prefill call continuing the first, and a decode
step taking over from the prefilled cache.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import quantized_gemv_flash_amd as rra
import synth
from gpu_common import (DEV, LOGIT_ATOL, assert_close, assert_tokens, banner, host, u32)
from quantized_gemv_flash_amd.loader import load_decoder

pytestmark = pytest.mark.gpu

SMALL_Q8 = dataclasses.replace(synth.SMALL_LLAMA_FP8, name="small-llama-q8", fmt="q8")
SMALL_Q4 = dataclasses.replace(synth.SMALL_LLAMA_FP8, name="small-llama-q4", fmt="q4")


@pytest.fixture(autouse=True)
def side_stream():
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        yield s
    s.synchronize()


def prompt(S, n, seed, tag):
    return synth.uniform_int((n,), 0, S.vocab - 1, seed, tag)


def check_cache(dd, orc, slot, rows, what):
    for l in range(len(dd.k_caches)):
        assert_close(dd.k_caches[l][slot, :, :rows], orc.kc[l][slot, :, :rows],
                     what=f"{what} layer {l} K")
        assert_close(dd.v_caches[l][slot, :, :rows], orc.vc[l][slot, :, :rows],
                     what=f"{what} layer {l} V")


def check_last(next_tok, logits, o, what):
    assert_close(logits, o["logits"][-1], rtol=0.0, atol=LOGIT_ATOL, what=f"{what} logits")
    assert_tokens([int(next_tok.item())], o["tok"][-1:], o["gap"][-1:], o["logits"][-1:],
                  what=f"{what} next token")


@pytest.mark.parametrize("S", [synth.TINY_LLAMA_F32, SMALL_Q8, SMALL_Q4, synth.SMALL_LLAMA_FP8],
                         ids=lambda S: S.name)
def test_prefill_matches_oracle_then_decode_takes_over(S):
    # 19 tokens in chunks of 8 (8 + 8 + 3) into slot 1 of three; slots 0 and 2
    # keep their (zero) caches; then one decode step for slot 1 alone.
    banner("prefill", S.name)
    max_len, m_max, slot, T = 32, 3, 1, 19
    W = synth.decoder_weights(S, seed=0, device=DEV, gamma="random")
    dd = load_decoder(S, W, m_max=m_max, max_len=max_len, prefill_rows=8)
    orc = oracle.DecoderOracle(S, W, m_max, max_len)
    toks = prompt(S, T, 0, "prefill")
    nt = torch.zeros(1, dtype=torch.int32, device=DEV)
    lg = torch.empty(S.vocab, device=DEV)
    dd.model.rra_prefill(toks.to(DEV, torch.int32), T, slot, 0, next_tok=nt, logits=lg)
    o = orc.prefill(slot, host(W.embed[toks.to(DEV)]), 0)
    torch.cuda.current_stream().synchronize()
    check_cache(dd, orc, slot, T, "prefill")
    check_last(nt, lg, o, "prefill")
    for other in (0, 2):
        for l in range(S.n_layers):
            assert not dd.k_caches[l][other].any() and not dd.v_caches[l][other].any()
    # decode takes over at position T with the oracle's next token; the other
    # slots are empty
    nxt = int(o["tok"][-1])
    x = torch.zeros((m_max, S.hidden), device=DEV)
    x[slot] = W.embed[nxt]
    pos = u32([0, 0, 0])
    pos[:] = rra.POS_NONE_I32
    pos[slot] = T
    tok = torch.zeros(m_max, dtype=torch.int32, device=DEV)
    logits = torch.empty((m_max, S.vocab), device=DEV)
    ids = dd.model.rra_decode_step(x, pos, tok, m_max, logits=logits, tok_host=True)
    od = orc.step(host(W.embed[nxt])[None], [T], [slot])
    assert_close(x[slot:slot + 1], od["hidden"], what="decode hidden")
    assert_close(logits[slot:slot + 1], od["logits"], rtol=0.0, atol=LOGIT_ATOL, what="decode logits")
    assert_tokens([ids[slot]], od["tok"], od["gap"], od["logits"], what="decode token")
    check_cache(dd, orc, slot, T + 1, "after decode")


def test_prefill_continues_a_context_across_calls():
    # 10 tokens, then 13 more at start 10 (chunks 8 + 2, then 8 + 5): the cache
    # and the last token equal one oracle prefill of all 23 tokens.
    S = SMALL_Q4
    banner("prefill", S.name, "two calls")
    W = synth.decoder_weights(S, seed=1, device=DEV, gamma="random")
    dd = load_decoder(S, W, m_max=2, max_len=32, prefill_rows=8)
    orc = oracle.DecoderOracle(S, W, 2, 32)
    toks = prompt(S, 23, 1, "prefill2").to(DEV, torch.int32)
    nt = torch.zeros(1, dtype=torch.int32, device=DEV)
    lg = torch.empty(S.vocab, device=DEV)
    dd.model.rra_prefill(toks[:10], 10, 0, 0)
    dd.model.rra_prefill(toks[10:], 13, 0, 10, next_tok=nt, logits=lg)
    o = orc.prefill(0, host(W.embed[toks.long()]), 0)
    torch.cuda.current_stream().synchronize()
    check_cache(dd, orc, 0, 23, "two calls")
    check_last(nt, lg, o, "two calls")


def test_prefill_chunk_of_one_equals_decode_steps_bitwise():
    # prefill_rows = 1 makes every chunk a one-row step: the cache must be
    # bit-identical to feeding the same tokens through rra_decode_step.
    S = synth.TINY_LLAMA_F32
    W = synth.decoder_weights(S, seed=2, device=DEV, gamma="random")
    a = load_decoder(S, W, m_max=1, max_len=16, prefill_rows=1)
    b = load_decoder(S, W, m_max=1, max_len=16)
    toks = prompt(S, 9, 2, "prefill3").to(DEV, torch.int32)
    a.model.rra_prefill(toks, 9, 0, 0)
    x = torch.empty((1, S.hidden), device=DEV)
    pos = u32([0])
    tok = torch.zeros(1, dtype=torch.int32, device=DEV)
    for t in range(9):
        tok[0] = toks[t]
        pos[0] = t
        b.model.rra_decode_step(x, pos, tok, 1, flags=rra.RRA_STEP_GATHER)
    torch.cuda.current_stream().synchronize()
    for l in range(S.n_layers):
        assert torch.equal(a.k_caches[l], b.k_caches[l]) and torch.equal(a.v_caches[l], b.v_caches[l])


def test_prefill_rejects_bad_arguments_without_enqueueing():
    S = synth.TINY_LLAMA_F32
    W = synth.decoder_weights(S, seed=0, device=DEV)
    dd = load_decoder(S, W, m_max=2, max_len=16, prefill_rows=4)
    toks = prompt(S, 8, 0, "prefill4").to(DEV, torch.int32)
    with pytest.raises(rra.RraError, match="seq=2"):
        dd.model.rra_prefill(toks, 8, 2, 0)
    with pytest.raises(rra.RraError, match="exceed max_len"):
        dd.model.rra_prefill(toks, 8, 0, 9)
    with pytest.raises(rra.RraError, match="no tokens"):
        dd.model.rra_prefill(toks, 0, 0, 0)
    torch.cuda.current_stream().synchronize()
    for l in range(S.n_layers):
        assert not dd.k_caches[l].any()


def test_qwen15b_q4_prefill_33_tokens_rows32():
    # The 1.5B-shaped Q4 decoder with 32-row prefill chunks (32 + 1 tokens)
    # into slot 2 of four.
    S = synth.QWEN25_15B_Q4
    banner("prefill", S.name)
    W = synth.decoder_weights(S, seed=0, device=DEV)
    dd = load_decoder(S, W, m_max=4, max_len=64, prefill_rows=32)
    orc = oracle.DecoderOracle(S, W, 4, 64)
    T, slot = 33, 2
    toks = prompt(S, T, 0, "prefill5")
    nt = torch.zeros(1, dtype=torch.int32, device=DEV)
    lg = torch.empty(S.vocab, device=DEV)
    dd.model.rra_prefill(toks.to(DEV, torch.int32), T, slot, 0, next_tok=nt, logits=lg)
    o = orc.prefill(slot, host(W.embed[toks.to(DEV)]), 0)
    torch.cuda.current_stream().synchronize()
    check_cache(dd, orc, slot, T, "1.5B prefill")
    check_last(nt, lg, o, "1.5B prefill")
