"""Parity of prompt ingestion (rra_prefill) with the CPU oracle's prefill.

Prefill runs a sequence's prompt tokens through the model in chunks of up to
`prefill_rows` (<= 128) tokens: per layer a GEMM that streams the weights
once for the chunk's rows, RoPE and the chunk's K/V rows into the sequence's
cache slot, and a matrix-core causal attention over the slot's rows.
Checked: every layer's K/V cache rows of the slot, the last token's logits
and greedy id, the other slots untouched, ragged last chunks, a second
prefill call continuing the first, and a decode step taking over from the
prefilled cache.
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


@pytest.mark.parametrize("S", [synth.TINY_LLAMA_F32, SMALL_Q8, SMALL_Q4, synth.SMALL_LLAMA_FP8],
                         ids=lambda S: S.name)
def test_prefill_128_row_chunks_match_oracle(S):
    # 150 tokens in chunks of 128 + 22 into slot 1 of three (the 128-row GEMMs
    # and five 32-key blocks of the matrix-core attention), then 60 more from
    # position 150 in chunks of 60 (a chunk starting past the slot's first
    # rows), each call's last token's logits and id against the oracle.
    banner("prefill 128", S.name)
    max_len, m_max, slot = 256, 3, 1
    W = synth.decoder_weights(S, seed=4, device=DEV, gamma="random")
    dd = load_decoder(S, W, m_max=m_max, max_len=max_len, prefill_rows=128)
    orc = oracle.DecoderOracle(S, W, m_max, max_len)
    toks = prompt(S, 210, 4, "prefill128")
    nt = torch.zeros(1, dtype=torch.int32, device=DEV)
    lg = torch.empty(S.vocab, device=DEV)
    dd.model.rra_prefill(toks[:150].to(DEV, torch.int32), 150, slot, 0, next_tok=nt, logits=lg)
    o = orc.prefill(slot, host(W.embed[toks[:150].to(DEV)]), 0, head="last")
    torch.cuda.current_stream().synchronize()
    check_cache(dd, orc, slot, 150, "first call")
    check_last(nt, lg, o, "first call")
    dd.model.rra_prefill(toks[150:].to(DEV, torch.int32), 60, slot, 150, next_tok=nt, logits=lg)
    o = orc.prefill(slot, host(W.embed[toks[150:].to(DEV)]), 150, head="last")
    torch.cuda.current_stream().synchronize()
    check_cache(dd, orc, slot, 210, "second call")
    check_last(nt, lg, o, "second call")
    for other in (0, 2):
        for l in range(S.n_layers):
            assert not dd.k_caches[l][other].any() and not dd.v_caches[l][other].any()
    dd.model.rra_model_check()


def test_prefill_chunk_sizes_agree():
    # The same 70-token prompt in chunks of 1, 16, 33 and 128 rows (the
    # 1-, 2-, 4- and 8-column-tile GEMMs and their attention tiles): every
    # cache row and the next token within the tolerance of each other and of
    # the oracle.
    S = SMALL_Q4
    W = synth.decoder_weights(S, seed=2, device=DEV, gamma="random")
    toks = prompt(S, 70, 2, "prefill3")
    orc = oracle.DecoderOracle(S, W, 1, 80)
    o = orc.prefill(0, host(W.embed[toks.to(DEV)]), 0, head="last")
    for rows in (1, 16, 33, 128):
        dd = load_decoder(S, W, m_max=1, max_len=80, prefill_rows=rows)
        nt = torch.zeros(1, dtype=torch.int32, device=DEV)
        lg = torch.empty(S.vocab, device=DEV)
        dd.model.rra_prefill(toks.to(DEV, torch.int32), 70, 0, 0, next_tok=nt, logits=lg)
        torch.cuda.current_stream().synchronize()
        check_cache(dd, orc, 0, 70, f"rows {rows}")
        check_last(nt, lg, o, f"rows {rows}")


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


@pytest.mark.parametrize("T,rows", [(33, 32), (96, 128)])
def test_qwen15b_q4_prefill(T, rows):
    # The 1.5B-shaped Q4 decoder into slot 2 of four: 33 tokens in 32-row
    # chunks (32 + 1), and a 96-token prompt in one chunk (the 8-column-tile
    # GEMMs, three 32-key blocks of attention per 16-row tile).
    S = synth.QWEN25_15B_Q4
    banner("prefill", S.name, T, rows)
    W = synth.decoder_weights(S, seed=0, device=DEV)
    dd = load_decoder(S, W, m_max=4, max_len=128, prefill_rows=rows)
    orc = oracle.DecoderOracle(S, W, 4, 128)
    slot = 2
    toks = prompt(S, T, 0, "prefill5")
    nt = torch.zeros(1, dtype=torch.int32, device=DEV)
    lg = torch.empty(S.vocab, device=DEV)
    dd.model.rra_prefill(toks.to(DEV, torch.int32), T, slot, 0, next_tok=nt, logits=lg)
    o = orc.prefill(slot, host(W.embed[toks.to(DEV)]), 0, head="last")
    torch.cuda.current_stream().synchronize()
    check_cache(dd, orc, slot, T, "1.5B prefill")
    check_last(nt, lg, o, "1.5B prefill")
