"""Parity of the Q6K (6-bit K-quant) weight format on the GEMV, through the C ABI:
repack/unpack, the GEMV against the oracle (random and exact-integer cases,
LM-head shapes) and a decoder whose LM head is Q6K."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import quantized_gemv_flash_amd as rra
import synth
from gpu_common import DEV, LOGIT_ATOL, assert_close, assert_tokens, banner, host
from quantized_gemv_flash_amd.loader import load_decoder

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def side_stream():
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        yield s
    s.synchronize()


def _gemv(data, scale, x, m):
    n = data.shape[0]
    w = rra.device_weight(data, scale, "q6k")
    y = torch.full((m, n), float("nan"), device=DEV)
    nb = rra.rra_batched_gemv_workspace_bytes(w, m)
    ws = torch.full((max(nb, 4),), 0xFF, dtype=torch.uint8, device=DEV)
    rra.rra_batched_gemv(w, x, y, m, ws)
    torch.cuda.current_stream().synchronize()
    return y


@pytest.mark.parametrize("n,k", [(16, 256), (37, 512), (300, 768), (33, 256)])
def test_q6k_repack_roundtrip_bit_exact(n, k):
    banner("repack q6k", n, k)
    data, scale = synth.weight(n, k, "q6k", 0.02, 0, f"q6rp{n}x{k}", DEV)
    w = rra.device_weight(data, scale, "q6k")
    assert w.layout == rra.RRA_TILED and w.data.numel() == rra.rra_tiled_bytes("q6k", n, k)
    d2, s2 = torch.full_like(data, 0x5A), torch.full_like(scale, 0x33)
    rra.rra_unpack_weight(w, d2, s2)
    torch.cuda.current_stream().synchronize()
    assert torch.equal(d2, data) and torch.equal(s2, scale)


def test_q6k_rejects_k_not_multiple_of_256():
    assert rra.rra_tiled_bytes("q6k", 16, 128) == 0
    data = torch.zeros((16, 96), dtype=torch.uint8, device=DEV)   # as if k = 128
    scale = torch.zeros((16, 9), dtype=torch.uint8, device=DEV)
    w = rra.Weight("q6k", 16, 128, data, scale)
    with pytest.raises(rra.RraError):
        rra.rra_repack_weight(w)


@pytest.mark.parametrize("m", [1, 3, 16, 17, 32])
@pytest.mark.parametrize("n,k", [(16, 256), (37, 512), (300, 768), (1000, 2048), (64, 14336)])
def test_q6k_gemv_matches_oracle(n, k, m):
    banner("gemv q6k", n, k, m)
    data, scale = synth.weight(n, k, "q6k", 0.02, 0, f"q6g{n}x{k}", DEV)
    x = synth.normal((m, k), 1.0, 0, f"q6gx{m}x{k}", DEV)
    y = _gemv(data, scale, x, m)
    ref = oracle.gemv("q6k", data, scale, n, k, host(x))
    assert_close(y, ref, what=f"gemv q6k {n}x{k} m={m}")


@pytest.mark.parametrize("m", [1, 5, 32])
def test_q6k_gemv_integer_exact(m):
    # Power-of-two d, small-integer x, sub-scales including the extremes -128
    # and 127 and codes over all of 0..63: every operand and partial sum is
    # exact in fp32 as in the oracle's fp64, so the results must be equal.
    banner("gemv exact q6k", m)
    n, k = 70, 768
    g = np.random.default_rng(13)
    nsb = k // 256
    data = g.integers(0, 256, size=(n, nsb * 192), dtype=np.uint8)
    rec = np.zeros((n, nsb, 18), np.uint8)
    rec[:, :, :16] = g.choice(np.array([-128, 127, -1, 0, 1, 5, -7], np.int8),
                              size=(n, nsb, 16)).view(np.uint8)
    pow2 = np.array([0x3C00, 0x3800, 0x2C00, 0x2400], np.uint16)  # 1, 1/2, 1/16, 1/64
    rec[:, :, 16:18] = pow2[g.integers(0, 4, size=(n, nsb))].view(np.uint8).reshape(n, nsb, 2)
    x = g.integers(-4, 5, size=(m, k)).astype(np.float32)
    dt, st = torch.from_numpy(data).to(DEV), torch.from_numpy(rec.reshape(n, nsb * 18)).to(DEV)
    y = _gemv(dt, st, torch.from_numpy(x).to(DEV), m)
    ref = oracle.gemv("q6k", data, rec.reshape(n, nsb * 18), n, k, x)
    assert np.array_equal(host(y).astype(np.float64), ref)


@pytest.mark.parametrize("n,k", [(128256, 4096), (151936, 1536)])
def test_q6k_lm_head_shapes_sampled_rows(n, k):
    banner("gemv full q6k", n, k)
    data, scale = synth.weight(n, k, "q6k", 0.02, 0, f"q6full{n}x{k}", DEV)
    hd, hs = host(data), host(scale)
    rows = sorted(set(np.random.default_rng(n).integers(0, n, 120).tolist()) | {0, n - 1, n - 17})
    for m in (1, 17, 32):
        x = synth.normal((m, k), 1.0, 0, f"q6fullx{m}x{k}", DEV)
        y = _gemv(data, scale, x, m)
        ref = oracle.gemv("q6k", hd, hs, n, k, host(x), rows=rows)
        assert_close(host(y)[:, rows], ref, what=f"gemv q6k {n}x{k} m={m}")


SMALL_Q4_Q6K_HEAD = dataclasses.replace(synth.SMALL_LLAMA_Q4_FP8_HEAD,
                                        name="small-llama-q4-q6k-head", lm_fmt="q6k")


def test_q6k_lm_head_small_decoder():
    # A Q4 decoder with a Q6K LM head: two sequences, greedy steps in one
    # graph, against the oracle.
    S = SMALL_Q4_Q6K_HEAD
    banner("decode", S.name)
    W = synth.decoder_weights(S, seed=0, device=DEV, gamma="random")
    dd = load_decoder(S, W, m_max=S.m, max_len=S.max_len)
    orc = oracle.DecoderOracle(S, W, S.m, S.max_len)
    x = torch.empty((S.m, S.hidden), device=DEV)
    pos = torch.zeros(S.m, dtype=torch.int32, device=DEV)
    tok_d = torch.zeros(S.m, dtype=torch.int32, device=DEV)
    logits = torch.empty((S.m, S.vocab), device=DEV)
    tok = synth.first_tokens(S, S.m).tolist()
    for step in range(S.steps):
        p = [step, step + 3]
        x.copy_(W.embed[torch.as_tensor(tok, device=DEV)])
        pos.copy_(torch.as_tensor(p, dtype=torch.int32))
        ids = dd.model.rra_decode_step(x, pos, tok_d, S.m, flags=rra.RRA_GRAPH, logits=logits,
                                       tok_host=True)
        o = orc.step(host(W.embed[torch.as_tensor(tok, device=DEV)]), p)
        assert_close(x, o["hidden"], what=f"step {step} hidden")
        assert_close(logits, o["logits"], rtol=0.0, atol=LOGIT_ATOL, what=f"step {step} logits")
        assert_tokens(ids, o["tok"], o["gap"], o["logits"], what=f"step {step} tokens")
        tok = o["tok"].tolist()
