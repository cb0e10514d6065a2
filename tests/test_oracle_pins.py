"""Pins of the CPU oracle against facts other than itself.

Each test compares the oracle with a library routine, a closed form, a
worked example from the block-format definition, an independently written
bit-level decoding, or brute force on tiny inputs -- chosen so that a dropped
term, a wrong sign, a swapped nibble, a wrong head mapping or a transposed
operand in the oracle fails at least one of them.
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth


# ---------------------------------------------------------------- fp16 decode
def test_f16_decode_matches_numpy_for_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ---------------------------------------------------------------- dequant
def test_q4_worked_example():
    # One row, K = 64 (two blocks).  Block 0 scale 0.5 (fp16 0x3800), block 1
    # scale 0.125 (0x3000).  Byte 0x9F: low nibble 15 -> element 0 = 0.5*(15-8)
    # = 3.5; high nibble 9 -> element 1 = 0.5*(9-8) = 0.5.  Byte 0x08: element 2
    # = 0 (q=8), element 3 = 0.5*(0-8) = -4.  Byte 0x7E in block 1 (byte 16):
    # element 32 = 0.125*(14-8) = 0.75, element 33 = 0.125*(7-8) = -0.125.
    row = np.full(32, 0x88, np.uint8)  # every other element q = 8 -> 0
    row[0], row[1], row[16] = 0x9F, 0x08, 0x7E
    scale = np.array([[0x3800, 0x3000]], np.uint16)
    w = oracle.dequant("q4", row.reshape(1, 32), scale, 1, 64, [0])[0]
    expect = np.zeros(64)
    expect[0], expect[1], expect[2], expect[3] = 3.5, 0.5, 0.0, -4.0
    expect[32], expect[33] = 0.75, -0.125
    assert np.array_equal(w, expect)


def test_q8_worked_example():
    # Scale 0.25 (fp16 0x3400); q = -127, 0, 5, 127 -> -31.75, 0, 1.25, 31.75.
    q = np.zeros((1, 32), np.int8)
    q[0, :4] = [-127, 0, 5, 127]
    w = oracle.dequant("q8", q, np.array([[0x3400]], np.uint16), 1, 32, [0])[0]
    assert np.array_equal(w[:4], [-31.75, 0.0, 1.25, 31.75])
    assert not w[4:].any()


def _brute_row_q4(row_bytes: bytes, scales, k):
    """Element i of a packed Q4 row is nibble i of the row read as one
    little-endian integer; value = scale * (nibble - 8).  Exact rationals."""
    big = int.from_bytes(row_bytes, "little")
    out = []
    for i in range(k):
        nib = (big >> (4 * i)) & 0xF
        s = Fraction(np.array([scales[i // 32]], np.uint16).view(np.float16).item())
        out.append(s * (nib - 8))
    return out


def _brute_row_q8(row_bytes: bytes, scales, k):
    vals = struct.unpack(f"{k}b", row_bytes)
    return [Fraction(np.array([scales[i // 32]], np.uint16).view(np.float16).item()) * v
            for i, v in enumerate(vals)]


def _e4m3_exact(code: int) -> Fraction:
    # OCP E4M3 written out from its bit fields: sign, exponent bias 7, 3-bit
    # fraction, exponent 0 subnormal (2^-6 * f/8).
    sign = -1 if code & 0x80 else 1
    e, f = (code >> 3) & 0xF, code & 0x7
    assert not (e == 15 and f == 7), "NaN code"
    mag = Fraction(f, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(f, 8)) * Fraction(2) ** (e - 7)
    return sign * mag


def _brute_row_fp8(row_bytes: bytes, scales, k):
    return [Fraction(np.array([scales[i // 32]], np.uint16).view(np.float16).item()) * _e4m3_exact(c)
            for i, c in enumerate(row_bytes)]


def _brute_row_q6k(codes: bytes, recs: bytes, k):
    # The 6-bit code of element i: low 4 bits are nibble i of the super-block's
    # first 128 bytes read as one little-endian integer, high 2 bits are 2-bit
    # field i of its last 64 bytes read the same way; value = d * sc * (q - 32)
    # with sc the signed byte i // 16 of the record and d its fp16 tail.
    out = []
    for sb in range(k // 256):
        c = codes[sb * 192:(sb + 1) * 192]
        r = recs[sb * 18:(sb + 1) * 18]
        lo, hi = int.from_bytes(c[:128], "little"), int.from_bytes(c[128:], "little")
        d = Fraction(np.frombuffer(r[16:18], np.float16).item())
        for i in range(256):
            q = ((lo >> (4 * i)) & 0xF) | (((hi >> (2 * i)) & 0x3) << 4)
            sc = struct.unpack("b", r[i // 16:i // 16 + 1])[0]
            out.append(d * sc * (q - 32))
    return out


def _pack_q6k_superblock(q, sc, d_bits):
    # Bytes of one super-block from 256 codes (0..63), 16 signed sub-scales and
    # the fp16 bits of d, packed bit by bit (no vector tricks).
    lo = sum((qi & 0xF) << (4 * i) for i, qi in enumerate(q)).to_bytes(128, "little")
    hi = sum((qi >> 4) << (2 * i) for i, qi in enumerate(q)).to_bytes(64, "little")
    rec = struct.pack("16b", *sc) + struct.pack("<H", d_bits)
    return lo + hi, rec


def test_q6k_worked_example():
    # One row, K = 256.  d = 0.5 (fp16 0x3800); sub-block j has scale sc[j];
    # code q of element i is chosen so each value is easy to check by hand:
    # element 0 (sub-block 0, sc = 1): q = 63 -> 0.5 * 1 * 31 = 15.5
    # element 1 (sc = 1): q = 0 -> 0.5 * 1 * -32 = -16
    # element 16 (sub-block 1, sc = -2): q = 33 -> 0.5 * -2 * 1 = -1
    # element 255 (sub-block 15, sc = 127): q = 48 -> 0.5 * 127 * 16 = 1016
    # element 200 (sub-block 12, sc = -128): q = 31 -> 0.5 * -128 * -1 = 64
    # every other element: q = 32 -> 0.
    q = [32] * 256
    q[0], q[1], q[16], q[255], q[200] = 63, 0, 33, 48, 31
    sc = [1, -2] + [0] * 10 + [-128, 0, 0, 127]
    codes, rec = _pack_q6k_superblock(q, sc, 0x3800)
    got = oracle.dequant("q6k", np.frombuffer(codes, np.uint8).reshape(1, 192),
                         np.frombuffer(rec, np.uint8).reshape(1, 18), 1, 256, [0])[0]
    want = np.zeros(256)
    want[[0, 1, 16, 255, 200]] = [15.5, -16.0, -1.0, 1016.0, 64.0]
    assert np.array_equal(got, want)


def test_e4m3_decode_matches_torch_for_every_code():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_to_f64(c) for c in range(256)])
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(np.isnan(got), nan)  # 0x7F, 0xFF
    assert np.array_equal(got[~nan], ref[~nan])


def test_fp8_worked_example():
    # One row, K = 64 (two blocks).  Block 0 scale 0.5 (fp16 0x3800), block 1
    # scale 2 (0x4000).  E4M3 0x7E = 1.75 * 2^8 = 448 (the largest finite),
    # 0xFE = -448, 0x38 = 1.0, 0x3C = 1.5, 0x08 = 2^-6 (smallest normal),
    # 0x01 = 2^-9 (smallest subnormal), 0x80 = -0.
    row = np.zeros(64, np.uint8)
    row[[0, 1, 2, 3, 4, 5, 6, 32, 33]] = [0x7E, 0xFE, 0x38, 0x3C, 0x08, 0x01, 0x80, 0x3C, 0x01]
    scale = np.array([[0x3800, 0x4000]], np.uint16)
    got = oracle.dequant("fp8", row.reshape(1, 64), scale, 1, 64, [0])[0]
    want = np.zeros(64)
    want[[0, 1, 2, 3, 4, 5, 6]] = [224.0, -224.0, 0.5, 0.75, 2.0 ** -7, 2.0 ** -10, -0.0]
    want[[32, 33]] = [3.0, 2.0 ** -8]
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fmt", ["q4", "q8", "fp8", "q6k"])
def test_gemv_integer_exact_brute_force(fmt):
    # Power-of-two scales and small-integer x make every partial sum exact in
    # fp64, so the oracle must equal exact rational arithmetic bit for bit.
    rng = np.random.default_rng(7)
    n, k, m = 5, (512 if fmt == "q6k" else 96), 3
    scales = (np.array([0x3C00, 0x3800, 0x4000, 0x3400, 0x2C00], np.uint16)[
        rng.integers(0, 5, size=(n, k // 32))]).astype(np.uint16)
    if fmt == "q4":
        data = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
        rows = [_brute_row_q4(data[r].tobytes(), scales[r], k) for r in range(n)]
    elif fmt == "q8":
        data = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
        rows = [_brute_row_q8(data[r].tobytes(), scales[r], k) for r in range(n)]
    elif fmt == "fp8":
        codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)  # no NaN
        data = codes[rng.integers(0, codes.size, size=(n, k))]
        rows = [_brute_row_fp8(data[r].tobytes(), scales[r], k) for r in range(n)]
    else:
        nsb = k // 256
        data = rng.integers(0, 256, size=(n, nsb * 192), dtype=np.uint8)
        scales = np.zeros((n, nsb * 18), np.uint8)
        for r in range(n):
            for sb in range(nsb):
                scales[r, sb * 18:sb * 18 + 16] = rng.integers(-128, 128, 16).astype(np.int8).view(np.uint8)
                d = np.array([[0x3C00, 0x3800, 0x4000, 0x2C00][rng.integers(0, 4)]], np.uint16)
                scales[r, sb * 18 + 16:sb * 18 + 18] = d.view(np.uint8)
        rows = [_brute_row_q6k(data[r].tobytes(), scales[r].tobytes(), k) for r in range(n)]
    x = rng.integers(-9, 10, size=(m, k)).astype(np.float64)
    y = oracle.gemv(fmt, data, scales, n, k, x)
    for mi in range(m):
        for r in range(n):
            exact = sum(w * int(xv) for w, xv in zip(rows[r], x[mi]))
            assert y[mi, r] == float(exact)


def test_gemv_f32_is_matmul():
    # For fp32 weights the GEMV is a plain matrix product (library routine).
    rng = np.random.default_rng(3)
    n, k, m = 33, 70, 4  # non-square: a transposed operand cannot pass
    w = rng.standard_normal((n, k)).astype(np.float32)
    x = rng.standard_normal((m, k))
    y = oracle.gemv("f32", w, None, n, k, x)
    ref = x @ w.astype(np.float64).T
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_gemv_row_subset_and_batch_independence():
    w, s = synth.weight(40, 128, "q4", 0.02, 0, "pin_gemv")
    x = synth.normal((6, 128), 1.0, 0, "pin_x").numpy()
    full = oracle.gemv("q4", w, s, 40, 128, x)
    sub = oracle.gemv("q4", w, s, 40, 128, x, rows=[39, 0, 17])
    assert np.array_equal(sub, full[:, [39, 0, 17]])
    for mi in range(6):  # M-batched == M separate M=1 products
        one = oracle.gemv("q4", w, s, 40, 128, x[mi:mi + 1])
        assert np.array_equal(one[0], full[mi])


def test_quantiser_roundtrip_is_close():
    # The producer's blocks dequantise to within half a step of the draw.
    w = synth.normal((8, 64), 0.02, 0, "pin_quant")
    for fmt, qmax in (("q8", 127), ("q4", 7)):
        d, s = synth.quantize(w, fmt)
        deq = oracle.dequant(fmt, d, s, 8, 64, range(8))
        step = np.repeat(s.numpy().view(np.float16).astype(np.float64), 32, axis=1)
        assert np.all(np.abs(deq - w.numpy()) <= 0.5 * step * (1 + 1e-3) + 1e-9)
    # Q6K: within half a step d * sc of each sub-block of 16.
    w2 = synth.normal((4, 512), 0.02, 0, "pin_quant6")
    d, r = synth.quantize(w2, "q6k")
    deq = oracle.dequant("q6k", d, r, 4, 512, range(4))
    rec = r.numpy().reshape(4, 2, 18)
    dd = rec[:, :, 16:18].copy().view(np.float16).astype(np.float64)      # [4][2][1]
    step = np.repeat((dd * rec[:, :, :16].view(np.int8)).reshape(4, 32), 16, axis=1)
    assert np.all(np.abs(deq - w2.numpy()) <= 0.5 * step * (1 + 1e-3) + 1e-9)
    # FP8: within half a unit in the last place of E4M3 (3 fraction bits, so a
    # relative 2^-4), or half the subnormal step (2^-10) times the scale.
    d, s = synth.quantize(w, "fp8")
    deq = oracle.dequant("fp8", d, s, 8, 64, range(8))
    sc = np.repeat(s.numpy().view(np.float16).astype(np.float64), 32, axis=1)
    bound = np.maximum(np.abs(w.numpy()) * 2.0 ** -4, sc * 2.0 ** -10)
    assert np.all(np.abs(deq - w.numpy()) <= bound * (1 + 1e-3) + 1e-12)


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_constant_vector_closed_form():
    c, eps, h = 0.37, 1e-6, 64
    g = np.linspace(0.5, 1.5, h)
    out = oracle.rmsnorm(np.full((1, h), c), g, eps)
    np.testing.assert_allclose(out[0], c / math.sqrt(c * c + eps) * g, rtol=1e-15)


def test_rmsnorm_matches_torch():
    x = torch.randn(3, 256, dtype=torch.float64)
    g = torch.rand(256, dtype=torch.float64) + 0.5
    ref = F.rms_norm(x, (256,), g, eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.rmsnorm(x.numpy(), g.numpy(), 1e-6), ref, rtol=1e-13)


# ---------------------------------------------------------------- RoPE
def test_rope_position_zero_is_identity():
    z = np.random.default_rng(0).standard_normal((3, 64))
    assert np.array_equal(oracle.rope(z, 0, 1e4), z)


def test_rope_pairs_are_half_split_and_angles_closed_form():
    # hd = 4: theta_0 = 1, theta_1 = theta^(-1/2).  e_0 rotates into slot 2 (not
    # slot 1) by angle p; e_1 rotates into slot 3 by angle p * theta^-0.5.
    p, theta = 5, 1e4
    out = oracle.rope(np.eye(4), p, theta)
    a1 = p * theta ** -0.5
    np.testing.assert_allclose(out[0], [math.cos(p), 0, math.sin(p), 0], atol=1e-15)
    np.testing.assert_allclose(out[1], [0, math.cos(a1), 0, math.sin(a1)], atol=1e-15)
    np.testing.assert_allclose(out[2], [-math.sin(p), 0, math.cos(p), 0], atol=1e-15)


def test_rope_matches_complex_rotation_and_relative_position():
    rng = np.random.default_rng(1)
    hd, theta = 128, 1e4
    q, k = rng.standard_normal(hd), rng.standard_normal(hd)
    half = hd // 2
    freq = theta ** (-np.arange(half) * 2.0 / hd)
    for p in (1, 77, 8191):
        zc = (q[:half] + 1j * q[half:]) * np.exp(1j * p * freq)
        np.testing.assert_allclose(oracle.rope(q, p, theta),
                                   np.concatenate([zc.real, zc.imag]), atol=1e-12)
    # <R(p+s) q, R(p'+s) k> depends only on p - p'
    d0 = oracle.rope(q, 10, theta) @ oracle.rope(k, 3, theta)
    d1 = oracle.rope(q, 1010, theta) @ oracle.rope(k, 1003, theta)
    assert abs(d0 - d1) < 1e-10
    # per-pair norm is preserved
    r = oracle.rope(q, 4321, theta)
    np.testing.assert_allclose(r[:half] ** 2 + r[half:] ** 2, q[:half] ** 2 + q[half:] ** 2,
                               rtol=1e-12)


# ---------------------------------------------------------------- attention
def _cache(nkv, ld, hd, seed):
    g = np.random.default_rng(seed)
    return g.standard_normal((nkv, ld, hd)), g.standard_normal((nkv, ld, hd))


def test_attention_single_row_returns_that_value_row():
    kc, vc = _cache(2, 8, 16, 0)
    q = np.random.default_rng(1).standard_normal((4, 16))
    out = oracle.attention(q, kc, vc, 1)
    assert np.array_equal(out, vc[[0, 0, 1, 1], 0])  # exactly v_0 of each group


def test_attention_zero_query_is_mean_of_values():
    kc, vc = _cache(2, 10, 8, 2)
    out = oracle.attention(np.zeros((6, 8)), kc, vc, 7)
    np.testing.assert_allclose(out, vc[[0, 0, 0, 1, 1, 1], :7].mean(axis=1), rtol=1e-14)


def test_attention_two_rows_closed_form():
    hd = 4
    kc = np.zeros((1, 2, hd)); vc = np.zeros((1, 2, hd))
    kc[0, 0] = [1, 0, 0, 0]; kc[0, 1] = [0, 2, 0, 0]
    vc[0, 0] = [1, 2, 3, 4]; vc[0, 1] = [-1, 0, 5, 1]
    q = np.array([[3.0, 1.0, 0, 0]])
    s0, s1 = 3.0 / 2, 2.0 / 2  # <q, k_t> / sqrt(4)
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    np.testing.assert_allclose(oracle.attention(q, kc, vc, 2)[0],
                               w0 * vc[0, 0] + (1 - w0) * vc[0, 1], rtol=1e-15)


def test_attention_gqa_head_map_is_contiguous_groups():
    # Constant value rows per KV head: head h must return the constant of KV
    # head h // (nq/nkv).
    nq, nkv, hd, ld = 6, 3, 8, 5
    kc = np.random.default_rng(3).standard_normal((nkv, ld, hd))
    vc = np.zeros((nkv, ld, hd))
    for g in range(nkv):
        vc[g] = g + 1.0
    out = oracle.attention(np.random.default_rng(4).standard_normal((nq, hd)), kc, vc, ld)
    np.testing.assert_allclose(out[:, 0], [1, 1, 2, 2, 3, 3], rtol=1e-14)


def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(5)
    nq, nkv, hd, ld, L = 8, 2, 32, 50, 37
    kc, vc = rng.standard_normal((nkv, ld, hd)), rng.standard_normal((nkv, ld, hd))
    q = rng.standard_normal((nq, hd))
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None], torch.from_numpy(kc[:, :L])[None],
        torch.from_numpy(vc[:, :L])[None], enable_gqa=True)[0, :, 0].numpy()
    np.testing.assert_allclose(oracle.attention(q, kc, vc, L), ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("chunk", [1, 3, 32, 64, 128, 256, 300, 4096])
def test_splitk_equals_unsplit_for_every_chunk(chunk):
    rng = np.random.default_rng(chunk)
    nq, nkv, hd, ld, L = 4, 1, 16, 300, 299
    kc, vc = rng.standard_normal((nkv, ld, hd)) * 3, rng.standard_normal((nkv, ld, hd))
    q = rng.standard_normal((nq, hd))
    np.testing.assert_allclose(oracle.attention_splitk(q, kc, vc, L, chunk),
                               oracle.attention(q, kc, vc, L), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- SwiGLU, argmax
def test_silu_matches_torch():
    z = torch.linspace(-30, 30, 1001, dtype=torch.float64)
    np.testing.assert_allclose(oracle.silu(z.numpy()), F.silu(z).numpy(), rtol=1e-14, atol=1e-300)
    assert oracle.swiglu(np.array([0.0]), np.array([5.0]))[0] == 0.0


def test_argmax_lowest_index_on_ties_and_gap():
    l = np.array([[0.0, 3.0, 1.0, 3.0], [5.0, -1.0, 5.0, 4.0], [-2.0, -1.0, -3.0, -4.0]])
    tok, gap = oracle.argmax(l)
    assert tok.tolist() == [1, 0, 1]
    assert gap.tolist() == [0.0, 0.0, 1.0]
    perm = np.random.default_rng(0).permutation(1000)
    onehot = np.zeros(1000); onehot[perm[0]] = 1.0
    assert oracle.argmax(onehot)[0] == perm[0]
    with pytest.raises(ValueError):
        oracle.argmax(np.array([1.0, np.nan]))


# ---------------------------------------------------------------- whole step
def _torch_llama_step(shape, wts, xs, pos_list, caches):
    """An independent float64 forward written with torch library routines
    (rms_norm, sdpa with GQA, silu, matmul) and RoPE as a complex rotation."""
    S = shape
    nq, nkv, hd, I, H = S.n_heads, S.n_kv_heads, S.head_dim, S.intermediate, S.hidden
    half = hd // 2
    freq = torch.tensor(S.rope_theta, dtype=torch.float64) ** (
        -torch.arange(half, dtype=torch.float64) * 2.0 / hd)

    def rot(z, p):
        c = torch.complex(z[..., :half], z[..., half:]) * torch.polar(
            torch.ones(half, dtype=torch.float64), p * freq)
        return torch.cat([c.real, c.imag], -1)

    W = lambda t: t[0].to(torch.float64)
    x = torch.as_tensor(xs, dtype=torch.float64).clone()
    for l, lw in enumerate(wts.layers):
        u = F.rms_norm(x, (H,), lw.attn_gamma.double(), eps=S.rms_eps)
        qkv = u @ W(lw.wqkv).T
        att = []
        for i, p in enumerate(pos_list):
            q = rot(qkv[i, :nq * hd].view(nq, hd), p)
            k = rot(qkv[i, nq * hd:(nq + nkv) * hd].view(nkv, hd), p)
            v = qkv[i, (nq + nkv) * hd:].view(nkv, hd)
            caches[l][0][i][:, p] = k
            caches[l][1][i][:, p] = v
            o = F.scaled_dot_product_attention(
                q[None, :, None], caches[l][0][i][None, :, :p + 1],
                caches[l][1][i][None, :, :p + 1], enable_gqa=True)
            att.append(o[0, :, 0].reshape(-1))
        x = x + torch.stack(att) @ W(lw.wo).T
        u = F.rms_norm(x, (H,), lw.ffn_gamma.double(), eps=S.rms_eps)
        gu = u @ W(lw.wgu).T
        x = x + (F.silu(gu[:, :I]) * gu[:, I:]) @ W(lw.wd).T
    u = F.rms_norm(x, (H,), wts.out_gamma.double(), eps=S.rms_eps)
    return x, u @ W(wts.lm_head).T


def test_decoder_oracle_matches_independent_torch_forward():
    S = synth.TINY_LLAMA_F32
    wts = synth.decoder_weights(S, seed=0, gamma="random")
    m, steps = 2, 4
    orc = oracle.DecoderOracle(S, wts, m, S.max_len)
    caches = [(torch.zeros(m, S.n_kv_heads, S.max_len, S.head_dim, dtype=torch.float64),
               torch.zeros(m, S.n_kv_heads, S.max_len, S.head_dim, dtype=torch.float64))
              for _ in wts.layers]
    tok = synth.first_tokens(S, m).tolist()
    for step in range(steps):
        x = wts.embed[tok].double().numpy()
        pos = [step, step + 3]  # sequences at different positions
        got = orc.step(x, pos)
        hid, logits = _torch_llama_step(S, wts, x, pos, caches)
        np.testing.assert_allclose(got["hidden"], hid.numpy(), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(got["logits"], logits.numpy(), rtol=1e-10, atol=1e-12)
        tok = got["tok"].tolist()


def test_decoder_oracle_batched_equals_separate_sequences():
    S = synth.TINY_LLAMA_F32
    wts = synth.decoder_weights(S, seed=1)
    x = synth.normal((3, S.hidden), 1.0, 1, "pin_x3").numpy()
    pos = [0, 0, 0]
    both = oracle.DecoderOracle(S, wts, 3, S.max_len).step(x, pos)
    for i in range(3):
        one = oracle.DecoderOracle(S, wts, 1, S.max_len).step(x[i:i + 1], pos[i:i + 1])
        assert np.array_equal(one["logits"][0], both["logits"][i])
        assert np.array_equal(one["hidden"][0], both["hidden"][i])


def _torch_llama_prefill(shape, wts, xs, start, ctx):
    """Prompt ingestion written independently in matrix form: all T rows of a
    layer at once, RoPE as a complex rotation at positions start..start+T-1,
    and attention as torch sdpa over [context rows; prompt rows] with an
    explicit causal mask (row t sees keys j <= start + t)."""
    S = shape
    nq, nkv, hd, I, H = S.n_heads, S.n_kv_heads, S.head_dim, S.intermediate, S.hidden
    half = hd // 2
    freq = torch.tensor(S.rope_theta, dtype=torch.float64) ** (
        -torch.arange(half, dtype=torch.float64) * 2.0 / hd)
    x = torch.as_tensor(xs, dtype=torch.float64).clone()
    T = x.shape[0]
    pos = torch.arange(start, start + T, dtype=torch.float64)

    def rot(z):  # z [T][heads][hd]
        c = torch.complex(z[..., :half], z[..., half:]) * torch.polar(
            torch.ones(T, 1, half, dtype=torch.float64), pos[:, None, None] * freq)
        return torch.cat([c.real, c.imag], -1)

    W = lambda t: t[0].to(torch.float64)
    mask = torch.arange(start + T)[None, :] <= (start + torch.arange(T))[:, None]
    ks, vs = [], []
    for l, lw in enumerate(wts.layers):
        u = F.rms_norm(x, (H,), lw.attn_gamma.double(), eps=S.rms_eps)
        qkv = u @ W(lw.wqkv).T
        q = rot(qkv[:, :nq * hd].view(T, nq, hd))
        k = rot(qkv[:, nq * hd:(nq + nkv) * hd].view(T, nkv, hd))
        v = qkv[:, (nq + nkv) * hd:].view(T, nkv, hd)
        K = torch.cat([ctx[l][0], k.transpose(0, 1)], 1)  # [nkv][start+T][hd]
        V = torch.cat([ctx[l][1], v.transpose(0, 1)], 1)
        ks.append(K)
        vs.append(V)
        o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], K[None], V[None],
                                           attn_mask=mask, enable_gqa=True)
        x = x + o[0].transpose(0, 1).reshape(T, nq * hd) @ W(lw.wo).T
        u = F.rms_norm(x, (H,), lw.ffn_gamma.double(), eps=S.rms_eps)
        gu = u @ W(lw.wgu).T
        x = x + (F.silu(gu[:, :I]) * gu[:, I:]) @ W(lw.wd).T
    u = F.rms_norm(x, (H,), wts.out_gamma.double(), eps=S.rms_eps)
    return x, u @ W(wts.lm_head).T, ks, vs


@pytest.mark.parametrize("start", [0, 5])
def test_prefill_oracle_matches_masked_matrix_form(start):
    S = synth.TINY_LLAMA_F32
    wts = synth.decoder_weights(S, seed=3, gamma="random")
    T, seq = 7, 1
    ctx = [(synth.normal((S.n_kv_heads, start, S.head_dim), 1.0, 3, f"pf_k{l}").double(),
            synth.normal((S.n_kv_heads, start, S.head_dim), 1.0, 3, f"pf_v{l}").double())
           for l in range(S.n_layers)]
    orc = oracle.DecoderOracle(S, wts, 2, S.max_len)
    for l in range(S.n_layers):
        orc.set_context(l, seq, ctx[l][0], ctx[l][1])
    toks = synth.uniform_int((T,), 0, S.vocab - 1, 3, "pf_tok")
    x = wts.embed[toks].double().numpy()
    got = orc.prefill(seq, x, start)
    hid, logits, ks, vs = _torch_llama_prefill(S, wts, x, start, ctx)
    np.testing.assert_allclose(got["hidden"], hid.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(got["logits"], logits.numpy(), rtol=1e-10, atol=1e-12)
    for l in range(S.n_layers):
        np.testing.assert_allclose(orc.kc[l][seq, :, :start + T], ks[l].numpy(), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(orc.vc[l][seq, :, :start + T], vs[l].numpy(), rtol=1e-12, atol=1e-13)
        assert not orc.kc[l][0].any() and not orc.vc[l][0].any()  # the other slot is untouched


def test_prefill_oracle_equals_one_token_steps():
    S = synth.TINY_LLAMA_F32
    wts = synth.decoder_weights(S, seed=4)
    toks = synth.uniform_int((6,), 0, S.vocab - 1, 4, "pf_tok2")
    x = wts.embed[toks].double().numpy()
    a = oracle.DecoderOracle(S, wts, 1, S.max_len).prefill(0, x, 2)
    b = oracle.DecoderOracle(S, wts, 1, S.max_len)
    for t in range(6):
        one = b.step(x[t:t + 1], [2 + t])
        assert np.array_equal(one["hidden"][0], a["hidden"][t])
        assert np.array_equal(one["logits"][0], a["logits"][t])
