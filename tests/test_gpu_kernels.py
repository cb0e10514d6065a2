"""Parity of each HIP step kernel with the CPU oracle, called through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemv_flash_amd as rra
import synth
from gpu_common import DEV, assert_close, banner, host, u32

pytestmark = pytest.mark.gpu

POW2_SCALES = np.array([0x3C00, 0x3800, 0x4000, 0x3400, 0x2C00], np.uint16)  # 1, .5, 2, .25, 1/16


# ---------------------------------------------------------------- layout
@pytest.mark.parametrize("fmt", ["q4", "q8", "fp8"])
@pytest.mark.parametrize("n,k", [(16, 32), (37, 96), (300, 416), (33, 160)])
def test_repack_roundtrip_bit_exact(fmt, n, k):
    banner("repack", fmt, n, k)
    data, scale = synth.weight(n, k, fmt, 0.02, 0, f"rp{n}x{k}", DEV)
    w = rra.device_weight(data, scale, fmt)
    assert w.layout == rra.RRA_TILED and w.data.numel() == rra.rra_tiled_bytes(fmt, n, k)
    d2, s2 = torch.full_like(data, 0x5A), torch.full_like(scale, 0x1234)
    rra.rra_unpack_weight(w, d2, s2)
    torch.cuda.synchronize()
    assert torch.equal(d2, data) and torch.equal(s2, scale)


# ---------------------------------------------------------------- GEMV
def _gemv(fmt, data, scale, x, m):
    n = data.shape[0]
    w = rra.device_weight(data, scale, fmt)
    y = torch.full((m, n), float("nan"), device=DEV)
    nb = rra.rra_batched_gemv_workspace_bytes(w, m)
    # poisoned scratch: nothing may depend on its previous contents
    ws = torch.full((max(nb, 4),), 0xFF, dtype=torch.uint8, device=DEV)
    rra.rra_batched_gemv(w, x, y, m, ws)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("m", [1, 3, 16, 17, 32])
@pytest.mark.parametrize("n,k", [(16, 32), (37, 96), (300, 416), (1000, 2048), (64, 14336)])
@pytest.mark.parametrize("fmt", ["q4", "q8", "fp8", "f32"])
def test_gemv_matches_oracle(fmt, n, k, m):
    banner("gemv", fmt, n, k, m)
    data, scale = synth.weight(n, k, fmt, 0.02, 0, f"g{n}x{k}", DEV)
    x = synth.normal((m, k), 1.0, 0, f"gx{m}x{k}", DEV)
    y = _gemv(fmt, data, scale, x, m)
    ref = oracle.gemv(fmt, data, scale, n, k, host(x))
    assert_close(y, ref, what=f"gemv {fmt} {n}x{k} m={m}")


@pytest.mark.parametrize("m", [1, 5, 32])
@pytest.mark.parametrize("fmt", ["q4", "q8", "fp8"])
def test_gemv_integer_exact(fmt, m):
    # Power-of-two scales and small integer inputs: every partial sum is exact
    # in fp32 as well as in the oracle's fp64, so the results must be equal.
    # FP8: scale 1 and codes with exponents 6..9 (|value| in [0.5, 16), 4
    # significant bits) keep every sum within fp32's 24 bits.
    banner("gemv exact", fmt, m)
    n, k = 70, 640
    g = np.random.default_rng(11)
    scale = torch.from_numpy(POW2_SCALES[g.integers(0, 5, size=(n, k // 32))].view(np.int16)).to(DEV)
    if fmt == "q4":
        data = torch.from_numpy(g.integers(0, 256, size=(n, k // 2), dtype=np.uint8)).to(DEV)
    elif fmt == "q8":
        data = torch.from_numpy(g.integers(-127, 128, size=(n, k), dtype=np.int8)).to(DEV)
    else:
        codes = np.array([s << 7 | e << 3 | f for s in (0, 1) for e in range(6, 10) for f in range(8)],
                         np.uint8)
        data = torch.from_numpy(codes[g.integers(0, codes.size, size=(n, k))]).to(DEV)
        scale = torch.full((n, k // 32), 0x3C00, dtype=torch.int16, device=DEV)
    x = torch.from_numpy(g.integers(-8, 9, size=(m, k)).astype(np.float32)).to(DEV)
    y = _gemv(fmt, data, scale, x, m)
    ref = oracle.gemv(fmt, data, scale, n, k, host(x))
    assert np.array_equal(host(y).astype(np.float64), ref)


def test_gemv_batch_rows_independent():
    # Each sequence's result does not depend on the other sequences in the batch.
    data, scale = synth.weight(512, 1024, "q4", 0.02, 0, "gind", DEV)
    x = synth.normal((16, 1024), 1.0, 0, "gindx", DEV)
    full = _gemv("q4", data, scale, x, 16)
    for i in (0, 7, 15):
        one = _gemv("q4", data, scale, x[i:i + 1].contiguous(), 1)
        assert torch.equal(one[0], full[i])


FULL_SHAPES = [
    ("q8", 1152, 896), ("q8", 896, 896), ("q8", 9728, 896), ("q8", 896, 4864), ("q8", 151936, 896),
    ("q4", 2048, 1536), ("q4", 1536, 1536), ("q4", 17920, 1536), ("q4", 1536, 8960),
    ("q4", 151936, 1536),
    ("q4", 6144, 4096), ("q4", 4096, 4096), ("q4", 28672, 4096), ("q4", 4096, 14336),
    ("q4", 128256, 4096),
    ("fp8", 151936, 896), ("fp8", 128256, 4096), ("fp8", 4096, 14336),
]


@pytest.mark.parametrize("fmt,n,k", FULL_SHAPES)
def test_gemv_full_shapes_sampled_rows(fmt, n, k):
    # Every GEMV shape of the three quantised decoders at M = 1, 17 and 32, with
    # the split-K launch the decode step uses; the oracle computes sampled rows.
    banner("gemv full", fmt, n, k)
    data, scale = synth.weight(n, k, fmt, 0.02, 0, f"full{n}x{k}", DEV)
    hd, hs = host(data), host(scale)
    rows = sorted(set(np.random.default_rng(n).integers(0, n, 120).tolist()) | {0, n - 1, n - 17})
    for m in (1, 17, 32):
        x = synth.normal((m, k), 1.0, 0, f"fullx{m}x{k}", DEV)
        y = _gemv(fmt, data, scale, x, m)
        ref = oracle.gemv(fmt, hd, hs, n, k, host(x), rows=rows)
        assert_close(host(y)[:, rows], ref, what=f"gemv {fmt} {n}x{k} m={m}")


@pytest.mark.parametrize("m", [17, 32])
def test_gemv_three_row_tiles_ragged(m):
    # A short-split shape that takes three row tiles per wave at M > 16 (380
    # row tiles: 256 workgroups of 12 instead of 384 of 8), with a ragged
    # last workgroup (8 of its 12 row tiles) and a partial last row tile.
    n, k = 6075, 4096
    banner("gemv rpw3", n, k, m)
    data, scale = synth.weight(n, k, "q4", 0.02, 0, "rpw3", DEV)
    hd, hs = host(data), host(scale)
    rows = sorted(set(np.random.default_rng(3).integers(0, n, 80).tolist())
                  | set(range(n - 40, n)) | {0, 6063, 6064})
    x = synth.normal((m, k), 1.0, 0, f"rpw3x{m}", DEV)
    y = _gemv("q4", data, scale, x, m)
    ref = oracle.gemv("q4", hd, hs, n, k, host(x), rows=rows)
    assert_close(host(y)[:, rows], ref, what=f"gemv rpw3 m={m}")


@pytest.mark.parametrize("m", [17, 32])
def test_gemv_long_split_two_row_tiles_ragged(m):
    # A long-split shape (8 splits of 14 K tiles) whose plan has one row tile
    # per wave, launched with two at M > 16 (254 row tiles: 32 workgroups of
    # 8), with a ragged last workgroup (6 of its 8 row tiles) and a partial
    # last row tile (8 of 16 rows).
    n, k = 4056, 14336
    banner("gemv long rpw2", n, k, m)
    data, scale = synth.weight(n, k, "q4", 0.02, 0, "rpw2long", DEV)
    hd, hs = host(data), host(scale)
    rows = sorted(set(np.random.default_rng(2).integers(0, n, 80).tolist())
                  | set(range(n - 40, n)) | {0, 4031, 4032})
    x = synth.normal((m, k), 1.0, 0, f"rpw2longx{m}", DEV)
    y = _gemv("q4", data, scale, x, m)
    ref = oracle.gemv("q4", hd, hs, n, k, host(x), rows=rows)
    assert_close(host(y)[:, rows], ref, what=f"gemv long rpw2 m={m}")


# ---------------------------------------------------------------- KV scatter
@pytest.mark.parametrize("m,nkv,hd,max_len", [(1, 2, 64, 16), (5, 8, 128, 300), (32, 2, 128, 1152)])
def test_kv_scatter_bit_exact(m, nkv, hd, max_len):
    banner("scatter", m, nkv, hd, max_len)
    # Sentinel rows: value encodes (sequence, head, column).
    i, g, d = np.meshgrid(np.arange(m), np.arange(nkv), np.arange(hd), indexing="ij")
    rows = (i * 1e6 + g * 1e3 + d).astype(np.float32).reshape(m, nkv * hd)
    k_rows = torch.from_numpy(rows).to(DEV)
    v_rows = -k_rows
    kc = torch.full((m, nkv, max_len, hd), 7.0, device=DEV)
    vc = torch.full_like(kc, 9.0)
    pos = [(3 * s + 1) % max_len for s in range(m)]
    pos[-1] = max_len - 1
    if m > 1:
        pos[0] = max_len + 5  # out of range: must not be written
    rra.rra_kv_scatter(k_rows, v_rows, kc, vc, u32(pos), m, nkv, hd, max_len)
    torch.cuda.synchronize()
    ek = np.full((m, nkv, max_len, hd), 7.0, np.float32)
    ev = np.full_like(ek, 9.0)
    for s in range(m):
        if pos[s] < max_len:
            ek[s, :, pos[s]] = rows[s].reshape(nkv, hd)
            ev[s, :, pos[s]] = -rows[s].reshape(nkv, hd)
    assert np.array_equal(host(kc), ek) and np.array_equal(host(vc), ev)


# ---------------------------------------------------------------- flash decode
def _fd_run(q, kc, vc, lens, m, nq, nkv, hd, max_len, chunk):
    out = torch.full((m, nq, hd), 123.0, device=DEV)
    nb = rra.rra_flash_decode_workspace_bytes(m, nq, nkv, hd, max_len, chunk)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    rra.rra_flash_decode(q, kc, vc, u32(lens), out, m, nq, nkv, hd, max_len, chunk, ws)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("chunk", [32, 64, 96, 256, 0])
@pytest.mark.parametrize("nq,nkv", [(8, 2), (14, 2), (4, 4), (16, 2), (12, 2)])
@pytest.mark.parametrize("hd", [64, 128])
def test_flash_decode_matches_unsplit_oracle(hd, nq, nkv, chunk):
    banner("fd", hd, nq, nkv, chunk)
    a = synth.Attention("t", 4, nq, nkv, hd, 300, 1, 300, ())
    q, kc, vc, _, _, _ = synth.attention_inputs(a, seed=hd + nq, device=DEV)
    lens = [1, 37, 300, 129]
    out = _fd_run(q, kc, vc, lens, 4, nq, nkv, hd, 300, chunk)
    hq, hk, hv = host(q), host(kc), host(vc)
    for s, L in enumerate(lens):
        ref = oracle.attention(hq[s], hk[s], hv[s], L)
        assert_close(out[s], ref, what=f"fd seq {s} L={L}")


def test_flash_decode_zero_length_leaves_output():
    a = synth.Attention("t", 2, 8, 2, 128, 64, 1, 64, ())
    q, kc, vc, _, _, _ = synth.attention_inputs(a, device=DEV)
    out = _fd_run(q, kc, vc, [0, 5], 2, 8, 2, 128, 64, 32)
    assert torch.all(out[0] == 123.0)
    assert_close(out[1], oracle.attention(host(q)[1], host(kc)[1], host(vc)[1], 5))


@pytest.mark.parametrize("hd,nq,nkv", [(64, 14, 2), (128, 32, 8), (128, 12, 2)])
def test_flash_decode_head_split_is_bitwise_neutral(hd, nq, nkv):
    # With a fixed chunk, one sequence alone runs on a small grid, where each
    # KV head's query heads are dealt to several workgroups; in a batch of 24
    # the grid is large and one workgroup serves the whole group.  Every head's
    # arithmetic is the same either way: the outputs must be equal bitwise.
    m, max_len, chunk = 24, 512, 32
    banner("fd head split", hd, nq, nkv)
    a = synth.Attention("t", m, nq, nkv, hd, max_len, 1, max_len, ())
    q, kc, vc, _, _, lens = synth.attention_inputs(a, seed=7, device=DEV)
    L = lens.tolist()
    both = _fd_run(q, kc, vc, L, m, nq, nkv, hd, max_len, chunk)
    for s in (0, 5, m - 1):
        one = _fd_run(q[s:s + 1].contiguous(), kc[s:s + 1].contiguous(), vc[s:s + 1].contiguous(),
                      L[s:s + 1], 1, nq, nkv, hd, max_len, chunk)
        assert torch.equal(one[0], both[s]), f"seq {s} L={L[s]}"


@pytest.mark.parametrize("m", [7, 32])
def test_flash_decode_batch_order_is_bitwise_neutral(m):
    # The standalone call's workgroups take the sequences longest first.
    # Which workgroup serves a sequence must not change its result: the
    # batch in reverse order gives the same rows, reversed, bit for bit.
    hd, nq, nkv, max_len, chunk = 64, 8, 2, 512, 64
    banner("fd batch order", m)
    a = synth.Attention("t", m, nq, nkv, hd, max_len, 1, max_len, ())
    q, kc, vc, _, _, lens = synth.attention_inputs(a, seed=11, device=DEV)
    L = lens.tolist()
    fwd = _fd_run(q, kc, vc, L, m, nq, nkv, hd, max_len, chunk)
    r = list(range(m - 1, -1, -1))
    rev = _fd_run(q[r].contiguous(), kc[r].contiguous(), vc[r].contiguous(), L[::-1], m, nq, nkv,
                  hd, max_len, chunk)
    assert torch.equal(rev.flip(0), fwd)


def test_flash_decode_full_size_every_chunk():
    # 32 sequences, 32 Q / 8 KV heads, hd 128, lengths uniform in [1, 8192],
    # cache 8192 rows; the new row is scattered at L-1 first.  Each split-K
    # chunk size must equal unsplit softmax attention.
    a = synth.FLASH_DECODE_M32
    banner("fd full", a.name)
    q, kc, vc, kn, vn, lens = synth.attention_inputs(a, seed=0, device=DEV)
    L = lens.tolist()
    rra.rra_kv_scatter(kn.reshape(a.m, -1), vn.reshape(a.m, -1), kc, vc, u32([l - 1 for l in L]),
                       a.m, a.n_kv_heads, a.head_dim, a.max_len)
    torch.cuda.synchronize()
    hq = host(q)
    refs = []
    for s in range(a.m):
        refs.append(oracle.attention(hq[s], host(kc[s, :, :L[s]]), host(vc[s, :, :L[s]]), L[s]))
    ref = np.stack(refs)
    for chunk in list(a.chunks) + [0]:
        out = _fd_run(q, kc, vc, L, a.m, a.n_heads, a.n_kv_heads, a.head_dim, a.max_len, chunk)
        assert_close(out, ref, what=f"fd full chunk={chunk}")


def test_flash_decode_llama8b_shape_split_cap():
    # The 8B-shaped decode step's attention launch: 32 sequences, 32 Q / 8 KV
    # heads, hd 128, a 4160-row cache, where the library's choice is 5 splits of
    # <= 832 rows (the split cap).  Lengths straddle the split and row-count
    # boundaries; the library's choice and the 8-split size both must equal
    # unsplit softmax attention.
    m, nq, nkv, hd, max_len = 32, 32, 8, 128, 4160
    banner("fd 8b shape", m, nq, nkv, hd, max_len)
    assert rra.rra_flash_decode_chunk(m, nkv, max_len, 0) == 832
    a = synth.Attention("t", m, nq, nkv, hd, max_len, 1, max_len, ())
    q, kc, vc, _, _, lens = synth.attention_inputs(a, seed=11, device=DEV)
    edge = [1, 2, 4, 5, 6, 831, 832, 833, 1664, 1665, 4159, 4160]
    L = edge + [int(v) for v in lens.tolist()[len(edge):]]
    hq = host(q)
    ref = np.stack([oracle.attention(hq[s], host(kc[s, :, :L[s]]), host(vc[s, :, :L[s]]), L[s])
                    for s in range(m)])
    for chunk in (0, 544):
        out = _fd_run(q, kc, vc, L, m, nq, nkv, hd, max_len, chunk)
        assert_close(out, ref, what=f"fd 8b shape chunk={chunk}")


# ---------------------------------------------------------------- HBM read probe
@pytest.mark.parametrize("n,blocks", [(4, 1), (1000, 3), (1 << 20, 37), ((1 << 20) + 12, 256)])
def test_hbm_read_reads_every_value(n, blocks):
    # Small integers: every block sum and the total are exact in fp32.
    g = torch.Generator(device="cpu").manual_seed(n)
    buf = torch.randint(-3, 4, (n,), generator=g).to(torch.float32)
    sums = torch.full((blocks,), float("nan"), device=DEV)
    rra.rra_hbm_read(buf.to(DEV), sums)
    torch.cuda.synchronize()
    assert host(sums).astype(np.float64).sum() == float(buf.double().sum())


def test_hbm_read_rejects_bad_arguments():
    sums = torch.zeros(4, device=DEV)
    buf = torch.zeros(8, device=DEV)
    with pytest.raises(rra.RraError, match="multiple of 16"):
        rra.rra_hbm_read(buf[:3], sums)
    with pytest.raises(rra.RraError, match="multiple of 16"):
        rra.rra_hbm_read(buf[1:5], sums)
    with pytest.raises(rra.RraError, match="blocks=0"):
        rra.rra_hbm_read(buf, sums, blocks=0)


# ---------------------------------------------------------------- elementwise
@pytest.mark.parametrize("m,h", [(1, 256), (3, 896), (32, 4096), (2, 4100)])
def test_rmsnorm(m, h):
    x = synth.normal((m, h), 1.0, 0, f"rn{h}", DEV) * 3.0
    gamma = 1.0 + synth.normal((h,), 0.1, 0, f"rng{h}", DEV)
    out = torch.empty_like(x)
    rra.rra_rmsnorm(x, gamma, out, m, h, 1e-6)
    torch.cuda.synchronize()
    assert_close(out, oracle.rmsnorm(host(x), host(gamma), 1e-6))


@pytest.mark.parametrize("hd,heads", [(64, 14), (128, 32)])
def test_rope(hd, heads):
    m, max_len, theta = 4, 8192, 1e4
    table = torch.empty(max_len * hd, device=DEV)
    rra.rra_rope_table(table, max_len, hd, theta)
    z = synth.normal((m, heads, hd), 1.0, 0, f"rope{hd}", DEV)
    pos = [0, 1, 777, 8191]
    zz = z.clone()
    rra.rra_rope(zz, u32(pos), table, m, heads, hd, max_len)
    torch.cuda.synchronize()
    hz = host(z)
    for s in range(m):
        assert_close(zz[s], oracle.rope(hz[s], pos[s], theta), what=f"rope pos {pos[s]}")


def test_swiglu():
    m, n = 3, 4864
    gate = synth.normal((m, n), 4.0, 0, "swg", DEV)
    up = synth.normal((m, n), 1.0, 0, "swu", DEV)
    out = torch.empty_like(gate)
    rra.rra_swiglu(gate, up, out, m, n)
    torch.cuda.synchronize()
    assert_close(out, oracle.swiglu(host(gate), host(up)))


@pytest.mark.parametrize("v", [1024, 128256, 151936, 4097])
def test_argmax_bit_exact(v):
    m = 5
    l = synth.normal((m, v), 1.0, 0, f"am{v}", DEV)
    l[1, 100] = 50.0
    l[1, v - 1] = 50.0          # tie: lowest index wins
    l[2, :] = -3.0              # all equal
    l[3, v - 1] = 1e30          # maximum in the ragged tail
    tok = torch.full((m,), -1, dtype=torch.int32, device=DEV)
    ws = torch.empty(rra.rra_argmax_workspace_bytes(m, v), dtype=torch.uint8, device=DEV)
    rra.rra_argmax(l, tok, m, v, ws)
    torch.cuda.synchronize()
    ref, _ = oracle.argmax(host(l))
    assert host(tok).tolist() == ref.tolist()
    assert host(tok)[1] == 100 and host(tok)[2] == 0 and host(tok)[3] == v - 1


@pytest.mark.parametrize("fmt,n,k", [("q4", 300, 416), ("q8", 1152, 896), ("q4", 4096, 14336),
                                     ("q8", 896, 4864), ("q4", 37, 128)])
@pytest.mark.parametrize("m", [1, 3, 8])
def test_valu_gemv_matches_oracle(fmt, n, k, m):
    # the vector-ALU comparison GEMV on the same tiled weights
    data, scale = synth.weight(n, k, fmt, 0.02, 5, f"valu_{fmt}_{n}", DEV)
    w = rra.device_weight(data, scale, fmt)
    x = synth.normal((m, k), 1.0, 5, f"valu_x{m}", DEV)
    y = torch.full((m, n), float("nan"), device=DEV)
    ws = torch.empty(max(4, rra.rra_batched_gemv_workspace_bytes(w, m)), dtype=torch.uint8,
                     device=DEV)
    rra.rra_batched_gemv_valu(w, x, y, m, ws)
    torch.cuda.synchronize()
    ref = oracle.gemv(fmt, data, scale, n, k, host(x))
    assert_close(y, ref, what=f"valu {fmt} {n}x{k} m={m}")
