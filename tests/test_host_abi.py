"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/rra.h declares, and rejects bad arguments before any
device work."""
import ctypes

import pytest
import torch

import quantized_gemv_flash_amd as rra


def test_library_exports_every_declared_function():
    names = rra.header_functions()
    assert len(names) >= 20
    missing = [n for n in names if not hasattr(rra.lib, n)]
    assert not missing, missing
    assert rra.lib.rra_version() == 1


def test_status_names():
    assert rra.lib.rra_status_name(0) == b"RRA_OK"
    assert rra.lib.rra_status_name(4) == b"RRA_ECAPTURE"


@pytest.mark.parametrize("fmt,n,k,expect", [
    ("q4", 37, 96, 3 * 1 * 1152),        # ragged rows and a partial K tile
    ("q4", 128256, 4096, 8016 * 32 * 1152),
    ("q8", 1152, 896, 72 * 14 * 1088),
    ("q8", 16, 32, 1 * 1 * 1088),
    ("q4", 16, 33, 0),                     # K not a multiple of 32
    ("f32", 16, 32, 0),                    # fp32 is never tiled
])
def test_tiled_bytes(fmt, n, k, expect):
    assert rra.rra_tiled_bytes(fmt, n, k) == expect


def _fake_weight(fmt, n, k, layout=rra.RRA_TILED):
    t = torch.zeros(16, dtype=torch.uint8)  # never dereferenced: validation fails first
    return rra.Weight(fmt, n, k, t, t if layout == rra.RRA_PLANAR and fmt != "f32" else None, layout)


@pytest.mark.parametrize("m", [0, 33, -1])
def test_gemv_rejects_bad_batch(m):
    w = _fake_weight("q4", 64, 128)
    x = torch.zeros(4)
    with pytest.raises(rra.RraError) as e:
        rra.rra_batched_gemv(w, x, x, m)
    assert e.value.status == rra.RRA_EINVAL and "1..32" in str(e.value)


def test_gemv_rejects_planar_quantised_weight():
    w = _fake_weight("q8", 64, 128, rra.RRA_PLANAR)
    x = torch.zeros(4)
    with pytest.raises(rra.RraError) as e:
        rra.rra_batched_gemv(w, x, x, 1)
    assert "rra_repack_weight" in str(e.value)


def test_gemv_rejects_k_not_multiple_of_32():
    w = _fake_weight("q4", 64, 100)
    x = torch.zeros(4)
    with pytest.raises(rra.RraError, match="multiple of 32"):
        rra.rra_batched_gemv(w, x, x, 1)


def test_gemv_workspace_sizes():
    # Q8/Q4: the activation image (per 32-column block, 16 sequences per column
    # tile, an fp16 high and low part: 2 x 1 KiB), then the split-K partial sums.
    w = _fake_weight("q4", 4096, 14336)
    nb = rra.rra_batched_gemv_workspace_bytes(w, 32)
    img = (14336 // 32) * 2 * 2 * 1024
    assert nb > img and (nb - img) % (32 * 4096 * 4) == 0
    assert rra.rra_batched_gemv_workspace_bytes(w, 0) == 0
    # a short matrix is not split: the image alone (one column tile for m <= 16)
    w = _fake_weight("q8", 16, 64)
    assert rra.rra_batched_gemv_workspace_bytes(w, 1) == 2 * 1 * 2 * 1024
    assert rra.rra_batched_gemv_workspace_bytes(w, 17) == 2 * 2 * 2 * 1024
    w = _fake_weight("f32", 16, 64, rra.RRA_PLANAR)
    assert rra.rra_batched_gemv_workspace_bytes(w, 1) == 0


def test_gemv_requires_workspace():
    w = _fake_weight("q8", 64, 128)
    x = torch.zeros(4)
    with pytest.raises(rra.RraError) as e:
        rra.rra_batched_gemv(w, x, x, 1)
    assert e.value.status == rra.RRA_ENOTINIT and "workspace" in str(e.value)


def test_flash_decode_sizes_and_validation():
    # chunk chosen from (m, nkv, max_len); partials are m*nq*nc*(hd+1) floats
    c = rra.rra_flash_decode_chunk(32, 8, 8192, 0)
    assert c % 32 == 0 and 64 <= c <= 1024
    # chunk 0: enough for the default rule and for every tuner candidate (the
    # smallest candidate rows per split give the most partials)
    nc = -(-8192 // min([c] + [ch for ch, _ in rra.rra_flash_decode_candidates(32, 32, 8, 8192)]))
    assert rra.rra_flash_decode_workspace_bytes(32, 32, 8, 128, 8192, 0) == 32 * 32 * nc * 129 * 4
    assert rra.rra_flash_decode_workspace_bytes(32, 32, 8, 128, 8192, c) == \
        32 * 32 * -(-8192 // c) * 129 * 4
    assert rra.rra_flash_decode_workspace_bytes(1, 14, 2, 64, 768, 64) == 14 * 12 * 65 * 4
    assert rra.rra_flash_decode_workspace_bytes(1, 12, 8, 128, 64, 0) == 0   # nq % nkv
    assert rra.rra_flash_decode_workspace_bytes(1, 8, 1, 96, 64, 0) == 0     # hd
    assert rra.rra_flash_decode_workspace_bytes(1, 8, 1, 64, 64, 48) == 0    # chunk % 32
    t = torch.zeros(4)
    with pytest.raises(rra.RraError, match="group size|nq/nkv"):
        rra.rra_flash_decode(t, t, t, t, t, 1, 18, 2, 64, 16, 0, t)


def test_kv_scatter_and_step_kernels_validate_before_launch():
    t = torch.zeros(4)
    with pytest.raises(rra.RraError, match="1..32"):
        rra.rra_kv_scatter(t, t, t, t, t, 0, 1, 64, 16)
    with pytest.raises(rra.RraError):
        rra.rra_rmsnorm(t, t, t, 1, 0, 1e-6)
    with pytest.raises(rra.RraError):
        rra.rra_rope(t, t, t, 1, 1, 63, 16)
    with pytest.raises(rra.RraError):
        rra.rra_swiglu(t, t, t, 40, 4)
    ws = torch.zeros(4)
    with pytest.raises(rra.RraError) as e:
        rra.rra_argmax(t, t, 2, 100000, ws)   # workspace too small
    assert e.value.status == rra.RRA_ENOTINIT


def test_model_descriptor_validation():
    t = torch.zeros(16)
    w = _fake_weight("q4", 64, 128)
    layer = dict(wqkv=w, wo=w, wgu=w, wd=w, attn_gamma=t, ffn_gamma=t, k_cache=t, v_cache=t)
    with pytest.raises(rra.RraError, match="shape"):
        rra.Model(n_layers=1, hidden=128, n_heads=2, n_kv_heads=1, head_dim=64, intermediate=256,
                  vocab=64, rms_eps=1e-6, rope_theta=1e4, max_len=16, m_max=1, layers=[layer],
                  out_gamma=t, lm_head=w)
    with pytest.raises(rra.RraError, match="head_dim"):
        rra.Model(n_layers=1, hidden=128, n_heads=2, n_kv_heads=1, head_dim=96, intermediate=256,
                  vocab=64, rms_eps=1e-6, rope_theta=1e4, max_len=16, m_max=1, layers=[layer],
                  out_gamma=t, lm_head=w)
    with pytest.raises(rra.RraError, match="m_max"):
        rra.Model(n_layers=1, hidden=128, n_heads=2, n_kv_heads=1, head_dim=64, intermediate=256,
                  vocab=64, rms_eps=1e-6, rope_theta=1e4, max_len=16, m_max=40, layers=[layer],
                  out_gamma=t, lm_head=w)


def test_decode_step_rejects_null_model():
    st = rra.lib.rra_decode_step(None, None, None, None, None, None, 1, 0, None)
    assert st == rra.RRA_ENOTINIT


def test_attention_events_need_a_model():
    # rra_model_set_attention_events on no model: RRA_ENOTINIT, no GPU call
    assert rra.lib.rra_model_set_attention_events(None, None, 0) == rra.RRA_ENOTINIT
    assert b"null model" in rra.lib.rra_last_error()


def test_phase_events_need_a_model():
    assert rra.lib.rra_model_set_phase_events(None, None, 0) == rra.RRA_ENOTINIT
    assert b"null model" in rra.lib.rra_last_error()


@pytest.mark.parametrize("m,nkv,max_len,splits", [
    (32, 8, 4160, 5),    # 8B-shaped, M=32: 1280 workgroups, capped at 5 splits per sequence
    (32, 8, 8192, 8),    # 8192-row cache: 1024-row splits (the row cap) give 8
    (16, 8, 4160, 8),    # 1040 workgroups at 8 splits: the cap is max(5, 1024 / 128) = 8
    (1, 2, 768, 12),     # small grids: at least 256 workgroups, 64-row splits
    (32, 2, 1152, 4),    # 1.5B-shaped, M=32
])
def test_flash_decode_split_choice(m, nkv, max_len, splits):
    c = rra.rra_flash_decode_chunk(m, nkv, max_len, 0)
    assert c % 32 == 0 and 64 <= c <= 1024
    assert -(-max_len // c) == splits
    assert rra.rra_flash_decode_chunk(m, nkv, max_len, 96) == 96  # an explicit size is kept


def test_decode_workspace_bytes_is_the_model_workspace_size():
    # the decode-step contract's name for rra_model_workspace_bytes
    assert rra.lib.rra_decode_workspace_bytes(None) == 0
    assert rra.lib.rra_model_workspace_bytes(None) == 0


@pytest.mark.parametrize("m,nq,nkv,max_len", [(32, 32, 8, 4160), (32, 12, 2, 1152), (1, 14, 2, 768),
                                              (1, 12, 2, 1152), (32, 32, 8, 8192), (7, 8, 8, 33)])
def test_flash_decode_candidates_are_valid(m, nq, nkv, max_len):
    # Every (rows per split, head split) the tuner may try: rows a multiple of
    # 32 in 32..1024 covering max_len in at most 256 splits, distinct, head
    # splits dividing the group, grids within 8192 workgroups (head splits only
    # below 1024), and the list is a pure function of the shape.
    c = rra.rra_flash_decode_candidates(m, nq, nkv, max_len)
    assert c and c == rra.rra_flash_decode_candidates(m, nq, nkv, max_len)
    assert len(set(c)) == len(c)
    group = nq // nkv
    for chunk, hs in c:
        assert chunk % 32 == 0 and 32 <= chunk <= 1024
        nc = -(-max_len // chunk)
        assert nc <= 256 and group % hs == 0
        base = nc * nkv * m
        assert base <= 8192 and (hs == 1 or base * hs <= 4096 and base < 1024)
    assert any(hs == 1 for _, hs in c)
    assert rra.rra_flash_decode_candidates(m, nq + 1, nkv, max_len) == [] or (nq + 1) % nkv == 0
