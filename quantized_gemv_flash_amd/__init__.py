"""Python binding of librra (the MI355X batched decode step).

Argument marshalling only: every function forwards to the C ABI declared in
``include/rra.h`` under the same name, passing torch tensors' device
addresses and the current HIP stream.  All computation runs in librra's HIP
kernels; there is no fallback.  Importing this package fails if librra.so has
not been built (``python quantized_gemv_flash_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import POINTER, c_double, c_float, c_int32, c_int64, c_size_t, c_uint32, c_uint64, c_void_p
from typing import Optional, Sequence

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librra.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "rra.h")

RRA_OK, RRA_EINVAL, RRA_ENOTINIT, RRA_EHIP, RRA_ECAPTURE = 0, 1, 2, 3, 4
RRA_F32, RRA_Q8, RRA_Q4, RRA_FP8, RRA_Q6K = 0, 1, 2, 3, 4
RRA_PLANAR, RRA_TILED = 0, 1
RRA_GRAPH, RRA_STEP_GATHER, RRA_STEP_ADVANCE = 1, 2, 4
RRA_POS_NONE = 0xFFFFFFFF  # empty batch slot; -1 in an int32 position tensor
POS_NONE_I32 = -1
FMT = {"f32": RRA_F32, "q8": RRA_Q8, "q4": RRA_Q4, "fp8": RRA_FP8, "q6k": RRA_Q6K}


class RraError(RuntimeError):
    def __init__(self, call: str, status: int, message: str):
        super().__init__(f"{call}: status {status}: {message}")
        self.status = status


class rra_weight(ctypes.Structure):
    _fields_ = [("fmt", c_int32), ("layout", c_int32), ("n", c_int64), ("k", c_int64),
                ("data", c_void_p), ("scale", c_void_p)]


class rra_layer_desc(ctypes.Structure):
    _fields_ = [("wqkv", rra_weight), ("wo", rra_weight), ("wgu", rra_weight), ("wd", rra_weight),
                ("attn_gamma", c_void_p), ("ffn_gamma", c_void_p),
                ("k_cache", c_void_p), ("v_cache", c_void_p)]


class rra_model_desc(ctypes.Structure):
    _fields_ = [("n_layers", c_int32), ("hidden", c_int32), ("n_heads", c_int32),
                ("n_kv_heads", c_int32), ("head_dim", c_int32), ("intermediate", c_int32),
                ("vocab", c_int32), ("rms_eps", c_float), ("rope_theta", c_double),
                ("max_len", c_int32), ("m_max", c_int32), ("layers", POINTER(rra_layer_desc)),
                ("out_gamma", c_void_p), ("lm_head", rra_weight), ("embed", c_void_p),
                ("attn_chunk", c_int32), ("prefill_rows", c_int32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python quantized_gemv_flash_amd/build.py`")
    L = ctypes.CDLL(LIB_PATH)
    P, S, I, U = c_void_p, c_size_t, c_int32, c_uint32
    W = POINTER(rra_weight)
    sig = {
        "rra_last_error": ([], ctypes.c_char_p),
        "rra_status_name": ([I], ctypes.c_char_p),
        "rra_version": ([], I),
        "rra_tiled_bytes": ([I, c_int64, c_int64], S),
        "rra_repack_weight": ([W, P, S, W, P], I),
        "rra_unpack_weight": ([W, P, P, P], I),
        "rra_batched_gemv_workspace_bytes": ([W, I], S),
        "rra_batched_gemv": ([W, P, P, I, P, S, P], I),
        "rra_batched_gemv_noalloc": ([W, P, P, I, P], I),
        "rra_batched_gemv_valu": ([W, P, P, I, P, S, P], I),
        "rra_kv_scatter": ([P, P, P, P, P, I, I, I, I, P], I),
        "rra_flash_decode_workspace_bytes": ([I, I, I, I, I, I], S),
        "rra_flash_decode_chunk": ([I, I, I, I], I),
        "rra_flash_decode": ([P, P, P, P, P, I, I, I, I, I, I, P, S, P], I),
        "rra_flash_decode_candidates": ([I, I, I, I, P, P, I], I),
        "rra_flash_decode_ex": ([P, P, P, P, P, I, I, I, I, I, I, I, P, S, P], I),
        "rra_flash_decode_tune": ([P, P, P, P, P, I, I, I, I, I, P, S, P, POINTER(c_int32),
                                   POINTER(c_int32)], I),
        "rra_model_attention_plan": ([P, I, POINTER(c_int32), POINTER(c_int32)], I),
        "rra_model_set_attention_plan": ([P, I, I, I], I),
        "rra_model_tune_attention": ([P, P, I, P, P], I),
        "rra_rmsnorm": ([P, P, P, I, I, c_float, P], I),
        "rra_rope_table": ([P, I, I, c_double, P], I),
        "rra_rope": ([P, P, P, I, I, I, I, P], I),
        "rra_swiglu": ([P, P, P, I, I, P], I),
        "rra_argmax_workspace_bytes": ([I, I], S),
        "rra_argmax": ([P, P, I, I, P, S, P], I),
        "rra_hbm_read": ([P, S, P, I, P], I),
        "rra_model_workspace_bytes": ([POINTER(rra_model_desc)], S),
        "rra_decode_workspace_bytes": ([POINTER(rra_model_desc)], S),
        "rra_model_create": ([POINTER(rra_model_desc), P, S, P, POINTER(c_void_p)], I),
        "rra_decode_step": ([P, P, P, P, P, P, I, I, P], I),
        "rra_decode_step_async": ([P, P, P, P, P, P, P, I, I, P], I),
        "rra_prefill": ([P, P, I, I, U, P, P, P], I),
        "rra_model_check": ([P, P], I),
        "rra_graph_stats": ([P, POINTER(c_uint64), POINTER(c_uint64), POINTER(c_uint32)], I),
        "rra_model_set_attention_events": ([P, P, I], I),
        "rra_model_set_phase_events": ([P, P, I], I),
        "rra_model_destroy": ([P], None),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    return L


lib = _load()


def header_functions() -> list:
    """Names of the functions declared in include/rra.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(rra_[a-z0-9_]+)\s*\(", text)))


def _check(call: str, st: int):
    if st != RRA_OK:
        raise RraError(call, st, lib.rra_last_error().decode())


def _p(t: Optional[torch.Tensor]):
    return None if t is None else c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        if not torch.cuda.is_available():
            return None
        stream = torch.cuda.current_stream()
    return c_void_p(stream.cuda_stream) if hasattr(stream, "cuda_stream") else c_void_p(stream)


# ---------------------------------------------------------------- weights
class Weight:
    """An rra_weight plus the tensors it points into (kept alive)."""

    def __init__(self, fmt: str, n: int, k: int, data: torch.Tensor,
                 scale: Optional[torch.Tensor] = None, layout: int = RRA_PLANAR):
        self.fmt, self.n, self.k = fmt, n, k
        self.data, self.scale = data, scale
        self.c = rra_weight(FMT[fmt], layout, n, k, data.data_ptr(),
                            scale.data_ptr() if scale is not None else None)

    @property
    def layout(self) -> int:
        return self.c.layout

    @property
    def nbytes(self) -> int:
        return self.data.numel() * self.data.element_size() + (
            0 if self.scale is None else self.scale.numel() * self.scale.element_size())


def rra_tiled_bytes(fmt: str, n: int, k: int) -> int:
    return lib.rra_tiled_bytes(FMT[fmt], n, k)


def rra_repack_weight(planar: Weight, stream=None) -> Weight:
    """Planar quantised weight -> tiled copy in a new device tensor."""
    nbytes = rra_tiled_bytes(planar.fmt, planar.n, planar.k)
    if nbytes == 0:
        raise RraError("rra_repack_weight", RRA_EINVAL, "invalid shape or format")
    tiled = torch.empty(nbytes, dtype=torch.uint8, device=planar.data.device)
    out = rra_weight()
    _check("rra_repack_weight", lib.rra_repack_weight(ctypes.byref(planar.c), _p(tiled), nbytes,
                                                      ctypes.byref(out), _stream(stream)))
    return Weight(planar.fmt, planar.n, planar.k, tiled, None, RRA_TILED)


def rra_unpack_weight(tiled: Weight, data: torch.Tensor, scale: torch.Tensor, stream=None):
    _check("rra_unpack_weight", lib.rra_unpack_weight(ctypes.byref(tiled.c), _p(data), _p(scale),
                                                      _stream(stream)))


def device_weight(data: torch.Tensor, scale: Optional[torch.Tensor], fmt: str, stream=None) -> Weight:
    """A GEMV-ready weight from planar tensors already on the device: F32 as is,
    Q8/Q4/FP8/Q6K repacked into the tiled layout."""
    n = data.shape[0]
    k = data.shape[1] * 2 if fmt == "q4" else (data.shape[1] // 192 * 256 if fmt == "q6k"
                                                else data.shape[1])
    w = Weight(fmt, n, k, data, scale)
    return w if fmt == "f32" else rra_repack_weight(w, stream)


# ---------------------------------------------------------------- GEMV
def rra_batched_gemv_workspace_bytes(w: Weight, m: int) -> int:
    return lib.rra_batched_gemv_workspace_bytes(ctypes.byref(w.c), m)


def rra_batched_gemv(w: Weight, x: torch.Tensor, y: torch.Tensor, m: int,
                     ws: Optional[torch.Tensor] = None, stream=None):
    nb = 0 if ws is None else ws.numel() * ws.element_size()
    _check("rra_batched_gemv", lib.rra_batched_gemv(ctypes.byref(w.c), _p(x), _p(y), m, _p(ws), nb,
                                                    _stream(stream)))


def rra_batched_gemv_valu(w: Weight, x: torch.Tensor, y: torch.Tensor, m: int,
                          ws: Optional[torch.Tensor] = None, stream=None):
    nb = 0 if ws is None else ws.numel() * ws.element_size()
    _check("rra_batched_gemv_valu", lib.rra_batched_gemv_valu(ctypes.byref(w.c), _p(x), _p(y), m,
                                                              _p(ws), nb, _stream(stream)))


def rra_batched_gemv_noalloc(w: Weight, x: torch.Tensor, y: torch.Tensor, m: int, stream=None):
    _check("rra_batched_gemv_noalloc", lib.rra_batched_gemv_noalloc(ctypes.byref(w.c), _p(x), _p(y),
                                                                    m, _stream(stream)))


# ---------------------------------------------------------------- attention
def rra_kv_scatter(k_rows, v_rows, k_cache, v_cache, pos, m, nkv, hd, max_len, stream=None):
    _check("rra_kv_scatter", lib.rra_kv_scatter(_p(k_rows), _p(v_rows), _p(k_cache), _p(v_cache),
                                                _p(pos), m, nkv, hd, max_len, _stream(stream)))


def rra_flash_decode_workspace_bytes(m, nq, nkv, hd, max_len, chunk=0) -> int:
    return lib.rra_flash_decode_workspace_bytes(m, nq, nkv, hd, max_len, chunk)


def rra_flash_decode_chunk(m, nkv, max_len, chunk=0) -> int:
    return lib.rra_flash_decode_chunk(m, nkv, max_len, chunk)


def rra_flash_decode(q, k_cache, v_cache, seq_len, out, m, nq, nkv, hd, max_len, chunk, ws,
                     stream=None):
    _check("rra_flash_decode", lib.rra_flash_decode(
        _p(q), _p(k_cache), _p(v_cache), _p(seq_len), _p(out), m, nq, nkv, hd, max_len, chunk,
        _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def rra_flash_decode_candidates(m, nq, nkv, max_len):
    """[(chunk, head_split), ...] the tuner tries for this shape."""
    n = lib.rra_flash_decode_candidates(m, nq, nkv, max_len, None, None, 0)
    ch, hs = (c_int32 * max(n, 1))(), (c_int32 * max(n, 1))()
    lib.rra_flash_decode_candidates(m, nq, nkv, max_len, ch, hs, n)
    return [(ch[i], hs[i]) for i in range(n)]


def rra_flash_decode_ex(q, k_cache, v_cache, seq_len, out, m, nq, nkv, hd, max_len, chunk,
                        head_split, ws, stream=None):
    _check("rra_flash_decode_ex", lib.rra_flash_decode_ex(
        _p(q), _p(k_cache), _p(v_cache), _p(seq_len), _p(out), m, nq, nkv, hd, max_len, chunk,
        head_split, _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def rra_flash_decode_tune(q, k_cache, v_cache, seq_len, out, m, nq, nkv, hd, max_len, ws,
                          stream=None):
    """Times every candidate on these inputs; returns the cached (chunk, head_split)."""
    c, h = c_int32(), c_int32()
    _check("rra_flash_decode_tune", lib.rra_flash_decode_tune(
        _p(q), _p(k_cache), _p(v_cache), _p(seq_len), _p(out), m, nq, nkv, hd, max_len, _p(ws),
        ws.numel() * ws.element_size(), _stream(stream), ctypes.byref(c), ctypes.byref(h)))
    return c.value, h.value


# ---------------------------------------------------------------- step kernels
def rra_rmsnorm(x, gamma, out, m, h, eps, stream=None):
    _check("rra_rmsnorm", lib.rra_rmsnorm(_p(x), _p(gamma), _p(out), m, h, eps, _stream(stream)))


def rra_rope_table(table, max_len, hd, theta, stream=None):
    _check("rra_rope_table", lib.rra_rope_table(_p(table), max_len, hd, theta, _stream(stream)))


def rra_rope(z, pos, table, m, n_heads, hd, max_len, stream=None):
    _check("rra_rope", lib.rra_rope(_p(z), _p(pos), _p(table), m, n_heads, hd, max_len,
                                    _stream(stream)))


def rra_swiglu(gate, up, out, m, n, stream=None):
    _check("rra_swiglu", lib.rra_swiglu(_p(gate), _p(up), _p(out), m, n, _stream(stream)))


def rra_argmax_workspace_bytes(m, v) -> int:
    return lib.rra_argmax_workspace_bytes(m, v)


def rra_argmax(logits, tok, m, v, ws, stream=None):
    _check("rra_argmax", lib.rra_argmax(_p(logits), _p(tok), m, v, _p(ws),
                                        ws.numel() * ws.element_size(), _stream(stream)))


def rra_hbm_read(buf, sums, blocks=None, stream=None):
    """Streaming read of the whole of `buf` (a device tensor); sums: device
    fp32 tensor of at least `blocks` elements (default: all of it)."""
    blocks = sums.numel() if blocks is None else blocks
    if sums.numel() < blocks:
        raise RraError(f"rra_hbm_read: sums holds {sums.numel()} floats, needs {blocks}")
    _check("rra_hbm_read", lib.rra_hbm_read(_p(buf), buf.numel() * buf.element_size(), _p(sums),
                                            blocks, _stream(stream)))


# ---------------------------------------------------------------- decode step
class Model:
    """Owns the descriptor structs, the workspace tensor and the rra_model handle.

    `layers` is a sequence of dicts with keys wqkv, wo, wgu, wd (Weight),
    attn_gamma, ffn_gamma, k_cache, v_cache (tensors)."""

    def __init__(self, *, n_layers, hidden, n_heads, n_kv_heads, head_dim, intermediate, vocab,
                 rms_eps, rope_theta, max_len, m_max, layers: Sequence[dict], out_gamma,
                 lm_head: Weight, embed: Optional[torch.Tensor] = None, attn_chunk: int = 0,
                 prefill_rows: int = 0, stream=None):
        self._keep = [layers, out_gamma, lm_head, embed]
        arr = (rra_layer_desc * n_layers)()
        for i, l in enumerate(layers):
            arr[i] = rra_layer_desc(l["wqkv"].c, l["wo"].c, l["wgu"].c, l["wd"].c,
                                    l["attn_gamma"].data_ptr(), l["ffn_gamma"].data_ptr(),
                                    l["k_cache"].data_ptr(), l["v_cache"].data_ptr())
        self._layers = arr
        self.desc = rra_model_desc(
            n_layers, hidden, n_heads, n_kv_heads, head_dim, intermediate, vocab, rms_eps,
            rope_theta, max_len, m_max, ctypes.cast(arr, POINTER(rra_layer_desc)),
            out_gamma.data_ptr(), lm_head.c, embed.data_ptr() if embed is not None else None,
            attn_chunk, prefill_rows)
        nbytes = lib.rra_model_workspace_bytes(ctypes.byref(self.desc))
        if nbytes == 0:
            # re-run creation on a null workspace to surface the validation message
            h = c_void_p()
            _check("rra_model_create", lib.rra_model_create(ctypes.byref(self.desc), None, 0,
                                                            _stream(stream), ctypes.byref(h)))
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=out_gamma.device)
        self.handle = c_void_p()
        _check("rra_model_create", lib.rra_model_create(
            ctypes.byref(self.desc), _p(self.ws), nbytes, _stream(stream), ctypes.byref(self.handle)))
        self.vocab, self.hidden, self.m_max = vocab, hidden, m_max
        self.prefill_rows = prefill_rows or 128

    def rra_decode_step(self, x, pos, tok, m: int, flags: int = 0, logits=None,
                        tok_host: bool = False, stream=None):
        """One decode step; returns the host token ids when tok_host is set."""
        host = (c_uint32 * m)() if tok_host else None
        _check("rra_decode_step", lib.rra_decode_step(
            self.handle, _p(x), _p(pos), _p(tok), host, _p(logits), m, flags, _stream(stream)))
        return list(host) if host is not None else None

    def rra_decode_step_async(self, x, pos, tok, tok_pinned, done, m: int, flags: int = 0,
                              logits=None, stream=None):
        """One decode step whose ids are copied asynchronously into tok_pinned (a
        pinned host int32 tensor of >= m elements) and followed by a record of
        `done` (a torch.cuda.Event already recorded once, so that it exists);
        returns at once.  Read tok_pinned after done.synchronize()/query()."""
        _check("rra_decode_step_async", lib.rra_decode_step_async(
            self.handle, _p(x), _p(pos), _p(tok), c_void_p(tok_pinned.data_ptr()),
            c_void_p(done.cuda_event), _p(logits), m, flags, _stream(stream)))

    def rra_prefill(self, tokens, n_tokens: int, seq: int, start: int, next_tok=None,
                    logits=None, stream=None):
        """Ingests n_tokens prompt tokens (device uint32) into cache slot seq at
        positions start...; the last token's greedy id / logits go to next_tok /
        logits when given."""
        _check("rra_prefill", lib.rra_prefill(self.handle, _p(tokens), n_tokens, seq, start,
                                              _p(next_tok), _p(logits), _stream(stream)))

    def rra_model_attention_plan(self, m: int):
        c, h = c_int32(), c_int32()
        _check("rra_model_attention_plan", lib.rra_model_attention_plan(
            self.handle, m, ctypes.byref(c), ctypes.byref(h)))
        return c.value, h.value

    def rra_model_set_attention_plan(self, m: int, chunk: int, head_split: int):
        _check("rra_model_set_attention_plan",
               lib.rra_model_set_attention_plan(self.handle, m, chunk, head_split))

    def rra_model_tune_attention(self, ms=None, lengths=None, stream=None):
        """Times the flash-decode candidates for each batch size in ms (default:
        1..m_max) at the given per-slot lengths (default: max_len); returns
        {m: (chunk, head_split)}."""
        arr = None if not ms else (c_int32 * len(ms))(*ms)
        lens = None if lengths is None else (c_uint32 * self.m_max)(
            *[int(v) for v in lengths] + [0] * (self.m_max - len(lengths)))
        _check("rra_model_tune_attention", lib.rra_model_tune_attention(
            self.handle, arr, len(ms) if ms else 0, lens, _stream(stream)))
        return {m: self.rra_model_attention_plan(m) for m in (ms or range(1, self.m_max + 1))}

    def rra_model_check(self, stream=None):
        _check("rra_model_check", lib.rra_model_check(self.handle, _stream(stream)))

    def rra_graph_stats(self):
        c, r, k = c_uint64(), c_uint64(), c_uint32()
        _check("rra_graph_stats", lib.rra_graph_stats(self.handle, ctypes.byref(c), ctypes.byref(r),
                                                      ctypes.byref(k)))
        return dict(captures=c.value, replays=r.value, kernels=k.value)

    def rra_model_set_attention_events(self, events=None):
        """events: None (stop) or 2 x n_layers torch.cuda.Event(enable_timing=True),
        each already recorded once (so that it exists); kept alive here."""
        if not events:
            self._attn_events = None
            _check("rra_model_set_attention_events",
                   lib.rra_model_set_attention_events(self.handle, None, 0))
            return
        handles = (c_void_p * len(events))(*[e.cuda_event for e in events])
        self._attn_events = (list(events), handles)
        _check("rra_model_set_attention_events",
               lib.rra_model_set_attention_events(self.handle, handles, len(events)))

    def rra_model_set_phase_events(self, events=None):
        """events: None (stop) or 4 x n_layers + 3 torch.cuda.Event(enable_timing=True),
        each already recorded once (so that it exists); kept alive here."""
        if not events:
            self._phase_events = None
            _check("rra_model_set_phase_events",
                   lib.rra_model_set_phase_events(self.handle, None, 0))
            return
        handles = (c_void_p * len(events))(*[e.cuda_event for e in events])
        self._phase_events = (list(events), handles)
        _check("rra_model_set_phase_events",
               lib.rra_model_set_phase_events(self.handle, handles, len(events)))

    def close(self):
        if getattr(self, "handle", None):
            lib.rra_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
