"""CPU oracle for the batched single-token decode step.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the HIP path (``quantized_gemv_flash_amd``) and never imports it.

Everything is computed in fp64 from the plain definition of each step.  The
heavy loops (dequantising GEMV, attention) are plain C in ``oracle.c``; the
elementwise steps and the layer composition are numpy fp64 here.

Sources (docs.rs source pages):
  [reduces]          realizar 0.8.5, src/cuda/executor/layers/reduces.rs
  [batched_forward]  realizar 0.8.5, src/cuda/executor/layers/batched_forward.rs
  [head_dim]         realizar 0.8.5, src/cuda/executor/head_dim.rs
  [graph]            aprender-serve 0.70.2, src/gguf/cuda/forward_qwen35_cuda_graph.rs

Readings where the pages name a step without defining it (each is listed, with
its reason, in the design notes):
  * layer body: Llama pre-norm block -- x += Wo attn(rope(Wqkv rmsnorm(x)));
    x += Wd (silu(Wg u) * Wu u) with u = rmsnorm(x);
  * RMSNorm: x / sqrt(mean(x^2) + eps) * gamma;
  * RoPE: pairs (i, i + hd/2), theta_i = theta^(-2i/hd), angle pos*theta_i in
    fp64;
  * attention scale 1/sqrt(hd); query head h reads KV head h // (nq/nkv);
  * the current token attends to itself: seq_len = pos + 1;
  * greedy token: the lowest index among the maximal logits.

parity unpinned: the whole-model greedy run beyond the invariants listed in
the tests (the pages print no worked example for any model).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "oracle.c")
_LIB = os.path.join(_DIR, "liboracle.so")

F32, Q8, Q4, FP8, Q6K = 0, 1, 2, 3, 4
_FMT = {"f32": F32, "q8": Q8, "q4": Q4, "fp8": FP8, "q6k": Q6K}


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc, OpenMP, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
                        "-fno-fast-math", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"],
                       check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P, I64, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double
        L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f64.restype = D
        L.orc_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_to_f64.restype = D
        L.orc_dequant_row.argtypes = [ctypes.c_int, P, P, I64, I64, P]
        L.orc_dequant_row.restype = None
        L.orc_gemv.argtypes = [ctypes.c_int, P, P, I64, I64, P, I64, P, I64, P]
        L.orc_gemv.restype = None
        L.orc_attention.argtypes = [P, P, P, I64, I64, I64, I64, I64, P]
        L.orc_attention.restype = None
        L.orc_attention_splitk.argtypes = [P, P, P, I64, I64, I64, I64, I64, I64, P]
        L.orc_attention_splitk.restype = None
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _np(t):
    """torch tensor or array -> contiguous numpy array (host copy if needed)."""
    if t is None:
        return None
    if hasattr(t, "detach"):
        t = t.detach().cpu()
        if str(t.dtype) == "torch.int16":  # fp16 bit patterns
            return np.ascontiguousarray(t.numpy().view(np.uint16))
        return np.ascontiguousarray(t.numpy())
    a = np.ascontiguousarray(t)
    return a.view(np.uint16) if a.dtype == np.int16 else a


# --------------------------------------------------------------------------
# Steps
# --------------------------------------------------------------------------
def f16_to_f64(bits: int) -> float:
    return lib().orc_f16_to_f64(int(bits) & 0xFFFF)


def e4m3_to_f64(code: int) -> float:
    return lib().orc_e4m3_to_f64(int(code) & 0xFF)


def dequant(fmt: str, data, scale, n: int, k: int, rows: Sequence[int]) -> np.ndarray:
    """Dequantised rows [len(rows)][k] in fp64."""
    d, s = _np(data), _np(scale)
    out = np.empty((len(rows), k), np.float64)
    for i, r in enumerate(rows):
        lib().orc_dequant_row(_FMT[fmt], _ptr(d), _ptr(s), k, int(r), _ptr(out[i]))
    return out


def gemv(fmt: str, data, scale, n: int, k: int, x, rows: Optional[Sequence[int]] = None):
    """y[m][r] = sum_i W[rows[r]][i] x[m][i] in fp64 ([batched_forward]
    forward_batched_to_token_ids: one weight read serves all M inputs)."""
    d, s = _np(data), _np(scale)
    xx = np.ascontiguousarray(np.asarray(_np(x), dtype=np.float64).reshape(-1, k))
    m = xx.shape[0]
    if rows is None:
        r, nr = None, n
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nr = r.shape[0]
    y = np.empty((m, nr), np.float64)
    lib().orc_gemv(_FMT[fmt], _ptr(d), _ptr(s), n, k, _ptr(xx), m, _ptr(r), nr, _ptr(y))
    return y


def rmsnorm(x: np.ndarray, gamma, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gamma over the last axis ([batched_forward]
    batched_output_norm_lm_head_argmax names the norm and its epsilon)."""
    x = np.asarray(x, np.float64)
    g = np.asarray(_np(gamma), np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope(z: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotate every head of z [..., heads, hd] by position `pos` ([graph] module
    doc: the position drives RoPE).  Pairs (i, i + hd/2); angle pos*theta_i,
    theta_i = theta^(-2i/hd), all in fp64."""
    z = np.asarray(z, np.float64)
    hd = z.shape[-1]
    half = hd // 2
    i = np.arange(half, dtype=np.float64)
    ang = float(pos) * theta ** (-2.0 * i / hd)
    c, s = np.cos(ang), np.sin(ang)
    a, b = z[..., :half], z[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def attention(q, kc, vc, length: int) -> np.ndarray:
    """One sequence: q [nq][hd], kc/vc [nkv][ld][hd] -> out [nq][hd] over cache
    rows [0, length) ([head_dim] flash_decoding_attention_into)."""
    q = np.ascontiguousarray(np.asarray(q, np.float64))
    kc = np.ascontiguousarray(np.asarray(kc, np.float64))
    vc = np.ascontiguousarray(np.asarray(vc, np.float64))
    nq, hd = q.shape
    nkv, ld, _ = kc.shape
    out = np.zeros((nq, hd), np.float64)
    lib().orc_attention(_ptr(q), _ptr(kc), _ptr(vc), nq, nkv, hd, ld, int(length), _ptr(out))
    return out


def attention_splitk(q, kc, vc, length: int, chunk: int) -> np.ndarray:
    """The split-K form of `attention` with chunk size `chunk`."""
    q = np.ascontiguousarray(np.asarray(q, np.float64))
    kc = np.ascontiguousarray(np.asarray(kc, np.float64))
    vc = np.ascontiguousarray(np.asarray(vc, np.float64))
    nq, hd = q.shape
    nkv, ld, _ = kc.shape
    out = np.zeros((nq, hd), np.float64)
    lib().orc_attention_splitk(_ptr(q), _ptr(kc), _ptr(vc), nq, nkv, hd, ld, int(length),
                               int(chunk), _ptr(out))
    return out


def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z) = z / (1 + e^-z)."""
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """silu(gate) * up ([graph] module doc names the fused SwiGLU)."""
    return silu(gate) * np.asarray(up, np.float64)


def argmax(logits: np.ndarray):
    """(token, top-2 gap) per row: the lowest index among the maximal values
    ([reduces] gpu_argmax returns the token with the maximum logit).  A NaN
    logit is an error."""
    l = np.asarray(logits, np.float64)
    if np.isnan(l).any():
        raise ValueError("NaN logit")
    l2 = l.reshape(-1, l.shape[-1])
    tok = np.argmax(l2, axis=-1)  # first occurrence of the maximum
    top2 = np.sort(l2, axis=-1)[:, -2:] if l2.shape[-1] > 1 else np.concatenate([l2, l2], -1)
    gap = top2[:, 1] - top2[:, 0]
    return tok.reshape(l.shape[:-1]), gap.reshape(l.shape[:-1])


# --------------------------------------------------------------------------
# The decode step ([batched_forward] forward_batched_to_token_ids: M
# embeddings and M positions in, M greedy token ids out)
# --------------------------------------------------------------------------
class DecoderOracle:
    """fp64 decoder over a subset of sequences, with its own fp64 KV cache.

    `weights` is a synth.DecoderWeights (tensors on any device; copied to host
    once).  Sequences are independent, so the oracle may hold only the ones a
    test samples; index i here is the i-th sequence handed to it.
    """

    def __init__(self, shape, weights, n_seq: int, max_len: int):
        self.s = shape
        self.fmt = shape.fmt
        self.lm_fmt = getattr(shape, "lm_format", shape.fmt)
        self.n_seq = n_seq
        self.max_len = max_len

        def host(wt):
            d, sc = wt
            return _np(d), _np(sc)

        self.layers = []
        for lw in weights.layers:
            self.layers.append(dict(
                wqkv=host(lw.wqkv), wo=host(lw.wo), wgu=host(lw.wgu), wd=host(lw.wd),
                attn_gamma=_np(lw.attn_gamma).astype(np.float64),
                ffn_gamma=_np(lw.ffn_gamma).astype(np.float64)))
        self.out_gamma = _np(weights.out_gamma).astype(np.float64)
        self.lm_head = host(weights.lm_head)
        S = shape
        self.kc = [np.zeros((n_seq, S.n_kv_heads, max_len, S.head_dim)) for _ in self.layers]
        self.vc = [np.zeros((n_seq, S.n_kv_heads, max_len, S.head_dim)) for _ in self.layers]

    def set_context(self, layer: int, seq: int, k_rows, v_rows):
        """Cache rows [0, L) of sequence `seq` in `layer` (k/v [nkv][L][hd])."""
        k, v = _np(k_rows).astype(np.float64), _np(v_rows).astype(np.float64)
        L = k.shape[1]
        self.kc[layer][seq, :, :L] = k
        self.vc[layer][seq, :, :L] = v

    def _mv(self, w, n, k, x):
        return gemv(self.fmt, w[0], w[1], n, k, x)

    def layer(self, l: int, x: np.ndarray, pos: Sequence[int],
              slots: Optional[Sequence[int]] = None) -> np.ndarray:
        """Row i sits at position pos[i] of the oracle's sequence slots[i]
        (default i).  Rows are taken in order, each writing its K/V row and then
        attending to rows [0, pos[i]] of its sequence, so rows that share a
        sequence at consecutive positions attend causally (a prefill)."""
        S, Lw = self.s, self.layers[l]
        M, H = x.shape
        nq, nkv, hd, I = S.n_heads, S.n_kv_heads, S.head_dim, S.intermediate
        u = rmsnorm(x, Lw["attn_gamma"], S.rms_eps)
        qkv = self._mv(Lw["wqkv"], S.qkv_rows, H, u)
        attn = np.empty((M, nq * hd))
        for i in range(M):
            q = qkv[i, :nq * hd].reshape(nq, hd)
            k = qkv[i, nq * hd:(nq + nkv) * hd].reshape(nkv, hd)
            v = qkv[i, (nq + nkv) * hd:].reshape(nkv, hd)
            p = int(pos[i])
            c = i if slots is None else int(slots[i])
            q, k = rope(q, p, S.rope_theta), rope(k, p, S.rope_theta)
            self.kc[l][c, :, p] = k
            self.vc[l][c, :, p] = v
            attn[i] = attention(q, self.kc[l][c], self.vc[l][c], p + 1).reshape(-1)
        x = x + self._mv(Lw["wo"], H, nq * hd, attn)
        u = rmsnorm(x, Lw["ffn_gamma"], S.rms_eps)
        gu = self._mv(Lw["wgu"], 2 * I, H, u)
        a = swiglu(gu[:, :I], gu[:, I:])
        return x + self._mv(Lw["wd"], H, I, a)

    def step(self, x, pos: Sequence[int], slots: Optional[Sequence[int]] = None,
             head: str = "all"):
        """One decode step for the oracle's sequences.  x [n][H] (embedding rows),
        pos [n], slots [n] (sequence of each row, default row i -> sequence i).
        Returns dict(hidden [n][H], logits [r][V], tok [r], gap [r]) where the
        r rows taken through the output norm and LM head are every row
        (head="all") or only the last one (head="last"; the same values for that
        row, the others are simply not computed)."""
        x = np.asarray(_np(x), np.float64).reshape(len(pos), self.s.hidden)
        for l in range(len(self.layers)):
            x = self.layer(l, x, pos, slots)
        if head not in ("all", "last"):
            raise ValueError(f"head={head!r}")
        xh = x if head == "all" else x[-1:]
        u = rmsnorm(xh, self.out_gamma, self.s.rms_eps)
        logits = gemv(self.lm_fmt, self.lm_head[0], self.lm_head[1], self.s.vocab, self.s.hidden, u)
        tok, gap = argmax(logits)
        return dict(hidden=x, logits=logits, tok=tok, gap=gap)

    def prefill(self, seq: int, x, start: int, head: str = "all"):
        """Prompt ingestion ([head_dim] tensor_core_attention: causal
        attention over the prompt): the T embedding rows x [T][H] at positions
        start .. start+T-1 of sequence `seq`, every layer over all T rows, row t
        attending to rows [0, start + t] of the sequence.  Returns step()'s dict
        for the T rows (with head="last", logits of the last row only); the
        last row's tok is the next greedy token."""
        T = np.asarray(_np(x)).reshape(-1, self.s.hidden).shape[0]
        return self.step(x, [start + t for t in range(T)], [seq] * T, head=head)
