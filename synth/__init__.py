"""Seeded synthetic inputs for the batched decode step.

This module is shared by the CPU oracle side (tests, cpu baseline) and the HIP
side (tests, bench).  It holds no arithmetic of the decode step itself: only

* the workload shape table (five decoder / attention workloads),
* seeded normal draws (torch generators, one independent stream per tensor),
* the block quantiser that turns N(0, std) draws into Q8 / Q4 test weights
  (the weight *producer*; the consumer-side dequantisation lives in the oracle
  and in the kernels, separately).

Every draw is keyed by (seed, tensor name), so any tensor can be regenerated on
its own, on any device.  A test generates each tensor once and hands the same
bytes to both sides.
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Optional, Sequence

import torch

QBLOCK = 32  # elements per quantisation block, both formats


# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Decoder:
    """Shape of a Llama-style pre-norm decoder and the run made on it."""

    name: str
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    fmt: str  # "f32" | "q8" | "q4" | "fp8" (and "q6k" for an LM head)
    rms_eps: float = 1e-6
    rope_theta: float = 1e4
    weight_std: float = 0.02
    m: int = 1
    steps: int = 16
    max_len: int = 16
    # context before the greedy steps:
    #   "none"      decode starts at position 0
    #   "decode:N"  N teacher-forced decode steps on random token ids
    #   "kv:N"      cache rows [0, N) filled with seeded N(0,1) K and V
    #   "kv:A-B"    per-sequence length drawn uniformly from [A, B]
    context: str = "none"
    lm_fmt: Optional[str] = None  # LM-head format when it differs from `fmt`

    @property
    def qkv_rows(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def lm_format(self) -> str:
        return self.lm_fmt or self.fmt


@dataclasses.dataclass(frozen=True)
class Attention:
    """Standalone split-K flash-decode workload."""

    name: str
    m: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    max_len: int
    len_lo: int
    len_hi: int
    chunks: Sequence[int]


TINY_LLAMA_F32 = Decoder(
    name="tiny-llama-f32", n_layers=2, hidden=256, n_heads=4, n_kv_heads=2,
    head_dim=64, intermediate=688, vocab=1024, fmt="f32", m=1, steps=16,
    max_len=16, context="none")

QWEN25_05B_Q8 = Decoder(
    name="qwen2.5-0.5b-shaped-q8", n_layers=24, hidden=896, n_heads=14,
    n_kv_heads=2, head_dim=64, intermediate=4864, vocab=151936, fmt="q8",
    m=1, steps=256, max_len=768, context="decode:512")

FLASH_DECODE_M32 = Attention(
    name="flash-decode-m32-gqa4-hd128", m=32, n_heads=32, n_kv_heads=8,
    head_dim=128, max_len=8192, len_lo=1, len_hi=8192, chunks=(32, 64, 128, 256))

QWEN25_15B_Q4 = Decoder(
    name="qwen2.5-1.5b-shaped-q4", n_layers=28, hidden=1536, n_heads=12,
    n_kv_heads=2, head_dim=128, intermediate=8960, vocab=151936, fmt="q4",
    m=32, steps=128, max_len=1152, context="kv:1024")

LLAMA3_8B_Q4 = Decoder(
    name="llama3-8b-shaped-q4", n_layers=32, hidden=4096, n_heads=32,
    n_kv_heads=8, head_dim=128, intermediate=14336, vocab=128256, fmt="q4",
    m=32, steps=64, max_len=4160, context="kv:2048-4096")

WORKLOADS = {w.name: w for w in (TINY_LLAMA_F32, QWEN25_05B_Q8, FLASH_DECODE_M32,
                                 QWEN25_15B_Q4, LLAMA3_8B_Q4)}

# Test shapes for the FP8 block format (not workloads of the pages): a small
# all-FP8 decoder, and a Q4 decoder with an FP8 LM head (the pages' split).
SMALL_LLAMA_FP8 = Decoder(
    name="small-llama-fp8", n_layers=2, hidden=256, n_heads=4, n_kv_heads=2,
    head_dim=64, intermediate=704, vocab=1024, fmt="fp8", m=2, steps=8, max_len=16)
SMALL_LLAMA_Q4_FP8_HEAD = Decoder(
    name="small-llama-q4-fp8-head", n_layers=2, hidden=256, n_heads=4, n_kv_heads=2,
    head_dim=64, intermediate=704, vocab=1024, fmt="q4", lm_fmt="fp8", m=2, steps=8,
    max_len=16)


# --------------------------------------------------------------------------
# Seeded draws
# --------------------------------------------------------------------------
def stream_seed(seed: int, name: str) -> int:
    """A 63-bit generator seed for tensor `name` under run seed `seed`."""
    h = zlib.crc32(name.encode()) & 0xFFFFFFFF
    return ((seed & 0x7FFFFFFF) << 32 | h) & 0x7FFFFFFFFFFFFFFF


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(stream_seed(seed, name))
    return g


def normal(shape, std: float, seed: int, name: str, device="cpu") -> torch.Tensor:
    """fp32 draws from N(0, std^2), one independent stream per (seed, name)."""
    g = _gen(seed, name, device)
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def uniform_int(shape, lo: int, hi: int, seed: int, name: str, device="cpu") -> torch.Tensor:
    """int64 draws uniform on the closed range [lo, hi]."""
    g = _gen(seed, name, device)
    return torch.randint(lo, hi + 1, tuple(shape), generator=g, device=device,
                         dtype=torch.int64)


# --------------------------------------------------------------------------
# Block quantiser (weight producer)
# --------------------------------------------------------------------------
def quantize_q8(w: torch.Tensor):
    """fp32 [N][K] -> (q int8 [N][K], scale fp16-bits int16 [N][K/32]).

    Per block of 32 consecutive K elements of one row: scale = maxabs/127,
    stored as fp16 (round to nearest even); q = clamp(rint(w / scale), -127, 127)
    with the division by the stored (fp16-rounded) scale.  An all-zero block gets
    scale 0 and q 0.
    """
    n, k = w.shape
    assert k % QBLOCK == 0, "Q8 needs K to be a multiple of 32"
    b = w.reshape(n, k // QBLOCK, QBLOCK)
    s16 = (b.abs().amax(dim=2) / 127.0).to(torch.float16)
    s = s16.to(torch.float32).unsqueeze(2)
    safe = torch.where(s > 0, s, torch.ones_like(s))
    q = torch.where(s > 0, torch.round(b / safe), torch.zeros_like(b))
    q = q.clamp_(-127, 127).to(torch.int8).reshape(n, k)
    return q.contiguous(), s16.view(torch.int16).contiguous()


E4M3_MAX = 448.0


def quantize_fp8(w: torch.Tensor):
    """fp32 [N][K] -> (E4M3 codes uint8 [N][K], scale fp16-bits int16 [N][K/32]).

    Per block of 32: scale = maxabs/448 (the largest finite E4M3 magnitude),
    stored as fp16 (round to nearest even); q = E4M3(w / scale), round to
    nearest even, clamped to +-448 first (the fp16 rounding of the scale can
    push a ratio just past 448).  All-zero block: scale 0, every code 0.
    """
    n, k = w.shape
    assert k % QBLOCK == 0, "FP8 blocks need K to be a multiple of 32"
    b = w.reshape(n, k // QBLOCK, QBLOCK)
    s16 = (b.abs().amax(dim=2) / E4M3_MAX).to(torch.float16)
    s = s16.to(torch.float32).unsqueeze(2)
    safe = torch.where(s > 0, s, torch.ones_like(s))
    r = torch.where(s > 0, b / safe, torch.zeros_like(b)).clamp_(-E4M3_MAX, E4M3_MAX)
    q = r.to(torch.float8_e4m3fn).view(torch.uint8).reshape(n, k)
    return q.contiguous(), s16.view(torch.int16).contiguous()


def quantize_q4(w: torch.Tensor):
    """fp32 [N][K] -> (packed uint8 [N][K/2], scale fp16-bits int16 [N][K/32]).

    Per block of 32: scale = maxabs/7 (fp16, round to nearest even);
    q = clamp(rint(w / scale) + 8, 0, 15).  Byte j of a row holds element 2j in
    its low nibble and element 2j+1 in its high nibble.  All-zero block: scale
    0, every q = 8.
    """
    n, k = w.shape
    assert k % QBLOCK == 0, "Q4 needs K to be a multiple of 32"
    b = w.reshape(n, k // QBLOCK, QBLOCK)
    s16 = (b.abs().amax(dim=2) / 7.0).to(torch.float16)
    s = s16.to(torch.float32).unsqueeze(2)
    safe = torch.where(s > 0, s, torch.ones_like(s))
    q = torch.where(s > 0, torch.round(b / safe), torch.zeros_like(b)) + 8
    q = q.clamp_(0, 15).to(torch.uint8).reshape(n, k)
    packed = q[:, 0::2] | (q[:, 1::2] << 4)
    return packed.contiguous(), s16.view(torch.int16).contiguous()


Q6K_SUPER = 256


def quantize_q6k(w: torch.Tensor):
    """fp32 [N][K] -> (codes uint8 [N][K/256*192], scale records uint8
    [N][K/256*18]) in the 6-bit K-quant layout (see the oracle's dequant).

    Per sub-block of 16: s = maxabs/31.5; per super-block of 256: d = max s /
    126.5, stored as fp16 (round to nearest even; the margin below 127 absorbs
    that rounding); sub-scale sc = min(ceil(s / d), 127) with the stored d, so
    the step d*sc >= s and |w| / (d sc) <= 31.5; q = clamp(rint(w / (d sc)) + 32,
    0, 63).  A sub-block whose sc is 0 gets every q = 32; an all-zero
    super-block gets d = 0.
    """
    n, k = w.shape
    assert k % Q6K_SUPER == 0, "Q6K needs K to be a multiple of 256"
    nsb = k // Q6K_SUPER
    b = w.reshape(n, nsb, 16, 16)
    s = b.abs().amax(dim=3) / 31.5                       # [n][nsb][16]
    d16 = (s.amax(dim=2) / 126.5).to(torch.float16)      # [n][nsb]
    d = d16.to(torch.float32).unsqueeze(2)
    sc = torch.where(d > 0, torch.ceil(s / torch.where(d > 0, d, torch.ones_like(d))),
                     torch.zeros_like(s)).clamp_(0, 127)
    step = (d * sc).unsqueeze(3)                           # [n][nsb][16][1]
    safe = torch.where(step > 0, step, torch.ones_like(step))
    q = torch.where(step > 0, torch.round(b / safe), torch.zeros_like(b)) + 32
    q = q.clamp_(0, 63).to(torch.uint8).reshape(n, nsb, Q6K_SUPER)
    low = q & 0xF
    lo = low[:, :, 0::2] | (low[:, :, 1::2] << 4)         # [n][nsb][128]
    high = q >> 4
    hi = (high[:, :, 0::4] | (high[:, :, 1::4] << 2) | (high[:, :, 2::4] << 4)
          | (high[:, :, 3::4] << 6))                      # [n][nsb][64]
    codes = torch.cat([lo, hi], dim=2).reshape(n, nsb * 192)
    dbytes = d16.view(torch.int16).unsqueeze(2)
    dlo = (dbytes & 0xFF).to(torch.uint8)
    dhi = ((dbytes >> 8) & 0xFF).to(torch.uint8)
    rec = torch.cat([sc.to(torch.uint8), dlo, dhi], dim=2).reshape(n, nsb * 18)
    return codes.contiguous(), rec.contiguous()


def quantize(w: torch.Tensor, fmt: str):
    """Returns (data, scale-or-None) in the planar layout for `fmt`."""
    if fmt == "f32":
        return w.contiguous(), None
    if fmt == "q8":
        return quantize_q8(w)
    if fmt == "q4":
        return quantize_q4(w)
    if fmt == "fp8":
        return quantize_fp8(w)
    if fmt == "q6k":
        return quantize_q6k(w)
    raise ValueError(f"unknown weight format {fmt!r}")


def weight(rows: int, cols: int, fmt: str, std: float, seed: int, name: str, device="cpu"):
    """A seeded [rows][cols] weight, N(0, std^2) then quantised to `fmt`."""
    return quantize(normal((rows, cols), std, seed, name, device), fmt)


# --------------------------------------------------------------------------
# Whole decoder inputs
# --------------------------------------------------------------------------
@dataclasses.dataclass
class LayerWeights:
    wqkv: tuple  # rows: q heads, then k heads, then v heads
    wo: tuple
    wgu: tuple   # rows: gate [0, I), then up [I, 2I)
    wd: tuple
    attn_gamma: torch.Tensor
    ffn_gamma: torch.Tensor


@dataclasses.dataclass
class DecoderWeights:
    layers: list
    out_gamma: torch.Tensor
    lm_head: tuple
    embed: torch.Tensor  # [vocab][hidden] fp32, gathered, not streamed


def decoder_layer(w: Decoder, layer: int, seed: int = 0, device="cpu",
                  gamma: str = "ones") -> LayerWeights:
    std = w.weight_std
    p = f"layer{layer}."
    H, I = w.hidden, w.intermediate
    return LayerWeights(
        wqkv=weight(w.qkv_rows, H, w.fmt, std, seed, p + "wqkv", device),
        wo=weight(H, w.n_heads * w.head_dim, w.fmt, std, seed, p + "wo", device),
        wgu=weight(2 * I, H, w.fmt, std, seed, p + "wgu", device),
        wd=weight(H, I, w.fmt, std, seed, p + "wd", device),
        attn_gamma=_gamma(H, gamma, seed, p + "attn_gamma", device),
        ffn_gamma=_gamma(H, gamma, seed, p + "ffn_gamma", device),
    )


def _gamma(h: int, kind: str, seed: int, name: str, device) -> torch.Tensor:
    if kind == "ones":
        return torch.ones(h, dtype=torch.float32, device=device)
    if kind == "random":  # 1 + N(0, 0.1^2): exercises a kernel that drops gamma
        return 1.0 + normal((h,), 0.1, seed, name, device)
    raise ValueError(kind)


def decoder_weights(w: Decoder, seed: int = 0, device="cpu", gamma: str = "ones",
                    layers: Optional[int] = None) -> DecoderWeights:
    n = w.n_layers if layers is None else layers
    return DecoderWeights(
        layers=[decoder_layer(w, l, seed, device, gamma) for l in range(n)],
        out_gamma=_gamma(w.hidden, gamma, seed, "out_gamma", device),
        lm_head=weight(w.vocab, w.hidden, w.lm_format, w.weight_std, seed, "lm_head", device),
        embed=normal((w.vocab, w.hidden), 1.0, seed, "embed", device),
    )


def first_tokens(w: Decoder, m: int, seed: int = 0, device="cpu") -> torch.Tensor:
    """Per-sequence first token ids; sequence i is drawn from its own stream so
    that the sets for smaller M are prefixes of the sets for larger M."""
    out = [uniform_int((1,), 0, w.vocab - 1, seed, f"tok0.seq{i}", device) for i in range(m)]
    return torch.cat(out)


def context_tokens(w: Decoder, m: int, n: int, seed: int = 0, device="cpu") -> torch.Tensor:
    """[m][n] random token ids for a teacher-forced decode context."""
    out = [uniform_int((n,), 0, w.vocab - 1, seed, f"ctx_tok.seq{i}", device) for i in range(m)]
    return torch.stack(out)


def context_lengths(w: Decoder, m: int, seed: int = 0) -> list:
    """Per-sequence context length (cache rows already filled at step 0)."""
    c = w.context
    if c == "none":
        return [0] * m
    kind, _, arg = c.partition(":")
    if kind == "decode":
        return [int(arg)] * m
    if kind == "kv":
        if "-" in arg:
            lo, hi = (int(v) for v in arg.split("-"))
            return [int(uniform_int((1,), lo, hi, seed, f"ctx_len.seq{i}")[0]) for i in range(m)]
        return [int(arg)] * m
    raise ValueError(c)


def kv_context_rows(w: Decoder, layer: int, seq: int, length: int, seed: int = 0,
                    device="cpu"):
    """Synthetic context rows for one (layer, sequence): K and V [nkv][length][hd]
    drawn from N(0,1)."""
    shape = (w.n_kv_heads, length, w.head_dim)
    k = normal(shape, 1.0, seed, f"ctx_k.l{layer}.s{seq}", device)
    v = normal(shape, 1.0, seed, f"ctx_v.l{layer}.s{seq}", device)
    return k, v


# --------------------------------------------------------------------------
# Standalone attention inputs
# --------------------------------------------------------------------------
def attention_inputs(a: Attention, seed: int = 0, device="cpu", m: Optional[int] = None,
                     max_len: Optional[int] = None, lengths=None):
    """q [M][nq][hd], k/v caches [M][nkv][max_len][hd] (rows >= len hold N(0,1)
    too, so an over-read shows), new rows k_new/v_new [M][nkv][hd], and
    per-sequence lengths L_m (the new row goes to position L_m - 1)."""
    m = a.m if m is None else m
    max_len = a.max_len if max_len is None else max_len
    if lengths is None:
        hi = min(a.len_hi, max_len)
        lengths = uniform_int((m,), a.len_lo, hi, seed, "fd_len", "cpu")
    lengths = torch.as_tensor(lengths, dtype=torch.int64)
    q = normal((m, a.n_heads, a.head_dim), 1.0, seed, "fd_q", device)
    kc = normal((m, a.n_kv_heads, max_len, a.head_dim), 1.0, seed, "fd_kc", device)
    vc = normal((m, a.n_kv_heads, max_len, a.head_dim), 1.0, seed, "fd_vc", device)
    kn = normal((m, a.n_kv_heads, a.head_dim), 1.0, seed, "fd_kn", device)
    vn = normal((m, a.n_kv_heads, a.head_dim), 1.0, seed, "fd_vn", device)
    return q, kc, vc, kn, vn, lengths
