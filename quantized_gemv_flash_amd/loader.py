"""Places a decoder's weights on the device for librra and creates the model.

Takes planar weights as (data, scale) tensor pairs on the target device (the
layout of include/rra.h's RRA_PLANAR), repacks the quantised ones into the tiled
GEMV layout with rra_repack_weight, allocates zeroed KV caches
[m_max][nkv][max_len][hd] per layer, and builds the rra_model descriptor.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import torch

from . import Model, Weight, device_weight


@dataclasses.dataclass
class DeviceDecoder:
    model: Model
    k_caches: List[torch.Tensor]
    v_caches: List[torch.Tensor]
    weights: list          # per layer dict of tiled Weights (kept alive)
    lm_head: Weight
    embed: Optional[torch.Tensor]

    def weight_bytes(self) -> int:
        """Bytes of weights one decode step streams (every layer + LM head)."""
        n = self.lm_head.nbytes
        for l in self.weights:
            n += sum(l[k].nbytes for k in ("wqkv", "wo", "wgu", "wd"))
        return n


def load_decoder(shape, weights, m_max: int, max_len: int, attn_chunk: int = 0,
                 drop_planar: bool = False, prefill_rows: int = 0, stream=None) -> DeviceDecoder:
    """`shape` has the decoder dimensions (n_layers, hidden, n_heads, n_kv_heads,
    head_dim, intermediate, vocab, fmt, rms_eps, rope_theta); `weights` has
    .layers (each with wqkv, wo, wgu, wd as (data, scale) pairs, attn_gamma,
    ffn_gamma), .out_gamma, .lm_head and .embed, all on one device."""
    S = shape
    dev = weights.out_gamma.device
    layers, kcs, vcs, keep = [], [], [], []
    for lw in weights.layers:
        d = {}
        for name in ("wqkv", "wo", "wgu", "wd"):
            data, scale = getattr(lw, name)
            d[name] = device_weight(data, scale, S.fmt, stream)
            if drop_planar and S.fmt != "f32":
                setattr(lw, name, (None, None))
        kc = torch.zeros((m_max, S.n_kv_heads, max_len, S.head_dim), dtype=torch.float32, device=dev)
        vc = torch.zeros_like(kc)
        kcs.append(kc)
        vcs.append(vc)
        d.update(attn_gamma=lw.attn_gamma, ffn_gamma=lw.ffn_gamma, k_cache=kc, v_cache=vc)
        layers.append(d)
        keep.append(d)
    lm_fmt = getattr(S, "lm_format", S.fmt)
    lm = device_weight(weights.lm_head[0], weights.lm_head[1], lm_fmt, stream)
    if drop_planar and lm_fmt != "f32":
        weights.lm_head = (None, None)
    model = Model(n_layers=len(layers), hidden=S.hidden, n_heads=S.n_heads,
                  n_kv_heads=S.n_kv_heads, head_dim=S.head_dim, intermediate=S.intermediate,
                  vocab=S.vocab, rms_eps=S.rms_eps, rope_theta=S.rope_theta, max_len=max_len,
                  m_max=m_max, layers=layers, out_gamma=weights.out_gamma, lm_head=lm,
                  embed=weights.embed, attn_chunk=attn_chunk, prefill_rows=prefill_rows,
                  stream=stream)
    return DeviceDecoder(model, kcs, vcs, keep, lm, weights.embed)
