"""Synthetic workloads: the flat parameter groups and step settings.

Shape-only stand-ins for the models the ZeRO pages train (a ToyModel of
Linear layers, BERT-base, LLaMA-class decoders) and a fragmented-bucket case.
Values come from ``synth`` (seeded); no dataset or checkpoint is involved.
Names follow the usual module naming of each architecture.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

from . import BF16, FP16, KIND_GRAD, KIND_INIT, KIND_INJECT, KIND_SIZES, NormalSpec
from . import hash64, normal_spec, scaled, stream_key

WEIGHT, BIAS, NORM = "weight", "bias", "norm"


@dataclass
class Workload:
    name: str
    tensors: List[Tuple[str, int, str]]      # (name, numel, kind)
    world: int                               # N data-parallel ranks
    dtype: int                               # FP16 / BF16 gradient and parameter copy
    grad_sigma: float
    steps: int
    align: int = 2                           # start-alignment factor, in elements
    init_sigma: float = 0.02
    scale0: float = 1.0                      # initial loss scale
    dynamic: bool = False                    # dynamic loss scaling
    window: int = 1000
    min_scale: float = 1.0
    clip: float = 0.0                        # max grad norm, 0 = off
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    owners: str = "first"                    # "first": owner 0 only; "all": every owner
    bucket_cap: Optional[int] = None         # reduce bucket size, elements
    inject_every: int = 0                    # inject inf/NaN every k-th step (1-based)
    rank_shift: int = 0                      # rank r's draw is scaled by 2^-(r * rank_shift)
    seed: int = 1
    description: str = ""

    @property
    def numels(self) -> np.ndarray:
        return np.array([t[1] for t in self.tensors], dtype=np.int64)

    @property
    def phi(self) -> int:
        return int(sum(t[1] for t in self.tensors))

    def grad_spec(self, scale: float, rank: int = 0) -> NormalSpec:
        """The draw of rank `rank`'s gradient at loss scale `scale`.  With
        rank_shift the ranks' values sit on binary grids rank_shift binades
        apart, so their sums in fp32 are no longer exact."""
        base = normal_spec(self.grad_sigma, self.dtype)
        factor = scale * 2.0 ** (-rank * self.rank_shift)
        return scaled(base, factor) if factor != 1.0 else base

    def init_spec(self) -> NormalSpec:
        return normal_spec(self.init_sigma, self.dtype)

    def grad_key(self, step: int, rank: int) -> int:
        return stream_key(self.seed, KIND_GRAD, step, rank)

    def init_key(self) -> int:
        return stream_key(self.seed, KIND_INIT, 0, 0)


def _linear(prefix: str, n_in: int, n_out: int, bias: bool = True):
    out = [(prefix + ".weight", n_out * n_in, WEIGHT)]
    if bias:
        out.append((prefix + ".bias", n_out, BIAS))
    return out


def toy_tensors(hidden: int = 1024, layers: int = 12, classes: int = 10):
    """ToyModel of the wmrh.cn ZeRO article, section 3.1: `layers` blocks of
    Linear(h, 4h) -> GELU -> Linear(4h, h) and a Linear(h, classes) head."""
    t = []
    for i in range(layers):
        t += _linear(f"layers.{i}.0", hidden, 4 * hidden)
        t += _linear(f"layers.{i}.2", 4 * hidden, hidden)
    t += _linear("classifier", hidden, classes)
    return t


def bert_tensors(hidden: int = 768, layers: int = 12, ffn: int = 3072, vocab: int = 30522,
                 max_pos: int = 512, types: int = 2):
    t = [("embeddings.word_embeddings.weight", vocab * hidden, WEIGHT),
         ("embeddings.position_embeddings.weight", max_pos * hidden, WEIGHT),
         ("embeddings.token_type_embeddings.weight", types * hidden, WEIGHT),
         ("embeddings.LayerNorm.weight", hidden, NORM),
         ("embeddings.LayerNorm.bias", hidden, BIAS)]
    for i in range(layers):
        p = f"encoder.layer.{i}"
        t += _linear(p + ".attention.self.query", hidden, hidden)
        t += _linear(p + ".attention.self.key", hidden, hidden)
        t += _linear(p + ".attention.self.value", hidden, hidden)
        t += _linear(p + ".attention.output.dense", hidden, hidden)
        t += [(p + ".attention.output.LayerNorm.weight", hidden, NORM),
              (p + ".attention.output.LayerNorm.bias", hidden, BIAS)]
        t += _linear(p + ".intermediate.dense", hidden, ffn)
        t += _linear(p + ".output.dense", ffn, hidden)
        t += [(p + ".output.LayerNorm.weight", hidden, NORM),
              (p + ".output.LayerNorm.bias", hidden, BIAS)]
    t += _linear("pooler.dense", hidden, hidden)
    return t


def llama_tensors(d: int, layers: int, ffn: int, vocab: int = 32000, kv_dim: Optional[int] = None):
    kv = d if kv_dim is None else kv_dim
    t = [("model.embed_tokens.weight", vocab * d, WEIGHT)]
    for i in range(layers):
        p = f"model.layers.{i}"
        t += [(p + ".self_attn.q_proj.weight", d * d, WEIGHT),
              (p + ".self_attn.k_proj.weight", kv * d, WEIGHT),
              (p + ".self_attn.v_proj.weight", kv * d, WEIGHT),
              (p + ".self_attn.o_proj.weight", d * d, WEIGHT),
              (p + ".mlp.gate_proj.weight", ffn * d, WEIGHT),
              (p + ".mlp.up_proj.weight", ffn * d, WEIGHT),
              (p + ".mlp.down_proj.weight", d * ffn, WEIGHT),
              (p + ".input_layernorm.weight", d, NORM),
              (p + ".post_attention_layernorm.weight", d, NORM)]
    t += [("model.norm.weight", d, NORM), ("lm_head.weight", vocab * d, WEIGHT)]
    return t


def bucket_tensors(n: int = 10000, lo: int = 64, hi: int = 1 << 20, seed: int = 5):
    """n tensors, sizes log-uniform in [lo, hi], drawn from the seeded hash."""
    key = stream_key(seed, KIND_SIZES, 0, 0)
    span = math.log2(hi / lo)
    t = []
    for k in range(n):
        u = (hash64(key, k) >> 11) * 2.0 ** -53
        size = int(math.floor(lo * 2.0 ** (span * u)))
        t.append((f"bucket_tensor.{k}", max(lo, min(hi, size)), WEIGHT))
    return t


def _make() -> dict:
    w = {}
    w["toy"] = Workload(
        name="toy", tensors=toy_tensors(), world=8, dtype=FP16, grad_sigma=1e-3, steps=10,
        scale0=2.0 ** 16, dynamic=True, seed=1,
        description="ToyModel flat buffer (12x[Linear 1024->4096, Linear 4096->1024] + "
                    "Linear 1024->10), N=8, fp16 grads N(0,1e-3)x2^16")
    w["bert"] = Workload(
        name="bert", tensors=bert_tensors(), world=8, dtype=FP16, grad_sigma=1e-3, steps=20,
        scale0=2.0 ** 16, dynamic=True, clip=1.0, seed=2,
        description="BERT-base-shaped flat buffer (12 layers, hidden 768, FFN 3072, "
                    "vocab 30522), N=8, fp16 grads, clip 1.0")
    w["llama7b"] = Workload(
        name="llama7b", tensors=llama_tensors(4096, 32, 11008), world=8, dtype=BF16,
        grad_sigma=1e-4, steps=5, clip=1.0, bucket_cap=500_000_000, seed=3,
        description="LLaMA-7B-shaped flat buffer (32 layers, d=4096, FFN 11008, vocab 32000), "
                    "N=8, bf16 grads N(0,1e-4), clip 1.0, 5e8-element reduce buckets")
    w["llama70b"] = Workload(
        name="llama70b", tensors=llama_tensors(8192, 80, 28672, kv_dim=1024), world=8,
        dtype=BF16, grad_sigma=1e-4, steps=3, clip=1.0, bucket_cap=500_000_000, seed=4,
        description="LLaMA-70B-shaped flat buffer (80 layers, d=8192, FFN 28672, GQA 8 KV heads, "
                    "vocab 32000), N=8, bf16 grads N(0,1e-4), clip 1.0, 5e8-element reduce "
                    "buckets")
    w["buckets"] = Workload(
        name="buckets", tensors=bucket_tensors(), world=16, dtype=FP16, grad_sigma=1e-3,
        steps=40, scale0=2.0 ** 16, dynamic=True, owners="all", bucket_cap=500_000_000,
        inject_every=4, seed=5,
        description="10,000 tensors log-uniform in [64, 2^20] in 5e8-element reduce buckets, "
                    "N=16, fp16 grads x dynamic loss scale, inf/NaN every 4th step")
    # the same structure at a size the oracle runs in full in seconds
    w["buckets_small"] = Workload(
        name="buckets_small", tensors=bucket_tensors(400, 64, 1 << 14, seed=6), world=16,
        dtype=FP16, grad_sigma=1e-3, steps=40, scale0=2.0 ** 16, dynamic=True, owners="all",
        bucket_cap=400_000, inject_every=4, seed=6,
        description="400 tensors log-uniform in [64, 2^14] in 4e5-element reduce buckets, "
                    "N=16, dynamic loss scale, inf/NaN every 4th step")
    # ToyModel whose ranks' gradients sit on grids 3 binades apart (rank 7's
    # values are 2^-21 times rank 0's): the fp32 sums of the reduce round
    w["toy_offgrid"] = Workload(
        name="toy_offgrid", tensors=toy_tensors(), world=8, dtype=FP16, grad_sigma=1e-3,
        steps=3, scale0=2.0 ** 16, dynamic=True, rank_shift=3, seed=11,
        description="ToyModel flat buffer, N=8, fp16 grads N(0,1e-3)x2^16x2^-3r for rank r "
                    "(off one common grid)")
    w["toy_tiny"] = Workload(
        name="toy_tiny", tensors=toy_tensors(hidden=64, layers=2, classes=10), world=8,
        dtype=FP16, grad_sigma=1e-3, steps=3, scale0=2.0 ** 16, dynamic=True, seed=9,
        description="ToyModel with hidden 64 and 2 layers (smoke size)")
    return w


WORKLOADS = _make()


def bucket_windows(wl: Workload, offsets: np.ndarray, padded: int, bucket_first: np.ndarray):
    """Element ranges [a, b) of the reduce buckets; the last one takes the
    alignment padding."""
    out = []
    nb = bucket_first.size - 1
    for k in range(nb):
        a = int(offsets[bucket_first[k]]) if bucket_first[k] < len(offsets) else wl.phi
        b = int(offsets[bucket_first[k + 1]]) if k + 1 < nb else padded
        out.append((a, b))
    return out


def tensor_segments(wl: Workload, offsets: np.ndarray, begin: int, end: int):
    """(start, stop, kind) pieces of the flat range [begin, end) that lie in a
    tensor; padding past the last tensor is not listed (it stays zero)."""
    out = []
    numels = wl.numels
    k = int(np.searchsorted(offsets, begin, side="right")) - 1
    k = max(k, 0)
    while k < len(numels) and offsets[k] < end:
        a = max(begin, int(offsets[k]))
        b = min(end, int(offsets[k] + numels[k]))
        if a < b:
            out.append((a, b, wl.tensors[k][2]))
        k += 1
    return out


def injections(wl: Workload, padded: int):
    """{step: (rank, index, kind)} for the inf/NaN injections (1-based steps).
    kind is "inf" on odd occurrences and "nan" on even ones."""
    if not wl.inject_every:
        return {}
    out = {}
    key = stream_key(wl.seed, KIND_INJECT, 0, 0)
    phi = wl.phi
    occ = 0
    for s in range(wl.inject_every, wl.steps + 1, wl.inject_every):
        occ += 1
        h = hash64(key, 2 * s)
        g = hash64(key, 2 * s + 1)
        out[s] = (int(h % wl.world), int(g % phi), "inf" if occ % 2 == 1 else "nan")
    return out
