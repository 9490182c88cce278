"""Seeded synthetic inputs for the ZeRO shard step: layouts and random draws.

This module is the only code the HIP path and the oracle both use.  It holds
none of the method's arithmetic (no flatten, norm, loss scaling or Adam): it
describes which parameters one data-parallel rank owns and draws the seeded
values that stand in for a real model's state and gradients.

Layouts.  A model is a list of named tensors in a fixed flat order.  ZeRO
partitions the flat model state across the Nd data-parallel ranks instead of
replicating it (ZeRO paper card, "Method"; DeepSpeed article on ZeRO); here
rank r owns the contiguous range [r*P, min((r+1)*P, psi)) with P = ceil(psi/Nd).
The tensors that intersect that range give the flatten segments
(tensor, src_off, dst_off, count).

Shapes:
  * GPT-2 1.5B-like: 48 layers, hidden 1600, vocab 50257, 1024 positions; the
    page on the ZeRO paper uses a 1.5B GPT-2-like model for its memory
    arithmetic ("Bottleneck").  Order: wte, wpe, 48 blocks, ln_f.
  * 100B GPT-like: 125 layers, hidden 8192, 64 heads, 16-way model parallel
    (the paper card's configuration table, "Evidence").  The shard is one
    model-parallel rank's slice of the layer stack (Megatron column/row
    split, biases and layer norms of row-split layers replicated); the table
    gives no embedding, so none is included.
  * 1T: a stack of hidden-8192 GPT blocks with psi taken as exactly 10^12 (the
    paper card's trillion-parameter arithmetic, "Evidence"; no shapes are
    printed), so each of 1024 ranks owns 976,562,500 parameters.

Draws.  Every array is filled in chunks of 2^22 elements; chunk j of stream
(seed, *words) comes from its own PCG64 generator seeded with
SeedSequence([seed, *words, j]), so the values do not depend on how many
threads fill them.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

CHUNK = 1 << 22
F16_NAN_SENTINEL = 0x7E00      # fills source-tensor elements outside the shard
F16_POS_INF = 0x7C00

# --------------------------------------------------------------------------
# tensor lists
# --------------------------------------------------------------------------


def _gpt_block(h: int, mp: int = 1, prefix: str = "") -> List[Tuple[str, int]]:
    """One GPT block's tensors as a model-parallel rank holds them."""
    return [
        (prefix + "ln1.w", h), (prefix + "ln1.b", h),
        (prefix + "attn.qkv.w", h * 3 * h // mp), (prefix + "attn.qkv.b", 3 * h // mp),
        (prefix + "attn.proj.w", (h // mp) * h), (prefix + "attn.proj.b", h),
        (prefix + "ln2.w", h), (prefix + "ln2.b", h),
        (prefix + "mlp.fc.w", h * 4 * h // mp), (prefix + "mlp.fc.b", 4 * h // mp),
        (prefix + "mlp.proj.w", (4 * h // mp) * h), (prefix + "mlp.proj.b", h),
    ]


def gpt2_1p5b_tensors() -> List[Tuple[str, int]]:
    h, layers, vocab, ctx = 1600, 48, 50257, 1024
    out = [("wte", vocab * h), ("wpe", ctx * h)]
    for layer in range(layers):
        out += _gpt_block(h, 1, f"h{layer}.")
    out += [("ln_f.w", h), ("ln_f.b", h)]
    return out


def gpt_100b_mp16_tensors() -> List[Tuple[str, int]]:
    h, layers, mp = 8192, 125, 16
    out = []
    for layer in range(layers):
        out += _gpt_block(h, mp, f"h{layer}.")
    return out


class _BlockStack:
    """Lazy tensor list of an unbounded stack of GPT blocks (the 1T model)."""

    def __init__(self, h: int):
        self.block = _gpt_block(h)
        self.per_block = sum(c for _, c in self.block)

    def tensors_in(self, begin: int, end: int):
        """Yield (flat_offset, name, numel) of tensors intersecting [begin, end)."""
        layer = begin // self.per_block
        off = layer * self.per_block
        while off < end:
            for name, numel in self.block:
                if off + numel > begin and off < end:
                    yield off, f"h{layer}.{name}", numel
                off += numel
            layer += 1


# --------------------------------------------------------------------------
# shard layout
# --------------------------------------------------------------------------


@dataclass
class ShardLayout:
    """One rank's share of a flat model state and the tensors it comes from."""
    model: str
    psi: int
    nd: int
    rank: int
    start: int                       # first owned flat index
    n: int                           # owned element count
    tensor_names: List[str]          # source tensors that intersect the shard
    tensor_numels: List[int]
    segments: List[Tuple[int, int, int, int]]   # (tensor index, src_off, dst_off, count)


def _layout_from(model: str, psi: int, nd: int, rank: int, tensors_with_offsets) -> ShardLayout:
    P = -(-psi // nd)
    start = rank * P
    end = min(psi, start + P)
    names, numels, segs = [], [], []
    for off, name, numel in tensors_with_offsets:
        lo, hi = max(off, start), min(off + numel, end)
        if lo >= hi:
            continue
        segs.append((len(names), lo - off, lo - start, hi - lo))
        names.append(name)
        numels.append(numel)
    return ShardLayout(model, psi, nd, rank, start, end - start, names, numels, segs)


def _with_offsets(tensors):
    off = 0
    for name, numel in tensors:
        yield off, name, numel
        off += numel


def layout_from_tensors(model: str, tensors: Sequence[Tuple[str, int]], nd: int, rank: int) -> ShardLayout:
    psi = sum(c for _, c in tensors)
    return _layout_from(model, psi, nd, rank, _with_offsets(tensors))


def gpt2_layout(nd: int = 16, rank: Optional[int] = None) -> ShardLayout:
    return layout_from_tensors("gpt2-1.5b", gpt2_1p5b_tensors(), nd, nd // 2 if rank is None else rank)


def gpt100b_layout(nd: int = 25, rank: Optional[int] = None) -> ShardLayout:
    return layout_from_tensors("gpt-100b-mp16", gpt_100b_mp16_tensors(), nd,
                               nd // 2 if rank is None else rank)


def gpt1t_layout(nd: int = 1024, rank: Optional[int] = None) -> ShardLayout:
    psi = 10 ** 12
    rank = nd // 2 if rank is None else rank
    P = -(-psi // nd)
    start = rank * P
    stack = _BlockStack(8192)
    return _layout_from("gpt-1t-h8192", psi, nd, rank,
                        stack.tensors_in(start, min(psi, start + P)))


def single_tensor_layout(n: int) -> ShardLayout:
    return layout_from_tensors(f"flat-{n}", [("flat", n)], 1, 0)


# --------------------------------------------------------------------------
# workload configurations
# --------------------------------------------------------------------------


@dataclass
class HParams:
    lr: float = 1e-4
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    max_grad_norm: float = 1.0
    backoff: float = 0.5
    growth: float = 2.0
    min_scale: float = 1.0
    growth_interval: int = 20


@dataclass
class Workload:
    name: str
    layout: ShardLayout
    sigma_p: float                  # master params ~ N(0, sigma_p), fp32
    sigma_g: float                  # unscaled grads ~ N(0, sigma_g), fp32 before scaling
    scale0: float                   # initial loss scale S
    steps: int
    seed: int = 0
    hp: HParams = field(default_factory=HParams)
    inject: Dict[int, int] = field(default_factory=dict)   # 1-based step -> fp16 bit pattern
    bucket_elems: int = 0           # 0: one flatten call for the whole shard

    @property
    def n(self) -> int:
        return self.layout.n


def workload(name: str) -> Workload:
    """The five synthetic workloads (tiny, gpt2, stress, 100b, 1t)."""
    if name == "tiny":
        return Workload("tiny", single_tensor_layout(1 << 20), 0.02, 1e-3, 2.0 ** 16, 10)
    if name == "gpt2":
        return Workload("gpt2", gpt2_layout(), 0.02, 1e-3, 2.0 ** 16, 100)
    if name == "stress":
        return Workload("stress", gpt2_layout(), 0.02, 1e-4, 2.0 ** 24, 100,
                        inject={3: F16_POS_INF, 7: F16_NAN_SENTINEL})
    if name == "100b":
        return Workload("100b", gpt100b_layout(), 0.02, 1e-4, 2.0 ** 16, 50)
    if name == "1t":
        return Workload("1t", gpt1t_layout(), 0.006, 1e-4, 2.0 ** 16, 20,
                        bucket_elems=25_000_000)
    raise KeyError(name)


WORKLOADS = ("tiny", "gpt2", "stress", "100b", "1t")

# --------------------------------------------------------------------------
# seeded draws
# --------------------------------------------------------------------------

_THREADS = max(1, min(16, os.cpu_count() or 1))


def standard_normal_f32(n: int, words: Sequence[int]) -> np.ndarray:
    """n standard-normal float32 draws of stream `words`, chunked as above."""
    out = np.empty(n, np.float32)

    def fill(j: int) -> None:
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([*words, j])))
        lo = j * CHUNK
        g.standard_normal(out=out[lo:min(n, lo + CHUNK)], dtype=np.float32)

    chunks = range(-(-n // CHUNK))
    if n > CHUNK and _THREADS > 1:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, chunks))
    else:
        for j in chunks:
            fill(j)
    return out


def master_params(w: Workload) -> np.ndarray:
    """fp32 master parameters ~ N(0, sigma_p)."""
    x = standard_normal_f32(w.n, [w.seed, 1])
    x *= np.float32(w.sigma_p)
    return x


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> binary16 bit patterns via numpy (round to nearest even)."""
    with np.errstate(over="ignore"):
        return x.astype(np.float16).view(np.uint16)


def injection_position(w: Workload, step: int) -> int:
    return int(np.random.default_rng(np.random.SeedSequence([w.seed, 3, step])).integers(w.n))


def scaled_f16_normals(n: int, words: Sequence[int], sigma: float, scale: float) -> np.ndarray:
    """f16(z * sigma * scale) bit patterns for the standard normals z of
    stream `words` (same draws as standard_normal_f32); the fp32 products and
    the numpy round-to-nearest-even cast are done chunk by chunk in threads."""
    out = np.empty(n, np.uint16)
    sig, sc = np.float32(sigma), np.float32(scale)

    def fill(j: int) -> None:
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([*words, j])))
        lo, hi = j * CHUNK, min(n, (j + 1) * CHUNK)
        z = g.standard_normal(hi - lo, dtype=np.float32)
        z *= sig
        z *= sc
        out[lo:hi] = to_f16_bits(z)

    chunks = range(-(-n // CHUNK))
    if n > CHUNK and _THREADS > 1:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, chunks))
    else:
        for j in chunks:
            fill(j)
    return out


def grad_partition(w: Workload, step: int, scale: float) -> np.ndarray:
    """The rank's flat binary16 gradient for 1-based `step`, scaled by the
    current loss scale: f16(g_true * S) with g_true ~ N(0, sigma_g) in fp32.
    Injected inf/NaN patterns are written after the conversion."""
    bits = scaled_f16_normals(w.n, [w.seed, 2, step], w.sigma_g, scale)
    if step in w.inject:
        bits[injection_position(w, step)] = w.inject[step]
    return bits


def source_tensors(layout: ShardLayout, gpart: np.ndarray) -> List[np.ndarray]:
    """Per-layer binary16 tensors (uint16) holding gpart at the shard's
    segments; every element outside the shard holds a NaN sentinel, so a
    flatten that reads outside its segments shows up as an overflow."""
    out = []
    for numel in layout.tensor_numels:
        out.append(np.full(numel, F16_NAN_SENTINEL, np.uint16))
    for t, so, do, cnt in layout.segments:
        out[t][so:so + cnt] = gpart[do:do + cnt]
    return out


def random_segments(rng: np.random.Generator, n: int, max_seg: int, misalign: bool = True):
    """A random cover of [0, n) by segments, each from its own small source
    tensor at a random (possibly unaligned) offset.  Returns
    (tensor_numels, segments)."""
    numels, segs = [], []
    d = 0
    while d < n:
        cnt = int(min(n - d, rng.integers(1, max_seg + 1)))
        pad_lo = int(rng.integers(0, 9)) if misalign else 0
        pad_hi = int(rng.integers(0, 9)) if misalign else 0
        segs.append((len(numels), pad_lo, d, cnt))
        numels.append(pad_lo + cnt + pad_hi)
        d += cnt
    return numels, segs


def layout_summary(layout: ShardLayout) -> str:
    counts = [c for *_, c in layout.segments]
    return (f"{layout.model}: psi={layout.psi:,} nd={layout.nd} rank={layout.rank} "
            f"n={layout.n:,} segments={len(counts)} (min {min(counts):,}, max {max(counts):,})")


def expected_norm_estimate(w: Workload) -> float:
    """sqrt(n) * sigma_g: the typical unscaled gradient norm (for reports only)."""
    return math.sqrt(w.n) * w.sigma_g
