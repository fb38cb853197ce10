"""Seeded synthetic inputs for the routed MoE FFN workloads.

This module is the only code that both the CPU oracle (``oracle/``) and the
HIP library's callers (tests, bench) use.  It draws random numbers and
writes them into the storage formats the library consumes; it computes
nothing of the method itself (no routing, no dequantisation, no matmul).

Random numbers
--------------
Every tensor is a counter-based stream: value ``c`` of the stream with key
``K`` is the SplitMix64 output ``mix64(K + (c + 1) * GAMMA)`` (Steele, Lea and
Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014; the
constants are those of the public-domain reference ``splitmix64.c``).  Keys
are derived from (seed, family, layer, tensor, expert) so that any single
expert can be regenerated on its own, on the host here or on the GPU by the
twin kernel in ``gpu_gen.hip`` (bit-identical by construction and by test).

Normal draws use inverse-CDF sampling from a 65,536-entry table of standard
normal quantiles: 16 bits of a SplitMix64 output pick the quantile of
probability ``(i + 0.5) / 65536``.  Each 64-bit output therefore gives four
N(0, 1) samples; a sample of N(0, sigma) is ``float32(sigma) * table[i]``
rounded once in fp32.  Only IEEE-exact operations follow the table lookup,
which is what lets the GPU twin reproduce the host bytes exactly.

Stored weight formats (the library's input contract)
-----------------------------------------------------
A matrix used as ``x @ W`` with ``W`` of shape [K x N] is stored output-major:
row ``n`` holds the K reduction weights in blocks of 32 consecutive k.

* codes ``q``: uint32 ``[N][K/32][words]`` (words = 2 for 2-bit, 3 for 3-bit)
* scales ``s``: uint16 ``[N][K/32]`` holding IEEE binary16 bits

2-bit: code = level + 2 for levels -2..1; weight i of a block sits in word
i // 16 at bits [2 (i mod 16), +2).  3-bit: code = level + 4 for levels -4..3;
the three words are one little-endian 96-bit string and weight i occupies
bits [3 i, 3 i + 3) (weights 10 and 21 straddle a word boundary).

Quantiser (input preparation only; the library never quantises): per block
``a = max |w|`` in fp32, ``s = fp16_rne(a / 2)`` (2-bit) or ``a / 4`` (3-bit),
``level = clamp(rint_half_even(w / s), lo, hi)`` with the division rounded
once in fp32, and every level 0 when ``s == 0``.

The pages (Strata write-ups, e.g. aiproducthub "Strata Skill", section
功能与原则; bnskd "Strata：把 125B 大模型塞进 12GB 显卡", table 实测数据) name
the 2-bit "Q2_0" tier and 3-bit tiers but print no bit layout; the layout
above is this library's own definition of those block formats.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "GAMMA", "M1", "M2", "mix64", "derive_key", "splitmix_stream",
    "NORMAL_TABLE", "normal", "bf16_bits_from_f32", "f32_from_bf16_bits",
    "quantize_blocks", "pack_codes", "expert_tensor_host",
    "Workload", "WORKLOADS", "router_host", "activations_host",
    "GATE", "UP", "DOWN", "ROUTER", "BIAS_PERM", "ACT",
    "expert_key", "tensor_shape",
]

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB

# tensor ids used in key derivation
GATE, UP, DOWN, ROUTER, BIAS_PERM, ACT = 0, 1, 2, 3, 4, 5
# model families: the tiny shapes and the full 2048/768/512 shapes
FAMILY_TINY, FAMILY_FULL, FAMILY_CODER = 1, 2, 3


def mix64(z: int) -> int:
    """SplitMix64 finaliser on a Python int (mod 2**64)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * M1) & MASK64
    z = ((z ^ (z >> 27)) * M2) & MASK64
    return z ^ (z >> 31)


def derive_key(*fields: int) -> int:
    """Fold integer fields into a 64-bit stream key."""
    h = 0
    for f in fields:
        h = mix64(((h ^ (int(f) & MASK64)) + GAMMA) & MASK64)
    return h


def splitmix_stream(key: int, start: int, n: int) -> np.ndarray:
    """Outputs ``start .. start+n-1`` of the SplitMix64 stream with ``key``."""
    with np.errstate(over="ignore"):
        c = np.arange(start + 1, start + n + 1, dtype=np.uint64)
        z = np.uint64(key) + c * np.uint64(GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(M2)
        z = z ^ (z >> np.uint64(31))
    return z


def _normal_table() -> np.ndarray:
    from scipy.special import ndtri
    p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
    return ndtri(p).astype(np.float32)


NORMAL_TABLE = _normal_table()


def normal(key: int, n: int, sigma: float = 1.0, start: int = 0) -> np.ndarray:
    """``n`` fp32 samples of N(0, sigma) from stream ``key``; sample c uses
    16-bit lane ``c % 4`` of stream output ``c // 4``.  ``start`` must be a
    multiple of 4."""
    assert start % 4 == 0
    nh = (n + 3) // 4
    h = splitmix_stream(key, start // 4, nh)
    idx = (h[:, None] >> np.array([0, 16, 32, 48], dtype=np.uint64)) & np.uint64(0xFFFF)
    v = NORMAL_TABLE[idx.reshape(-1)[:n].astype(np.int64)]
    return (np.float32(sigma) * v).astype(np.float32)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- quantiser

def quantize_blocks(v: np.ndarray, bits: int):
    """Quantise ``v`` [N][K] fp32 along K in blocks of 32.

    Returns (levels int8 [N][K/32][32], scale bits uint16 [N][K/32])."""
    assert bits in (2, 3)
    n, k = v.shape
    assert k % 32 == 0
    blk = v.reshape(n, k // 32, 32).astype(np.float32)
    half = np.float32(2.0 if bits == 2 else 4.0)
    lo, hi = (-2, 1) if bits == 2 else (-4, 3)
    a = np.max(np.abs(blk), axis=-1)
    s16 = (a / half).astype(np.float16)
    sf = s16.astype(np.float32)
    safe = np.where(sf > 0, sf, np.float32(1.0))
    with np.errstate(divide="ignore", invalid="ignore"):
        q = blk / safe[..., None]
    lev = np.clip(np.rint(q), lo, hi)
    lev = np.where(sf[..., None] > 0, lev, 0).astype(np.int8)
    return lev, s16.view(np.uint16)


def pack_codes(levels: np.ndarray, bits: int) -> np.ndarray:
    """Pack levels [..., 32] into uint32 words [..., words] (format above)."""
    bias = 2 if bits == 2 else 4
    codes = (levels.astype(np.int64) + bias).astype(np.uint64)
    shp = codes.shape[:-1]
    if bits == 2:
        out = np.zeros(shp + (2,), dtype=np.uint64)
        for i in range(32):
            out[..., i // 16] |= codes[..., i] << np.uint64(2 * (i % 16))
    else:
        out = np.zeros(shp + (3,), dtype=np.uint64)
        for i in range(32):
            pos = 3 * i
            w, off = divmod(pos, 32)
            out[..., w] |= (codes[..., i] << np.uint64(off)) & np.uint64(0xFFFFFFFF)
            if off > 29:
                out[..., w + 1] |= codes[..., i] >> np.uint64(32 - off)
    return (out & np.uint64(0xFFFFFFFF)).astype(np.uint32)


# ---------------------------------------------------------------- workloads

@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, formats and the seed of every stream."""
    name: str
    family: int
    n_layers: int
    n_experts: int
    d_model: int
    d_ff: int
    top_k: int
    n_tokens: int
    bits: int
    x_dtype: str          # "f32" or "bf16"
    zipf_bias: bool
    chained: bool         # residual stream + RMSNorm between layers
    seed: int = 0
    act_tag: int = 0
    note: str = field(default="", compare=False)

    @property
    def words(self) -> int:
        return 2 if self.bits == 2 else 3

    def expert_bytes(self) -> int:
        """Packed bytes of one expert (codes + scales of gate, up, down)."""
        w = 3 * self.d_model * self.d_ff
        return w // 32 * (4 * self.words + 2)


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny", FAMILY_TINY, 1, 16, 256, 128, 2, 8, 2, "f32", False, False, act_tag=1,
                 note="1 layer, 16 experts, d_model 256, d_ff 128, top-2, 8 tokens"),
        Workload("decode_1layer", FAMILY_FULL, 1, 512, 2048, 768, 10, 1, 2, "bf16", True, False, act_tag=2,
                 note="single-layer decode, batch 1"),
        Workload("decode_48layer", FAMILY_FULL, 48, 512, 2048, 768, 10, 1, 2, "f32", True, True, act_tag=3,
                 note="48-layer decode step, batch 1, RMSNorm chain"),
        Workload("prefill_8192", FAMILY_FULL, 1, 512, 2048, 768, 10, 8192, 2, "bf16", True, False, act_tag=4,
                 note="one 8,192-token prefill chunk through one layer"),
        Workload("verify4_3bit", FAMILY_FULL, 48, 512, 2048, 768, 10, 4, 3, "f32", True, True, act_tag=5,
                 note="4-token verify batch through 48 layers, 3-bit experts"),
        # the pages' Coder build keeps about half of the experts; a short
        # stack of such layers is a shape variant for the tests
        Workload("coder_256", FAMILY_CODER, 4, 256, 2048, 768, 10, 2, 2, "f32", True, True, act_tag=6,
                 note="4 layers x 256 experts, 2 tokens, 2-bit"),
        # a prompt cut into chunks through a short stack of tiny layers
        Workload("tiny_stack", FAMILY_TINY, 3, 16, 256, 128, 2, 40, 2, "f32", True, True, act_tag=7,
                 note="3 layers x 16 experts, 40 tokens, chunked prefill"),
    ]
}


def tensor_shape(wl: Workload, tensor: int):
    """(N, K) of a stored expert tensor: rows are outputs, K the reduction."""
    if tensor in (GATE, UP):
        return wl.d_ff, wl.d_model
    return wl.d_model, wl.d_ff


def expert_key(wl: Workload, layer: int, tensor: int, expert: int) -> int:
    # no workload tag: every full-shape workload shares layer 0 draws and the
    # 3-bit workload quantises the same normal draws as the 2-bit ones
    return derive_key(wl.seed, wl.family, layer, tensor, expert)


def expert_tensor_host(wl: Workload, layer: int, tensor: int, expert: int, bits: int | None = None):
    """Packed (codes uint32 [N][K/32][words], scales uint16 [N][K/32]) of one
    expert tensor, generated on the host."""
    bits = wl.bits if bits is None else bits
    n, k = tensor_shape(wl, tensor)
    v = normal(expert_key(wl, layer, tensor, expert), n * k, 0.02).reshape(n, k)
    lev, s = quantize_blocks(v, bits)
    return pack_codes(lev, bits), s


def router_host(wl: Workload, layer: int):
    """Router weight [d_model][n_experts] fp32 ~ N(0, 0.02) and bias [n_experts].

    The bias gives the router a Zipf(1.1) prior over experts:
    ``b_e = -1.1 ln(rank_e)`` with ``rank`` a seeded permutation of 1..E
    (zero bias for workloads without the skew)."""
    e, d = wl.n_experts, wl.d_model
    w = normal(derive_key(wl.seed, wl.family, layer, ROUTER, 0), d * e, 0.02).reshape(d, e)
    if wl.zipf_bias:
        h = splitmix_stream(derive_key(wl.seed, wl.family, layer, BIAS_PERM, 0), 0, e)
        rank = np.empty(e, dtype=np.int64)
        rank[np.argsort(h, kind="stable")] = np.arange(1, e + 1)
        b = (-1.1 * np.log(rank.astype(np.float64))).astype(np.float32)
    else:
        b = np.zeros(e, dtype=np.float32)
    return w, b


def activations_host(wl: Workload, n_tokens: int | None = None, stream: int = 0):
    """Activations [T][d_model] ~ N(0, 1): fp32, or bf16 bits (uint16) when
    the workload's activations are bf16 (fp32 draw rounded to nearest even)."""
    t = wl.n_tokens if n_tokens is None else n_tokens
    x = normal(derive_key(wl.seed, wl.family, ACT, wl.act_tag, stream), t * wl.d_model, 1.0)
    x = x.reshape(t, wl.d_model)
    if wl.x_dtype == "bf16":
        return bf16_bits_from_f32(x)
    return x
