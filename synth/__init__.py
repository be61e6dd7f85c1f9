"""Seeded synthetic attention inputs, shared bit-for-bit by the GPU path and the oracle.

This module holds no attention arithmetic: it only draws numbers.  Every tensor is
a deterministic function of (seed, element index), so any subset of it can be
regenerated independently of the rest:

* uniform bits: SplitMix64 used as a counter-based generator.  Output n of the
  stream for ``seed`` is ``mix64(seed + (n + 1) * 0x9E3779B97F4A7C15)`` with the
  published SplitMix64 finaliser (Steele, Lea and Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014; constants as in Vigna's
  reference code).  This is exactly the sequence the stateful SplitMix64 gives
  when seeded with ``seed``.
* normals: Box-Muller on consecutive output pairs (2p, 2p+1), with
  u = (x >> 11) * 2**-53, r = sqrt(-2 ln(1 - u1)), theta = 2 pi u2,
  z[2p] = r cos theta, z[2p+1] = r sin theta, evaluated in float64.
* storage: float64 -> float32 (round to nearest even) -> bfloat16 (round to
  nearest even on the float32 bit pattern).  Optional multiplier applied in
  float64 before the float32 rounding (the "x3" peaky-row workload).

Workloads follow the shapes the pages benchmark: d=128, 16 heads, 4K-32K tokens
(page "AVO算法优化Transformer注意力机制性能解析", section 1 and 4.1), and d=128,
N=2048, batch 8, 16 heads with MQA and GQA (page "GPU注意力算子性能优化"
(QiMeng-Attention), section 4.1).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 21


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Outputs ``start .. start+count-1`` of the SplitMix64 stream seeded with ``seed``."""
    n = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + n * GAMMA
        return _mix64(z)


def normal_f64(seed: int, start_pair: int, n_pairs: int) -> np.ndarray:
    """2*n_pairs standard normals (float64), pairs ``start_pair ..`` of the stream."""
    x = splitmix64(seed, 2 * start_pair, 2 * n_pairs)
    u = (x >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
    u1 = u[0::2]
    u2 = u[1::2]
    r = np.sqrt(-2.0 * np.log1p(-u1))
    th = (2.0 * math.pi) * u2
    out = np.empty(2 * n_pairs, dtype=np.float64)
    out[0::2] = r * np.cos(th)
    out[1::2] = r * np.sin(th)
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> bfloat16 bit patterns (uint16), round to nearest even.

    NaN inputs are not produced by this module and are not handled specially.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 values (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _fill(out: np.ndarray, seed: int, pos: int, cnt: int, mult: float) -> None:
    # pairs cover elements [pos, pos+cnt); chunk starts are even so pairs align.
    z = normal_f64(seed, pos // 2, (cnt + 1) // 2)[:cnt]
    if mult != 1.0:
        z = z * mult
    out[pos:pos + cnt] = f32_to_bf16_bits(z.astype(np.float32))


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_bf16(seed: int, shape, mult: float = 1.0) -> np.ndarray:
    """bf16 bits of ``bf16(f32(mult * z))`` for iid standard normals z, C-order ``shape``.

    Element e is always drawn from stream outputs 2*(e//2) and 2*(e//2)+1, so the
    result does not depend on how the work is chunked or threaded.
    """
    total = int(np.prod(shape, dtype=np.int64))
    out = np.empty(total, dtype=np.uint16)
    starts = list(range(0, total, _CHUNK))
    jobs = [(p, min(_CHUNK, total - p)) for p in starts]
    if len(jobs) <= 1:
        for p, c in jobs:
            _fill(out, seed, p, c, mult)
    else:
        with ThreadPoolExecutor(max_workers=_workers()) as ex:
            list(ex.map(lambda j: _fill(out, seed, j[0], j[1], mult), jobs))
    return out.reshape(shape)


# --------------------------------------------------------------------------
# Workload catalogue.  Each workload has its own seed block; the Q, K and V
# tensors use seed_base + 0, + 1 and + 2.
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H_q: int
    H_kv: int
    N: int
    D: int = 128
    causal: bool = False
    qk_mult: float = 1.0
    seed_base: int = 0
    scale: float = field(default=float(np.float32(1.0 / math.sqrt(128.0))))

    @property
    def flops(self) -> float:
        """4*B*H_q*N^2*D, halved for causal (the counting convention of the metric)."""
        f = 4.0 * self.B * self.H_q * self.N * self.N * self.D
        return f / 2 if self.causal else f

    @property
    def pairs(self) -> int:
        """Number of allowed (query, key) pairs, exact."""
        per_head = self.N * (self.N + 1) // 2 if self.causal else self.N * self.N
        return self.B * self.H_q * per_head

    def shapes(self):
        return ((self.B, self.H_q, self.N, self.D), (self.B, self.H_kv, self.N, self.D))

    def generate(self):
        """(q, k, v) as uint16 bf16 bit arrays in [B, H, N, D] layout."""
        qs, ks = self.shapes()
        q = normal_bf16(self.seed_base + 0, qs, self.qk_mult)
        k = normal_bf16(self.seed_base + 1, ks, self.qk_mult)
        v = normal_bf16(self.seed_base + 2, ks, 1.0)
        return q, k, v


def _sweep(base: int, causal: bool):
    out = []
    tag = "causal" if causal else "noncausal"
    for i, (b, n) in enumerate(((8, 4096), (4, 8192), (2, 16384), (1, 32768))):
        out.append(Workload(f"mha_{tag}_b{b}_h16_n{n}", b, 16, 16, n, causal=causal,
                            seed_base=base + 10 * i))
    return out


WORKLOADS = {w.name: w for w in [
    # tiny MHA, the size the oracle finishes in well under a second
    Workload("mha_tiny_b1_h2_n256", 1, 2, 2, 256, seed_base=1000),
    # the pages' mid shape (d=128, N=2048, batch 8, 16 heads): GQA with 8 query
    # heads per KV head, and MQA
    Workload("gqa_b8_hq16_hkv2_n2048", 8, 16, 2, 2048, seed_base=2000),
    Workload("mqa_b8_hq16_hkv1_n2048", 8, 16, 1, 2048, seed_base=2010),
    # 32768 tokens per step split as (batch, length), 16 heads, both mask modes
    *_sweep(3000, False),
    *_sweep(4000, True),
    # causal long-context MQA with Q and K scaled x3 before rounding: peaky rows
    Workload("mqa_causal_peaky_b1_hq16_n32768", 1, 16, 1, 32768, causal=True, qk_mult=3.0,
             seed_base=5000),
]}

# The headline workload: non-causal MHA, B=2, N=16384, 16 heads, d=128.
HEADLINE = "mha_noncausal_b2_h16_n16384"


def config_of(w: Workload) -> str:
    """Label of the forward configuration a workload belongs to: C1 the tiny
    MHA case, C2 the mid-shape GQA/MQA pair, C3 and C4 the non-causal and causal
    MHA sweeps at 32768 tokens, C5 the peaky causal long-context MQA case."""
    if w.N <= 256:
        return "C1"
    if w.qk_mult != 1.0:
        return "C5"
    if w.H_kv < w.H_q:
        return "C2"
    return "C4" if w.causal else "C3"


# --------------------------------------------------------------------------
# FP8 (e4m3) inputs.  e4m3 (the OCP 8-bit format): sign, 4 exponent bits with
# bias 7, 3 mantissa bits, subnormals at exponent field 0, no infinities, codes
# 0x7F and 0xFF are NaN, largest finite value 448.  Inputs are drawn as
# normals z, divided by a per-tensor descale factor s and rounded to the nearest
# e4m3 value (ties to the even code, saturating at +-448): the tensor the codes
# stand for is s * value(code).
# --------------------------------------------------------------------------
def _e4m3_positive_values() -> np.ndarray:
    """Values of the codes 0x00 .. 0x7E (increasing)."""
    c = np.arange(127)
    e, m = c >> 3, c & 7
    return np.where(e == 0, m * 2.0 ** -9, (8.0 + m) * np.exp2(e - 10.0))


_E4M3_POS = _e4m3_positive_values()


def f64_to_e4m3(x: np.ndarray) -> np.ndarray:
    """float64 -> e4m3 codes (uint8), round to nearest with ties to the even code,
    saturating at +-448.  NaN inputs are not produced by this module."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 126)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)


def _fill_e4m3(out: np.ndarray, seed: int, pos: int, cnt: int, inv_descale: float) -> None:
    z = normal_f64(seed, pos // 2, (cnt + 1) // 2)[:cnt]
    out[pos:pos + cnt] = f64_to_e4m3(z * inv_descale)


def normal_e4m3(seed: int, shape, descale: float) -> np.ndarray:
    """e4m3 codes of ``z / descale`` for iid standard normals z, C-order ``shape``
    (same element-to-stream rule as ``normal_bf16``)."""
    total = int(np.prod(shape, dtype=np.int64))
    out = np.empty(total, dtype=np.uint8)
    inv = 1.0 / float(descale)
    jobs = [(p, min(_CHUNK, total - p)) for p in range(0, total, _CHUNK)]
    if len(jobs) <= 1:
        for p, c in jobs:
            _fill_e4m3(out, seed, p, c, inv)
    else:
        with ThreadPoolExecutor(max_workers=_workers()) as ex:
            list(ex.map(lambda j: _fill_e4m3(out, seed, j[0], j[1], inv), jobs))
    return out.reshape(shape)


# Descale of the FP8 workloads: unit normals up to |z| = 6 map onto the full
# e4m3 range (per-tensor amax scaling with amax taken as 6).
FP8_DESCALE = float(np.float32(6.0 / 448.0))


@dataclass(frozen=True)
class Fp8Workload:
    name: str
    B: int
    H_q: int
    H_kv: int
    N: int
    D: int = 128
    causal: bool = False
    seed_base: int = 0
    scale: float = field(default=float(np.float32(1.0 / math.sqrt(128.0))))
    descale_q: float = FP8_DESCALE
    descale_k: float = FP8_DESCALE
    descale_v: float = FP8_DESCALE

    @property
    def flops(self) -> float:
        f = 4.0 * self.B * self.H_q * self.N * self.N * self.D
        return f / 2 if self.causal else f

    def shapes(self):
        return ((self.B, self.H_q, self.N, self.D), (self.B, self.H_kv, self.N, self.D))

    def generate(self):
        """(q8, k8, v8) as uint8 e4m3 codes in [B, H, N, D] layout."""
        qs, ks = self.shapes()
        return (normal_e4m3(self.seed_base + 0, qs, self.descale_q),
                normal_e4m3(self.seed_base + 1, ks, self.descale_k),
                normal_e4m3(self.seed_base + 2, ks, self.descale_v))


FP8_WORKLOADS = {w.name: w for w in [
    Fp8Workload("fp8_mha_tiny_b1_h2_n256", 1, 2, 2, 256, seed_base=8000),
    Fp8Workload("fp8_gqa_b8_hq16_hkv2_n2048", 8, 16, 2, 2048, seed_base=8010),
    Fp8Workload("fp8_mha_noncausal_b2_h16_n16384", 2, 16, 16, 16384, seed_base=8020),
    Fp8Workload("fp8_mha_causal_b2_h16_n16384", 2, 16, 16, 16384, causal=True, seed_base=8030),
]}

# The FP8 counterpart of the headline workload (non-causal MHA, B=2, N=16384).
FP8_HEADLINE = "fp8_mha_noncausal_b2_h16_n16384"


# --------------------------------------------------------------------------
# Block-sparse masks: per (mask head, query block) lists of key blocks, in
# block-compressed-row form (kb_ptr offsets, kb_idx indices).
# --------------------------------------------------------------------------
def lists_to_csr(lists):
    """[[key blocks of list 0], [.. of list 1], ...] -> (kb_ptr, kb_idx) int32."""
    ptr = np.zeros(len(lists) + 1, np.int32)
    ptr[1:] = np.cumsum([len(x) for x in lists], dtype=np.int64)
    idx = np.array([j for x in lists for j in x], np.int32)
    return ptr, idx


def sparse_pattern(seed: int, n_blocks: int, mask_heads: int, local: int, n_global: int,
                   n_random: int, causal: bool):
    """Lists of key blocks for each (mask head, query block): the `local` blocks
    ending at the diagonal block, the first `n_global` blocks, and `n_random`
    seeded random blocks (at or below the diagonal when causal), sorted, unique."""
    rng = np.random.default_rng(seed)
    lists = []
    for _ in range(mask_heads):
        for qb in range(n_blocks):
            hi = qb if causal else n_blocks - 1
            s = set(range(max(0, qb - local + 1), qb + 1)) if local > 0 else set()
            s |= set(range(min(n_global, hi + 1)))
            if n_random > 0 and hi >= 0:
                s |= set(rng.integers(0, hi + 1, n_random).tolist())
            lists.append(sorted(s))
    return lists


@dataclass(frozen=True)
class SparseWorkload:
    """Block-sparse forward: 128 x 128 blocks, local + global + random pattern."""
    name: str
    B: int
    H_q: int
    H_kv: int
    N: int
    local: int
    n_global: int
    n_random: int
    causal: bool = False
    per_head: bool = False
    D: int = 128
    block: int = 128
    seed_base: int = 0
    scale: float = field(default=float(np.float32(1.0 / math.sqrt(128.0))))

    def lists(self):
        nb = -(-self.N // self.block)
        return sparse_pattern(self.seed_base + 7, nb, self.H_q if self.per_head else 1, self.local,
                              self.n_global, self.n_random, self.causal)

    def csr(self):
        return lists_to_csr(self.lists())

    def pairs(self) -> int:
        """Allowed (query, key) pairs, exact."""
        nb = -(-self.N // self.block)
        lists = self.lists()
        total = 0
        for h in range(self.H_q):
            for qb in range(nb):
                ls = lists[(h if self.per_head else 0) * nb + qb]
                q0, q1 = qb * self.block, min(self.N, (qb + 1) * self.block)
                for kb in ls:
                    k0, k1 = kb * self.block, min(self.N, (kb + 1) * self.block)
                    if not self.causal or k1 <= q0:
                        total += (q1 - q0) * (k1 - k0)
                    else:   # pairs j <= i within the two ranges
                        for i in range(q0, q1):
                            total += max(0, min(k1, i + 1) - k0)
        return self.B * total

    @property
    def flops(self) -> float:
        """4*D per allowed (row, key) pair."""
        return 4.0 * self.D * self.pairs()

    def generate(self):
        qs = (self.B, self.H_q, self.N, self.D)
        ks = (self.B, self.H_kv, self.N, self.D)
        return (normal_bf16(self.seed_base + 0, qs), normal_bf16(self.seed_base + 1, ks),
                normal_bf16(self.seed_base + 2, ks))


SPARSE_WORKLOADS = {w.name: w for w in [
    # local window of 4 blocks + 1 global block + 2 random blocks per query block
    SparseWorkload("bsparse_local4_global1_rand2_b2_h16_n16384", 2, 16, 16, 16384, 4, 1, 2,
                   seed_base=9000),
    SparseWorkload("bsparse_causal_local8_global2_b2_h16_n16384", 2, 16, 16, 16384, 8, 2, 2,
                   causal=True, seed_base=9010),
    SparseWorkload("bsparse_perhead_gqa_hq16_hkv2_n8192", 1, 16, 2, 8192, 3, 1, 3, per_head=True,
                   seed_base=9020),
]}


# --------------------------------------------------------------------------
# Decode workloads: M new query rows per (batch, query head) against a cache
# of L keys and values (the last M positions of the sequence).  Same seeding
# rule: Q, K, V use seed_base + 0, + 1, + 2.
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    H_q: int
    H_kv: int
    M: int
    L: int
    D: int = 128
    causal: bool = False
    seed_base: int = 0
    scale: float = field(default=float(np.float32(1.0 / math.sqrt(128.0))))

    @property
    def pairs(self) -> int:
        """Allowed (query row, key) pairs."""
        per_head = self.M * self.L - (self.M * (self.M - 1) // 2 if self.causal else 0)
        return self.B * self.H_q * per_head

    @property
    def flops(self) -> float:
        return 4.0 * self.D * self.pairs

    @property
    def bytes(self) -> int:
        """Algorithmic HBM bytes: K and V read once, Q read once, O written once
        (bf16) and LSE written once (fp32)."""
        kv = 2 * self.B * self.H_kv * self.L * self.D * 2
        qo = 2 * self.B * self.H_q * self.M * self.D * 2
        return kv + qo + self.B * self.H_q * self.M * 4

    def shapes(self):
        return ((self.B, self.H_q, self.M, self.D), (self.B, self.H_kv, self.L, self.D))

    def generate(self):
        """(q, k, v) as uint16 bf16 bit arrays: q [B, H_q, M, D], k, v [B, H_kv, L, D]."""
        qs, ks = self.shapes()
        return (normal_bf16(self.seed_base + 0, qs), normal_bf16(self.seed_base + 1, ks),
                normal_bf16(self.seed_base + 2, ks))


DECODE_WORKLOADS = {w.name: w for w in [
    # one new token, the pages' GQA head shape (16 query heads, 8 per K/V head),
    # batch 8, a 32K-token cache: 256 MiB of K/V per step
    DecodeWorkload("decode_gqa_b8_hq16_hkv2_m1_l32768", 8, 16, 2, 1, 32768, seed_base=6000),
    # four new tokens (causal among themselves), same shape
    DecodeWorkload("decode_gqa_b8_hq16_hkv2_m4_l32768", 8, 16, 2, 4, 32768, causal=True,
                   seed_base=6010),
    # MHA decode, batch 8, 8K cache: 512 MiB of K/V
    DecodeWorkload("decode_mha_b8_h16_m1_l8192", 8, 16, 16, 1, 8192, seed_base=6020),
    # MQA, one sequence, 32K cache
    DecodeWorkload("decode_mqa_b1_hq16_hkv1_m1_l32768", 1, 16, 1, 1, 32768, seed_base=6030),
]}

DECODE_HEADLINE = "decode_gqa_b8_hq16_hkv2_m1_l32768"


# --------------------------------------------------------------------------
# Packed variable-length batches: sequences concatenated along the token axis
# (q [H_q, total, D], k, v [H_kv, total, D]) with an optional sliding window.
# Lengths come from the same counter-based generator (seed_base + 3), so the
# batch is reproducible.  Q, K, V use seed_base + 0, + 1, + 2.
# --------------------------------------------------------------------------
def _seq_lengths(seed: int, total: int, lo: int, hi: int) -> np.ndarray:
    """Lengths in [lo, hi] summing exactly to ``total``, drawn from uniforms
    derived from the generator's bf16 normals (|z| mapped through exp)."""
    z = bf16_bits_to_f32(normal_bf16(seed, (4096,))).astype(np.float64)
    u = 1.0 - np.exp(-np.abs(z))          # in [0, 1), deterministic
    out, acc, t = [], 0, 0
    while acc < total:
        n = int(lo + u[t % u.size] * (hi - lo + 1))
        n = min(max(n, lo), hi, total - acc)
        out.append(n)
        acc += n
        t += 1
    return np.array(out, dtype=np.int32)


@dataclass(frozen=True)
class VarlenWorkload:
    name: str
    H_q: int
    H_kv: int
    total: int
    min_len: int
    max_len: int
    causal: bool = True
    left: int = -1
    right: int = -1
    D: int = 128
    seed_base: int = 0
    scale: float = field(default=float(np.float32(1.0 / math.sqrt(128.0))))

    def lengths(self) -> np.ndarray:
        return _seq_lengths(self.seed_base + 3, self.total, self.min_len, self.max_len)

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths())]).astype(np.int32)

    @property
    def pairs(self) -> int:
        """Allowed (row, key) pairs of one head, times H_q."""
        tot = 0
        for n in self.lengths().tolist():
            i = np.arange(n, dtype=np.int64)
            lo = np.maximum(0, i - self.left) if self.left >= 0 else np.zeros(n, np.int64)
            hi = np.full(n, n - 1, np.int64)
            if self.causal:
                hi = np.minimum(hi, i)
            if self.right >= 0:
                hi = np.minimum(hi, i + self.right)
            tot += int(np.maximum(hi - lo + 1, 0).sum())
        return tot * self.H_q

    @property
    def flops(self) -> float:
        return 4.0 * self.D * self.pairs

    def generate(self):
        """(q, k, v) as uint16 bf16 bits: q [H_q, total, D], k, v [H_kv, total, D]."""
        qs, ks = (self.H_q, self.total, self.D), (self.H_kv, self.total, self.D)
        return (normal_bf16(self.seed_base + 0, qs), normal_bf16(self.seed_base + 1, ks),
                normal_bf16(self.seed_base + 2, ks))


VARLEN_WORKLOADS = {w.name: w for w in [
    # 32768 tokens in sequences of 512..8192 tokens, 16 heads, causal
    VarlenWorkload("varlen_causal_h16_t32768", 16, 16, 32768, 512, 8192, seed_base=7000),
    # same tokens, GQA (8 query heads per K/V head), causal with a 4096-token window
    VarlenWorkload("varlen_swa4096_gqa_hq16_hkv2_t32768", 16, 2, 32768, 512, 16384, left=4096,
                   seed_base=7010),
    # one 32768-token sequence, 16 heads, a symmetric local window of 1024 tokens
    VarlenWorkload("local1024_h16_t32768", 16, 16, 32768, 32768, 32768, causal=False, left=1024,
                   right=1024, seed_base=7020),
    # eight sequences of exactly 4096 tokens, 16 heads, causal: the packed form of
    # dense causal B = 8, N = 4096
    VarlenWorkload("varlen_causal_equal_h16_8x4096", 16, 16, 32768, 4096, 4096, seed_base=7030),
]}
