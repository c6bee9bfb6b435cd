"""The synthetic attention workloads: shapes, scales, masking and seeds.

Shapes follow the pages' problem statement (Learning FlashAttention the Hard
Way, Part 2, workload definitions: SDPA_L = [1,4,128,64] for listings and
SDPA_P = [1,8,4096,64] for timing, fp16 Q/K/V in [B,H,S,D] from randn, default
scale 1/sqrt(D)), widened with a long-sequence case, two causal cases at
head_dim 128, and one with Q and K drawn three times wider so the softmax is
peaked and the running max moves often. A sweep over sequence lengths 4k, 8k
and 16k (batch 1, 8 heads, head_dim 64, with and without the causal mask)
follows the sequence lengths at which "Three kernels for a chip the ecosystem
skipped" (Kernel one: FlashAttention-2) reports its attention throughput.

Q, K and V use generator streams 0, 1 and 2 under the workload's seed.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .gen import normal_f16

STREAM_Q, STREAM_K, STREAM_V = 0, 1, 2
SEED_BASE = 0xA77E0000


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S: int
    D: int
    causal: bool
    seed: int
    qk_mult: float = 1.0  # Q and K are fp16(qk_mult * N(0,1))
    v_mult: float = 1.0

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(D), rounded to fp32 (both sides use this value)."""
        return float(np.float32(1.0 / np.sqrt(self.D)))

    @property
    def shape(self):
        return (self.B, self.H, self.S, self.D)

    @property
    def flops(self) -> float:
        """4*B*H*S^2*D, halved when causal (the pages' FLOP convention)."""
        f = 4.0 * self.B * self.H * self.S * self.S * self.D
        return f / 2 if self.causal else f

    @property
    def algorithmic_bytes(self) -> int:
        """Q, K, V and O in fp16 plus LSE in fp32, each moved once."""
        n = self.B * self.H * self.S * self.D
        return 4 * n * 2 + self.B * self.H * self.S * 4

    def describe(self) -> str:
        m = "causal" if self.causal else "non-causal"
        return f"B{self.B} H{self.H} S{self.S} D{self.D} fp16 {m}"


WORKLOADS = {
    "listing_b1h4s128d64": Workload("listing_b1h4s128d64", 1, 4, 128, 64, False, SEED_BASE + 1),
    "sdpa_b1h8s4096d64": Workload("sdpa_b1h8s4096d64", 1, 8, 4096, 64, False, SEED_BASE + 2),
    "long_b1h8s16384d64": Workload("long_b1h8s16384d64", 1, 8, 16384, 64, False, SEED_BASE + 3),
    "causal_b2h16s8192d128": Workload("causal_b2h16s8192d128", 2, 16, 8192, 128, True, SEED_BASE + 4),
    "peaked_causal_b4h32s4096d128": Workload(
        "peaked_causal_b4h32s4096d128", 4, 32, 4096, 128, True, SEED_BASE + 5, qk_mult=3.0),
    "sweep_b1h8s8192d64": Workload("sweep_b1h8s8192d64", 1, 8, 8192, 64, False, SEED_BASE + 6),
    "sweep_causal_b1h8s4096d64": Workload(
        "sweep_causal_b1h8s4096d64", 1, 8, 4096, 64, True, SEED_BASE + 7),
    "sweep_causal_b1h8s8192d64": Workload(
        "sweep_causal_b1h8s8192d64", 1, 8, 8192, 64, True, SEED_BASE + 8),
    "sweep_causal_b1h8s16384d64": Workload(
        "sweep_causal_b1h8s16384d64", 1, 8, 16384, 64, True, SEED_BASE + 9),
    # One head: 128 query tiles leave half of 256 CUs idle in a single pass.
    "single_head_b1h1s16384d64": Workload(
        "single_head_b1h1s16384d64", 1, 1, 16384, 64, False, SEED_BASE + 10),
}

# Workloads on which the split-KV path is timed against the single pass.
SPLITKV_BENCH = ("single_head_b1h1s16384d64", "sweep_causal_b1h8s4096d64")

HEADLINE = "sdpa_b1h8s4096d64"

# The five problem configurations: the tiny listing case, the headline, the
# long sequence, causal D = 128, and causal D = 128 with peaked scores.
CONFIGS = ("listing_b1h4s128d64", "sdpa_b1h8s4096d64", "long_b1h8s16384d64",
           "causal_b2h16s8192d128", "peaked_causal_b4h32s4096d128")

# Sequence-length sweep at batch 1, 8 heads, head_dim 64: (S, causal) -> name.
SWEEP = {
    (4096, False): "sdpa_b1h8s4096d64",
    (8192, False): "sweep_b1h8s8192d64",
    (16384, False): "long_b1h8s16384d64",
    (4096, True): "sweep_causal_b1h8s4096d64",
    (8192, True): "sweep_causal_b1h8s8192d64",
    (16384, True): "sweep_causal_b1h8s16384d64",
}


def make_qkv(B: int, H: int, S: int, D: int, seed: int,
             qk_mult: float = 1.0, v_mult: float = 1.0):
    """fp16 numpy Q, K, V of shape [B,H,S,D] from streams 0, 1, 2 of ``seed``."""
    shape = (B, H, S, D)
    q = normal_f16(seed, STREAM_Q, shape, qk_mult)
    k = normal_f16(seed, STREAM_K, shape, qk_mult)
    v = normal_f16(seed, STREAM_V, shape, v_mult)
    return q, k, v


def workload_inputs(w: Workload):
    return make_qkv(w.B, w.H, w.S, w.D, w.seed, w.qk_mult, w.v_mult)


@dataclass(frozen=True)
class CacheWorkload:
    """S_q queries per head against an S_k-key cache (the queries are the
    last S_q positions). Q uses stream 0 of ``seed``, K and V streams 1 and 2
    of ``seed + 1``."""
    name: str
    B: int
    H: int
    Sq: int
    Sk: int
    D: int
    causal: bool
    seed: int

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.D)))

    @property
    def algorithmic_bytes(self) -> int:
        """K and V read once, Q read and O written once (fp16), LSE (fp32)."""
        bh = self.B * self.H
        return 2 * bh * self.Sk * self.D * 2 + 2 * bh * self.Sq * self.D * 2 + bh * self.Sq * 4

    @property
    def flops(self) -> float:
        """4 * D per visible (query, key) pair."""
        off = self.Sk - self.Sq
        if self.causal:
            vis = sum(min(self.Sk, off + i + 1) for i in range(self.Sq))
        else:
            vis = self.Sq * self.Sk
        return 4.0 * self.B * self.H * self.D * vis

    def describe(self) -> str:
        m = "causal" if self.causal else "non-causal"
        return f"B{self.B} H{self.H} S_q{self.Sq} S_k{self.Sk} D{self.D} fp16 {m}"


def cache_inputs(w: CacheWorkload):
    q = normal_f16(w.seed, STREAM_Q, (w.B, w.H, w.Sq, w.D))
    k = normal_f16(w.seed + 1, STREAM_K, (w.B, w.H, w.Sk, w.D))
    v = normal_f16(w.seed + 1, STREAM_V, (w.B, w.H, w.Sk, w.D))
    return q, k, v


# Decoding against a key/value cache (the Emmy comments page closes on it): one
# new token for 8 sequences x 32 heads over an 8k-token cache at D = 128, and
# 16 new tokens of one sequence x 8 heads over a 128k-token cache at D = 64.
DECODE = {
    "decode_b8h32q1k8192d128": CacheWorkload("decode_b8h32q1k8192d128", 8, 32, 1, 8192, 128,
                                             True, SEED_BASE + 20),
    "decode_b1h8q16k131072d64": CacheWorkload("decode_b1h8q16k131072d64", 1, 8, 16, 131072, 64,
                                              True, SEED_BASE + 22),
}
