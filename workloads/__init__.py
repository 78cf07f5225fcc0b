"""Seeded synthetic inputs for the MoE dispatch + combine step.

Shared by the tests, the benchmark and the smoke check. Holds no part of the
method's arithmetic: it draws tokens, routings, weights and expert outputs,
and nothing else. Which expert-output rows are filled is passed in by the
caller (the tests take it from the oracle).

Workloads (sizes and distributions of the step on a decode micro-batch):

  tiny        N=128,  h=1024, E=8,   K=2, bf16, uniform distinct experts
  decode      N=128,  h=7168, E=256, K=8, bf16, uniform distinct experts
  decode_fp8  as decode, dispatch payload fp8 e4m3 + fp32 scale per 128
  wide_zipf   N=512,  h=4096, E=64,  K=6, bf16, Zipf(s=1.2) over experts
  worst_fill  N=1024, h=7168, E=256, K=8, bf16, half the tokens on a fixed
              hot set of 8 experts, the rest uniform distinct

Recipe: tokens are N(0,1) fp32 samples rounded to bf16 (nearest even);
weights are a softmax of N(0,1) logits over the K picks, computed in fp64 and
rounded to fp32; expert outputs are N(0,1) rounded to bf16 on filled rows and
the bf16 quiet NaN 0x7FC0 elsewhere. Seed 0 by default, with one independent
stream per input kind (numpy SeedSequence.spawn).
"""
from dataclasses import dataclass, replace

import numpy as np

BF16 = 0
FP8_E4M3 = 1
BF16_QNAN = 0x7FC0


@dataclass(frozen=True)
class Workload:
    name: str
    num_tokens: int
    hidden: int
    num_experts: int
    topk: int
    dtype: int
    routing: str          # "uniform" | "zipf" | "hotset"
    max_tokens: int = 0   # layout capacity; 0 means = num_tokens
    zipf_s: float = 1.2
    hot_experts: int = 8
    seed: int = 0

    @property
    def capacity(self) -> int:
        return self.max_tokens if self.max_tokens else self.num_tokens

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 128, 1024, 8, 2, BF16, "uniform"),
    "decode": Workload("decode", 128, 7168, 256, 8, BF16, "uniform"),
    "decode_fp8": Workload("decode_fp8", 128, 7168, 256, 8, FP8_E4M3, "uniform"),
    "wide_zipf": Workload("wide_zipf", 512, 4096, 64, 6, BF16, "zipf"),
    "worst_fill": Workload("worst_fill", 1024, 7168, 256, 8, BF16, "hotset"),
}


def _streams(w: Workload):
    ss = np.random.SeedSequence(w.seed)
    kids = ss.spawn(4)
    return [np.random.Generator(np.random.PCG64(k)) for k in kids]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def tokens(w: Workload) -> np.ndarray:
    """bf16 bits [N, h]."""
    rng = _streams(w)[0]
    return f32_to_bf16_bits(rng.standard_normal((w.num_tokens, w.hidden), dtype=np.float32))


def routing(w: Workload) -> np.ndarray:
    """int32 [N, K] expert ids, K distinct per token."""
    rng = _streams(w)[1]
    n, e, k = w.num_tokens, w.num_experts, w.topk
    if w.routing == "uniform":
        keys = rng.random((n, e))
        idx = np.argsort(keys, axis=1, kind="stable")[:, :k]
    elif w.routing == "zipf":
        # expert r-1 has weight r^-s; K distinct draws without replacement,
        # taken as Gumbel-top-k on log-weights (the order of sequential draws)
        logp = -w.zipf_s * np.log(np.arange(1, e + 1, dtype=np.float64))
        g = rng.gumbel(size=(n, e))
        idx = np.argsort(-(logp[None, :] + g), axis=1, kind="stable")[:, :k]
    elif w.routing == "hotset":
        hot = rng.permutation(e)[: w.hot_experts]
        assert k <= w.hot_experts
        hot_tokens = rng.permutation(n)[: n // 2]
        keys = rng.random((n, e))
        idx = np.argsort(keys, axis=1, kind="stable")[:, :k]
        for t in hot_tokens:
            idx[t] = rng.permutation(hot)[:k]
    else:
        raise ValueError(w.routing)
    return np.ascontiguousarray(idx.astype(np.int32))


def weights(w: Workload) -> np.ndarray:
    """fp32 [N, K]: softmax of N(0,1) logits over the K picks (fp64, rounded)."""
    rng = _streams(w)[2]
    logits = rng.standard_normal((w.num_tokens, w.topk))
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    return np.ascontiguousarray((z / z.sum(axis=1, keepdims=True)).astype(np.float32))


def expert_outputs(w: Workload, filled_rows=None) -> np.ndarray:
    """bf16 bits [E * capacity, h] in receive-slot order.

    `filled_rows` is a boolean mask over the E * capacity rows; rows it marks
    get N(0,1) values, the others the bf16 NaN poison. None fills every row.
    """
    rng = _streams(w)[3]
    rows = w.num_experts * w.capacity
    if filled_rows is None:
        return f32_to_bf16_bits(rng.standard_normal((rows, w.hidden), dtype=np.float32))
    filled_rows = np.asarray(filled_rows, dtype=bool)
    assert filled_rows.shape == (rows,)
    y = np.full((rows, w.hidden), BF16_QNAN, dtype=np.uint16)
    nf = int(filled_rows.sum())
    y[filled_rows] = f32_to_bf16_bits(rng.standard_normal((nf, w.hidden), dtype=np.float32))
    return y
