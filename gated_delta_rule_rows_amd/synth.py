"""Seeded synthetic inputs for the KDA verify-row scan workloads.

This module draws inputs only; it holds none of the scan's arithmetic.  The
HIP path and the CPU oracle both consume what it returns.

Recipe (every workload):
  * q, k ~ N(0, 1) per element, then L2-normalised over the 128 key channels
    of each (layer, row, head), in f64, then rounded to f32;
  * v ~ N(0, 1), rounded to f32;
  * g ~ U(-5, 0) per key channel (a log-decay), rounded to f32;
  * beta = sigmoid(N(0, 1)) per (layer, row, head), in f64, rounded to f32;
  * bf16 workloads round those f32 values to bf16 (round to nearest even).

Draw order inside one call: q, k, v, g, beta, each a C-order block of its full
shape.  One call is keyed by (seed, stream, index): numpy's PCG64 seeded from
``SeedSequence([seed, stream, index])``, so a test can regenerate any single
round or step without drawing the ones before it.

Greedy-accept inputs: logits ~ N(0, 3^2) per (row, vocabulary entry), f32,
with one planted token per row raised to 64.0 (far above every normal draw,
so it is the row's unique maximum), and draft tokens equal to the planted
tokens of the rows before them, except for a planted mismatch at the
accepted-draft count j.  Vocabulary size 150,000 mirrors the pages' head
(about 600k floats over the four rows of a K = 3 round).

Pre-scan row-op inputs (the projections ahead of the scan): raw q/k/v
projections x ~ N(0, 1) over 3 * H * 128 channels, gate pre-activations
a ~ N(0, 2^2) (so about 2% of channels reach the -5 bound), beta
pre-activations b ~ N(0, 1) (beta = sigmoid(N(0, 1)), as above), conv taps
~ U(-0.5, 0.5) and conv-ring rows ~ N(0, 1), all f32.

Streams: 0 = verify rows, 1 = accept draws, 2 = warm-up rows, 3 = logits,
4 = row-op inputs.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

D = 128
T_MAX = 15
B_MAX = 15
GATE_LO = -5.0

STREAM_ROWS = 0
STREAM_ACCEPT = 1
STREAM_WARMUP = 2
STREAM_LOGITS = 3
STREAM_ROW_OPS = 4
VOCAB = 150_000
PLANTED_LOGIT = 64.0


def _rng(seed: int, stream: int, index: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(stream), int(index)]))


def _unit_rows(rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.standard_normal(shape)
    x /= np.linalg.norm(x, axis=-1, keepdims=True)
    return x.astype(np.float32)


def rows(seed: int, index: int, L: int, T: int, H: int, d: int = D,
         stream: int = STREAM_ROWS) -> dict:
    """Row inputs of one round (or step): q,k,v,g [L][T][H][d], beta [L][T][H], f32."""
    rng = _rng(seed, stream, index)
    shape = (L, T, H, d)
    q = _unit_rows(rng, shape)
    k = _unit_rows(rng, shape)
    v = rng.standard_normal(shape).astype(np.float32)
    g = rng.uniform(GATE_LO, 0.0, shape).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((L, T, H))))).astype(np.float32)
    return {"q": q, "k": k, "v": v, "g": g, "beta": beta}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round f32 to bf16 (nearest even); return the 16-bit patterns as uint16."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def rows_bf16(seed: int, index: int, L: int, T: int, H: int, d: int = D) -> dict:
    """Same draws as rows(), rounded to bf16; arrays hold uint16 bit patterns."""
    r = rows(seed, index, L, T, H, d)
    return {name: to_bf16_bits(a) for name, a in r.items()}


def accepts(seed: int, n: int, K: int) -> np.ndarray:
    """n accept counts j ~ U{0..K} (accepted drafts per round)."""
    return _rng(seed, STREAM_ACCEPT, 0).integers(0, K + 1, size=n)


def serving_ks(seed: int, n: int, choices=(1, 3, 5, 7, 14)) -> np.ndarray:
    """Per-round draft counts K drawn uniformly from `choices`."""
    rng = _rng(seed, STREAM_ACCEPT, 1)
    return np.asarray(choices)[rng.integers(0, len(choices), size=n)]


def accept_round(seed: int, index: int, t: int, V: int, j: int):
    """One greedy-accept round: (logits [t][V] f32, drafts [t-1] uint32, planted [t] uint32).

    Row r's planted token is its unique maximum; drafts[r] = planted[r] for
    r < j and drafts[j] != planted[j] (when j < t - 1), so exactly j drafts
    are accepted and the bonus token is planted[j].
    """
    if not (1 <= t and 1 <= V and 0 <= j <= t - 1):
        raise ValueError("need t >= 1, V >= 1, 0 <= j <= t - 1")
    rng = _rng(seed, STREAM_LOGITS, index)
    logits = (rng.standard_normal((t, V)) * 3.0).astype(np.float32)
    planted = rng.integers(0, V, size=t).astype(np.uint32)
    logits[np.arange(t), planted] = PLANTED_LOGIT
    drafts = planted[: t - 1].copy()
    if j < t - 1:
        drafts[j] = (planted[j] + 1 + rng.integers(0, max(V - 1, 1))) % max(V, 2)
        if V == 1:
            drafts[j] = 1   # the only token is 0, so any other id misses
    return logits, drafts, planted


def row_op_inputs(seed: int, index: int, L: int, T: int, H: int, d: int = D) -> dict:
    """Projections for one round of row ops: x [L][T][3*H*d], a [L][T][H*d],
    b [L][T][H], w [L][3*H*d][4], ring [L][3][3*H*d], all f32.  Draw order:
    x, a, b, w, ring."""
    rng = _rng(seed, STREAM_ROW_OPS, index)
    C = 3 * H * d
    x = rng.standard_normal((L, T, C)).astype(np.float32)
    a = (rng.standard_normal((L, T, H * d)) * 2.0).astype(np.float32)
    b = rng.standard_normal((L, T, H)).astype(np.float32)
    w = rng.uniform(-0.5, 0.5, (L, C, 4)).astype(np.float32)
    ring = rng.standard_normal((L, 3, C)).astype(np.float32)
    return {"x": x, "a": a, "b": b, "w": w, "ring": ring}


def warmup_rows(seed: int, n_rows: int, L: int, H: int, d: int = D) -> dict:
    """n_rows warm-up rows, drawn like verify rows, on their own stream."""
    return rows(seed, 0, L, n_rows, H, d, stream=STREAM_WARMUP)


@dataclass(frozen=True)
class Workload:
    name: str
    L: int
    H: int
    T: int          # verify rows per round (K + 1); 1 for the batched arm
    rounds: int     # rounds, or steps for the batched arm
    seed: int
    B: int = 0      # sessions (batched arm only)
    warmup_rows: int = 0
    bf16: bool = False
    note: str = ""


# The five synthetic workloads the scan is built and measured on.
WORKLOADS = {
    "tiny": Workload("tiny", L=1, H=1, T=8, rounds=4, seed=0,
                     note="zero state, 4 rounds of T=8 (K=7), j~U{0..7}, replay every round"),
    "one_layer": Workload("one_layer", L=1, H=64, T=8, rounds=1, seed=1, warmup_rows=256,
                          note="64x128x128 state warmed by 256 rows; replay sweep j=0..7"),
    "verify_k14": Workload("verify_k14", L=34, H=64, T=15, rounds=32, seed=2,
                           note="34 layers x 64 heads, T=15 (K=14), j~U{0..14}"),
    "batched_b15": Workload("batched_b15", L=34, H=64, T=1, rounds=64, seed=3, B=15,
                            note="15 sessions x 34 layers x 64 heads, one row each per step"),
    "serving_mix_bf16": Workload("serving_mix_bf16", L=34, H=64, T=15, rounds=256, seed=4,
                                 bf16=True,
                                 note="bf16 rows, f32 state, K per round from {1,3,5,7,14}"),
}
