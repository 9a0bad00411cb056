"""Seeded synthetic workloads for the balanced expert-parallel plan.

This module only draws inputs: router ids and weights, hidden rows, expert weight
blocks and gradients. It holds none of the method's arithmetic (no histogram, no
plan, no copy, no combine, no reduce), so both the HIP path and the CPU oracle
may take their inputs from it.

The five workloads follow the shapes the MoonEP write-ups give: E = 896 experts
with 16 active per token for Kimi K3 ("Verso l'ottimizzazione dei modelli
multimodali giganti", alextech.ai page), and B = E/R for training and 3-4 for
inference ("Key facts about the release", news.hamidun.com EN page). Routing is
skewed on purpose, since skew is what the method removes ("Why expert
parallelism is needed", same page).

Router ids are top-K of (logits + per-expert bias); the k order of a token's
ids is descending score. Combine weights are the softmax over the K selected
scores (renormalised top-K). Dense tensors are drawn with torch's seeded
generator on the device they are needed on; ids and weights are drawn with
numpy on the host, because the oracle needs them there.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, Tuple

import numpy as np

F32 = 0
BF16 = 1
_DT_BYTES = {F32: 4, BF16: 2}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    R: int              # virtual expert-parallel ranks
    E: int              # experts
    K: int              # experts per token
    S: int              # tokens per rank
    H: int              # hidden size
    dtype: int          # element type of hidden rows: F32 or BF16
    B: int              # duplicate-expert slots per rank
    block_shape: Tuple[int, ...]   # one expert's weight block
    block_dtype: int    # F32 or BF16
    routing: str        # "bias", "uniform" or "zipf"
    bias_std: float = 1.0
    zipf_s: float = 1.2
    weight_std: float = 0.02

    @property
    def G(self) -> int:
        return self.E // self.R

    @property
    def SK(self) -> int:
        return self.S * self.K

    @property
    def n_tok(self) -> int:
        return self.R * self.S

    @property
    def n_ent(self) -> int:
        return self.R * self.S * self.K

    @property
    def row_bytes(self) -> int:
        return self.H * _DT_BYTES[self.dtype]

    @property
    def block_elems(self) -> int:
        return int(np.prod(self.block_shape))

    @property
    def block_bytes(self) -> int:
        return self.block_elems * _DT_BYTES[self.block_dtype]

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    # R=4, E=16, K=2, S=64, H=128 fp32, B=4; weights [16,128,256] fp32 N(0,0.02)
    "tiny": Workload("tiny", R=4, E=16, K=2, S=64, H=128, dtype=F32, B=4,
                     block_shape=(128, 256), block_dtype=F32,
                     routing="bias", bias_std=1.0),
    # R=8, E=64, K=8, S=4096, H=2048 bf16, B=8; uniform top-8 without replacement.
    # No weight block is given for this workload; 3x2048x1024 bf16 is used.
    "uniform": Workload("uniform", R=8, E=64, K=8, S=4096, H=2048, dtype=BF16, B=8,
                        block_shape=(3, 2048, 1024), block_dtype=BF16,
                        routing="uniform"),
    # R=16, E=256, K=8, S=8192, H=4096 bf16, B=16; popularity ~ rank^-1.2
    "zipf": Workload("zipf", R=16, E=256, K=8, S=8192, H=4096, dtype=BF16, B=16,
                     block_shape=(3, 4096, 1024), block_dtype=BF16,
                     routing="zipf", zipf_s=1.2),
    # Kimi-K3-shaped training layer: E=896, K=16, R=32, S=4096, H=7168 bf16, B=28
    "k3": Workload("k3", R=32, E=896, K=16, S=4096, H=7168, dtype=BF16, B=28,
                   block_shape=(3, 7168, 512), block_dtype=BF16,
                   routing="bias", bias_std=1.5),
    # Inference decode: E=896, K=16, R=64, S=128, H=7168 bf16, B=4.
    # The K3 model's weight block is used for its duplicates.
    "decode": Workload("decode", R=64, E=896, K=16, S=128, H=7168, dtype=BF16, B=4,
                       block_shape=(3, 7168, 512), block_dtype=BF16,
                       routing="bias", bias_std=0.75),
}

_CHUNK_TOK = 8192


def _softmax_rows(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float64)
    x = x - x.max(axis=1, keepdims=True)
    ex = np.exp(x)
    return (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)


def _topk_desc(scores: np.ndarray, K: int) -> np.ndarray:
    """Indices of the K largest scores of each row, highest first (ties: lower index)."""
    n, E = scores.shape
    if K < E:
        part = np.argpartition(-scores, K - 1, axis=1)[:, :K]
        part.sort(axis=1)  # index order, so the stable sort below breaks ties by index
    else:
        part = np.broadcast_to(np.arange(E), (n, E)).copy()
    sel = np.take_along_axis(scores, part, axis=1)
    order = np.argsort(-sel, axis=1, kind="stable")
    return np.take_along_axis(part, order, axis=1)


def make_routing(wl: Workload, seed: int) -> Tuple[np.ndarray, np.ndarray]:
    """Router output of one step: ids int32 [R,S,K] and weights float32 [R,S,K].

    Draw order is fixed: per-expert terms (bias or popularity permutation), then
    per token chunk the selection scores, then the weight logits where they are
    drawn separately.
    """
    rng = np.random.default_rng(seed)
    n, E, K = wl.n_tok, wl.E, wl.K
    ids = np.empty((n, K), dtype=np.int32)
    w = np.empty((n, K), dtype=np.float32)
    if wl.routing == "bias":
        bias = rng.normal(0.0, wl.bias_std, size=E).astype(np.float32)
    elif wl.routing == "zipf":
        perm = rng.permutation(E)
        pop = np.empty(E, dtype=np.float64)
        pop[perm] = np.arange(1, E + 1, dtype=np.float64) ** (-wl.zipf_s)
        logp = np.log(pop / pop.sum()).astype(np.float32)
    elif wl.routing != "uniform":
        raise ValueError(wl.routing)
    for t0 in range(0, n, _CHUNK_TOK):
        m = min(_CHUNK_TOK, n - t0)
        if wl.routing == "bias":
            scores = rng.standard_normal((m, E), dtype=np.float32) + bias[None, :]
            sel = _topk_desc(scores, K)
            ids[t0:t0 + m] = sel
            w[t0:t0 + m] = _softmax_rows(np.take_along_axis(scores, sel, axis=1))
        else:
            if wl.routing == "uniform":
                # equal scores + Gumbel noise: a uniformly random ordered K-subset
                keys = rng.random((m, E), dtype=np.float32)
            else:
                # Gumbel-top-k sampling without replacement, probabilities ~ pop
                u = rng.random((m, E), dtype=np.float64)
                u = np.clip(u, 1e-300, 1.0)
                keys = (logp[None, :].astype(np.float64) - np.log(-np.log(u))).astype(np.float32)
            ids[t0:t0 + m] = _topk_desc(keys, K)
            w[t0:t0 + m] = _softmax_rows(rng.standard_normal((m, K), dtype=np.float32))
    return ids.reshape(wl.R, wl.S, K), w.reshape(wl.R, wl.S, K)


def make_consecutive_ids(R: int, E: int, K: int, S: int, seed: int,
                         zipf_s: float = 1.0) -> np.ndarray:
    """Router ids int32 [R,S,K] that are cheap to draw at billions of entries, for
    shapes near the largest entry count: token g takes the K experts f_g, f_g + 1,
    ..., f_g + K - 1 (mod E), distinct as long as K <= E, after a first expert f_g
    drawn with popularity proportional to rank^-zipf_s over a seeded permutation
    of the experts. Tokens are drawn in chunks, so the only large array is the
    result."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(E)
    pop = np.empty(E, dtype=np.float64)
    pop[perm] = np.arange(1, E + 1, dtype=np.float64) ** (-zipf_s)
    cdf = np.cumsum(pop / pop.sum())
    n = R * S
    ids = np.empty((n, K), dtype=np.int32)
    step = np.arange(K, dtype=np.int32)[None, :]
    for t0 in range(0, n, 1 << 24):
        m = min(1 << 24, n - t0)
        first = np.minimum(np.searchsorted(cdf, rng.random(m)), E - 1).astype(np.int32)
        blk = ids[t0:t0 + m]
        np.add(first[:, None], step, out=blk)
        np.remainder(blk, E, out=blk)
    return ids.reshape(R, S, K)


def manifest(*arrays: np.ndarray) -> str:
    """sha256 over the raw bytes of the given host arrays (reproducibility record)."""
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


# ---------------------------------------------------------------- dense tensors

_STREAM_IDS = {"hidden": 1, "y": 2, "expert_w": 3, "dup_grads": 4, "home_grads": 5}


def torch_dtype(dt: int):
    import torch
    return {F32: torch.float32, BF16: torch.bfloat16}[dt]


def dense(shape, dt: int, std: float, seed: int, stream: str, device) -> "torch.Tensor":
    """Seeded N(0, std^2) tensor of element type dt, drawn chunk by chunk along dim 0
    in float32 with torch's generator on `device`, then rounded (RNE) to dt."""
    import torch
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed) * 1009 + _STREAM_IDS[stream])
    out = torch.empty(shape, dtype=torch_dtype(dt), device=dev)
    flat = out.view(shape[0], -1)
    per = max(1, (1 << 26) // max(1, flat.shape[1]))
    for i in range(0, shape[0], per):
        j = min(shape[0], i + per)
        t = torch.randn((j - i, flat.shape[1]), generator=g, device=dev, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        flat[i:j].copy_(t)
    return out


def make_hidden(wl: Workload, seed: int, device="cpu"):
    return dense((wl.R, wl.S, wl.H), wl.dtype, 1.0, seed, "hidden", device)


def make_expert_out(wl: Workload, seed: int, device="cpu"):
    """Stand-in expert outputs y [R, S*K, H] (the input of combine)."""
    return dense((wl.R, wl.SK, wl.H), wl.dtype, 1.0, seed, "y", device)


def make_expert_weights(wl: Workload, seed: int, device="cpu"):
    return dense((wl.E,) + tuple(wl.block_shape), wl.block_dtype, wl.weight_std, seed,
                 "expert_w", device)


def make_grads(wl: Workload, seed: int, device="cpu"):
    """fp32 gradients: duplicate slots [R, B, n] and home experts [E, n]."""
    n = wl.block_elems
    dup = dense((wl.R, wl.B, n), F32, 1.0, seed, "dup_grads", device)
    home = dense((wl.E, n), F32, 1.0, seed, "home_grads", device)
    return dup, home
