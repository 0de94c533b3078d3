"""Seeded synthetic inputs for the expert-parallel dispatch/combine workloads.

This module only draws inputs: routing (``topk_idx``), gate weights, hidden rows
and fp8 scale factors, plus a stand-in for the experts' outputs.  It performs no
step of the layout, scatter, copy epilogue or combine, so both the HIP path and
the CPU oracle can consume its arrays without sharing any of the method's
arithmetic.  Every array is produced on the host with
``numpy.random.Generator(PCG64(seed))``; conversions to bf16 and fp8 e4m3fn use
PyTorch's own casts (round-to-nearest-even), not code of this project.

Shapes follow the DeepEP v2 pages: the deterministic-dispatch PR (issue #757,
section "Performance") benchmarks 4096 tokens, hidden 7168, top-8 of 256
experts over EP16; the other workloads are the tiny, fp8, skewed and
receive-side variants of that share.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "generate", "draw_expert_outputs", "row_bytes", "sf_per_row", "seed_for"]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic dispatch/combine problem on one GPU's share.

    S source partitions of T tokens each, hidden size H, top-K routing over E
    experts placed in contiguous blocks of E/R on R logical ranks; Nmax is
    num_max_tokens_per_rank.  ``dtype`` is the dispatched hidden format ("bf16",
    or "fp8" = OCP e4m3fn bytes with one fp32 scale per 128 columns).
    """
    name: str
    S: int
    T: int
    H: int
    K: int
    E: int
    R: int
    Nmax: int
    dtype: str = "bf16"
    expand: bool = False
    alignment: int = 1
    routing: str = "uniform"      # "uniform" distinct experts, or "zipf"
    zipf_s: float = 1.2
    n_out: int = 1                # num_scaleout_ranks: > 1 = hybrid row form, S = n_out * n_up

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[int, Workload] = {
    1: Workload("tiny", S=1, T=128, H=256, K=4, E=32, R=8, Nmax=128),
    2: Workload("dsv3_share", S=1, T=4096, H=7168, K=8, E=256, R=16, Nmax=4096),
    3: Workload("dsv3_share_fp8", S=1, T=4096, H=7168, K=8, E=256, R=16, Nmax=4096, dtype="fp8"),
    4: Workload("zipf_skew", S=1, T=8192, H=4096, K=8, E=128, R=16, Nmax=8192, routing="zipf"),
    5: Workload("recv_side_expand", S=16, T=2048, H=7168, K=8, E=256, R=16, Nmax=2048, expand=True),
}


def row_bytes(w: Workload) -> int:
    """Bytes of one dispatched hidden row."""
    return w.H * (1 if w.dtype == "fp8" else 2)


def sf_per_row(w: Workload) -> int:
    """fp32 scale factors per row (one per 128 columns for fp8, else none)."""
    return w.H // 128 if w.dtype == "fp8" else 0


def _route(w: Workload, rng: np.random.Generator) -> np.ndarray:
    n = w.S * w.T
    if w.K > w.E:
        raise ValueError(f"{w.K} distinct experts per token need E >= K (E = {w.E})")
    if w.routing == "uniform":
        # K distinct experts, uniform: the first K of a random permutation per token.
        keys = rng.random((n, w.E))
        return np.argsort(keys, axis=1, kind="stable")[:, : w.K].astype(np.int64)
    if w.routing == "zipf":
        # K experts without replacement from p_e proportional to (e+1)^-s
        # (Gumbel-top-k, which samples successively without replacement).
        logp = -w.zipf_s * np.log(np.arange(1, w.E + 1, dtype=np.float64))
        g = rng.gumbel(size=(n, w.E))
        return np.argsort(-(logp[None, :] + g), axis=1, kind="stable")[:, : w.K].astype(np.int64)
    raise ValueError(f"unknown routing {w.routing!r}")


def generate(w: Workload, seed: int, *, with_x: bool = True, masked_frac: float = 0.0,
             invalid_frac: float = 0.0, dup_frac: float = 0.0) -> Dict[str, np.ndarray]:
    """Draw one seeded input set for ``w``.

    Draw order: routing keys, logits, x, scales; then the optional edge-case
    perturbations (masked lanes = -1, out-of-range lanes = E + j, duplicated
    experts inside a token), each from the same generator.

    Returns host arrays: ``topk_idx`` int64 [S][T][K], ``topk_weights`` fp32
    [S][T][K], ``x`` uint8 view of the rows [S][T][row_bytes], ``x_sf`` fp32
    [S][T][H/128] (fp8 only, else shape [S][T][0]).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    n = w.S * w.T
    topk = _route(w, rng) if n > 0 else np.zeros((0, w.K), np.int64)
    logits = rng.standard_normal((n, w.K))
    z = np.exp(logits - logits.max(axis=1, keepdims=True)) if n > 0 else logits
    weights = (z / z.sum(axis=1, keepdims=True)).astype(np.float32) if n > 0 else z.astype(np.float32)
    out: Dict[str, np.ndarray] = {}
    if with_x:
        xf = rng.standard_normal((n, w.H), dtype=np.float32)
        xt = torch.from_numpy(xf)
        if w.dtype == "fp8":
            xb = xt.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        else:
            xb = xt.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint8)
        out["x"] = np.ascontiguousarray(xb).reshape(w.S, w.T, row_bytes(w))
        del xf, xt
        if w.dtype == "fp8":
            sf = rng.uniform(0.5, 2.0, (n, w.H // 128)).astype(np.float32)
        else:
            sf = np.zeros((n, 0), np.float32)
        out["x_sf"] = sf.reshape(w.S, w.T, sf_per_row(w))
    if masked_frac > 0 and n > 0:
        m = rng.random((n, w.K)) < masked_frac
        topk[m] = -1
    if invalid_frac > 0 and n > 0:
        m = rng.random((n, w.K)) < invalid_frac
        topk[m] = w.E + rng.integers(0, 3, size=int(m.sum()))
    if dup_frac > 0 and n > 0 and w.K > 1:
        m = rng.random(n) < dup_frac
        rows = np.nonzero(m)[0]
        src = rng.integers(0, w.K, size=rows.size)
        dst = rng.integers(0, w.K, size=rows.size)
        topk[rows, dst] = topk[rows, src]
    out["topk_idx"] = np.ascontiguousarray(topk.reshape(w.S, w.T, w.K))
    out["topk_weights"] = np.ascontiguousarray(weights.reshape(w.S, w.T, w.K))
    return out


def draw_expert_outputs(rows: int, H: int, seed: int) -> np.ndarray:
    """Stand-in for the experts' bf16 outputs ``y``: ``rows`` x H N(0,1) draws as bf16 bits (uint16)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    yf = rng.standard_normal((rows, H), dtype=np.float32)
    return torch.from_numpy(yf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def seed_for(config_id: int, sweep: int = 0) -> int:
    """Seeds: 1000+id for the headline draw, 2000+id and 3000+id for parity sweeps."""
    return (1 + sweep) * 1000 + config_id
