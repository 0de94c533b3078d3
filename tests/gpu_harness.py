"""Helpers of the GPU tests: upload seeded inputs, run the HIP path through the
C ABI (the ``combine_ep_layout_07_amd.ep`` binding), bring results back, and
compare them with the oracle element by element."""
from __future__ import annotations

import sys
from typing import Dict

import numpy as np
import torch

import combine_ep_layout_07_amd.ep as ep
import oracle


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def upload(w, inputs: Dict[str, np.ndarray], device="cuda"):
    d = dict(
        x=torch.from_numpy(inputs["x"].reshape(w.S * w.T, inputs["x"].shape[-1])).to(device),
        topk_idx=torch.from_numpy(inputs["topk_idx"]).to(device),
        topk_weights=torch.from_numpy(inputs["topk_weights"]).to(device),
        x_sf=torch.from_numpy(inputs["x_sf"]).to(device) if w.dtype == "fp8" else None,
    )
    return d


def run_layout(w, dev, num_layout_cus=0, direct=False):
    cfg = ep.config_for(w, num_layout_cus, direct)
    L = ep.alloc_layout(cfg)
    ep.ep_layout(cfg, dev["topk_idx"], L)
    torch.cuda.synchronize()
    return cfg, L


def layout_host(L) -> Dict[str, np.ndarray]:
    return {k: v.cpu().numpy() for k, v in L.tables().items()}


def compare_tables(got: Dict[str, np.ndarray], want: Dict[str, np.ndarray]):
    for key, wv in want.items():
        g = np.asarray(got[key]).reshape(-1).astype(np.int64)
        v = np.asarray(wv).reshape(-1).astype(np.int64)
        assert g.shape == v.shape, f"{key}: shape {g.shape} vs {v.shape}"
        bad = np.nonzero(g != v)[0]
        assert bad.size == 0, f"{key}: {bad.size} mismatches; first at {bad[0]}: gpu {g[bad[0]]} oracle {v[bad[0]]}"


def filled_staging_mask(w, lay) -> np.ndarray:
    """[R][S][Nmax] mask of the staging rows the layout fills: j < tokens_per_rank
    of the source whose region it is (regions reordered on the hybrid path)."""
    from tests.brute import staging_region
    tpr = np.asarray(lay["tokens_per_rank"]).reshape(w.S, w.R)
    cnt = np.zeros((w.R * w.S,), np.int64)
    for d in range(w.R):
        for s in range(w.S):
            cnt[staging_region(d, s, w.S, w.n_out)] = tpr[s, d]
    j = np.arange(w.Nmax)[None, None, :]
    return j < cnt.reshape(w.R, w.S)[:, :, None]


def compare_dispatch(w, lay, gpu: "ep.RecvBuffers", want: Dict[str, np.ndarray], direct: bool = False):
    """Bit-exact comparison of staging (filled rows) and receive buffers (filled
    rows).  With Direct Recv X the staging rows hold no hidden bytes."""
    mask = filled_staging_mask(w, lay)
    if not direct:
        sx = gpu.staging_x.cpu().numpy()
        assert (sx[mask] == want["staging_x"][mask]).all(), "staging_x differs"
        del sx
    sm = gpu.staging_meta.cpu().numpy()
    assert (sm[mask] == want["staging_meta"][mask]).all(), "staging_meta differs"
    if w.dtype == "fp8":
        ssf = gpu.staging_sf.cpu().numpy()
        assert (ssf[mask].view(np.int32) == want["staging_sf"][mask].view(np.int32)).all(), "staging_sf differs"
    n = oracle.recv_rows(w.S, w.T, w.K, w.E, w.R, lay, w.expand)
    rx = gpu.recv_x[:n].cpu().numpy()
    bad = np.nonzero((rx != want["recv_x"][:n]).any(axis=1))[0]
    assert bad.size == 0, f"recv_x: {bad.size} rows differ, first {bad[0]}"
    del rx
    assert (gpu.recv_src_idx[:n].cpu().numpy() == want["recv_src_idx"][:n]).all(), "recv_src_idx differs"
    assert (gpu.recv_topk_weights[:n].cpu().numpy().view(np.int32)
            == want["recv_topk_weights"][:n].view(np.int32)).all(), "recv_topk_weights differ"
    if not w.expand:
        assert (gpu.recv_topk_idx[:n].cpu().numpy() == want["recv_topk_idx"][:n]).all(), "recv_topk_idx differs"
    if w.dtype == "fp8":
        assert (gpu.recv_sf[:n].cpu().numpy().view(np.int32) == want["recv_sf"][:n].view(np.int32)).all()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def compare_combine(got_bits: np.ndarray, want_bits: np.ndarray, rtol=1e-2, atol=1e-5) -> float:
    """Elementwise |gpu - oracle| <= rtol*|oracle| + atol; returns the bit-equal share."""
    g = bf16_to_f64(got_bits.reshape(-1))
    o = bf16_to_f64(want_bits.reshape(-1))
    err = np.abs(g - o)
    lim = rtol * np.abs(o) + atol
    bad = np.nonzero(~(err <= lim))[0]
    assert bad.size == 0, f"combine: {bad.size} elements out of tolerance; first {bad[0]}: gpu {g[bad[0]]} oracle {o[bad[0]]}"
    return float((got_bits.reshape(-1) == want_bits.reshape(-1)).mean()) if g.size else 1.0


def seeded_y(rows: int, H: int, seed: int, device="cuda") -> torch.Tensor:
    """Expert-output stand-in: N(0,1) bf16 drawn on the device from a seeded generator."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return torch.randn((max(rows, 1), H), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
