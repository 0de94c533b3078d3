"""ep_layout_no_alloc (the layout for callers that cannot allocate: its scratch
is the library's own per-GPU array) against ep_layout, through the C ABI.

Two calls in a row on the one GPU, the second with a smaller input, each
compared table by table, bit for bit, with ep_layout's tables for the same
routing (and with the oracle's).  The array keeps the first call's contents,
so the second call also shows that no stale word of it is read."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import combine_ep_layout_07_amd.ep as ep  # noqa: E402
import oracle  # noqa: E402
from combine_ep_layout_07_amd.workloads import WORKLOADS, Workload, generate, seed_for  # noqa: E402
from tests.gpu_harness import compare_tables, layout_host, say  # noqa: E402


def _layout_both(w, seed, num_layout_cus=0, one_launch=False):
    inputs = generate(w, seed, with_x=False, masked_frac=0.1, invalid_frac=0.01, dup_frac=0.2)
    topk = torch.from_numpy(inputs["topk_idx"]).cuda()
    cfg = ep.config_for(w, num_layout_cus, layout_one_launch=one_launch)
    say(f"[case] {w.name} ep_layout vs ep_layout_no_alloc (cus={num_layout_cus}, one_launch={one_launch}, "
        f"scratch {int(ep.ep_query_sizes(cfg).layout_scratch)} B)")
    want = ep.alloc_layout(cfg)
    ep.ep_layout(cfg, topk, want)
    got = ep.alloc_layout(cfg)
    for t in got.tables().values():
        t.fill_(-7)
    got.scratch = None
    got.struct.scratch_dev = None  # the caller's scratch is not used
    ep.ep_layout_no_alloc(cfg, topk, got)
    torch.cuda.synchronize()
    compare_tables(layout_host(got), layout_host(want))
    lay_o = oracle.layout(w.S, w.T, w.K, w.E, w.R, w.Nmax, inputs["topk_idx"], w.expand, w.alignment, w.n_out)
    compare_tables(layout_host(got), lay_o)


def test_no_alloc_layout_two_calls_second_smaller():
    # the receive-side expand workload (16 sources x 2048 tokens: the largest
    # scratch of the workloads), then the headline compact one (4096 tokens)
    _layout_both(WORKLOADS[5], seed_for(5))
    _layout_both(WORKLOADS[2], seed_for(2))


def test_no_alloc_layout_small_after_large_geometry():
    # many layout workgroups first (a large scratch footprint), then a small
    # hybrid problem with few units and a one-workgroup single-source layout
    _layout_both(WORKLOADS[4], seed_for(4), num_layout_cus=1000)
    _layout_both(Workload("hybrid_small", S=6, T=97, H=64, K=6, E=24, R=6, Nmax=100, n_out=3), 5)
    _layout_both(WORKLOADS[1], seed_for(1))


def test_no_alloc_one_launch_layout_two_calls_second_smaller():
    # the one-launch layout keeps its exchange words in the library's array
    # too (after the counts, so their place moves with the geometry)
    _layout_both(WORKLOADS[2], seed_for(2), one_launch=True)
    _layout_both(WORKLOADS[2].with_(name="dsv3_half", T=2048, Nmax=2048), 3, one_launch=True)
    _layout_both(WORKLOADS[2], seed_for(2), num_layout_cus=300, one_launch=True)
