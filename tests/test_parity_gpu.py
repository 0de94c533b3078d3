"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Layout tables, staging rows, receive rows and metadata are compared bit-exactly;
combine within |gpu - oracle| <= 1e-2 * |oracle| + 1e-5 (fp32 accumulation of at
most K products vs the oracle's double accumulation, both rounded once to bf16:
they differ by at most one bf16 ulp, 2^-8..2^-7 relative, except where
cancellation leaves a result below the fp32 accumulation error
K * 2^-24 * sum|w*y| ~ 3e-6, which the absolute term covers).

The five workloads run at their full sizes in the launch configuration the
benchmark times; the small cases cover edge lanes, ragged sizes and limits.
"""
import os
import types

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import combine_ep_layout_07_amd.ep as ep  # noqa: E402
import oracle  # noqa: E402
from combine_ep_layout_07_amd.workloads import WORKLOADS, Workload, generate, seed_for  # noqa: E402
from tests.gpu_harness import (bf16_to_f64, compare_combine, compare_dispatch, compare_tables, layout_host,  # noqa: E402
                               run_layout, say, seeded_y, upload)


def _without_scratch(L):
    """The same layout buffers, with no scratch pointer for the dispatch and
    the combine (the copy epilogue then has no receive-row index).  Holds L,
    whose tensors the copied pointers address."""
    st = ep.EpLayoutT.from_buffer_copy(L.struct)
    st.scratch_dev = None
    return types.SimpleNamespace(struct=st, buffers=L)


def _full_case(w, seed, edge=None, num_layout_cus=0, check_combine=True, direct=False, scratch=True):
    edge = edge or {}
    say(f"[case] {w.name} S={w.S} T={w.T} H={w.H} K={w.K} E={w.E} R={w.R} Nmax={w.Nmax} {w.dtype} "
        f"expand={w.expand} A={w.alignment} seed={seed} edge={edge} cus={num_layout_cus} direct={direct} "
        f"scratch={scratch}")
    inputs = generate(w, seed, **edge)
    lay_o = oracle.layout(w.S, w.T, w.K, w.E, w.R, w.Nmax, inputs["topk_idx"], w.expand, w.alignment, w.n_out)
    dev = upload(w, inputs)
    say("  ep_layout")
    cfg, L = run_layout(w, dev, num_layout_cus, direct)
    compare_tables(layout_host(L), lay_o)
    if not scratch:
        L = _without_scratch(L)
    say("  ep_dispatch")
    R = ep.alloc_recv(cfg)
    ep.ep_dispatch(cfg, dev["x"], dev["x_sf"], dev["topk_idx"], dev["topk_weights"], L, R)
    torch.cuda.synchronize()
    want = oracle.dispatch(w.S, w.T, w.H, w.K, w.E, w.R, w.Nmax, w.dtype == "fp8", w.expand, w.alignment,
                           inputs["x"], inputs.get("x_sf"), inputs["topk_idx"], inputs["topk_weights"], lay_o,
                           w.n_out)
    compare_dispatch(w, lay_o, R, want, direct)
    del want
    if not check_combine:
        return
    say("  ep_combine")
    rows = int(ep.ep_query_sizes(cfg).recv_rows)
    y = seeded_y(rows, w.H, seed + 17)
    out = torch.empty((w.S * w.T, w.H), dtype=torch.bfloat16, device="cuda")
    ep.ep_combine(cfg, L, dev["topk_idx"], dev["topk_weights"], y, out)
    torch.cuda.synchronize()
    y_h = y.view(torch.int16).cpu().numpy().view(np.uint16)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.combine(w.S, w.T, w.H, w.K, w.E, w.R, w.Nmax, w.expand, inputs["topk_idx"],
                         inputs["topk_weights"], lay_o, y_h, w.n_out).reshape(-1, w.H)
    share = compare_combine(got, ref)
    say(f"  combine bit-equal share {share:.6f}")
    assert share > 0.99


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4, 5])
def test_workload_full_size(cfg_id):
    w = WORKLOADS[cfg_id]
    _full_case(w, seed_for(cfg_id))


@pytest.mark.parametrize("cfg_id", [1, 3, 4])
@pytest.mark.parametrize("sweep", [1, 2])
def test_workload_sweep_seeds(cfg_id, sweep):
    w = WORKLOADS[cfg_id]
    _full_case(w, seed_for(cfg_id, sweep), check_combine=(cfg_id == 1))


EDGE = dict(masked_frac=0.15, invalid_frac=0.03, dup_frac=0.3)
SMALL = [
    Workload("ragged", S=3, T=301, H=264, K=6, E=24, R=6, Nmax=310),
    Workload("k1", S=1, T=130, H=64, K=1, E=16, R=16, Nmax=130),
    Workload("k3", S=2, T=97, H=128, K=3, E=32, R=8, Nmax=100),
    Workload("k32", S=1, T=77, H=64, K=32, E=128, R=64, Nmax=80),
    Workload("r1", S=2, T=200, H=64, K=4, E=8, R=1, Nmax=200),
    Workload("e1024", S=1, T=300, H=64, K=8, E=1024, R=64, Nmax=300),
    Workload("row16B", S=2, T=150, H=8, K=4, E=16, R=4, Nmax=150),
    Workload("fp8_small", S=2, T=120, H=256, K=5, E=20, R=5, Nmax=128, dtype="fp8"),
    Workload("expand_small", S=4, T=90, H=128, K=4, E=32, R=8, Nmax=96, expand=True),
    Workload("expand_a4_fp8", S=3, T=70, H=128, K=4, E=16, R=4, Nmax=70, expand=True, alignment=4, dtype="fp8"),
    Workload("expand_a128", S=2, T=64, H=64, K=8, E=32, R=8, Nmax=64, expand=True, alignment=128),
    Workload("empty", S=2, T=0, H=64, K=4, E=16, R=4, Nmax=0),
    Workload("empty_expand", S=1, T=0, H=64, K=4, E=16, R=4, Nmax=4, expand=True, alignment=2),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
@pytest.mark.parametrize("edge", [False, True], ids=["clean", "edge_lanes"])
def test_small_cases(w, edge):
    _full_case(w, 7, EDGE if edge else None)


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4])
def test_direct_recv_x_full_size(cfg_id):
    """Direct Recv X writes the same receive rows, scales and metadata."""
    _full_case(WORKLOADS[cfg_id], seed_for(cfg_id, 1), direct=True, check_combine=(cfg_id == 1))


@pytest.mark.parametrize("w", [SMALL[0], SMALL[3], SMALL[4], SMALL[7], SMALL[11]], ids=lambda w: w.name)
def test_direct_recv_x_small(w):
    _full_case(w, 11, EDGE, direct=True)


@pytest.mark.parametrize("w", [
    Workload("sources_1000_fits", S=1000, T=3, H=8, K=2, E=1024, R=2, Nmax=3),
    Workload("sources_600_fits_expand", S=600, T=4, H=8, K=2, E=1024, R=2, Nmax=4, expand=True),
    Workload("sources_700_hybrid", S=700, T=3, H=8, K=2, E=256, R=4, Nmax=3, n_out=7),
], ids=lambda w: w.name)
def test_receiver_tables_of_many_sources(w):
    """Many sources for few destinations: the receiver tables' prefix over
    sources is a workgroup scan per destination instead of one thread's walk
    (per-source totals gathered in LDS, or -- the hybrid case's 700 sources x 4
    destinations -- straight from the unit counts); the row form's segments
    on top."""
    _full_case(w, 37, EDGE)


@pytest.mark.parametrize("mode", ["staging", "direct", "expand"])
def test_receiver_tables_beyond_lds(mode):
    """R * (S + 1) > 8192 table entries: the epilogues search recv_base and
    recv_psum in global memory instead of staging them in LDS."""
    w = Workload("many_sources", S=160, T=5, H=64, K=3, E=64, R=64, Nmax=6, expand=mode == "expand",
                 alignment=2 if mode == "expand" else 1)
    assert w.R * (w.S + 1) + w.R + 1 > 8192
    _full_case(w, 31, EDGE, direct=mode == "direct")


@pytest.mark.parametrize("case", ["tiny", "dsv3_share", "expand_small", "expand_a4_fp8"])
@pytest.mark.parametrize("nb", [1, 2])
def test_combine_bias(case, nb):
    """ep_combine_bias: bias rows added before the single rounding."""
    w = {x.name: x for x in list(WORKLOADS.values()) + SMALL}[case]
    inputs = generate(w, 23, masked_frac=0.1)
    lay_o = oracle.layout(w.S, w.T, w.K, w.E, w.R, w.Nmax, inputs["topk_idx"], w.expand, w.alignment)
    dev = upload(w, inputs)
    say(f"[case] {w.name} ep_combine_bias nb={nb}")
    cfg, L = run_layout(w, dev)
    rows = int(ep.ep_query_sizes(cfg).recv_rows)
    y = seeded_y(rows, w.H, 5)
    biases = [seeded_y(w.S * w.T, w.H, 6 + i) for i in range(nb)]
    out = torch.empty((w.S * w.T, w.H), dtype=torch.bfloat16, device="cuda")
    ep.ep_combine_bias(cfg, L, dev["topk_idx"], dev["topk_weights"], y, biases[0], biases[1] if nb > 1 else None,
                       out)
    torch.cuda.synchronize()
    hb = [b.view(torch.int16).cpu().numpy().view(np.uint16).reshape(w.S, w.T, w.H) for b in biases]
    ref = oracle.combine_bias(w.S, w.T, w.H, w.K, w.E, w.R, w.Nmax, w.expand, inputs["topk_idx"],
                              inputs["topk_weights"], lay_o, y.view(torch.int16).cpu().numpy().view(np.uint16),
                              hb[0], hb[1] if nb > 1 else None)
    share = compare_combine(out.view(torch.int16).cpu().numpy().view(np.uint16), ref)
    assert share > 0.99


def test_cached_layout_replay():
    """One layout (the pages' handle) serves several dispatches of different
    hidden states with the same routing."""
    w = WORKLOADS[3]
    inputs = generate(w, seed_for(3, 1))
    other = generate(w, seed_for(3, 2))
    say("[case] dsv3_share_fp8 cached layout replay")
    lay_o = oracle.layout(w.S, w.T, w.K, w.E, w.R, w.Nmax, inputs["topk_idx"], w.expand, w.alignment)
    dev = upload(w, inputs)
    cfg, L = run_layout(w, dev)
    for x_np, sf_np in ((inputs["x"], inputs["x_sf"]), (other["x"], other["x_sf"]), (inputs["x"], inputs["x_sf"])):
        x = torch.from_numpy(x_np.reshape(w.S * w.T, -1)).cuda()
        sf = torch.from_numpy(sf_np).cuda()
        R = ep.alloc_recv(cfg)
        ep.ep_dispatch(cfg, x, sf, dev["topk_idx"], dev["topk_weights"], L, R)
        torch.cuda.synchronize()
        want = oracle.dispatch(w.S, w.T, w.H, w.K, w.E, w.R, w.Nmax, True, False, 1, x_np, sf_np,
                               inputs["topk_idx"], inputs["topk_weights"], lay_o)
        compare_dispatch(w, lay_o, R, want)


@pytest.mark.parametrize("w", [
    WORKLOADS[2].with_(name="dsv3_share_expand_a128", expand=True, alignment=128),
    Workload("expand_a4_fp8_replay", S=3, T=70, H=128, K=4, E=16, R=4, Nmax=70, expand=True, alignment=4,
             dtype="fp8"),
], ids=lambda w: w.name)
def test_cached_expand_layout_replay(w):
    """The cached-expand path: one expand layout (with alignment padding) serves
    three dispatches of different hidden states into the same receive buffers,
    then a combine; every receive row, padding row, scale and weight is
    bit-exact against the oracle each time, and the combine within tolerance."""
    inputs = generate(w, seed_for(2, 6), masked_frac=0.05)
    say(f"[case] {w.name} cached expand layout replay")
    lay_o = oracle.layout(w.S, w.T, w.K, w.E, w.R, w.Nmax, inputs["topk_idx"], w.expand, w.alignment)
    dev = upload(w, inputs)
    cfg, L = run_layout(w, dev)
    compare_tables(layout_host(L), lay_o)
    R = ep.alloc_recv(cfg)
    for rep, seed in enumerate((seed_for(2, 7), seed_for(2, 8), seed_for(2, 7))):
        other = generate(w, seed)
        say(f"  dispatch {rep} (x seed {seed})")
        x = torch.from_numpy(other["x"].reshape(w.S * w.T, -1)).cuda()
        sf = torch.from_numpy(other["x_sf"]).cuda() if w.dtype == "fp8" else None
        ep.ep_dispatch(cfg, x, sf, dev["topk_idx"], dev["topk_weights"], L, R)
        torch.cuda.synchronize()
        want = oracle.dispatch(w.S, w.T, w.H, w.K, w.E, w.R, w.Nmax, w.dtype == "fp8", True, w.alignment,
                               other["x"], other.get("x_sf"), inputs["topk_idx"], inputs["topk_weights"], lay_o)
        compare_dispatch(w, lay_o, R, want)
        del want
    say("  ep_combine")
    rows = int(ep.ep_query_sizes(cfg).recv_rows)
    y = seeded_y(rows, w.H, 29)
    out = torch.empty((w.S * w.T, w.H), dtype=torch.bfloat16, device="cuda")
    ep.ep_combine(cfg, L, dev["topk_idx"], dev["topk_weights"], y, out)
    torch.cuda.synchronize()
    ref = oracle.combine(w.S, w.T, w.H, w.K, w.E, w.R, w.Nmax, True, inputs["topk_idx"], inputs["topk_weights"],
                         lay_o, y.view(torch.int16).cpu().numpy().view(np.uint16))
    assert compare_combine(out.view(torch.int16).cpu().numpy().view(np.uint16), ref) > 0.99


HYBRID = [
    # the deterministic-dispatch page's 2 x 8 topology (EP16 over two scale-out groups)
    Workload("hybrid_2x8", S=16, T=512, H=7168, K=8, E=256, R=16, Nmax=512, n_out=2),
    Workload("hybrid_3x2_edge", S=6, T=97, H=264, K=6, E=24, R=6, Nmax=100, n_out=3),
    Workload("hybrid_2x2_fp8_expand", S=4, T=80, H=256, K=4, E=16, R=4, Nmax=80, n_out=2, dtype="fp8", expand=True,
             alignment=4),
]


@pytest.mark.parametrize("w", HYBRID, ids=lambda w: w.name)
def test_hybrid_row_form(w):
    _full_case(w, 19, EDGE if "edge" in w.name else None)


def test_hybrid_direct_recv_x():
    _full_case(HYBRID[0], 21, direct=True, check_combine=False)


@pytest.mark.parametrize("cus", [0, 1200])
def test_expand_widest_expert_and_topk_limits(cus):
    """Expand at the limits: E = 1024 experts (16 expert-scan workgroups), K = 32
    lanes per token (two tokens per wave step), R = 64, alignment 3; 1200
    layout workgroups give 300 units, more per scan segment than it keeps in
    registers."""
    w = Workload("expand_e1024_k32", S=3, T=400, H=64, K=32, E=1024, R=64, Nmax=400, expand=True, alignment=3)
    _full_case(w, 41, EDGE, num_layout_cus=cus)


@pytest.mark.parametrize("mode", ["staging", "direct", "expand", "fp8"])
def test_rows_wider_than_one_pass(mode):
    """H = 10240 bf16 (or 16512 fp8): 1280 (1032) 16-byte chunks per row, more
    than one pass of 64 lanes x 16 chunks, so the scatter, the epilogues and
    the combine loop over column passes (the pipelined one-pass kernels are
    not used)."""
    fp8 = mode == "fp8"
    w = Workload(f"wide_{mode}", S=2, T=45, H=16512 if fp8 else 10240, K=4, E=16, R=4, Nmax=48,
                 expand=mode == "expand", alignment=2 if mode == "expand" else 1, dtype="fp8" if fp8 else "bf16")
    _full_case(w, 51, EDGE, direct=mode == "direct")


PIECES = [
    Workload("pieces_bf16_ragged", S=5, T=2048, H=7000, K=8, E=256, R=16, Nmax=2048),
    Workload("pieces_fp8_ragged", S=8, T=2048, H=8320, K=8, E=256, R=16, Nmax=2048, dtype="fp8"),
    Workload("pieces_hybrid_2x4", S=8, T=2048, H=7000, K=8, E=256, R=16, Nmax=2048, n_out=2),
]


@pytest.mark.parametrize("w,direct", [(w, d) for w in PIECES for d in (False, True)] +
                         [(Workload("pieces_expand_a4", S=8, T=2048, H=7000, K=8, E=256, R=16, Nmax=2048,
                                    expand=True, alignment=4), False)],
                         ids=lambda c: getattr(c, "name", None) or ("direct" if c else "staging"))
def test_scatter_in_pieces(w, direct):
    """Rows of more than 1 GiB (bound S*T*min(K,R) rows) take the staging
    scatter in 1 KiB pieces per wave, and Direct Recv X (from 512 MiB) in 2 KiB
    pieces: ragged last pieces (875 and 520 chunks per row), fp8 scales, the
    hybrid row form, a padded expand layout, masked and duplicate lanes."""
    _full_case(w, 61, EDGE, direct=direct)


@pytest.mark.parametrize("w", [WORKLOADS[3], SMALL[0], SMALL[1], SMALL[7], SMALL[8], SMALL[9], HYBRID[1], HYBRID[2],
                               Workload("wide_bf16", S=2, T=45, H=10240, K=4, E=16, R=4, Nmax=48),
                               WORKLOADS[5].with_(name="expand_quarter", S=4)],
                         ids=lambda w: w.name)
def test_dispatch_without_layout_scratch(w):
    """Dispatch and combine given the layout without its scratch: the copy
    epilogues have no index and search the receiver tables for each row's
    source (compact and expand, one-pass rows, rows wider than one pass, fp8,
    the hybrid row form, edge lanes); the oracle's results either way."""
    _full_case(w, 73, EDGE, scratch=False)


def test_expand_alignment_128_at_dsv3_shape():
    """The expand layout at the pages' benchmark alignment (128, zero padding)
    on the 4096-token H=7168 shape: ~32k padding rows next to 32k lane rows."""
    _full_case(WORKLOADS[2].with_(name="dsv3_share_expand_a128", expand=True, alignment=128), seed_for(2, 5))


def test_hybrid_2x8_at_dsv3_token_count():
    """16 sources of 256 tokens (2 scale-out x 8 scale-up): the same 4096
    tokens as the headline shape, in the hybrid row form."""
    _full_case(WORKLOADS[2].with_(name="hybrid_2x8", S=16, T=256, Nmax=256, n_out=2), seed_for(2, 5))


def test_error_flag_for_out_of_range_ids():
    w = Workload("bad_ids", S=1, T=64, H=64, K=4, E=16, R=4, Nmax=64)
    inputs = generate(w, 3, invalid_frac=0.2)
    assert (inputs["topk_idx"] >= w.E).any()
    dev = upload(w, inputs)
    say("[case] bad_ids ep_layout")
    _, L = run_layout(w, dev)
    assert int(L.error_flags.item()) == 1
    inputs = generate(w, 3)
    dev = upload(w, inputs)
    _, L = run_layout(w, dev)
    assert int(L.error_flags.item()) == 0


SINGLE = {  # one-launch layout at num_layout_cus = 0 (8 waves up to 1024 items, 16 up to 2048)
    "single8_expand": Workload("single8_expand", S=1, T=200, H=64, K=4, E=32, R=8, Nmax=200, expand=True,
                               alignment=4),
    "single16": Workload("single16", S=1, T=250, H=64, K=8, E=64, R=16, Nmax=250),
    "single16_expand": Workload("single16_expand", S=1, T=250, H=64, K=8, E=64, R=16, Nmax=250, expand=True,
                                alignment=3),
}


@pytest.mark.parametrize("cfg_id", [1, 2, 4, 5] + list(SINGLE))
def test_layout_independent_of_workgroup_count(cfg_id):
    """Slots are a pure function of topk_idx: the number of layout workgroups
    (the pages' num_prologue_sms) changes nothing.  Workload 1 and the small
    single-source cases take the one-launch layout at num_layout_cus = 0 and
    the two-pass one otherwise."""
    w = SINGLE[cfg_id] if cfg_id in SINGLE else WORKLOADS[cfg_id]
    inputs = generate(w, seed_for(cfg_id) if cfg_id not in SINGLE else 61, with_x=False, masked_frac=0.1,
                      invalid_frac=0.02, dup_frac=0.2)
    inputs["x"] = np.zeros((w.S, w.T, 16), np.uint8)
    dev = upload(w, inputs)
    ref = None
    for cus in (0, 1, 3, 16, 64, 1000):
        say(f"[case] {w.name} ep_layout num_layout_cus={cus}")
        _, L = run_layout(w, dev, cus)
        tabs = layout_host(L)
        if ref is None:
            ref = tabs
        else:
            compare_tables(tabs, ref)


ONE_LAUNCH = [WORKLOADS[2], WORKLOADS[4], Workload("ragged_sources", S=3, T=301, H=64, K=6, E=24, R=6, Nmax=310),
              Workload("hybrid_2x8_small", S=16, T=96, H=64, K=8, E=256, R=16, Nmax=96, n_out=2),
              Workload("k32_r64", S=2, T=500, H=64, K=32, E=1024, R=64, Nmax=500)]


@pytest.mark.parametrize("w", ONE_LAUNCH, ids=lambda w: w.name)
def test_one_launch_layout_equals_two_launches(w):
    """The compact layout's one-launch form (count pass, grid-wide exchange,
    slot pass in one kernel) and its default two-launch form give the
    oracle's tables for several workgroup counts; three layouts in a row on
    one scratch buffer (each launch derives fresh exchange tokens) stay exact."""
    inputs = generate(w, 71, with_x=False, masked_frac=0.1, invalid_frac=0.02, dup_frac=0.2)
    inputs["x"] = np.zeros((w.S, w.T, 16), np.uint8)
    dev = upload(w, inputs)
    lay_o = oracle.layout(w.S, w.T, w.K, w.E, w.R, w.Nmax, inputs["topk_idx"], w.expand, w.alignment, w.n_out)
    for cus in (0, 7, 300):
        for one in (True, False):
            say(f"[case] {w.name} layout cus={cus} one_launch={one}")
            cfg = ep.config_for(w, cus, layout_one_launch=one)
            L = ep.alloc_layout(cfg)
            for _ in range(3):
                for t in L.tables().values():
                    t.fill_(-7)
                ep.ep_layout(cfg, dev["topk_idx"], L)
                torch.cuda.synchronize()
                compare_tables(layout_host(L), lay_o)


@pytest.mark.parametrize("mode", ["1", "2"])
def test_one_launch_layout_time_out_is_reported(mode, monkeypatch):
    """A forced time-out of the one-launch layout's exchange (EP_LAYOUT_SYNC_TEST:
    1 = the coordinator waits for words no unit writes, 2 = every unit does and
    gives up) ends the kernel normally with bit 1 of error_flags set (which
    also shows that the one-launch form ran); the next layout on the same
    scratch is exact again, and the default two-launch form never waits."""
    w = WORKLOADS[2]
    inputs = generate(w, seed_for(2), with_x=False)
    inputs["x"] = np.zeros((w.S, w.T, 16), np.uint8)
    dev = upload(w, inputs)
    lay_o = oracle.layout(w.S, w.T, w.K, w.E, w.R, w.Nmax, inputs["topk_idx"])
    cfg = ep.config_for(w, layout_one_launch=True)
    L = ep.alloc_layout(cfg)
    monkeypatch.setenv("EP_LAYOUT_SYNC_TEST", mode)
    say(f"[case] forced layout exchange time-out, mode {mode}")
    ep.ep_layout(cfg, dev["topk_idx"], L)
    torch.cuda.synchronize()
    assert int(L.error_flags.item()) & 2, "the time-out must be reported"
    cfg2 = ep.config_for(w)
    L2 = ep.alloc_layout(cfg2)
    ep.ep_layout(cfg2, dev["topk_idx"], L2)
    torch.cuda.synchronize()
    assert int(L2.error_flags.item()) == 0
    compare_tables(layout_host(L2), lay_o)
    monkeypatch.delenv("EP_LAYOUT_SYNC_TEST")
    ep.ep_layout(cfg, dev["topk_idx"], L)
    torch.cuda.synchronize()
    assert int(L.error_flags.item()) == 0
    compare_tables(layout_host(L), lay_o)


@pytest.mark.parametrize("name", list(SINGLE))
def test_one_launch_layout_parity(name):
    """The one-launch layout (8 and 16 waves) against the oracle, with edge lanes."""
    _full_case(SINGLE[name], 62, EDGE)


SOURCE_TOP8 = [  # one source, compact, top-8, from just above the one-workgroup layout to 16385 tokens
    Workload("top8_257", S=1, T=257, H=64, K=8, E=256, R=16, Nmax=257),
    Workload("top8_ragged_4097", S=1, T=4097, H=64, K=8, E=256, R=16, Nmax=4100),
    Workload("top8_r64_e1024", S=1, T=3000, H=64, K=8, E=1024, R=64, Nmax=3000),
    Workload("top8_r64_e64", S=1, T=2000, H=64, K=8, E=64, R=64, Nmax=2000),
    Workload("top8_r1", S=1, T=5000, H=64, K=8, E=8, R=1, Nmax=5000),
    Workload("top8_r3_e24", S=1, T=700, H=64, K=8, E=24, R=3, Nmax=700),
    Workload("top8_16384", S=1, T=16384, H=64, K=8, E=256, R=16, Nmax=16384),
    Workload("top8_16385", S=1, T=16385, H=64, K=8, E=256, R=16, Nmax=16385),
]


@pytest.mark.parametrize("w", SOURCE_TOP8, ids=lambda w: w.name)
def test_single_source_layout_sizes(w):
    """One source at top-8: ragged unit counts, one to 64 destinations, 64 to
    1024 experts, up to 16385 tokens, with masked, out-of-range and duplicate
    lanes; dispatch and combine follow from its tables.  Three layouts in a
    row into tables filled with junk stay exact, and so does routing that
    starts 8 bytes off a 16-byte boundary (the alignment the ABI requires)."""
    _full_case(w, 83, EDGE)
    inputs = generate(w, 84, with_x=False, masked_frac=0.1, invalid_frac=0.02, dup_frac=0.2)
    inputs["x"] = np.zeros((w.S, w.T, 16), np.uint8)
    dev = upload(w, inputs)
    lay_o = oracle.layout(w.S, w.T, w.K, w.E, w.R, w.Nmax, inputs["topk_idx"], w.expand, w.alignment, w.n_out)
    cfg = ep.config_for(w)
    L = ep.alloc_layout(cfg)
    for _ in range(3):
        for t in L.tables().values():
            t.fill_(-7)
        ep.ep_layout(cfg, dev["topk_idx"], L)
        torch.cuda.synchronize()
        compare_tables(layout_host(L), lay_o)
    flat = torch.empty(dev["topk_idx"].numel() + 1, dtype=torch.int64, device="cuda")
    off = flat[1:].view(dev["topk_idx"].shape)
    off.copy_(dev["topk_idx"])
    assert off.data_ptr() % 16 == 8
    for t in L.tables().values():
        t.fill_(-7)
    ep.ep_layout(cfg, off, L)
    torch.cuda.synchronize()
    compare_tables(layout_host(L), lay_o)


def test_dispatch_is_bitwise_reproducible():
    w = WORKLOADS[4]
    inputs = generate(w, seed_for(4))
    dev = upload(w, inputs)
    say("[case] zipf_skew reproducibility")
    cfg, L = run_layout(w, dev)
    outs = []
    for _ in range(2):
        R = ep.alloc_recv(cfg)
        ep.ep_dispatch(cfg, dev["x"], None, dev["topk_idx"], dev["topk_weights"], L, R)
        torch.cuda.synchronize()
        n = int(L.recv_base[-1].item())
        outs.append((R.recv_x[:n].clone(), R.recv_src_idx[:n].clone(), R.recv_topk_weights[:n].clone()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("cfg_id", [2, 5])
def test_combine_is_bitwise_reproducible(cfg_id):
    """The combine sums each output element in one lane in a fixed order, so
    repeated runs, and runs on layouts computed with different workgroup counts,
    give bitwise equal outputs (the property the deterministic path exists for)."""
    w = WORKLOADS[cfg_id]
    inputs = generate(w, seed_for(cfg_id))
    dev = upload(w, inputs)
    say(f"[case] {w.name} combine reproducibility")
    rows = None
    outs = []
    for cus in (0, 0, 37):
        cfg, L = run_layout(w, dev, num_layout_cus=cus)
        if rows is None:
            rows = int(ep.ep_query_sizes(cfg).recv_rows)
            y = seeded_y(rows, w.H, 11)
        out = torch.empty((w.S * w.T, w.H), dtype=torch.bfloat16, device="cuda")
        ep.ep_combine(cfg, L, dev["topk_idx"], dev["topk_weights"], y, out)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    assert torch.equal(outs[0].view(torch.int16), outs[2].view(torch.int16))


@pytest.mark.parametrize("w", [WORKLOADS[1], Workload("expand_specials", S=2, T=100, H=256, K=4, E=16, R=4, Nmax=100,
                                                     expand=True)], ids=lambda w: w.name)
def test_combine_special_values(w):
    """Expert outputs with NaN, +-Inf, -0, subnormals and large finite values:
    non-finite results match the oracle's class (NaN, +Inf, -Inf; NaN payloads
    may differ), finite ones stay within the combine tolerance."""
    inputs = generate(w, 555)
    dev = upload(w, inputs)
    say(f"[case] {w.name} combine special values")
    cfg, L = run_layout(w, dev)
    lay_o = oracle.layout(w.S, w.T, w.K, w.E, w.R, w.Nmax, inputs["topk_idx"], w.expand, w.alignment)
    rows = int(ep.ep_query_sizes(cfg).recv_rows)
    y_h = seeded_y(rows, w.H, 21).view(torch.int16).cpu().numpy().view(np.uint16).copy()
    rng = np.random.default_rng(7)
    specials = np.array([0x7FC0, 0x7F80, 0xFF80, 0x8000, 0x0001, 0x007F, 0x8005, 0x7149, 0xF149], np.uint16)
    pick = rng.random(y_h.shape) < 0.002
    y_h[pick] = specials[rng.integers(0, specials.size, int(pick.sum()))]
    y = torch.from_numpy(y_h.view(np.int16)).to("cuda").view(torch.bfloat16)
    out = torch.empty((w.S * w.T, w.H), dtype=torch.bfloat16, device="cuda")
    ep.ep_combine(cfg, L, dev["topk_idx"], dev["topk_weights"], y, out)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
    ref = oracle.combine(w.S, w.T, w.H, w.K, w.E, w.R, w.Nmax, w.expand, inputs["topk_idx"], inputs["topk_weights"],
                         lay_o, y_h).reshape(-1)
    g, o = bf16_to_f64(got), bf16_to_f64(ref)
    assert np.isnan(o).any() and np.isinf(o).any(), "the draw must reach NaN and Inf outputs"
    assert (np.isnan(g) == np.isnan(o)).all()
    assert (np.isposinf(g) == np.isposinf(o)).all() and (np.isneginf(g) == np.isneginf(o)).all()
    fin = np.isfinite(o)
    compare_combine(got[fin], ref[fin])


def test_phases_split_equals_all():
    w = WORKLOADS[2]
    inputs = generate(w, seed_for(2, 1))
    dev = upload(w, inputs)
    say("[case] dsv3_share split phases")
    cfg, L = run_layout(w, dev)
    R1 = ep.alloc_recv(cfg)
    ep.ep_dispatch(cfg, dev["x"], None, dev["topk_idx"], dev["topk_weights"], L, R1, ep.EP_PHASE_ALL)
    R2 = ep.alloc_recv(cfg)
    ep.ep_dispatch(cfg, dev["x"], None, dev["topk_idx"], dev["topk_weights"], L, R2, ep.EP_PHASE_SCATTER)
    ep.ep_dispatch(cfg, dev["x"], None, dev["topk_idx"], dev["topk_weights"], L, R2, ep.EP_PHASE_EPILOGUE)
    torch.cuda.synchronize()
    n = int(L.recv_base[-1].item())
    assert torch.equal(R1.recv_x[:n], R2.recv_x[:n])
    assert torch.equal(R1.recv_topk_idx[:n], R2.recv_topk_idx[:n])


@pytest.mark.parametrize("w", [WORKLOADS[1], SMALL[7],
                               Workload("hybrid_small_fused", S=6, T=80, H=128, K=6, E=24, R=6, Nmax=80, n_out=3),
                               Workload("k32_fused", S=1, T=300, H=512, K=32, E=1024, R=64, Nmax=300)],
                         ids=lambda w: w.name)
def test_small_dispatch_one_launch_equals_two(w):
    """A small compact-layout problem dispatches in one launch when both
    phases are asked for; its staging rows, records, receive rows and
    metadata equal those of the two phases enqueued separately, and the
    oracle's (edge lanes included)."""
    inputs = generate(w, 808, masked_frac=0.1, invalid_frac=0.02, dup_frac=0.2)
    dev = upload(w, inputs)
    say(f"[case] {w.name} one-launch dispatch")
    cfg, L = run_layout(w, dev)
    R1, R2 = ep.alloc_recv(cfg), ep.alloc_recv(cfg)
    ep.ep_dispatch(cfg, dev["x"], dev["x_sf"], dev["topk_idx"], dev["topk_weights"], L, R1, ep.EP_PHASE_ALL)
    ep.ep_dispatch(cfg, dev["x"], dev["x_sf"], dev["topk_idx"], dev["topk_weights"], L, R2, ep.EP_PHASE_SCATTER)
    ep.ep_dispatch(cfg, dev["x"], dev["x_sf"], dev["topk_idx"], dev["topk_weights"], L, R2, ep.EP_PHASE_EPILOGUE)
    torch.cuda.synchronize()
    lay_o = oracle.layout(w.S, w.T, w.K, w.E, w.R, w.Nmax, inputs["topk_idx"], w.expand, w.alignment, w.n_out)
    want = oracle.dispatch(w.S, w.T, w.H, w.K, w.E, w.R, w.Nmax, w.dtype == "fp8", False, 1, inputs["x"],
                           inputs.get("x_sf"), inputs["topk_idx"], inputs["topk_weights"], lay_o, w.n_out)
    compare_dispatch(w, lay_o, R1, want)
    compare_dispatch(w, lay_o, R2, want)


LAYOUT_DISPATCH = [WORKLOADS[1], SMALL[1], Workload("one_token", S=1, T=1, H=64, K=4, E=16, R=4, Nmax=1),
                   Workload("fp8_single", S=1, T=200, H=512, K=6, E=48, R=12, Nmax=205, dtype="fp8"),
                   Workload("k32_single", S=1, T=64, H=512, K=32, E=512, R=64, Nmax=64),
                   Workload("ragged_16x", S=1, T=131, H=128, K=8, E=64, R=16, Nmax=131),
                   WORKLOADS[2], WORKLOADS[5].with_(name="expand_quarter", S=4)]


@pytest.mark.parametrize("w", LAYOUT_DISPATCH, ids=lambda w: w.name)
def test_layout_dispatch_in_one_call(w):
    """ep_layout_dispatch (one kernel for one small source in the compact
    layout, the two calls' launches otherwise) gives the same tables, staging
    rows, records, receive rows and metadata as ep_layout + ep_dispatch, and
    the oracle's (edge lanes included)."""
    inputs = generate(w, 909, masked_frac=0.1, invalid_frac=0.02, dup_frac=0.2)
    dev = upload(w, inputs)
    say(f"[case] {w.name} ep_layout_dispatch")
    cfg = ep.config_for(w)
    L1, R1 = ep.alloc_layout(cfg), ep.alloc_recv(cfg)
    for t in L1.tables().values():
        t.fill_(-7)
    ep.ep_layout_dispatch(cfg, dev["x"], dev["x_sf"], dev["topk_idx"], dev["topk_weights"], L1, R1)
    L2, R2 = ep.alloc_layout(cfg), ep.alloc_recv(cfg)
    ep.ep_layout(cfg, dev["topk_idx"], L2)
    ep.ep_dispatch(cfg, dev["x"], dev["x_sf"], dev["topk_idx"], dev["topk_weights"], L2, R2)
    torch.cuda.synchronize()
    lay_o = oracle.layout(w.S, w.T, w.K, w.E, w.R, w.Nmax, inputs["topk_idx"], w.expand, w.alignment, w.n_out)
    compare_tables(layout_host(L1), lay_o)
    compare_tables(layout_host(L2), lay_o)
    want = oracle.dispatch(w.S, w.T, w.H, w.K, w.E, w.R, w.Nmax, w.dtype == "fp8", w.expand, w.alignment,
                           inputs["x"], inputs.get("x_sf"), inputs["topk_idx"], inputs["topk_weights"], lay_o, w.n_out)
    compare_dispatch(w, lay_o, R1, want)
    compare_dispatch(w, lay_o, R2, want)


@pytest.mark.parametrize("cfg_id", [2, 3, 5])
def test_identity_expert_round_trip(cfg_id):
    """dispatch -> identity expert -> combine gives bf16(sum(w) * x), any size."""
    w = WORKLOADS[cfg_id]
    inputs = generate(w, seed_for(cfg_id, 2))
    dev = upload(w, inputs)
    say(f"[case] {w.name} identity round trip")
    cfg, L = run_layout(w, dev)
    R = ep.alloc_recv(cfg)
    ep.ep_dispatch(cfg, dev["x"], dev["x_sf"], dev["topk_idx"], dev["topk_weights"], L, R)
    if w.dtype == "fp8":
        dec = R.recv_x.view(torch.float8_e4m3fn).float() * R.recv_sf.repeat_interleave(128, dim=1)
        y = dec.to(torch.bfloat16)
        xv = (dev["x"].view(torch.float8_e4m3fn).float() * dev["x_sf"].reshape(-1, w.H // 128)
              .repeat_interleave(128, dim=1)).to(torch.bfloat16).float()
    else:
        y = R.recv_x.view(torch.bfloat16)
        xv = dev["x"].view(torch.bfloat16).float()
    out = torch.empty((w.S * w.T, w.H), dtype=torch.bfloat16, device="cuda")
    ep.ep_combine(cfg, L, dev["topk_idx"], dev["topk_weights"], y, out)
    torch.cuda.synchronize()
    valid = (dev["topk_idx"] >= 0) & (dev["topk_idx"] < w.E)
    sw = (dev["topk_weights"] * valid).sum(dim=-1).reshape(-1, 1).double()
    want = (sw * xv.double())
    got = out.double()
    err = (got - want).abs()
    assert bool((err <= 1e-2 * want.abs() + 1e-5).all()), float(err.max())


GRAPH_CASES = [(WORKLOADS[1], False), (WORKLOADS[2], False), (WORKLOADS[2], True),
               (Workload("expand_a4_fp8_graph", S=3, T=70, H=128, K=4, E=16, R=4, Nmax=70, expand=True, alignment=4,
                         dtype="fp8"), False)]


@pytest.mark.parametrize("w,direct", GRAPH_CASES, ids=lambda c: getattr(c, "name", "direct" if c else "staging"))
def test_graph_replay_matches_eager(w, direct):
    """A step (layout, dispatch, combine) captured in a HIP graph and replayed
    several times, with eager work and synchronisation between the replays,
    gives the eager result every time (the library enqueues kernels only;
    the expand case covers the launches that request LDS to cap residency,
    the Direct Recv X case its pipelined scatter and metadata-only epilogue)."""
    inputs = generate(w, 4242)
    dev = upload(w, inputs)
    say(f"[case] {w.name} graph replay direct={direct}")
    cfg, L = run_layout(w, dev, direct=direct)
    R = ep.alloc_recv(cfg)
    rows = int(ep.ep_query_sizes(cfg).recv_rows)
    y = seeded_y(rows, w.H, 3)
    out = torch.empty((w.S * w.T, w.H), dtype=torch.bfloat16, device="cuda")

    def step(stream=None):
        ep.ep_layout(cfg, dev["topk_idx"], L, stream)
        ep.ep_dispatch(cfg, dev["x"], dev["x_sf"], dev["topk_idx"], dev["topk_weights"], L, R, ep.EP_PHASE_ALL, stream)
        ep.ep_combine(cfg, L, dev["topk_idx"], dev["topk_weights"], y, out, stream)

    step()
    torch.cuda.synchronize()
    n = int((L.expert_base if w.expand else L.recv_base)[-1].item())
    ref = (L.dst_slot.clone(), R.recv_x[:n].clone(), R.recv_topk_weights[:n].clone(), out.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step(s)  # warm the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step(s)
    torch.cuda.synchronize()
    for rep in range(3):
        L.dst_slot.fill_(-7)
        R.recv_x.zero_()
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (L.dst_slot, R.recv_x[:n], R.recv_topk_weights[:n], out)
        for a_, b_ in zip(got, ref):
            assert torch.equal(a_, b_), f"replay {rep} differs from the eager step"


def _random_workload(rng):
    R = int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
    El = int(rng.choice([1, 2, 3, 4, 8]))
    K = int(rng.integers(1, 9))
    El = max(El, -(-K // R))  # distinct experts per token need K <= E
    n_out = int(rng.choice([1, 1, 2, 3]))
    S = n_out * int(rng.integers(1, 4))
    T = int(rng.integers(0, 200))
    dtype = "fp8" if rng.random() < 0.3 else "bf16"
    # row sizes that reach every chunks-per-lane instantiation below the full-size workloads' (1, 2, 4, 7)
    H = int(rng.choice([128, 256, 384, 1152])) if dtype == "fp8" else int(rng.choice([8, 64, 136, 512, 1024, 1032,
                                                                                         3072]))
    expand = bool(rng.random() < 0.3)
    return Workload(f"rand", S=S, T=T, H=H, K=K, E=R * El, R=R, Nmax=T + int(rng.integers(0, 5)), dtype=dtype,
                    expand=expand, alignment=int(rng.choice([1, 2, 8])) if expand else 1, n_out=n_out)


@pytest.mark.parametrize("seed", range(60))
def test_random_small_configurations(seed):
    """Random shapes, dtypes, layouts, topologies and edge lanes against the oracle."""
    rng = np.random.default_rng(9000 + seed)
    w = _random_workload(rng)
    direct = (not w.expand) and rng.random() < 0.4
    edge = dict(masked_frac=float(rng.random() * 0.3), invalid_frac=float(rng.random() * 0.05),
                dup_frac=float(rng.random() * 0.4))
    _full_case(w, 100 + seed, edge, num_layout_cus=int(rng.choice([0, 0, 1, 5])), direct=direct)


MAX_CASES = [
    Workload("h_max_bf16", S=1, T=16, H=262144, K=2, E=8, R=4, Nmax=16),        # 512 KiB rows
    Workload("h_max_fp8", S=2, T=8, H=262144, K=3, E=12, R=4, Nmax=9, dtype="fp8"),  # 256 KiB rows + 2048 scales
    Workload("h_max_expand", S=1, T=8, H=262144, K=2, E=8, R=4, Nmax=8, expand=True, alignment=3),
    Workload("s_max", S=65535, T=1, H=8, K=1, E=2, R=2, Nmax=1),                # layout grid y = 65535
]


@pytest.mark.parametrize("w", MAX_CASES, ids=lambda w: w.name)
def test_maximum_sizes(w):
    """The largest hidden size (H = 262144) in both layouts and dtypes, and the
    largest number of sources (S = 65535, receiver tables far beyond LDS)."""
    _full_case(w, 4321, dict(masked_frac=0.1, dup_frac=0.2))


@pytest.mark.parametrize("mode", ["staging", "direct", "expand"])
def test_grid_stride_loops(mode):
    """4.5 M tokens of 16-byte rows at top-2: about 8.5 M receive rows, more work
    units than the 2^20-workgroup grids hold, so every kernel's grid-stride
    loop (scatter, copy epilogue and its pipelined next-row path, metadata-only
    and expand epilogues, combine) runs more than one iteration."""
    w = Workload(f"many_rows_{mode}", S=1, T=4_500_000, H=8, K=2, E=2, R=2, Nmax=4_500_000, expand=mode == "expand")
    _full_case(w, 99, dict(masked_frac=0.05), direct=mode == "direct")


def _random_large_workload(rng):
    """Larger random shapes: up to 3000 tokens per source, H up to 7168, up to
    64 ranks and 1024 experts, staging kept under 4 GiB."""
    while True:
        R = int(rng.choice([1, 2, 8, 16, 32, 64]))
        El = int(rng.choice([1, 2, 4, 8, 16]))
        if R * El > 1024:
            continue
        K = int(rng.integers(1, min(8, R * El) + 1))
        n_out = int(rng.choice([1, 1, 2]))
        S = n_out * int(rng.choice([1, 2]))
        T = int(rng.integers(0, 3001))
        dtype = "fp8" if rng.random() < 0.3 else "bf16"
        H = int(rng.choice([1024, 7168])) if dtype == "fp8" else int(rng.choice([128, 1024, 2048, 4096, 7168]))
        expand = bool(rng.random() < 0.3)
        Nmax = T + int(rng.integers(0, 9))
        if R * S * Nmax * (H if dtype == "fp8" else 2 * H) <= 4 << 30:
            return Workload("rand_large", S=S, T=T, H=H, K=K, E=R * El, R=R, Nmax=Nmax, dtype=dtype, expand=expand,
                            alignment=int(rng.choice([1, 4, 128])) if expand else 1, n_out=n_out)


@pytest.mark.parametrize("seed", range(8))
def test_random_large_configurations(seed):
    """Random larger shapes (layouts, fp8, hybrid, Direct Recv X, edge lanes,
    layout workgroup counts up to 300) against the oracle."""
    rng = np.random.default_rng(77000 + seed)
    w = _random_large_workload(rng)
    direct = (not w.expand) and rng.random() < 0.4
    edge = dict(masked_frac=float(rng.random() * 0.2), invalid_frac=float(rng.random() * 0.02),
                dup_frac=float(rng.random() * 0.2))
    _full_case(w, 500 + seed, edge, num_layout_cus=int(rng.choice([0, 0, 7, 300])), direct=direct)


def test_readme_example_runs():
    """The Python example in README.md, executed as written: with an identity
    expert the combine returns bf16(sum_k w_k * x) = x up to rounding."""
    import re

    text = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")).read()
    code = re.search(r"```python\n(.*?)```", text, flags=re.S).group(1)
    say("[case] README example")
    env = {}
    exec(compile(code, "README.md", "exec"), env)
    torch.cuda.synchronize()
    x, out, w = env["x"].float(), env["out"].float(), env["topk_w"]
    want = x * w.sum(-1).reshape(-1, 1)
    assert torch.allclose(out, want, rtol=1e-2, atol=1e-2)


def test_plain_c_example_runs():
    """combine_ep_layout_07_amd/examples/ep_example.c: the ABI driven from C11
    with hipMalloc'd buffers (built by build()); it checks its own results."""
    import subprocess

    from combine_ep_layout_07_amd import _build

    assert os.path.exists(_build.EXAMPLE_BIN), "the C example is not built; run __graft_entry__.build()"
    say("[case] plain C example")
    r = subprocess.run([_build.EXAMPLE_BIN], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ep_example: ok" in r.stdout


def test_two_streams_with_disjoint_buffers():
    """Calls on different streams with disjoint buffers may run concurrently:
    two workloads enqueued alternately on two streams (default priority) give
    the same results as the same steps run one after the other."""
    cases = [WORKLOADS[3], WORKLOADS[5].with_(name="expand_quarter", S=4)]
    setups = []
    for w in cases:
        inputs = generate(w, seed_for(2, 9))
        dev = upload(w, inputs)
        cfg, L = run_layout(w, dev)
        R = ep.alloc_recv(cfg)
        rows = int(ep.ep_query_sizes(cfg).recv_rows)
        y = seeded_y(rows, w.H, 5)
        out = torch.empty((w.S * w.T, w.H), dtype=torch.bfloat16, device="cuda")
        setups.append((w, dev, cfg, L, R, y, out))

    def step(setup, stream):
        w, dev, cfg, L, R, y, out = setup
        ep.ep_layout(cfg, dev["topk_idx"], L, stream)
        ep.ep_dispatch(cfg, dev["x"], dev["x_sf"], dev["topk_idx"], dev["topk_weights"], L, R, ep.EP_PHASE_ALL,
                       stream)
        ep.ep_combine(cfg, L, dev["topk_idx"], dev["topk_weights"], y, out, stream)

    def snapshot(setup):
        w, dev, cfg, L, R, y, out = setup
        n = int(L.recv_base[-1].item()) if not w.expand else int(L.expert_base[-1].item())
        return [L.dst_slot.clone(), R.recv_x[:n].clone(), R.recv_src_idx[:n].clone(), out.clone()]

    say("[case] two streams, serial reference")
    for st in setups:
        step(st, torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [snapshot(st) for st in setups]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in setups:
        st[4].recv_x.zero_()
        st[6].zero_()
    torch.cuda.synchronize()
    say("[case] two streams, interleaved")
    for _ in range(3):
        for st, stream in zip(setups, streams):
            step(st, stream)
    torch.cuda.synchronize()
    for st, want in zip(setups, ref):
        for a_, b_ in zip(snapshot(st), want):
            assert torch.equal(a_, b_), f"{st[0].name}: concurrent result differs from the serial one"
