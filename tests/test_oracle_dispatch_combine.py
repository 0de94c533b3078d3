"""Pins of the oracle's scatter, copy epilogue and combine.

Rows are checked against the inputs at the positions the layout fixes (bytes of
x, scales, metadata), the receive order against a sort by global source token
index (the order the pages' post-hoc deterministic sort produced), and combine
against exact rational arithmetic, one-hot and dyadic weights, and the
identity-expert round trip (dispatch, identity expert, combine gives
sum(w) * x).
"""
import numpy as np
import pytest
import torch

import oracle
from combine_ep_layout_07_amd.workloads import WORKLOADS, Workload, draw_expert_outputs, generate, seed_for
from tests.brute import (bf16_bits_to_fraction, check_dispatch, combine_rows_for_token, exact_combine_row,
                         f32_to_fraction, fraction_to_bf16_bits)

SMALL = [
    Workload("s1", S=1, T=37, H=64, K=4, E=16, R=4, Nmax=40),
    Workload("s2", S=3, T=29, H=128, K=3, E=12, R=6, Nmax=29, expand=True),
    Workload("s3", S=2, T=31, H=256, K=5, E=20, R=5, Nmax=33, dtype="fp8"),
    Workload("s4", S=2, T=23, H=128, K=4, E=16, R=4, Nmax=23, expand=True, alignment=4, dtype="fp8"),
    Workload("s5", S=1, T=0, H=64, K=2, E=4, R=2, Nmax=0),
]


def _run(w, seed, **edge):
    d = generate(w, seed, **edge)
    lay = oracle.layout(w.S, w.T, w.K, w.E, w.R, w.Nmax, d["topk_idx"], w.expand, w.alignment)
    disp = oracle.dispatch(w.S, w.T, w.H, w.K, w.E, w.R, w.Nmax, w.dtype == "fp8", w.expand, w.alignment,
                           d["x"], d.get("x_sf"), d["topk_idx"], d["topk_weights"], lay)
    return d, lay, disp


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
@pytest.mark.parametrize("edge", [{}, dict(masked_frac=0.2, invalid_frac=0.05, dup_frac=0.3)],
                         ids=["clean", "edge_lanes"])
def test_dispatch_rows_match_inputs(w, edge):
    d, lay, disp = _run(w, 42, **edge)
    check_dispatch(w.S, w.T, w.H, w.K, w.E, w.R, w.Nmax, w.dtype == "fp8", w.expand, w.alignment, d, lay, disp)


def test_dispatch_tiny_workload():
    w = WORKLOADS[1]
    d, lay, disp = _run(w, seed_for(1))
    check_dispatch(w.S, w.T, w.H, w.K, w.E, w.R, w.Nmax, False, False, 1, d, lay, disp)


def test_each_deduplicated_entry_placed_once():
    w = SMALL[0]
    d, lay, disp = _run(w, 9, dup_frac=0.5)
    n = int(lay["recv_base"][-1])
    src = disp["recv_src_idx"][:n]
    El = w.E // w.R
    pairs = set()
    for i, g in enumerate(src):
        dd = int(np.searchsorted(lay["recv_base"], i, side="right") - 1)
        assert (g, dd) not in pairs
        pairs.add((g, dd))
    topk = d["topk_idx"].reshape(-1, w.K)
    want = {(g, int(e) // El) for g in range(w.S * w.T) for e in topk[g] if 0 <= e < w.E}
    assert pairs == want


# ---------------------------------------------------------------- combine

def _combine(w, d, lay, y):
    return oracle.combine(w.S, w.T, w.H, w.K, w.E, w.R, w.Nmax, w.expand, d["topk_idx"], d["topk_weights"], lay, y)


@pytest.mark.parametrize("w", SMALL[:4], ids=lambda w: w.name)
def test_combine_exact_rational(w):
    d, lay, disp = _run(w, 5, masked_frac=0.1, dup_frac=0.3)
    rows = oracle.recv_rows(w.S, w.T, w.K, w.E, w.R, lay, w.expand)
    H = 32
    w2 = w.with_(H=H, dtype="bf16")
    y = draw_expert_outputs(max(rows, 1), H, 77)
    out = _combine(w2, d, lay, y)
    for s in range(w.S):
        for t in range(w.T):
            pairs = combine_rows_for_token(w.S, w.T, w.K, w.E, w.R, w.Nmax, d["topk_idx"], lay, s, t, w.expand)
            want = exact_combine_row([y[r] for r, _ in pairs], [d["topk_weights"][s, t, k] for _, k in pairs]) \
                if pairs else np.zeros(H, np.uint16)
            assert (out[s, t] == want).all(), f"token ({s},{t})"


@pytest.mark.parametrize("w", [SMALL[0], SMALL[1]], ids=lambda w: w.name)
@pytest.mark.parametrize("nb", [1, 2])
def test_combine_bias_exact_rational(w, nb):
    """Bias rows are added to the reduced sum before the single rounding."""
    from fractions import Fraction
    d, lay, disp = _run(w, 13, masked_frac=0.2, dup_frac=0.2)
    rows = oracle.recv_rows(w.S, w.T, w.K, w.E, w.R, lay, w.expand)
    H = 24
    y = draw_expert_outputs(max(rows, 1), H, 31)
    biases = [draw_expert_outputs(w.S * w.T, H, 40 + i).reshape(w.S, w.T, H) for i in range(nb)]
    out = oracle.combine_bias(w.S, w.T, H, w.K, w.E, w.R, w.Nmax, w.expand, d["topk_idx"], d["topk_weights"],
                              lay, y, biases[0], biases[1] if nb > 1 else None)
    for s in range(w.S):
        for t in range(w.T):
            pairs = combine_rows_for_token(w.S, w.T, w.K, w.E, w.R, w.Nmax, d["topk_idx"], lay, s, t, w.expand)
            want = []
            for h in range(H):
                acc = sum((f32_to_fraction(d["topk_weights"][s, t, k]) * bf16_bits_to_fraction(int(y[r, h]))
                           for r, k in pairs), Fraction(0))
                acc += sum((bf16_bits_to_fraction(int(bb[s, t, h])) for bb in biases), Fraction(0))
                want.append(fraction_to_bf16_bits(acc))
            assert (out[s, t] == np.array(want, np.uint16)).all(), f"token ({s},{t})"


def test_combine_bias_alone_when_no_lane_is_valid():
    w = Workload("nb", S=1, T=5, H=16, K=2, E=4, R=2, Nmax=5)
    topk = np.full((1, 5, 2), -1, np.int64)
    wts = np.full((1, 5, 2), 0.5, np.float32)
    lay = oracle.layout(1, 5, 2, 4, 2, 5, topk)
    y = draw_expert_outputs(1, 16, 1)
    b0 = draw_expert_outputs(5, 16, 2).reshape(1, 5, 16)
    b1 = draw_expert_outputs(5, 16, 3).reshape(1, 5, 16)
    out = oracle.combine_bias(1, 5, 16, 2, 4, 2, 5, False, topk, wts, lay, y, b0, b1)
    f0 = torch.from_numpy(b0.view(np.int16).copy()).view(torch.bfloat16).double()
    f1 = torch.from_numpy(b1.view(np.int16).copy()).view(torch.bfloat16).double()
    want = (f0 + f1).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)  # b0+b1 exact in fp32
    assert (out == want).all()
    assert (oracle.combine_bias(1, 5, 16, 2, 4, 2, 5, False, topk, wts, lay, y, b0, None) == b0).all()


def test_combine_one_hot_returns_row_bitwise():
    w = Workload("oh", S=2, T=20, H=64, K=4, E=16, R=4, Nmax=20, expand=False)
    rng = np.random.default_rng(1)
    topk = np.full((w.S, w.T, w.K), -1, np.int64)
    hot = rng.integers(0, w.K, size=(w.S, w.T))
    for s in range(w.S):
        for t in range(w.T):
            topk[s, t, hot[s, t]] = rng.integers(0, w.E)
    wts = np.zeros((w.S, w.T, w.K), np.float32)
    for s in range(w.S):
        for t in range(w.T):
            wts[s, t, hot[s, t]] = 1.0
    d = dict(topk_idx=topk, topk_weights=wts)
    for expand in (False, True):
        ww = w.with_(expand=expand)
        lay = oracle.layout(w.S, w.T, w.K, w.E, w.R, w.Nmax, topk, expand, 1)
        rows = oracle.recv_rows(w.S, w.T, w.K, w.E, w.R, lay, expand)
        y = draw_expert_outputs(rows, w.H, 3)
        out = _combine(ww, d, lay, y)
        for s in range(w.S):
            for t in range(w.T):
                (r, _), = combine_rows_for_token(w.S, w.T, w.K, w.E, w.R, w.Nmax, topk, lay, s, t, expand)
                assert (out[s, t] == y[r]).all()


def test_combine_dyadic_weights_exact():
    # weights 1/2, 1/4, 1/8, 1/8 on small-integer rows: every sum is exact in
    # bf16, so the result is known without rounding.
    w = Workload("dy", S=1, T=16, H=32, K=4, E=8, R=8, Nmax=16)
    rng = np.random.default_rng(2)
    topk = np.stack([rng.permutation(w.E)[: w.K] for _ in range(w.T)])[None].astype(np.int64)
    wts = np.tile(np.array([0.5, 0.25, 0.125, 0.125], np.float32), (1, w.T, 1))
    lay = oracle.layout(w.S, w.T, w.K, w.E, w.R, w.Nmax, topk)
    rows = int(lay["recv_base"][-1])
    yi = rng.integers(-8, 9, size=(rows, w.H)).astype(np.float32)
    y = torch.from_numpy(yi).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    out = _combine(w, dict(topk_idx=topk, topk_weights=wts), lay, y)
    for t in range(w.T):
        pairs = combine_rows_for_token(w.S, w.T, w.K, w.E, w.R, w.Nmax, topk, lay, 0, t, False)
        exact = sum(float(wts[0, t, k]) * yi[r] for r, k in pairs)
        want = torch.from_numpy(np.asarray(exact, np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
        assert (out[0, t].view(np.int16) == want).all()


def test_combine_token_without_valid_lane_is_positive_zero():
    w = Workload("z", S=1, T=6, H=16, K=3, E=6, R=3, Nmax=6)
    topk = np.array([[[-1, -1, -1], [0, 7, -1], [6, 6, 6], [1, -1, 2], [-5, -1, 9], [5, 4, 3]]], np.int64)
    wts = np.full((1, 6, 3), 0.3, np.float32)
    lay = oracle.layout(1, 6, 3, 6, 3, 6, topk)
    y = draw_expert_outputs(int(lay["recv_base"][-1]), 16, 4)
    out = _combine(w, dict(topk_idx=topk, topk_weights=wts), lay, y)
    for t in (0, 2, 4):
        assert (out[0, t] == 0).all()
    assert lay["error_flags"][0] == 1


@pytest.mark.parametrize("w", [SMALL[0], SMALL[1], SMALL[2], SMALL[3]], ids=lambda w: w.name)
def test_identity_expert_round_trip(w):
    """dispatch -> identity expert -> combine returns bf16(sum(w) * x)."""
    d, lay, disp = _run(w, 21, masked_frac=0.1, dup_frac=0.2)
    rows = oracle.recv_rows(w.S, w.T, w.K, w.E, w.R, lay, w.expand)
    if w.dtype == "fp8":
        dec = torch.from_numpy(disp["recv_x"].copy()).view(torch.float8_e4m3fn).float()
        scale = torch.from_numpy(disp["recv_sf"]).repeat_interleave(128, dim=1)
        y = (dec * scale).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        xv = torch.from_numpy(d["x"].reshape(-1, w.H).copy()).view(torch.float8_e4m3fn).double() \
            * torch.from_numpy(d["x_sf"].reshape(-1, w.H // 128)).double().repeat_interleave(128, dim=1)
        xv = torch.from_numpy(xv.float().to(torch.bfloat16).float().numpy()).double()
    else:
        y = disp["recv_x"].view(np.uint16).reshape(rows, w.H)
        xv = torch.from_numpy(d["x"].reshape(-1, w.H * 2).copy()).view(torch.bfloat16).double()
    out = _combine(w.with_(dtype="bf16"), d, lay, y)
    topk = d["topk_idx"].reshape(-1, w.K)
    valid = (topk >= 0) & (topk < w.E)
    sw = torch.from_numpy((d["topk_weights"].reshape(-1, w.K).astype(np.float64) * valid).sum(axis=1))
    want = (sw[:, None] * xv).float()
    got = torch.from_numpy(out.reshape(-1, w.H).view(np.int16).copy()).view(torch.bfloat16).float()
    # sum of lanes vs sum of weights times the row: equal up to one bf16 rounding
    assert torch.allclose(got, want, rtol=2 ** -7, atol=1e-6)
    exact_share = (got == want.to(torch.bfloat16).float()).float().mean().item()
    assert exact_share > 0.98


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_rounding_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    vals = np.concatenate([rng.standard_normal(3000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 3000),
                           np.array([0.0, -0.0, 1.0, -2.5, 3.0e38, 1e-40, -1e-42], np.float32)])
    want = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_from_double(float(v)) for v in vals], np.uint16)
    assert (got == want).all()


def test_bf16_rounding_exact_rational_ties_and_limits():
    from fractions import Fraction
    cases = []
    one = Fraction(1)
    q = Fraction(1, 128)
    cases += [one + q / 2, one + 3 * q / 2, one + q / 2 + Fraction(1, 2 ** 40), -(one + q / 2)]
    max_bf16 = (2 - Fraction(1, 128)) * Fraction(2) ** 127  # 0x7F7F, the largest finite bf16
    cases += [max_bf16, max_bf16 + Fraction(2) ** 119 - Fraction(2) ** 80]
    cases += [Fraction(2) ** -133, Fraction(3, 2) * Fraction(2) ** -133, Fraction(2) ** -127 * Fraction(255, 128)]
    for c in cases:
        assert oracle.bf16_from_double(float(c)) == fraction_to_bf16_bits(Fraction(float(c)))
    # just past the largest finite bf16 by half a unit -> +inf; NaN stays NaN
    assert oracle.bf16_from_double(float(max_bf16 + Fraction(2) ** 119)) == 0x7F80
    assert oracle.bf16_from_double(float("nan")) & 0x7FC0 == 0x7FC0
    assert oracle.bf16_from_double(float("-inf")) == 0xFF80
    assert bf16_bits_to_fraction(0x3F80) == 1 and f32_to_fraction(np.float32(0.5)) == Fraction(1, 2)


@pytest.mark.parametrize("expand", [False, True])
def test_hybrid_dispatch_rows_and_combine(expand):
    """Hybrid row form: staging rows sit at segment = scale-up index, offset =
    scale-out index * Nmax + slot; the receive rows and combine are unchanged."""
    w = Workload("hyb", S=6, T=25, H=64, K=4, E=24, R=6, Nmax=27, n_out=2, expand=expand, alignment=2)
    d = generate(w, 8, masked_frac=0.1, dup_frac=0.3)
    lay = oracle.layout(w.S, w.T, w.K, w.E, w.R, w.Nmax, d["topk_idx"], expand, 2, 2)
    disp = oracle.dispatch(w.S, w.T, w.H, w.K, w.E, w.R, w.Nmax, False, expand, 2, d["x"], None, d["topk_idx"],
                           d["topk_weights"], lay, 2)
    check_dispatch(w.S, w.T, w.H, w.K, w.E, w.R, w.Nmax, False, expand, 2, d, lay, disp, n_out=2)
    dlay = oracle.layout(w.S, w.T, w.K, w.E, w.R, w.Nmax, d["topk_idx"], expand, 2)
    ddisp = oracle.dispatch(w.S, w.T, w.H, w.K, w.E, w.R, w.Nmax, False, expand, 2, d["x"], None, d["topk_idx"],
                            d["topk_weights"], dlay)
    rows = oracle.recv_rows(w.S, w.T, w.K, w.E, w.R, lay, expand)
    assert (disp["recv_x"][:rows] == ddisp["recv_x"][:rows]).all()
    assert (disp["recv_src_idx"][:rows] == ddisp["recv_src_idx"][:rows]).all()
    y = draw_expert_outputs(rows, w.H, 3)
    a = oracle.combine(w.S, w.T, w.H, w.K, w.E, w.R, w.Nmax, expand, d["topk_idx"], d["topk_weights"], lay, y, 2)
    b = oracle.combine(w.S, w.T, w.H, w.K, w.E, w.R, w.Nmax, expand, d["topk_idx"], d["topk_weights"], dlay, y)
    assert (a == b).all()


def combine_tokens_pin(w, seed):
    """oracle.combine_tokens against the exact rational combine of each selected
    token, and bitwise against the rows of the full oracle.combine it samples.

    The selection is unsorted, repeats tokens and includes a token with no
    valid lane (its row is +0); a selected index g names token (s, t) with
    g = s*T + t (the global source token index)."""
    d = generate(w, seed, masked_frac=0.2, dup_frac=0.3)
    topk = d["topk_idx"].copy()
    topk[w.S - 1, min(1, w.T - 1), :] = -1  # a token with no valid lane
    lay = oracle.layout(w.S, w.T, w.K, w.E, w.R, w.Nmax, topk, w.expand, w.alignment, w.n_out)
    rows = oracle.recv_rows(w.S, w.T, w.K, w.E, w.R, lay, w.expand)
    H = 16
    y = draw_expert_outputs(max(rows, 1), H, seed + 1)
    n = w.S * w.T
    rng = np.random.default_rng(seed)
    empty_tok = (w.S - 1) * w.T + min(1, w.T - 1)
    sel = np.concatenate([rng.permutation(n)[: max(1, n // 2)], rng.integers(0, n, 5), [empty_tok, n - 1, 0]])
    got = oracle.combine_tokens(w.S, w.T, H, w.K, w.E, w.R, w.Nmax, w.expand, topk, d["topk_weights"], lay, y, sel,
                                w.n_out)
    assert got.shape == (sel.size, H)
    for i, g in enumerate(sel):
        s, t = divmod(int(g), w.T)
        pairs = combine_rows_for_token(w.S, w.T, w.K, w.E, w.R, w.Nmax, topk, lay, s, t, w.expand, w.n_out)
        want = exact_combine_row([y[r] for r, _ in pairs], [d["topk_weights"][s, t, k] for _, k in pairs]) \
            if pairs else np.zeros(H, np.uint16)
        assert (got[i] == want).all(), f"combine_tokens row {i} (token {g} = ({s}, {t})) differs"
    assert (got[sel == empty_tok] == 0).all()
    full = oracle.combine(w.S, w.T, H, w.K, w.E, w.R, w.Nmax, w.expand, topk, d["topk_weights"], lay, y,
                          w.n_out).reshape(n, H)
    assert (got == full[sel]).all()


COMBINE_TOKENS_CASES = [
    Workload("ct_direct", S=3, T=19, H=16, K=4, E=16, R=4, Nmax=21),
    Workload("ct_hybrid", S=6, T=11, H=16, K=3, E=12, R=6, Nmax=12, n_out=2),
    Workload("ct_hybrid3", S=6, T=7, H=16, K=4, E=16, R=4, Nmax=7, n_out=3),
    Workload("ct_expand", S=2, T=17, H=16, K=3, E=12, R=6, Nmax=17, expand=True, alignment=4),
    Workload("ct_expand_hybrid", S=4, T=9, H=16, K=4, E=16, R=4, Nmax=9, expand=True, alignment=2, n_out=2),
]


@pytest.mark.parametrize("w", COMBINE_TOKENS_CASES, ids=lambda w: w.name)
def test_combine_tokens_matches_exact_and_full_combine(w):
    combine_tokens_pin(w, 1234)


def test_combine_tokens_edge_arguments():
    w = COMBINE_TOKENS_CASES[0]
    d = generate(w, 3)
    lay = oracle.layout(w.S, w.T, w.K, w.E, w.R, w.Nmax, d["topk_idx"])
    y = draw_expert_outputs(int(lay["recv_base"][-1]), 8, 2)
    empty = oracle.combine_tokens(w.S, w.T, 8, w.K, w.E, w.R, w.Nmax, False, d["topk_idx"], d["topk_weights"], lay,
                                  y, np.zeros(0, np.int64))
    assert empty.shape == (0, 8)
    for bad in (-1, w.S * w.T):
        with pytest.raises(ValueError):
            oracle.combine_tokens(w.S, w.T, 8, w.K, w.E, w.R, w.Nmax, False, d["topk_idx"], d["topk_weights"], lay,
                                  y, np.array([0, bad], np.int64))
