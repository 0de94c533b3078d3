"""Independent characterisations of the dispatch layout, dispatch and combine.

These pin the CPU oracle to something other than itself:

* ``brute_layout`` restates each definition as an O(T^2) count over Python
  lists (no running counters, no prefix arrays);
* ``sorted_layout`` derives the same tables from a stable sort (numpy
  ``argsort(kind="stable")``): a destination's slots are the token order of the
  senders, and an expert's expand rows are the lex order of its lanes;
* ``check_dispatch`` / ``check_combine_*`` check the oracle's rows against the
  inputs directly (bytes of x at the mapped position, exact rational sums).

Sources: DeepEP v2 "Kernel-side deterministic dispatch for the non-expand
layout" (PR #753, sections Motivation, Approach, Direct vs hybrid dispatch,
Compatibility) and "Add experimental direct recv_x dispatch path" (PR #690,
sections Background and Direct Recv X design).
"""
from __future__ import annotations

from fractions import Fraction
from typing import Dict

import numpy as np


def _valid(e, E):
    return 0 <= e < E


def token_dests(topk, s, t, K, E, El):
    return {int(topk[s, t, k]) // El for k in range(K) if _valid(int(topk[s, t, k]), E)}


def row_base(s, S, n_out):
    """Row base of source s: s on the direct path, its scale-out index s // n_up on the hybrid path."""
    return s // (S // n_out) if n_out > 1 else s


def staging_region(d, s, S, n_out):
    """Region of source s in destination d's staging buffer: d*S + s on the direct
    path; on the hybrid path segment = scale-up index, then the scale-out index."""
    if n_out > 1:
        n_up = S // n_out
        return (d * n_up + s % n_up) * n_out + s // n_up
    return d * S + s


def brute_layout(S, T, K, E, R, Nmax, topk, expand=False, A=1, n_out=1) -> Dict[str, np.ndarray]:
    """Each output restated literally, by counting (O(T^2), tiny sizes only)."""
    El = E // R
    topk = np.asarray(topk).reshape(S, T, K)
    dst_slot = np.full((S, T, K), -1, np.int64)
    for s in range(S):
        for t in range(T):
            for k in range(K):
                e = int(topk[s, t, k])
                if not _valid(e, E):
                    continue
                d = e // El
                if any(_valid(int(topk[s, t, k2]), E) and int(topk[s, t, k2]) // El == d for k2 in range(k)):
                    continue  # a lower lane already carries this destination
                earlier = sum(1 for t2 in range(t) if d in token_dests(topk, s, t2, K, E, El))
                dst_slot[s, t, k] = row_base(s, S, n_out) * Nmax + earlier
    tpr = np.array([[sum(1 for t in range(T) if d in token_dests(topk, s, t, K, E, El)) for d in range(R)]
                    for s in range(S)], np.int64).reshape(S, R)
    tpe = np.array([[sum(1 for t in range(T) for k in range(K) if int(topk[s, t, k]) == e) for e in range(E)]
                    for s in range(S)], np.int64).reshape(S, E)
    recv_psum = np.array([[sum(tpr[s2, d] for s2 in range(s)) for s in range(S + 1)] for d in range(R)],
                         np.int64)
    recv_base = np.array([sum(tpr[s, d2] for s in range(S) for d2 in range(d)) for d in range(R + 1)], np.int64)
    out = dict(dst_slot=dst_slot, tokens_per_rank=tpr, tokens_per_expert=tpe, recv_psum=recv_psum,
               recv_base=recv_base, error_flags=np.array([1 if (topk >= E).any() else 0]))
    if n_out > 1:
        n_up = S // n_out
        out["recv_psum_scaleup"] = np.array(
            [[sum(tpr[s2, d] for s2 in range(S) if s2 % n_up < u) for u in range(n_up + 1)] for d in range(R)],
            np.int64)
    if expand:
        cnt = [int(tpe[:, e].sum()) for e in range(E)]
        expert_base = np.array([sum(-(-cnt[e2] // A) * A for e2 in range(e)) for e in range(E + 1)], np.int64)
        pos = np.full((S, T, K), -1, np.int64)
        lanes = [(s, t, k) for s in range(S) for t in range(T) for k in range(K)]
        for idx, (s, t, k) in enumerate(lanes):
            e = int(topk[s, t, k])
            if not _valid(e, E):
                continue
            before = sum(1 for (s2, t2, k2) in lanes[:idx] if int(topk[s2, t2, k2]) == e)
            pos[s, t, k] = expert_base[e] + before
        out["expert_base"] = expert_base
        out["expand_pos"] = pos
    return out


def sorted_layout(S, T, K, E, R, Nmax, topk, expand=False, A=1, n_out=1) -> Dict[str, np.ndarray]:
    """The same tables from stable sorts and bincounts (vectorised numpy)."""
    El = E // R
    topk = np.asarray(topk, np.int64).reshape(S, T, K)
    valid = (topk >= 0) & (topk < E)
    rank = np.where(valid, topk // El, -1)
    # owner: first occurrence of a rank among the token's lanes
    owner = np.zeros_like(valid)
    for k in range(K):
        prev = np.zeros(valid.shape[:2], bool)
        for k2 in range(k):
            prev |= valid[:, :, k2] & (rank[:, :, k2] == rank[:, :, k])
        owner[:, :, k] = valid[:, :, k] & ~prev
    s_idx, t_idx, k_idx = np.nonzero(owner)           # C order: ascending (s, t, k)
    d_idx = rank[s_idx, t_idx, k_idx]
    order = np.argsort(s_idx * R + d_idx, kind="stable")   # groups (s, d), t ascending inside
    group = (s_idx * R + d_idx)[order]
    start = np.searchsorted(group, group, side="left")
    pos_in_group = np.arange(group.size) - start
    dst_slot = np.full((S, T, K), -1, np.int64)
    base = np.array([row_base(s, S, n_out) for s in range(S)], np.int64)
    dst_slot[s_idx[order], t_idx[order], k_idx[order]] = base[s_idx[order]] * Nmax + pos_in_group
    tpr = np.bincount(s_idx * R + d_idx, minlength=S * R).reshape(S, R)
    vs, vt, vk = np.nonzero(valid)
    tpe = np.bincount(vs * E + topk[vs, vt, vk], minlength=S * E).reshape(S, E)
    recv_psum = np.zeros((R, S + 1), np.int64)
    recv_psum[:, 1:] = np.cumsum(tpr.T, axis=1)
    recv_base = np.zeros(R + 1, np.int64)
    recv_base[1:] = np.cumsum(tpr.sum(axis=0))
    out = dict(dst_slot=dst_slot, tokens_per_rank=tpr, tokens_per_expert=tpe, recv_psum=recv_psum,
               recv_base=recv_base, error_flags=np.array([1 if (topk >= E).any() else 0]))
    if expand:
        cnt = tpe.sum(axis=0)
        padded = -(-cnt // A) * A
        expert_base = np.concatenate([[0], np.cumsum(padded)])
        ex = topk[vs, vt, vk]
        order = np.argsort(ex, kind="stable")
        exs = ex[order]
        start = np.searchsorted(exs, exs, side="left")
        pos = np.full((S, T, K), -1, np.int64)
        pos[vs[order], vt[order], vk[order]] = expert_base[exs] + (np.arange(exs.size) - start)
        out["expert_base"] = expert_base
        out["expand_pos"] = pos
    return out


def assert_tables_equal(got: Dict[str, np.ndarray], want: Dict[str, np.ndarray], keys=None):
    for key in keys or want.keys():
        g = np.asarray(got[key]).astype(np.int64).ravel()
        w = np.asarray(want[key]).astype(np.int64).ravel()
        assert g.shape == w.shape, f"{key}: shape {g.shape} != {w.shape}"
        bad = np.nonzero(g != w)[0]
        assert bad.size == 0, f"{key}: {bad.size} mismatches, first at {bad[0]}: got {g[bad[0]]} want {w[bad[0]]}"


def check_layout_invariants(S, T, K, E, R, Nmax, topk, lay, expand=False, A=1, n_out=1):
    """Properties that hold at any size (each one a statement of the pages)."""
    El = E // R
    topk = np.asarray(topk, np.int64).reshape(S, T, K)
    slot = np.asarray(lay["dst_slot"]).reshape(S, T, K).astype(np.int64)
    tpr = np.asarray(lay["tokens_per_rank"]).reshape(S, R).astype(np.int64)
    tpe = np.asarray(lay["tokens_per_expert"]).reshape(S, E).astype(np.int64)
    valid = (topk >= 0) & (topk < E)
    rank = np.where(valid, topk // El, -1)
    has = slot >= 0
    # only valid lanes carry slots; one slot per (token, destination)
    assert not (has & ~valid).any(), "a masked or invalid lane carries a slot"
    n_owner = has.sum()
    for d in range(R):
        per_tok = (has & (rank == d)).sum(axis=2)
        any_d = (valid & (rank == d)).any(axis=2)
        assert (per_tok == any_d.astype(int)).all(), f"destination {d}: not exactly one owner per token"
    assert n_owner == tpr.sum(), "sum of tokens_per_rank != number of owner lanes"
    # rows never overflow and are dense: per (s, d) the slots are s*Nmax + 0..count-1
    for s in range(S):
        for d in range(R):
            sl = np.sort(slot[s][has[s] & (rank[s] == d)])
            assert (sl == row_base(s, S, n_out) * Nmax + np.arange(tpr[s, d])).all(), f"(s={s}, d={d}) not dense"
            assert tpr[s, d] <= min(T, Nmax), "a row overflows Nmax"
            # ascending token order inside a row
            ts = np.nonzero((has[s] & (rank[s] == d)).any(axis=1))[0]
            ss = slot[s][has[s] & (rank[s] == d)]
            assert (np.diff(ss) > 0).all() and ts.size == ss.size
    # tokens_per_expert bounds tokens_per_rank
    for d in range(R):
        blk = tpe[:, d * El:(d + 1) * El]
        assert (blk.max(axis=1, initial=0) <= tpr[:, d]).all() and (tpr[:, d] <= blk.sum(axis=1)).all()
    rp = np.asarray(lay["recv_psum"]).reshape(R, S + 1).astype(np.int64)
    rb = np.asarray(lay["recv_base"]).reshape(R + 1).astype(np.int64)
    assert rp[:, S].sum() == n_owner and rb[R] == n_owner
    assert (rp[:, 0] == 0).all() and (np.diff(rp, axis=1) == tpr.T).all()
    assert (np.diff(rb) == rp[:, S]).all() and rb[0] == 0
    assert int(np.asarray(lay["error_flags"]).ravel()[0]) == int((topk >= E).any())
    if expand:
        eb = np.asarray(lay["expert_base"]).astype(np.int64)
        pos = np.asarray(lay["expand_pos"]).reshape(S, T, K).astype(np.int64)
        cnt = tpe.sum(axis=0)
        assert eb[0] == 0 and (np.diff(eb) == -(-cnt // A) * A).all()
        assert ((pos >= 0) == valid).all()
        p = pos[valid]
        assert np.unique(p).size == p.size, "two lanes share an expand row"
        for e in range(E):
            pe = pos[valid & (topk == e)]          # C order = ascending (s, t, k)
            assert (pe == eb[e] + np.arange(cnt[e])).all(), f"expert {e} rows not dense/ordered"


def check_dispatch(S, T, H, K, E, R, Nmax, is_fp8, expand, A, inputs, lay, disp, rows_to_check=None, n_out=1):
    """Staging and receive rows against the inputs at the positions the layout fixes."""
    El = E // R
    Rw = H if is_fp8 else 2 * H
    x = np.asarray(inputs["x"]).reshape(S, T, Rw)
    sf = np.asarray(inputs["x_sf"]).reshape(S, T, -1) if is_fp8 else None
    topk = np.asarray(inputs["topk_idx"]).reshape(S, T, K)
    w = np.asarray(inputs["topk_weights"]).reshape(S, T, K)
    slot = np.asarray(lay["dst_slot"]).reshape(S, T, K)
    tpr = np.asarray(lay["tokens_per_rank"]).reshape(S, R)
    rp = np.asarray(lay["recv_psum"]).reshape(R, S + 1)
    rb = np.asarray(lay["recv_base"]).reshape(R + 1)
    valid = (topk >= 0) & (topk < E)
    # staging: owner lane (s,t,k) -> row j = slot - row_base*Nmax of source s's region in destination d
    sx = disp["staging_x"].reshape(R * S, Nmax, disp["staging_x"].shape[-1])
    ssf = disp["staging_sf"].reshape(R * S, Nmax, disp["staging_sf"].shape[-1])
    smeta = disp["staging_meta"].reshape(R * S, Nmax, disp["staging_meta"].shape[-1])
    for s, t, k in zip(*np.nonzero(slot >= 0)):
        d = int(topk[s, t, k]) // El
        j = int(slot[s, t, k]) - row_base(s, S, n_out) * Nmax
        g = staging_region(d, s, S, n_out)
        assert (sx[g, j] == x[s, t]).all(), f"staging_x ({d},{s},{j}) != x[{s},{t}]"
        if is_fp8:
            assert (ssf[g, j] == sf[s, t]).all()
        meta = smeta[g, j]
        assert meta[0] == t
        assert (meta[1:1 + K] == np.where(valid[s, t], topk[s, t], -1)).all()
        assert (meta[1 + K:1 + 2 * K] == w[s, t].view(np.int32)).all()
    if not expand:
        for d in range(R):
            src = [s * T + t for s in range(S) for t in range(T)
                   if (valid[s, t] & (topk[s, t] // El == d)).any()]
            got = disp["recv_src_idx"][rb[d]:rb[d + 1]]
            assert list(got) == src, f"destination {d}: receive order is not ascending source token index"
            for s in range(S):
                assert rb[d] + rp[d, s] == rb[d] + sum(tpr[s2, d] for s2 in range(s))
        n = int(rb[R])
        for i in range(n) if rows_to_check is None else rows_to_check:
            g = int(disp["recv_src_idx"][i])
            s, t = divmod(g, T)
            d = int(np.searchsorted(rb, i, side="right") - 1)
            assert (disp["recv_x"][i] == x[s, t]).all(), f"recv_x[{i}] != x[{s},{t}]"
            if is_fp8:
                assert (disp["recv_sf"][i] == sf[s, t]).all()
            for k in range(K):
                on_d = valid[s, t, k] and int(topk[s, t, k]) // El == d
                assert disp["recv_topk_idx"][i, k] == (int(topk[s, t, k]) - d * El if on_d else -1)
                want = w[s, t, k] if on_d else np.float32(0.0)
                assert disp["recv_topk_weights"][i, k].view(np.int32) == np.float32(want).view(np.int32)
    else:
        eb = np.asarray(lay["expert_base"]).astype(np.int64)
        tpe = np.asarray(lay["tokens_per_expert"]).reshape(S, E)
        for e in range(E):
            lanes = [(s, t, k) for s in range(S) for t in range(T) for k in range(K) if topk[s, t, k] == e]
            seg_src = disp["recv_src_idx"][eb[e]:eb[e] + len(lanes)]
            assert list(seg_src) == [s * T + t for (s, t, k) in lanes], f"expert {e}: wrong expand order"
            for r, (s, t, k) in zip(range(eb[e], eb[e] + len(lanes)), lanes):
                assert (disp["recv_x"][r] == x[s, t]).all()
                if is_fp8:
                    assert (disp["recv_sf"][r] == sf[s, t]).all()
                assert disp["recv_topk_weights"][r].view(np.int32) == w[s, t, k].view(np.int32)
            assert int(tpe[:, e].sum()) == len(lanes)
            for r in range(eb[e] + len(lanes), eb[e + 1]):
                assert (disp["recv_x"][r] == 0).all() and disp["recv_src_idx"][r] == -1
                assert disp["recv_topk_weights"][r].view(np.int32) == 0


# --- exact arithmetic for combine -------------------------------------------------

def bf16_bits_to_fraction(b: int) -> Fraction:
    b &= 0xFFFF
    sign = -1 if b & 0x8000 else 1
    ex = (b >> 7) & 0xFF
    man = b & 0x7F
    assert ex != 0xFF, "no inf/nan in these inputs"
    if ex == 0:
        return sign * Fraction(man, 1 << 7) * Fraction(1, 1 << 126)
    return sign * (1 + Fraction(man, 1 << 7)) * (Fraction(2) ** (ex - 127))


def f32_to_fraction(v) -> Fraction:
    return Fraction(float(np.float32(v)))


def fraction_to_bf16_bits(q: Fraction) -> int:
    """Nearest bf16 to an exact rational, ties to even (finite inputs only)."""
    if q == 0:
        return 0
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 7)
    n_float = a / quantum
    n = n_float.numerator // n_float.denominator
    rem = n_float - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * quantum
    if val >= Fraction(2) ** 128:
        return sign | 0x7F80
    # encode val (a bf16 value) into bits
    if val < Fraction(2) ** -126:
        man = int(val / (Fraction(2) ** -133))
        return sign | man
    ex = val.numerator.bit_length() - val.denominator.bit_length()
    if Fraction(2) ** ex > val:
        ex -= 1
    man = int((val / (Fraction(2) ** ex) - 1) * 128)
    return sign | ((ex + 127) << 7) | man


def exact_combine_row(y_rows, weights):
    """bf16(sum_k w_k * y_k) with exact rational accumulation and one rounding."""
    H = len(y_rows[0]) if y_rows else 0
    out = []
    for h in range(H):
        acc = Fraction(0)
        for yr, wk in zip(y_rows, weights):
            acc += f32_to_fraction(wk) * bf16_bits_to_fraction(int(yr[h]))
        out.append(fraction_to_bf16_bits(acc))
    return np.array(out, np.uint16)


def combine_rows_for_token(S, T, K, E, R, Nmax, topk, lay, s, t, expand, n_out=1):
    """(row, k) pairs of Y that token (s, t) combines: the owner's receive row per rank, or the lane's expand row
    (the owner's slot minus its row base, s or, on the hybrid path, s's scale-out index, times Nmax)."""
    El = E // R
    topk = np.asarray(topk).reshape(S, T, K)
    pairs = []
    for k in range(K):
        e = int(topk[s, t, k])
        if not _valid(e, E):
            continue
        if expand:
            pairs.append((int(np.asarray(lay["expand_pos"]).reshape(S, T, K)[s, t, k]), k))
        else:
            d = e // El
            k0 = next(k2 for k2 in range(K) if _valid(int(topk[s, t, k2]), E) and int(topk[s, t, k2]) // El == d)
            j = int(np.asarray(lay["dst_slot"]).reshape(S, T, K)[s, t, k0]) - row_base(s, S, n_out) * Nmax
            rb = np.asarray(lay["recv_base"]).ravel()
            rp = np.asarray(lay["recv_psum"]).reshape(R, S + 1)
            pairs.append((int(rb[d] + rp[d, s] + j), k))
    return pairs
