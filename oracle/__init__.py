"""ctypes wrapper around the plain C oracle (``oracle/ep_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` are the only callers.  The HIP library never loads
this module and this module never loads the HIP library.

``build()`` compiles ``libep_oracle.so`` next to this file with gcc
(``-O2 -ffp-contract=off``); the functions below load it and marshal numpy
arrays.  Layouts are the ones documented in ``ep_oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ep_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libep_oracle.so")
_libs: Dict[str, ctypes.CDLL] = {}
_active: Optional[str] = None


def compile_oracle(src: str, out: str) -> str:
    """gcc -O2 -ffp-contract=off one oracle source into a shared library."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-std=c11", "-Wall", "-Wextra", "-shared",
           "-fPIC", "-I", _HERE, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle with gcc; returns the library path."""
    if force or not os.path.exists(_LIB_PATH):
        compile_oracle(_SRC, _LIB_PATH)
    return _LIB_PATH


def _open(path: str) -> ctypes.CDLL:
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.epo_layout.argtypes = [I] * 9 + [P] * 10
    lib.epo_layout.restype = I
    lib.epo_dispatch.argtypes = [I] * 11 + [P] * 19
    lib.epo_dispatch.restype = I
    lib.epo_combine.argtypes = [I] * 9 + [P] * 8
    lib.epo_combine.restype = I
    lib.epo_combine_bias.argtypes = [I] * 9 + [P] * 10
    lib.epo_combine_bias.restype = I
    lib.epo_combine_tokens.argtypes = [I] * 9 + [P] * 7 + [I, P, P]
    lib.epo_combine_tokens.restype = I
    lib.epo_bf16_from_double.argtypes = [ctypes.c_double]
    lib.epo_bf16_from_double.restype = ctypes.c_uint16
    return lib


def use_library(path: Optional[str]) -> None:
    """Route the functions below to another build of the oracle (``None`` = the
    default one).  Only the mutation tests use this, to show that the pins
    reject deliberately broken oracles."""
    global _active
    _active = path


def _load() -> ctypes.CDLL:
    path = _active or _LIB_PATH
    if path not in _libs:
        if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
            build()
        _libs[path] = _open(path)
    return _libs[path]


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def bf16_from_double(v: float) -> int:
    return int(_load().epo_bf16_from_double(float(v)))


def layout(S, T, K, E, R, Nmax, topk_idx: np.ndarray, expand: bool = False, A: int = 1,
           n_out: int = 1) -> Dict[str, np.ndarray]:
    """Run the oracle layout; returns the tables as numpy int32 arrays
    (``n_out`` = num_scaleout_ranks; > 1 selects the hybrid row form)."""
    lib = _load()
    topk = np.ascontiguousarray(topk_idx, dtype=np.int64).reshape(S, T, K)
    out = {
        "dst_slot": np.empty((S, T, K), np.int32),
        "tokens_per_rank": np.empty((S, R), np.int32),
        "tokens_per_expert": np.empty((S, E), np.int32),
        "recv_psum": np.empty((R, S + 1), np.int32),
        "recv_base": np.empty((R + 1,), np.int32),
        "error_flags": np.zeros((1,), np.int32),
    }
    if expand:
        out["expert_base"] = np.empty((E + 1,), np.int32)
        out["expand_pos"] = np.empty((S, T, K), np.int32)
    if n_out > 1:
        out["recv_psum_scaleup"] = np.empty((R, S // n_out + 1), np.int32)
    rc = lib.epo_layout(S, T, K, E, R, Nmax, int(expand), A, n_out, _p(topk), _p(out["dst_slot"]),
                        _p(out["tokens_per_rank"]), _p(out["tokens_per_expert"]), _p(out["recv_psum"]),
                        _p(out["recv_base"]), _p(out.get("expert_base")), _p(out.get("expand_pos")),
                        _p(out.get("recv_psum_scaleup")), _p(out["error_flags"]))
    if rc != 0:
        raise ValueError(f"epo_layout rejected the sizes (rc={rc})")
    return out


def recv_rows(S, T, K, E, R, lay: Dict[str, np.ndarray], expand: bool) -> int:
    """Number of receive rows the layout fills (deduplicated rows, or expand rows incl. padding)."""
    return int(lay["expert_base"][E]) if expand else int(lay["recv_base"][R])


def dispatch(S, T, H, K, E, R, Nmax, is_fp8: bool, expand: bool, A: int, x: np.ndarray,
             x_sf: Optional[np.ndarray], topk_idx: np.ndarray, topk_weights: np.ndarray,
             lay: Dict[str, np.ndarray], n_out: int = 1) -> Dict[str, np.ndarray]:
    """Run the oracle scatter + copy epilogue; returns staging and receive arrays.

    Staging rows that no lane fills keep the value 0 here; they are unspecified
    and never compared."""
    lib = _load()
    Rw = H if is_fp8 else 2 * H
    F = H // 128 if is_fp8 else 0
    M = 1 + 2 * K
    rows = recv_rows(S, T, K, E, R, lay, expand)
    out = {
        "staging_x": np.zeros((R, S, Nmax, Rw), np.uint8),
        "staging_sf": np.zeros((R, S, Nmax, F), np.float32),
        "staging_meta": np.zeros((R, S, Nmax, M), np.int32),
        "recv_x": np.zeros((rows, Rw), np.uint8),
        "recv_sf": np.zeros((rows, F), np.float32),
        "recv_src_idx": np.zeros((rows,), np.int32),
    }
    if expand:
        out["recv_topk_weights"] = np.zeros((rows,), np.float32)
    else:
        out["recv_topk_idx"] = np.zeros((rows, K), np.int32)
        out["recv_topk_weights"] = np.zeros((rows, K), np.float32)
    xs = np.ascontiguousarray(x, dtype=np.uint8).reshape(S, T, Rw)
    sf = np.ascontiguousarray(x_sf, dtype=np.float32).reshape(S, T, F) if is_fp8 else None
    rc = lib.epo_dispatch(S, T, H, K, E, R, Nmax, int(is_fp8), int(expand), A, n_out, _p(xs), _p(sf),
                          _p(np.ascontiguousarray(topk_idx, dtype=np.int64)),
                          _p(np.ascontiguousarray(topk_weights, dtype=np.float32)),
                          _p(lay["dst_slot"]), _p(lay["tokens_per_rank"]), _p(lay["tokens_per_expert"]),
                          _p(lay["recv_psum"]), _p(lay["recv_base"]), _p(lay.get("expert_base")),
                          _p(lay.get("expand_pos")), _p(out["staging_x"]), _p(out["staging_sf"]),
                          _p(out["staging_meta"]), _p(out["recv_x"]), _p(out["recv_sf"]),
                          _p(out["recv_src_idx"]), _p(out.get("recv_topk_idx")), _p(out["recv_topk_weights"]))
    if rc != 0:
        raise ValueError(f"epo_dispatch rejected the sizes (rc={rc})")
    return out


def combine(S, T, H, K, E, R, Nmax, expand: bool, topk_idx: np.ndarray, topk_weights: np.ndarray,
            lay: Dict[str, np.ndarray], y: np.ndarray, n_out: int = 1) -> np.ndarray:
    """Run the oracle combine; ``y`` is bf16 bits (uint16) [rows][H]; returns uint16 [S][T][H]."""
    lib = _load()
    out = np.empty((S, T, H), np.uint16)
    yy = np.ascontiguousarray(y, dtype=np.uint16)
    rc = lib.epo_combine(S, T, H, K, E, R, Nmax, int(expand), n_out,
                         _p(np.ascontiguousarray(topk_idx, dtype=np.int64)),
                         _p(np.ascontiguousarray(topk_weights, dtype=np.float32)),
                         _p(lay["dst_slot"]), _p(lay["recv_psum"]), _p(lay["recv_base"]),
                         _p(lay.get("expand_pos")), _p(yy), _p(out))
    if rc != 0:
        raise ValueError(f"epo_combine rejected the sizes (rc={rc})")
    return out


def combine_bias(S, T, H, K, E, R, Nmax, expand: bool, topk_idx: np.ndarray, topk_weights: np.ndarray,
                 lay: Dict[str, np.ndarray], y: np.ndarray, bias0: Optional[np.ndarray],
                 bias1: Optional[np.ndarray], n_out: int = 1) -> np.ndarray:
    """Combine plus up to two bf16 bias tensors (uint16 [S][T][H] or None)."""
    lib = _load()
    out = np.empty((S, T, H), np.uint16)
    b0 = None if bias0 is None else np.ascontiguousarray(bias0, dtype=np.uint16)
    b1 = None if bias1 is None else np.ascontiguousarray(bias1, dtype=np.uint16)
    rc = lib.epo_combine_bias(S, T, H, K, E, R, Nmax, int(expand), n_out,
                              _p(np.ascontiguousarray(topk_idx, dtype=np.int64)),
                              _p(np.ascontiguousarray(topk_weights, dtype=np.float32)),
                              _p(lay["dst_slot"]), _p(lay["recv_psum"]), _p(lay["recv_base"]),
                              _p(lay.get("expand_pos")), _p(np.ascontiguousarray(y, dtype=np.uint16)),
                              _p(b0), _p(b1), _p(out))
    if rc != 0:
        raise ValueError(f"epo_combine_bias rejected the sizes (rc={rc})")
    return out


def combine_tokens(S, T, H, K, E, R, Nmax, expand: bool, topk_idx: np.ndarray, topk_weights: np.ndarray,
                   lay: Dict[str, np.ndarray], y: np.ndarray, sel: np.ndarray, n_out: int = 1) -> np.ndarray:
    """Combine for the global token indices ``sel`` only; returns uint16 [len(sel)][H]."""
    lib = _load()
    sel = np.ascontiguousarray(sel, dtype=np.int64)
    out = np.empty((sel.size, H), np.uint16)
    yy = np.ascontiguousarray(y, dtype=np.uint16)
    rc = lib.epo_combine_tokens(S, T, H, K, E, R, Nmax, int(expand), n_out,
                                _p(np.ascontiguousarray(topk_idx, dtype=np.int64)),
                                _p(np.ascontiguousarray(topk_weights, dtype=np.float32)),
                                _p(lay["dst_slot"]), _p(lay["recv_psum"]), _p(lay["recv_base"]),
                                _p(lay.get("expand_pos")), _p(yy), int(sel.size), _p(sel), _p(out))
    if rc != 0:
        raise ValueError(f"epo_combine_tokens rejected the arguments (rc={rc})")
    return out

