"""Python binding of libep (include/ep.h): deterministic MoE expert-parallel
dispatch layout, dispatch and combine on one MI355X.

Argument marshalling only: every step runs in the HIP kernels of ``libep.so``.
PyTorch provides device memory and the current stream.  The functions keep
the C names (``ep_query_sizes``, ``ep_layout``, ``ep_dispatch``,
``ep_combine``, ``ep_status_string``); ``alloc_layout`` / ``alloc_recv``
allocate the caller-owned buffers the sizes call describes.

Importing this package fails loudly (ImportError) when ``libep.so`` has not
been built; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# EP_LIBRARY selects another build of the same library (e.g. one compiled with
# different tuning constants); the default is the in-tree build.
LIB_PATH = os.environ.get("EP_LIBRARY") or os.path.join(_HERE, "libep.so")

EP_OK, EP_ERR_INVALID_ARG, EP_ERR_CAPACITY, EP_ERR_UNSUPPORTED, EP_ERR_HIP = 0, -1, -2, -3, -4
EP_DTYPE_BF16, EP_DTYPE_FP8_E4M3FN = 0, 1
EP_PHASE_SCATTER, EP_PHASE_EPILOGUE, EP_PHASE_ALL = 1, 2, 3
EP_FLAG_DIRECT_RECV_X, EP_FLAG_LAYOUT_ONE_LAUNCH = 1, 2


class EpError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {ep_status_string(status)} ({status})")
        self.status = status


class EpConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_src_ranks", "num_tokens", "hidden", "num_topk", "num_experts", "num_ranks",
        "num_max_tokens_per_rank", "x_dtype", "expand", "expert_alignment", "num_layout_cus", "flags",
        "num_scaleout_ranks")]


class EpSizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "dst_slot", "tokens_per_rank", "tokens_per_expert", "recv_psum", "recv_base",
        "expert_base", "expand_pos", "error_flags", "layout_scratch", "recv_psum_scaleup",
        "staging_x", "staging_sf", "staging_meta", "recv_rows",
        "recv_x", "recv_sf", "recv_src_idx", "recv_topk_idx", "recv_topk_weights", "y", "out")]


class EpLayoutT(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "dst_slot_dev", "tokens_per_rank_dev", "tokens_per_expert_dev", "recv_psum_dev", "recv_base_dev",
        "expert_base_dev", "expand_pos_dev", "error_flags_dev", "scratch_dev", "recv_psum_scaleup_dev")]


class EpRecvT(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "staging_x_dev", "staging_sf_dev", "staging_meta_dev", "recv_x_dev", "recv_sf_dev",
        "recv_src_idx_dev", "recv_topk_idx_dev", "recv_topk_weights_dev")] + [("recv_capacity_rows", ctypes.c_int64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    lib.ep_query_sizes.argtypes = [ctypes.POINTER(EpConfig), ctypes.POINTER(EpSizes)]
    lib.ep_layout.argtypes = [ctypes.POINTER(EpConfig), P, ctypes.POINTER(EpLayoutT), P]
    lib.ep_layout_no_alloc.argtypes = [ctypes.POINTER(EpConfig), P, ctypes.POINTER(EpLayoutT), P]
    lib.ep_dispatch.argtypes = [ctypes.POINTER(EpConfig), P, P, P, P, ctypes.POINTER(EpLayoutT),
                                ctypes.POINTER(EpRecvT), ctypes.c_int32, P]
    lib.ep_layout_dispatch.argtypes = [ctypes.POINTER(EpConfig), P, P, P, P, ctypes.POINTER(EpLayoutT),
                                       ctypes.POINTER(EpRecvT), P]
    lib.ep_combine.argtypes = [ctypes.POINTER(EpConfig), ctypes.POINTER(EpLayoutT), P, P, P, P, P]
    lib.ep_combine_bias.argtypes = [ctypes.POINTER(EpConfig), ctypes.POINTER(EpLayoutT), P, P, P, P, P, P, P]
    for f in ("ep_query_sizes", "ep_layout", "ep_layout_no_alloc", "ep_dispatch", "ep_layout_dispatch", "ep_combine",
              "ep_combine_bias", "ep_version"):
        getattr(lib, f).restype = ctypes.c_int
    lib.ep_status_string.argtypes = [ctypes.c_int]
    lib.ep_status_string.restype = ctypes.c_char_p
    return lib


_lib = _load()


def ep_status_string(status: int) -> str:
    return _lib.ep_status_string(int(status)).decode()


def ep_version() -> int:
    return int(_lib.ep_version())


def make_config(S: int, T: int, H: int, K: int, E: int, R: int, Nmax: int, dtype: str = "bf16",
                expand: bool = False, alignment: int = 1, num_layout_cus: int = 0,
                direct_recv_x: bool = False, num_scaleout_ranks: int = 1, layout_one_launch: bool = False) -> EpConfig:
    flags = (EP_FLAG_DIRECT_RECV_X if direct_recv_x else 0) | (EP_FLAG_LAYOUT_ONE_LAUNCH if layout_one_launch else 0)
    return EpConfig(S, T, H, K, E, R, Nmax, EP_DTYPE_FP8_E4M3FN if dtype == "fp8" else EP_DTYPE_BF16,
                    int(bool(expand)), alignment, num_layout_cus, flags, num_scaleout_ranks)


def config_for(w, num_layout_cus: int = 0, direct_recv_x: bool = False, layout_one_launch: bool = False) -> EpConfig:
    """EpConfig of a ``workloads.Workload``."""
    return make_config(w.S, w.T, w.H, w.K, w.E, w.R, w.Nmax, w.dtype, w.expand, w.alignment, num_layout_cus,
                       direct_recv_x, getattr(w, "n_out", 1), layout_one_launch)


def ep_query_sizes(cfg: EpConfig) -> EpSizes:
    sz = EpSizes()
    rc = _lib.ep_query_sizes(ctypes.byref(cfg), ctypes.byref(sz))
    if rc != EP_OK:
        raise EpError(rc, "ep_query_sizes")
    return sz


# The helpers below run on every call, so they stay cheap: plain integers for
# pointers and streams (the argtypes convert them), one size property.
def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr(t: Optional[torch.Tensor], name: str, nbytes: int = 0) -> Optional[int]:
    """Device pointer of a contiguous CUDA tensor holding at least ``nbytes``."""
    if t is None:
        if nbytes:
            raise ValueError(f"{name} is required")
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    nb = t.nbytes
    if nb < nbytes:
        raise ValueError(f"{name} holds {nb} bytes, needs {nbytes}")
    return t.data_ptr() if nb else None


def _recv_rows(cfg: EpConfig) -> int:
    """Receive-row bound of cfg (ep_query_sizes), kept on cfg with the bytes it
    was computed from and recomputed when any field has changed since."""
    key = bytes(cfg)
    memo = getattr(cfg, "_rows_memo", None)
    if memo is None or memo[0] != key:
        memo = (key, int(ep_query_sizes(cfg).recv_rows))
        cfg._rows_memo = memo
    return memo[1]


def _check_elem(t: Optional[torch.Tensor], name: str, size: int) -> None:
    """Rows are read as elements of ``size`` bytes (bf16 2, e4m3fn 1, fp32
    scales 4): a tensor of that element width (any dtype, a bit view included)
    or of raw bytes is accepted, so that e.g. fp32 activations passed for bf16
    rows are refused instead of being read as bf16 bits."""
    if t is not None and t.element_size() not in (1, size):
        raise ValueError(f"{name} must have {size}-byte elements (or be raw bytes), got {t.dtype}")


def _empty(nbytes: int, dtype: torch.dtype, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    esz = torch.empty((), dtype=dtype).element_size()
    return torch.empty(max(1, nbytes // esz), dtype=dtype, device=device)


class LayoutBuffers:
    """Device tensors of the layout tables plus the ep_layout_t that points at them."""

    def __init__(self, cfg: EpConfig, device="cuda"):
        sz = ep_query_sizes(cfg)
        S, T, K, E, R = cfg.num_src_ranks, cfg.num_tokens, cfg.num_topk, cfg.num_experts, cfg.num_ranks
        i32 = dict(dtype=torch.int32, device=device)
        self.dst_slot = torch.empty((S, T, K), **i32)
        self.tokens_per_rank = torch.empty((S, R), **i32)
        self.tokens_per_expert = torch.empty((S, E), **i32)
        self.recv_psum = torch.empty((R, S + 1), **i32)
        self.recv_base = torch.empty((R + 1,), **i32)
        self.expert_base = torch.empty((E + 1,), **i32) if cfg.expand else None
        self.expand_pos = torch.empty((S, T, K), **i32) if cfg.expand else None
        self.error_flags = torch.zeros((1,), **i32)
        self.scratch = _empty(sz.layout_scratch, torch.int32, device)
        n_out = cfg.num_scaleout_ranks
        self.recv_psum_scaleup = torch.empty((R, S // n_out + 1), **i32) if n_out > 1 else None
        self.struct = EpLayoutT(
            _ptr(self.dst_slot, "dst_slot"), _ptr(self.tokens_per_rank, "tokens_per_rank"),
            _ptr(self.tokens_per_expert, "tokens_per_expert"), _ptr(self.recv_psum, "recv_psum"),
            _ptr(self.recv_base, "recv_base"), _ptr(self.expert_base, "expert_base"),
            _ptr(self.expand_pos, "expand_pos"), _ptr(self.error_flags, "error_flags"),
            _ptr(self.scratch, "scratch"), _ptr(self.recv_psum_scaleup, "recv_psum_scaleup"))

    def tables(self):
        out = dict(dst_slot=self.dst_slot, tokens_per_rank=self.tokens_per_rank,
                   tokens_per_expert=self.tokens_per_expert, recv_psum=self.recv_psum, recv_base=self.recv_base,
                   error_flags=self.error_flags)
        if self.expert_base is not None:
            out.update(expert_base=self.expert_base, expand_pos=self.expand_pos)
        if self.recv_psum_scaleup is not None:
            out.update(recv_psum_scaleup=self.recv_psum_scaleup)
        return out


class RecvBuffers:
    """Device tensors of the staging and receive buffers plus their ep_recv_t."""

    def __init__(self, cfg: EpConfig, device="cuda"):
        sz = ep_query_sizes(cfg)
        S, K, R, Nmax, H = cfg.num_src_ranks, cfg.num_topk, cfg.num_ranks, cfg.num_max_tokens_per_rank, cfg.hidden
        fp8 = cfg.x_dtype == EP_DTYPE_FP8_E4M3FN
        rw = H if fp8 else 2 * H
        F = H // 128 if fp8 else 0
        rows = int(sz.recv_rows)
        self.rows = rows
        direct = bool(cfg.flags & EP_FLAG_DIRECT_RECV_X)
        self.staging_x = None if direct else torch.empty((R, S, Nmax, rw), dtype=torch.uint8, device=device)
        self.staging_sf = torch.empty((R, S, Nmax, F), dtype=torch.float32, device=device) if fp8 else None
        self.staging_meta = torch.empty((R, S, Nmax, 1 + 2 * K), dtype=torch.int32, device=device)
        self.recv_x = torch.empty((rows, rw), dtype=torch.uint8, device=device)
        self.recv_sf = torch.empty((rows, F), dtype=torch.float32, device=device) if fp8 else None
        self.recv_src_idx = torch.empty((rows,), dtype=torch.int32, device=device)
        if cfg.expand:
            self.recv_topk_idx = None
            self.recv_topk_weights = torch.empty((rows,), dtype=torch.float32, device=device)
        else:
            self.recv_topk_idx = torch.empty((rows, K), dtype=torch.int32, device=device)
            self.recv_topk_weights = torch.empty((rows, K), dtype=torch.float32, device=device)
        self.struct = EpRecvT(
            _ptr(self.staging_x, "staging_x"), _ptr(self.staging_sf, "staging_sf"),
            _ptr(self.staging_meta, "staging_meta"), _ptr(self.recv_x, "recv_x"), _ptr(self.recv_sf, "recv_sf"),
            _ptr(self.recv_src_idx, "recv_src_idx"), _ptr(self.recv_topk_idx, "recv_topk_idx"),
            _ptr(self.recv_topk_weights, "recv_topk_weights"), rows)


def alloc_layout(cfg: EpConfig, device="cuda") -> LayoutBuffers:
    return LayoutBuffers(cfg, device)


def alloc_recv(cfg: EpConfig, device="cuda") -> RecvBuffers:
    return RecvBuffers(cfg, device)


def ep_layout(cfg: EpConfig, topk_idx: torch.Tensor, layout: LayoutBuffers, stream=None) -> None:
    S, T, K = cfg.num_src_ranks, cfg.num_tokens, cfg.num_topk
    if topk_idx.dtype != torch.int64:
        raise ValueError("topk_idx must be int64")
    rc = _lib.ep_layout(ctypes.byref(cfg), _ptr(topk_idx, "topk_idx", S * T * K * 8), ctypes.byref(layout.struct),
                        _stream(stream))
    if rc != EP_OK:
        raise EpError(rc, "ep_layout")


def ep_layout_no_alloc(cfg: EpConfig, topk_idx: torch.Tensor, layout: LayoutBuffers, stream=None) -> None:
    """ep_layout on the library's own per-GPU scratch (layout.scratch is not used)."""
    S, T, K = cfg.num_src_ranks, cfg.num_tokens, cfg.num_topk
    if topk_idx.dtype != torch.int64:
        raise ValueError("topk_idx must be int64")
    rc = _lib.ep_layout_no_alloc(ctypes.byref(cfg), _ptr(topk_idx, "topk_idx", S * T * K * 8),
                                 ctypes.byref(layout.struct), _stream(stream))
    if rc != EP_OK:
        raise EpError(rc, "ep_layout_no_alloc")


def ep_dispatch(cfg: EpConfig, x: torch.Tensor, x_sf: Optional[torch.Tensor], topk_idx: torch.Tensor,
                topk_weights: torch.Tensor, layout: LayoutBuffers, recv: RecvBuffers, phases: int = EP_PHASE_ALL,
                stream=None) -> None:
    S, T, K, H = cfg.num_src_ranks, cfg.num_tokens, cfg.num_topk, cfg.hidden
    fp8 = cfg.x_dtype == EP_DTYPE_FP8_E4M3FN
    rw = H if fp8 else 2 * H
    if topk_weights.dtype != torch.float32 or topk_idx.dtype != torch.int64:
        raise ValueError("topk_idx must be int64 and topk_weights float32")
    _check_elem(x, "x", 1 if fp8 else 2)
    _check_elem(x_sf, "x_sf", 4)
    rc = _lib.ep_dispatch(ctypes.byref(cfg), _ptr(x, "x", S * T * rw),
                          _ptr(x_sf, "x_sf", S * T * (H // 128) * 4 if fp8 else 0),
                          _ptr(topk_idx, "topk_idx", S * T * K * 8), _ptr(topk_weights, "topk_weights", S * T * K * 4),
                          ctypes.byref(layout.struct), ctypes.byref(recv.struct), int(phases), _stream(stream))
    if rc != EP_OK:
        raise EpError(rc, "ep_dispatch")


def ep_layout_dispatch(cfg: EpConfig, x: torch.Tensor, x_sf: Optional[torch.Tensor], topk_idx: torch.Tensor,
                       topk_weights: torch.Tensor, layout: LayoutBuffers, recv: RecvBuffers, stream=None) -> None:
    """ep_layout then ep_dispatch (both phases) in one call; one kernel for small single sources."""
    S, T, K, H = cfg.num_src_ranks, cfg.num_tokens, cfg.num_topk, cfg.hidden
    fp8 = cfg.x_dtype == EP_DTYPE_FP8_E4M3FN
    rw = H if fp8 else 2 * H
    if topk_weights.dtype != torch.float32 or topk_idx.dtype != torch.int64:
        raise ValueError("topk_idx must be int64 and topk_weights float32")
    _check_elem(x, "x", 1 if fp8 else 2)
    _check_elem(x_sf, "x_sf", 4)
    rc = _lib.ep_layout_dispatch(ctypes.byref(cfg), _ptr(x, "x", S * T * rw),
                                 _ptr(x_sf, "x_sf", S * T * (H // 128) * 4 if fp8 else 0),
                                 _ptr(topk_idx, "topk_idx", S * T * K * 8),
                                 _ptr(topk_weights, "topk_weights", S * T * K * 4),
                                 ctypes.byref(layout.struct), ctypes.byref(recv.struct), _stream(stream))
    if rc != EP_OK:
        raise EpError(rc, "ep_layout_dispatch")


def ep_combine(cfg: EpConfig, layout: LayoutBuffers, topk_idx: torch.Tensor, topk_weights: torch.Tensor,
               y: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    S, T, K, H = cfg.num_src_ranks, cfg.num_tokens, cfg.num_topk, cfg.hidden
    rows = _recv_rows(cfg)
    if topk_weights.dtype != torch.float32 or topk_idx.dtype != torch.int64:
        raise ValueError("topk_idx must be int64 and topk_weights float32")
    _check_elem(y, "y", 2)
    _check_elem(out, "out", 2)
    rc = _lib.ep_combine(ctypes.byref(cfg), ctypes.byref(layout.struct), _ptr(topk_idx, "topk_idx", S * T * K * 8),
                         _ptr(topk_weights, "topk_weights", S * T * K * 4), _ptr(y, "y", rows * H * 2),
                         _ptr(out, "out", S * T * H * 2), _stream(stream))
    if rc != EP_OK:
        raise EpError(rc, "ep_combine")


def ep_combine_bias(cfg: EpConfig, layout: LayoutBuffers, topk_idx: torch.Tensor, topk_weights: torch.Tensor,
                    y: torch.Tensor, bias0: Optional[torch.Tensor], bias1: Optional[torch.Tensor],
                    out: torch.Tensor, stream=None) -> None:
    """Combine plus up to two bf16 [S][T][H] bias tensors added before the rounding."""
    S, T, K, H = cfg.num_src_ranks, cfg.num_tokens, cfg.num_topk, cfg.hidden
    rows = _recv_rows(cfg)
    if topk_weights.dtype != torch.float32 or topk_idx.dtype != torch.int64:
        raise ValueError("topk_idx must be int64 and topk_weights float32")
    for t, name in ((y, "y"), (bias0, "bias0"), (bias1, "bias1"), (out, "out")):
        _check_elem(t, name, 2)
    nb = S * T * H * 2
    rc = _lib.ep_combine_bias(ctypes.byref(cfg), ctypes.byref(layout.struct), _ptr(topk_idx, "topk_idx", S * T * K * 8),
                              _ptr(topk_weights, "topk_weights", S * T * K * 4), _ptr(y, "y", rows * H * 2),
                              _ptr(bias0, "bias0", nb if bias0 is not None else 0),
                              _ptr(bias1, "bias1", nb if bias1 is not None else 0),
                              _ptr(out, "out", S * T * H * 2), _stream(stream))
    if rc != EP_OK:
        raise EpError(rc, "ep_combine_bias")
