"""Python binding of the MI355X fused all-reduce-sum (+ residual + RMSNorm) library.

Thin marshalling over the C ABI in ``include/ar_fused.h`` (``libar_fused.so``, built from
``csrc/`` for gfx950): each function takes torch tensors on the GPU, checks that they are
contiguous, of one element type and of the [M, H] shape the call implies, and passes their
device pointers, sizes and the current HIP stream to the function of the same name.  Every
step of the computation runs in the library's HIP kernels; there is no other code path.  If the
library has not been built, every call raises.

Operations (fusion patterns kAllReduce and kARResidualRMSNorm):
  ar_sum(inputs, out)                    out = sum of the W partials (binary32, rank order)
  ar_residual_rmsnorm(inputs, residual, gamma, eps, residual_out, norm_out)
                                         residual_out = sum + residual
                                         norm_out = RMSNorm(residual_out) * gamma
  ar_residual_rmsnorm_ws(..., workspace) the same; few-row calls split each row over
                                         several blocks (caller-owned workspace)
"""
from __future__ import annotations

import ctypes
import os
import re
import threading
from typing import Dict, Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libar_fused.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "ar_fused.h")

DTYPE_FP32, DTYPE_FP16, DTYPE_BF16 = 0, 1, 2
PATTERN_ALLREDUCE, PATTERN_AR_RESIDUAL_RMSNORM = 0, 1
AR_OK, AR_ERR_INVALID_ARG, AR_ERR_UNSUPPORTED, AR_ERR_MISALIGNED = 0, 1, 2, 3
AR_ERR_ALIAS, AR_ERR_LAUNCH, AR_ERR_DEVICE = 4, 5, 6
SUPPORTED_W = (1, 2, 4, 8, 16, 32, 64)

_lib = None
_lock = threading.Lock()


class ArError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))


ROUTE_ONE_SHOT, ROUTE_TWO_SHOT, ROUTE_FALLBACK, ROUTE_UNFUSED = 0, 1, 2, 3


class Policy(ctypes.Structure):
    _fields_ = [("min_tokens", ctypes.c_int64), ("two_shot_min_bytes", ctypes.c_int64),
                ("max_payload_bytes", ctypes.c_int64)]

    def as_dict(self) -> Dict[str, int]:
        return {name: int(getattr(self, name)) for name, _ in self._fields_}


class LaunchConfig(ctypes.Structure):
    _fields_ = [("threads_per_block", ctypes.c_int32), ("vecs_per_thread", ctypes.c_int32),
                ("lanes_per_row", ctypes.c_int32), ("rows_per_block", ctypes.c_int32),
                ("grid", ctypes.c_int32), ("flat", ctypes.c_int32), ("nt_store", ctypes.c_int32),
                ("ranks_per_batch", ctypes.c_int32)]

    def as_dict(self) -> Dict[str, int]:
        return {name: int(getattr(self, name)) for name, _ in self._fields_}

    @classmethod
    def from_dict(cls, d: Dict[str, int]) -> "LaunchConfig":
        return cls(**{name: int(d.get(name, 0)) for name, _ in cls._fields_})


class SplitConfig(ctypes.Structure):
    _fields_ = [("threads_per_block", ctypes.c_int32), ("vecs_per_thread", ctypes.c_int32),
                ("segments", ctypes.c_int32), ("max_polls", ctypes.c_uint32)]

    def as_dict(self) -> Dict[str, int]:
        return {name: int(getattr(self, name)) for name, _ in self._fields_}

    @classmethod
    def from_dict(cls, d: Dict[str, int]) -> "SplitConfig":
        return cls(**{name: int(d.get(name, 0)) for name, _ in cls._fields_})


SPLIT_SLOTS = 64


def lib():
    """The loaded library (ctypes.CDLL); raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("HIP library %s is not built; run __graft_entry__.build() or "
                               "python all_reduce_residual_amd/_build.py" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        cfgp = ctypes.POINTER(LaunchConfig)
        sig = {
            "ar_sum": [vp, i32, i64, i64, i32, vp, vp],
            "ar_sum_with_config": [vp, i32, i64, i64, i32, vp, vp, cfgp],
            "ar_residual_rmsnorm": [vp, i32, i64, i64, i32, vp, vp, f32, vp, vp, vp],
            "ar_residual_rmsnorm_with_config": [vp, i32, i64, i64, i32, vp, vp, f32, vp, vp, vp,
                                                cfgp],
            "ar_supports": [i32, i32, i64, i64, i32],
            "ar_launch_config": [i32, i32, i64, i64, i32, i32, cfgp],
            "ar_status_string": [i32],
            "ar_lamport_arm": [vp, i32, i64, i64, i32, vp],
            "ar_lamport_push": [vp, i32, vp, i32, i64, i64, i32, i64, vp],
            "ar_lamport_sum": [vp, i32, i64, i64, i32, i64, vp, vp, ctypes.c_uint32, vp],
            "ar_lamport_residual_rmsnorm": [vp, i32, i64, i64, i32, i64, vp, vp, f32, vp, vp, vp,
                                            ctypes.c_uint32, vp],
            "ar_policy_default": [i32, ctypes.POINTER(Policy)],
            "ar_route": [i32, i32, i64, i64, i32, ctypes.POINTER(Policy),
                         ctypes.POINTER(ctypes.c_int)],
            "ar_allreduce_routed": [i32, vp, i32, i64, i64, i32, vp, vp, f32, vp, vp, i32,
                                    ctypes.POINTER(Policy), ctypes.POINTER(ctypes.c_int), vp],
            "ar_row_partition": [i32, i64, i32, ctypes.POINTER(ctypes.c_int64),
                                 ctypes.POINTER(ctypes.c_int64)],
            "ar_all_gather": [vp, i32, i64, i64, i32, vp, vp],
            "ar_device_cu_count": [ctypes.POINTER(ctypes.c_int)],
            "ar_rmsnorm": [vp, i64, i64, i32, vp, f32, vp, vp],
            "ar_residual_rmsnorm_unfused": [vp, i32, i64, i64, i32, vp, vp, f32, vp, vp, vp],
            "ar_split_workspace_bytes": [i64],
            "ar_workspace_clear": [vp, i64, vp],
            "ar_split_config": [i32, i64, i64, i32, i32, ctypes.POINTER(SplitConfig)],
            "ar_residual_rmsnorm_ws": [vp, i32, i64, i64, i32, vp, vp, f32, vp, vp, vp, i64, vp],
            "ar_residual_rmsnorm_noalloc": [vp, i32, i64, i64, i32, vp, vp, f32, vp, vp, vp],
            "ar_residual_rmsnorm_split_with_config": [vp, i32, i64, i64, i32, vp, vp, f32, vp,
                                                      vp, vp, i64, vp,
                                                      ctypes.POINTER(SplitConfig)],
        }
        for name, argtypes in sig.items():
            fn = getattr(L, name)
            fn.argtypes = argtypes
            fn.restype = {"ar_status_string": ctypes.c_char_p,
                          "ar_split_workspace_bytes": ctypes.c_int64}.get(name, ctypes.c_int)
        _lib = L
        return L


def header_functions() -> Sequence[str]:
    """Names of the functions include/ar_fused.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ar_\w+)\s*\(", text, flags=re.M)))


def status_string(status: int) -> str:
    return lib().ar_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != AR_OK:
        raise ArError(status, where)


def dtype_code(torch_dtype) -> int:
    import torch
    codes = {torch.float32: DTYPE_FP32, torch.float16: DTYPE_FP16, torch.bfloat16: DTYPE_BF16}
    if torch_dtype not in codes:
        raise TypeError("unsupported element type %s" % (torch_dtype,))
    return codes[torch_dtype]


def _stream_handle(stream, device) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _marshal_inputs(inputs, out_like):
    """Check the partials against the [M, H] output and return (ptr array, W, M, H, dtype)."""
    if len(inputs) == 0:
        raise ValueError("need at least one partial")
    if out_like.dim() != 2:
        raise ValueError("tensors must be [M, H]")
    M, H = out_like.shape
    for t in list(inputs) + [out_like]:
        if t.dtype != out_like.dtype or tuple(t.shape) != (M, H):
            raise ValueError("every tensor must be [%d, %d] %s" % (M, H, out_like.dtype))
        if not t.is_cuda or t.device != out_like.device:
            raise ValueError("every tensor must be on %s" % out_like.device)
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    ptrs = (ctypes.c_void_p * len(inputs))(*[t.data_ptr() for t in inputs])
    return ptrs, len(inputs), M, H, dtype_code(out_like.dtype)


def ar_sum(inputs, out, stream=None, config: Optional[Dict[str, int]] = None) -> None:
    """kAllReduce: out = RN_T(x_0 + ... + x_{W-1}), binary32 in rank order."""
    ptrs, W, M, H, dt = _marshal_inputs(inputs, out)
    s = _stream_handle(stream, out.device)
    if config is None:
        st = lib().ar_sum(ptrs, W, M, H, dt, out.data_ptr(), s)
    else:
        cfg = LaunchConfig.from_dict(config)
        st = lib().ar_sum_with_config(ptrs, W, M, H, dt, out.data_ptr(), s, ctypes.byref(cfg))
    _check(st, "ar_sum")


def ar_residual_rmsnorm(inputs, residual, gamma, eps: float, residual_out, norm_out,
                        stream=None, config: Optional[Dict[str, int]] = None) -> None:
    """kARResidualRMSNorm: residual_out = RN_T(sum + residual); norm_out = RMSNorm * gamma."""
    import torch
    ptrs, W, M, H, dt = _marshal_inputs(inputs, residual_out)
    _marshal_inputs([residual], norm_out)
    _marshal_inputs([residual], residual_out)
    if gamma.dtype != torch.float32 or tuple(gamma.shape) != (H,) or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous float32 [%d] tensor" % H)
    if gamma.device != residual_out.device:
        raise ValueError("gamma must be on %s" % residual_out.device)
    s = _stream_handle(stream, residual_out.device)
    args = (ptrs, W, M, H, dt, residual.data_ptr(), gamma.data_ptr(), float(eps),
            residual_out.data_ptr(), norm_out.data_ptr(), s)
    if config is None:
        st = lib().ar_residual_rmsnorm(*args)
    else:
        cfg = LaunchConfig.from_dict(config)
        st = lib().ar_residual_rmsnorm_with_config(*args, ctypes.byref(cfg))
    _check(st, "ar_residual_rmsnorm")


def split_workspace_bytes(M: int) -> int:
    """Bytes of workspace ar_residual_rmsnorm_ws needs for calls of up to M rows."""
    n = int(lib().ar_split_workspace_bytes(int(M)))
    if n < 0:
        raise ValueError("bad row count %d" % M)
    return n


def ar_workspace_clear(workspace, stream=None) -> None:
    """Zero-fills a workspace tensor (a kernel, so it may be captured in a graph)."""
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("the workspace must be a contiguous device tensor")
    nbytes = workspace.numel() * workspace.element_size()
    s = _stream_handle(stream, workspace.device)
    _check(lib().ar_workspace_clear(workspace.data_ptr(), nbytes, s), "ar_workspace_clear")


def new_workspace(M: int, device):
    """A zero-filled uint8 tensor of split_workspace_bytes(M) bytes on `device` (torch's
    allocator; the library allocates nothing)."""
    import torch
    return torch.zeros(split_workspace_bytes(M), dtype=torch.uint8, device=device)


def ar_split_config(W: int, M: int, H: int, dtype: int, cu_count: int = 0) -> Dict[str, int]:
    """The split launch shape the heuristic picks (all zeros: one block per row)."""
    c = SplitConfig()
    _check(lib().ar_split_config(W, M, H, dtype, cu_count, ctypes.byref(c)), "ar_split_config")
    return c.as_dict()


def ar_residual_rmsnorm_ws(inputs, residual, gamma, eps: float, residual_out, norm_out,
                           workspace, stream=None, config: Optional[Dict[str, int]] = None) -> None:
    """kARResidualRMSNorm with a workspace: few-row calls split each row over several blocks
    (results as ar_residual_rmsnorm).  `workspace`: a contiguous device tensor of at least
    split_workspace_bytes(M) bytes, zero-filled before its first use (new_workspace).  With
    `config` the split kernel runs with that shape (ar_residual_rmsnorm_split_with_config)."""
    ptrs, W, M, H, dt = _marshal_inputs(inputs, residual_out)
    _marshal_inputs([residual], norm_out)
    _marshal_inputs([residual], residual_out)
    _check_gamma(gamma, H, residual_out.device)
    if not workspace.is_cuda or workspace.device != residual_out.device or \
            not workspace.is_contiguous():
        raise ValueError("the workspace must be a contiguous tensor on %s" % residual_out.device)
    nbytes = workspace.numel() * workspace.element_size()
    s = _stream_handle(stream, residual_out.device)
    args = (ptrs, W, M, H, dt, residual.data_ptr(), gamma.data_ptr(), float(eps),
            residual_out.data_ptr(), norm_out.data_ptr(), workspace.data_ptr(), nbytes, s)
    if config is None:
        _check(lib().ar_residual_rmsnorm_ws(*args), "ar_residual_rmsnorm_ws")
    else:
        cfg = SplitConfig.from_dict(config)
        _check(lib().ar_residual_rmsnorm_split_with_config(*args, ctypes.byref(cfg)),
               "ar_residual_rmsnorm_split_with_config")


NOALLOC_MAX_ROWS = 512


def ar_residual_rmsnorm_noalloc(inputs, residual, gamma, eps: float, residual_out, norm_out,
                                stream=None) -> None:
    """kARResidualRMSNorm with the split form's exchange slots inside the library (no workspace
    argument, nothing allocated; at most NOALLOC_MAX_ROWS rows).  Calls that overlap in time on
    one GPU share those slots and race: issue them on one stream."""
    ptrs, W, M, H, dt = _marshal_inputs(inputs, residual_out)
    _marshal_inputs([residual], norm_out)
    _marshal_inputs([residual], residual_out)
    _check_gamma(gamma, H, residual_out.device)
    s = _stream_handle(stream, residual_out.device)
    _check(lib().ar_residual_rmsnorm_noalloc(ptrs, W, M, H, dt, residual.data_ptr(),
                                             gamma.data_ptr(), float(eps),
                                             residual_out.data_ptr(), norm_out.data_ptr(), s),
           "ar_residual_rmsnorm_noalloc")


def _check_gamma(gamma, H, device):
    import torch
    if gamma.dtype != torch.float32 or tuple(gamma.shape) != (H,) or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous float32 [%d] tensor" % H)
    if gamma.device != device:
        raise ValueError("gamma must be on %s" % device)


def ar_residual_rmsnorm_unfused(inputs, residual, gamma, eps: float, residual_out, norm_out,
                                stream=None) -> None:
    """kARResidualRMSNorm as two kernels (sum with the residual as last addend, then RMSNorm of
    residual_out): the fallback for rows of any width, with the fused path's results."""
    ptrs, W, M, H, dt = _marshal_inputs(inputs, residual_out)
    _marshal_inputs([residual], norm_out)
    _marshal_inputs([residual], residual_out)
    _check_gamma(gamma, H, residual_out.device)
    s = _stream_handle(stream, residual_out.device)
    _check(lib().ar_residual_rmsnorm_unfused(ptrs, W, M, H, dt, residual.data_ptr(),
                                             gamma.data_ptr(), float(eps),
                                             residual_out.data_ptr(), norm_out.data_ptr(), s),
           "ar_residual_rmsnorm_unfused")


def ar_rmsnorm(x, gamma, eps: float, y, stream=None) -> None:
    """y = RMSNorm(x) * gamma row by row (the normalisation step alone); any row width."""
    _marshal_inputs([x], y)
    M, H = y.shape
    _check_gamma(gamma, H, y.device)
    s = _stream_handle(stream, y.device)
    _check(lib().ar_rmsnorm(x.data_ptr(), M, H, dtype_code(y.dtype), gamma.data_ptr(),
                            float(eps), y.data_ptr(), s), "ar_rmsnorm")


def ar_row_partition(W: int, M: int, rank: int):
    """(row_begin, row_count) of `rank`'s slice in the W-way row partition (two-shot share)."""
    b, c = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(lib().ar_row_partition(W, M, rank, ctypes.byref(b), ctypes.byref(c)),
           "ar_row_partition")
    return int(b.value), int(c.value)


def ar_all_gather(slices, out, stream=None) -> None:
    """All-gather share: out[row_begin(j):row_begin(j)+row_count(j)] = slices[j] for all j."""
    if out.dim() != 2:
        raise ValueError("out must be [M, H]")
    M, H = out.shape
    W = len(slices)
    if W == 0:
        raise ValueError("need at least one slice")
    ptrs = []
    for j, t in enumerate(slices):
        b, c = ar_row_partition(W, M, j)
        if t.dtype != out.dtype or tuple(t.shape) != (c, H):
            raise ValueError("slice %d must be [%d, %d] %s" % (j, c, H, out.dtype))
        if c and (not t.is_cuda or t.device != out.device or not t.is_contiguous()):
            raise ValueError("slice %d must be a contiguous tensor on %s" % (j, out.device))
        ptrs.append(t.data_ptr() if c else 0)
    if not out.is_contiguous() or not out.is_cuda:
        raise ValueError("out must be a contiguous GPU tensor")
    arr = (ctypes.c_void_p * W)(*ptrs)
    st = lib().ar_all_gather(arr, W, M, H, dtype_code(out.dtype), out.data_ptr(),
                             _stream_handle(stream, out.device))
    _check(st, "ar_all_gather")


LAMPORT_BUFFERS = 3


def _check_rbuf(rbuf, like=None):
    if rbuf.dim() != 4 or rbuf.shape[0] != LAMPORT_BUFFERS or not rbuf.is_cuda \
            or not rbuf.is_contiguous():
        raise ValueError("rbuf must be a contiguous [%d, W, M, H] GPU tensor" % LAMPORT_BUFFERS)
    if like is not None and (like.dtype != rbuf.dtype or tuple(like.shape) != tuple(rbuf.shape[2:])
                             or like.device != rbuf.device or not like.is_contiguous()):
        raise ValueError("tensor must be a contiguous [M, H] %s on %s" % (rbuf.dtype, rbuf.device))
    _, W, M, H = rbuf.shape
    return W, M, H, dtype_code(rbuf.dtype)


def _check_status(status, device):
    import torch
    if status.dtype != torch.int32 or status.numel() < 1 or status.device != device:
        raise ValueError("status must be an int32 GPU tensor on %s" % device)


def ar_lamport_arm(rbuf, stream=None) -> None:
    """Empty every slot of the receive buffers rbuf ([3, W, M, H])."""
    W, M, H, dt = _check_rbuf(rbuf)
    _check(lib().ar_lamport_arm(rbuf.data_ptr(), W, M, H, dt, _stream_handle(stream, rbuf.device)),
           "ar_lamport_arm")


def ar_lamport_push(partial, rank: int, rbuf, round: int, stream=None) -> None:
    """Producer of `rank` in round `round`: write `partial` ([M, H]) into its slot of buffer
    round % 3 and empty its slot of buffer (round + 1) % 3."""
    W, M, H, dt = _check_rbuf(rbuf, partial)
    _check(lib().ar_lamport_push(partial.data_ptr(), rank, rbuf.data_ptr(), W, M, H, dt, round,
                                 _stream_handle(stream, rbuf.device)), "ar_lamport_push")


def ar_lamport_sum(rbuf, round: int, out, status, spin_limit: int = 0, stream=None) -> None:
    """Consumer of round `round`, kAllReduce: out = sum of the W slots of buffer round % 3."""
    W, M, H, dt = _check_rbuf(rbuf, out)
    _check_status(status, rbuf.device)
    _check(lib().ar_lamport_sum(rbuf.data_ptr(), W, M, H, dt, round, out.data_ptr(),
                                status.data_ptr(), spin_limit, _stream_handle(stream, rbuf.device)),
           "ar_lamport_sum")


def ar_lamport_residual_rmsnorm(rbuf, round: int, residual, gamma, eps: float, residual_out,
                                norm_out, status, spin_limit: int = 0, stream=None) -> None:
    """Consumer of round `round`, kARResidualRMSNorm over the W slots of buffer round % 3."""
    import torch
    W, M, H, dt = _check_rbuf(rbuf, residual)
    _check_rbuf(rbuf, residual_out)
    _check_rbuf(rbuf, norm_out)
    _check_status(status, rbuf.device)
    if gamma.dtype != torch.float32 or tuple(gamma.shape) != (H,) or not gamma.is_contiguous() \
            or gamma.device != rbuf.device:
        raise ValueError("gamma must be a contiguous float32 [%d] tensor on %s" % (H, rbuf.device))
    st = lib().ar_lamport_residual_rmsnorm(
        rbuf.data_ptr(), W, M, H, dt, round, residual.data_ptr(), gamma.data_ptr(), float(eps),
        residual_out.data_ptr(), norm_out.data_ptr(), status.data_ptr(), spin_limit,
        _stream_handle(stream, rbuf.device))
    _check(st, "ar_lamport_residual_rmsnorm")


def ar_policy_default(W: int) -> Dict[str, int]:
    p = Policy()
    _check(lib().ar_policy_default(W, ctypes.byref(p)), "ar_policy_default")
    return p.as_dict()


def ar_route(pattern: int, W: int, M: int, H: int, dtype: int,
             policy: Optional[Dict[str, int]] = None) -> int:
    """ROUTE_ONE_SHOT, ROUTE_TWO_SHOT, ROUTE_FALLBACK or ROUTE_UNFUSED for this call (default
    policy if None)."""
    p = Policy(**(policy if policy is not None else ar_policy_default(W if W >= 1 else 1)))
    r = ctypes.c_int(-1)
    _check(lib().ar_route(pattern, W, M, H, dtype, ctypes.byref(p), ctypes.byref(r)), "ar_route")
    return int(r.value)


def ar_allreduce_routed(inputs, out, residual=None, gamma=None, eps: float = 1e-6,
                        norm_out=None, rank: int = 0, policy: Optional[Dict[str, int]] = None,
                        stream=None) -> int:
    """Run the call on the path ar_route picks (kARResidualRMSNorm when `residual` is given,
    `out` then being residual_out; else kAllReduce) and return the route taken.  A two-shot route
    writes only this rank's row slice; a fallback route raises ArError (AR_ERR_UNSUPPORTED)."""
    import torch
    ptrs, W, M, H, dt = _marshal_inputs(inputs, out)
    pattern = PATTERN_ALLREDUCE
    res_p = gam_p = no_p = None
    if residual is not None:
        pattern = PATTERN_AR_RESIDUAL_RMSNORM
        if norm_out is None or gamma is None:
            raise ValueError("kARResidualRMSNorm needs gamma and norm_out")
        _marshal_inputs([residual], norm_out)
        _marshal_inputs([residual], out)
        if gamma.dtype != torch.float32 or tuple(gamma.shape) != (H,) \
                or not gamma.is_contiguous() or gamma.device != out.device:
            raise ValueError("gamma must be a contiguous float32 [%d] tensor on %s"
                             % (H, out.device))
        res_p, gam_p, no_p = residual.data_ptr(), gamma.data_ptr(), norm_out.data_ptr()
    p = Policy(**(policy if policy is not None else ar_policy_default(W)))
    r = ctypes.c_int(-1)
    st = lib().ar_allreduce_routed(pattern, ptrs, W, M, H, dt, res_p, gam_p, float(eps),
                                   out.data_ptr(), no_p, rank, ctypes.byref(p), ctypes.byref(r),
                                   _stream_handle(stream, out.device))
    _check(st, "ar_allreduce_routed")
    return int(r.value)


def ar_supports(pattern: int, W: int, M: int, H: int, dtype: int) -> int:
    """Status the pattern would return for this shape (AR_OK if supported); no device access."""
    return int(lib().ar_supports(pattern, W, M, H, dtype))


def ar_launch_config(pattern: int, W: int, M: int, H: int, dtype: int,
                     cu_count: int = 0) -> Dict[str, int]:
    """The launch shape the library picks (cu_count <= 0: query the current device)."""
    cfg = LaunchConfig()
    _check(lib().ar_launch_config(pattern, W, M, H, dtype, cu_count, ctypes.byref(cfg)),
           "ar_launch_config")
    return cfg.as_dict()


def ar_device_cu_count() -> int:
    n = ctypes.c_int(0)
    _check(lib().ar_device_cu_count(ctypes.byref(n)), "ar_device_cu_count")
    return int(n.value)


def ar_status_string(status: int) -> str:
    return status_string(status)
