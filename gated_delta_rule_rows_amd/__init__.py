"""MI355X KDA verify-row scan: Python binding of libkda.so.

Argument marshalling only.  Every step of the scan, the snapshot, the replay
and the batched arm runs in the gfx950 kernels behind the C ABI declared in
include/kda.h; this module turns torch tensors into device pointers and
sizes, passes torch's current HIP stream, and raises on a nonzero status.
There is no CPU path: if libkda.so is missing or was built for another GPU
the calls fail loudly.

Shapes (D = 128):
  state            [L][H][D][D] float32
  q, k, v, g       [L][T][H][D] float32 or bfloat16 (all five the same dtype)
  beta             [L][T][H]
  o                [L][T][H][D] float32 or None
  batched arm      rows [L][B][H][D], beta [L][B][H], o [L][B][H][D];
                   s_ptrs = state_table(...) -> int64 device tensor [L*B]
"""
from __future__ import annotations

import ctypes
import os

import torch

D = 128
T_MAX = 15
B_MAX = 15
KDA_IN_F32 = 0
KDA_IN_BF16 = 1

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")
_lib = None


class KdaError(RuntimeError):
    """A refusal or launch failure reported by libkda.so (message from kda_last_error)."""

    def __init__(self, status: int, message: str):
        super().__init__(f"[status {status}] {message}")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libkda.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is not built; run `python -m gated_delta_rule_rows_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    p, i = ctypes.c_void_p, ctypes.c_int
    lib.kda_scan_rows.argtypes = [p, p, p, p, p, p, p, p, i, i, i, i, p]
    lib.kda_snapshot.argtypes = [p, p, i, i, p]
    lib.kda_replay.argtypes = [p, p, p, p, p, p, p, i, i, i, i, i, p]
    lib.kda_scan_batched.argtypes = [p, p, p, p, p, p, p, i, i, i, i, p]
    for fn in (lib.kda_scan_rows, lib.kda_snapshot, lib.kda_replay, lib.kda_scan_batched,
               lib.kda_abi_version):
        fn.restype = i
    lib.kda_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != 0:
        raise KdaError(rc, _lib.kda_last_error().decode())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(t: torch.Tensor | None, name: str):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _in_dtype(rows) -> int:
    dt = rows[0].dtype
    if any(x.dtype != dt for x in rows):
        raise TypeError("q, k, v, g, beta must share one dtype")
    if dt == torch.float32:
        return KDA_IN_F32
    if dt == torch.bfloat16:
        return KDA_IN_BF16
    raise TypeError(f"row inputs must be float32 or bfloat16, got {dt}")


def _shape(t: torch.Tensor, shape, name: str):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _f32(t: torch.Tensor, name: str):
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")


def _rows_shape(q, k, v, g, beta):
    if q.dim() != 4 or q.shape[-1] != D:
        raise ValueError(f"q must be [L][T][H][{D}], got {tuple(q.shape)}")
    L, T, H, _ = q.shape
    for x, n in ((k, "k"), (v, "v"), (g, "g")):
        _shape(x, q.shape, n)
    _shape(beta, (L, T, H), "beta")
    return L, T, H


def kda_scan_rows(s_in, s_out, q, k, v, g, beta, o=None, stream=None) -> None:
    """Scan the T rows of q/k/v/g/beta over every (layer, head) state.

    s_out may be s_in (in place); a distinct s_out leaves s_in as the snapshot.
    """
    lib = load()
    L, T, H = _rows_shape(q, k, v, g, beta)
    for st, n in ((s_in, "s_in"), (s_out, "s_out")):
        _shape(st, (L, H, D, D), n)
        _f32(st, n)
    if o is not None:
        _shape(o, (L, T, H, D), "o")
        _f32(o, "o")
    dt = _in_dtype((q, k, v, g, beta))
    _check(lib.kda_scan_rows(_dev(s_in, "s_in"), _dev(s_out, "s_out"), _dev(q, "q"), _dev(k, "k"),
                             _dev(v, "v"), _dev(g, "g"), _dev(beta, "beta"), _dev(o, "o"),
                             L, T, H, dt, _stream(stream)))


def kda_snapshot(s, snap, stream=None) -> None:
    """snap = s (device copy of [L][H][D][D] states)."""
    lib = load()
    if s.dim() != 4 or tuple(s.shape[2:]) != (D, D):
        raise ValueError(f"s must be [L][H][{D}][{D}], got {tuple(s.shape)}")
    _shape(snap, s.shape, "snap")
    _f32(s, "s")
    _f32(snap, "snap")
    L, H = s.shape[0], s.shape[1]
    _check(lib.kda_snapshot(_dev(s, "s"), _dev(snap, "snap"), L, H, _stream(stream)))


def kda_replay(snap, s_out, q, k, v, g, beta, keep: int, stream=None) -> None:
    """s_out = state after rows 0..keep-1 of the round, rebuilt from snap.

    q..beta are the round's retained inputs ([L][T_round][H]...); keep = j + 1.
    """
    lib = load()
    L, T_round, H = _rows_shape(q, k, v, g, beta)
    for st, n in ((snap, "snap"), (s_out, "s_out")):
        _shape(st, (L, H, D, D), n)
        _f32(st, n)
    dt = _in_dtype((q, k, v, g, beta))
    _check(lib.kda_replay(_dev(snap, "snap"), _dev(s_out, "s_out"), _dev(q, "q"), _dev(k, "k"),
                          _dev(v, "v"), _dev(g, "g"), _dev(beta, "beta"), L, T_round, int(keep), H,
                          dt, _stream(stream)))


def state_table(states, device=None) -> torch.Tensor:
    """Device pointer table for the batched arm.

    states: nested list [L][B] of [H][D][D] float32 device tensors (session b's
    layer-l state), or one tensor [L][B][H][D][D].  Returns int64 [L*B].
    """
    if isinstance(states, torch.Tensor):
        if states.dim() != 5 or tuple(states.shape[3:]) != (D, D):
            raise ValueError("state tensor must be [L][B][H][D][D]")
        _f32(states, "states")
        if not (states.is_cuda and states.is_contiguous()):
            raise ValueError("states must be a contiguous device tensor")
        L, B, H = states.shape[:3]
        base = states.data_ptr()
        ptrs = [base + (lb * H * D * D) * 4 for lb in range(L * B)]
        device = states.device
    else:
        ptrs = []
        for row in states:
            for t in row:
                if not (t.is_cuda and t.is_contiguous()) or t.dtype != torch.float32:
                    raise ValueError("each state must be a contiguous float32 device tensor")
                if t.dim() != 3 or tuple(t.shape[1:]) != (D, D):
                    raise ValueError("each state must be [H][D][D]")
                ptrs.append(t.data_ptr())
                device = device or t.device
    return torch.tensor(ptrs, dtype=torch.int64, device=device)


def kda_scan_batched(s_ptrs, q, k, v, g, beta, o=None, stream=None) -> None:
    """Batched-decode arm: rows [L][B][H][D], one per session, states updated in place."""
    lib = load()
    L, B, H = _rows_shape(q, k, v, g, beta)
    if s_ptrs.dtype != torch.int64:
        raise TypeError("s_ptrs must be an int64 device tensor")
    _shape(s_ptrs, (L * B,), "s_ptrs")
    if o is not None:
        _shape(o, (L, B, H, D), "o")
        _f32(o, "o")
    dt = _in_dtype((q, k, v, g, beta))
    _check(lib.kda_scan_batched(_dev(s_ptrs, "s_ptrs"), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"),
                                _dev(g, "g"), _dev(beta, "beta"), _dev(o, "o"), L, B, H, dt,
                                _stream(stream)))


def kda_abi_version() -> int:
    return int(load().kda_abi_version())


def kda_last_error() -> str:
    return load().kda_last_error().decode()


__all__ = [
    "D", "T_MAX", "B_MAX", "KdaError", "load", "lib_path", "kda_scan_rows", "kda_snapshot",
    "kda_replay", "kda_scan_batched", "state_table", "kda_abi_version", "kda_last_error",
]
