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
  e (stash plane)  [L][T][H][D] float32 or None: per-row delta vectors a scan
                   writes and a replay (or the next fused round) reads
  batched arm      rows [L][B][H][D], beta [L][B][H], o [L][B][H][D];
                   s_ptrs = state_table(...) -> int64 device tensor [L*B]
  row ops          x [L][T][3*H*D], a [L][T][H*D], b [L][T][H] (float32 or
                   bfloat16), conv_w [L][3*H*D][4], ring [L][3][3*H*D] float32
  conv ring        ring [L][3][C] float32, raw conv input rows [L][T][C]
  batched copy     table = copy_table(srcs, dsts) -> int64 device tensor [2n]
  greedy accept    logits [t][V] (row stride free, elements contiguous),
                   drafts [t-1], vam [t], out2 [2] as int32 or uint32,
                   work = accept_workspace()
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
ACCEPT_WORK_BYTES = 12288
NO_TOKEN = 0xFFFFFFFF
RING_ROWS = 3
MAX_PREV_ROUNDS = 4


class _PrevRound(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("g", ctypes.c_void_p),
                ("beta", ctypes.c_void_p), ("e", ctypes.c_void_p), ("T", ctypes.c_int),
                ("keep", ctypes.c_int)]

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
    lib.kda_scan_rows_stash.argtypes = [p, p, p, p, p, p, p, p, p, i, i, i, i, p]
    lib.kda_scan_rows_columns.argtypes = [p, p, p, p, p, p, p, p, p, i, i, i, i, p]
    lib.kda_snapshot.argtypes = [p, p, i, i, p]
    lib.kda_replay.argtypes = [p, p, p, p, p, p, p, i, i, i, i, i, p]
    lib.kda_replay_stash.argtypes = [p, p, p, p, p, i, i, i, i, i, p]
    lib.kda_scan_batched.argtypes = [p, p, p, p, p, p, p, i, i, i, i, p]
    lib.kda_verify_round.argtypes = [p, p, p, p, p, p, p, i, i, p, p, p, p, p, p, p,
                                     i, i, i, i, p]
    lib.kda_accept_greedy.argtypes = [p, i, i, ctypes.c_longlong, i, p, p, p, p, p]
    lib.kda_accept_greedy_noalloc.argtypes = [p, i, i, ctypes.c_longlong, i, p, p, p, p]
    lib.kda_conv_reroll.argtypes = [p, p, p, i, i, i, ctypes.c_longlong, i, p]
    lib.kda_conv_reroll_dev.argtypes = [p, p, p, i, i, p, ctypes.c_longlong, i, p]
    lib.kda_verify_round_dev.argtypes = [p, p, p, p, p, p, p, i, p, p, p, p, p, p, p, p,
                                         i, i, i, i, p]
    lib.kda_copy_batch.argtypes = [p, i, ctypes.c_longlong, p]
    lib.kda_row_ops.argtypes = [p] * 11 + [i, i, i, i, p]
    lib.kda_verify_round_multi.argtypes = [p, p, ctypes.POINTER(_PrevRound), i, p, p, p, p, p,
                                           p, p, i, i, i, i, p]
    for fn in (lib.kda_scan_rows, lib.kda_snapshot, lib.kda_replay, lib.kda_scan_batched,
               lib.kda_verify_round, lib.kda_accept_greedy, lib.kda_conv_reroll,
               lib.kda_copy_batch, lib.kda_row_ops, lib.kda_verify_round_multi,
               lib.kda_scan_rows_columns, lib.kda_verify_round_dev, lib.kda_conv_reroll_dev,
               lib.kda_scan_rows_stash, lib.kda_replay_stash, lib.kda_accept_greedy_noalloc,
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


def _state(t, shape, name):
    _shape(t, shape, name)
    _f32(t, name)


def _plane(t, shape, name):
    """An optional f32 [.., D] plane (o or the stash e)."""
    if t is not None:
        _shape(t, shape, name)
        _f32(t, name)


def kda_scan_rows(s_in, s_out, q, k, v, g, beta, o=None, stream=None) -> None:
    """Scan the T rows of q/k/v/g/beta over every (layer, head) state.

    s_out may be s_in (in place); a distinct s_out leaves s_in as the snapshot.
    o (optional) receives the outputs.
    """
    lib = load()
    L, T, H = _rows_shape(q, k, v, g, beta)
    _state(s_in, (L, H, D, D), "s_in")
    _state(s_out, (L, H, D, D), "s_out")
    _plane(o, (L, T, H, D), "o")
    dt = _in_dtype((q, k, v, g, beta))
    _check(lib.kda_scan_rows(_dev(s_in, "s_in"), _dev(s_out, "s_out"), _dev(q, "q"), _dev(k, "k"),
                             _dev(v, "v"), _dev(g, "g"), _dev(beta, "beta"), _dev(o, "o"),
                             L, T, H, dt, _stream(stream)))


def kda_scan_rows_stash(s_in, s_out, q, k, v, g, beta, o, e, stream=None) -> None:
    """kda_scan_rows that also writes the stash plane e [L][T][H][D] (float32,
    required): each row's delta vector, read by kda_replay_stash and the fused
    round.  o may be None."""
    lib = load()
    L, T, H = _rows_shape(q, k, v, g, beta)
    _state(s_in, (L, H, D, D), "s_in")
    _state(s_out, (L, H, D, D), "s_out")
    _plane(o, (L, T, H, D), "o")
    if e is None:
        raise ValueError("e is required")
    _plane(e, (L, T, H, D), "e")
    dt = _in_dtype((q, k, v, g, beta))
    _check(lib.kda_scan_rows_stash(_dev(s_in, "s_in"), _dev(s_out, "s_out"), _dev(q, "q"),
                                   _dev(k, "k"), _dev(v, "v"), _dev(g, "g"), _dev(beta, "beta"),
                                   _dev(o, "o"), _dev(e, "e"), L, T, H, dt, _stream(stream)))


def kda_scan_rows_columns(s_in, s_cols, q, k, v, g, beta, o, e=None, stream=None) -> None:
    """The state-column variant: scan T rows and keep the state after every row.

    s_cols is [T][L][H][D][D]; s_cols[t] is the state after rows 0..t, so a
    round that accepts keep rows continues from s_cols[keep - 1].  s_in is
    left untouched; o is required.
    """
    lib = load()
    L, T, H = _rows_shape(q, k, v, g, beta)
    _state(s_in, (L, H, D, D), "s_in")
    _state(s_cols, (T, L, H, D, D), "s_cols")
    if o is None:
        raise ValueError("o is required")
    _plane(o, (L, T, H, D), "o")
    _plane(e, (L, T, H, D), "e")
    dt = _in_dtype((q, k, v, g, beta))
    _check(lib.kda_scan_rows_columns(_dev(s_in, "s_in"), _dev(s_cols, "s_cols"), _dev(q, "q"),
                                     _dev(k, "k"), _dev(v, "v"), _dev(g, "g"),
                                     _dev(beta, "beta"), _dev(o, "o"), _dev(e, "e"), L, T, H, dt,
                                     _stream(stream)))


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


def _kept_rows(k, v, g, beta, e, what):
    """Shape check of a round's retained rows; v and beta may be None when e is given."""
    if k.dim() != 4 or k.shape[-1] != D:
        raise ValueError(f"{what} k must be [L][T][H][{D}], got {tuple(k.shape)}")
    L, T, H, _ = k.shape
    _shape(g, k.shape, f"{what} g")
    present = [k, g]
    if e is None or v is not None:
        if v is None or beta is None:
            raise ValueError(f"{what}: v and beta are needed without the stash plane e")
        _shape(v, k.shape, f"{what} v")
        _shape(beta, (L, T, H), f"{what} beta")
        present += [v, beta]
    _plane(e, (L, T, H, D), f"{what} e")
    return L, T, H, _in_dtype(present)


def kda_replay(snap, s_out, q, k, v, g, beta, keep: int, stream=None) -> None:
    """s_out = state after rows 0..keep-1 of the round, rebuilt from snap.

    q, k, v, g [L][T_round][H][D] and beta [L][T_round][H] are the round's
    retained inputs, the tensors given to its kda_scan_rows (q is not read);
    keep = j + 1.
    """
    lib = load()
    L, T_round, H = _rows_shape(q, k, v, g, beta)
    dt = _in_dtype((q, k, v, g, beta))
    _state(snap, (L, H, D, D), "snap")
    _state(s_out, (L, H, D, D), "s_out")
    _check(lib.kda_replay(_dev(snap, "snap"), _dev(s_out, "s_out"), _dev(q, "q"), _dev(k, "k"),
                          _dev(v, "v"), _dev(g, "g"), _dev(beta, "beta"), L, T_round, int(keep),
                          H, dt, _stream(stream)))


def kda_replay_stash(snap, s_out, k, g, e, keep: int, stream=None) -> None:
    """kda_replay from the round's stash plane e (written by kda_scan_rows_stash):
    only k, g [L][T_round][H][D] and e are read; same bits as kda_replay."""
    lib = load()
    if e is None:
        raise ValueError("e is required")
    L, T_round, H, dt = _kept_rows(k, None, g, None, e, "replay")
    _state(snap, (L, H, D, D), "snap")
    _state(s_out, (L, H, D, D), "s_out")
    _check(lib.kda_replay_stash(_dev(snap, "snap"), _dev(s_out, "s_out"), _dev(k, "k"),
                                _dev(g, "g"), _dev(e, "e"), L, T_round, int(keep), H, dt,
                                _stream(stream)))


def _j_dev(j):
    """The accepted-draft count on the device: a 1-element (or out2-style) int32
    or uint32 tensor whose first element is j."""
    if not (isinstance(j, torch.Tensor) and j.is_cuda):
        raise TypeError("a device keep is given as j, a device tensor (kda_accept_greedy's out2)")
    if j.dtype not in (torch.int32, torch.uint32) or j.numel() < 1 or not j.is_contiguous():
        raise ValueError("j must be a contiguous int32 tensor with j at element 0")
    return ctypes.c_void_p(j.data_ptr())


def kda_verify_round(snap_prev, snap_out, prev, keep, q, k, v, g, beta, o, e=None,
                     stream=None) -> None:
    """One fused verify round.

    prev = (k, v, g, beta, e) of the previous round (v/beta may be None when its
    stash e is given; prev may be None when keep == 0).  snap_out receives
    snap_prev advanced by the previous round's first `keep` rows (this round's
    snapshot); o receives this round's outputs, e (optional) its stash plane.
    keep is an int, or a device tensor j (kda_accept_greedy's out2) for keep =
    j + 1 read on the device (kda_verify_round_dev).
    """
    lib = load()
    L, T, H = _rows_shape(q, k, v, g, beta)
    dt = _in_dtype((q, k, v, g, beta))
    _state(snap_prev, (L, H, D, D), "snap_prev")
    _state(snap_out, (L, H, D, D), "snap_out")
    _plane(o, (L, T, H, D), "o")
    _plane(e, (L, T, H, D), "e")
    if prev is None:
        if keep != 0:
            raise ValueError("keep > 0 needs the previous round's rows")
        pk = pv = pg = pb = pe = None
        T_prev = 0
    else:
        pk, pv, pg, pb, pe = prev
        Lp, T_prev, Hp, pdt = _kept_rows(pk, pv, pg, pb, pe, "prev")
        if (Lp, Hp) != (L, H) or pdt != dt:
            raise ValueError("previous round's rows do not match this round's L, H, dtype")
    if isinstance(keep, torch.Tensor):
        if prev is None:
            raise ValueError("a device keep needs the previous round's rows")
        _check(lib.kda_verify_round_dev(
            _dev(snap_prev, "snap_prev"), _dev(snap_out, "snap_out"), _dev(pk, "pk"),
            _dev(pv, "pv"), _dev(pg, "pg"), _dev(pb, "pbeta"), _dev(pe, "pe"), int(T_prev),
            _j_dev(keep), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(g, "g"),
            _dev(beta, "beta"), _dev(o, "o"), _dev(e, "e"), L, T, H, dt, _stream(stream)))
        return
    _check(lib.kda_verify_round(
        _dev(snap_prev, "snap_prev"), _dev(snap_out, "snap_out"), _dev(pk, "pk"), _dev(pv, "pv"),
        _dev(pg, "pg"), _dev(pb, "pbeta"), _dev(pe, "pe"), int(T_prev), int(keep), _dev(q, "q"),
        _dev(k, "k"), _dev(v, "v"), _dev(g, "g"), _dev(beta, "beta"), _dev(o, "o"),
        _dev(e, "e"), L, T, H, dt, _stream(stream)))


def kda_verify_round_multi(snap_base, snap_out, prevs, q, k, v, g, beta, o, e=None,
                           stream=None) -> None:
    """A fused round replaying several earlier rounds.

    prevs: up to 4 tuples (k, v, g, beta, e, keep), oldest first, each an earlier
    round's retained rows ([L][T_i][H][D]; v/beta may be None when its stash e is
    given) and how many of them to replay.  snap_base is the committed state
    before prevs[0].  snap_out (or None to skip the store) receives the
    committed state after all of them; o (and e) this round's outputs.
    """
    lib = load()
    L, T, H = _rows_shape(q, k, v, g, beta)
    dt = _in_dtype((q, k, v, g, beta))
    _state(snap_base, (L, H, D, D), "snap_base")
    if snap_out is not None:
        _state(snap_out, (L, H, D, D), "snap_out")
    _plane(o, (L, T, H, D), "o")
    _plane(e, (L, T, H, D), "e")
    if len(prevs) > MAX_PREV_ROUNDS:
        raise ValueError(f"at most {MAX_PREV_ROUNDS} earlier rounds")
    arr = (_PrevRound * max(1, len(prevs)))()
    for n, (pk, pv, pg, pb, pe, keep) in enumerate(prevs):
        Lp, Tp, Hp, pdt = _kept_rows(pk, pv, pg, pb, pe, f"prevs[{n}]")
        if (Lp, Hp) != (L, H) or pdt != dt:
            raise ValueError(f"prevs[{n}] does not match this round's L, H, dtype")
        ptr = lambda t, nm: None if t is None else _dev(t, f"prevs[{n}] {nm}").value
        arr[n] = _PrevRound(ptr(pk, "k"), ptr(pv, "v"), ptr(pg, "g"), ptr(pb, "beta"),
                            ptr(pe, "e"), Tp, int(keep))
    _check(lib.kda_verify_round_multi(
        _dev(snap_base, "snap_base"), _dev(snap_out, "snap_out"), arr, len(prevs), _dev(q, "q"),
        _dev(k, "k"), _dev(v, "v"), _dev(g, "g"), _dev(beta, "beta"), _dev(o, "o"),
        _dev(e, "e"), L, T, H, dt, _stream(stream)))


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


def accept_workspace(device=None) -> torch.Tensor:
    """Scratch for kda_accept_greedy (uint8 [ACCEPT_WORK_BYTES], contents irrelevant).

    One workspace serves any number of calls issued on one stream; calls that
    may run at the same time on different streams need their own.
    """
    return torch.empty(ACCEPT_WORK_BYTES, dtype=torch.uint8,
                       device=device if device is not None else "cuda")


def _u32(t, n, name):
    if t.dtype not in (torch.int32, torch.uint32):
        raise TypeError(f"{name} must be int32 or uint32")
    _shape(t, (n,), name)


def _accept_args(logits, drafts, vam, out2):
    if not isinstance(logits, torch.Tensor) or logits.dim() != 2:
        raise ValueError("logits must be a [t][V] tensor")
    if not logits.is_cuda:
        raise ValueError("logits must be a device tensor")
    t, V = logits.shape
    if logits.dtype == torch.float32:
        dt = KDA_IN_F32
    elif logits.dtype == torch.bfloat16:
        dt = KDA_IN_BF16
    else:
        raise TypeError(f"logits must be float32 or bfloat16, got {logits.dtype}")
    if V > 1 and logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous")
    ld = logits.stride(0) if t > 1 else V
    if drafts is not None:
        _u32(drafts, max(t - 1, 0), "drafts")
    _u32(vam, t, "vam")
    _u32(out2, 2, "out2")
    lp = ctypes.c_void_p(logits.data_ptr())
    dp = _dev(drafts, "drafts") if drafts is not None and t > 1 else None
    return lp, int(t), int(V), int(ld), dt, dp, _dev(vam, "vam"), _dev(out2, "out2")


def kda_accept_greedy_noalloc(logits, drafts, vam, out2, stream=None) -> None:
    """kda_accept_greedy without a workspace: the partial argmaxes go to the
    library's static device array (one per GPU, shared by every call on it, so
    calls that may overlap on one GPU must not use this form)."""
    lib = load()
    _check(lib.kda_accept_greedy_noalloc(*_accept_args(logits, drafts, vam, out2),
                                         _stream(stream)))


def kda_accept_greedy(logits, drafts, vam, out2, work, stream=None) -> None:
    """Greedy accept: vam[r] = argmax of logits row r (lowest index on ties,
    NO_TOKEN for a row holding a NaN), out2 = (j, bonus) with j the number of
    leading drafts equal to vam and bonus = vam[j].

    logits: [t][V] float32 or bfloat16, unit element stride (any row stride).
    drafts: [t-1] token ids (None allowed when t == 1).
    """
    lib = load()
    args = _accept_args(logits, drafts, vam, out2)
    if work.dtype != torch.uint8 or work.numel() < ACCEPT_WORK_BYTES:
        raise ValueError(f"work must be a uint8 tensor of >= {ACCEPT_WORK_BYTES} bytes")
    _check(lib.kda_accept_greedy(*args, _dev(work, "work"), _stream(stream)))


def kda_row_ops(x, a, b, conv_w, ring_in, q, k, v, g, beta, ring_out=None, stream=None) -> None:
    """Scan inputs from one round's projections: causal short conv + SiLU over the
    ring, q/k L2 norm, bounded gate, beta sigmoid (see include/kda.h).  ring_out
    (optional, may be ring_in) receives the ring after all T rows."""
    lib = load()
    if x.dim() != 3 or x.shape[2] % (3 * D) != 0:
        raise ValueError(f"x must be [L][T][3*H*{D}], got {tuple(x.shape)}")
    L, T, C = x.shape
    H = C // (3 * D)
    _shape(a, (L, T, H * D), "a")
    _shape(b, (L, T, H), "b")
    _state(conv_w, (L, C, 4), "conv_w")
    _state(ring_in, (L, RING_ROWS, C), "ring_in")
    if ring_out is not None:
        _state(ring_out, (L, RING_ROWS, C), "ring_out")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (g, "g")):
        _state(t, (L, T, H, D), n)
    _state(beta, (L, T, H), "beta")
    dt = _in_dtype((x, a, b))
    _check(lib.kda_row_ops(_dev(x, "x"), _dev(a, "a"), _dev(b, "b"), _dev(conv_w, "conv_w"),
                           _dev(ring_in, "ring_in"), _dev(ring_out, "ring_out"), _dev(q, "q"),
                           _dev(k, "k"), _dev(v, "v"), _dev(g, "g"), _dev(beta, "beta"),
                           L, T, H, dt, _stream(stream)))


def kda_conv_reroll(ring_snap, raw, keep, ring_out, stream=None) -> None:
    """ring_out = the short-conv ring after `keep` accepted rows: ring_snap [L][3][C]
    rolled once per kept row over the round's raw conv inputs raw [L][T_round][C].
    keep is an int, or a device tensor j for keep = j + 1 read on the device."""
    lib = load()
    if raw.dim() != 3:
        raise ValueError(f"raw must be [L][T_round][C], got {tuple(raw.shape)}")
    L, T, C = raw.shape
    _state(ring_snap, (L, RING_ROWS, C), "ring_snap")
    _state(ring_out, (L, RING_ROWS, C), "ring_out")
    dt = _in_dtype((raw,))
    if isinstance(keep, torch.Tensor):
        _check(lib.kda_conv_reroll_dev(_dev(ring_snap, "ring_snap"), _dev(raw, "raw"),
                                       _dev(ring_out, "ring_out"), L, T, _j_dev(keep), C, dt,
                                       _stream(stream)))
        return
    _check(lib.kda_conv_reroll(_dev(ring_snap, "ring_snap"), _dev(raw, "raw"),
                               _dev(ring_out, "ring_out"), L, T, int(keep), C, dt,
                               _stream(stream)))


def copy_table(srcs, dsts, device=None) -> torch.Tensor:
    """Device pointer table [src_0..src_{n-1}, dst_0..dst_{n-1}] (int64) for
    kda_copy_batch.  Every buffer is a contiguous float32 device tensor of one size."""
    if len(srcs) != len(dsts) or not srcs:
        raise ValueError("need as many destinations as sources, at least one")
    words = srcs[0].numel()
    for t in list(srcs) + list(dsts):
        if not (isinstance(t, torch.Tensor) and t.is_cuda and t.is_contiguous()):
            raise ValueError("copy buffers must be contiguous device tensors")
        if t.dtype != torch.float32 or t.numel() != words:
            raise ValueError("copy buffers must be float32 tensors of one size")
    ptrs = [t.data_ptr() for t in srcs] + [t.data_ptr() for t in dsts]
    return torch.tensor(ptrs, dtype=torch.int64, device=device or srcs[0].device)


def kda_copy_batch(table, n: int, words: int, stream=None) -> None:
    """Copy n buffers of `words` float32, named by a copy_table, in one launch."""
    lib = load()
    if table.dtype != torch.int64:
        raise TypeError("table must be an int64 device tensor")
    _shape(table, (2 * n,), "table")
    _check(lib.kda_copy_batch(_dev(table, "table"), int(n), int(words), _stream(stream)))


def kda_abi_version() -> int:
    return int(load().kda_abi_version())


def kda_last_error() -> str:
    return load().kda_last_error().decode()


__all__ = [
    "D", "T_MAX", "B_MAX", "KdaError", "load", "lib_path", "kda_scan_rows", "kda_snapshot",
    "kda_replay", "kda_scan_batched", "kda_verify_round", "state_table", "kda_abi_version",
    "kda_last_error", "kda_accept_greedy", "accept_workspace", "ACCEPT_WORK_BYTES", "NO_TOKEN",
    "kda_conv_reroll", "copy_table", "kda_copy_batch", "RING_ROWS", "kda_row_ops",
    "kda_verify_round_multi", "MAX_PREV_ROUNDS", "kda_scan_rows_columns", "kda_scan_rows_stash",
    "kda_replay_stash", "kda_accept_greedy_noalloc",
]
