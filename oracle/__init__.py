"""CPU oracle for the KDA verify-row scan (test infrastructure only).

Only the tests, the smoke check and the bench's CPU-baseline leg use this
package.  It wraps ``kda_oracle.c`` -- a plain, scalar, f64 restatement of the
recurrence (see that file's header for the definition and its sources) --
with numpy arrays in and out.  It imports nothing from the HIP library and
the HIP library imports nothing from it.

Functions
---------
scan_rows(s_in, q, k, v, g, beta, T=None, want_o=True, threads=1)
    Scan rows 0..T-1 of every (layer, head) chain; returns (s_out, o).
replay(snap, q, k, v, g, beta, keep, threads=1)
    The state after rows 0..keep-1, rebuilt from the pre-round snapshot.
batched(states, q, k, v, g, beta, want_o=True, threads=1)
    B independent sessions, one row each; returns (new_states, o).
accept_greedy(logits, drafts)
    Per-row argmax (lowest index wins; NaN row -> 0xFFFFFFFF) and the accepted
    draft count j with its bonus token; returns (vam, j, bonus).

Inputs are float32 arrays, or uint16 arrays holding bf16 bit patterns (all
five row inputs in the same dtype); the oracle widens bf16 itself.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")

D = 128

_lib = None


def build(out: str = _LIB) -> str:
    """Compile the oracle with gcc (strict IEEE: no fast-math, no contraction)."""
    cmd = [
        "gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-pthread",
        "-fno-fast-math", "-ffp-contract=off", "-fno-strict-aliasing",
        _SRC, "-o", out + ".tmp", "-lm", "-lpthread",
    ]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def load():
    """Load the built oracle library, building it first only if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    p = ctypes.c_void_p
    i = ctypes.c_int
    lib.kda_oracle_scan_rows.argtypes = [p, p, p, p, p, p, p, p, i, i, i, i, i, i, i]
    lib.kda_oracle_scan_rows.restype = i
    lib.kda_oracle_batched.argtypes = [p, p, p, p, p, p, p, i, i, i, i, i, i]
    lib.kda_oracle_batched.restype = i
    lib.kda_oracle_accept_greedy.argtypes = [p, i, i, ctypes.c_long, i, p, p, p]
    lib.kda_oracle_accept_greedy.restype = i
    lib.kda_oracle_conv_reroll.argtypes = [p, p, p, i, i, i, ctypes.c_long, i]
    lib.kda_oracle_conv_reroll.restype = i
    lib.kda_oracle_row_ops.argtypes = [p] * 11 + [i, i, i, i, i]
    lib.kda_oracle_row_ops.restype = i
    lib.kda_oracle_version.restype = i
    lib.kda_oracle_max_threads.restype = i
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _rows(q, k, v, g, beta):
    arrs = [np.ascontiguousarray(x) for x in (q, k, v, g, beta)]
    dt = arrs[0].dtype
    if any(a.dtype != dt for a in arrs):
        raise TypeError("q, k, v, g, beta must share one dtype")
    if dt == np.float32:
        bf16 = 0
    elif dt == np.uint16:
        bf16 = 1
    else:
        raise TypeError(f"oracle inputs must be float32 or uint16 (bf16 bits), got {dt}")
    return arrs, bf16


def scan_rows(s_in, q, k, v, g, beta, T=None, want_o=True, threads=1):
    """Scan the first T rows of q/k/v/g [L][T_stride][H][d] and beta [L][T_stride][H].

    s_in: [L][H][d][d] float32 (not modified).  Returns (s_out, o) with o of
    shape [L][T][H][d] (None when want_o is False).
    """
    lib = load()
    (q, k, v, g, beta), bf16 = _rows(q, k, v, g, beta)
    s_in = np.ascontiguousarray(s_in, dtype=np.float32)
    L, T_stride, H, d = q.shape
    if T is None:
        T = T_stride
    if not (0 <= T <= T_stride):
        raise ValueError("T outside 0..T_stride")
    if s_in.shape != (L, H, d, d) or beta.shape != (L, T_stride, H):
        raise ValueError("shape mismatch")
    for x in (k, v, g):
        if x.shape != q.shape:
            raise ValueError("shape mismatch")
    s_out = np.empty_like(s_in)
    o = np.empty((L, T, H, d), np.float32) if want_o else None
    rc = lib.kda_oracle_scan_rows(
        _ptr(s_in), _ptr(s_out), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(o),
        L, T_stride, T, H, d, bf16, int(threads))
    if rc != 0:
        raise MemoryError("oracle work buffer allocation failed")
    return s_out, o


def replay(snap, q, k, v, g, beta, keep, threads=1):
    """State after rows 0..keep-1 of the round, rebuilt from the snapshot; no outputs."""
    s_out, _ = scan_rows(snap, q, k, v, g, beta, T=keep, want_o=False, threads=threads)
    return s_out


def batched(states, q, k, v, g, beta, want_o=True, threads=1):
    """Batched arm.  states: [L][B][H][d][d] float32; rows [L][B][H][d]; beta [L][B][H].

    Returns (new_states, o) without modifying the input array.
    """
    lib = load()
    (q, k, v, g, beta), bf16 = _rows(q, k, v, g, beta)
    L, B, H, d = q.shape
    st = np.array(states, dtype=np.float32, copy=True, order="C")
    if st.shape != (L, B, H, d, d) or beta.shape != (L, B, H):
        raise ValueError("shape mismatch")
    table = (ctypes.c_void_p * (L * B))()
    base = st.ctypes.data
    for lb in range(L * B):
        table[lb] = base + lb * H * d * d * 4
    o = np.empty((L, B, H, d), np.float32) if want_o else None
    rc = lib.kda_oracle_batched(
        ctypes.cast(table, ctypes.c_void_p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        _ptr(o), L, B, H, d, bf16, int(threads))
    if rc != 0:
        raise MemoryError("oracle work buffer allocation failed")
    return st, o


def accept_greedy(logits, drafts):
    """logits [t][V] float32 (or uint16 bf16 bits); drafts: t - 1 token ids."""
    lib = load()
    lg = np.ascontiguousarray(logits)
    if lg.dtype == np.float32:
        bf16 = 0
    elif lg.dtype == np.uint16:
        bf16 = 1
    else:
        raise TypeError("logits must be float32 or uint16 (bf16 bits)")
    t, V = lg.shape
    dr = np.ascontiguousarray(np.asarray(drafts, dtype=np.uint32).reshape(-1))
    if dr.size != t - 1:
        raise ValueError("need t - 1 drafts")
    if dr.size == 0:
        dr = np.zeros(1, np.uint32)
    vam = np.empty(t, np.uint32)
    out2 = np.empty(2, np.uint32)
    rc = lib.kda_oracle_accept_greedy(_ptr(lg), t, V, V, bf16, _ptr(dr), _ptr(vam), _ptr(out2))
    if rc != 0:
        raise ValueError("bad accept arguments")
    return vam, int(out2[0]), int(out2[1])


RING_ROWS = 3   # short-conv kernel size 4 keeps 3 prior raw rows


def conv_reroll(ring_snap, raw, keep):
    """Conv ring after `keep` accepted rows: ring_snap [L][3][C] f32 rolled once per
    kept row over raw [L][T_round][C] (float32, or uint16 bf16 bits)."""
    lib = load()
    rs = np.ascontiguousarray(ring_snap, np.float32)
    rw = np.ascontiguousarray(raw)
    if rw.dtype == np.float32:
        bf16 = 0
    elif rw.dtype == np.uint16:
        bf16 = 1
    else:
        raise TypeError("raw must be float32 or uint16 (bf16 bits)")
    L, T, C = rw.shape
    if rs.shape != (L, RING_ROWS, C):
        raise ValueError("ring_snap must be [L][3][C] matching raw")
    out = np.empty_like(rs)
    if lib.kda_oracle_conv_reroll(_ptr(rs), _ptr(rw), _ptr(out), L, T, int(keep), C, bf16) != 0:
        raise ValueError("bad conv_reroll arguments")
    return out


def row_ops(x, a, b, w, ring_in, H, d=128, want_ring=True):
    """Pre-scan row ops of one round.  x [L][T][3*H*d], a [L][T][H*d], b [L][T][H]
    (float32, or uint16 bf16 bits, all alike), w [L][3*H*d][4] f32, ring_in
    [L][3][3*H*d] f32.  Returns dict q, k, v, g [L][T][H][d], beta [L][T][H] (f32)
    and ring (the ring after all T rows, or None)."""
    lib = load()
    xs = [np.ascontiguousarray(z) for z in (x, a, b)]
    if all(z.dtype == np.float32 for z in xs):
        bf16 = 0
    elif all(z.dtype == np.uint16 for z in xs):
        bf16 = 1
    else:
        raise TypeError("x, a, b must all be float32 or all uint16 (bf16 bits)")
    L, T, C = xs[0].shape
    if C != 3 * H * d or xs[1].shape != (L, T, H * d) or xs[2].shape != (L, T, H):
        raise ValueError("row-op input shapes do not match H, d")
    wc = np.ascontiguousarray(w, np.float32)
    rc = np.ascontiguousarray(ring_in, np.float32)
    if wc.shape != (L, C, 4) or rc.shape != (L, RING_ROWS, C):
        raise ValueError("w must be [L][3*H*d][4] and ring_in [L][3][3*H*d]")
    out = {n: np.empty((L, T, H, d), np.float32) for n in ("q", "k", "v", "g")}
    out["beta"] = np.empty((L, T, H), np.float32)
    ring = np.empty_like(rc) if want_ring else None
    rcode = lib.kda_oracle_row_ops(_ptr(xs[0]), _ptr(xs[1]), _ptr(xs[2]), _ptr(wc), _ptr(rc),
                                   _ptr(ring) if want_ring else None, _ptr(out["q"]),
                                   _ptr(out["k"]), _ptr(out["v"]), _ptr(out["g"]),
                                   _ptr(out["beta"]), L, T, H, d, bf16)
    if rcode != 0:
        raise ValueError("bad row_ops arguments")
    out["ring"] = ring
    return out


def max_threads() -> int:
    return int(load().kda_oracle_max_threads())
