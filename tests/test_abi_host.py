"""The C-ABI library loads, exports what include/kda.h declares, and refuses
bad arguments on the host before anything is enqueued.

No compute happens here: every call below is one that validation must refuse.
Without a GPU the pointers are plain aligned integers (validation never
dereferences them); with a GPU they are real device buffers large enough for
every shape used, so even a validation bug could not read out of bounds.
"""
import ctypes
import os
import re

import pytest

import gated_delta_rule_rows_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, ERR_ARG, ERR_RANGE, ERR_ALIGN, ERR_ALIAS, ERR_HIP = range(6)


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|int)\s+(kda_\w+)\s*\(", text, re.M)))


def _header_constant(name):
    m = re.search(rf"#define\s+{name}\s+(\d+)", open(HEADER).read())
    return int(m.group(1))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.lib_path()):
        from gated_delta_rule_rows_amd import build
        build.build()
    return kda.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) >= {"kda_scan_rows", "kda_snapshot", "kda_replay", "kda_scan_batched",
                          "kda_scan_rows_stash", "kda_replay_stash",
                          "kda_verify_round", "kda_accept_greedy", "kda_conv_reroll",
                          "kda_copy_batch", "kda_row_ops", "kda_verify_round_multi",
                          "kda_scan_rows_columns", "kda_verify_round_dev", "kda_conv_reroll_dev",
                          "kda_last_error", "kda_abi_version"}
    for n in names:
        assert hasattr(lib, n), f"libkda.so does not export {n}"


def test_abi_version_matches_header(lib):
    assert lib.kda_abi_version() == _header_constant("KDA_ABI_VERSION")
    assert _header_constant("KDA_HEAD_DIM") == kda.D == 128
    assert _header_constant("KDA_T_MAX") == kda.T_MAX == 15
    assert _header_constant("KDA_B_MAX") == kda.B_MAX == 15
    assert _header_constant("KDA_ACCEPT_WORK_BYTES") == kda.ACCEPT_WORK_BYTES
    assert re.search(r"#define\s+KDA_NO_TOKEN\s+0xFFFFFFFFu", open(HEADER).read())
    assert kda.NO_TOKEN == 0xFFFFFFFF
    assert _header_constant("KDA_CONV_RING_ROWS") == kda.RING_ROWS == 3
    assert _header_constant("KDA_MAX_PREV_ROUNDS") == kda.MAX_PREV_ROUNDS == 4


class Bufs:
    """Named buffers: real device memory when a GPU is visible, else fake aligned addresses."""

    SIZE = 64 << 20   # bytes per buffer, enough for every shape below

    def __init__(self):
        self.keep = []
        try:
            import torch
            self.gpu = torch.cuda.is_available()
        except Exception:
            self.gpu = False
        self.addr = {}
        for i, n in enumerate(["s_in", "s_out", "q", "k", "v", "g", "beta", "o", "snap", "ptrs"]):
            if self.gpu:
                import torch
                t = torch.zeros(self.SIZE // 4, dtype=torch.float32, device="cuda")
                self.keep.append(t)
                self.addr[n] = t.data_ptr()
            else:
                self.addr[n] = 0x7F0000000000 + i * (1 << 32)

    def __getitem__(self, n):
        return ctypes.c_void_p(self.addr[n])


@pytest.fixture(scope="module")
def b():
    return Bufs()


def _scan(lib, b, **kw):
    a = dict(s_in=b["s_in"], s_out=b["s_out"], q=b["q"], k=b["k"], v=b["v"], g=b["g"],
             beta=b["beta"], o=b["o"], L=2, T=8, H=2, dt=0)
    a.update(kw)
    return lib.kda_scan_rows(a["s_in"], a["s_out"], a["q"], a["k"], a["v"], a["g"], a["beta"],
                             a["o"], a["L"], a["T"], a["H"], a["dt"], None)


def _scan_stash(lib, b, **kw):
    a = dict(s_in=b["s_in"], s_out=b["s_out"], q=b["q"], k=b["k"], v=b["v"], g=b["g"],
             beta=b["beta"], o=b["o"], e=b["ptrs"], L=2, T=8, H=2, dt=0)
    a.update(kw)
    return lib.kda_scan_rows_stash(a["s_in"], a["s_out"], a["q"], a["k"], a["v"], a["g"],
                                   a["beta"], a["o"], a["e"], a["L"], a["T"], a["H"], a["dt"],
                                   None)


def _columns(lib, b, **kw):
    a = dict(s_in=b["s_in"], s_cols=b["s_out"], q=b["q"], k=b["k"], v=b["v"], g=b["g"],
             beta=b["beta"], o=b["o"], e=None, L=2, T=8, H=2, dt=0)
    a.update(kw)
    return lib.kda_scan_rows_columns(a["s_in"], a["s_cols"], a["q"], a["k"], a["v"], a["g"],
                                     a["beta"], a["o"], a["e"], a["L"], a["T"], a["H"], a["dt"],
                                     None)


def _replay(lib, b, **kw):
    a = dict(snap=b["snap"], s_out=b["s_out"], q=b["q"], k=b["k"], v=b["v"], g=b["g"],
             beta=b["beta"], L=2, T=8, keep=3, H=2, dt=0)
    a.update(kw)
    return lib.kda_replay(a["snap"], a["s_out"], a["q"], a["k"], a["v"], a["g"], a["beta"],
                          a["L"], a["T"], a["keep"], a["H"], a["dt"], None)


def _replay_stash(lib, b, **kw):
    a = dict(snap=b["snap"], s_out=b["s_out"], k=b["k"], g=b["g"], e=b["ptrs"], L=2, T=8,
             keep=3, H=2, dt=0)
    a.update(kw)
    return lib.kda_replay_stash(a["snap"], a["s_out"], a["k"], a["g"], a["e"], a["L"], a["T"],
                                a["keep"], a["H"], a["dt"], None)


def _round(lib, b, **kw):
    a = dict(snap_prev=b["snap"], snap_out=b["s_out"], pk=b["k"], pv=b["v"], pg=b["g"],
             pbeta=b["beta"], pe=None, T_prev=8, keep=3, q=b["q"], k=b["k"], v=b["v"],
             g=b["g"], beta=b["beta"], o=b["o"], e=None, L=2, T=8, H=2, dt=0)
    a.update(kw)
    return lib.kda_verify_round(a["snap_prev"], a["snap_out"], a["pk"], a["pv"], a["pg"],
                                a["pbeta"], a["pe"], a["T_prev"], a["keep"], a["q"], a["k"],
                                a["v"], a["g"], a["beta"], a["o"], a["e"], a["L"], a["T"],
                                a["H"], a["dt"], None)


def _batched(lib, b, **kw):
    a = dict(ptrs=b["ptrs"], q=b["q"], k=b["k"], v=b["v"], g=b["g"], beta=b["beta"], o=b["o"],
             L=2, B=4, H=2, dt=0)
    a.update(kw)
    return lib.kda_scan_batched(a["ptrs"], a["q"], a["k"], a["v"], a["g"], a["beta"], a["o"],
                                a["L"], a["B"], a["H"], a["dt"], None)


def _accept(lib, b, **kw):
    a = dict(logits=b["q"], t=4, V=1000, ld=1000, dt=0, drafts=b["k"], vam=b["o"], out2=b["v"],
             work=b["snap"])
    a.update(kw)
    return lib.kda_accept_greedy(a["logits"], a["t"], a["V"], a["ld"], a["dt"], a["drafts"],
                                 a["vam"], a["out2"], a["work"], None)


def _msg(lib):
    return lib.kda_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(T=0), ERR_RANGE, "T=0"),
    (dict(T=16), ERR_RANGE, "T=16"),
    (dict(L=0), ERR_RANGE, "L=0"),
    (dict(H=0), ERR_RANGE, "H=0"),
    (dict(H=-3), ERR_RANGE, "H=-3"),
    (dict(dt=2), ERR_ARG, "in_dtype"),
    (dict(q=None), ERR_ARG, "q is NULL"),
    (dict(beta=None), ERR_ARG, "beta is NULL"),
    (dict(s_in=None), ERR_ARG, "s_in is NULL"),
    (dict(s_out=None), ERR_ARG, "s_out is NULL"),
])
def test_scan_rows_refusals(lib, b, kw, code, needle):
    assert _scan(lib, b, **kw) == code
    assert needle in _msg(lib)


def test_scan_rows_alignment_and_alias(lib, b):
    off = lambda n, k: ctypes.c_void_p(b.addr[n] + k)
    assert _scan(lib, b, k=off("k", 4)) == ERR_ALIGN and "k is not 16-byte aligned" in _msg(lib)
    assert _scan(lib, b, o=off("o", 8)) == ERR_ALIGN
    # beta is read per element: it needs element alignment only
    assert _scan(lib, b, beta=off("beta", 2)) == ERR_ALIGN and "4-byte" in _msg(lib)
    assert _scan(lib, b, beta=off("beta", 1), dt=1) == ERR_ALIGN and "2-byte" in _msg(lib)
    assert _batched(lib, b, beta=off("beta", 2)) == ERR_ALIGN
    # s_out partially over s_in
    assert _scan(lib, b, s_out=off("s_in", 4096)) == ERR_ALIAS and "partially" in _msg(lib)
    # s_out over a row input, o over the state
    assert _scan(lib, b, s_out=b["v"]) == ERR_ALIAS and "s_out overlaps v" in _msg(lib)
    assert _scan(lib, b, o=b["s_in"]) == ERR_ALIAS and "o overlaps s_in" in _msg(lib)
    assert _scan(lib, b, o=off("q", 1024)) == ERR_ALIAS
    assert _scan_stash(lib, b, e=b["o"]) == ERR_ALIAS and "o overlaps e" in _msg(lib)
    assert _scan_stash(lib, b, e=off("ptrs", 8)) == ERR_ALIGN
    assert _scan_stash(lib, b, e=None) == ERR_ARG and "e is NULL" in _msg(lib)
    assert _scan_stash(lib, b, T=16) == ERR_RANGE and "kda_scan_rows_stash" in _msg(lib)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(keep=0), ERR_RANGE, "keep=0"),
    (dict(keep=9), ERR_RANGE, "keep=9"),
    (dict(T=0, keep=1), ERR_RANGE, "T_round=0"),
    (dict(T=16, keep=1), ERR_RANGE, "T_round=16"),
    (dict(snap=None), ERR_ARG, "snap is NULL"),
    (dict(q=None), ERR_ARG, "q is NULL"),
    (dict(v=None), ERR_ARG, "v is NULL"),
    (dict(beta=None), ERR_ARG, "beta is NULL"),
    (dict(dt=-1), ERR_ARG, "in_dtype"),
])
def test_replay_refusals(lib, b, kw, code, needle):
    assert _replay(lib, b, **kw) == code
    assert needle in _msg(lib)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(T=0), ERR_RANGE, "T=0"),
    (dict(T=16), ERR_RANGE, "T=16"),
    (dict(L=0), ERR_RANGE, "L=0"),
    (dict(dt=3), ERR_ARG, "in_dtype"),
    (dict(o=None), ERR_ARG, "o is NULL"),
    (dict(s_cols=None), ERR_ARG, "s_cols is NULL"),
    (dict(s_in=None), ERR_ARG, "s_in is NULL"),
    (dict(g=None), ERR_ARG, "g is NULL"),
])
def test_scan_rows_columns_refusals(lib, b, kw, code, needle):
    assert _columns(lib, b, **kw) == code
    assert needle in _msg(lib)


def test_scan_rows_columns_alignment_and_alias(lib, b):
    off = lambda n, k: ctypes.c_void_p(b.addr[n] + k)
    assert _columns(lib, b, s_cols=off("s_out", 4)) == ERR_ALIGN
    assert "s_cols is not 16-byte aligned" in _msg(lib)
    # no in-place form: the columns may not even be s_in itself
    assert _columns(lib, b, s_cols=b["s_in"]) == ERR_ALIAS and "s_cols overlaps s_in" in _msg(lib)
    # T columns of L*H states reach past the first state: a row input there is refused
    cols_bytes = 8 * 2 * 2 * 128 * 128 * 4
    assert _columns(lib, b, s_cols=off("q", -(cols_bytes - 16))) == ERR_ALIAS
    assert "s_cols overlaps q" in _msg(lib)
    assert _columns(lib, b, e=off("s_out", cols_bytes - 16)) == ERR_ALIAS
    assert "s_cols overlaps e" in _msg(lib)
    assert _columns(lib, b, o=b["k"]) == ERR_ALIAS and "o overlaps k" in _msg(lib)


def _round_dev(lib, b, **kw):
    a = dict(snap_prev=b["snap"], snap_out=b["s_out"], pk=b["k"], pv=b["v"], pg=b["g"],
             pbeta=b["beta"], pe=None, T_prev=8, j=b["ptrs"], q=b["q"], k=b["k"], v=b["v"],
             g=b["g"], beta=b["beta"], o=b["o"], e=None, L=2, T=8, H=2, dt=0)
    a.update(kw)
    return lib.kda_verify_round_dev(a["snap_prev"], a["snap_out"], a["pk"], a["pv"], a["pg"],
                                    a["pbeta"], a["pe"], a["T_prev"], a["j"], a["q"], a["k"],
                                    a["v"], a["g"], a["beta"], a["o"], a["e"], a["L"], a["T"],
                                    a["H"], a["dt"], None)


def _reroll_dev(lib, b, **kw):
    a = dict(ring=b["snap"], raw=b["q"], out=b["s_out"], L=2, T=8, j=b["ptrs"], C=384, dt=0)
    a.update(kw)
    return lib.kda_conv_reroll_dev(a["ring"], a["raw"], a["out"], a["L"], a["T"], a["j"], a["C"],
                                   a["dt"], None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(j=None), ERR_ARG, "j is NULL"),
    (dict(T_prev=0), ERR_RANGE, "T_prev=0"),
    (dict(T_prev=16), ERR_RANGE, "T_prev=16"),
    (dict(snap_out=None), ERR_ARG, "snap_out is NULL"),
    (dict(T=0), ERR_RANGE, "T=0"),
    (dict(pk=None), ERR_ARG, "pk is NULL"),
])
def test_verify_round_dev_refusals(lib, b, kw, code, needle):
    assert _round_dev(lib, b, **kw) == code
    assert needle in _msg(lib)


def test_verify_round_dev_alignment_and_alias(lib, b):
    off = lambda n, k: ctypes.c_void_p(b.addr[n] + k)
    assert _round_dev(lib, b, j=off("ptrs", 2)) == ERR_ALIGN and "j is not 4-byte" in _msg(lib)
    # j is read by every workgroup: no output may cover it
    assert _round_dev(lib, b, j=off("o", 64)) == ERR_ALIAS and "o overlaps j" in _msg(lib)
    assert _round_dev(lib, b, j=off("s_out", 4)) == ERR_ALIAS and "snap_out overlaps j" in _msg(lib)
    assert _round_dev(lib, b, e=b["ptrs"]) == ERR_ALIAS and "e overlaps j" in _msg(lib)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(j=None), ERR_ARG, "j is NULL"),
    (dict(T=0), ERR_RANGE, "T_round=0"),
    (dict(C=0), ERR_RANGE, "C=0"),
    (dict(out=None), ERR_ARG, "ring_out is NULL"),
])
def test_conv_reroll_dev_refusals(lib, b, kw, code, needle):
    assert _reroll_dev(lib, b, **kw) == code
    assert needle in _msg(lib)


def test_conv_reroll_dev_alignment_and_alias(lib, b):
    off = lambda n, k: ctypes.c_void_p(b.addr[n] + k)
    assert _reroll_dev(lib, b, j=off("ptrs", 1)) == ERR_ALIGN
    assert _reroll_dev(lib, b, j=off("s_out", 8)) == ERR_ALIAS and "ring_out overlaps j" in _msg(lib)


def test_replay_alias(lib, b):
    assert _replay(lib, b, s_out=b["snap"]) == ERR_ALIAS and "s_out overlaps snap" in _msg(lib)
    assert _replay(lib, b, s_out=b["g"]) == ERR_ALIAS
    assert _replay(lib, b, s_out=b["q"]) == ERR_ALIAS and "s_out overlaps q" in _msg(lib)
    off = lambda n, k: ctypes.c_void_p(b.addr[n] + k)
    assert _replay(lib, b, q=off("q", 4)) == ERR_ALIGN and "q is not 16-byte" in _msg(lib)


def test_replay_stash_refusals(lib, b):
    off = lambda n, k: ctypes.c_void_p(b.addr[n] + k)
    assert _replay_stash(lib, b, e=None) == ERR_ARG and "e is NULL" in _msg(lib)
    assert _replay_stash(lib, b, keep=0) == ERR_RANGE and "keep=0" in _msg(lib)
    assert _replay_stash(lib, b, keep=9) == ERR_RANGE and "kda_replay_stash" in _msg(lib)
    assert _replay_stash(lib, b, k=None) == ERR_ARG and "k is NULL" in _msg(lib)
    assert _replay_stash(lib, b, g=None) == ERR_ARG and "g is NULL" in _msg(lib)
    assert _replay_stash(lib, b, e=off("ptrs", 4)) == ERR_ALIGN
    assert _replay_stash(lib, b, s_out=b["ptrs"]) == ERR_ALIAS and "overlaps e" in _msg(lib)
    assert _replay_stash(lib, b, s_out=b["snap"]) == ERR_ALIAS


@pytest.mark.parametrize("kw,code,needle", [
    (dict(T=0), ERR_RANGE, "T=0"),
    (dict(T=16), ERR_RANGE, "T=16"),
    (dict(T_prev=-1), ERR_RANGE, "T_prev=-1"),
    (dict(T_prev=16), ERR_RANGE, "T_prev=16"),
    (dict(keep=-1), ERR_RANGE, "keep=-1"),
    (dict(keep=9), ERR_RANGE, "keep=9"),
    (dict(o=None), ERR_ARG, "o is NULL"),
    (dict(pk=None), ERR_ARG, "pk is NULL"),
    (dict(pv=None), ERR_ARG, "pv is NULL"),
    (dict(snap_prev=None), ERR_ARG, "snap_prev is NULL"),
    (dict(dt=3), ERR_ARG, "in_dtype"),
])
def test_verify_round_refusals(lib, b, kw, code, needle):
    assert _round(lib, b, **kw) == code
    assert needle in _msg(lib)


def test_verify_round_alias(lib, b):
    off = lambda n, k: ctypes.c_void_p(b.addr[n] + k)
    assert _round(lib, b, snap_out=off("snap", 64)) == ERR_ALIAS and "partially" in _msg(lib)
    assert _round(lib, b, o=b["k"]) == ERR_ALIAS and "o overlaps" in _msg(lib)
    assert _round(lib, b, e=b["o"]) == ERR_ALIAS and "o overlaps e" in _msg(lib)
    assert _round(lib, b, snap_out=b["g"]) == ERR_ALIAS
    # keep == 0 needs no previous rows: with those NULL the refusal is the o alias
    assert _round(lib, b, keep=0, pk=None, pv=None, pg=None, pbeta=None, o=b["q"]) == ERR_ALIAS


@pytest.mark.parametrize("kw,code,needle", [
    (dict(B=0), ERR_RANGE, "B=0"),
    (dict(B=16), ERR_RANGE, "B=16"),
    (dict(L=0), ERR_RANGE, "L=0"),
    (dict(ptrs=None), ERR_ARG, "s_ptrs is NULL"),
    (dict(dt=7), ERR_ARG, "in_dtype"),
])
def test_batched_refusals(lib, b, kw, code, needle):
    assert _batched(lib, b, **kw) == code
    assert needle in _msg(lib)


def test_batched_alias(lib, b):
    assert _batched(lib, b, o=b["q"]) == ERR_ALIAS and "o overlaps q" in _msg(lib)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(t=0), ERR_RANGE, "t=0"),
    (dict(t=16), ERR_RANGE, "t=16"),
    (dict(V=0), ERR_RANGE, "V=0"),
    (dict(V=-5), ERR_RANGE, "V=-5"),
    (dict(ld=999), ERR_RANGE, "ld=999"),
    (dict(dt=2), ERR_ARG, "in_dtype"),
    (dict(logits=None), ERR_ARG, "logits is NULL"),
    (dict(drafts=None), ERR_ARG, "drafts is NULL"),
    (dict(vam=None), ERR_ARG, "vam is NULL"),
    (dict(out2=None), ERR_ARG, "out2 is NULL"),
    (dict(work=None), ERR_ARG, "work is NULL"),
    # t == 1 needs no drafts and ignores ld: the refusal comes from the NULL vam
    (dict(t=1, drafts=None, ld=0, vam=None), ERR_ARG, "vam is NULL"),
])
def test_accept_refusals(lib, b, kw, code, needle):
    assert _accept(lib, b, **kw) == code
    assert needle in _msg(lib)


def test_accept_alignment_and_alias(lib, b):
    off = lambda n, k: ctypes.c_void_p(b.addr[n] + k)
    assert _accept(lib, b, work=off("snap", 4)) == ERR_ALIGN and "work is not 16" in _msg(lib)
    assert _accept(lib, b, vam=off("o", 2)) == ERR_ALIGN and "vam is not 4" in _msg(lib)
    assert _accept(lib, b, logits=off("q", 2)) == ERR_ALIGN and "logits is not 4" in _msg(lib)
    assert _accept(lib, b, logits=off("q", 1), dt=1) == ERR_ALIGN and "2-byte" in _msg(lib)
    assert _accept(lib, b, vam=off("q", 3996)) == ERR_ALIAS and "vam overlaps logits" in _msg(lib)
    assert _accept(lib, b, out2=b["k"]) == ERR_ALIAS and "out2 overlaps drafts" in _msg(lib)
    assert _accept(lib, b, out2=off("snap", 64)) == ERR_ALIAS and "out2 overlaps work" in _msg(lib)
    assert _accept(lib, b, vam=b["v"]) == ERR_ALIAS and "vam overlaps out2" in _msg(lib)


def _reroll(lib, b, **kw):
    a = dict(snap=b["s_in"], raw=b["q"], out=b["s_out"], L=2, T=8, keep=3, C=1000, dt=0)
    a.update(kw)
    return lib.kda_conv_reroll(a["snap"], a["raw"], a["out"], a["L"], a["T"], a["keep"], a["C"],
                               a["dt"], None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(keep=0), ERR_RANGE, "keep=0"),
    (dict(keep=9), ERR_RANGE, "keep=9"),
    (dict(T=0, keep=1), ERR_RANGE, "T_round=0"),
    (dict(T=16, keep=1), ERR_RANGE, "T_round=16"),
    (dict(L=0), ERR_RANGE, "L=0"),
    (dict(C=0), ERR_RANGE, "C=0"),
    (dict(dt=5), ERR_ARG, "in_dtype"),
    (dict(snap=None), ERR_ARG, "ring_snap is NULL"),
    (dict(raw=None), ERR_ARG, "raw is NULL"),
    (dict(out=None), ERR_ARG, "ring_out is NULL"),
])
def test_conv_reroll_refusals(lib, b, kw, code, needle):
    assert _reroll(lib, b, **kw) == code
    assert needle in _msg(lib)


def test_conv_reroll_alignment_and_alias(lib, b):
    off = lambda n, k: ctypes.c_void_p(b.addr[n] + k)
    assert _reroll(lib, b, snap=off("s_in", 2)) == ERR_ALIGN and "ring_snap is not 4" in _msg(lib)
    assert _reroll(lib, b, raw=off("q", 1), dt=1) == ERR_ALIGN and "raw is not 2" in _msg(lib)
    assert _reroll(lib, b, out=off("s_in", 4)) == ERR_ALIAS and "ring_out overlaps ring_snap" in _msg(lib)
    assert _reroll(lib, b, out=off("q", 400)) == ERR_ALIAS and "ring_out overlaps raw" in _msg(lib)


def test_copy_batch_refusals(lib, b):
    assert lib.kda_copy_batch(b["ptrs"], 0, 100, None) == ERR_RANGE and "n=0" in _msg(lib)
    assert lib.kda_copy_batch(b["ptrs"], 65536, 100, None) == ERR_RANGE
    assert lib.kda_copy_batch(b["ptrs"], 2, 0, None) == ERR_RANGE and "words=0" in _msg(lib)
    assert lib.kda_copy_batch(None, 2, 100, None) == ERR_ARG and "table is NULL" in _msg(lib)
    assert lib.kda_copy_batch(ctypes.c_void_p(b.addr["ptrs"] + 4), 2, 100, None) == ERR_ALIGN


def _ops(lib, b, **kw):
    a = dict(x=b["q"], a=b["k"], bb=b["beta"], w=b["ptrs"], ring=b["snap"], ring_out=None,
             q=b["o"], k=b["s_out"], v=b["v"], g=b["g"], beta=b["s_in"], L=2, T=8, H=2, dt=0)
    a.update(kw)
    return lib.kda_row_ops(a["x"], a["a"], a["bb"], a["w"], a["ring"], a["ring_out"], a["q"],
                           a["k"], a["v"], a["g"], a["beta"], a["L"], a["T"], a["H"], a["dt"],
                           None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(T=0), ERR_RANGE, "T=0"),
    (dict(T=16), ERR_RANGE, "T=16"),
    (dict(L=0), ERR_RANGE, "L=0"),
    (dict(H=0), ERR_RANGE, "H=0"),
    (dict(dt=4), ERR_ARG, "in_dtype"),
    (dict(x=None), ERR_ARG, "x is NULL"),
    (dict(w=None), ERR_ARG, "conv_w is NULL"),
    (dict(ring=None), ERR_ARG, "ring_in is NULL"),
    (dict(g=None), ERR_ARG, "g is NULL"),
    (dict(beta=None), ERR_ARG, "beta is NULL"),
])
def test_row_ops_refusals(lib, b, kw, code, needle):
    assert _ops(lib, b, **kw) == code
    assert needle in _msg(lib)


def test_row_ops_alignment_and_alias(lib, b):
    off = lambda n, k: ctypes.c_void_p(b.addr[n] + k)
    assert _ops(lib, b, w=off("ptrs", 4)) == ERR_ALIGN and "conv_w is not 16" in _msg(lib)
    assert _ops(lib, b, q=off("o", 4)) == ERR_ALIGN and "q is not 16" in _msg(lib)
    assert _ops(lib, b, x=off("q", 1), dt=1) == ERR_ALIGN and "x is not 2" in _msg(lib)
    assert _ops(lib, b, v=b["q"]) == ERR_ALIAS and "v overlaps x" in _msg(lib)
    assert _ops(lib, b, g=b["o"]) == ERR_ALIAS and "q overlaps g" in _msg(lib)
    # rows run in parallel and the early ones read ring_in: no in-place ring
    assert _ops(lib, b, ring_out=b["snap"]) == ERR_ALIAS and "ring_out overlaps ring_in" in _msg(lib)
    assert _ops(lib, b, ring_out=off("snap", 64)) == ERR_ALIAS


def _multi(lib, b, prevs, **kw):
    arr = (kda._PrevRound * max(1, len(prevs)))(*prevs)
    a = dict(base=b["snap"], out=b["s_out"], n=len(prevs), q=b["q"], k=b["k"], v=b["v"],
             g=b["g"], beta=b["beta"], o=b["o"], e=None, L=2, T=8, H=2, dt=0)
    a.update(kw)
    return lib.kda_verify_round_multi(a["base"], a["out"], arr, a["n"], a["q"], a["k"], a["v"],
                                      a["g"], a["beta"], a["o"], a["e"], a["L"], a["T"], a["H"],
                                      a["dt"], None)


def _pr(b, T=8, keep=3, stash=True):
    return kda._PrevRound(b.addr["k"], None if stash else b.addr["v"], b.addr["g"],
                          None if stash else b.addr["beta"], b.addr["ptrs"] if stash else None,
                          T, keep)


def test_verify_round_multi_refusals(lib, b):
    assert _multi(lib, b, [_pr(b)] * 4, n=5) == ERR_RANGE and "n_prev=5" in _msg(lib)
    assert _multi(lib, b, [], n=-1) == ERR_RANGE
    assert _multi(lib, b, [_pr(b, T=16)]) == ERR_RANGE and "prev[0].T=16" in _msg(lib)
    assert _multi(lib, b, [_pr(b), _pr(b, T=4, keep=5)]) == ERR_RANGE and "prev[1].keep=5" in _msg(lib)
    assert _multi(lib, b, [_pr(b), _pr(b, stash=False)]) == ERR_ARG and "all or none" in _msg(lib)
    # a round with nothing kept is not read: its mismatch does not matter, the alias does
    assert _multi(lib, b, [_pr(b), _pr(b, keep=0, stash=False)], o=b["k"]) == ERR_ALIAS
    assert _multi(lib, b, [_pr(b)], out=ctypes.c_void_p(b.addr["snap"] + 64)) == ERR_ALIAS
    bad = kda._PrevRound(None, None, b.addr["g"], None, b.addr["ptrs"], 8, 2)
    assert _multi(lib, b, [bad]) == ERR_ARG and "prev[0].k is NULL" in _msg(lib)
    arr_null = lib.kda_verify_round_multi(b["snap"], b["s_out"], None, 1, b["q"], b["k"], b["v"],
                                          b["g"], b["beta"], b["o"], None, 2, 8, 2, 0, None)
    assert arr_null == ERR_ARG and "prev is NULL" in _msg(lib)


def test_snapshot_refusals(lib, b):
    assert lib.kda_snapshot(b["s_in"], b["s_in"], 2, 2, None) == ERR_ALIAS
    assert lib.kda_snapshot(b["s_in"], None, 2, 2, None) == ERR_ARG
    assert lib.kda_snapshot(b["s_in"], b["snap"], 0, 2, None) == ERR_RANGE
    assert lib.kda_snapshot(ctypes.c_void_p(b.addr["s_in"] + 8), b["snap"], 1, 1, None) == ERR_ALIGN


def test_binding_rejects_bad_shapes_before_the_library():
    torch = pytest.importorskip("torch")
    # host tensors are refused by the marshalling layer (no CPU path exists)
    q = torch.zeros(1, 2, 1, 128)
    s = torch.zeros(1, 1, 128, 128)
    beta = torch.zeros(1, 2, 1)
    with pytest.raises(ValueError, match="device tensor"):
        kda.kda_scan_rows(s, s.clone(), q, q, q, q, beta)
    with pytest.raises(ValueError, match="shape"):
        kda.kda_scan_rows(s, s.clone(), q, q, q, q, torch.zeros(1, 3, 1))
    with pytest.raises(TypeError, match="dtype"):
        kda.kda_scan_rows(s, s.clone(), q, q, q, q, beta.double())
