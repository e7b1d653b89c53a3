"""kda_accept_greedy_noalloc, the greedy accept on the library's static device
scratch, gives the bits of kda_accept_greedy with a caller workspace.

Two calls in a row on one GPU, the second with a smaller round (fewer rows,
a shorter vocabulary, bf16), so a stale partial left by the first call would
show.  Both calls are compared with kda_accept_greedy on the same inputs (exact:
argmax indices and the accept count are integers) and with the planted tokens.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_rows_amd as kda
from gated_delta_rule_rows_amd import synth

pytestmark = pytest.mark.gpu


def _round(seed, t, V, j, bf16):
    lg, dr, planted = synth.accept_round(seed, 0, t, V, j)
    x = torch.from_numpy(lg).cuda()
    if bf16:
        x = x.to(torch.bfloat16)
    return x, torch.from_numpy(dr.view(np.int32)).cuda(), planted


def _both(x, dr, t):
    out = {}
    for name in ("noalloc", "work"):
        vam = torch.full((t,), -7, dtype=torch.int32, device="cuda")
        out2 = torch.full((2,), -7, dtype=torch.int32, device="cuda")
        if name == "noalloc":
            kda.kda_accept_greedy_noalloc(x, dr, vam, out2)
        else:
            kda.kda_accept_greedy(x, dr, vam, out2, kda.accept_workspace())
        torch.cuda.synchronize()
        out[name] = (vam.cpu().numpy().view(np.uint32), out2.cpu().numpy().view(np.uint32))
    return out


def test_noalloc_accept_equals_workspace_accept_twice_shrinking():
    cases = [(15, 150_000, 9, False), (4, 5_000, 2, True)]   # the second call is smaller
    for t, V, j, bf16 in cases:
        x, dr, planted = _round(31, t, V, j, bf16)
        got = _both(x, dr, t)
        np.testing.assert_array_equal(got["noalloc"][0], got["work"][0])
        np.testing.assert_array_equal(got["noalloc"][1], got["work"][1])
        assert int(got["noalloc"][1][0]) == j
        assert int(got["noalloc"][1][1]) == int(planted[j])


def test_noalloc_refuses_rows_beyond_the_static_scratch():
    x = torch.zeros(16, 64, device="cuda")
    vam = torch.empty(16, dtype=torch.int32, device="cuda")
    out2 = torch.empty(2, dtype=torch.int32, device="cuda")
    with pytest.raises(kda.KdaError, match="static scratch"):
        kda.kda_accept_greedy_noalloc(x, torch.zeros(15, dtype=torch.int32, device="cuda"),
                                      vam, out2)
