"""include/kda.h is a C header: a C99 program compiles against it, links
libkda.so and calls the entry points through plain C.

The program declares the four hot-path calls itself, with the argument lists
of the boundary as it is specified (scan, snapshot, replay, batched arm), and
those declarations must agree with the header's: a C compiler rejects a
redeclaration with different parameter types.

No GPU is needed: the program checks the ABI version and that validation
refuses bad arguments (null pointers, ranges) with the documented status codes
before anything reaches the device.
"""
import os
import shutil
import subprocess

import pytest

import gated_delta_rule_rows_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_SRC = r"""
#include <stdio.h>
#include <string.h>
#include "kda.h"

/* The boundary's four hot-path calls, written out from their specification.
   Redeclaring a function with an incompatible prototype is a compile error. */
int kda_scan_rows(const float* s_in, float* s_out,
                  const void* q, const void* k, const void* v, const void* g,
                  const void* beta, float* o,
                  int L, int T, int H, int in_dtype, void* stream);
int kda_snapshot(const float* s, float* snap, int L, int H, void* stream);
int kda_replay(const float* snap, float* s_out,
               const void* q, const void* k, const void* v, const void* g,
               const void* beta,
               int L, int T_round, int keep, int H, int in_dtype, void* stream);
int kda_scan_batched(float* const* s_ptrs,
                     const void* q, const void* k, const void* v, const void* g,
                     const void* beta, float* o,
                     int L, int B, int H, int in_dtype, void* stream);
const char* kda_last_error(void);
int kda_abi_version(void);

static int expect(int got, int want, const char* what) {
    if (got != want) {
        printf("FAIL %s: status %d, want %d (%s)\n", what, got, want, kda_last_error());
        return 1;
    }
    return 0;
}

int main(void) {
    int bad = 0;
    if (kda_abi_version() != KDA_ABI_VERSION) {
        printf("FAIL abi version %d != %d\n", kda_abi_version(), KDA_ABI_VERSION);
        return 1;
    }
    /* refusals happen on the host, before any device work */
    bad |= expect(kda_scan_rows(0, 0, 0, 0, 0, 0, 0, 0, 1, 16, 1, KDA_IN_F32, 0),
                  KDA_ERR_RANGE, "scan T=16");
    bad |= expect(kda_scan_rows(0, 0, 0, 0, 0, 0, 0, 0, 1, 8, 1, KDA_IN_F32, 0),
                  KDA_ERR_ARG, "scan null state");
    bad |= expect(kda_snapshot(0, 0, 0, 1, 0), KDA_ERR_RANGE, "snapshot L=0");
    bad |= expect(kda_replay(0, 0, 0, 0, 0, 0, 0, 1, 8, 0, 1, KDA_IN_F32, 0),
                  KDA_ERR_RANGE, "replay keep=0");
    bad |= expect(kda_replay(0, 0, 0, 0, 0, 0, 0, 1, 8, 9, 1, KDA_IN_F32, 0),
                  KDA_ERR_RANGE, "replay keep=9");
    bad |= expect(kda_scan_rows_stash(0, 0, 0, 0, 0, 0, 0, 0, 0, 1, 8, 1, KDA_IN_F32, 0),
                  KDA_ERR_ARG, "scan_stash null e");
    bad |= expect(kda_replay_stash(0, 0, 0, 0, 0, 1, 8, 3, 1, KDA_IN_F32, 0),
                  KDA_ERR_ARG, "replay_stash null e");
    bad |= expect(kda_scan_batched(0, 0, 0, 0, 0, 0, 0, 1, KDA_B_MAX + 1, 1, KDA_IN_BF16, 0),
                  KDA_ERR_RANGE, "batched B=16");
    bad |= expect(kda_verify_round(0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 1, 8, 1, 7, 0),
                  KDA_ERR_ARG, "round dtype");
    bad |= expect(kda_accept_greedy(0, 0, 10, 10, KDA_IN_F32, 0, 0, 0, 0, 0),
                  KDA_ERR_RANGE, "accept t=0");
    bad |= expect(kda_conv_reroll(0, 0, 0, 1, 8, 9, 100, KDA_IN_F32, 0),
                  KDA_ERR_RANGE, "reroll keep=9");
    bad |= expect(kda_copy_batch(0, 1, 10, 0), KDA_ERR_ARG, "copy null table");
    bad |= expect(kda_row_ops(0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 1, 0, 1, KDA_IN_F32, 0),
                  KDA_ERR_RANGE, "row ops T=0");
    if (strlen(kda_last_error()) == 0) {
        printf("FAIL empty message after a refusal\n");
        bad = 1;
    }
    if (!bad) printf("OK\n");
    return bad;
}
"""


def test_header_compiles_as_c99_and_links(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(kda.lib_path()):
        from gated_delta_rule_rows_amd import build
        build.build()
    src = tmp_path / "abi.c"
    src.write_text(C_SRC)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(kda.lib_path())
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                    str(kda.lib_path()), f"-Wl,-rpath,{libdir}"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.strip().endswith("OK")
