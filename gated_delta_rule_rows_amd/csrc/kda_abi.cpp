// C ABI of libkda.so: host-side argument validation, then one enqueue.
//
// Every refusal happens before anything touches the device; the message is
// kept per thread for kda_last_error().  The validation follows the source
// pages' refusals: an empty verify row set or one wider than the decode-exact
// knee of 15 rows is refused (memra-engine 0.123.0 glm_spec.rs, fn
// glm5_verify_rows), and keep outside 1..=rows is refused (fn
// glm5_verify_rollback).

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "kda.h"
#include "kda_launch.h"

namespace {

thread_local char g_err[512] = "";

int refuse(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

// A byte range [p, p + n) of device memory, with the alignment it needs.
struct Span {
    const char* name;
    const void* ptr;
    unsigned long long n;
    unsigned align;
    bool optional;   // may be NULL
};

uintptr_t addr(const Span& s) { return reinterpret_cast<uintptr_t>(s.ptr); }

bool overlap(const Span& a, const Span& b) {
    if (!a.ptr || !b.ptr || a.n == 0 || b.n == 0) return false;
    return addr(a) < addr(b) + b.n && addr(b) < addr(a) + a.n;
}

int check_spans(const char* fn, const Span* s, int n) {
    for (int i = 0; i < n; ++i) {
        if (!s[i].ptr) {
            if (s[i].optional) continue;
            return refuse(KDA_ERR_ARG, "%s: %s is NULL", fn, s[i].name);
        }
        if (addr(s[i]) % s[i].align != 0)
            return refuse(KDA_ERR_ALIGN, "%s: %s is not %u-byte aligned", fn, s[i].name, s[i].align);
    }
    return KDA_OK;
}

// No output may overlap an input or another output.  `same_out`/`same_in`
// name one (output, input) pair that may be the identical buffer (a state
// updated in place); a partial overlap of that pair is still refused.
int check_alias(const char* fn, const Span* out, int n_out, const Span* in, int n_in,
                const Span* same_out = nullptr, const Span* same_in = nullptr) {
    for (int i = 0; i < n_out; ++i) {
        for (int j = 0; j < n_in; ++j) {
            const bool pair = &out[i] == same_out && &in[j] == same_in;
            if (pair && out[i].ptr == in[j].ptr) continue;
            if (overlap(out[i], in[j])) {
                if (pair)
                    return refuse(KDA_ERR_ALIAS, "%s: %s partially overlaps %s", fn, out[i].name,
                                  in[j].name);
                return refuse(KDA_ERR_ALIAS, "%s: %s overlaps %s", fn, out[i].name, in[j].name);
            }
        }
        for (int j = i + 1; j < n_out; ++j) {
            if (overlap(out[i], out[j]))
                return refuse(KDA_ERR_ALIAS, "%s: %s overlaps %s", fn, out[i].name, out[j].name);
        }
    }
    return KDA_OK;
}

int check_counts(const char* fn, long long L, long long H) {
    if (L < 1) return refuse(KDA_ERR_RANGE, "%s: L=%lld, need L >= 1", fn, L);
    if (H < 1) return refuse(KDA_ERR_RANGE, "%s: H=%lld, need H >= 1", fn, H);
    if (L * H > INT_MAX) return refuse(KDA_ERR_RANGE, "%s: L*H=%lld too large", fn, L * H);
    return KDA_OK;
}

int check_dtype(const char* fn, int in_dtype) {
    if (in_dtype != KDA_IN_F32 && in_dtype != KDA_IN_BF16)
        return refuse(KDA_ERR_ARG, "%s: in_dtype=%d is neither KDA_IN_F32 nor KDA_IN_BF16", fn,
                      in_dtype);
    return KDA_OK;
}

int check_rows(const char* fn, const char* what, int T) {
    if (T < 1 || T > KDA_T_MAX)
        return refuse(KDA_ERR_RANGE, "%s: %s=%d outside 1..%d (K+1 verify rows, K <= 14)", fn, what,
                      T, KDA_T_MAX);
    return KDA_OK;
}

int launched(const char* fn, hipError_t e) {
    if (e != hipSuccess) return refuse(KDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    g_err[0] = '\0';
    return KDA_OK;
}

constexpr unsigned long long kStateBytes = 4ull * kda::kD * kda::kD;
constexpr unsigned long long kRowElems = kda::kD;
static_assert(sizeof(kda::AcceptScratch) <= KDA_ACCEPT_WORK_BYTES, "accept workspace too small");
static_assert(kda::kNoToken == KDA_NO_TOKEN, "one sentinel");
static_assert(kda::kRingRows == KDA_CONV_RING_ROWS, "one ring depth");

// The fused round behind kda_verify_round and kda_verify_round_multi.
// keep_j (one_round only): the kept rows of prev[0] come from device memory.
int verify_round(const char* fn, bool one_round, const float* snap_base, float* snap_out,
                 const kda_prev_round* prev, int n_prev, const void* q, const void* k,
                 const void* v, const void* g, const void* beta, float* o, float* e, int L,
                 int T, int H, int in_dtype, void* stream, const uint32_t* keep_j = nullptr) {
    int rc;
    if ((rc = check_dtype(fn, in_dtype)) || (rc = check_counts(fn, L, H)) ||
        (rc = check_rows(fn, "T", T)))
        return rc;
    if (n_prev < 0 || n_prev > KDA_MAX_PREV_ROUNDS)
        return refuse(KDA_ERR_RANGE, "%s: n_prev=%d outside 0..%d", fn, n_prev,
                      KDA_MAX_PREV_ROUNDS);
    if (n_prev > 0 && !prev) return refuse(KDA_ERR_ARG, "%s: prev is NULL", fn);
    const unsigned long long chains = static_cast<unsigned long long>(L) * H;
    const unsigned es = in_dtype == KDA_IN_BF16 ? 2 : 4;
    const unsigned long long rows = chains * T;
    // earlier rounds: validate each, keep those with rows to replay
    kda::ScanArgs a{};
    int stash = -1;   // all replayed rounds read the stash plane (1) or none does (0)
    Span in[7 + 5 * KDA_MAX_PREV_ROUNDS];
    int n_in = 0;
    in[n_in++] = {one_round ? "snap_prev" : "snap_base", snap_base, chains * kStateBytes, 16,
                  false};
    in[n_in++] = {"q", q, rows * kRowElems * es, 16, false};
    in[n_in++] = {"k", k, rows * kRowElems * es, 16, false};
    in[n_in++] = {"v", v, rows * kRowElems * es, 16, false};
    in[n_in++] = {"g", g, rows * kRowElems * es, 16, false};
    in[n_in++] = {"beta", beta, rows * es, es, false};
    static const char* const one[5] = {"pk", "pg", "pv", "pbeta", "pe"};
    static const char* const names[KDA_MAX_PREV_ROUNDS][5] = {
        {"prev[0].k", "prev[0].g", "prev[0].v", "prev[0].beta", "prev[0].e"},
        {"prev[1].k", "prev[1].g", "prev[1].v", "prev[1].beta", "prev[1].e"},
        {"prev[2].k", "prev[2].g", "prev[2].v", "prev[2].beta", "prev[2].e"},
        {"prev[3].k", "prev[3].g", "prev[3].v", "prev[3].beta", "prev[3].e"},
    };
    for (int i = 0; i < n_prev; ++i) {
        const kda_prev_round& pr = prev[i];
        if (pr.T < 1 || pr.T > KDA_T_MAX)
            return refuse(KDA_ERR_RANGE, "%s: prev[%d].T=%d outside 1..%d", fn, i, pr.T, KDA_T_MAX);
        if (pr.keep < 0 || pr.keep > pr.T)
            return refuse(KDA_ERR_RANGE, "%s: prev[%d].keep=%d outside 0..=%d", fn, i, pr.keep,
                          pr.T);
        if (pr.keep == 0) continue;   // nothing of that round is replayed
        const int st = pr.e != nullptr ? 1 : 0;
        if (stash >= 0 && st != stash)
            return refuse(KDA_ERR_ARG,
                          st ? "%s: prev[%d] brings the stash plane e and an earlier replayed "
                               "round does not (all or none)"
                             : "%s: prev[%d] has no stash plane e and an earlier replayed round "
                               "has one (all or none)",
                          fn, i);
        stash = st;
        const unsigned long long prow = chains * pr.T;
        const char* const* nm = one_round ? one : names[i];
        in[n_in++] = {nm[0], pr.k, prow * kRowElems * es, 16, false};
        in[n_in++] = {nm[1], pr.g, prow * kRowElems * es, 16, false};
        if (st) {
            in[n_in++] = {nm[4], pr.e, prow * kRowElems * 4, 16, false};
        } else {
            in[n_in++] = {nm[2], pr.v, prow * kRowElems * es, 16, false};
            in[n_in++] = {nm[3], pr.beta, prow * es, es, false};
        }
        kda::PrevRows& d = a.prev[a.n_prev++];
        d.k = pr.k; d.g = pr.g; d.T = pr.T; d.keep = pr.keep;
        if (st) d.e = pr.e; else { d.v = pr.v; d.beta = pr.beta; }
    }
    if (keep_j) in[n_in++] = {"j", keep_j, 4, 4, false};   // read by every workgroup
    const Span out[] = {
        {"snap_out", snap_out, chains * kStateBytes, 16, true},
        {"o", o, rows * kRowElems * 4, 16, false},
        {"e", e, rows * kRowElems * 4, 16, true},
    };
    if ((rc = check_spans(fn, in, n_in)) || (rc = check_spans(fn, out, 3)) ||
        (rc = check_alias(fn, out, 3, in, n_in, &out[0], &in[0])))
        return rc;
    a.s_in = snap_base; a.s_out = snap_out;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.o = o; a.e_out = e;
    a.n_chains = static_cast<long long>(chains); a.H = H; a.T = T; a.T_stride = T;
    a.keep_j = keep_j;
    const kda::Launch kind = stash == 1 ? kda::Launch::kRoundStash : kda::Launch::kRound;
    return launched(fn, kda::launch_scan(a, kind, in_dtype == KDA_IN_BF16,
                                         static_cast<hipStream_t>(stream)));
}

int conv_reroll(const char* fn, const float* ring_snap, const void* raw, float* ring_out, int L,
                int T_round, int keep, const uint32_t* keep_j, long long C, int in_dtype,
                void* stream) {
    int rc;
    if ((rc = check_dtype(fn, in_dtype)) || (rc = check_rows(fn, "T_round", T_round))) return rc;
    if (L < 1) return refuse(KDA_ERR_RANGE, "%s: L=%d, need L >= 1", fn, L);
    if (keep < 1 || keep > T_round)
        return refuse(KDA_ERR_RANGE, "%s: keep=%d outside 1..T_round=%d", fn, keep, T_round);
    if (C < 1 || C > (1ll << 40) / (static_cast<long long>(L) * T_round))
        return refuse(KDA_ERR_RANGE, "%s: C=%lld outside 1..%lld", fn, C,
                      (1ll << 40) / (static_cast<long long>(L) * T_round));
    const unsigned es = in_dtype == KDA_IN_BF16 ? 2 : 4;
    const unsigned long long ring = static_cast<unsigned long long>(L) * KDA_CONV_RING_ROWS * C;
    const Span in[] = {
        {"ring_snap", ring_snap, ring * 4, 4, false},
        {"raw", raw, static_cast<unsigned long long>(L) * T_round * C * es, es, false},
    };
    const Span out[] = {{"ring_out", ring_out, ring * 4, 4, false}};
    if ((rc = check_spans(fn, in, 2)) || (rc = check_spans(fn, out, 1)) ||
        (rc = check_alias(fn, out, 1, in, 2)))
        return rc;
    if (keep_j) {
        const Span js[] = {{"j", keep_j, 4, 4, false}};
        if ((rc = check_alias(fn, out, 1, js, 1))) return rc;
    }
    kda::RerollArgs a{};
    a.ring_snap = ring_snap; a.raw = raw; a.ring_out = ring_out;
    a.C = C; a.L = L; a.T = T_round; a.keep = keep; a.keep_j = keep_j;
    return launched(fn, kda::launch_reroll(a, in_dtype == KDA_IN_BF16,
                                           static_cast<hipStream_t>(stream)));
}

// kda_scan_rows / kda_scan_rows_stash: e (the stash plane) is written when given.
int scan_rows(const char* fn, const float* s_in, float* s_out, const void* q, const void* k,
              const void* v, const void* g, const void* beta, float* o, float* e, int L, int T,
              int H, int in_dtype, void* stream) {
    int rc;
    if ((rc = check_dtype(fn, in_dtype)) || (rc = check_counts(fn, L, H)) ||
        (rc = check_rows(fn, "T", T)))
        return rc;
    const unsigned long long chains = static_cast<unsigned long long>(L) * H;
    const unsigned es = in_dtype == KDA_IN_BF16 ? 2 : 4;
    const unsigned long long rows = chains * T;
    const Span in[] = {
        {"s_in", s_in, chains * kStateBytes, 16, false},
        {"q", q, rows * kRowElems * es, 16, false},
        {"k", k, rows * kRowElems * es, 16, false},
        {"v", v, rows * kRowElems * es, 16, false},
        {"g", g, rows * kRowElems * es, 16, false},
        {"beta", beta, rows * es, es, false},
    };
    const Span out[] = {
        {"s_out", s_out, chains * kStateBytes, 16, false},
        {"o", o, rows * kRowElems * 4, 16, true},
        {"e", e, rows * kRowElems * 4, 16, true},
    };
    if ((rc = check_spans(fn, in, 6)) || (rc = check_spans(fn, out, 3)) ||
        (rc = check_alias(fn, out, 3, in, 6, &out[0], &in[0])))
        return rc;
    kda::ScanArgs a{};
    a.s_in = s_in; a.s_out = s_out;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.o = o; a.e_out = e;
    a.n_chains = static_cast<long long>(chains); a.H = H; a.T = T; a.T_stride = T;
    const kda::Launch kind = o ? kda::Launch::kScanOut : kda::Launch::kScanState;
    return launched(fn, kda::launch_scan(a, kind, in_dtype == KDA_IN_BF16,
                                         static_cast<hipStream_t>(stream)));
}

// kda_replay (q, v, beta given, e NULL) / kda_replay_stash (e given; q, v,
// beta NULL and not read).  q is validated like the other rows although a
// replay never reads it: the caller passes the round's own buffers.
int replay(const char* fn, const float* snap, float* s_out, const void* q, const void* k,
           const void* v, const void* g, const void* beta, const float* e, int L, int T_round,
           int keep, int H, int in_dtype, void* stream) {
    int rc;
    if ((rc = check_dtype(fn, in_dtype)) || (rc = check_counts(fn, L, H)) ||
        (rc = check_rows(fn, "T_round", T_round)))
        return rc;
    if (keep < 1 || keep > T_round)
        return refuse(KDA_ERR_RANGE,
                      "%s: keep=%d outside 1..=%d (the anchor row is always committed; "
                      "keep = accepted drafts + 1)",
                      fn, keep, T_round);
    const unsigned long long chains = static_cast<unsigned long long>(L) * H;
    const unsigned es = in_dtype == KDA_IN_BF16 ? 2 : 4;
    const unsigned long long rows = chains * T_round;
    const bool stash = e != nullptr;   // with the stash plane, q, v and beta are not passed
    const Span in[] = {
        {"snap", snap, chains * kStateBytes, 16, false},
        {"q", q, rows * kRowElems * es, 16, stash},
        {"k", k, rows * kRowElems * es, 16, false},
        {"v", v, rows * kRowElems * es, 16, stash},
        {"g", g, rows * kRowElems * es, 16, false},
        {"beta", beta, rows * es, es, stash},
        {"e", e, rows * kRowElems * 4, 16, true},
    };
    const Span out[] = {{"s_out", s_out, chains * kStateBytes, 16, false}};
    if ((rc = check_spans(fn, in, 7)) || (rc = check_spans(fn, out, 1)) ||
        (rc = check_alias(fn, out, 1, in, 7)))
        return rc;
    kda::ScanArgs a{};
    a.s_in = snap; a.s_out = s_out;
    a.k = k; a.v = v; a.g = g; a.beta = beta; a.e_in = e;
    a.n_chains = static_cast<long long>(chains); a.H = H; a.T = keep; a.T_stride = T_round;
    const kda::Launch kind = stash ? kda::Launch::kReplayStash : kda::Launch::kReplay;
    return launched(fn, kda::launch_scan(a, kind, in_dtype == KDA_IN_BF16,
                                         static_cast<hipStream_t>(stream)));
}

int accept_greedy(const char* fn, const void* logits, int t, int V, long long ld, int in_dtype,
                  const uint32_t* drafts, uint32_t* vam, uint32_t* out2, void* work, void* stream,
                  bool static_work = false);

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_last_error(void) { return g_err; }

int kda_scan_rows(const float* s_in, float* s_out, const void* q, const void* k, const void* v,
                  const void* g, const void* beta, float* o, int L, int T, int H, int in_dtype,
                  void* stream) {
    return scan_rows("kda_scan_rows", s_in, s_out, q, k, v, g, beta, o, nullptr, L, T, H,
                     in_dtype, stream);
}

int kda_scan_rows_stash(const float* s_in, float* s_out, const void* q, const void* k,
                        const void* v, const void* g, const void* beta, float* o, float* e, int L,
                        int T, int H, int in_dtype, void* stream) {
    if (!e) return refuse(KDA_ERR_ARG, "kda_scan_rows_stash: e is NULL");
    return scan_rows("kda_scan_rows_stash", s_in, s_out, q, k, v, g, beta, o, e, L, T, H,
                     in_dtype, stream);
}

int kda_scan_rows_columns(const float* s_in, float* s_cols, const void* q, const void* k,
                          const void* v, const void* g, const void* beta, float* o, float* e,
                          int L, int T, int H, int in_dtype, void* stream) {
    const char* fn = "kda_scan_rows_columns";
    int rc;
    if ((rc = check_dtype(fn, in_dtype)) || (rc = check_counts(fn, L, H)) ||
        (rc = check_rows(fn, "T", T)))
        return rc;
    const unsigned long long chains = static_cast<unsigned long long>(L) * H;
    const unsigned es = in_dtype == KDA_IN_BF16 ? 2 : 4;
    const unsigned long long rows = chains * T;
    const Span in[] = {
        {"s_in", s_in, chains * kStateBytes, 16, false},
        {"q", q, rows * kRowElems * es, 16, false},
        {"k", k, rows * kRowElems * es, 16, false},
        {"v", v, rows * kRowElems * es, 16, false},
        {"g", g, rows * kRowElems * es, 16, false},
        {"beta", beta, rows * es, es, false},
    };
    const Span out[] = {
        {"s_cols", s_cols, rows * kStateBytes, 16, false},
        {"o", o, rows * kRowElems * 4, 16, false},
        {"e", e, rows * kRowElems * 4, 16, true},
    };
    if ((rc = check_spans(fn, in, 6)) || (rc = check_spans(fn, out, 3)) ||
        (rc = check_alias(fn, out, 3, in, 6)))
        return rc;
    kda::ScanArgs a{};
    a.s_in = s_in; a.s_cols = s_cols; a.col_stride = chains * kda::kD * kda::kD;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.o = o; a.e_out = e;
    a.n_chains = static_cast<long long>(chains); a.H = H; a.T = T; a.T_stride = T;
    return launched(fn, kda::launch_scan(a, kda::Launch::kScanColumns, in_dtype == KDA_IN_BF16,
                                         static_cast<hipStream_t>(stream)));
}

int kda_snapshot(const float* s, float* snap, int L, int H, void* stream) {
    const char* fn = "kda_snapshot";
    int rc;
    if ((rc = check_counts(fn, L, H))) return rc;
    const unsigned long long chains = static_cast<unsigned long long>(L) * H;
    const Span in[] = {{"s", s, chains * kStateBytes, 16, false}};
    const Span out[] = {{"snap", snap, chains * kStateBytes, 16, false}};
    if ((rc = check_spans(fn, in, 1)) || (rc = check_spans(fn, out, 1)) ||
        (rc = check_alias(fn, out, 1, in, 1)))
        return rc;
    return launched(fn, kda::launch_copy(s, snap, static_cast<size_t>(chains) * kda::kD * kda::kD,
                                         static_cast<hipStream_t>(stream)));
}

int kda_replay(const float* snap, float* s_out, const void* q, const void* k, const void* v,
               const void* g, const void* beta, int L, int T_round, int keep, int H, int in_dtype,
               void* stream) {
    return replay("kda_replay", snap, s_out, q, k, v, g, beta, nullptr, L, T_round, keep, H,
                  in_dtype, stream);
}

int kda_replay_stash(const float* snap, float* s_out, const void* k, const void* g,
                     const float* e, int L, int T_round, int keep, int H, int in_dtype,
                     void* stream) {
    if (!e) return refuse(KDA_ERR_ARG, "kda_replay_stash: e is NULL");
    return replay("kda_replay_stash", snap, s_out, nullptr, k, nullptr, g, nullptr, e, L, T_round,
                  keep, H, in_dtype, stream);
}

int kda_scan_batched(float* const* s_ptrs, const void* q, const void* k, const void* v,
                     const void* g, const void* beta, float* o, int L, int B, int H, int in_dtype,
                     void* stream) {
    const char* fn = "kda_scan_batched";
    int rc;
    if ((rc = check_dtype(fn, in_dtype)) || (rc = check_counts(fn, L, H))) return rc;
    if (B < 1 || B > KDA_B_MAX)
        return refuse(KDA_ERR_RANGE, "%s: B=%d outside 1..%d (per-row exactness knee)", fn, B,
                      KDA_B_MAX);
    const unsigned long long chains = static_cast<unsigned long long>(L) * B * H;
    if (chains > INT_MAX) return refuse(KDA_ERR_RANGE, "%s: L*B*H=%llu too large", fn, chains);
    const unsigned es = in_dtype == KDA_IN_BF16 ? 2 : 4;
    const Span in[] = {
        {"s_ptrs", s_ptrs, static_cast<unsigned long long>(L) * B * 8, 8, false},
        {"q", q, chains * kRowElems * es, 16, false},
        {"k", k, chains * kRowElems * es, 16, false},
        {"v", v, chains * kRowElems * es, 16, false},
        {"g", g, chains * kRowElems * es, 16, false},
        {"beta", beta, chains * es, es, false},
    };
    const Span out[] = {{"o", o, chains * kRowElems * 4, 16, true}};
    if ((rc = check_spans(fn, in, 6)) || (rc = check_spans(fn, out, 1)) ||
        (rc = check_alias(fn, out, 1, in, 6)))
        return rc;
    kda::ScanArgs a{};
    a.s_ptrs = s_ptrs;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.o = o;
    a.n_chains = static_cast<long long>(chains); a.H = H; a.T = 1; a.T_stride = 1;
    const kda::Launch kind = o ? kda::Launch::kBatchedOut : kda::Launch::kBatchedState;
    return launched(fn, kda::launch_scan(a, kind, in_dtype == KDA_IN_BF16,
                                         static_cast<hipStream_t>(stream)));
}

int kda_verify_round(const float* snap_prev, float* snap_out, const void* pk, const void* pv,
                     const void* pg, const void* pbeta, const float* pe, int T_prev, int keep,
                     const void* q, const void* k, const void* v, const void* g, const void* beta,
                     float* o, float* e, int L, int T, int H, int in_dtype, void* stream) {
    const char* fn = "kda_verify_round";
    if (T_prev < 0 || T_prev > KDA_T_MAX)
        return refuse(KDA_ERR_RANGE, "%s: T_prev=%d outside 0..%d", fn, T_prev, KDA_T_MAX);
    if (keep < 0 || keep > T_prev)
        return refuse(KDA_ERR_RANGE, "%s: keep=%d outside 0..=%d (previous-round rows to replay)",
                      fn, keep, T_prev);
    if (!snap_out) return refuse(KDA_ERR_ARG, "%s: snap_out is NULL", fn);
    const kda_prev_round pr = {pk, pv, pg, pbeta, pe, T_prev, keep};
    return verify_round(fn, true, snap_prev, snap_out, &pr, keep > 0 ? 1 : 0, q, k, v, g, beta,
                        o, e, L, T, H, in_dtype, stream);
}

int kda_verify_round_dev(const float* snap_prev, float* snap_out, const void* pk, const void* pv,
                         const void* pg, const void* pbeta, const float* pe, int T_prev,
                         const uint32_t* j, const void* q, const void* k, const void* v,
                         const void* g, const void* beta, float* o, float* e, int L, int T,
                         int H, int in_dtype, void* stream) {
    const char* fn = "kda_verify_round_dev";
    if (T_prev < 1 || T_prev > KDA_T_MAX)
        return refuse(KDA_ERR_RANGE, "%s: T_prev=%d outside 1..%d", fn, T_prev, KDA_T_MAX);
    if (!j) return refuse(KDA_ERR_ARG, "%s: j is NULL", fn);
    if (reinterpret_cast<uintptr_t>(j) % 4 != 0)
        return refuse(KDA_ERR_ALIGN, "%s: j is not 4-byte aligned", fn);
    if (!snap_out) return refuse(KDA_ERR_ARG, "%s: snap_out is NULL", fn);
    // validated for the most rows the device value can select
    const kda_prev_round pr = {pk, pv, pg, pbeta, pe, T_prev, T_prev};
    return verify_round(fn, true, snap_prev, snap_out, &pr, 1, q, k, v, g, beta, o, e, L, T, H,
                        in_dtype, stream, j);
}

int kda_verify_round_multi(const float* snap_base, float* snap_out, const kda_prev_round* prev,
                           int n_prev, const void* q, const void* k, const void* v,
                           const void* g, const void* beta, float* o, float* e, int L, int T,
                           int H, int in_dtype, void* stream) {
    return verify_round("kda_verify_round_multi", false, snap_base, snap_out, prev, n_prev, q, k,
                        v, g, beta, o, e, L, T, H, in_dtype, stream);
}

int kda_accept_greedy(const void* logits, int t, int V, long long ld, int in_dtype,
                      const uint32_t* drafts, uint32_t* vam, uint32_t* out2, void* work,
                      void* stream) {
    return accept_greedy("kda_accept_greedy", logits, t, V, ld, in_dtype, drafts, vam, out2, work,
                         stream);
}

int kda_accept_greedy_noalloc(const void* logits, int t, int V, long long ld, int in_dtype,
                              const uint32_t* drafts, uint32_t* vam, uint32_t* out2,
                              void* stream) {
    const char* fn = "kda_accept_greedy_noalloc";
    if (t < 1 || t > KDA_T_MAX)
        return refuse(KDA_ERR_RANGE,
                      "%s: t=%d outside 1..%d (the static scratch holds partial argmaxes for "
                      "at most %d rows)",
                      fn, t, KDA_T_MAX, KDA_T_MAX);
    kda::AcceptScratch* ws = nullptr;
    const hipError_t e = kda::accept_static_scratch(&ws);
    if (e != hipSuccess)
        return refuse(KDA_ERR_HIP, "%s: no static scratch on the current device: %s", fn,
                      hipGetErrorString(e));
    return accept_greedy(fn, logits, t, V, ld, in_dtype, drafts, vam, out2, ws, stream, true);
}

}  // extern "C"

namespace {

// kda_accept_greedy and its variant on the static scratch (static_work: the
// workspace is the library's own, so it is not checked as a caller buffer).
int accept_greedy(const char* fn, const void* logits, int t, int V, long long ld, int in_dtype,
                  const uint32_t* drafts, uint32_t* vam, uint32_t* out2, void* work, void* stream,
                  bool static_work) {
    int rc;
    if ((rc = check_dtype(fn, in_dtype)) || (rc = check_rows(fn, "t", t))) return rc;
    if (V < 1) return refuse(KDA_ERR_RANGE, "%s: V=%d, need V >= 1", fn, V);
    if (t == 1) ld = V;
    if (ld < V) return refuse(KDA_ERR_RANGE, "%s: ld=%lld < V=%d (rows would overlap)", fn, ld, V);
    if (ld > (1ll << 40)) return refuse(KDA_ERR_RANGE, "%s: ld=%lld too large", fn, ld);
    const unsigned es = in_dtype == KDA_IN_BF16 ? 2 : 4;
    const unsigned long long n_logits = static_cast<unsigned long long>(t - 1) * ld + V;
    const Span in[] = {
        {"logits", logits, n_logits * es, es, false},
        {"drafts", t > 1 ? drafts : nullptr, (t - 1) * 4ull, 4, t == 1},
    };
    const Span out[] = {
        {"vam", vam, t * 4ull, 4, false},
        {"out2", out2, 8, 4, false},
        {"work", work, KDA_ACCEPT_WORK_BYTES, 16, false},
    };
    const int n_out = static_work ? 2 : 3;
    if ((rc = check_spans(fn, in, 2)) || (rc = check_spans(fn, out, n_out)) ||
        (rc = check_alias(fn, out, n_out, in, 2)))
        return rc;
    auto* ws = static_cast<kda::AcceptScratch*>(work);
    kda::AcceptArgs a{};
    a.logits = logits; a.ld = ld; a.t = t; a.V = V;
    a.drafts = drafts; a.vam = vam; a.out2 = out2;
    a.pv = ws->pv; a.pi = ws->pi; a.pn = ws->pn;
    return launched(fn, kda::launch_accept(a, in_dtype == KDA_IN_BF16,
                                           static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int kda_row_ops(const void* x, const void* a, const void* b, const float* conv_w,
                const float* ring_in, float* ring_out, float* q, float* k, float* v, float* g,
                float* beta, int L, int T, int H, int in_dtype, void* stream) {
    const char* fn = "kda_row_ops";
    int rc;
    if ((rc = check_dtype(fn, in_dtype)) || (rc = check_counts(fn, L, H)) ||
        (rc = check_rows(fn, "T", T)))
        return rc;
    const unsigned es = in_dtype == KDA_IN_BF16 ? 2 : 4;
    const unsigned long long LH = static_cast<unsigned long long>(L) * H;
    const unsigned long long chans = LH * kda::kD;          // per row, all layers
    const unsigned long long ring = 3ull * KDA_CONV_RING_ROWS * chans * 4;
    const Span in[] = {
        {"x", x, 3 * chans * T * es, es, false},
        {"a", a, chans * T * es, es, false},
        {"b", b, LH * T * es, es, false},
        {"conv_w", conv_w, 3 * chans * 4 * 4, 16, false},
        {"ring_in", ring_in, ring, 4, false},
    };
    const Span out[] = {
        {"ring_out", ring_out, ring, 4, true},
        {"q", q, chans * T * 4, 16, false},
        {"k", k, chans * T * 4, 16, false},
        {"v", v, chans * T * 4, 16, false},
        {"g", g, chans * T * 4, 16, false},
        {"beta", beta, LH * T * 4, 4, false},
    };
    if ((rc = check_spans(fn, in, 5)) || (rc = check_spans(fn, out, 6)) ||
        (rc = check_alias(fn, out, 6, in, 5)))
        return rc;
    kda::RowOpsArgs r{};
    r.x = x; r.a = a; r.b = b; r.w = conv_w; r.ring_in = ring_in; r.ring_out = ring_out;
    r.q = q; r.k = k; r.v = v; r.g = g; r.beta = beta; r.L = L; r.T = T; r.H = H;
    return launched(fn, kda::launch_row_ops(r, in_dtype == KDA_IN_BF16,
                                            static_cast<hipStream_t>(stream)));
}

int kda_conv_reroll(const float* ring_snap, const void* raw, float* ring_out, int L,
                    int T_round, int keep, long long C, int in_dtype, void* stream) {
    return conv_reroll("kda_conv_reroll", ring_snap, raw, ring_out, L, T_round, keep, nullptr, C,
                       in_dtype, stream);
}

int kda_conv_reroll_dev(const float* ring_snap, const void* raw, float* ring_out, int L,
                        int T_round, const uint32_t* j, long long C, int in_dtype, void* stream) {
    const char* fn = "kda_conv_reroll_dev";
    if (!j) return refuse(KDA_ERR_ARG, "%s: j is NULL", fn);
    if (reinterpret_cast<uintptr_t>(j) % 4 != 0)
        return refuse(KDA_ERR_ALIGN, "%s: j is not 4-byte aligned", fn);
    // keep = T_round passes the host range check; the kernel reads the real one
    return conv_reroll(fn, ring_snap, raw, ring_out, L, T_round, T_round, j, C, in_dtype, stream);
}

int kda_copy_batch(const uint64_t* table, int n, long long words, void* stream) {
    const char* fn = "kda_copy_batch";
    int rc;
    if (n < 1 || n > 65535) return refuse(KDA_ERR_RANGE, "%s: n=%d outside 1..65535", fn, n);
    if (words < 1 || words > (1ll << 40))
        return refuse(KDA_ERR_RANGE, "%s: words=%lld outside 1..2^40", fn, words);
    const Span in[] = {{"table", table, 16ull * n, 8, false}};
    if ((rc = check_spans(fn, in, 1))) return rc;
    return launched(fn, kda::launch_copy_batch(table, n, words, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
