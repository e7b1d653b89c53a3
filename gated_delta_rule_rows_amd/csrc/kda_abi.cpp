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

// A byte range [p, p + n) of device memory.
struct Span {
    const char* name;
    uintptr_t p;
    unsigned long long n;
};

bool overlap(const Span& a, const Span& b) {
    if (a.p == 0 || b.p == 0 || a.n == 0 || b.n == 0) return false;
    return a.p < b.p + b.n && b.p < a.p + a.n;
}

// Every pointer must be non-null and 16-byte aligned, except beta (the last
// span when `beta_elem` is nonzero), which is read one element at a time and
// only needs element alignment.
int check_ptrs(const char* fn, const Span* s, int n, unsigned beta_elem = 0) {
    for (int i = 0; i < n; ++i) {
        if (s[i].p == 0) return refuse(KDA_ERR_ARG, "%s: %s is NULL", fn, s[i].name);
        const unsigned align = (beta_elem && i == n - 1) ? beta_elem : 16;
        if (s[i].p % align != 0)
            return refuse(KDA_ERR_ALIGN, "%s: %s is not %u-byte aligned", fn, s[i].name, align);
    }
    return KDA_OK;
}

int check_counts(const char* fn, long long L, long long H) {
    if (L < 1) return refuse(KDA_ERR_RANGE, "%s: L=%lld, need L >= 1", fn, L);
    if (H < 1) return refuse(KDA_ERR_RANGE, "%s: H=%lld, need H >= 1", fn, H);
    return KDA_OK;
}

int check_dtype(const char* fn, int in_dtype) {
    if (in_dtype != KDA_IN_F32 && in_dtype != KDA_IN_BF16)
        return refuse(KDA_ERR_ARG, "%s: in_dtype=%d is neither KDA_IN_F32 nor KDA_IN_BF16", fn,
                      in_dtype);
    return KDA_OK;
}

int launched(const char* fn, hipError_t e) {
    if (e != hipSuccess) return refuse(KDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    g_err[0] = '\0';
    return KDA_OK;
}

constexpr unsigned long long kStateBytes = 4ull * kda::kD * kda::kD;

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_last_error(void) { return g_err; }

int kda_scan_rows(const float* s_in, float* s_out, const void* q, const void* k, const void* v,
                  const void* g, const void* beta, float* o, int L, int T, int H, int in_dtype,
                  void* stream) {
    const char* fn = "kda_scan_rows";
    int rc;
    if ((rc = check_dtype(fn, in_dtype))) return rc;
    if ((rc = check_counts(fn, L, H))) return rc;
    if (T < 1 || T > KDA_T_MAX)
        return refuse(KDA_ERR_RANGE, "%s: T=%d outside 1..%d (K+1 verify rows, K <= 14)", fn, T,
                      KDA_T_MAX);
    const long long chains = static_cast<long long>(L) * H;
    if (chains > INT_MAX) return refuse(KDA_ERR_RANGE, "%s: L*H=%lld too large", fn, chains);
    const unsigned long long es = in_dtype == KDA_IN_BF16 ? 2 : 4;
    const unsigned long long rows = static_cast<unsigned long long>(chains) * T;
    const Span sp[] = {
        {"s_in", reinterpret_cast<uintptr_t>(s_in), chains * kStateBytes},
        {"s_out", reinterpret_cast<uintptr_t>(s_out), chains * kStateBytes},
        {"q", reinterpret_cast<uintptr_t>(q), rows * kda::kD * es},
        {"k", reinterpret_cast<uintptr_t>(k), rows * kda::kD * es},
        {"v", reinterpret_cast<uintptr_t>(v), rows * kda::kD * es},
        {"g", reinterpret_cast<uintptr_t>(g), rows * kda::kD * es},
        {"beta", reinterpret_cast<uintptr_t>(beta), rows * es},
    };
    if ((rc = check_ptrs(fn, sp, 7, static_cast<unsigned>(es)))) return rc;
    const Span so = {"o", reinterpret_cast<uintptr_t>(o), rows * kda::kD * 4};
    if (o && so.p % 16 != 0) return refuse(KDA_ERR_ALIGN, "%s: o is not 16-byte aligned", fn);
    // s_out: identical to s_in (in place) or disjoint from it; never over a row input
    if (sp[1].p != sp[0].p && overlap(sp[0], sp[1]))
        return refuse(KDA_ERR_ALIAS, "%s: s_out partially overlaps s_in", fn);
    for (int i = 2; i < 7; ++i) {
        if (overlap(sp[1], sp[i]))
            return refuse(KDA_ERR_ALIAS, "%s: s_out overlaps %s", fn, sp[i].name);
    }
    if (o) {
        for (int i = 0; i < 7; ++i) {
            if (overlap(so, sp[i]))
                return refuse(KDA_ERR_ALIAS, "%s: o overlaps %s", fn, sp[i].name);
        }
    }
    kda::ScanArgs a{};
    a.s_in = s_in; a.s_out = s_out; a.s_ptrs = nullptr;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.o = o;
    a.n_chains = chains; a.H = H; a.T = T; a.T_stride = T;
    return launched(fn, kda::launch_scan(a, in_dtype == KDA_IN_BF16, o != nullptr, false,
                                         static_cast<hipStream_t>(stream)));
}

int kda_snapshot(const float* s, float* snap, int L, int H, void* stream) {
    const char* fn = "kda_snapshot";
    int rc;
    if ((rc = check_counts(fn, L, H))) return rc;
    const long long chains = static_cast<long long>(L) * H;
    const Span sp[] = {
        {"s", reinterpret_cast<uintptr_t>(s), chains * kStateBytes},
        {"snap", reinterpret_cast<uintptr_t>(snap), chains * kStateBytes},
    };
    if ((rc = check_ptrs(fn, sp, 2))) return rc;
    if (overlap(sp[0], sp[1])) return refuse(KDA_ERR_ALIAS, "%s: snap overlaps s", fn);
    return launched(fn, kda::launch_copy(s, snap, static_cast<size_t>(chains) * kda::kD * kda::kD,
                                         static_cast<hipStream_t>(stream)));
}

int kda_replay(const float* snap, float* s_out, const void* q, const void* k, const void* v,
               const void* g, const void* beta, int L, int T_round, int keep, int H, int in_dtype,
               void* stream) {
    const char* fn = "kda_replay";
    int rc;
    if ((rc = check_dtype(fn, in_dtype))) return rc;
    if ((rc = check_counts(fn, L, H))) return rc;
    if (T_round < 1 || T_round > KDA_T_MAX)
        return refuse(KDA_ERR_RANGE, "%s: T_round=%d outside 1..%d", fn, T_round, KDA_T_MAX);
    if (keep < 1 || keep > T_round)
        return refuse(KDA_ERR_RANGE,
                      "%s: keep=%d outside 1..=%d (the anchor row is always committed; "
                      "keep = accepted drafts + 1)",
                      fn, keep, T_round);
    const long long chains = static_cast<long long>(L) * H;
    if (chains > INT_MAX) return refuse(KDA_ERR_RANGE, "%s: L*H=%lld too large", fn, chains);
    const unsigned long long es = in_dtype == KDA_IN_BF16 ? 2 : 4;
    const unsigned long long rows = static_cast<unsigned long long>(chains) * T_round;
    const Span sp[] = {
        {"snap", reinterpret_cast<uintptr_t>(snap), chains * kStateBytes},
        {"s_out", reinterpret_cast<uintptr_t>(s_out), chains * kStateBytes},
        {"q", reinterpret_cast<uintptr_t>(q), rows * kda::kD * es},
        {"k", reinterpret_cast<uintptr_t>(k), rows * kda::kD * es},
        {"v", reinterpret_cast<uintptr_t>(v), rows * kda::kD * es},
        {"g", reinterpret_cast<uintptr_t>(g), rows * kda::kD * es},
        {"beta", reinterpret_cast<uintptr_t>(beta), rows * es},
    };
    if ((rc = check_ptrs(fn, sp, 7, static_cast<unsigned>(es)))) return rc;
    for (int i = 0; i < 7; ++i) {
        if (i != 1 && overlap(sp[1], sp[i]))
            return refuse(KDA_ERR_ALIAS, "%s: s_out overlaps %s", fn, sp[i].name);
    }
    kda::ScanArgs a{};
    a.s_in = snap; a.s_out = s_out; a.s_ptrs = nullptr;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.o = nullptr;
    a.n_chains = chains; a.H = H; a.T = keep; a.T_stride = T_round;
    return launched(fn, kda::launch_scan(a, in_dtype == KDA_IN_BF16, false, false,
                                         static_cast<hipStream_t>(stream)));
}

int kda_scan_batched(float* const* s_ptrs, const void* q, const void* k, const void* v,
                     const void* g, const void* beta, float* o, int L, int B, int H, int in_dtype,
                     void* stream) {
    const char* fn = "kda_scan_batched";
    int rc;
    if ((rc = check_dtype(fn, in_dtype))) return rc;
    if ((rc = check_counts(fn, L, H))) return rc;
    if (B < 1 || B > KDA_B_MAX)
        return refuse(KDA_ERR_RANGE, "%s: B=%d outside 1..%d (per-row exactness knee)", fn, B,
                      KDA_B_MAX);
    const long long chains = static_cast<long long>(L) * B * H;
    if (chains > INT_MAX) return refuse(KDA_ERR_RANGE, "%s: L*B*H=%lld too large", fn, chains);
    const unsigned long long es = in_dtype == KDA_IN_BF16 ? 2 : 4;
    const unsigned long long rows = static_cast<unsigned long long>(chains);
    const Span sp[] = {
        {"s_ptrs", reinterpret_cast<uintptr_t>(s_ptrs), static_cast<unsigned long long>(L) * B * 8},
        {"q", reinterpret_cast<uintptr_t>(q), rows * kda::kD * es},
        {"k", reinterpret_cast<uintptr_t>(k), rows * kda::kD * es},
        {"v", reinterpret_cast<uintptr_t>(v), rows * kda::kD * es},
        {"g", reinterpret_cast<uintptr_t>(g), rows * kda::kD * es},
        {"beta", reinterpret_cast<uintptr_t>(beta), rows * es},
    };
    if ((rc = check_ptrs(fn, sp, 6, static_cast<unsigned>(es)))) return rc;
    const Span so = {"o", reinterpret_cast<uintptr_t>(o), rows * kda::kD * 4};
    if (o) {
        if (so.p % 16 != 0) return refuse(KDA_ERR_ALIGN, "%s: o is not 16-byte aligned", fn);
        for (int i = 0; i < 6; ++i) {
            if (overlap(so, sp[i]))
                return refuse(KDA_ERR_ALIAS, "%s: o overlaps %s", fn, sp[i].name);
        }
    }
    kda::ScanArgs a{};
    a.s_in = nullptr; a.s_out = nullptr; a.s_ptrs = s_ptrs;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.o = o;
    a.n_chains = chains; a.H = H; a.T = 1; a.T_stride = 1;
    return launched(fn, kda::launch_scan(a, in_dtype == KDA_IN_BF16, o != nullptr, true,
                                         static_cast<hipStream_t>(stream)));
}

}  // extern "C"
