// Drives the host side of libkda (kda_abi.cpp) in a build with AddressSanitizer
// and UndefinedBehaviorSanitizer.  The kernel launchers are replaced by the
// stubs below, which record what the C ABI handed them and touch no device:
// every entry point is called with valid arguments (checking the launch it
// asks for) and with refused ones (checking the status and that nothing was
// launched), and two threads refuse at once to exercise the per-thread error
// message.  Returns 0 and prints OK when every check holds.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <thread>

#include "kda.h"
#include "kda_launch.h"

namespace {
int g_launches = 0;
kda::ScanArgs g_scan{};
kda::Launch g_kind{};
bool g_bf16 = false;
kda::AcceptArgs g_accept{};
kda::RerollArgs g_reroll{};
kda::RowOpsArgs g_ops{};
long long g_copy_words = 0;
int g_copy_n = 0;
}  // namespace

namespace kda {
hipError_t launch_scan(const ScanArgs& a, Launch kind, bool bf16, hipStream_t) {
    ++g_launches; g_scan = a; g_kind = kind; g_bf16 = bf16;
    return hipSuccess;
}
hipError_t launch_copy(const float*, float*, size_t n, hipStream_t) {
    ++g_launches; g_copy_words = static_cast<long long>(n);
    return hipSuccess;
}
hipError_t launch_reroll(const RerollArgs& a, bool, hipStream_t) {
    ++g_launches; g_reroll = a;
    return hipSuccess;
}
hipError_t launch_row_ops(const RowOpsArgs& a, bool, hipStream_t) {
    ++g_launches; g_ops = a;
    return hipSuccess;
}
hipError_t launch_copy_batch(const uint64_t*, int n, long long words, hipStream_t) {
    ++g_launches; g_copy_n = n; g_copy_words = words;
    return hipSuccess;
}
int accept_workgroups_per_row(int V) { return V < 64 ? 1 : 64; }
hipError_t launch_accept(const AcceptArgs& a, bool, hipStream_t) {
    ++g_launches; g_accept = a;
    return hipSuccess;
}
AcceptScratch g_static_scratch;   // stands in for the library's device array
float* kda_static_probe() { return g_static_scratch.pv; }
hipError_t accept_static_scratch(AcceptScratch** out) {
    *out = &g_static_scratch;
    return hipSuccess;
}
}  // namespace kda

extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }

static int bad = 0;
#define CHECK(c, what)                                                       \
    do {                                                                     \
        if (!(c)) {                                                          \
            std::printf("FAIL %s (line %d): %s\n", what, __LINE__, kda_last_error()); \
            bad = 1;                                                         \
        }                                                                    \
    } while (0)

// Host buffers stand in for device memory: validation never dereferences them.
static char* buf(size_t n) { return static_cast<char*>(std::aligned_alloc(256, (n + 255) / 256 * 256)); }

int main() {
    const int L = 2, T = 8, H = 3;
    const size_t state = 4ull * L * H * 128 * 128, rows = 4ull * L * T * H * 128,
                 betas = 4ull * L * T * H;
    char *s0 = buf(state), *s1 = buf(state), *q = buf(rows), *k = buf(rows), *v = buf(rows),
         *g = buf(rows), *be = buf(betas), *o = buf(rows), *e = buf(rows), *pe = buf(rows);

    // scan, scan with the stash plane, state only
    int before = g_launches;
    CHECK(kda_scan_rows((float*)s0, (float*)s1, q, k, v, g, be, (float*)o, L, T, H, KDA_IN_F32,
                        nullptr) == KDA_OK, "scan");
    CHECK(g_launches == before + 1 && g_kind == kda::Launch::kScanOut && g_scan.n_chains == L * H &&
          g_scan.T == T && g_scan.e_out == nullptr, "scan launch");
    CHECK(kda_scan_rows_stash((float*)s0, (float*)s0, q, k, v, g, be, nullptr, (float*)e, L, T, H,
                              KDA_IN_BF16, nullptr) == KDA_OK, "scan stash in place");
    CHECK(g_kind == kda::Launch::kScanState && g_scan.e_out == (float*)e && g_bf16, "stash launch");
    // replay and replay from the stash plane
    CHECK(kda_replay((float*)s0, (float*)s1, q, k, v, g, be, L, T, 5, H, KDA_IN_F32, nullptr) ==
          KDA_OK, "replay");
    CHECK(g_kind == kda::Launch::kReplay && g_scan.T == 5 && g_scan.T_stride == T, "replay launch");
    CHECK(kda_replay_stash((float*)s0, (float*)s1, k, g, (const float*)e, L, T, 3, H, KDA_IN_F32,
                           nullptr) == KDA_OK, "replay stash");
    CHECK(g_kind == kda::Launch::kReplayStash && g_scan.e_in == (const float*)e && g_scan.T == 3,
          "replay stash launch");
    // snapshot, columns, batched
    CHECK(kda_snapshot((float*)s0, (float*)s1, L, H, nullptr) == KDA_OK, "snapshot");
    CHECK(g_copy_words == 1ll * L * H * 128 * 128, "snapshot words");
    char* cols = buf(state * T);
    CHECK(kda_scan_rows_columns((float*)s0, (float*)cols, q, k, v, g, be, (float*)o, nullptr, L, T,
                                H, KDA_IN_F32, nullptr) == KDA_OK, "columns");
    CHECK(g_kind == kda::Launch::kScanColumns && g_scan.col_stride == 1ull * L * H * 128 * 128,
          "columns launch");
    char* table = buf(8 * 15 * L);
    CHECK(kda_scan_batched((float* const*)table, q, k, v, g, be, (float*)o, L, 4, H, KDA_IN_F32,
                           nullptr) == KDA_OK, "batched");
    CHECK(g_kind == kda::Launch::kBatchedOut && g_scan.n_chains == 4ll * L * H, "batched launch");
    // fused rounds: one earlier round, several, device keep
    CHECK(kda_verify_round((float*)s0, (float*)s1, k, nullptr, g, nullptr, (const float*)pe, T, 4, q,
                           k, v, g, be, (float*)o, (float*)e, L, T, H, KDA_IN_F32, nullptr) ==
          KDA_OK, "round");
    CHECK(g_kind == kda::Launch::kRoundStash && g_scan.n_prev == 1 && g_scan.prev[0].keep == 4,
          "round launch");
    CHECK(kda_verify_round((float*)s0, (float*)s1, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0,
                           q, k, v, g, be, (float*)o, nullptr, L, T, H, KDA_IN_F32, nullptr) ==
          KDA_OK, "round keep 0");
    CHECK(g_scan.n_prev == 0, "round keep 0 launch");
    kda_prev_round prev[4];
    for (int i = 0; i < 4; ++i) prev[i] = {k, v, g, be, nullptr, T, i == 2 ? 0 : i + 1};
    CHECK(kda_verify_round_multi((float*)s0, nullptr, prev, 4, q, k, v, g, be, (float*)o, nullptr,
                                 L, T, H, KDA_IN_F32, nullptr) == KDA_OK, "multi");
    CHECK(g_kind == kda::Launch::kRound && g_scan.n_prev == 3 && g_scan.s_out == nullptr, "multi launch");
    char* j = buf(4);
    CHECK(kda_verify_round_dev((float*)s0, (float*)s1, k, v, g, be, nullptr, T, (const uint32_t*)j, q,
                               k, v, g, be, (float*)o, nullptr, L, T, H, KDA_IN_F32, nullptr) ==
          KDA_OK, "round dev");
    CHECK(g_scan.keep_j == (const uint32_t*)j, "round dev launch");
    // beside the scan
    char *lg = buf(4ull * 3 * 1000), *work = buf(KDA_ACCEPT_WORK_BYTES), *vam = buf(16), *out2 = buf(8);
    CHECK(kda_accept_greedy(lg, 3, 1000, 1000, KDA_IN_F32, (const uint32_t*)q, (uint32_t*)vam,
                            (uint32_t*)out2, work, nullptr) == KDA_OK, "accept");
    CHECK(g_accept.t == 3 && (char*)g_accept.pv >= work &&
          (char*)(g_accept.pn + 15 * 64) <= work + KDA_ACCEPT_WORK_BYTES, "accept workspace");
    CHECK(kda_accept_greedy_noalloc(lg, 3, 1000, 1000, KDA_IN_F32, (const uint32_t*)q,
                                    (uint32_t*)vam, (uint32_t*)out2, nullptr) == KDA_OK,
          "accept noalloc");
    CHECK(g_accept.pv == kda::kda_static_probe(), "accept noalloc uses the static scratch");
    CHECK(kda_accept_greedy_noalloc(lg, 16, 1000, 1000, KDA_IN_F32, (const uint32_t*)q,
                                    (uint32_t*)vam, (uint32_t*)out2, nullptr) == KDA_ERR_RANGE &&
          std::strstr(kda_last_error(), "static scratch") != nullptr, "accept noalloc t=16");
    const long long C = 3ll * H * 128;
    char *ring = buf(4ull * L * 3 * C), *ring2 = buf(4ull * L * 3 * C), *raw = buf(4ull * L * T * C);
    CHECK(kda_conv_reroll((float*)ring, raw, (float*)ring2, L, T, 6, C, KDA_IN_F32, nullptr) == KDA_OK,
          "reroll");
    CHECK(g_reroll.keep == 6 && g_reroll.C == C, "reroll launch");
    CHECK(kda_conv_reroll_dev((float*)ring, raw, (float*)ring2, L, T, (const uint32_t*)j, C,
                              KDA_IN_BF16, nullptr) == KDA_OK, "reroll dev");
    char *a = buf(4ull * L * T * H * 128), *b = buf(4ull * L * T * H), *w = buf(16ull * L * C);
    CHECK(kda_row_ops(raw, a, b, (float*)w, (float*)ring, (float*)ring2, (float*)q, (float*)k,
                      (float*)v, (float*)g, (float*)be, L, T, H, KDA_IN_F32, nullptr) == KDA_OK,
          "row ops");
    CHECK(g_ops.T == T && g_ops.H == H, "row ops launch");
    CHECK(kda_copy_batch((const uint64_t*)table, 4, 1000, nullptr) == KDA_OK && g_copy_n == 4,
          "copy batch");

    // refusals: nothing is launched
    before = g_launches;
    CHECK(kda_scan_rows((float*)s0, (float*)s1, q, k, v, g, be, (float*)o, L, 16, H, KDA_IN_F32,
                        nullptr) == KDA_ERR_RANGE, "T=16");
    CHECK(kda_scan_rows((float*)s0, (float*)(s0 + 4096), q, k, v, g, be, nullptr, L, T, H,
                        KDA_IN_F32, nullptr) == KDA_ERR_ALIAS, "partial overlap");
    CHECK(std::strstr(kda_last_error(), "partially") != nullptr, "overlap message");
    CHECK(kda_scan_rows_stash((float*)s0, (float*)s1, q, k, v, g, be, (float*)o, (float*)o, L, T, H,
                              KDA_IN_F32, nullptr) == KDA_ERR_ALIAS, "e over o");
    CHECK(kda_replay((float*)s0, (float*)s1, nullptr, k, v, g, be, L, T, 3, H, KDA_IN_F32, nullptr) ==
          KDA_ERR_ARG, "replay q NULL");
    CHECK(kda_replay((float*)s0, (float*)s1, q, k, v, g, be, L, T, 0, H, KDA_IN_F32, nullptr) ==
          KDA_ERR_RANGE, "replay keep 0");
    CHECK(kda_replay_stash((float*)s0, (float*)s1, k, g, (const float*)(e + 4), L, T, 3, H,
                           KDA_IN_F32, nullptr) == KDA_ERR_ALIGN, "stash e misaligned");
    CHECK(kda_scan_batched((float* const*)table, q, k, v, g, be, (float*)o, L, 16, H, KDA_IN_F32,
                           nullptr) == KDA_ERR_RANGE, "B=16");
    prev[1].keep = 9;
    CHECK(kda_verify_round_multi((float*)s0, (float*)s1, prev, 4, q, k, v, g, be, (float*)o,
                                 nullptr, L, T, H, KDA_IN_F32, nullptr) == KDA_ERR_RANGE,
          "multi keep");
    prev[1].keep = 2;
    prev[0].e = (const float*)pe;
    CHECK(kda_verify_round_multi((float*)s0, (float*)s1, prev, 4, q, k, v, g, be, (float*)o,
                                 nullptr, L, T, H, KDA_IN_F32, nullptr) == KDA_ERR_ARG,
          "multi stash mix");
    CHECK(kda_accept_greedy(lg, 3, 1000, 999, KDA_IN_F32, (const uint32_t*)q, (uint32_t*)vam,
                            (uint32_t*)out2, work, nullptr) == KDA_ERR_RANGE, "accept ld");
    CHECK(kda_row_ops(raw, a, b, (float*)w, (float*)ring, (float*)ring, (float*)q, (float*)k,
                      (float*)v, (float*)g, (float*)be, L, T, H, KDA_IN_F32, nullptr) ==
          KDA_ERR_ALIAS, "row ops ring in place");
    CHECK(kda_copy_batch((const uint64_t*)(table + 4), 4, 1000, nullptr) == KDA_ERR_ALIGN,
          "copy table misaligned");
    CHECK(kda_scan_rows((float*)s0, (float*)s1, q, k, v, g, be, nullptr, 1 << 20, T, 1 << 12,
                        KDA_IN_F32, nullptr) == KDA_ERR_RANGE, "L*H overflow");
    CHECK(g_launches == before, "a refusal launched nothing");

    // the last-error message is per thread
    int ta = -1, tb = -1;
    char ma[256] = "", mb[256] = "";
    std::thread t1([&] {
        for (int i = 0; i < 200; ++i)
            ta = kda_replay((float*)s0, (float*)s1, q, k, v, g, be, L, T, 0, H, KDA_IN_F32, nullptr);
        std::snprintf(ma, sizeof ma, "%s", kda_last_error());
    });
    std::thread t2([&] {
        for (int i = 0; i < 200; ++i)
            tb = kda_scan_batched((float* const*)table, q, k, v, g, be, (float*)o, L, 0, H,
                                  KDA_IN_F32, nullptr);
        std::snprintf(mb, sizeof mb, "%s", kda_last_error());
    });
    t1.join();
    t2.join();
    CHECK(ta == KDA_ERR_RANGE && std::strstr(ma, "kda_replay") != nullptr, "thread 1 message");
    CHECK(tb == KDA_ERR_RANGE && std::strstr(mb, "kda_scan_batched") != nullptr, "thread 2 message");

    for (char* p : {s0, s1, q, k, v, g, be, o, e, pe, cols, table, j, lg, work, vam, out2, ring,
                    ring2, raw, a, b, w})
        std::free(p);
    if (!bad) std::printf("OK\n");
    return bad;
}
