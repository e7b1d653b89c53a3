/*
 * Drives the CPU oracle (oracle/kda_oracle.c) over small pin-style cases in a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer.  Every buffer is
 * malloc'd at its exact size, so a read or write past any tensor the oracle
 * indexes (rows, strides, the batched pointer table, the ring, the logits) is
 * reported; the checks below make sure each entry point really ran.
 * Returns 0 and prints OK when every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int kda_oracle_scan_rows(const float* s_in, float* s_out, const void* q, const void* k,
                         const void* v, const void* g, const void* beta, float* o, int L,
                         int T_stride, int T, int H, int d, int in_bf16, int threads);
int kda_oracle_batched(float* const* states, const void* q, const void* k, const void* v,
                       const void* g, const void* beta, float* o, int L, int B, int H, int d,
                       int in_bf16, int threads);
int kda_oracle_accept_greedy(const void* logits, int t, int V, long ld, int in_bf16,
                             const uint32_t* drafts, uint32_t* vam, uint32_t* out2);
int kda_oracle_conv_reroll(const float* ring_snap, const void* raw, float* ring_out, int L,
                           int T_round, int keep, long C, int in_bf16);
int kda_oracle_row_ops(const void* x, const void* a, const void* b, const float* w,
                       const float* ring_in, float* ring_out, float* q, float* k, float* v,
                       float* g, float* beta, int L, int T, int H, int d, int in_bf16);

static int bad = 0;
#define CHECK(c, what)                                   \
    do {                                                 \
        if (!(c)) {                                      \
            printf("FAIL %s (line %d)\n", what, __LINE__); \
            bad = 1;                                     \
        }                                                \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void) {   /* splitmix64 -> [0, 1) */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) / 9007199254740992.0;
}

static float* fbuf(long n) { return (float*)malloc(sizeof(float) * (size_t)n); }

static void fill(float* x, long n, double lo, double hi) {
    for (long i = 0; i < n; ++i) x[i] = (float)(lo + (hi - lo) * urand());
}

static uint16_t* to_bf16(const float* x, long n) {
    uint16_t* b = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)n);
    for (long i = 0; i < n; ++i) {
        uint32_t u;
        memcpy(&u, &x[i], 4);
        b[i] = (uint16_t)(u >> 16);
    }
    return b;
}

/* A round of inputs [L][T][H][d] (beta [L][T][H]). */
typedef struct {
    float *q, *k, *v, *g, *beta;
} rows_t;

static rows_t make_rows(int L, int T, int H, int d) {
    const long n = (long)L * T * H * d, nb = (long)L * T * H;
    rows_t r = {fbuf(n), fbuf(n), fbuf(n), fbuf(n), fbuf(nb)};
    fill(r.q, n, -0.2, 0.2);
    fill(r.k, n, -0.2, 0.2);
    fill(r.v, n, -1, 1);
    fill(r.g, n, -6, 0.5);   /* both clamp bounds are reached */
    fill(r.beta, nb, 0, 1);
    return r;
}

static void free_rows(rows_t* r) {
    free(r->q); free(r->k); free(r->v); free(r->g); free(r->beta);
}

static void scan_cases(int threads) {
    const int L = 2, T = 5, H = 3, d = 8;
    const long ns = (long)L * H * d * d;
    rows_t r = make_rows(L, T, H, d);
    float* s0 = fbuf(ns);
    fill(s0, ns, -1, 1);
    float* s1 = fbuf(ns);
    float* o = fbuf((long)L * T * H * d);
    CHECK(kda_oracle_scan_rows(s0, s1, r.q, r.k, r.v, r.g, r.beta, o, L, T, T, H, d, 0, threads) == 0,
          "scan status");
    /* replay of keep rows = scan of keep rows out of the same T-row layout */
    for (int keep = 1; keep <= T; ++keep) {
        float* rep = fbuf(ns);
        CHECK(kda_oracle_scan_rows(s0, rep, r.q, r.k, r.v, r.g, r.beta, NULL, L, T, keep, H, d, 0,
                                   threads) == 0,
              "replay status");
        if (keep == T) CHECK(memcmp(rep, s1, sizeof(float) * ns) == 0, "replay(T) == scan");
        free(rep);
    }
    /* chained one-row scans equal the T-row scan */
    float* c = fbuf(ns);
    memcpy(c, s0, sizeof(float) * ns);
    for (int t = 0; t < T; ++t) {
        const long rn = (long)L * H * d, bn = (long)L * H;
        float *q1 = fbuf(rn), *k1 = fbuf(rn), *v1 = fbuf(rn), *g1 = fbuf(rn), *b1 = fbuf(bn);
        for (int l = 0; l < L; ++l) {
            const long src = ((long)l * T + t) * H * d, dst = (long)l * H * d;
            memcpy(q1 + dst, r.q + src, sizeof(float) * H * d);
            memcpy(k1 + dst, r.k + src, sizeof(float) * H * d);
            memcpy(v1 + dst, r.v + src, sizeof(float) * H * d);
            memcpy(g1 + dst, r.g + src, sizeof(float) * H * d);
            memcpy(b1 + (long)l * H, r.beta + ((long)l * T + t) * H, sizeof(float) * H);
        }
        CHECK(kda_oracle_scan_rows(c, c, q1, k1, v1, g1, b1, NULL, L, 1, 1, H, d, 0, threads) == 0,
              "chained status");
        free(q1); free(k1); free(v1); free(g1); free(b1);
    }
    CHECK(memcmp(c, s1, sizeof(float) * ns) == 0, "chained one-row scans == T-row scan");
    /* bf16 inputs through the same entry point */
    const long n = (long)L * T * H * d, nb = (long)L * T * H;
    uint16_t *bq = to_bf16(r.q, n), *bk = to_bf16(r.k, n), *bv = to_bf16(r.v, n),
             *bg = to_bf16(r.g, n), *bb = to_bf16(r.beta, nb);
    CHECK(kda_oracle_scan_rows(s0, c, bq, bk, bv, bg, bb, o, L, T, T, H, d, 1, threads) == 0,
          "bf16 scan status");
    free(bq); free(bk); free(bv); free(bg); free(bb);
    /* identity: beta = 0, g = 0 leaves the state bit for bit */
    memset(r.beta, 0, sizeof(float) * nb);
    memset(r.g, 0, sizeof(float) * n);
    CHECK(kda_oracle_scan_rows(s0, c, r.q, r.k, r.v, r.g, r.beta, o, L, T, T, H, d, 0, threads) == 0,
          "identity status");
    CHECK(memcmp(c, s0, sizeof(float) * ns) == 0, "identity leaves the state");
    free(c); free(s0); free(s1); free(o);
    free_rows(&r);
}

static void batched_case(int threads) {
    const int L = 2, B = 3, H = 2, d = 8;
    rows_t r = make_rows(L, B, H, d);   /* [L][B][H][d]: the batched row layout */
    float* states[6];
    float* iso[6];
    for (int i = 0; i < L * B; ++i) {
        states[i] = fbuf((long)H * d * d);
        fill(states[i], (long)H * d * d, -1, 1);
        iso[i] = fbuf((long)H * d * d);
        memcpy(iso[i], states[i], sizeof(float) * H * d * d);
    }
    float* o = fbuf((long)L * B * H * d);
    CHECK(kda_oracle_batched(states, r.q, r.k, r.v, r.g, r.beta, o, L, B, H, d, 0, threads) == 0,
          "batched status");
    /* each session alone, as a one-layer one-row scan */
    for (int l = 0; l < L; ++l)
        for (int b = 0; b < B; ++b) {
            const long ro = ((long)l * B + b) * H * d, bo = ((long)l * B + b) * H;
            float* out = fbuf((long)H * d * d);
            CHECK(kda_oracle_scan_rows(iso[l * B + b], out, r.q + ro, r.k + ro, r.v + ro, r.g + ro,
                                       r.beta + bo, NULL, 1, 1, 1, H, d, 0, 1) == 0,
                  "isolated status");
            CHECK(memcmp(out, states[l * B + b], sizeof(float) * H * d * d) == 0,
                  "batched == isolated");
            free(out);
        }
    for (int i = 0; i < L * B; ++i) { free(states[i]); free(iso[i]); }
    free(o);
    free_rows(&r);
}

static void accept_case(void) {
    const int t = 4, V = 1000;
    const long ld = 1003;
    float* lg = fbuf((t - 1) * ld + V);
    fill(lg, (t - 1) * ld + V, -3, 3);
    uint32_t want[4] = {17, 999, 0, 512};
    for (int r = 0; r < t; ++r) lg[r * ld + want[r]] = 50.0f;
    uint32_t drafts[3] = {17, 999, 5};   /* the third draft misses: j = 2 */
    uint32_t vam[4], out2[2];
    CHECK(kda_oracle_accept_greedy(lg, t, V, ld, 0, drafts, vam, out2) == 0, "accept status");
    for (int r = 0; r < t; ++r) CHECK(vam[r] == want[r], "argmax");
    CHECK(out2[0] == 2 && out2[1] == 0, "j and bonus");
    lg[2 * ld + 7] = NAN;
    CHECK(kda_oracle_accept_greedy(lg, t, V, ld, 0, drafts, vam, out2) == 0, "accept NaN status");
    CHECK(vam[2] == 0xFFFFFFFFu, "NaN row sentinel");
    free(lg);
}

static void ring_cases(void) {
    const int L = 2, T = 4, H = 2, d = 8;
    const long C = 3L * H * d;
    float* ring = fbuf(L * 3 * C);
    fill(ring, L * 3 * C, -1, 1);
    float* raw = fbuf(L * T * C);
    fill(raw, L * T * C, -1, 1);
    float* out = fbuf(L * 3 * C);
    for (int keep = 1; keep <= T; ++keep) {
        CHECK(kda_oracle_conv_reroll(ring, raw, out, L, T, keep, C, 0) == 0, "reroll status");
        /* output row 2 is raw row keep-1 */
        for (int l = 0; l < L; ++l)
            CHECK(memcmp(out + (l * 3 + 2) * C, raw + ((long)l * T + keep - 1) * C,
                         sizeof(float) * C) == 0,
                  "reroll newest row");
    }
    const long HD = (long)H * d;
    float* a = fbuf(L * T * HD);
    fill(a, L * T * HD, -3, 3);
    float* b = fbuf((long)L * T * H);
    fill(b, (long)L * T * H, -2, 2);
    float* w = fbuf(L * C * 4);
    fill(w, L * C * 4, -0.5, 0.5);
    float *q = fbuf(L * T * HD), *k = fbuf(L * T * HD), *v = fbuf(L * T * HD),
          *g = fbuf(L * T * HD), *beta = fbuf((long)L * T * H);
    CHECK(kda_oracle_row_ops(raw, a, b, w, ring, out, q, k, v, g, beta, L, T, H, d, 0) == 0,
          "row ops status");
    for (long i = 0; i < L * T * H; ++i) {
        double nq = 0;
        for (int j = 0; j < d; ++j) nq += (double)q[i * d + j] * q[i * d + j];
        CHECK(nq <= 1.0 + 1e-5, "normalised q");
        CHECK(beta[i] > 0 && beta[i] < 1, "beta in (0, 1)");
    }
    for (long i = 0; i < L * T * HD; ++i) CHECK(g[i] >= -5.0f && g[i] <= 0.0f, "gate bound");
    uint16_t *xb = to_bf16(raw, L * T * C), *ab = to_bf16(a, L * T * HD),
             *bb = to_bf16(b, (long)L * T * H);
    CHECK(kda_oracle_row_ops(xb, ab, bb, w, ring, NULL, q, k, v, g, beta, L, T, H, d, 1) == 0,
          "bf16 row ops status");
    CHECK(kda_oracle_conv_reroll(ring, xb, out, L, T, 3, C, 1) == 0, "bf16 reroll status");
    free(xb); free(ab); free(bb);
    free(ring); free(raw); free(out); free(a); free(b); free(w);
    free(q); free(k); free(v); free(g); free(beta);
}

int main(void) {
    scan_cases(1);
    scan_cases(4);
    batched_case(1);
    batched_case(3);
    accept_case();
    ring_cases();
    if (!bad) printf("OK\n");
    return bad;
}
