/*
 * kda_oracle.c -- plain sequential CPU reference for the KDA verify-row scan.
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.  Only the test suite, the
 * smoke check and the bench's CPU-baseline leg may load this library.  It
 * shares no source, header, table or helper with the HIP library: it is the
 * recurrence written out from its definition, scalar, one row after another.
 *
 * What it computes (one chain = one (session, layer, head)):
 *   The state S is a d x d f32 matrix, S[i][j], i = key channel (decayed and
 *   reduced over), j = value channel.  Each verify row t with inputs
 *   q_t, k_t, v_t, g_t (d-vectors) and beta_t (scalar) does
 *       gc_i  = min(max(g_t[i], -5), 0)            (clamp in f32)
 *       S'    = diag(exp(gc)) S                    (decay per key channel)
 *       u     = S'^T k_t                           (u_j = sum_i k_i S'_ij)
 *       S_new = S' + beta_t k_t (v_t - u)^T        (delta-rule write)
 *       o_t   = S_new^T q_t / sqrt(d)              (read from the updated S)
 *   all in f64, with S rounded to f32 at the end of every row.
 *
 *   Sources.  memra-engine 0.123.0 glm_spec.rs (docs.rs source page): the
 *   module doc's VERIFY-ROW BATCHING section says the t=K+1 recurrence runs
 *   sequentially and equals the chained t=1 program; its ROLLBACK section and
 *   the Glm5VerifyCkpt doc give the snapshot-before-row-0 plus replay of rows
 *   0..keep-1.  glm5_spec_ppn_gate.rs (same crate) fixes head_dim 128 and
 *   gate_lower_bound -5.0 in its mini fixture config.  The pages name the scan
 *   kernel but never print its recurrence; the update rule, the upper clamp
 *   bound 0 and the 1/sqrt(d) output scale are the delta-rule reading stated
 *   above (plain reading; the pages are silent).
 *
 *   bf16 inputs are widened exactly, bits << 16, as dflash.rs (memra-engine
 *   0.98.0, fn bf16_to_f32) does on the host.
 *
 * Layouts (row-major, contiguous):
 *   state           [L][H][d][d] f32
 *   q, k, v, g      [L][T_stride][H][d]   f32 or bf16 bits
 *   beta            [L][T_stride][H]      f32 or bf16 bits
 *   o               [L][T][H][d] f32 (T rows scanned; may be NULL)
 *   batched arm:    rows [L][B][H][d], beta [L][B][H], o [L][B][H][d],
 *                   states given as a host pointer table [L*B] -> [H][d][d].
 *
 * Threads: chains are independent, so the multi-chain entry points may run
 * chains on several POSIX threads; each chain's rows stay strictly
 * sequential on one thread.
 */
#define _POSIX_C_SOURCE 200809L
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <pthread.h>
#include <unistd.h>

#define ORACLE_GATE_LO (-5.0f) /* gate_lower_bound of the glm5_next fixture */
#define ORACLE_GATE_HI (0.0f)  /* a log-decay never grows the state */

/* Exact bf16 -> f32: the 16 bf16 bits become the high half of the f32. */
static float widen_bf16(uint16_t bits) {
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static float fetch(const void* base, long idx, int in_bf16) {
    if (in_bf16) return widen_bf16(((const uint16_t*)base)[idx]);
    return ((const float*)base)[idx];
}

/* Clamp in f32, as the gate bound is an f32 constant of the model config. */
static float clamp_gate(float g) {
    float x = g;
    if (x < ORACLE_GATE_LO) x = ORACLE_GATE_LO;
    if (x > ORACLE_GATE_HI) x = ORACLE_GATE_HI;
    return x;
}

/*
 * One chain: T rows, sequential.  S (d*d f32) is read and written in place.
 * Row t's vectors start at element offset t*row_stride of q/k/v/g and its
 * beta at t*beta_stride.  o (if not NULL) gets row t at o + t*o_stride.
 * work must hold d*d + 3*d doubles.
 */
static void chain(float* S, const void* q, const void* k, const void* v, const void* g,
                  const void* beta, int in_bf16, long row_stride, long beta_stride, int T,
                  int d, float* o, long o_stride, double* work) {
    double* Sp = work;            /* d*d: decayed, then updated state (f64) */
    double* u = work + (long)d * d;
    double* e = u + d;
    double* dec = e + d;
    const double inv_norm = 1.0 / sqrt((double)d);
    for (int t = 0; t < T; ++t) {
        const long rb = (long)t * row_stride;
        const double b = (double)fetch(beta, (long)t * beta_stride, in_bf16);
        /* decay per key channel */
        for (int i = 0; i < d; ++i) dec[i] = exp((double)clamp_gate(fetch(g, rb + i, in_bf16)));
        for (int i = 0; i < d; ++i)
            for (int j = 0; j < d; ++j) Sp[(long)i * d + j] = dec[i] * (double)S[(long)i * d + j];
        /* u = S'^T k, summed over ascending key index */
        for (int j = 0; j < d; ++j) u[j] = 0.0;
        for (int i = 0; i < d; ++i) {
            const double ki = (double)fetch(k, rb + i, in_bf16);
            for (int j = 0; j < d; ++j) u[j] += ki * Sp[(long)i * d + j];
        }
        /* e = beta (v - u) */
        for (int j = 0; j < d; ++j) e[j] = b * ((double)fetch(v, rb + j, in_bf16) - u[j]);
        /* S_new = S' + k e^T */
        for (int i = 0; i < d; ++i) {
            const double ki = (double)fetch(k, rb + i, in_bf16);
            for (int j = 0; j < d; ++j) Sp[(long)i * d + j] += ki * e[j];
        }
        /* o = S_new^T q / sqrt(d), from the updated state */
        if (o) {
            for (int j = 0; j < d; ++j) u[j] = 0.0;
            for (int i = 0; i < d; ++i) {
                const double qi = (double)fetch(q, rb + i, in_bf16);
                for (int j = 0; j < d; ++j) u[j] += qi * Sp[(long)i * d + j];
            }
            for (int j = 0; j < d; ++j) o[(long)t * o_stride + j] = (float)(u[j] * inv_norm);
        }
        /* the state is f32: round once per row */
        for (long x = 0; x < (long)d * d; ++x) S[x] = (float)Sp[x];
    }
}

int kda_oracle_version(void) { return 1; }

/* Element size in bytes of an input tensor. */
static long esz(int in_bf16) { return in_bf16 ? 2 : 4; }

/* Where one chain's data lives. */
typedef struct {
    float* S;
    const char *q, *k, *v, *g, *beta;
    long row_stride, beta_stride;
    int T;
    float* o;
    long o_stride;
} chain_ref;

/* A chain set: either the [L][H] scan layout or the batched [L][B][H] layout. */
typedef struct {
    int batched;
    float* s_out;
    float* const* states;
    const void *q, *k, *v, *g, *beta;
    float* o;
    int L, T_stride, T, B, H, d, in_bf16;
} chain_set;

static chain_ref locate(const chain_set* cs, long c) {
    chain_ref r;
    const long d = cs->d, dd = d * d, e = esz(cs->in_bf16);
    if (!cs->batched) {
        const long l = c / cs->H, h = c % cs->H;
        const long row0 = (l * cs->T_stride * cs->H + h) * d; /* element offset of row 0 */
        const long b0 = l * cs->T_stride * cs->H + h;
        r.S = cs->s_out + c * dd;
        r.q = (const char*)cs->q + row0 * e;
        r.k = (const char*)cs->k + row0 * e;
        r.v = (const char*)cs->v + row0 * e;
        r.g = (const char*)cs->g + row0 * e;
        r.beta = (const char*)cs->beta + b0 * e;
        r.row_stride = (long)cs->H * d;
        r.beta_stride = cs->H;
        r.T = cs->T;
        r.o = cs->o ? cs->o + (l * cs->T * cs->H + h) * d : NULL;
        r.o_stride = (long)cs->H * d;
    } else {
        const long lb = c / cs->H, h = c % cs->H;
        const long row0 = c * d;
        r.S = cs->states[lb] + h * dd;
        r.q = (const char*)cs->q + row0 * e;
        r.k = (const char*)cs->k + row0 * e;
        r.v = (const char*)cs->v + row0 * e;
        r.g = (const char*)cs->g + row0 * e;
        r.beta = (const char*)cs->beta + c * e;
        r.row_stride = d;
        r.beta_stride = 1;
        r.T = 1;
        r.o = cs->o ? cs->o + row0 : NULL;
        r.o_stride = d;
    }
    return r;
}

typedef struct {
    const chain_set* cs;
    long nchain;
    int tid, nthreads;
    int fail;
} worker_arg;

/* Thread `tid` runs chains tid, tid + n, tid + 2n, ...; each chain on one thread. */
static void* worker(void* p) {
    worker_arg* a = (worker_arg*)p;
    const long d = a->cs->d;
    double* work = (double*)malloc(sizeof(double) * (d * d + 3 * d));
    if (!work) {
        a->fail = 1;
        return NULL;
    }
    for (long c = a->tid; c < a->nchain; c += a->nthreads) {
        chain_ref r = locate(a->cs, c);
        chain(r.S, r.q, r.k, r.v, r.g, r.beta, a->cs->in_bf16, r.row_stride, r.beta_stride, r.T,
              (int)d, r.o, r.o_stride, work);
    }
    free(work);
    return NULL;
}

static int run_chains(const chain_set* cs, long nchain, int threads) {
    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    if ((long)threads > nchain) threads = nchain > 0 ? (int)nchain : 1;
    worker_arg args[256];
    pthread_t tids[256];
    int started[256];
    int fail = 0;
    for (int t = 0; t < threads; ++t) {
        args[t].cs = cs;
        args[t].nchain = nchain;
        args[t].tid = t;
        args[t].nthreads = threads;
        args[t].fail = 0;
        started[t] = 0;
    }
    for (int t = 1; t < threads; ++t)
        started[t] = pthread_create(&tids[t], NULL, worker, &args[t]) == 0;
    /* chains of a thread that failed to start run here, after thread 0's own */
    worker(&args[0]);
    for (int t = 1; t < threads; ++t) {
        if (started[t])
            pthread_join(tids[t], NULL);
        else
            worker(&args[t]);
        fail |= args[t].fail;
    }
    fail |= args[0].fail;
    return fail ? -1 : 0;
}

/*
 * Scan T rows (T <= T_stride) of L x H independent chains.
 * s_out receives the state after the T rows (s_in is left untouched unless
 * s_out == s_in).  o may be NULL.  Returns 0, or -1 if a work buffer could
 * not be allocated.
 */
int kda_oracle_scan_rows(const float* s_in, float* s_out, const void* q, const void* k,
                         const void* v, const void* g, const void* beta, float* o, int L,
                         int T_stride, int T, int H, int d, int in_bf16, int threads) {
    const long nchain = (long)L * H;
    if (s_out != s_in) memcpy(s_out, s_in, sizeof(float) * (long)d * d * nchain);
    chain_set cs = {0, s_out, NULL, q, k, v, g, beta, o, L, T_stride, T, 0, H, d, in_bf16};
    return run_chains(&cs, nchain, threads);
}

/*
 * Batched arm: B sessions, one row each, per layer.  states[l*B + b] points at
 * session b's layer-l state [H][d][d], updated in place.
 */
int kda_oracle_batched(float* const* states, const void* q, const void* k, const void* v,
                       const void* g, const void* beta, float* o, int L, int B, int H, int d,
                       int in_bf16, int threads) {
    chain_set cs = {1, NULL, states, q, k, v, g, beta, o, L, 1, 1, B, H, d, in_bf16};
    return run_chains(&cs, (long)L * B * H, threads);
}

/* Host threads available to the multi-chain entry points. */
int kda_oracle_max_threads(void) {
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

/*
 * Greedy accept over t verify rows (glm_spec.rs, 0.123.0, the greedy branch
 * of glm5_spec_round: per-row device argmax with the host argmax's tie-break,
 * lowest index wins, then the longest matching prefix; a device argmax emits
 * a sentinel on a NaN row).
 *   logits : t rows of V values (f32, or bf16 bits when in_bf16), row r at
 *            element offset r * ld.
 *   drafts : the t - 1 drafted tokens (draft r is compared with row r's argmax).
 *   vam    : out, t entries: argmax of row r, lowest index among equal maxima,
 *            or 0xFFFFFFFF if the row holds a NaN.
 *   out2   : out, {j, bonus}: j = leading drafts equal to vam[0..], bonus = vam[j].
 */
int kda_oracle_accept_greedy(const void* logits, int t, int V, long ld, int in_bf16,
                             const uint32_t* drafts, uint32_t* vam, uint32_t* out2) {
    if (t < 1 || V < 1) return -1;
    for (int r = 0; r < t; ++r) {
        uint32_t best = 0;
        float bv = fetch(logits, (long)r * ld, in_bf16);
        int nan = bv != bv;
        for (int i = 1; i < V; ++i) {
            const float x = fetch(logits, (long)r * ld + i, in_bf16);
            if (x != x) nan = 1;
            if (x > bv) {
                bv = x;
                best = (uint32_t)i;
            }
        }
        vam[r] = nan ? 0xFFFFFFFFu : best;
    }
    int j = 0;
    while (j < t - 1 && drafts[j] == vam[j]) ++j;
    out2[0] = (uint32_t)j;
    out2[1] = vam[j];
    return 0;
}

/*
 * Conv-ring rollback (glm_spec.rs, 0.123.0, module doc VERIFY-ROW BATCHING and
 * the Glm5VerifyCkpt doc): the short-conv ring of a KDA layer holds the last
 * W-1 = 3 raw conv inputs (kernel size 4, glm5_spec_ppn_gate.rs fixture
 * short_conv_kernel_size); after accepting keep rows it is rebuilt from the
 * pre-round ring snapshot by rolling it forward once per kept row over the
 * round's raw input rows.
 *   ring_snap, ring_out : [L][3][C] f32, row 0 the oldest
 *   raw                 : [L][T_round][C] f32 or bf16 bits
 * Each roll drops the oldest ring row and appends the next raw row.
 */
#define ORACLE_RING_ROWS 3

int kda_oracle_conv_reroll(const float* ring_snap, const void* raw, float* ring_out, int L,
                           int T_round, int keep, long C, int in_bf16) {
    if (L < 1 || T_round < 1 || keep < 1 || keep > T_round || C < 1) return -1;
    for (long l = 0; l < L; ++l) {
        float* ring = ring_out + l * ORACLE_RING_ROWS * C;
        memcpy(ring, ring_snap + l * ORACLE_RING_ROWS * C, sizeof(float) * ORACLE_RING_ROWS * C);
        for (int r = 0; r < keep; ++r) {
            for (int m = 0; m + 1 < ORACLE_RING_ROWS; ++m)
                memcpy(ring + m * C, ring + (m + 1) * C, sizeof(float) * C);
            for (long c = 0; c < C; ++c)
                ring[(ORACLE_RING_ROWS - 1) * C + c] =
                    fetch(raw, (l * T_round + r) * C + c, in_bf16);
        }
    }
    return 0;
}

/*
 * Pre-scan row ops of one verify round (glm_spec.rs, 0.123.0, module doc
 * VERIFY-ROW BATCHING: projections, gates and the short conv of one KDA layer
 * run batched over the t = K+1 rows; glm5_spec_ppn_gate.rs fixture:
 * short_conv_kernel_size 4, gate_lower_bound -5.0).  The pages fix those two
 * numbers and the order; the rest is the plain reading:
 *   conv  : per channel c of the 3*H*d raw q/k/v channels, causal over the
 *           sequence (3 ring rows, then the round's rows):
 *           y_t[c] = sum_{m=0..3} w[c][m] x_{t-3+m}[c], no bias, then SiLU
 *           y * sigmoid(y);
 *   q, k  : per (row, head) L2-normalised over d: x / sqrt(sum x^2 + 1e-6);
 *   v     : the conv output;
 *   g     : max(-softplus(a), -5), the log-decay with the fixture's bound;
 *   beta  : sigmoid(b).
 * Layouts: x [L][T][3*H*d] (q, k, v channel blocks of H*d), a [L][T][H*d],
 * b [L][T][H], w [L][3*H*d][4] f32, ring_in/ring_out [L][3][3*H*d] f32 (row 0
 * the oldest; ring_out = the ring after all T rows, may be NULL); outputs
 * q, k, v, g [L][T][H][d] and beta [L][T][H], f32.  f64 inside, f32 out.
 */
#define ORACLE_NORM_EPS 1e-6
#define ORACLE_CONV_TAPS 4

static double silu(double y) { return y / (1.0 + exp(-y)); }

static double softplus(double a) { return a > 0 ? a + log1p(exp(-a)) : log1p(exp(a)); }

int kda_oracle_row_ops(const void* x, const void* a, const void* b, const float* w,
                       const float* ring_in, float* ring_out, float* q, float* k, float* v,
                       float* g, float* beta, int L, int T, int H, int d, int in_bf16) {
    if (L < 1 || T < 1 || H < 1 || d < 1) return -1;
    const long HD = (long)H * d, C = 3 * HD;
    double* ring = malloc(sizeof(double) * ORACLE_RING_ROWS * C);
    double* y = malloc(sizeof(double) * C);
    if (!ring || !y) { free(ring); free(y); return -2; }
    for (long l = 0; l < L; ++l) {
        for (long i = 0; i < ORACLE_RING_ROWS * C; ++i) ring[i] = ring_in[l * ORACLE_RING_ROWS * C + i];
        const float* wl = w + l * C * ORACLE_CONV_TAPS;
        for (long t = 0; t < T; ++t) {
            const long xr = (l * T + t) * C;
            /* causal conv over (ring rows 0..2, this row), then SiLU */
            for (long c = 0; c < C; ++c) {
                const double xt = fetch(x, xr + c, in_bf16);
                double acc = 0.0;
                for (int m = 0; m < ORACLE_RING_ROWS; ++m)
                    acc += (double)wl[c * ORACLE_CONV_TAPS + m] * ring[m * C + c];
                acc += (double)wl[c * ORACLE_CONV_TAPS + ORACLE_RING_ROWS] * xt;
                y[c] = silu(acc);
            }
            /* the ring rolls by this row's raw input */
            for (int m = 0; m + 1 < ORACLE_RING_ROWS; ++m)
                for (long c = 0; c < C; ++c) ring[m * C + c] = ring[(m + 1) * C + c];
            for (long c = 0; c < C; ++c) ring[(ORACLE_RING_ROWS - 1) * C + c] = fetch(x, xr + c, in_bf16);
            for (long h = 0; h < H; ++h) {
                const long o = ((l * T + t) * H + h) * d;
                double sq = 0.0, sk = 0.0;
                for (long j = 0; j < d; ++j) {
                    sq += y[h * d + j] * y[h * d + j];
                    sk += y[HD + h * d + j] * y[HD + h * d + j];
                }
                const double nq = 1.0 / sqrt(sq + ORACLE_NORM_EPS);
                const double nk = 1.0 / sqrt(sk + ORACLE_NORM_EPS);
                for (long j = 0; j < d; ++j) {
                    q[o + j] = (float)(y[h * d + j] * nq);
                    k[o + j] = (float)(y[HD + h * d + j] * nk);
                    v[o + j] = (float)y[2 * HD + h * d + j];
                    double gg = -softplus(fetch(a, (l * T + t) * HD + h * d + j, in_bf16));
                    if (gg < ORACLE_GATE_LO) gg = ORACLE_GATE_LO;
                    g[o + j] = (float)gg;
                }
                beta[(l * T + t) * H + h] =
                    (float)(1.0 / (1.0 + exp(-(double)fetch(b, (l * T + t) * H + h, in_bf16))));
            }
        }
        if (ring_out)
            for (long i = 0; i < ORACLE_RING_ROWS * C; ++i)
                ring_out[l * ORACLE_RING_ROWS * C + i] = (float)ring[i];
    }
    free(ring);
    free(y);
    return 0;
}
