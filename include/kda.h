/*
 * kda.h -- C ABI of libkda.so, the MI355X (gfx950) KDA verify-row scan.
 *
 * The library runs the hot path of speculative verification on the KDA
 * (Kimi delta attention) layers of a hybrid model: per head a 128 x 128 f32
 * recurrent state S[i][j] (i = key channel, j = value channel) advanced by
 * verify rows, plus the rollback seam (snapshot before row 0, retained row
 * inputs, accept-j replay) and the batched-decode arm.
 *
 * One row t of one head, inputs q_t, k_t, v_t, g_t (128-vectors), beta_t:
 *     gc   = min(max(g_t, -5), 0)            per key channel, in f32
 *     S'   = diag(exp(gc)) S
 *     u    = S'^T k_t
 *     S    = S' + beta_t k_t (v_t - u)^T
 *     o_t  = S^T q_t / sqrt(128)             (from the updated state)
 * memra-engine 0.123.0 glm_spec.rs, module doc VERIFY-ROW BATCHING: the
 * t = K+1 recurrence is sequential inside one scan launch and equals the
 * chained t = 1 program; glm5_spec_ppn_gate.rs mini fixture: head_dim 128,
 * gate_lower_bound -5.0.  The update rule itself is the delta-rule reading
 * (the pages name the scan but do not print it).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers, row-major and contiguous, 16-byte
 *     aligned -- except beta, which needs only its element alignment (4 bytes
 *     for f32, 2 for bf16).  The caller owns every buffer; the library never allocates,
 *     frees or synchronizes.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL means
 *     the null stream).
 *   - Arguments are validated on the host before anything is enqueued.  On a
 *     refusal nothing is enqueued, a nonzero KDA_ERR_* status is returned and
 *     kda_last_error() describes it.  A failed launch returns KDA_ERR_HIP.
 *     Faults inside a kernel surface at the caller's next synchronization.
 *   - Row inputs (q, k, v, g, beta) are all f32 (KDA_IN_F32) or all bf16
 *     (KDA_IN_BF16, widened exactly by bits << 16 as dflash.rs, memra-engine
 *     0.98.0, fn bf16_to_f32, does).  State and outputs are always f32.
 *   - Inputs must be finite; NaN/Inf are not checked on the hot path.
 *   - Results are deterministic: for a given input every entry point gives
 *     the same bits on every call, and a T-row scan gives the same bits as T
 *     chained one-row scans, a replay of keep rows the same bits as a
 *     keep-row scan, and the batched arm the same bits per row as isolated
 *     one-row scans.
 */
#ifndef KDA_H
#define KDA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_HEAD_DIM 128   /* d_k = d_v; glm5_spec_ppn_gate.rs fixture head_dim */
#define KDA_T_MAX 15       /* verify rows per round: K + 1 <= 15 (glm_spec.rs, WALK-REUSE) */
#define KDA_B_MAX 15       /* batched-decode sessions per step (same knee) */
#define KDA_ABI_VERSION 10
#define KDA_ACCEPT_WORK_BYTES 12288   /* workspace of kda_accept_greedy */
#define KDA_NO_TOKEN 0xFFFFFFFFu      /* argmax slot of a logits row holding a NaN */
#define KDA_CONV_RING_ROWS 3          /* short-conv history: kernel size 4 keeps 3 raw rows */
#define KDA_MAX_PREV_ROUNDS 4         /* earlier rounds one kda_verify_round_multi can replay */

enum { KDA_IN_F32 = 0, KDA_IN_BF16 = 1 };

enum {
    KDA_OK = 0,
    KDA_ERR_ARG = 1,   /* null pointer or unknown dtype */
    KDA_ERR_RANGE = 2, /* a count outside its range (T, keep, B, L, H, C, n, words) */
    KDA_ERR_ALIGN = 3, /* a pointer not 16-byte aligned */
    KDA_ERR_ALIAS = 4, /* an output overlaps an input (or another output) */
    KDA_ERR_HIP = 5    /* the HIP runtime refused a launch */
};

/*
 * Scan T verify rows of L independent layer-states x H heads.
 *   glm_spec.rs (0.123.0), VERIFY-ROW BATCHING: one t = K+1 scan per layer,
 *   rows chained sequentially; ROLLBACK: the state before row 0 is the
 *   snapshot.
 *   s_in, s_out : [L][H][128][128] f32.  s_out == s_in scans in place;
 *                 disjoint buffers leave s_in untouched, so s_in then IS the
 *                 pre-round snapshot at no cost.  Partial overlap is refused.
 *   q, k, v, g  : [L][T][H][128] in in_dtype.
 *   beta        : [L][T][H] in in_dtype.
 *   o           : [L][T][H][128] f32, or NULL to skip the outputs.
 *   L, H >= 1;  1 <= T <= KDA_T_MAX.
 * The caller keeps q, k, v, g, beta alive until it has either replayed or
 * accepted every row: they are the round's stash (glm_spec.rs, ROLLBACK: the
 * row inputs are retained with zero copies), and kda_replay takes the same
 * pointers.
 */
int kda_scan_rows(const float* s_in, float* s_out, const void* q, const void* k,
                  const void* v, const void* g, const void* beta, float* o, int L, int T, int H,
                  int in_dtype, void* stream);

/*
 * kda_scan_rows that also writes the round's stash plane e.
 *   e           : [L][T][H][128] f32, required: row t's delta vector
 *                 e_t = beta_t (v_t - S'^T k_t), the exact value the scan
 *                 added (S = S' + k_t e_t^T).  kda_replay_stash and the fused
 *                 round rebuild the state from k, g and e without the two
 *                 reductions, bit for bit.  The pages size their stash at
 *                 about 160 KB per row per layer (glm_spec.rs, ROLLBACK):
 *                 one such f32 plane (32 KiB at 64 heads) above the five row
 *                 inputs.
 *   The rest as kda_scan_rows.  e must not overlap any other argument.
 */
int kda_scan_rows_stash(const float* s_in, float* s_out, const void* q, const void* k,
                        const void* v, const void* g, const void* beta, float* o, float* e,
                        int L, int T, int H, int in_dtype, void* stream);

/*
 * The per-row state-column variant of a verify scan: T rows as kda_scan_rows,
 * keeping the state after every row, so that accepting keep rows commits
 * column keep-1 by pointer, with no replay.
 *   glm_spec.rs (0.123.0), module doc ROLLBACK and the Glm5VerifyCkpt doc:
 *   the column clones per row (restore column keep-1) that the pages later
 *   retired for snapshot plus replay.  It serves as the comparison arm of
 *   kda_replay / kda_verify_round: it writes T states per round instead of
 *   one.
 *   s_in        : [L][H][128][128] f32, left untouched.
 *   s_cols      : [T][L][H][128][128] f32.  Column t, the L x H states at
 *                 s_cols + t*L*H*128*128, is the state after rows 0..t: the
 *                 bits of kda_scan_rows over rows 0..t and of kda_replay with
 *                 keep = t + 1.  Column T-1 is the state after the round.
 *   q..beta     : as kda_scan_rows.
 *   e           : as kda_scan_rows_stash, or NULL.
 *   o           : [L][T][H][128] f32, required.
 *   No output may overlap an input.  L, H >= 1;  1 <= T <= KDA_T_MAX.
 */
int kda_scan_rows_columns(const float* s_in, float* s_cols, const void* q, const void* k,
                          const void* v, const void* g, const void* beta, float* o, float* e,
                          int L, int T, int H, int in_dtype, void* stream);

/*
 * snap = s, a device copy of L x H states [L][H][128][128] f32.
 *   glm_spec.rs (0.123.0), walk per KDA layer: the state is cloned once per
 *   layer per round before row 0.  Only callers that scan in place need it.
 *   s and snap must not overlap.  L, H >= 1.
 */
int kda_snapshot(const float* s, float* snap, int L, int H, void* stream);

/*
 * Accept-j rollback: s_out = the state after rows 0..keep-1 of the round,
 * rebuilt from the pre-round snapshot `snap` by re-running those rows on the
 * round's retained inputs.  keep = j + 1 (the anchor row plus j accepted
 * drafts), 1 <= keep <= T_round <= KDA_T_MAX.
 *   glm_spec.rs (0.123.0), fn glm5_verify_rollback / glm5_rollback_layer and
 *   the Glm5VerifyCkpt doc: keep outside 1..=rows is an error; the replay is
 *   the same row program over the same inputs, so the rebuilt state is
 *   identical to the one the scan held after row keep-1.  In serving keep ==
 *   T_round needs no replay (the resident state already is it); the call stays
 *   legal and then returns the scan's final state bits.
 *   snap, s_out : [L][H][128][128] f32; they must not overlap.
 *   q, k, v, g  : the round's row buffers [L][T_round][H][128] (in_dtype),
 *   beta        : [L][T_round][H] -- the very pointers passed to the round's
 *                 kda_scan_rows.  q is not read (a replay writes no outputs)
 *                 but must be a valid non-NULL aligned pointer, like the
 *                 others; rows keep..T_round-1 are not read.
 *   No outputs are written.
 */
int kda_replay(const float* snap, float* s_out, const void* q, const void* k, const void* v,
               const void* g, const void* beta, int L, int T_round, int keep, int H,
               int in_dtype, void* stream);

/*
 * kda_replay from the stash plane: the same rollback, reading each kept row's
 * delta vector e from the plane kda_scan_rows_stash wrote instead of
 * recomputing it from v, beta and S'^T k.  Each row is then only the decay
 * and the rank-1 update, and s_out carries the same bits as kda_replay.
 *   glm_spec.rs (0.123.0), ROLLBACK: accept-j replays the stolen scan inputs
 *   from the snapshot.
 *   k, g : [L][T_round][H][128] in in_dtype;  e : [L][T_round][H][128] f32.
 *   The rest as kda_replay.
 */
int kda_replay_stash(const float* snap, float* s_out, const void* k, const void* g,
                     const float* e, int L, int T_round, int keep, int H, int in_dtype,
                     void* stream);

/*
 * Batched-decode arm: B independent sessions, one row each (t = 1), each
 * against its own state, updated in place.
 *   glm_spec.rs (0.123.0), WALK-REUSE: B sessions, each row to its own cache
 *   at its own position, each row bit-identical to the isolated t = 1 step,
 *   for B <= 15.
 *   s_ptrs      : DEVICE array of L*B pointers; s_ptrs[l*B + b] points at
 *                 session b's layer-l state [H][128][128] f32 (16-byte
 *                 aligned).  Entries must be distinct and must not overlap
 *                 each other or any input/output; the library cannot check
 *                 them (they live on the device).
 *   q, k, v, g  : [L][B][H][128] in in_dtype.    beta: [L][B][H].
 *   o           : [L][B][H][128] f32, or NULL.
 *   L, H >= 1;  1 <= B <= KDA_B_MAX.
 */
int kda_scan_batched(float* const* s_ptrs, const void* q, const void* k, const void* v,
                     const void* g, const void* beta, float* o, int L, int B, int H,
                     int in_dtype, void* stream);

/*
 * One fused verify round: roll the previous round back to its kept rows, store
 * that committed state (this round's snapshot), then scan this round's rows
 * for their outputs.  The state crosses HBM once per round.
 *   glm_spec.rs (0.123.0), ROLLBACK: accept-j replays rows 0..j of the
 *   previous round from its snapshot; VERIFY-ROW BATCHING: this round's rows
 *   are scanned sequentially.  Here the replay of round r-1 and the scan of
 *   round r share one launch and one pass over the state.
 *   snap_prev   : [L][H][128][128] f32, the previous round's snapshot (its
 *                 committed state before its rows).
 *   snap_out    : [L][H][128][128] f32, receives snap_prev advanced by rows
 *                 0..keep-1 of the previous round -- the committed state and
 *                 this round's snapshot.  == snap_prev updates in place.
 *                 The state after this round's rows is NOT stored: the next
 *                 round (or kda_replay) rebuilds what the accept keeps.
 *   pk, pv, pg, pbeta, pe : the previous round's retained rows and stash, as
 *                 for kda_replay (kda_replay_stash with pe), in a
 *                 [L][T_prev][H] layout.  With pe, pv and pbeta are not read.  All may be NULL when keep == 0.
 *   T_prev      : the previous round's row count, 0..KDA_T_MAX.
 *   keep        : previous-round rows to keep, 0..T_prev (0: snap_prev is
 *                 already committed; then snap_out is a copy of it).
 *   q..beta, o  : this round's rows and outputs, as for kda_scan_rows; o is
 *                 required.  e (optional) receives this round's stash plane,
 *                 as kda_scan_rows_stash writes it.
 *   1 <= T <= KDA_T_MAX.
 * Bit for bit, snap_out equals kda_replay(snap_prev, ..., keep) and o equals
 * kda_scan_rows(snap_out, ...)'s outputs.
 */
int kda_verify_round(const float* snap_prev, float* snap_out, const void* pk, const void* pv,
                     const void* pg, const void* pbeta, const float* pe, int T_prev, int keep,
                     const void* q, const void* k, const void* v, const void* g,
                     const void* beta, float* o, float* e, int L, int T, int H, int in_dtype,
                     void* stream);

/*
 * The retained rows of an earlier verify round, for kda_verify_round_multi:
 * k, g and either its stash plane e or v and beta, all in that round's
 * layout [L][T][H][128] ([L][T][H] for beta), in the launch's in_dtype.
 */
typedef struct {
    const void* k;
    const void* v;      /* may be NULL when e is given */
    const void* g;
    const void* beta;   /* may be NULL when e is given */
    const float* e;     /* that round's stash plane, or NULL */
    int T;              /* that round's rows per layer, 1..KDA_T_MAX */
    int keep;           /* its rows to replay, 0..T (0: nothing of that round) */
} kda_prev_round;

/*
 * A fused verify round that replays several earlier rounds.
 *   glm_spec.rs (0.123.0), ROLLBACK: a rolled-back state is rebuilt by
 *   replaying kept rows from a snapshot, and the replay is the scan's own row
 *   program.  Extending kda_verify_round, the snapshot may be older than the
 *   previous round: snap_base is the committed state before prev[0], and the
 *   kept rows of prev[0], prev[1], ... are replayed in that order before this
 *   round's rows are scanned.  A caller can so store the committed state only
 *   every few rounds (snap_out = NULL in between) and save that write, which
 *   dominates the HBM bytes of a round at small K.
 *   snap_out : the committed state after all n_prev rounds (this round's
 *              snapshot), or NULL to not store it.  May be snap_base.
 *   prev     : HOST array of n_prev descriptors, 0 <= n_prev <= 4; either
 *              every replayed round (keep > 0) brings e or none does.
 *   The rest as for kda_verify_round.  Bit for bit, the result equals
 *   kda_replay of each round in turn, then kda_scan_rows of this round.
 */
int kda_verify_round_multi(const float* snap_base, float* snap_out, const kda_prev_round* prev,
                           int n_prev, const void* q, const void* k, const void* v,
                           const void* g, const void* beta, float* o, float* e, int L, int T,
                           int H, int in_dtype, void* stream);

/*
 * Greedy accept of one verify round.
 *   glm_spec.rs (0.123.0), glm5_spec_round step 4, greedy branch: one device
 *   argmax per verify row, the lowest index winning among equal maxima; then
 *   j = the length of the longest prefix of drafts that equal the argmaxes of
 *   their rows, and the bonus token is the argmax of row j.  A row holding a
 *   NaN has no argmax: its slot is KDA_NO_TOKEN, which the caller must refuse
 *   (the same file's sentinel guard on device argmaxes).
 *   logits : t rows of V logits in in_dtype (bf16 widens exactly by bits << 16);
 *            row r starts at element r*ld, ld >= V when t > 1 (ignored when
 *            t == 1).  Element alignment; 16-byte aligned rows (and ld a
 *            multiple of 4) take the vector-load kernel.
 *   t      : verify rows, 1..KDA_T_MAX (K + 1).
 *   drafts : t-1 u32 draft tokens, drafts[r] being the token fed after row r;
 *            may be NULL when t == 1.
 *   vam    : t u32, receives each row's argmax (or KDA_NO_TOKEN).
 *   out2   : 2 u32, receives {j, bonus}: 0 <= j <= t-1 accepted drafts and
 *            bonus = vam[j]; the round then commits keep = j + 1 rows.
 *   work   : KDA_ACCEPT_WORK_BYTES of device memory, 16-byte aligned, owned by
 *            the caller: scratch for per-row partial results, in any state on
 *            entry.  Calls that can run at the same time (on different
 *            streams) need different work buffers.
 * Comparisons are f32: -0 equals +0 (the lower index wins), -inf is an
 * ordinary value.  The outputs depend only on the inputs, never on timing.
 */
int kda_accept_greedy(const void* logits, int t, int V, long long ld, int in_dtype,
                      const uint32_t* drafts, uint32_t* vam, uint32_t* out2, void* work,
                      void* stream);

/*
 * kda_accept_greedy with no workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * forbid allocation, harnesses without an allocator).  The per-row partial
 * argmaxes go to a static device array inside the library, one per GPU,
 * sized for the largest call (KDA_T_MAX rows); its address is looked up on
 * the first call on each device.  The call itself allocates and frees
 * nothing.  Every call on one GPU shares that GPU's array: calls that can
 * overlap on one GPU (different streams, different host threads) race and
 * must use kda_accept_greedy with their own workspaces instead.  Arguments,
 * results and refusals are those of kda_accept_greedy; t outside
 * 1..KDA_T_MAX is refused as beyond the static array.
 */
int kda_accept_greedy_noalloc(const void* logits, int t, int V, long long ld, int in_dtype,
                              const uint32_t* drafts, uint32_t* vam, uint32_t* out2,
                              void* stream);

/*
 * Pre-scan row ops: one layer-set's projections to scan inputs, all t rows.
 *   glm_spec.rs (0.123.0), module doc VERIFY-ROW BATCHING: a KDA layer's
 *   gates and short conv run batched over the t = K+1 verify rows ahead of the
 *   scan; glm5_spec_ppn_gate.rs fixture: short_conv_kernel_size 4,
 *   gate_lower_bound -5.0.  Per row t, channel c, head h (d = 128):
 *     y_t[c] = SiLU(w[c][0] x_{t-3}[c] + w[c][1] x_{t-2}[c] + w[c][2] x_{t-1}[c]
 *                   + w[c][3] x_t[c])          x_{-3..-1} = the ring rows
 *     q, k   = the q, k blocks of y, each L2-normalised per (t, h):
 *              y / sqrt(sum y^2 + 1e-6);  v = the v block of y
 *     g      = max(-softplus(a_t), -5);  beta = sigmoid(b_t)
 *   (The pages fix the kernel size, the bound and the order of these ops;
 *   SiLU after the conv, no conv bias, the norm epsilon and -softplus as the
 *   gate's log-decay are this library's reading.)
 *   x        : [L][T][3*H*128] in in_dtype, the raw q | k | v projections
 *              (channel c = block*H*128 + h*128 + j).  Element alignment.
 *   a        : [L][T][H*128] gate pre-activations; b : [L][T][H].
 *   conv_w   : [L][3*H*128][4] f32 taps, oldest first, 16-byte aligned.
 *   ring_in  : [L][3][3*H*128] f32, the conv ring before row 0 (row 0 oldest).
 *   ring_out : [L][3][3*H*128] f32 or NULL: the ring after all T rows (the
 *              full-accept ring; kda_conv_reroll gives it for a partial
 *              accept).  Must not overlap ring_in: rows are computed in
 *              parallel, and the early rows read ring_in.
 *   q, k, v, g : [L][T][H][128] f32, beta : [L][T][H] f32 -- the scan's
 *              inputs, 16-byte aligned (beta: 4 bytes).
 *   1 <= T <= KDA_T_MAX, L, H >= 1.
 */
int kda_row_ops(const void* x, const void* a, const void* b, const float* conv_w,
                const float* ring_in, float* ring_out, float* q, float* k, float* v, float* g,
                float* beta, int L, int T, int H, int in_dtype, void* stream);

/*
 * Conv-ring rollback.
 *   glm_spec.rs (0.123.0), module doc VERIFY-ROW BATCHING and the
 *   Glm5VerifyCkpt doc: a KDA layer's short-conv ring holds the last
 *   KDA_CONV_RING_ROWS raw conv inputs (glm5_spec_ppn_gate.rs fixture:
 *   short_conv_kernel_size 4); on a partial accept it is rebuilt from the
 *   pre-round ring snapshot by rolling it once per kept row over the round's
 *   retained raw rows.
 *   ring_snap : [L][3][C] f32, the rings before the round, row 0 the oldest.
 *   raw       : [L][T_round][C] in in_dtype, the round's raw conv inputs
 *               (the q/k/v projections before the conv), element alignment.
 *   ring_out  : [L][3][C] f32, receives, in row m, entry keep + m of the
 *               sequence (ring_snap rows 0..2, raw rows 0..T_round-1).
 *   1 <= keep <= T_round <= KDA_T_MAX, L >= 1, C >= 1.  ring_out must not
 *   overlap ring_snap or raw.  16-byte aligned buffers with C a multiple of 4
 *   take the vector kernel; any element-aligned layout is accepted.
 */
int kda_conv_reroll(const float* ring_snap, const void* raw, float* ring_out, int L,
                    int T_round, int keep, long long C, int in_dtype, void* stream);

/*
 * The rollback with the accepted-draft count left on the device: as
 * kda_verify_round and kda_conv_reroll, with keep = min(*j, T - 1) + 1 read
 * by the kernels themselves (T = T_prev, or T_round), where j is the u32 that
 * kda_accept_greedy writes to out2[0].  The host then need not wait for j
 * between the accept and the rollback: a whole verify round, accept and
 * rollback included, can be enqueued (or captured in a HIP graph) before j
 * is read back.  glm_spec.rs (0.123.0), glm5_spec_round step 4 and
 * glm5_verify_rollback: the round commits keep = j + 1 rows.
 *   j        : device pointer to one uint32, 4-byte aligned; it must not
 *              overlap an output.  A j >= T (never produced by the accept) is
 *              clamped to keep = T.
 *   others   : as kda_verify_round (with 1 <= T_prev) and kda_conv_reroll;
 *              the retained rows are validated for all T_prev (T_round) rows.
 */
int kda_verify_round_dev(const float* snap_prev, float* snap_out, const void* pk, const void* pv,
                         const void* pg, const void* pbeta, const float* pe, int T_prev,
                         const uint32_t* j, const void* q, const void* k, const void* v,
                         const void* g, const void* beta, float* o, float* e, int L, int T,
                         int H, int in_dtype, void* stream);
int kda_conv_reroll_dev(const float* ring_snap, const void* raw, float* ring_out, int L,
                        int T_round, const uint32_t* j, long long C, int in_dtype, void* stream);

/*
 * Batched uniform copy: n buffers of `words` f32 each, in one launch.
 *   dflash.rs (memra-engine 0.98.0), DsparkSnapBatch / copy_batch_uniform_f32:
 *   the batched GDN state snapshot, where one pointer-table refresh and one
 *   launch replace a copy per layer.
 *   table : DEVICE array of 2n u64, [src_0 .. src_{n-1}, dst_0 .. dst_{n-1}],
 *           8-byte aligned; each entry a device address of `words` f32
 *           (4-byte aligned; pairs that are both 16-byte aligned, with words a
 *           multiple of 4, move 16 bytes per access).
 *   1 <= n <= 65535, words >= 1.
 * The library cannot read the table on the host: the caller guarantees that
 * every entry is a valid device buffer of that size and that no destination
 * overlaps a source or another destination.
 */
int kda_copy_batch(const uint64_t* table, int n, long long words, void* stream);

/* Message for the last nonzero status returned on the calling thread. */
const char* kda_last_error(void);

/* KDA_ABI_VERSION of the built library. */
int kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
