// Internal interface between the C-ABI layer (kda_abi.cpp) and the gfx950
// kernels (kda_kernels.hip).  Not installed; callers use include/kda.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace kda {

constexpr int kD = 128;        // head dim: d_k = d_v
constexpr int kTMax = 15;      // verify rows per launch
constexpr int kBMax = 15;      // batched-decode sessions

constexpr int kMaxPrev = 4;   // earlier rounds one fused launch can replay

// The retained rows of an earlier round: k, g and either e (the stash plane)
// or v and beta, in that round's layout [L][T][H][128].
struct PrevRows {
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    const float* e;
    int T;      // rows per layer in that round's layout
    int keep;   // rows to replay, 1..T
};

// One launch of the row kernel.  Either the contiguous layout
//   state [chain][128][128], chain = l*H + h, rows [L][T_stride][H][128]
// or (batched) the table layout
//   state s_ptrs[l*B + b] + h*128*128, chain = (l*B + b)*H + h, rows [L][B][H][128].
struct ScanArgs {
    const float* s_in;
    float* s_out;
    float* const* s_ptrs;
    // this launch's rows
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    const float* e_in;   // stash plane read by a stash replay
    float* o;            // per-row outputs (full rows)
    float* e_out;        // stash plane written by a scan, or nullptr
    // fused verify round only: earlier rounds' kept rows, replayed in order
    // from s_in before this launch's rows (entries with keep = 0 left out)
    PrevRows prev[kMaxPrev];
    int n_prev;
    // if set, prev[0] replays min(*keep_j, prev[0].T - 1) + 1 rows: j, the
    // accepted-draft count, as the greedy accept left it in device memory
    const uint32_t* keep_j;
    // state columns (kScanColumns): the state after row t of chain c at
    // s_cols + t * col_stride + c * 128 * 128
    float* s_cols;
    size_t col_stride;
    long long n_chains;  // (layer, head) or (layer, session, head) chains
    long long n_head_chains;   // chains run whole-head before a split tail (launcher)
    unsigned long long entry_mul;  // batched arm: table entries run in order (i * entry_mul) mod n
    int H;
    int T;               // rows this launch runs
    int T_stride;        // rows per layer in this launch's input layout
};

enum class Launch {
    kScanOut,       // T rows, outputs o (and e), state stored
    kScanState,     // T rows, state (and e) only
    kReplay,        // keep rows recomputed from the row inputs, state stored
    kReplayStash,   // keep rows from the stash plane e, state stored
    kBatchedOut,    // batched arm, one row per session, o
    kBatchedState,  // batched arm, state only
    kRound,         // fused verify round: replay (recomputed), store (if s_out), scan for o
    kRoundStash,    // fused verify round: replay from the stash, store (if s_out), scan for o
    kScanColumns,   // T rows, outputs o (and e), the state after every row stored
};

hipError_t launch_scan(const ScanArgs& a, Launch kind, bool bf16, hipStream_t stream);

hipError_t launch_copy(const float* src, float* dst, size_t n_floats, hipStream_t stream);

constexpr int kRingRows = 3;   // short-conv history rows (kernel size 4)

struct RerollArgs {
    const float* ring_snap;   // [L][3][C]
    const void* raw;          // [L][T][C] in the row dtype
    float* ring_out;          // [L][3][C]
    long long C;
    long long blocks_per_layer;   // set by launch_reroll
    const uint32_t* keep_j;       // if set, keep = min(*keep_j, T - 1) + 1
    int L;
    int T;
    int keep;
};

hipError_t launch_reroll(const RerollArgs& a, bool bf16, hipStream_t stream);

struct RowOpsArgs {
    const void* x;          // [L][T][3*H*128] raw q, k, v projections (row dtype)
    const void* a;          // [L][T][H*128] gate pre-activations
    const void* b;          // [L][T][H] beta pre-activations
    const float* w;         // [L][3*H*128][4] conv taps, oldest first
    const float* ring_in;   // [L][3][3*H*128]
    float* ring_out;        // [L][3][3*H*128] after all T rows, or nullptr
    float* q;               // [L][T][H][128]
    float* k;
    float* v;
    float* g;
    float* beta;            // [L][T][H]
    long long nwork;        // workgroups with work: L*H*ceil(T/3), set by launch_row_ops
    int L;
    int T;
    int H;
};

hipError_t launch_row_ops(const RowOpsArgs& a, bool bf16, hipStream_t stream);

// n uniform copies of `words` floats from a device table [src.., dst..].
hipError_t launch_copy_batch(const uint64_t* table, int n, long long words, hipStream_t stream);

constexpr uint32_t kNoToken = 0xFFFFFFFFu;   // argmax of a row that holds a NaN
constexpr int kAcceptPMax = 64;              // workgroups per row, at most

// Scratch of one greedy accept: the per-(row, workgroup) partial argmaxes
// the first launch writes and the second reads.  Nothing in it needs to be
// initialised.
struct AcceptScratch {
    float pv[kTMax * kAcceptPMax];
    uint32_t pi[kTMax * kAcceptPMax];
    uint32_t pn[kTMax * kAcceptPMax];
};

struct AcceptArgs {
    const void* logits;      // row r at element r*ld
    long long ld;
    int t;                   // rows, 1..kTMax
    int V;                   // logits per row, >= 1
    const uint32_t* drafts;  // t-1 draft tokens
    uint32_t* vam;           // t argmaxes
    uint32_t* out2;          // {j, bonus}
    float* pv;               // AcceptScratch members
    uint32_t* pi;
    uint32_t* pn;
};

int accept_workgroups_per_row(int V);
hipError_t launch_accept(const AcceptArgs& a, bool bf16, hipStream_t stream);

// The calling thread's current device's static accept scratch (device
// address), looked up on the first call for that device.
hipError_t accept_static_scratch(AcceptScratch** out);

}  // namespace kda
