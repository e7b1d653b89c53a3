// gfx950 kernels of the KDA verify-row scan.
//
// A workgroup owns one (layer, head) chain -- or, in the batched arm, one
// (layer, session, head) chain; in launches with few chains, a 32- or 64-column
// block of one -- and keeps that part of the head's 128 x 128 f32 state in
// VGPRs for the whole row loop: the state is read from HBM once and written
// once per launch, whatever the row count T.  This is what the source page
// (memra-engine 0.123.0 glm_spec.rs, module doc VERIFY-ROW BATCHING) means by
// the in-kernel T-loop over register state being the chained t=1 program.
//
// Per row of one head (i = key channel, j = value channel):
//   d_i = exp(clamp(g_i, -5, 0))                 (once per row, into LDS)
//   S'  = d_i * S_ij                              (VGPR, in place)
//   u_j = sum_i k_i S'_ij,  w_j = sum_i q_i S'_ij (in-lane FMA chains, then a
//                                                 fixed DPP butterfly)
//   e_j = beta (v_j - u_j)
//   S   = S' + k_i e_j                            (VGPR, in place)
//   o_j = (w_j + e_j * (q.k)) / sqrt(128)
// The last line is o = S^T q read from the updated state, expanded as
// q^T S' + (q.k) e so that both reductions of a row run in one phase.
//
// Tiling.  The recurrence reduces over i only; value columns never interact.
// A lane owns R consecutive key rows x C consecutive value columns; the NI =
// 128/R lanes that share a column group sit next to each other inside one
// 16-lane DPP row, so the reduction over i is an in-lane chain followed by a
// log2(NI)-step butterfly with no LDS traffic and no barrier.  R = 16 (NI = 8)
// throughout; a workgroup has 4 waves covering 4*(64/NI)*C columns, so a head
// takes 1, 2 or 4 workgroups for C = 4, 2, 1.  The whole-head verify scan and
// fused round place the 8 lanes of a column group across the wave's 16-lane
// rows instead and reduce with cross-row swaps (the swap layout, below): the
// same pairs in the same order, fewer VALU ops.
//
// Bit identity.  Every entry point (T-row scan, replay, batched t=1) runs the
// same row code with the same key split, explicit fmaf, -ffp-contract=off,
// one decay routine, and a reduction tree that does not depend on T, B, L, H,
// C or the entry point.  The state crosses HBM as exact f32 words, so a T-row
// launch equals T chained one-row launches bit for bit, and every tiling gives
// the same bits.
//
// Rollback.  A scan can also write each row's delta vector e (the "stash"
// plane beside the row inputs).  A replay that reads e skips both reductions:
// per element it is the decay multiply and the rank-1 FMA, with the very e
// bits the scan used, so it rebuilds the same state bits.  The fused verify
// round replays the previous round's kept rows from its snapshot (or several
// earlier rounds' from an older one), stores that committed state (this
// round's snapshot) and then scans the new rows for o, so the state crosses
// HBM once per round.
//
// No MFMA: each row is two matrix-vector products and a rank-1 update with a
// sequential dependency from row to row -- there is no dense contraction to
// feed the matrix cores.
//
// Memory.  State words stream past the caches (nontemporal loads and stores):
// each is read once and written once per launch.  Every row input of a phase
// and the state are in flight before the first wait; the fused round also
// issues this round's row loads before its replay.  The batched arm walks its
// table entries in a spread order, so that the workgroups in flight touch
// sessions far apart in memory.  The workgroups that split one head run on one
// XCD (workgroup indices equal mod 8), whose L2 then serves their repeated
// reads of the head's rows.
//
// No MFMA for the rank-1 write either: on gfx950 an f32 MFMA does not overlap
// independent VALU work (their times add), and the 4x4x1 form costs about as
// much as the four VALU FMAs it would replace.
//
// Beside the scan, all HBM- or latency-bound: the pre-scan row ops (short
// conv, norms, gate, beta) that produce the scan's inputs; the conv-ring
// rollback; a plain copy (snapshots) and a pointer-table batched copy; and the
// greedy accept (split-row argmax, then a one-workgroup prefix walk).

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kDD = kD * kD;
constexpr float kGateLo = -5.0f;   // gate_lower_bound of the glm5_next fixture
constexpr float kGateHi = 0.0f;    // a log-decay never grows the state
// 1/sqrt(128) rounded to f32
constexpr float kInvSqrtD = 0.0883883476483184405501055452631f;

template <int R, int C>
struct Tile {
    static constexpr int NI = kD / R;          // lanes reducing one column group
    static constexpr int NJG = 64 / NI;        // column groups per wave
    static constexpr int WCOLS = NJG * C;      // value columns per wave
    static constexpr int WAVES = 4;            // waves per workgroup
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int BCOLS = WAVES * WCOLS;   // value columns per workgroup
    static constexpr int BLOCKS = kD / BCOLS;     // workgroups per head
    static_assert(NI == 4 || NI == 8 || NI == 16, "the reduction must stay in one DPP row");
    static_assert(kD % BCOLS == 0, "workgroups must tile the head");
    static_assert(C == 1 || C == 2 || C == 4, "column vector width");
};

// The key split R = 16 (8 lanes per column group) fixes the rounding: each
// value column is an in-lane chain over its lane's 16 keys, in order, then
// the same 3-step butterfly, whatever C is.  C (value columns per lane) only
// sets how many workgroups share a head -- 1 at C = 4, 2 at C = 2, 4 at C = 1
// -- so launches with few chains can spread over the chip and still give the
// bits of every other launch.
constexpr int kKeysPerLane = 16;

// ------------------------------------------------------------------ lane ops

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over NI adjacent lanes, every lane ending with the same bits: each step
// adds a value to its partner's, and partners compute a+b and b+a.
template <int NI>
__device__ __forceinline__ float group_sum(float x) {
    x = x + dpp<0xB1>(x);                          // quad_perm [1,0,3,2]
    x = x + dpp<0x4E>(x);                          // quad_perm [2,3,0,1]
    if constexpr (NI >= 8) x = x + dpp<0x141>(x);  // row_half_mirror
    if constexpr (NI >= 16) x = x + dpp<0x140>(x); // row_mirror
    return x;
}

// The swap layout (whole-head launches that write o): the 8 key groups of a
// column group sit on lane bits 4, 5 and 3 (key-group bits 0, 1 and 2) and
// the column group on lane bits 0-2.  One 16-lane row then holds one value of
// key-group bits 0-1, so gfx950's cross-row swaps pair key groups g and g^1
// (v_permlane16_swap), then g^2 (v_permlane32_swap), and DPP row_ror:8 pairs
// g and g^4: the pairs of group_sum<8>, in its order, so every sum keeps its
// bits.  A reduce-scatter over the 4 columns of a lane costs 7 VALU ops
// instead of group_sum's 12, and the column each lane ends with is all that
// o needs.  (Written as asm: the compiler's swap builtins return the first
// register for both results.  The s_nop covers the VALU-write to swap-read
// wait states.)
__device__ __forceinline__ void swap16(float& a, float& b) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap32(float& a, float& b) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// Sum of x[0..3] over the 8 key groups; the lanes of row k (lane bits 4-5)
// end with column k's sum.
__device__ __forceinline__ float reduce_scatter4(const float (&x)[4]) {
    float a = x[0], b = x[1], c = x[2], d = x[3];
    swap16(a, b);   // even rows: column 0 of the row pair; odd rows: column 1
    swap16(c, d);   // even rows: column 2; odd rows: column 3
    float lo = a + b, hi = c + d;
    swap32(lo, hi); // row k: column k over rows k and k^2
    const float r = lo + hi;
    return r + dpp<0x128>(r);   // row_ror:8 pairs lane bit 3
}

// ------------------------------------------------------------------ input loads

template <bool BF16>
__device__ __forceinline__ float4 load4(const void* base, size_t off) {
    if constexpr (BF16) {
        const uint2 raw = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + off);
        float4 r;
        r.x = __builtin_bit_cast(float, raw.x << 16);
        r.y = __builtin_bit_cast(float, raw.x & 0xFFFF0000u);
        r.z = __builtin_bit_cast(float, raw.y << 16);
        r.w = __builtin_bit_cast(float, raw.y & 0xFFFF0000u);
        return r;
    } else {
        return *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* base, size_t off) {
    if constexpr (BF16) {
        return __builtin_bit_cast(float,
                                  static_cast<uint32_t>(static_cast<const uint16_t*>(base)[off]) << 16);
    } else {
        return static_cast<const float*>(base)[off];
    }
}

// An empty asm the compiler must assume rewrites x: arithmetic on x cannot
// move above this point.
__device__ __forceinline__ void opaque(float4& x) {
    asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w)::"memory");
}

// exp(clamp(g, -5, 0)) as 2^(gc * log2(e)) on the hardware exp2 (v_exp_f32,
// about 1 ulp on this range).  With the f32 rounding of gc * log2(e) the
// decay is within about 3 ulp of exp(gc) -- and it is the one decay routine
// every entry point uses, so their results stay bit-identical.
constexpr float kLog2e = 1.44269504088896340736f;
__device__ __forceinline__ float decay_of(float g) {
    return __builtin_amdgcn_exp2f(__builtin_amdgcn_fmed3f(g, kGateLo, kGateHi) * kLog2e);
}

// Pointers known to address global memory: loads and stores through them are
// global (not flat) instructions even when the pointer was read from memory.
using gfloat = __attribute__((address_space(1))) float;
typedef float vf2 __attribute__((ext_vector_type(2)));
typedef float vf4 __attribute__((ext_vector_type(4)));
using gvf2 = __attribute__((address_space(1))) vf2;
using gvf4 = __attribute__((address_space(1))) vf4;

// State words.  NT: nontemporal (streaming) access.  A launch reads each state
// word once and writes it once, and the next reader is a later launch, so
// keeping them out of the caches costs nothing; it measured 7-9% faster fused
// rounds and 14% faster batched steps.
template <int C, bool NT>
__device__ __forceinline__ void load_gcols(const gfloat* p, float (&x)[C]) {
    if constexpr (C == 4) {
        const vf4 v = NT ? __builtin_nontemporal_load((const gvf4*)p) : *(const gvf4*)p;
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    } else if constexpr (C == 2) {
        const vf2 v = NT ? __builtin_nontemporal_load((const gvf2*)p) : *(const gvf2*)p;
        x[0] = v.x; x[1] = v.y;
    } else {
        x[0] = NT ? __builtin_nontemporal_load(p) : *p;
    }
}

template <int C, bool NT>
__device__ __forceinline__ void store_gcols(gfloat* p, const float (&x)[C]) {
    if constexpr (C == 4) {
        const vf4 v{x[0], x[1], x[2], x[3]};
        if constexpr (NT) __builtin_nontemporal_store(v, (gvf4*)p); else *(gvf4*)p = v;
    } else if constexpr (C == 2) {
        const vf2 v{x[0], x[1]};
        if constexpr (NT) __builtin_nontemporal_store(v, (gvf2*)p); else *(gvf2*)p = v;
    } else {
        if constexpr (NT) __builtin_nontemporal_store(x[0], p); else *p = x[0];
    }
}

template <int C>
__device__ __forceinline__ void load_cols(const float* p, float (&x)[C]) {
    if constexpr (C == 4) {
        const float4 v = *reinterpret_cast<const float4*>(p);
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    } else if constexpr (C == 2) {
        const float2 v = *reinterpret_cast<const float2*>(p);
        x[0] = v.x; x[1] = v.y;
    } else {
        x[0] = *p;
    }
}

template <int C>
__device__ __forceinline__ void store_cols(float* p, const float (&x)[C]) {
    if constexpr (C == 4) {
        *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    } else if constexpr (C == 2) {
        *reinterpret_cast<float2*>(p) = make_float2(x[0], x[1]);
    } else {
        *p = x[0];
    }
}

// ------------------------------------------------------------------ the scan

// LDS row layout for the per-key vectors (decay, k, scaled q).  A lane reads
// the R consecutive keys of its group; group ig starts at ig*(R+4) floats so
// the NI groups of a wave land on distinct bank quads (a plain ig*R stride
// maps groups ig and ig+2 onto the same banks).
template <int R>
struct KeyRow {
    static constexpr int kPad = 4;
    static constexpr int kStride = (kD / R) * (R + kPad);   // floats per row
    __device__ static constexpr int at(int i) { return (i / R) * (R + kPad) + i % R; }
};

// What a phase of rows computes.
enum class Rows {
    kNone,
    kFull,    // u and w reductions: state, o and (optionally) e -- the verify scan
    kState,   // u reduction only: state and (optionally) e
    kStash,   // e read from the stash: decay and rank-1 update only
    kFullCols,   // kFull, and the state after every row stored (state columns)
};

// Modes that reduce S'^T q and write o.
constexpr bool has_q(Rows m) { return m == Rows::kFull || m == Rows::kFullCols; }

// Up to TM rows of one phase, staged in LDS (the batched arm stages one).
// The key-layout arrays of a multi-row stage hold one spare row past TM: the
// narrow tilings read the next row's keys during each row, and after the last
// row that read lands there (its values are never used).  The batched arm's
// one-row stage has none (it runs whole heads).
template <int R, int TM = kTMax>
struct Stage {
    static constexpr int kRows = TM > 1 ? TM + 1 : TM;
    float4 d[kRows * KeyRow<R>::kStride / 4];   // exp(clamp(g)), key layout
    float4 k[kRows * KeyRow<R>::kStride / 4];   // k, key layout
    float4 q[kRows * KeyRow<R>::kStride / 4];   // q / sqrt(128), key layout (kFull)
    float4 ve[TM * kD / 4];                  // beta * v, or e for kStash; [t][j]
    float2 bq[TM];                           // beta, (q / sqrt(128)) . k: one LDS read
};

// One phase's row inputs, located for one chain.
struct Src {
    const void *q, *k, *v, *g, *beta;
    const float* e;              // the stash plane (kStash)
    size_t row0, rstride;        // element offset of row 0, elements between rows
    size_t b0, bstride;          // beta
    int T;
};

// One phase's row inputs in flight: float4 loads per lane per input, enough
// for TMAX rows of 32 float4.
template <int R, int C, Rows M, int TMAX>
struct Staged {
    static constexpr int kPer = (TMAX * (kD / 4) + Tile<R, C>::THREADS - 1) / Tile<R, C>::THREADS;
    float4 k[kPer], v[kPer], g[kPer], q[kPer];
    float b[kPer];
};

// Issue every global load of a phase's rows (nothing waits on them here).
template <int R, int C, bool BF16, Rows M, int TMAX>
__device__ __forceinline__ void stage_issue(Staged<R, C, M, TMAX>& in, const Src& src, int tid) {
    using TL = Tile<R, C>;
    const int T = src.T;
#pragma unroll
    for (int p = 0; p < Staged<R, C, M, TMAX>::kPer; ++p) {
        // unconditional (row clamped into range, surplus values unused): a
        // branch here would make the merge copies wait on the loads
        const int idx = tid + p * TL::THREADS;
        const int t = min(idx >> 5, T - 1);
        const size_t off = src.row0 + t * src.rstride + (idx & 31) * 4;
        in.k[p] = load4<BF16>(src.k, off);
        in.g[p] = load4<BF16>(src.g, off);
        if constexpr (M == Rows::kStash) {
            in.v[p] = *reinterpret_cast<const float4*>(src.e + off);
        } else {
            in.v[p] = load4<BF16>(src.v, off);
            in.b[p] = load1<BF16>(src.beta, src.b0 + t * src.bstride);
        }
        if constexpr (has_q(M)) in.q[p] = load4<BF16>(src.q, off);
    }
}

// Keep the staging arithmetic from being hoisted between the loads (it would
// wait on the first input load before later loads are issued): the staged
// values pass through an empty asm placed after every load of the launch.
template <int R, int C, Rows M, int TMAX>
__device__ __forceinline__ void stage_fence(Staged<R, C, M, TMAX>& in) {
#pragma unroll
    for (int p = 0; p < Staged<R, C, M, TMAX>::kPer; ++p) {
        opaque(in.k[p]);
        opaque(in.v[p]);
        opaque(in.g[p]);
        if constexpr (has_q(M)) opaque(in.q[p]);
        if constexpr (M != Rows::kStash) asm volatile("" : "+v"(in.b[p])::"memory");
    }
}

// Write a phase's rows to LDS in the scan's layout (decay, q/sqrt(128), beta v
// or e) with (q/sqrt(128)).k per row.  With SYNC, ends with every lane past a
// barrier (without it, the caller places one before the rows are read).
template <int R, int C, Rows M, int TMAX, bool SYNC = true>
__device__ __forceinline__ void stage_commit(Stage<R, TMAX>& L, const Staged<R, C, M, TMAX>& in, int T,
                                             int tid) {
    using TL = Tile<R, C>;
    using KR = KeyRow<R>;
    float* sd = reinterpret_cast<float*>(L.d);
    float* sk = reinterpret_cast<float*>(L.k);
    float* sq = reinterpret_cast<float*>(L.q);
#pragma unroll
    for (int p = 0; p < Staged<R, C, M, TMAX>::kPer; ++p) {
        const int idx = tid + p * TL::THREADS;
        if (idx < T * (kD / 4)) {
            const int t = idx >> 5;
            const int c4 = idx & 31;
            const int kp = t * KR::kStride + KR::at(c4 * 4);   // 4 keys never straddle a group
            const float4 gg = in.g[p];
            *reinterpret_cast<float4*>(sk + kp) = in.k[p];
            *reinterpret_cast<float4*>(sd + kp) =
                make_float4(decay_of(gg.x), decay_of(gg.y), decay_of(gg.z), decay_of(gg.w));
            if constexpr (M == Rows::kStash) {
                L.ve[t * 32 + c4] = in.v[p];
            } else {
                const float bt = in.b[p];
                const float4 gv = in.v[p];
                L.ve[t * 32 + c4] = make_float4(bt * gv.x, bt * gv.y, bt * gv.z, bt * gv.w);
                if (c4 == 0) L.bq[t].x = bt;
            }
            if constexpr (has_q(M)) {
                const float4 gq = in.q[p];
                *reinterpret_cast<float4*>(sq + kp) = make_float4(
                    gq.x * kInvSqrtD, gq.y * kInvSqrtD, gq.z * kInvSqrtD, gq.w * kInvSqrtD);
            }
        }
        // (q/sqrt(128)).k per row, from the registers: the 32 lanes of a half
        // wave hold one row, 4 keys each; each lane's 4 keys in ascending
        // order, then a fixed butterfly over the 32 lanes.  Every lane takes
        // part (the loads were clamped into range), so the DPP and swap reads
        // see defined values; only rows in range are written.
        if constexpr (has_q(M)) {
            const float4 gq = in.q[p], gk = in.k[p];
            float d = fmaf(gq.x * kInvSqrtD, gk.x, 0.0f);
            d = fmaf(gq.y * kInvSqrtD, gk.y, d);
            d = fmaf(gq.z * kInvSqrtD, gk.z, d);
            d = fmaf(gq.w * kInvSqrtD, gk.w, d);
            d = group_sum<16>(d);
            float d2 = d;
            swap16(d, d2);   // even rows: (own, odd partner); odd rows: (even partner, own)
            d = d + d2;
            if (idx < T * (kD / 4) && (idx & 31) == 0) L.bq[idx >> 5].y = d;
        }
    }
    if constexpr (SYNC) __syncthreads();
}

// A phase's rows from HBM into LDS; `between` runs after the row loads are
// issued and before anything waits on them (the state loads go there, when
// this is the first phase).  Ends with the staged rows visible to every wave.
template <int R, int C, bool BF16, Rows M, int TMAX = kTMax, typename F>
__device__ __forceinline__ void stage(Stage<R, TMAX>& L, const Src& src, int tid, F&& between) {
    Staged<R, C, M, TMAX> in;
    stage_issue<R, C, BF16, M, TMAX>(in, src, tid);
    between();
    stage_fence<R, C, M, TMAX>(in);
    stage_commit<R, C, M, TMAX>(L, in, src.T, tid);
}

// ------------------------------------------------------------------ quad key broadcast
//
// Every tiling puts the column group on lane bits 0-2 and the key group on
// bits 3-5 (key-group bits 0, 1, 2 on lane bits 4, 5, 3: the swap layout), so
// the four lanes of a quad (bits 0-1) hold different value columns of the
// same 16 keys.  Quad lane n reads keys 4n..4n+3 of a row's per-key vectors
// (decay, k, scaled q) as one float4; key r of the group is then register
// r % 4 of quad lane r / 4, and each VALU op that consumes it reads it
// through a DPP quad_perm broadcast.  A lane reads 3 float4 per row instead of
// 12 (all 16 of its keys, for each vector), with the same arithmetic in the
// same order.

// x of quad lane N, as the first operand of the consuming op (the compiler
// folds this into v_mul_f32_dpp)
template <int N>
__device__ __forceinline__ float quad_lane(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), N * 0x55, 0xF, 0xF, true));
}

// acc = (x of quad lane N) * y + acc, one v_fmac_f32 with a DPP operand (the
// compiler does not fold a broadcast into fmac).  x is always a register an
// LDS read wrote, never a VALU op, so the DPP read needs no wait states.
template <int N>
__device__ __forceinline__ void fmac_quad(float& acc, float x, float y);
#define KDA_FMAC_QUAD(N)                                                                        \
    template <>                                                                                 \
    __device__ __forceinline__ void fmac_quad<N>(float& acc, float x, float y) {                \
        asm("v_fmac_f32_dpp %0, %1, %2 quad_perm:[" #N "," #N "," #N "," #N                     \
            "] row_mask:0xf bank_mask:0xf"                                                      \
            : "+v"(acc)                                                                         \
            : "v"(x), "v"(y));                                                                  \
    }
KDA_FMAC_QUAD(0)
KDA_FMAC_QUAD(1)
KDA_FMAC_QUAD(2)
KDA_FMAC_QUAD(3)
#undef KDA_FMAC_QUAD

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// A row's per-key values for this lane's 16 keys, and the ops that consume
// them.  Two sources with the same arithmetic, so every tiling gives the same
// bits:
//   DPP = false: all 16 keys of each vector read from LDS (12 float4 per row);
//   DPP = true:  3 float4 per row, each key broadcast within the quad.
// An op with a DPP operand issues in about 1.2x the cycles of a plain one
// (measured on gfx950), so the VALU-bound whole-head tiling reads its keys
// from LDS, and the narrow tilings -- one or two waves per SIMD, where a row's
// LDS traffic and latency dominate -- broadcast them.
template <bool DPP>
struct RowKeys;

template <>
struct RowKeys<false> {
    float k[16], d[16], q[16];
    template <int R, bool Q, int TM>
    __device__ __forceinline__ void read(const Stage<R, TM>& L, int t, int i0, int) {
        using KR = KeyRow<R>;
        const int kb = (t * KR::kStride + KR::at(i0)) / 4;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const float4 x = L.k[kb + r4], y = L.d[kb + r4];
            k[4 * r4 + 0] = x.x; k[4 * r4 + 1] = x.y; k[4 * r4 + 2] = x.z; k[4 * r4 + 3] = x.w;
            d[4 * r4 + 0] = y.x; d[4 * r4 + 1] = y.y; d[4 * r4 + 2] = y.z; d[4 * r4 + 3] = y.w;
            if constexpr (Q) {
                const float4 z = L.q[kb + r4];
                q[4 * r4 + 0] = z.x; q[4 * r4 + 1] = z.y; q[4 * r4 + 2] = z.z; q[4 * r4 + 3] = z.w;
            }
        }
    }
    template <int r> __device__ __forceinline__ float decay(float x) const { return d[r] * x; }
    template <int r> __device__ __forceinline__ float kmul(float x) const { return k[r] * x; }
    template <int r> __device__ __forceinline__ float qmul(float x) const { return q[r] * x; }
    template <int r> __device__ __forceinline__ void kfma(float& acc, float x) const { acc = fmaf(k[r], x, acc); }
    template <int r> __device__ __forceinline__ void qfma(float& acc, float x) const { acc = fmaf(q[r], x, acc); }
};

template <>
struct RowKeys<true> {
    float k[4], d[4], q[4];   // keys i0 + 4n .. i0 + 4n + 3 of quad lane n
    template <int R, bool Q, int TM>
    __device__ __forceinline__ void read(const Stage<R, TM>& L, int t, int i0, int n) {
        using KR = KeyRow<R>;
        const int at = (t * KR::kStride + KR::at(i0 + 4 * n)) / 4;
        const float4 kk = L.k[at], dd = L.d[at];
        k[0] = kk.x; k[1] = kk.y; k[2] = kk.z; k[3] = kk.w;
        d[0] = dd.x; d[1] = dd.y; d[2] = dd.z; d[3] = dd.w;
        if constexpr (Q) {
            const float4 qq = L.q[at];
            q[0] = qq.x; q[1] = qq.y; q[2] = qq.z; q[3] = qq.w;
        }
    }
    template <int r> __device__ __forceinline__ float decay(float x) const { return quad_lane<r / 4>(d[r % 4]) * x; }
    template <int r> __device__ __forceinline__ float kmul(float x) const { return quad_lane<r / 4>(k[r % 4]) * x; }
    template <int r> __device__ __forceinline__ float qmul(float x) const { return quad_lane<r / 4>(q[r % 4]) * x; }
    template <int r> __device__ __forceinline__ void kfma(float& acc, float x) const { fmac_quad<r / 4>(acc, k[r % 4], x); }
    template <int r> __device__ __forceinline__ void qfma(float& acc, float x) const { fmac_quad<r / 4>(acc, q[r % 4], x); }
};

// Decay, then the in-lane partial sums u (and w) over the 16 keys in order;
// the first key starts each sum with a plain product.
template <int C, bool Q>
__device__ __forceinline__ void decay_sums(const RowKeys<false>& x, float (&s)[16][C],
                                           float (&u)[C], float (&w)[C]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
            s[r][c] = x.d[r] * s[r][c];
            if (r == 0) {
                u[c] = x.k[0] * s[0][c];
                if constexpr (Q) w[c] = x.q[0] * s[0][c];
            } else {
                u[c] = fmaf(x.k[r], s[r][c], u[c]);
                if constexpr (Q) w[c] = fmaf(x.q[r], s[r][c], w[c]);
            }
        }
    }
}

template <int C, bool Q>
__device__ __forceinline__ void decay_sums(const RowKeys<true>& x, float (&s)[16][C],
                                           float (&u)[C], float (&w)[C]) {
    static_for<0, 16>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            s[r][c] = x.template decay<r>(s[r][c]);
            if constexpr (r == 0) {
                u[c] = x.template kmul<0>(s[0][c]);
                if constexpr (Q) w[c] = x.template qmul<0>(s[0][c]);
            } else {
                x.template kfma<r>(u[c], s[r][c]);
                if constexpr (Q) x.template qfma<r>(w[c], s[r][c]);
            }
        }
    });
}

// The rank-1 write S += k e^T.
template <int C>
__device__ __forceinline__ void write_rows(const RowKeys<false>& x, float (&s)[16][C],
                                           const float (&e)[C]) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int c = 0; c < C; ++c) s[r][c] = fmaf(x.k[r], e[c], s[r][c]);
}

template <int C>
__device__ __forceinline__ void write_rows(const RowKeys<true>& x, float (&s)[16][C],
                                           const float (&e)[C]) {
    static_for<0, 16>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
#pragma unroll
        for (int c = 0; c < C; ++c) x.template kfma<r>(s[r][c], e[c]);
    });
}

// A stash replay row: decay, then the rank-1 write, key by key.  From LDS
// the keys come four at a time: few live registers, which leaves room for the
// next phase's row loads the fused round holds meanwhile.
template <int C, bool Q, int R, int TM>
__device__ __forceinline__ void stash_rows_lds(const Stage<R, TM>& L, int t, int i0,
                                               float (&s)[16][C], const float (&e)[C]) {
    using KR = KeyRow<R>;
    const int kb = (t * KR::kStride + KR::at(i0)) / 4;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
        const float4 x = L.k[kb + r4];
        const float4 y = L.d[kb + r4];
        const float k4[4] = {x.x, x.y, x.z, x.w};
        const float d4[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int c = 0; c < C; ++c)
                s[4 * r4 + m][c] = fmaf(k4[m], e[c], d4[m] * s[4 * r4 + m][c]);
        asm volatile("" ::: "memory");   // the next four keys' reads wait here
    }
}

template <int C, typename K>
__device__ __forceinline__ void stash_rows(const K& x, float (&s)[16][C], const float (&e)[C]) {
    static_for<0, 16>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            s[r][c] = x.template decay<r>(s[r][c]);
            x.template kfma<r>(s[r][c], e[c]);
        }
    });
}

// Sum over the 8 key groups of one value in every lane: the pairs (g, g^1),
// (g, g^2), (g, g^4) on lane bits 4, 5, 3, each lane adding its partner's.
__device__ __forceinline__ float sum_groups(float x) {
    float y = x;
    swap16(x, y);   // even rows: (own, odd partner); odd rows: (even partner, own)
    x = x + y;
    y = x;
    swap32(x, y);
    x = x + y;
    return x + dpp<0x128>(x);   // row_ror:8
}

// Sums over the 8 key groups of two values a, b: rows with lane bit 4 clear
// end with a's sum, the others with b's.
__device__ __forceinline__ float sum_groups2(float a, float b) {
    swap16(a, b);   // even rows: (a own, a odd partner); odd rows: (b even partner, b own)
    float x = a + b;
    float y = x;
    swap32(x, y);
    x = x + y;
    return x + dpp<0x128>(x);
}

// A value of every lane in row r, copied to the lanes of row r ^ 1 (bit 4) and
// kept: the lane of row r gets (x of the even row of its pair, x of the odd).
__device__ __forceinline__ void gather_pair16(float& lo, float& hi) {
    hi = lo;
    swap16(lo, hi);
}

// Lane layouts.  Swap (every launch but the two below): column group on lane
// bits 0-2, key group on bits 4, 5, 3 (see reduce_scatter4 and quad_lane).
// Plain (the batched arm and the state-column arm at whole heads, which
// measured faster with it): key group on bits 0-2, column group on bits 3-5,
// each column reduced with group_sum<8>.  Both reduce with the same pairs in
// the same order, so they give the same bits.
template <int C, Rows M, bool TABLE>
constexpr bool plain_layout() {
    return C == 4 && (TABLE || M == Rows::kFullCols);
}

// o and e stores of the narrow tilings (C < 4): buffer stores from the
// chain's first row, one byte offset per lane, advanced a row at a time.  The
// lanes that do not store a value carry bit 31 in their offset; the resource
// covers 2^31 bytes, so their stores fall out of range and are dropped.  No
// exec-mask branch and no 64-bit address arithmetic per row: at one or two
// waves per SIMD every instruction of a row costs issue time.  A missing output gets
// an empty range, which drops every lane.
struct NarrowStores {
    __amdgpu_buffer_rsrc_t o, e;
    uint32_t oo, eo;   // this lane's byte offsets in the current row
    uint32_t step;     // bytes from one row to the next
    __device__ __forceinline__ void next() { oo += step; eo += step; }
};
constexpr int kBufferWords3 = 0x00020000;   // raw buffer, 32-bit data format

// s_waitcnt immediate that waits for vector memory only: vmcnt 0, expcnt and
// lgkmcnt at their maxima (gfx9 field layout).
constexpr int kWaitVmem = 0x0F70;

// One row t of one phase over the staged rows L.  The lane's key group starts
// at i0, its columns at j0 (ig: its key group, used by the plain layout).
// kFullCols: `cols` addresses this chain's state in column 0, and row t's
// state goes to cols + t * col_stride.
template <int R, int C, Rows M, bool PLAIN, int TM, bool PFK, typename K, typename F>
__device__ __forceinline__ void row_step(const Stage<R, TM>& L, const K& x, float (&s)[R][C], int t,
                                         float* o, float* e_out, size_t o0, size_t ostride,
                                         int ig, int i0, int j0, gfloat* cols, size_t col_stride,
                                         F&& next_keys, NarrowStores& ns) {
    const float* sve = reinterpret_cast<const float*>(L.ve);
    const int lane = threadIdx.x & 63;
    constexpr bool Q = has_q(M);
    if constexpr (M == Rows::kStash) {
        float e[C];
        load_cols<C>(sve + t * kD + j0, e);
        if constexpr (PFK) {
            next_keys();
            asm volatile("" ::: "memory");   // issued ahead of the row's arithmetic
        }
        if constexpr (C < 4) stash_rows<C>(x, s, e);
        else stash_rows_lds<C, false, R, TM>(L, t, i0, s, e);
        return;
    }
    const float2 bq = L.bq[t];
    const float nbt = -bq.x;
    // With the next row's keys read during this row, this row's beta*v is
    // read first: LDS reads return in order, so a read issued after those
    // would wait for them too.
    float ve1 = 0.0f;
    if constexpr (PFK) {
        static_assert(!PLAIN && C < 4, "the narrow tilings read keys ahead");
        ve1 = sve[t * kD + j0 + (C == 2 ? ((lane >> 4) & 1) : 0)];
        next_keys();
        asm volatile("" ::: "memory");   // issued ahead of the row's arithmetic
    }
    float u[C], w[C];
    decay_sums<C, Q>(x, s, u, w);
    float e[C];
    if constexpr (PLAIN) {
        float ve[C];   // beta * v
        load_cols<C>(sve + t * kD + j0, ve);
#pragma unroll
        for (int c = 0; c < C; ++c) {
            u[c] = group_sum<8>(u[c]);
            if constexpr (Q) w[c] = group_sum<8>(w[c]);
        }
#pragma unroll
        for (int c = 0; c < C; ++c) e[c] = fmaf(nbt, u[c], ve[c]);   // e = beta v - beta u
        const size_t row = o0 + t * ostride;
        if constexpr (Q) {
            // finish w's butterfly on every lane: sunk into the writer's
            // branch, its last DPP step would become mov 0, mov_dpp, add
#pragma unroll
            for (int c = 0; c < C; ++c) asm volatile("" : "+v"(w[c]));
            float ov[C];
#pragma unroll
            for (int c = 0; c < C; ++c) ov[c] = fmaf(e[c], bq.y, w[c]);
            if (ig == 0) store_cols<C>(o + row + j0, ov);
        }
        if (e_out != nullptr && ig == 0) store_cols<C>(e_out + row + j0, e);
    } else if constexpr (C == 4) {
        // row k (lane bits 4-5) ends with column k's sums; e comes back to
        // the lanes of its column group through a wave-private LDS slot
        const int kc = (lane >> 4) & 3;
        const uint32_t col = static_cast<uint32_t>(j0 + kc);
        float uo = reduce_scatter4(u);
        asm volatile("" : "+v"(uo));
        const float eo = fmaf(nbt, uo, sve[t * kD + col]);
        float ov = 0.0f;
        if constexpr (Q) {
            float wo = reduce_scatter4(w);
            asm volatile("" : "+v"(wo));
            ov = fmaf(eo, bq.y, wo);
        }
        // read back as one float4 per lane: 16-byte aligned
        __shared__ __attribute__((aligned(16))) float ex[4 * 8 * 4];
        float* slot = ex + (threadIdx.x >> 6) * 32 + (lane & 7) * 4;
        const size_t row = o0 + t * ostride;
        if ((lane & 8) == 0) {
            if constexpr (Q) {
                gfloat* orow = (gfloat*)(o + row);
                asm volatile("" : "+s"(orow));
                orow[col] = ov;
            }
            if (e_out != nullptr) {
                gfloat* erow = (gfloat*)(e_out + row);
                asm volatile("" : "+s"(erow));
                erow[col] = eo;
            }
            slot[kc] = eo;
        }
        __builtin_amdgcn_wave_barrier();   // one wave writes and reads the slots, in order
        load_cols<4>(slot, e);
    } else if constexpr (C == 2) {
        // column c = lane bit 4 (row & 1)
        static_assert(PFK, "the narrow tilings read keys ahead");
        float ec;
        if constexpr (Q) {
            // rows 0, 1 end with u of columns 0, 1; rows 2, 3 with w
            const float sums[4] = {u[0], u[1], w[0], w[1]};
            const float x4 = reduce_scatter4(sums);
            ec = fmaf(nbt, x4, ve1);                 // valid in rows 0, 1
            float e2 = ec;
            swap32(ec, e2);                          // rows 2, 3 take e from rows 0, 1
            const float ov = fmaf(ec, bq.y, x4);     // valid in rows 2, 3
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, ov), ns.o, ns.oo, 0, 0);
        } else {
            ec = fmaf(nbt, sum_groups2(u[0], u[1]), ve1);
        }
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, ec), ns.e, ns.eo, 0, 0);
        ns.next();
        gather_pair16(ec, e[1]);
        e[0] = ec;
    } else {
        static_assert(PFK, "the narrow tilings read keys ahead");
        if constexpr (Q) {
            const float x2 = sum_groups2(u[0], w[0]);   // even rows u, odd rows w
            float ec = fmaf(nbt, x2, ve1);              // valid in even rows
            float odd;
            gather_pair16(ec, odd);                     // ec: the even row's e, in all rows
            const float ov = fmaf(ec, bq.y, x2);        // valid in odd rows
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, ov), ns.o, ns.oo, 0, 0);
            e[0] = ec;
        } else {
            e[0] = fmaf(nbt, sum_groups(u[0]), ve1);
        }
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, e[0]), ns.e, ns.eo, 0, 0);
        ns.next();
    }
    // delta-rule write: S = S' + k e^T
    write_rows<C>(x, s, e);
    if constexpr (M == Rows::kFullCols) {
        gfloat* colp = cols + t * col_stride + (i0 * kD + j0);
#pragma unroll
        for (int r = 0; r < R; ++r) store_gcols<C, false>(colp + r * kD, s[r]);
    }
}

struct NoKeys {
    __device__ void operator()() const {}
};

// T rows of one phase.  The whole-head tiling (several waves per SIMD hide
// each other's latency) reads each row's keys when it starts it; at one chain
// per CU it runs one wave per SIMD, where reading them a row ahead measured 2%
// faster but needs 170 VGPRs.  The narrow tilings run one or two waves per
// SIMD, so each row's key reads are issued during the previous row (two
// register sets, used in turn: no copies between them).
template <int R, int C, Rows M, bool PLAIN, int TM>
__device__ __forceinline__ void run_rows(const Stage<R, TM>& L, float (&s)[R][C], int T,
                                         float* o, float* e_out, size_t o0, size_t ostride,
                                         int ig, int i0, int j0, gfloat* cols = nullptr,
                                         size_t col_stride = 0) {
    static_assert(R == 16, "a quad covers 16 keys");
    constexpr bool DPP = C < 4;
    constexpr bool Q = has_q(M);
    const int n = threadIdx.x & 3;
    if constexpr (!PLAIN) {
        // the key group again from an opaque copy of the thread index: held
        // from the launch's start instead, it spilled in one variant
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63;
        ig = ((lane >> 4) & 3) | ((lane >> 1) & 4);
        i0 = ig * R;
    }
    if constexpr (!DPP) {
        NarrowStores none;   // the whole-head tiling stores through its own path
#pragma unroll 1
        for (int t = 0; t < T; ++t) {
            RowKeys<DPP> x;   // a stash row reads its keys itself from LDS, four at a time
            if constexpr (M != Rows::kStash || DPP) x.template read<R, Q, TM>(L, t, i0, n);
            row_step<R, C, M, PLAIN, TM, false>(L, x, s, t, o, e_out, o0, ostride, ig, i0, j0,
                                                cols, col_stride, NoKeys{}, none);
        }
    } else {
        // The next row's keys go out at the start of each row, after that
        // row's own reads, unconditionally (the compiler then counts them
        // exactly instead of waiting on them at once): after the last row the
        // read lands in the stage's spare row.
        if (T <= 0) return;
        // o from the lanes with (lane & 0x38) == 0x10 (C = 1) or (lane & 0x28)
        // == 0x20 (C = 2), e from those where the same bits are 0.  The
        // launcher keeps T * H * 512 bytes under 2^31.
        NarrowStores ns;
        {
            const int lane = threadIdx.x & 63;
            constexpr int kMask = C == 2 ? 0x28 : 0x38, kOdd = C == 2 ? 0x20 : 0x10;
            constexpr uint32_t kOut = 0x80000000u;
            const uint32_t col4 = static_cast<uint32_t>(j0 + (C == 2 ? ((lane >> 4) & 1) : 0)) * 4;
            ns.o = __builtin_amdgcn_make_buffer_rsrc(o ? o + o0 : nullptr, 0, o ? kOut : 0, kBufferWords3);
            ns.e = __builtin_amdgcn_make_buffer_rsrc(e_out ? e_out + o0 : nullptr, 0, e_out ? kOut : 0,
                                                     kBufferWords3);
            ns.oo = col4 | ((lane & kMask) == kOdd ? 0u : kOut);
            ns.eo = col4 | ((lane & kMask) == 0 ? 0u : kOut);
            ns.step = static_cast<uint32_t>(ostride * 4);
        }
        RowKeys<true> xa, xb;
        xa.template read<R, Q, TM>(L, 0, i0, n);
#pragma unroll 1
        for (int t = 0; t < T; t += 2) {
            row_step<R, C, M, PLAIN, TM, true>(L, xa, s, t, o, e_out, o0, ostride, ig, i0, j0,
                                               cols, col_stride, [&] {
                xb.template read<R, Q, TM>(L, t + 1, i0, n);
            }, ns);
            if (t + 1 >= T) break;
            row_step<R, C, M, PLAIN, TM, true>(L, xb, s, t + 1, o, e_out, o0, ostride, ig, i0,
                                               j0, cols, col_stride, [&] {
                xa.template read<R, Q, TM>(L, t + 2, i0, n);   // t + 2 <= T
            }, ns);
        }
    }
}

// One launch: optionally a replay phase A (FUSED: the kept rows of up to
// kMaxPrev earlier rounds, oldest first, from the snapshot, then -- when
// a.s_out is set -- that committed state is stored), then phase B (this
// launch's rows).  Without FUSED the state after phase B is stored.
template <int R, int C, bool BF16, Rows MA, Rows MB, bool TABLE, bool DUAL>
__device__ __forceinline__ void scan_chain(const ScanArgs& a, Stage<R, TABLE ? 1 : kTMax>* Ls,
                                           size_t chain, int blk) {
    using TL = Tile<R, C>;
    constexpr bool FUSED = MA != Rows::kNone;
    static_assert(!DUAL || FUSED, "two stage areas serve the fused round only");
    auto& L = Ls[0];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    // the swap layout serves the launches whose time is VALU-bound: the
    // whole-head verify scan and fused round (batched and state-column
    // launches measured faster with the plain layout)
    constexpr bool PLAIN = plain_layout<C, MB, TABLE>();
    const int ig = PLAIN ? (lane & 7) : (((lane >> 4) & 3) | ((lane >> 1) & 4));
    const int jg = PLAIN ? (lane >> 3) : (lane & 7);
    const int i0 = ig * R;
    // --- this workgroup: column block blk of chain `chain`
    const int j0 = blk * TL::BCOLS + wave * TL::WCOLS + jg * C;
    // this lane's element offset inside a head's state; the per-head base
    // pointers are wave-uniform, so addresses are SGPR base + 32-bit offset
    const uint32_t lane_off = static_cast<uint32_t>(i0 * kD + j0);

    const gfloat* st_in;
    gfloat* st_out;
    Src b;   // this launch's rows
    size_t o0, ostride;
    b.q = a.q; b.k = a.k; b.v = a.v; b.g = a.g; b.beta = a.beta; b.e = a.e_in;
    if constexpr (TABLE) {
        const size_t lb = chain / a.H, h = chain % a.H;
        // the table entry is wave-uniform: keep it in scalar registers
        const uint64_t raw = reinterpret_cast<const uint64_t*>(a.s_ptrs)[lb];
        const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(raw)));
        const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(raw >> 32)));
        gfloat* p = reinterpret_cast<gfloat*>(lo | (hi << 32)) + h * kDD;
        st_in = p;
        st_out = p;
        b.row0 = chain * kD; b.rstride = 0;
        b.b0 = chain; b.bstride = 0;
        b.T = 1;
        o0 = chain * kD; ostride = 0;
    } else {
        const size_t l = chain / a.H, h = chain % a.H;
        st_in = (const gfloat*)a.s_in + chain * kDD;
        st_out = (gfloat*)a.s_out + chain * kDD;
        b.row0 = (l * a.T_stride * a.H + h) * kD; b.rstride = static_cast<size_t>(a.H) * kD;
        b.b0 = l * a.T_stride * a.H + h;           b.bstride = a.H;
        b.T = a.T;
        o0 = (l * a.T * a.H + h) * kD;              ostride = static_cast<size_t>(a.H) * kD;
    }

    // the state streams (see load_gcols), except in the state-column arm,
    // whose 2 GB of column writes measured faster through the caches
    constexpr bool kNT = MB != Rows::kFullCols;
    float s[R][C];
    auto load_state = [&] {
#pragma unroll
        for (int r = 0; r < R; ++r) load_gcols<C, kNT>(st_in + (lane_off + r * kD), s[r]);
    };
    auto store_state = [&] {
        if constexpr (TABLE) {
            // rows past the 4 KiB immediate-offset range get one shared base
            // pair: left to itself the compiler builds a 64-bit address per
            // row there, and those pairs spill
            constexpr int kNear = 4096 / (kD * 4);
            gfloat* near = st_out + lane_off;
            gfloat* far = near + kNear * kD;
            asm volatile("" : "+v"(far));
#pragma unroll
            for (int r = 0; r < R; ++r)
                store_gcols<C, kNT>(r < kNear ? near + r * kD : far + (r - kNear) * kD, s[r]);
        } else {
#pragma unroll
            for (int r = 0; r < R; ++r) store_gcols<C, kNT>(st_out + (lane_off + r * kD), s[r]);
        }
    };

    // an earlier round's kept rows (fused round), in that round's layout
    auto prev_src = [&](int i) {
        const PrevRows& pr = a.prev[i];
        const size_t l = chain / a.H, h = chain % a.H;
        Src p;
        p.q = nullptr; p.k = pr.k; p.v = pr.v; p.g = pr.g; p.beta = pr.beta; p.e = pr.e;
        p.row0 = (l * pr.T * a.H + h) * kD; p.rstride = static_cast<size_t>(a.H) * kD;
        p.b0 = l * pr.T * a.H + h;           p.bstride = a.H;
        p.T = pr.keep;
        if (i == 0 && a.keep_j != nullptr)   // device-side keep (wave-uniform scalar load)
            p.T = static_cast<int>(min(*a.keep_j, static_cast<uint32_t>(pr.T - 1))) + 1;
        return p;
    };

    if constexpr (DUAL) {
        // at most one earlier round (the launcher's rule)
        auto& LB = Ls[DUAL ? 1 : 0];
        Staged<R, C, MA, kTMax> inA;
        Staged<R, C, MB, kTMax> inB;
        const bool replay = a.n_prev > 0;
        Src p;
        if (replay) {
            p = prev_src(0);
            stage_issue<R, C, BF16, MA, kTMax>(inA, p, tid);
        }
        stage_issue<R, C, BF16, MB, kTMax>(inB, b, tid);
        load_state();
        if (replay) stage_fence<R, C, MA, kTMax>(inA);
        stage_fence<R, C, MB, kTMax>(inB);
        // both phases' rows go to LDS while the state is still arriving, so
        // the scan follows the replay and the snapshot store directly
        // two LDS areas: one barrier after both
        if (replay) stage_commit<R, C, MA, kTMax, false>(L, inA, p.T, tid);
        stage_commit<R, C, MB, kTMax>(LB, inB, b.T, tid);
        // the state has arrived during the commits: one wait for all of it
        // here, instead of a wait per state row that the row loop would issue
        // again on every pass (vmcnt 0; expcnt and lgkmcnt left at their
        // maxima; no stores are in flight yet)
        __builtin_amdgcn_s_waitcnt(kWaitVmem);
        if (replay) run_rows<R, C, MA, PLAIN>(L, s, p.T, nullptr, nullptr, 0, 0, ig, i0, j0);
        if (a.s_out) store_state();   // the committed state: this round's snapshot
        run_rows<R, C, MB, PLAIN>(LB, s, b.T, a.o, a.e_out, o0, ostride, ig, i0, j0);
        return;
    } else if constexpr (FUSED) {
        // With at most one stash replay, this launch's row loads go out
        // before the replay (the stash replay leaves registers for them) and
        // are waited on before the snapshot's stores are issued: a wait after
        // those stores would wait for them to complete as well.
        constexpr bool kEarlyRows = MA == Rows::kStash;
        if (a.n_prev == 0 || (kEarlyRows && a.n_prev == 1)) {
            Staged<R, C, MB, kTMax> inB;
            if (kEarlyRows && a.n_prev == 1) {
                const Src p0 = prev_src(0);
                Staged<R, C, MA, kTMax> inA;
                stage_issue<R, C, BF16, MA, kTMax>(inA, p0, tid);
                load_state();
                stage_fence<R, C, MA, kTMax>(inA);
                stage_commit<R, C, MA, kTMax>(L, inA, p0.T, tid);
                // narrow tilings: one wait for the state (see the dual stage)
                if constexpr (C < 4) __builtin_amdgcn_s_waitcnt(kWaitVmem);
                stage_issue<R, C, BF16, MB, kTMax>(inB, b, tid);
                asm volatile("" ::: "memory");   // keep those loads ahead of the replay
                run_rows<R, C, MA, PLAIN>(L, s, p0.T, nullptr, nullptr, 0, 0, ig, i0, j0);
            } else {
                stage_issue<R, C, BF16, MB, kTMax>(inB, b, tid);
                load_state();
            }
            stage_fence<R, C, MB, kTMax>(inB);
            if (a.s_out) store_state();   // the committed state: this round's snapshot
            __syncthreads();   // every wave is done with the replayed rows
            stage_commit<R, C, MB, kTMax>(L, inB, b.T, tid);
        } else {
            const Src p0 = prev_src(0);
            stage<R, C, BF16, MA>(L, p0, tid, load_state);
            if constexpr (C < 4) __builtin_amdgcn_s_waitcnt(kWaitVmem);
            run_rows<R, C, MA, PLAIN>(L, s, p0.T, nullptr, nullptr, 0, 0, ig, i0, j0);
            __syncthreads();   // every wave is done with these staged rows
            for (int i = 1; i < a.n_prev; ++i) {
                const Src pi = prev_src(i);
                stage<R, C, BF16, MA>(L, pi, tid, [] {});
                run_rows<R, C, MA, PLAIN>(L, s, pi.T, nullptr, nullptr, 0, 0, ig, i0, j0);
                __syncthreads();
            }
            if (a.s_out) store_state();   // the committed state: this round's snapshot
            stage<R, C, BF16, MB>(L, b, tid, [] {});
        }
    } else {
        // the batched arm always scans one row per session
        stage<R, C, BF16, MB, TABLE ? 1 : kTMax>(L, b, tid, load_state);
    }
    if constexpr (MB == Rows::kFullCols) {
        // the last column is the state after all rows: no separate store
        static_assert(!FUSED && !TABLE, "state columns serve the plain scan");
        run_rows<R, C, MB, PLAIN>(L, s, b.T, a.o, a.e_out, o0, ostride, ig, i0, j0,
                           (gfloat*)a.s_cols + chain * kDD, a.col_stride);
        return;
    }
    run_rows<R, C, MB, PLAIN>(L, s, b.T, a.o, TABLE ? nullptr : a.e_out, o0, ostride, ig, i0, j0);
    if constexpr (!FUSED) store_state();
}

// The B workgroups that split one head (C < 4) each read all of that head's
// row inputs.  The hardware hands workgroup i to XCD i mod 8, each XCD with
// its own L2, so the parts of a head get indices equal mod 8 (where the
// range allows): index i -> head (i / 8 / B) * 8 + i mod 8, part (i / 8) mod B.
// One XCD's L2 then serves the repeated row reads.  Any count of XCDs gives
// a correct mapping; 8 is MI355X's.
template <int B>
__device__ __forceinline__ void split_index(unsigned long long i, unsigned long long n,
                                            unsigned long long& head, int& part) {
    constexpr unsigned long long kXcd = 8, kGroup = kXcd * B;
    if (B > 1 && i < n - n % kGroup) {
        const unsigned long long k = i / kXcd;
        head = (k / B) * kXcd + i % kXcd;
        part = static_cast<int>(k % B);
    } else {
        head = i / B;
        part = static_cast<int>(i % B);
    }
}

// DUAL: phase A and phase B rows each get an LDS area, so both are loaded up
// front (one memory round trip fewer per launch, twice the LDS).
// TAILC (0, 1 or 2): the chains past a.n_head_chains -- the last, sparse fill
// of the chip -- run with TAILC value columns per lane, so over 4 or 2
// workgroups each (the same bits); that fill then spreads over the CUs and
// ends sooner.
template <int R, int C, bool BF16, Rows MA, Rows MB, bool TABLE, bool DUAL, int TAILC>
__global__ void __launch_bounds__((Tile<R, C>::THREADS))
__attribute__((amdgpu_waves_per_eu(DUAL ? 2 : 4)))   // DUAL: LDS allows 2 workgroups per CU
kda_scan_kernel(ScanArgs a) {
    using TL = Tile<R, C>;
    // the batched arm stages its one row: 2.4 KB of LDS instead of 38.5 KB
    __shared__ Stage<R, TABLE ? 1 : kTMax> Ls[DUAL ? 2 : 1];
    unsigned long long head_blocks = gridDim.x;
    if constexpr (TAILC != 0) {
        static_assert(C == 4 && !DUAL && !TABLE, "a split tail follows whole heads");
        head_blocks = static_cast<unsigned long long>(a.n_head_chains) * TL::BLOCKS;
        if (blockIdx.x >= head_blocks) {
            // head_blocks is a multiple of the CU count (256 on MI355X), so
            // there the tail index and the workgroup index agree mod 8
            constexpr int kSplit = Tile<R, TAILC>::BLOCKS;
            unsigned long long head;
            int part;
            split_index<kSplit>(blockIdx.x - head_blocks, gridDim.x - head_blocks, head, part);
            scan_chain<R, TAILC, BF16, MA, MB, TABLE, DUAL>(
                a, Ls, static_cast<size_t>(a.n_head_chains + head), part);
            return;
        }
    }
    unsigned long long bid = blockIdx.x;
    if constexpr (TABLE) {
        // the heads of one table entry stay together; the entries run in a
        // permuted order, so the workgroups in flight touch entries far apart
        // even when the caller's session buffers are one contiguous block
        static_assert(TL::BLOCKS == 1, "the batched arm runs whole heads");
        const unsigned long long h = static_cast<unsigned long long>(a.H);
        const unsigned long long entries = static_cast<unsigned long long>(a.n_chains) / h;
        bid = (bid / h) * a.entry_mul % entries * h + bid % h;
    }
    unsigned long long head;
    int part;
    split_index<TL::BLOCKS>(bid, head_blocks, head, part);
    scan_chain<R, C, BF16, MA, MB, TABLE, DUAL>(a, Ls, static_cast<size_t>(head), part);
}

// ------------------------------------------------------------------ copy

// Plain vector copy: each workgroup copies one contiguous 16 KiB chunk, 4
// float4 per thread 4 KiB apart.  On a 136 MiB state this measured 6.7 TB/s,
// against 6.2 TB/s for a grid-stride loop over the whole buffer.
__global__ void __launch_bounds__(256) kda_copy_kernel(const float4* __restrict__ src,
                                                       float4* __restrict__ dst, size_t n4) {
    const size_t base = static_cast<size_t>(blockIdx.x) * 1024 + threadIdx.x;
    if (base + 768 < n4) {
        const float4 a0 = src[base];
        const float4 a1 = src[base + 256];
        const float4 a2 = src[base + 512];
        const float4 a3 = src[base + 768];
        dst[base] = a0;
        dst[base + 256] = a1;
        dst[base + 512] = a2;
        dst[base + 768] = a3;
    } else {
        for (size_t i = base; i < n4 && i < base + 1024 - threadIdx.x; i += 256) dst[i] = src[i];
    }
}

// ------------------------------------------------------------------ conv ring

// The committed short-conv ring after `keep` accepted rows.  The ring holds
// the last 3 raw conv inputs (kernel size 4); rolling it once per kept row
// over the round's raw rows leaves, in output row m, entry keep + m of the
// sequence (ring rows 0..2, raw rows 0..T-1) -- memra-engine 0.123.0
// glm_spec.rs, module doc VERIFY-ROW BATCHING: ring snapshot plus re-roll at
// T = keep over the stolen raw rows.  Pure data movement: one thread moves
// four channels of all three output rows.
constexpr int kRerollThreads = 256;
constexpr int kRerollChans = kRerollThreads * 4;   // channels per workgroup

template <bool BF16, bool VEC>
__global__ void __launch_bounds__(kRerollThreads) kda_reroll_kernel(RerollArgs a) {
    const long long l = blockIdx.x / a.blocks_per_layer;
    const long long c = (blockIdx.x % a.blocks_per_layer) * kRerollChans +
                        static_cast<long long>(threadIdx.x) * 4;
    if (c >= a.C) return;
    const int keep = a.keep_j != nullptr
                         ? static_cast<int>(min(*a.keep_j, static_cast<uint32_t>(a.T - 1))) + 1
                         : a.keep;
#pragma unroll
    for (int m = 0; m < kRingRows; ++m) {
        const int sidx = keep + m;
        float4 x;
        if (sidx < kRingRows) {
            const float* src = a.ring_snap + (l * kRingRows + sidx) * a.C;
            if constexpr (VEC) {
                x = *reinterpret_cast<const float4*>(src + c);
            } else {
                x.x = src[c];
                x.y = c + 1 < a.C ? src[c + 1] : 0.f;
                x.z = c + 2 < a.C ? src[c + 2] : 0.f;
                x.w = c + 3 < a.C ? src[c + 3] : 0.f;
            }
        } else {
            const size_t off = static_cast<size_t>((l * a.T + (sidx - kRingRows)) * a.C + c);
            if constexpr (VEC) {
                x = load4<BF16>(a.raw, off);
            } else {
                x.x = load1<BF16>(a.raw, off);
                x.y = c + 1 < a.C ? load1<BF16>(a.raw, off + 1) : 0.f;
                x.z = c + 2 < a.C ? load1<BF16>(a.raw, off + 2) : 0.f;
                x.w = c + 3 < a.C ? load1<BF16>(a.raw, off + 3) : 0.f;
            }
        }
        float* dst = a.ring_out + (l * kRingRows + m) * a.C;
        if constexpr (VEC) {
            *reinterpret_cast<float4*>(dst + c) = x;
        } else {
            dst[c] = x.x;
            if (c + 1 < a.C) dst[c + 1] = x.y;
            if (c + 2 < a.C) dst[c + 2] = x.z;
            if (c + 3 < a.C) dst[c + 3] = x.w;
        }
    }
}

// ------------------------------------------------------------------ pre-scan row ops

// The per-row ops that turn one layer's projections into scan inputs for the
// t = K+1 verify rows (memra-engine 0.123.0 glm_spec.rs, module doc
// VERIFY-ROW BATCHING: gates and conv batched over the rows;
// glm5_spec_ppn_gate.rs fixture: short conv kernel 4, gate bound -5):
//   q, k, v : causal depthwise conv over (3 ring rows, the round's rows),
//             taps w[c][0..3] oldest first, then SiLU; q and k L2-normalised
//             per (row, head) with 1e-6 under the square root;
//   g       : max(-softplus(a), -5);     beta : sigmoid(b).
// Given the raw rows, every row's conv window x_{t-3..t} is known, so rows
// are independent: one workgroup of 128 lanes per (layer, head, 3 rows), a
// lane per head channel (q, k, v and g of that channel), the window's 6 raw
// or ring rows loaded once and every load issued before any arithmetic.
// Neighbouring row groups of a (layer, head) share 3 window rows; the
// blockIdx -> work mapping keeps them on one XCD (the dispatcher deals
// workgroups round-robin over the 8 XCDs), so those re-reads hit that XCD's
// L2.  The workgroup holding row T-1 also writes the ring after the round:
// the last three entries of the sequence.
constexpr int kOpsThreads = kD;   // 2 waves
constexpr int kXcds = 8;
constexpr float kNormEps = 1e-6f;

__device__ __forceinline__ float exp_f(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float rcp_f(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float silu_f(float y) { return y * rcp_f(1.0f + exp_f(-y)); }
__device__ __forceinline__ float softplus_f(float a) {
    // max(a, 0) + ln(1 + e^-|a|), the log on the hardware log2
    return fmaxf(a, 0.0f) + __builtin_amdgcn_logf(1.0f + exp_f(-fabsf(a))) * 0.69314718055994531f;
}

// Rows per workgroup: 3 measured fastest (28-29 us for 34 layers x 64 heads
// x 15 rows in f32, 35 us in bf16), against 29-30 and 30-34 us for 2, 4, 5
// or 8 rows, and 34-37 / 48-53 us for one row per workgroup.
constexpr int kRowsPerGroup = 3;

template <bool BF16>
__global__ void __launch_bounds__(kOpsThreads) kda_row_ops_kernel(RowOpsArgs a) {
    const int j = threadIdx.x;
    const int wave = j >> 6;
    const long long nwork = a.nwork;
    const long long per_xcd = (nwork + kXcds - 1) / kXcds;
    const long long bid = blockIdx.x;
    const long long work = (bid % kXcds) * per_xcd + bid / kXcds;
    if (work >= nwork) return;
    const int T = a.T;
    const int chunks = (T + kRowsPerGroup - 1) / kRowsPerGroup;
    const long long lh = work / chunks;
    const int r0 = static_cast<int>(work % chunks) * kRowsPerGroup;
    const int nr = min(kRowsPerGroup, T - r0);
    const long long l = lh / a.H;
    const long long h = lh % a.H;
    const long long HD = static_cast<long long>(a.H) * kD;
    const long long C = 3 * HD;
    const long long c0 = h * kD + j;

    // the conv window of these rows: sequence entries r0 .. r0 + kRowsPerGroup
    // + 2, where entries 0..2 are the ring rows and entry 3 + r is raw row r;
    // loads are unconditional, rows past T clamped
    float xw[3][kRowsPerGroup + kRingRows];
#pragma unroll
    for (int m = 0; m < kRowsPerGroup + kRingRows; ++m) {
        const int e = r0 + m;
#pragma unroll
        for (int blk = 0; blk < 3; ++blk) {
            if (e < kRingRows) {
                xw[blk][m] = a.ring_in[(l * kRingRows + e) * C + c0 + blk * HD];
            } else {
                const int rr = min(e - kRingRows, T - 1);
                xw[blk][m] = load1<BF16>(a.x, static_cast<size_t>((l * T + rr) * C + c0 + blk * HD));
            }
        }
    }
    float xa[kRowsPerGroup];
#pragma unroll
    for (int i = 0; i < kRowsPerGroup; ++i) {
        const int rr = min(r0 + i, T - 1);
        xa[i] = load1<BF16>(a.a, static_cast<size_t>((l * T + rr) * HD + c0));
    }
    float4 w[3];
#pragma unroll
    for (int blk = 0; blk < 3; ++blk)
        w[blk] = *reinterpret_cast<const float4*>(a.w + (l * C + c0 + blk * HD) * 4);
    float bt = 0.0f;
    if (j < nr) bt = load1<BF16>(a.b, static_cast<size_t>((l * T + r0 + j) * a.H + h));

    __shared__ float part[kRowsPerGroup][2][2];
    float yq[kRowsPerGroup], yk[kRowsPerGroup];
#pragma unroll
    for (int i = 0; i < kRowsPerGroup; ++i) {
        if (i < nr) {
            float y[3];
#pragma unroll
            for (int blk = 0; blk < 3; ++blk) {
                float acc = w[blk].x * xw[blk][i];
                acc = fmaf(w[blk].y, xw[blk][i + 1], acc);
                acc = fmaf(w[blk].z, xw[blk][i + 2], acc);
                acc = fmaf(w[blk].w, xw[blk][i + 3], acc);
                y[blk] = silu_f(acc);
            }
            const size_t o = static_cast<size_t>(((l * T + r0 + i) * a.H + h) * kD + j);
            a.v[o] = y[2];
            a.g[o] = fmaxf(-softplus_f(xa[i]), kGateLo);
            yq[i] = y[0];
            yk[i] = y[1];
            float sq = y[0] * y[0];
            float sk = y[1] * y[1];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                sq += __shfl_xor(sq, off);
                sk += __shfl_xor(sk, off);
            }
            if ((j & 63) == 0) {
                part[i][wave][0] = sq;
                part[i][wave][1] = sk;
            }
        }
    }
    if (j < nr) a.beta[(l * T + r0 + j) * a.H + h] = rcp_f(1.0f + exp_f(-bt));
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kRowsPerGroup; ++i) {
        if (i < nr) {
            const size_t o = static_cast<size_t>(((l * T + r0 + i) * a.H + h) * kD + j);
            a.q[o] = yq[i] * __builtin_amdgcn_rsqf(part[i][0][0] + part[i][1][0] + kNormEps);
            a.k[o] = yk[i] * __builtin_amdgcn_rsqf(part[i][0][1] + part[i][1][1] + kNormEps);
        }
    }
    if (a.ring_out && r0 + nr == T) {
        // entries T, T+1, T+2: the ring after all T rows (local index T - r0 + m)
#pragma unroll
        for (int m = 0; m < kRingRows; ++m)
#pragma unroll
            for (int blk = 0; blk < 3; ++blk) {
                float x = xw[blk][m];
#pragma unroll
                for (int n = 1; n <= kRowsPerGroup; ++n)
                    if (n == nr) x = xw[blk][m + n];
                a.ring_out[(l * kRingRows + m) * C + c0 + blk * HD] = x;
            }
    }
}

// ------------------------------------------------------------------ batched copy

// n copies of `words` floats, driven by a device table [src_0..src_{n-1},
// dst_0..dst_{n-1}] (memra-engine 0.98.0 dflash.rs, DsparkSnapBatch and its
// uniform batched f32 copy: one table refresh and one launch instead of a
// copy per layer of the GDN state snapshot).
// blockIdx.y picks the buffer pair; its pointers are wave-uniform, so the
// choice between 16-byte and 4-byte moves is made per pair at run time.
__global__ void __launch_bounds__(256) kda_copy_batch_kernel(const uint64_t* table, int n,
                                                             long long words) {
    const int b = blockIdx.y;
    const uint64_t s_raw = table[b];
    const uint64_t d_raw = table[n + b];
    const uint64_t s_lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(s_raw)));
    const uint64_t s_hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(s_raw >> 32)));
    const uint64_t d_lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(d_raw)));
    const uint64_t d_hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(d_raw >> 32)));
    const uint64_t sp = s_lo | (s_hi << 32);
    const uint64_t dp = d_lo | (d_hi << 32);
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (((sp | dp) & 15) == 0 && (words & 3) == 0) {
        const float4* s4 = reinterpret_cast<const float4*>(sp);
        float4* d4 = reinterpret_cast<float4*>(dp);
        const size_t n4 = static_cast<size_t>(words) / 4;
        for (; i + 3 * stride < n4; i += 4 * stride) {
            const float4 a0 = s4[i];
            const float4 a1 = s4[i + stride];
            const float4 a2 = s4[i + 2 * stride];
            const float4 a3 = s4[i + 3 * stride];
            d4[i] = a0;
            d4[i + stride] = a1;
            d4[i + 2 * stride] = a2;
            d4[i + 3 * stride] = a3;
        }
        for (; i < n4; i += stride) d4[i] = s4[i];
    } else {
        const float* src = reinterpret_cast<const float*>(sp);
        float* dst = reinterpret_cast<float*>(dp);
        for (; i < static_cast<size_t>(words); i += stride) dst[i] = src[i];
    }
}

// ------------------------------------------------------------------ greedy accept

// Per verify row, the argmax of its logits -- the lowest index among equal
// maxima, or kNoToken if the row holds a NaN -- then the greedy accept: j is
// the number of leading drafts equal to the argmaxes of their rows, and the
// bonus token is the argmax of row j (memra-engine 0.123.0 glm_spec.rs,
// glm5_spec_round step 4, the greedy branch: device argmaxes with the host
// argmax's tie-break, then the longest matching prefix).
//
// Two launches.  The first splits row r over P workgroups (blockIdx.y = r),
// each reducing its chunks to a (value, index, nan) partial; all of a row's
// loads are in flight at once, which is what an HBM-latency-bound read of a
// few MB needs.  The second, one workgroup with a wave per row, folds each
// row's P partials, then walks the drafts with one ballot.  The kernel
// boundary orders the two, so no atomics or fences are involved, and the
// lowest index of the maximum is unique, so the order partials meet in does
// not change the result.
constexpr int kArgThreads = 256;
constexpr int kArgChunk = kArgThreads * 16;   // elements per workgroup step

struct ArgBest {
    float v;
    uint32_t i;
    uint32_t nan;
};

__device__ __forceinline__ void take(ArgBest& b, float x, uint32_t i) {
    b.nan |= x != x ? 1u : 0u;
    if (x > b.v || (x == b.v && i < b.i)) {
        b.v = x;
        b.i = i;
    }
}

__device__ __forceinline__ void merge(ArgBest& b, const ArgBest& o) {
    b.nan |= o.nan;
    if (o.v > b.v || (o.v == b.v && o.i < b.i)) {
        b.v = o.v;
        b.i = o.i;
    }
}

__device__ __forceinline__ ArgBest wave_best(ArgBest b) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        ArgBest o;
        o.v = __shfl_xor(b.v, off);
        o.i = static_cast<uint32_t>(__shfl_xor(static_cast<int>(b.i), off));
        o.nan = static_cast<uint32_t>(__shfl_xor(static_cast<int>(b.nan), off));
        merge(b, o);
    }
    return b;
}

template <bool BF16, bool VEC>
__global__ void __launch_bounds__(kArgThreads) kda_argmax_part_kernel(AcceptArgs a) {
    const int tid = threadIdx.x;
    const int r = blockIdx.y;
    const int p = blockIdx.x;
    const int P = gridDim.x;
    const uint32_t n = static_cast<uint32_t>(a.V);
    const void* row = static_cast<const char*>(a.logits) +
                      static_cast<long long>(r) * a.ld * (BF16 ? 2 : 4);

    ArgBest b{-__builtin_inff(), kNoToken, 0u};
    for (uint32_t c0 = static_cast<uint32_t>(p) * kArgChunk; c0 < n;
         c0 += static_cast<uint32_t>(P) * kArgChunk) {
        if constexpr (VEC) {
            // four 4-element groups per lane, all issued before any compare
            float4 x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t i = c0 + (u * kArgThreads + tid) * 4;
                x[u] = i + 4 <= n ? load4<BF16>(row, i) : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t i = c0 + (u * kArgThreads + tid) * 4;
                if (i + 4 <= n) {
                    take(b, x[u].x, i);
                    take(b, x[u].y, i + 1);
                    take(b, x[u].z, i + 2);
                    take(b, x[u].w, i + 3);
                } else {
                    for (uint32_t m = i; m < n && m < i + 4; ++m) take(b, load1<BF16>(row, m), m);
                }
            }
        } else {
            float x[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const uint32_t i = c0 + u * kArgThreads + tid;
                x[u] = i < n ? load1<BF16>(row, i) : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const uint32_t i = c0 + u * kArgThreads + tid;
                if (i < n) take(b, x[u], i);
            }
        }
    }

    b = wave_best(b);
    __shared__ ArgBest wb[kArgThreads / 64];
    if ((tid & 63) == 0) wb[tid >> 6] = b;
    __syncthreads();
    if (tid == 0) {
#pragma unroll
        for (int w = 1; w < kArgThreads / 64; ++w) merge(b, wb[w]);
        const int slot = r * kAcceptPMax + p;
        a.pv[slot] = b.v;
        a.pi[slot] = b.i;
        a.pn[slot] = b.nan;
    }
}

// One workgroup of t waves: wave r folds row r's P partials into vam[r];
// then wave 0 finds the first draft that misses (a ballot) and the bonus.
__global__ void __launch_bounds__(64 * kTMax) kda_accept_finish_kernel(AcceptArgs a, int P) {
    const int lane = threadIdx.x & 63;
    const int r = threadIdx.x >> 6;
    __shared__ uint32_t vs[kTMax];
    ArgBest f{-__builtin_inff(), kNoToken, 0u};
    if (lane < P) {
        const int slot = r * kAcceptPMax + lane;
        f.v = a.pv[slot];
        f.i = a.pi[slot];
        f.nan = a.pn[slot];
    }
    f = wave_best(f);
    if (lane == 0) {
        const uint32_t v = f.nan ? kNoToken : f.i;
        a.vam[r] = v;
        vs[r] = v;
    }
    __syncthreads();
    if (r == 0) {
        const uint32_t v = lane < a.t ? vs[lane] : 0u;
        const bool miss = lane >= a.t - 1 || a.drafts[lane] != v;
        const int j = __builtin_ctzll(__ballot(miss));   // lane t-1 always misses
        const uint32_t bonus = static_cast<uint32_t>(__shfl(static_cast<int>(v), j));
        if (lane == 0) {
            a.out2[0] = static_cast<uint32_t>(j);
            a.out2[1] = bonus;
        }
    }
}

// Fused rounds of at most this many workgroups take two stage areas (about
// 74 KB of LDS each, so two workgroups per CU): they fit in one pass.
constexpr unsigned long long kDualStageMaxBlocks = 512;

// CUs of the current device, read once per device (a process may drive
// devices of different sizes, e.g. partitions); 256 if it cannot be read.  It
// picks tilings only: every tiling gives the same bits.
int chip_cus() {
    constexpr int kCached = 64;
    static std::atomic<int> cache[kCached];   // 0: not read yet
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < kCached) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    if (dev < kCached) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// a.n_head_chains chains with CH value columns per lane, then `tail` chains
// split TAILC-wide (2 or 4 workgroups each), in one launch
template <int CH, int TAILC, bool BF16, Rows MA, Rows MB>
hipError_t launch_split_tail(const ScanArgs& a, long long tail, hipStream_t stream) {
    using TL = Tile<kKeysPerLane, CH>;
    const unsigned long long tb = static_cast<unsigned long long>(a.n_head_chains) * TL::BLOCKS +
                                  static_cast<unsigned long long>(tail) *
                                      Tile<kKeysPerLane, TAILC>::BLOCKS;
    if (tb > 0x7FFFFFFFull) return hipErrorInvalidValue;
    kda_scan_kernel<kKeysPerLane, CH, BF16, MA, MB, false, false, TAILC>
        <<<dim3(static_cast<unsigned>(tb)), dim3(TL::THREADS), 0, stream>>>(a);
    return hipGetLastError();
}

// The batched arm's entry order: a multiplier coprime to the entry count n,
// near n / 7.  With one contiguous session block in [L][B] order, the plain
// order keeps the ~16 entries in flight in one contiguous 64 MiB span, and a
// step measured 790-800 us against 720-730 us with the entries spread
// (separately allocated sessions ran 705-710 us either way).
unsigned long long entry_mul_for(unsigned long long n) {
    unsigned long long m = n / 7;
    if (m < 1) m = 1;
    for (;;) {
        unsigned long long x = m, y = n;
        while (y) { const unsigned long long t = x % y; x = y; y = t; }
        if (x == 1) return m;
        ++m;
    }
}

template <int C, bool BF16, Rows MA, Rows MB, bool TABLE>
hipError_t launch_tiled(const ScanArgs& a0, hipStream_t stream) {
    using TL = Tile<kKeysPerLane, C>;
    ScanArgs a = a0;
    if constexpr (TABLE) a.entry_mul = entry_mul_for(static_cast<unsigned long long>(a.n_chains / a.H));
    const unsigned long long blocks = static_cast<unsigned long long>(a.n_chains) * TL::BLOCKS;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(blocks));
    if constexpr (MA != Rows::kNone && C != 4) {
        if (blocks <= kDualStageMaxBlocks && a.n_prev <= 1) {
            kda_scan_kernel<kKeysPerLane, C, BF16, MA, MB, TABLE, true, 0>
                <<<grid, dim3(TL::THREADS), 0, stream>>>(a);
            return hipGetLastError();
        }
    }
    if constexpr (C == 4 && !TABLE) {
        // a split tail stores o and e at 32-bit offsets from a chain's first
        // row (the narrow launches, at most one chain per CU, always fit)
        const bool narrow_ok = static_cast<unsigned long long>(a.T) * a.H * kD * 4 < (1ull << 31);
        const long long cus = chip_cus();
        const long long slots = 4 * cus;
        if (a.n_chains <= slots) {
            // up to one fill: whole rounds of one chain per CU, then a tail
            // of at most CUs/4 chains split 4 ways (a 2-way split of a larger
            // tail measured slower than whole heads: 384 chains 24.9 vs 24.1 us)
            const long long tail = a.n_chains % cus;
            if (narrow_ok && a.n_chains > cus && tail > 0 && tail <= cus / 4) {
                a.n_head_chains = a.n_chains - tail;
                return launch_split_tail<4, 1, BF16, MA, MB>(a, tail, stream);
            }
        } else {
            // several fills of 4 whole heads per CU (128 VGPRs, 4 waves per
            // SIMD): a sparse last fill splits 4 ways up to CUs/4 chains, 2
            // ways up to CUs/2, so that it has about one workgroup per CU
            const long long tail = a.n_chains % slots;
            if (narrow_ok && tail > 0 && tail <= cus / 2) {
                a.n_head_chains = a.n_chains - tail;
                return tail <= cus / 4 ? launch_split_tail<4, 1, BF16, MA, MB>(a, tail, stream)
                                       : launch_split_tail<4, 2, BF16, MA, MB>(a, tail, stream);
            }
        }
    }
    kda_scan_kernel<kKeysPerLane, C, BF16, MA, MB, TABLE, false, 0>
        <<<grid, dim3(TL::THREADS), 0, stream>>>(a);
    return hipGetLastError();
}

// The tiling by chain count n: up to CUs/2 chains a head splits over 4
// workgroups (C = 1), up to CUs over 2 (C = 2) -- at most 2 workgroups per CU
// either way -- and past that whole heads (C = 4), whose last partial round
// of one chain per CU splits 4 ways when it is at most CUs/4 chains.  Against
// half heads up to 512 chains and quarter heads up to 256, in one process:
// 240 chains 22.8 -> 18.3 us, 272 (the TP = 8 share) 23.7 -> 20.9, 384 27.7 ->
// 23.9, 448 31.5 -> 25.1, 544 35.6 -> 31.9; 128, 256, 640 and 768 unchanged.
// Half heads lose once every CU has a chain: their DPP key operands cost
// about 1.2x, and whole heads hide latency with 4 columns per lane.

template <bool BF16, Rows MA, Rows MB, bool TABLE>
hipError_t launch_one(const ScanArgs& a, hipStream_t stream) {
    if constexpr (!TABLE) {
        const long long cus = chip_cus();
        if (a.n_chains <= cus / 2) return launch_tiled<1, BF16, MA, MB, TABLE>(a, stream);
        if (a.n_chains <= cus) return launch_tiled<2, BF16, MA, MB, TABLE>(a, stream);
    }
    return launch_tiled<4, BF16, MA, MB, TABLE>(a, stream);
}

template <bool BF16>
hipError_t launch_dtype(const ScanArgs& a, Launch kind, hipStream_t stream) {
    switch (kind) {
        case Launch::kScanOut:      return launch_one<BF16, Rows::kNone, Rows::kFull, false>(a, stream);
        case Launch::kScanState:    return launch_one<BF16, Rows::kNone, Rows::kState, false>(a, stream);
        case Launch::kReplay:       return launch_one<BF16, Rows::kNone, Rows::kState, false>(a, stream);
        case Launch::kReplayStash:  return launch_one<BF16, Rows::kNone, Rows::kStash, false>(a, stream);
        case Launch::kBatchedOut:   return launch_one<BF16, Rows::kNone, Rows::kFull, true>(a, stream);
        case Launch::kBatchedState: return launch_one<BF16, Rows::kNone, Rows::kState, true>(a, stream);
        case Launch::kRound:        return launch_one<BF16, Rows::kState, Rows::kFull, false>(a, stream);
        case Launch::kRoundStash:   return launch_one<BF16, Rows::kStash, Rows::kFull, false>(a, stream);
        case Launch::kScanColumns:  return launch_one<BF16, Rows::kNone, Rows::kFullCols, false>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_scan(const ScanArgs& a, Launch kind, bool bf16, hipStream_t stream) {
    return bf16 ? launch_dtype<true>(a, kind, stream) : launch_dtype<false>(a, kind, stream);
}

// ------------------------------------------------------------------ accept scratch, no allocation
//
// The greedy accept's partial argmaxes for callers that cannot allocate: one
// file-scope device array per GPU, sized for the largest table any call needs
// (kTMax rows x kAcceptPMax partials, 11.25 KiB).  Its device address is
// looked up once per device with that device current and kept; host code
// passes that address to the kernels, never the array's name, which on the
// host is only a stand-in.  Every call on one device shares the array, so
// calls that overlap on a device race.  Nothing in it needs clearing: a call
// reads only the slots it has written.
static __device__ __align__(256) AcceptScratch scratch;

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
AcceptScratch* g_scratch[kScratchDevices];
}  // namespace

hipError_t accept_static_scratch(AcceptScratch** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = static_cast<AcceptScratch*>(p);
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

int accept_workgroups_per_row(int V) {
    const int chunks = (V + kArgChunk - 1) / kArgChunk;
    return chunks < kAcceptPMax ? chunks : kAcceptPMax;
}

hipError_t launch_accept(const AcceptArgs& a, bool bf16, hipStream_t stream) {
    const int es = bf16 ? 2 : 4;
    // whole 4-element groups are aligned loads when every row starts aligned
    const bool vec = reinterpret_cast<uintptr_t>(a.logits) % (4 * es) == 0 &&
                     (a.t == 1 || a.ld % 4 == 0);
    const int P = accept_workgroups_per_row(a.V);
    const dim3 grid(P, a.t);
    const dim3 block(kArgThreads);
    if (bf16) {
        if (vec)
            kda_argmax_part_kernel<true, true><<<grid, block, 0, stream>>>(a);
        else
            kda_argmax_part_kernel<true, false><<<grid, block, 0, stream>>>(a);
    } else {
        if (vec)
            kda_argmax_part_kernel<false, true><<<grid, block, 0, stream>>>(a);
        else
            kda_argmax_part_kernel<false, false><<<grid, block, 0, stream>>>(a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    kda_accept_finish_kernel<<<dim3(1), dim3(64 * a.t), 0, stream>>>(a, P);
    return hipGetLastError();
}

hipError_t launch_reroll(const RerollArgs& a0, bool bf16, hipStream_t stream) {
    RerollArgs a = a0;
    a.blocks_per_layer = (a.C + kRerollChans - 1) / kRerollChans;
    const unsigned long long blocks = static_cast<unsigned long long>(a.L) * a.blocks_per_layer;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
    const int es = bf16 ? 2 : 4;
    const bool vec = a.C % 4 == 0 && reinterpret_cast<uintptr_t>(a.ring_snap) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(a.ring_out) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(a.raw) % (4 * es) == 0;
    const dim3 grid(static_cast<unsigned>(blocks));
    if (bf16) {
        if (vec) kda_reroll_kernel<true, true><<<grid, kRerollThreads, 0, stream>>>(a);
        else kda_reroll_kernel<true, false><<<grid, kRerollThreads, 0, stream>>>(a);
    } else {
        if (vec) kda_reroll_kernel<false, true><<<grid, kRerollThreads, 0, stream>>>(a);
        else kda_reroll_kernel<false, false><<<grid, kRerollThreads, 0, stream>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_row_ops(const RowOpsArgs& a0, bool bf16, hipStream_t stream) {
    RowOpsArgs a = a0;
    a.nwork = static_cast<long long>(a.L) * a.H * ((a.T + kRowsPerGroup - 1) / kRowsPerGroup);
    const long long per_xcd = (a.nwork + kXcds - 1) / kXcds;
    const unsigned long long blocks = static_cast<unsigned long long>(per_xcd) * kXcds;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
    if (bf16)
        kda_row_ops_kernel<true><<<dim3(static_cast<unsigned>(blocks)), kOpsThreads, 0, stream>>>(a);
    else
        kda_row_ops_kernel<false><<<dim3(static_cast<unsigned>(blocks)), kOpsThreads, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_copy_batch(const uint64_t* table, int n, long long words, hipStream_t stream) {
    // about 16 KiB per workgroup per pass, at most 1024 workgroups per buffer
    const long long per = (words + 4095) / 4096;
    const unsigned gx = static_cast<unsigned>(per < 1 ? 1 : (per > 1024 ? 1024 : per));
    kda_copy_batch_kernel<<<dim3(gx, n), 256, 0, stream>>>(table, n, words);
    return hipGetLastError();
}

hipError_t launch_copy(const float* src, float* dst, size_t n_floats, hipStream_t stream) {
    const size_t n4 = n_floats / 4;   // n_floats is a multiple of 128*128
    size_t blocks = (n4 + 1023) / 1024;
    if (blocks < 1) blocks = 1;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
    kda_copy_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(
        reinterpret_cast<const float4*>(src), reinterpret_cast<float4*>(dst), n4);
    return hipGetLastError();
}

}  // namespace kda
