// Internal interface between the C-ABI layer (kda_abi.cpp) and the gfx950
// kernels (kda_kernels.hip).  Not installed; callers use include/kda.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

namespace kda {

constexpr int kD = 128;        // head dim: d_k = d_v
constexpr int kTMax = 15;      // verify rows per launch
constexpr int kBMax = 15;      // batched-decode sessions

// One launch of the row scan.  Either the contiguous layout
//   state [chain][128][128], chain = l*H + h, rows [L][T_stride][H][128]
// or (table) the batched layout
//   state s_ptrs[l*B + b] + h*128*128, chain = (l*B + b)*H + h, rows [L][B][H][128].
struct ScanArgs {
    const float* s_in;
    float* s_out;
    float* const* s_ptrs;
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    float* o;        // written only when write_o
    long long n_chains;  // (layer, head) or (layer, session, head) chains
    int H;
    int T;           // rows scanned by this launch
    int T_stride;    // rows per layer in the input layout (contiguous mode)
};

hipError_t launch_scan(const ScanArgs& a, bool bf16, bool write_o, bool table, hipStream_t stream);

hipError_t launch_copy(const float* src, float* dst, size_t n_floats, hipStream_t stream);

}  // namespace kda
