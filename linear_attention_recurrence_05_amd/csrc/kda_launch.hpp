// kda_launch.hpp -- host-side launchers shared between the C ABI (kda_api.hip)
// and the kernel files.  Arguments reaching these functions have already been
// validated by the ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace kda {

struct DecodeArgs {
    const void *q, *k, *v, *z;
    const float *beta, *A;
    float g_min;
    float* S;
    void* o;
    int B, H, d;
    bool is_bf16;
};

struct PrefillArgs {
    const void *q, *k, *v, *z;
    const float *beta, *A;
    float g_min;
    const float* S0;
    void* o;
    float* S_T;
    int B, T, H, d;
    bool is_bf16;
};

// How a prefill is executed.
enum class Plan {
    kFused,   // gate + intra + inter in one launch; one workgroup per (b, h, column tile)
    kSplit,   // intra kernel over all chunks -> workspace, then inter kernel
};

struct PlanInfo {
    Plan plan;
    int ncol;            // value columns per inter/fused workgroup
    int nb;              // split plan: 16-column blocks per state chain
    size_t ws_bytes;     // workspace needed
};

// Chosen execution plan for these sizes (pure function of the sizes).
PlanInfo choose_plan(int B, int T, int H, int d, bool is_bf16);
// Bytes of one chunk's factor block.
size_t factor_block_bytes(int d, bool is_bf16);

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, const PlanInfo& p, void* ws, hipStream_t stream);
hipError_t launch_gate_cumsum(const void* z, const float* A, float g_min, float* G, int B, int T,
                              int H, int d, bool is_bf16, hipStream_t stream);
hipError_t launch_intra_diag(const void* q, const void* k, const void* z, const float* beta,
                             const float* A, float g_min, float* Tm, float* Aqk, float* gamma,
                             int B, int T, int H, int d, bool is_bf16, hipStream_t stream);

}  // namespace kda
