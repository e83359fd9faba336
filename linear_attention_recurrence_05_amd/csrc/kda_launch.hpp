// kda_launch.hpp -- host-side launchers shared between the C ABI (kda_api.hip)
// and the kernel files.  Arguments reaching these functions have already been
// validated by the ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace kda {

// The states a launch reads and writes, for unit (b, h) of d x d fp32:
//   in  + (row_in(b) * H + h) * d * d,   out + (row_out(b) * H + h) * d * d,
// with row(b) = b when the slot table is null (dense [B, H, d, d]) and
// slot[b] otherwise (a pool of n_slots states).  A null in means zeros, a
// null out means no state written.  The caller's own slot tables (ck_in,
// ck_out) decide which sequences run: one whose slot lies outside
// [0, n_slots) is skipped -- no output row and no state is written for it.
// (A launch in the middle of a segmented prefill reads and writes a carry
// whose table differs from the caller's, hence the separate check tables.)
struct StateIO {
    const float* in;
    const int* in_slot;
    float* out;
    const int* out_slot;
    const int* ck_in;
    const int* ck_out;
    int n_slots;

    __device__ bool skip(int b) const {
        return (ck_in && (unsigned)ck_in[b] >= (unsigned)n_slots) ||
               (ck_out && (unsigned)ck_out[b] >= (unsigned)n_slots);
    }
    __device__ const float* in_at(int b, int h, int H, int d) const {
        return in ? in + ((size_t)(in_slot ? in_slot[b] : b) * H + h) * (size_t)d * d : nullptr;
    }
    __device__ float* out_at(int b, int h, int H, int d) const {
        return out ? out + ((size_t)(out_slot ? out_slot[b] : b) * H + h) * (size_t)d * d : nullptr;
    }
};

// Dense states (no slot tables).
inline StateIO dense_state(const float* in, float* out) {
    return StateIO{in, nullptr, out, nullptr, nullptr, nullptr, 0};
}

// Where a checkpointing pass stores the state entering every chunk: for the
// pass's row b' (= b R + r: segment r of sequence b when R segments run side
// by side) and head h, chunk n' of the row is chunk r NCs + n' of the
// sequence, whose state goes to base + ((b H + h) NC + r NCs + n') D D in
// the natural [D][D] layout; NC = R NCs chunks per sequence.
struct CkOut {
    float* base;
    int R, NC;
    template <int D>
    __device__ float* at(int bp, int h, int n, int H) const {
        const int b = bp / R, r = bp % R;
        return base + (((size_t)b * H + h) * NC + (size_t)r * (NC / R) + n) * (size_t)D * D;
    }
};

struct DecodeArgs {
    const void *q, *k, *v, *z;
    const float *beta, *A;
    float g_min;
    StateIO S;          // read and written in place (in == out)
    void* o;
    int B, H, d;
    bool is_bf16;
};

struct TokensArgs {
    const void *q, *k, *v, *z;
    const float *beta, *A;
    float g_min;
    StateIO S;          // the state before the tokens (in), after them (out)
    void* o;
    int B, T, H, d;
    bool is_bf16;
};

// Per-unit chunk counts of a fused-plan pass (unit u = b H + h of the pass):
// `in` (may be null) limits unit u to its first in[u] chunks; `out` (may be
// null; only state-only passes with v = 0 take it) makes the pass stop once
// the unit's state is exactly zero, and receives in out[u] the number of
// chunks it processed.
struct ChunkLim {
    const int* in;
    int* out;
};

struct PrefillArgs {
    const void *q, *k, *v, *z;
    const float *beta, *A;
    float g_min;
    StateIO S;          // S0 (in, may be null) and S_T (out, may be null)
    void* o;
    int B, T, H, d;
    bool is_bf16;
    ChunkLim lim{};     // fused plan only
};

// Gradients of a prefill: inputs of the forward call plus dO (and dST, may be
// null: zeros); outputs dq, dk, dv, dz (element type of the inputs), dbeta,
// dA (fp32) and dS0 (fp32, may be null: not written).
struct BackwardArgs {
    const void *q, *k, *v, *z;
    const float *beta, *A;
    float g_min;
    const float* S0;
    const void* dO;
    const float* dST;
    void *dq, *dk, *dv, *dz;
    float *dbeta, *dA, *dS0;
    int B, T, H, d;
    bool is_bf16;
};

// Backward geometry: value columns per workgroup, tokens per finalize block,
// and the bound on the per-segment partial sums in the workspace.
constexpr int kBwdCols = 8;
constexpr int kBwdTokBlock = 16;
constexpr size_t kBwdPartialBudget = (size_t)256 << 20;
// Threads of a chunk-level chain workgroup (16 value columns of one head).
constexpr int kBwdChainThreads = 512;
// Recompute window (tokens) of the chunk-parallel reverse sweep.
constexpr int kBwdHistPar = 4;
// Fewest tokens of one reverse-sweep launch (a multiple of kBwdTokBlock).
constexpr int kBwdSegTokensMin = 128;
// Shortest segment of a segment-parallel forward sweep in the backward.
constexpr int kBwdSegMin = 256;

// Byte offsets of the backward workspace regions (each 256-byte aligned).
struct BwdLayout {
    size_t ckpt, carry, ucor, pq, pk, pg, pb, dA_part, segws, oscr, Gc, Tm, Aqk, gam, dSend, fac,
        total;
    int R;       // segments of the forward sweep run side by side (1: one sweep)
    bool chain;  // reverse sweep by the chunk-level chain, chunks in parallel
    bool chunk;  // the chunkwise MFMA plan (kda_bwd_chunk.hip)
    int seg;     // tokens per reverse-sweep launch (multiple of kBwdTokBlock)
    int NC;      // chunks (checkpoints) per sequence
    int ntb;     // finalize token blocks per sequence
};
BwdLayout bwd_layout(int B, int T, int H, int d, bool is_bf16);
bool bwd_plan_chain(int T);
bool bwd_plan_chunk(int d, bool is_bf16);
// The chunkwise MFMA backward (bf16, d = 128): whether it applies, the bytes
// of one chunk's chain operand block, and its launches after the forward
// checkpoints (ckpt: bwd_ckpt_kernel's layout); fac, dSend and dA_part are
// workspace regions of units * NC blocks, states and floats.
bool bwd_chunk_ok(int d, bool is_bf16);
size_t bwd_chunk_fac_bytes();
hipError_t launch_bwd_chunk(const BackwardArgs& a, const float* ckpt, char* fac, float* dSend,
                            float* dA_part, hipStream_t stream);

// How a prefill is executed.
enum class Plan {
    kFused,   // gate + intra + inter in one launch; one workgroup per (b, h, column tile)
    kSplit,   // intra kernel over all chunk pairs -> workspace, then inter kernel
    kRing,    // pair producers and state chains in one launch, pairs passed through L2
};

struct PlanInfo {
    Plan plan;
    int ncol;            // value columns per inter/fused workgroup
    int nb;              // split plan: 16-column blocks per state chain
    size_t ws_bytes;     // workspace needed
};

// Chunks per split-plan segment (even, so no pair of chunks straddles two
// segments): the workspace holds this many chunks' factors per head; longer
// sequences run as consecutive segments carrying the state.
constexpr int kSegChunks = 1024;
static_assert(kSegChunks % 2 == 0, "segments hold whole pairs of chunks");

// Chosen execution plan for these sizes (pure function of the sizes).
PlanInfo choose_plan(int B, int T, int H, int d, bool is_bf16);
// Whether launch_prefill runs this plan as a state-only pass: a null o (no
// outputs; q is not read) and optionally a null v (v taken as zero).
bool prefill_state_only_ok(const PlanInfo& p, int d);
// A state-only pass of the fused kernel (bf16, d = 128, 128 columns per
// workgroup) over a.B rows of a.T tokens from a.S.in that stores the state
// entering every chunk into ck (a.o, a.v unused beyond v's reads).
hipError_t launch_ckpt_pass(const PrefillArgs& a, const CkOut& ck, hipStream_t stream);
// Bytes of one two-chunk factor block of the split plan.
size_t pair_block_bytes(int d, bool is_bf16);
// Whether the split plan compiles an inter kernel with ncol value columns per
// workgroup and nb 16-column blocks per state chain.
bool pair_variant_ok(int d, bool is_bf16, int ncol, int nb);

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_tokens(const TokensArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, const PlanInfo& p, void* ws, hipStream_t stream);
// Split plan: pair intra kernel -> workspace -> pair inter kernel, per segment.
hipError_t launch_split(const PrefillArgs& a, const PlanInfo& p, void* ws, hipStream_t stream);
// Ring plan (bf16, d = 128, at most one workgroup per CU: B * H * 8 <= CUs
// rounded to whole XCD groups): whether it runs on the current device, its
// workspace (flags and an L2-resident ring of pair blocks per unit), and the
// launch (a flag fill, then the ring kernel).  Needs o and v; no chunk limits.
bool ring_ok(int B, int H, int d, bool is_bf16);
size_t ring_ws_bytes(int B, int H, int d, bool is_bf16);
hipError_t launch_ring(const PrefillArgs& a, void* ws, hipStream_t stream);
hipError_t launch_backward(const BackwardArgs& a, void* ws, hipStream_t stream);

// Segment-scan prefill: the T tokens of each sequence as R segments of T / R
// (laid side by side as B * R batch rows), the state map of each segment,
// a scan over segments, and a last pass from the scanned start states.
struct SegLayout {
    PlanInfo inner;        // plan of the inner prefill calls (B * R rows of T / R)
    size_t inner_ws, vzero, ident, M, N, Sin, nch, total;   // byte offsets, 256-aligned
};
SegLayout seg_layout(int B, int T, int H, int d, bool is_bf16, int R);
// a.S: dense S0 (in, may be null) and S_T (out, may be null).
hipError_t launch_segmented(const PrefillArgs& a, int R, void* ws, hipStream_t stream);
// Segments the dense prefill entry point uses by itself for these sizes (1:
// none, the direct plan).
int auto_segments(int B, int T, int H, int d, bool is_bf16);
// The scan alone: the start state of every segment into the layout's Sin
// region ([B * R, H, d, d]) and S_T into a.S.out (if set); a.o is scratch.
hipError_t seg_start_states(const PrefillArgs& a, int R, const SegLayout& L, char* ws,
                            hipStream_t stream);
hipError_t launch_gate_cumsum(const void* z, const float* A, float g_min, float* G, int B, int T,
                              int H, int d, bool is_bf16, hipStream_t stream);
hipError_t launch_intra_diag(const void* q, const void* k, const void* z, const float* beta,
                             const float* A, float g_min, float* Tm, float* Aqk, float* gamma,
                             int B, int T, int H, int d, bool is_bf16, hipStream_t stream);

}  // namespace kda
