// kda_segscan.hip -- prefill of long sequences by a scan over segments: the
// one-GPU share of the pages' KDA context parallelism (dev.to "Kimi K3
// Architecture ...", section "Infrastructure and Training/Inference
// Mechanics": local state updates merged by a prefix scan over fixed-size
// states, exchanged by all-gathers).
//
// The state update is affine in the state: over a segment r of the sequence,
// S_end = M_r S_in + N_r, where M_r (d_k x d_k) is the product of the
// segment's (I - beta k k^T) Diag(a) factors and N_r the end state reached
// from zero.  Both come out of the ordinary chunkwise prefill, with the
// segments of every sequence laid side by side as batch rows (a contiguous
// [B, T, H, d] tensor is a [B * R, T / R, H, d] tensor):
//   M_r = prefill(q, k, v = 0, z, beta; S0 = I).S_T   (d_v = d_k columns of I)
//   N_r = prefill(q, k, v,     z, beta; S0 = 0).S_T
// A scan then gives every segment's start state,
//   S_in(0) = S0,   S_in(r + 1) = M_r S_in(r) + N_r,   S_T = S_in(R),
// and a last prefill of all segments from their start states writes o.  On
// P GPUs each would hold one segment and all-gather the (M_r, N_r) pairs;
// here the segments share one GPU, so the path costs three passes over the
// tokens plus the scan (the two map passes state-only where the plan has
// such passes: no q, no outputs, and no v for M_r), and its use on one GPU
// is more parallel work per launch (B * R * H units instead of B * H) for
// sequences whose own chains are too few to fill the chip.
#include <cstdlib>
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

// Zero n 16-byte words (a kernel rather than a memset, so that the call can be
// captured into a graph).
__global__ __launch_bounds__(256) void zero16_kernel(u32x4* __restrict__ p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        p[i] = u32x4{0u, 0u, 0u, 0u};
}

// n_states identity matrices of d x d fp32.
__global__ __launch_bounds__(256) void identity_kernel(float* __restrict__ p, size_t n_states,
                                                       int d) {
    const size_t per = (size_t)d * d, n = n_states * per;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
        const size_t e = i % per;
        p[i] = (e / d == e % d) ? 1.0f : 0.0f;
    }
}

// Start states of the two map passes with the segments of every sequence as
// rows b R + r ([B R, H, d, d] each): the M_r pass from the identity, except
// segment 0, whose map is taken as zero (it starts from the known S0); the
// other pass from zero, except segment 0, which starts from S0 (null: zero),
// so that its end state is already S_in(1).
__global__ __launch_bounds__(256) void seg_fill_kernel(float* __restrict__ ident,
                                                       float* __restrict__ nstart,
                                                       const float* __restrict__ S0, int B, int R,
                                                       int H, int d) {
    const size_t per = (size_t)d * d, n = (size_t)B * R * H * per;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
        const size_t st = i / per, e = i % per;
        const size_t row = st / H, h = st % H;
        const size_t b = row / R;
        const bool first = row % R == 0;
        ident[i] = (!first && e / d == e % d) ? 1.0f : 0.0f;
        nstart[i] = (first && S0) ? S0[(b * H + h) * per + e] : 0.0f;
    }
}

// Scan over the R segments of each (b, h), one workgroup per 16 value
// columns: S <- M_r S + N_r, with M_r staged in LDS and M_{r+1} loaded into
// registers while step r computes.  Writes S_in(r) of every segment to
// Sin[(b R + r), h] and the end state to S_T[b, h] (if given).  Reads S0
// (null: zeros) before any write, and only its own columns, so S_T may alias
// S0.  nch (may be null): chunks the map pass of unit (b R + r) H + h ran
// before its map was exactly zero; fewer than ncs (the segment's chunks)
// means M_r = 0, and the step is S <- N_r without reading M_r.
template <int D>
__global__ __launch_bounds__(256) void segscan_kernel(const float* __restrict__ M,
                                                      const float* __restrict__ Nst,
                                                      const float* S0, float* __restrict__ Sin,
                                                      float* S_T, int H, int R,
                                                      const int* __restrict__ nch, int ncs) {
    constexpr int CB = 16;                  // value columns per workgroup
    constexpr int OPT = D * CB / 256;       // outputs per thread
    constexpr int MPT = D * D / 256;        // elements of M per thread
    __shared__ float Ms[D][D + 1];
    __shared__ float Ss[D][CB];
    const int tid = (int)threadIdx.x;
    const int nct = D / CB;
    const int ct = (int)(blockIdx.x % nct);
    const size_t bh = blockIdx.x / nct;
    const size_t b = bh / H, h = bh % H;
    const int i = tid % D, j0 = (tid / D) * OPT;
    const size_t col0 = (size_t)ct * CB;
    auto state = [&](const float* base, size_t row) { return base + (row * H + h) * (size_t)D * D; };
    // S_in(0) = S0
    for (int e = tid; e < D * CB; e += 256) {
        const int c = e / CB, j = e % CB;
        Ss[c][j] = S0 ? S0[(bh * D + c) * D + col0 + j] : 0.0f;
    }
    // whether M_r is known to be zero (uniform over the workgroup)
    auto zero_map = [&](int r) { return nch && nch[(b * R + r) * H + h] < ncs; };
    float mreg[MPT];
    if (!zero_map(0)) {
        const float* m = state(M, b * R);
#pragma unroll
        for (int x = 0; x < MPT; ++x) mreg[x] = m[tid + 256 * x];
    }
    __syncthreads();
    for (int r = 0; r < R; ++r) {
        const size_t row = b * R + r;
        float* sin = const_cast<float*>(state(Sin, row));
        for (int e = tid; e < D * CB; e += 256) {
            const int c = e / CB, j = e % CB;
            sin[(size_t)c * D + col0 + j] = Ss[c][j];
        }
        const bool zr = zero_map(r);
        if (!zr) {
#pragma unroll
            for (int x = 0; x < MPT; ++x) {
                const int e = tid + 256 * x;
                Ms[e / D][e % D] = mreg[x];
            }
        }
        __syncthreads();
        if (r + 1 < R && !zero_map(r + 1)) {   // the next map, in flight while this step computes
            const float* m = state(M, row + 1);
#pragma unroll
            for (int x = 0; x < MPT; ++x) mreg[x] = m[tid + 256 * x];
        }
        const float* nr = state(Nst, row);
        float acc[OPT];
#pragma unroll
        for (int x = 0; x < OPT; ++x) acc[x] = nr[(size_t)i * D + col0 + j0 + x];
        if (!zr) {
            for (int c = 0; c < D; ++c) {
                const float mic = Ms[i][c];
#pragma unroll
                for (int x = 0; x < OPT; ++x) acc[x] += mic * Ss[c][j0 + x];
            }
        }
        __syncthreads();   // every thread has read Ss and Ms
#pragma unroll
        for (int x = 0; x < OPT; ++x) Ss[i][j0 + x] = acc[x];
        __syncthreads();
    }
    if (S_T)
        for (int e = tid; e < D * CB; e += 256) {
            const int c = e / CB, j = e % CB;
            S_T[(bh * D + c) * D + col0 + j] = Ss[c][j];
        }
}

static size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Segments kda_chunk_prefill splits a sequence into by itself.  A head's state
// chain runs its chunks one after another, so B * H heads of a long sequence
// keep only B * H * d / 16 chains busy; with 32 or fewer heads and bf16
// inputs at d = 128 the segment scan (R segments as B * R * H >= 128 units of
// the fused plan, whose map passes are state-only) was measured faster from
// 65,536 tokens on: 1.12-1.20x at B * H = 32 (R = 8), 1.26-1.70x at 16
// (R = 16), and slower at 64 heads or below 4,096 tokens per segment.  A
// plan forced by KDA_PREFILL_PLAN runs as forced (1: no segments).
int auto_segments(int B, int T, int H, int d, bool is_bf16) {
    if (std::getenv("KDA_PREFILL_PLAN")) return 1;
    if (!is_bf16 || d != 128 || T < 65536) return 1;
    const long units = (long)B * H;
    if (units > 32) return 1;
    int R = 1;
    while (units * R * 2 <= 256) R *= 2;
    while (R > 1 && (T % (kChunk * R) != 0 || T / R < 4096)) R /= 2;
    return units * R >= 128 ? R : 1;
}

SegLayout seg_layout(int B, int T, int H, int d, bool is_bf16, int R) {
    SegLayout L;
    const int Ts = T / R;
    L.inner = choose_plan(B * R, Ts, H, d, is_bf16);
    const size_t es = is_bf16 ? 2 : 4;
    const size_t states = (size_t)B * R * H * d * d * sizeof(float);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = round_up(off + bytes, 256);
        return o;
    };
    L.inner_ws = take(L.inner.ws_bytes);
    L.vzero = prefill_state_only_ok(L.inner, d) ? off : take((size_t)B * T * H * d * es);
    L.ident = take(states);
    L.M = take(states);
    L.N = take(states);
    L.Sin = take(states);
    L.nch = take((size_t)B * R * H * sizeof(int));
    L.total = off;
    return L;
}

// Fused inner plan (bf16 or fp32 at d = 128, state-only passes):
//   M_r: from the identity (zero for segment 0) with v = 0, stopping once the
//        map is exactly zero -- it only contracts, and for fast-decaying
//        gates it vanishes within a few chunks -- and recording how many
//        chunks that took (nch: the segment's first nch chunks depend on its
//        start state; the later ones do not);
//   N_r: from zero (segment 0 from S0), with the outputs when with_o;
//   the scan.
// Other plans: M_r and N_r in full, as ordinary prefills with a zero v.
static hipError_t start_states(const PrefillArgs& a, int R, const SegLayout& L, char* w,
                               bool with_o, hipStream_t stream) {
    void* inner = L.inner.ws_bytes ? (void*)(w + L.inner_ws) : nullptr;
    float* ident = (float*)(w + L.ident);
    float* M = (float*)(w + L.M);
    float* N = (float*)(w + L.N);
    float* Sin = (float*)(w + L.Sin);
    const int Bs = a.B * R, Ts = a.T / R;
    const size_t n_states = (size_t)Bs * a.H;
    const bool state_only = prefill_state_only_ok(L.inner, a.d);
    hipError_t e;
    const float* s_in0 = a.S.in;
    if (state_only) {
        hipLaunchKernelGGL(seg_fill_kernel, dim3(2048), dim3(256), 0, stream, ident, N, a.S.in, a.B,
                           R, a.H, a.d);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        PrefillArgs pm{a.q, a.k, nullptr, a.z, a.beta, a.A, a.g_min, dense_state(ident, M), nullptr,
                       Bs, Ts, a.H, a.d, a.is_bf16, ChunkLim{nullptr, (int*)(w + L.nch)}};
        if ((e = launch_prefill(pm, L.inner, inner, stream)) != hipSuccess) return e;
        PrefillArgs pn{a.q, a.k, a.v, a.z, a.beta, a.A, a.g_min, dense_state(N, N),
                       with_o ? a.o : nullptr, Bs, Ts, a.H, a.d, a.is_bf16};
        if ((e = launch_prefill(pn, L.inner, inner, stream)) != hipSuccess) return e;
    } else {
        // v has d (a multiple of 32) elements per token-head: whole 16-byte words
        const size_t vwords = (size_t)a.B * a.T * a.H * a.d * (a.is_bf16 ? 2 : 4) / 16;
        size_t zblocks = (vwords + 255) / 256;
        if (zblocks > 16384) zblocks = 16384;
        hipLaunchKernelGGL(zero16_kernel, dim3((unsigned)zblocks), dim3(256), 0, stream,
                           (u32x4*)(w + L.vzero), vwords);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(identity_kernel, dim3(2048), dim3(256), 0, stream, ident, n_states, a.d);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        // M_r: v = 0 from the identity; N_r: v from zero; o is scratch.
        PrefillArgs pm{a.q, a.k, (const void*)(w + L.vzero), a.z, a.beta, a.A, a.g_min,
                       dense_state(ident, M), a.o, Bs, Ts, a.H, a.d, a.is_bf16};
        if ((e = launch_prefill(pm, L.inner, inner, stream)) != hipSuccess) return e;
        PrefillArgs pn{a.q, a.k, a.v, a.z, a.beta, a.A, a.g_min, dense_state(nullptr, N), a.o,
                       Bs, Ts, a.H, a.d, a.is_bf16};
        if ((e = launch_prefill(pn, L.inner, inner, stream)) != hipSuccess) return e;
    }
    const unsigned grid = (unsigned)((size_t)a.B * a.H * (a.d / 16));
    const int* nch = state_only ? (const int*)(w + L.nch) : nullptr;
    const int ncs = (Ts + kChunk - 1) / kChunk;
    if (a.d == 128)
        hipLaunchKernelGGL(segscan_kernel<128>, dim3(grid), dim3(256), 0, stream, M, N, s_in0, Sin,
                           a.S.out, a.H, R, nch, ncs);
    else
        hipLaunchKernelGGL(segscan_kernel<32>, dim3(grid), dim3(256), 0, stream, M, N, s_in0, Sin,
                           a.S.out, a.H, R, nch, ncs);
    return hipGetLastError();
}

hipError_t seg_start_states(const PrefillArgs& a, int R, const SegLayout& L, char* w,
                            hipStream_t stream) {
    return start_states(a, R, L, w, false, stream);
}

// Fused inner plan: the start states with the outputs of every segment from
// its zero start (exact from each segment's nch-th chunk on, and in segment
// 0 throughout), then the first nch chunks of every segment again from its
// scanned start state, overwriting those outputs.  When a map does not
// vanish, nch is the whole segment and this last pass is a full one.  Other
// plans: the start states, then every segment in full from its start state.
hipError_t launch_segmented(const PrefillArgs& a, int R, void* ws, hipStream_t stream) {
    const SegLayout L = seg_layout(a.B, a.T, a.H, a.d, a.is_bf16, R);
    char* w = (char*)ws;
    const bool fast = prefill_state_only_ok(L.inner, a.d);
    hipError_t e = start_states(a, R, L, w, fast, stream);
    if (e != hipSuccess) return e;
    void* inner = L.inner.ws_bytes ? (void*)(w + L.inner_ws) : nullptr;
    PrefillArgs pf{a.q, a.k, a.v, a.z, a.beta, a.A, a.g_min, dense_state((float*)(w + L.Sin), nullptr),
                   a.o, a.B * R, a.T / R, a.H, a.d, a.is_bf16};
    if (fast) pf.lim = ChunkLim{(const int*)(w + L.nch), nullptr};
    return launch_prefill(pf, L.inner, inner, stream);
}

}  // namespace kda
