// kda_backward.hip -- gradients of the KDA prefill: the reverse sweep of the
// recurrence for dq, dk, dv, dz, dbeta, dA and dS0 given dO (and dS_T).
//
// The pages describe no backward pass (the dev.to page "Kimi K3 Architecture
// ...", section "The Sequence Bottleneck", mentions chunkwise parallel
// execution being stable, which training relies on).  What is computed is the
// exact gradient of the forward definition, per (b, h):
//   forward per token:  a = exp(g_min Sigmoid(e^{A_h} z)),  S' = Diag(a) S,
//                       u = v - S'^T k,  S <- S' + beta k u^T,  o = S^T q
//   reverse per token, with dS the gradient of the state after the token:
//     dS += q dO^T;          dq = S dO
//     de = dS^T k;           dk = beta dS u - beta S' de;   dbeta = de . u
//     dv = beta de;          dS' = dS - beta k de^T
//     dg = a rowsum(dS' o S_prev);   dS_prev = Diag(a) dS'
//   and through the gate: dx = dg g_min s (1 - s) with s = Sigmoid(x),
//   x = e^{A_h} z, so dz = e^{A_h} dx and dA_h = sum of dx x.
//
// Design.  The value columns of the state evolve independently (each column
// j of S sees only v_j), so the work splits over (b, h, block of 8 value
// columns) workgroups with no exchange between them; only the row sums over
// columns (dq, dk, dg) and dbeta need the blocks together, and they are
// summed afterwards in a fixed order.  A workgroup is one wave (64 lanes; 32
// for d_k = 32), lane l owning key rows RPT l .. RPT l + RPT - 1 of the 8
// columns in registers (RPT = d_k / 64, or 1), so every reduction over value
// columns stays in the lane and the one over key rows (dS^T k in the
// reverse, S'^T k in the forward) is a wave reduce-scatter by DPP row and
// half-row mirrors and quad permutes, two cross-row swaps and eight
// readlanes: no workgroup barrier and no LDS round trip per token.
//   bwd_ckpt_kernel   forward over the sequence, storing the state slice at
//                     the start of each 16-token chunk and the delta-rule
//                     correction u = v - S'^T k of every token (HBM).  When
//                     the sequence splits into R whole-chunk segments, the
//                     segments run side by side from their start states,
//                     which a segment scan of the chunkwise forward supplies
//                     (kda_segscan.hip).
//   bwd_seg_kernel    per chunk, last to first: recompute the chunk's states
//                     from its checkpoint and the stored u (no reduction),
//                     keeping them in LDS, then sweep the chunk in reverse;
//                     writes dv and per-block partials of dq, dk, dg, dbeta.
//                     Runs over segments of the sequence (last first), the
//                     state gradient carried between launches, so that the
//                     partials occupy a bounded workspace.
//   bwd_finalize_kernel  sums the partials over column blocks, applies the
//                     gate derivative (dz) and forms per-token-block dA terms.
//   bwd_dA_kernel     sums the dA terms of each head in a fixed order.
// Inputs of a chunk are loaded into registers one chunk ahead and parked in
// LDS, so the per-token chain never waits on HBM.  The sweep is a serial
// chain of VALU work per token (no contraction wide enough for MFMA: per
// token a lane does O(16) FMAs per product); it is bounded by latency, with
// HBM traffic for inputs, checkpoints, u and the partials.
#include <cstdlib>
#include <cstring>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <int D>
struct BwdGeom {
    static constexpr int N = kBwdCols;                  // value columns per workgroup
    static constexpr int W = D < kWave ? D : kWave;     // threads: one wave
    static constexpr int RPT = D / W;                   // key rows per thread
    static constexpr int NCB = D / N;                   // column blocks per head
    static_assert(N == 8, "the reduction hands out 8 columns over lanes 0, 2, .., 14");
    static_assert(W >= 16, "the reduction works on whole DPP rows of 16 lanes");
};

// ------------------------------------------------------------------ helpers

// Eight consecutive elements (16-byte aligned for bf16, 32 for fp32) as fp32.
template <typename E>
__device__ __forceinline__ void load8(const E* p, float (&x)[8]);
template <>
__device__ __forceinline__ void load8<bf16>(const bf16* p, float (&x)[8]) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
        x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&x)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = a[i];
        x[4 + i] = b[i];
    }
}

template <typename E>
__device__ __forceinline__ void store8(E* p, const float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = from_f32<E>(x[i]);
}

__device__ __forceinline__ void load8f(const float* p, float (&x)[8]) { load8<float>(p, x); }
__device__ __forceinline__ void store8f(float* p, const float (&x)[8]) {
    *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}

// R consecutive elements of a row-major vector, moved as one access.
template <typename E, int R>
struct alignas(sizeof(E) * R) Rows {
    E x[R];
};

// Value of the lane given by a DPP control inside each row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppRowMirror = 0x140;       // lane i <- lane 15 - i of its row (i ^ 15)
constexpr int kDppRowHalfMirror = 0x141;   // lane i <- lane 7 - i of its half-row (i ^ 7)
constexpr int kDppQuadXor2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int kDppQuadXor1 = 0xB1;         // quad_perm [1, 0, 3, 2]

// Sum over the W lanes of a wave of 8 per-lane values; every lane receives all
// 8 sums (wave-uniform).  Reduce-scatter: each step pairs a lane with one
// holding the same columns, the lane keeps half of them and adds the
// partner's copy of that half.  Partners i ^ 15, i ^ 7, i ^ 2 (bits 3, 2, 1
// select the kept half) cover 8 distinct lanes; i ^ 1 completes the row of
// 16, the cross-row swaps the wave.  Lane 2j then holds the sum of column j
// (j = 4 bit3 + 2 bit2 + bit1), which readlane broadcasts.
template <int W>
__device__ __forceinline__ void wave_sum8(const float (&part)[8], float (&out)[8]) {
    const int lane = (int)threadIdx.x & (W - 1);
    float a[4], b[2];
    const bool u3 = (lane & 8) != 0, u2 = (lane & 4) != 0, u1 = (lane & 2) != 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        a[i] = (u3 ? part[i + 4] : part[i]) + dpp<kDppRowMirror>(u3 ? part[i] : part[i + 4]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
        b[i] = (u2 ? a[i + 2] : a[i]) + dpp<kDppRowHalfMirror>(u2 ? a[i] : a[i + 2]);
    float c = (u1 ? b[1] : b[0]) + dpp<kDppQuadXor2>(u1 ? b[0] : b[1]);
    c += dpp<kDppQuadXor1>(c);
    if constexpr (W > 16) c += __shfl_xor(c, 16, W);
    if constexpr (W > 32) c += __shfl_xor(c, 32, W);
#pragma unroll
    for (int j = 0; j < 8; ++j)
        out[j] = __builtin_bit_cast(float,
                                    __builtin_amdgcn_readlane(__builtin_bit_cast(int, c), 2 * j));
}

// ------------------------------------------------------------------ staging

// One chunk's inputs for one workgroup, loaded into registers a chunk ahead of
// use and parked in LDS at the chunk's start.  Lane l holds its key rows' z,
// k (and q) for the chunk's tokens; lane r < 16 holds token r's 8-column
// slices of the shared vectors (v in the forward; u and dO in the reverse)
// and its beta.  Tokens past T read as zero.
template <typename E, int R, bool REV>
struct Stage {
    Rows<E, R> z[kChunk], k[kChunk], q[REV ? kChunk : 1];
    float x[8], dO[8], beta;
};

// The LDS side: z, k, q are private to their lane (lane l reads back only
// entry l); the shared vectors and beta are double-buffered by chunk parity.
template <typename E, int R, int W, bool REV>
struct StageLds {
    Rows<E, R> z[kChunk][W], k[kChunk][W], q[REV ? kChunk : 1][W];
    float x[2][kChunk][8], dO[2][REV ? kChunk : 1][8], beta[2][kChunk];
};

// x8 points at the shared vector of the chunk's first token for this
// column block (v, or u), with a stride of xstride elements per token.
template <typename E, typename X, int D, bool REV>
__device__ __forceinline__ void stage_load(Stage<E, BwdGeom<D>::RPT, REV>& s,
                                           const E* __restrict__ q, const E* __restrict__ k,
                                           const E* __restrict__ z,
                                           const float* __restrict__ beta,
                                           const E* __restrict__ dO, const X* __restrict__ x8,
                                           size_t xstride, int b, int h, int T, int H, int cb,
                                           int cs) {
    using G = BwdGeom<D>;
    constexpr int R = G::RPT;
    const int l = (int)threadIdx.x;
#pragma unroll
    for (int r = 0; r < kChunk; ++r) {
        const int t = cs + r;
        const size_t i = (((size_t)b * T + t) * H + h) * D + R * l;
        if (t < T) {
            s.z[r] = *reinterpret_cast<const Rows<E, R>*>(z + i);
            s.k[r] = *reinterpret_cast<const Rows<E, R>*>(k + i);
            if constexpr (REV) s.q[r] = *reinterpret_cast<const Rows<E, R>*>(q + i);
        } else {
#pragma unroll
            for (int e = 0; e < R; ++e) {
                s.z[r].x[e] = from_f32<E>(0.f);
                s.k[r].x[e] = from_f32<E>(0.f);
                if constexpr (REV) s.q[r].x[e] = from_f32<E>(0.f);
            }
        }
    }
    if (l < kChunk) {
        const int t = cs + l;
        if (t < T) {
            const size_t row = ((size_t)b * T + t) * H + h;
            load8(x8 + (size_t)l * xstride, s.x);
            if constexpr (REV) load8(dO + row * D + cb * kBwdCols, s.dO);
            s.beta = beta[row];
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) s.x[j] = s.dO[j] = 0.f;
            s.beta = 0.f;
        }
    }
}

template <typename E, int R, int W, bool REV>
__device__ __forceinline__ void stage_store(const Stage<E, R, REV>& s, StageLds<E, R, W, REV>& L,
                                            int buf) {
    const int l = (int)threadIdx.x;
#pragma unroll
    for (int r = 0; r < kChunk; ++r) {
        L.z[r][l] = s.z[r];
        L.k[r][l] = s.k[r];
        if constexpr (REV) L.q[r][l] = s.q[r];
    }
    if (l < kChunk) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            L.x[buf][l][j] = s.x[j];
            if constexpr (REV) L.dO[buf][l][j] = s.dO[j];
        }
        L.beta[buf][l] = s.beta;
    }
}

// ------------------------------------------------------------------ kernels

// Forward over the whole sequence.  The state slice of each chunk's start
// goes to ckpt[(u * NCB + cb) * NC + n] (D x 8 floats, row-major), the
// correction u of token t to ucor[((u * NCB + cb) * T + t) * 8].
template <typename E, int D>
__global__ __launch_bounds__(BwdGeom<D>::W) void bwd_ckpt_kernel(
    const E* __restrict__ k, const E* __restrict__ v, const E* __restrict__ z,
    const float* __restrict__ beta, const float* __restrict__ A, float g_min,
    const float* __restrict__ S0, const float* __restrict__ Sseg, int nseg,
    float* __restrict__ ckpt, float* __restrict__ ucor, int B, int T, int H) {
    using G = BwdGeom<D>;
    constexpr int N = G::N, R = G::RPT, W = G::W;
    __shared__ StageLds<E, R, W, false> sl;
    const int l = (int)threadIdx.x;
    const int cb = (int)(blockIdx.x % G::NCB);
    const size_t ur = blockIdx.x / G::NCB;
    const int sg = (int)(ur % (size_t)nseg);
    const size_t u = ur / nseg;
    const int b = (int)(u / (size_t)H), h = (int)(u % (size_t)H);
    const int NC = (T + kChunk - 1) / kChunk;
    // chunks [n_beg, n_end) of segment sg (whole chunks: T is a multiple of
    // 16 nseg when nseg > 1)
    const int n_beg = (int)((long)NC * sg / nseg), n_end = (int)((long)NC * (sg + 1) / nseg);
    const GateConsts gc = make_gate(A[h], g_min);
    // the segment's start state: S0 for one segment, else the scanned one
    const float* s_in = nseg > 1 ? Sseg + (((size_t)b * nseg + sg) * H + h) * (size_t)D * D
                                 : (S0 ? S0 + u * (size_t)D * D : nullptr);
    float S[R][N];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        if (s_in) load8f(s_in + (size_t)(R * l + i) * D + cb * N, S[i]);
        else
#pragma unroll
            for (int j = 0; j < N; ++j) S[i][j] = 0.f;
    }
    float* ck = ckpt + (u * G::NCB + cb) * (size_t)NC * (D * N) + (R * l) * N;
    float* uc = ucor ? ucor + (u * G::NCB + cb) * (size_t)T * N : nullptr;
    const size_t vstride = (size_t)H * D;     // elements between tokens of a head
    const E* vb = v + ((size_t)b * T * H + h) * D + cb * N;
    Stage<E, R, false> st;
    stage_load<E, E, D, false>(st, nullptr, k, z, beta, nullptr,
                               vb + (size_t)n_beg * kChunk * vstride, vstride, b, h, T, H, cb,
                               n_beg * kChunk);
    for (int n = n_beg; n < n_end; ++n) {
        const int buf = n & 1;
        stage_store(st, sl, buf);
        if (n + 1 < n_end)
            stage_load<E, E, D, false>(st, nullptr, k, z, beta, nullptr,
                                       vb + (size_t)(n + 1) * kChunk * vstride, vstride, b, h, T,
                                       H, cb, (n + 1) * kChunk);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < R; ++i) store8f(ck + (size_t)n * (D * N) + i * N, S[i]);
        const int L = min(kChunk, T - n * kChunk);
        for (int r = 0; r < L; ++r) {
            const Rows<E, R> zr = sl.z[r][l], kr = sl.k[r][l];
            float kc[R], part[N], p[N];
#pragma unroll
            for (int j = 0; j < N; ++j) part[j] = 0.f;
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const float a = gate_alpha(gc, gate_sigmoid(gc, to_f32(zr.x[i])));
                kc[i] = to_f32(kr.x[i]);
#pragma unroll
                for (int j = 0; j < N; ++j) {
                    S[i][j] *= a;
                    part[j] += kc[i] * S[i][j];
                }
            }
            wave_sum8<W>(part, p);
            const float bt = sl.beta[buf][r];
            float uu[N];
#pragma unroll
            for (int j = 0; j < N; ++j) uu[j] = sl.x[buf][r][j] - p[j];
            if (l == 0 && uc) store8f(uc + (size_t)(n * kChunk + r) * N, uu);
#pragma unroll
            for (int i = 0; i < R; ++i)
#pragma unroll
                for (int j = 0; j < N; ++j) S[i][j] += kc[i] * bt * uu[j];
        }
    }
}

// Reverse sweep over tokens [t0, t1) (t0 a multiple of the segment length, t1
// = T or the next segment's start).  Partials are indexed by the token's place
// in the segment.
//   PAR = false: one workgroup per (b, h, column block) walks the chunks last
//     to first; the state gradient starts from dS_T (t1 == T) or the carry of
//     the previous launch, and ends in dS0 (t0 == 0) or the carry.
//   PAR = true: one workgroup per (b, h, column block, chunk), all chunks of
//     the range at once; each starts from the gradient of its chunk's end
//     state, dSend (from bwd_chain_kernel), and the first chunk's workgroup
//     writes dS0.
// The chunk's states are recomputed and swept in windows of HW tokens (the
// LDS a workgroup holds scales with HW; each window recomputes from the
// chunk's checkpoint).
template <typename E, int D, bool PAR, int HW>
__global__ __launch_bounds__(BwdGeom<D>::W) void bwd_seg_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ z,
    const float* __restrict__ beta, const float* __restrict__ A, float g_min,
    const E* __restrict__ dO, const float* __restrict__ dST, const float* __restrict__ ckpt,
    const float* __restrict__ ucor, float* __restrict__ carry, float* __restrict__ dS0,
    E* __restrict__ dv, float* __restrict__ pq, float* __restrict__ pk, float* __restrict__ pg,
    float* __restrict__ pb, const float* __restrict__ dSend, int nch, int B, int T, int H,
    int t0, int t1, int seg) {
    using G = BwdGeom<D>;
    constexpr int N = G::N, R = G::RPT, W = G::W;
    static_assert(HW >= 1 && HW <= kChunk, "window within a chunk");
    // hist[r][m][l]: the state slice before token w0 + r of the chunk's
    // current window, lane l's rows, values 4m .. 4m+3 of row R l + m / 2
    // (lane l reads back only its own)
    __shared__ f32x4 hist[HW][R * N / 4][W];
    __shared__ StageLds<E, R, W, true> sl;
    const int l = (int)threadIdx.x;
    const int cb = (int)(blockIdx.x % G::NCB);
    const size_t rest = blockIdx.x / G::NCB;
    const int nl = PAR ? (int)(rest % (size_t)nch) : 0;
    const size_t u = PAR ? rest / (size_t)nch : rest;
    const int b = (int)(u / (size_t)H), h = (int)(u % (size_t)H);
    const int NC = (T + kChunk - 1) / kChunk;
    const GateConsts gc = make_gate(A[h], g_min);
    const int n_hi = PAR ? t0 / kChunk + nl : (t1 - 1) / kChunk;
    const int n_lo = PAR ? n_hi : t0 / kChunk;
    float dS[R][N];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const size_t slice = (u * D + R * l + i) * D + cb * N;   // [b, h, row, cb * N]
        if (PAR) {
            load8f(dSend + (((u * NC + n_hi) * D + R * l + i) * D + cb * N), dS[i]);
        } else if (t1 == T) {
            if (dST) load8f(dST + slice, dS[i]);
            else
#pragma unroll
                for (int j = 0; j < N; ++j) dS[i][j] = 0.f;
        } else {
            load8f(carry + slice, dS[i]);
        }
    }
    const float* ck = ckpt + (u * G::NCB + cb) * (size_t)NC * (D * N) + (R * l) * N;
    const float* uc = ucor + (u * G::NCB + cb) * (size_t)T * N;
    Stage<E, R, true> st;
    stage_load<E, float, D, true>(st, q, k, z, beta, dO, uc + (size_t)n_hi * kChunk * N, N, b, h,
                                  T, H, cb, n_hi * kChunk);
    for (int n = n_hi; n >= n_lo; --n) {
        const int cs = n * kChunk;
        const int L = min(kChunk, T - cs);
        const int buf = n & 1;
        stage_store(st, sl, buf);
        if (n > n_lo)
            stage_load<E, float, D, true>(st, q, k, z, beta, dO, uc + (size_t)(cs - kChunk) * N,
                                          N, b, h, T, H, cb, cs - kChunk);
        __syncthreads();
        // (with HW = kChunk a single window: w0 is 0 at compile time)
        for (int w0 = HW == kChunk ? 0 : ((L - 1) / HW) * HW; w0 >= 0; w0 -= HW) {
            const int w1 = HW == kChunk ? L : min(L, w0 + HW);
            float S[R][N];
#pragma unroll
            for (int i = 0; i < R; ++i) load8f(ck + (size_t)n * (D * N) + i * N, S[i]);
            // recompute the chunk's states up to the window's end from the stored
            // corrections, keeping those of the window
            for (int r = 0; r < w1; ++r) {
                if (HW == kChunk || r >= w0) {
#pragma unroll
                    for (int i = 0; i < R; ++i)
#pragma unroll
                        for (int m = 0; m < N / 4; ++m)
                            hist[r - w0][i * (N / 4) + m][l] =
                                f32x4{S[i][4 * m], S[i][4 * m + 1], S[i][4 * m + 2], S[i][4 * m + 3]};
                }
                const Rows<E, R> zr = sl.z[r][l], kr = sl.k[r][l];
                const float bt = sl.beta[buf][r];
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    const float a = gate_alpha(gc, gate_sigmoid(gc, to_f32(zr.x[i])));
                    const float kb = to_f32(kr.x[i]) * bt;
#pragma unroll
                    for (int j = 0; j < N; ++j) S[i][j] = a * S[i][j] + kb * sl.x[buf][r][j];
                }
            }
            // reverse sweep of the window
            for (int r = w1 - 1; r >= w0; --r) {
                const int t = cs + r;
                const Rows<E, R> zr = sl.z[r][l], kr = sl.k[r][l], qr = sl.q[r][l];
                const float bt = sl.beta[buf][r];
                float uu[N], dov[N], part[N], de[N];
#pragma unroll
                for (int j = 0; j < N; ++j) {
                    uu[j] = sl.x[buf][r][j];
                    dov[j] = sl.dO[buf][r][j];
                    part[j] = 0.f;
                }
                // S_t = a S_prev + k beta u^T (rows of this lane), so the products
                // with S_t and S' = a S_prev reduce to row sums of S_prev:
                //   dq = S_t dO = a (S_prev . dO) + k beta (u . dO)
                //   dk = beta (dS . u) - beta a (S_prev . de)
                //   dg = a (dS' . S_prev) = a ((dS . S_prev) - k beta (S_prev . de))
                //   dS_prev = a dS' = a dS - a k beta de^T
                float udo = 0.f;                         // u . dO, the same for every row
#pragma unroll
                for (int j = 0; j < N; ++j) udo += uu[j] * dov[j];
                float a[R], kb[R], Sprev[R][N], sdo[R];
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    a[i] = gate_alpha(gc, gate_sigmoid(gc, to_f32(zr.x[i])));
                    const float kc = to_f32(kr.x[i]);
                    const float qc = to_f32(qr.x[i]);
                    kb[i] = kc * bt;
#pragma unroll
                    for (int m = 0; m < N / 4; ++m) {
                        const f32x4 x = hist[r - w0][i * (N / 4) + m][l];
#pragma unroll
                        for (int e = 0; e < 4; ++e) Sprev[i][4 * m + e] = x[e];
                    }
                    float sd = 0.f;
#pragma unroll
                    for (int j = 0; j < N; ++j) {
                        dS[i][j] += qc * dov[j];
                        sd += Sprev[i][j] * dov[j];
                        part[j] += kc * dS[i][j];
                    }
                    sdo[i] = sd;
                }
                wave_sum8<W>(part, de);
                float dqc[R], dkc[R], dgc[R];
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    float sde = 0.f, dsu = 0.f, dss = 0.f;   // S_prev . de, dS . u, dS . S_prev
#pragma unroll
                    for (int j = 0; j < N; ++j) {
                        sde += Sprev[i][j] * de[j];
                        dsu += dS[i][j] * uu[j];
                        dss += dS[i][j] * Sprev[i][j];
                    }
                    dqc[i] = a[i] * sdo[i] + kb[i] * udo;
                    dkc[i] = bt * dsu - bt * a[i] * sde;
                    dgc[i] = a[i] * (dss - kb[i] * sde);
                    const float akb = a[i] * kb[i];
#pragma unroll
                    for (int j = 0; j < N; ++j) dS[i][j] = a[i] * dS[i][j] - akb * de[j];
                }
                const size_t prow = (((size_t)cb * B + b) * seg + (t - t0)) * H + h;
                *reinterpret_cast<Rows<float, R>*>(pq + prow * D + R * l) =
                    *reinterpret_cast<const Rows<float, R>*>(dqc);
                *reinterpret_cast<Rows<float, R>*>(pk + prow * D + R * l) =
                    *reinterpret_cast<const Rows<float, R>*>(dkc);
                *reinterpret_cast<Rows<float, R>*>(pg + prow * D + R * l) =
                    *reinterpret_cast<const Rows<float, R>*>(dgc);
                if (l == 0) {
                    float db = 0.f, dvv[N];
#pragma unroll
                    for (int j = 0; j < N; ++j) {
                        db += de[j] * uu[j];
                        dvv[j] = bt * de[j];
                    }
                    pb[prow] = db;
                    store8(dv + (((size_t)b * T + t) * H + h) * D + cb * N, dvv);
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const size_t slice = (u * D + R * l + i) * D + cb * N;
        if (PAR) {
            if (n_lo == 0 && dS0) store8f(dS0 + slice, dS[i]);
        } else if (t0 == 0) {
            if (dS0) store8f(dS0 + slice, dS[i]);
        } else {
            store8f(carry + slice, dS[i]);
        }
    }
}

// Gradients of the chunk end states, chunk by chunk from the last: with the
// chunk's factors K~ = k e^G, Q~ = q e^G, Kdec = k e^{G_L - G}, gamma = e^{G_L}
// (G the chunk-local cumulative log-decay), Tm and Aqk (the intra-chunk
// stage's exports), the state gradient at the chunk's start is
//   dS_start = Diag(gamma) dS_end + Q~^T dO - K~^T Tm^T (Kdec dS_end + Aqk^T dO)
// (the chunk equations differentiated; the same recurrence the token-level
// reverse sweep runs 16 steps at a time).  One workgroup of kBwdChainThreads per
// (b, h, 16 value columns); per chunk three small products through LDS, the
// inputs of chunks n - 1 .. n - 4 loading meanwhile.
// Writes dSend[(u * NC + n)] = the gradient of chunk n's end state.
template <typename E, int D>
__global__ __launch_bounds__(kBwdChainThreads) void bwd_chain_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const float* __restrict__ Gc,
    const float* __restrict__ Tm, const float* __restrict__ Aqk, const float* __restrict__ gam,
    const E* __restrict__ dO, const float* __restrict__ dST, float* __restrict__ dSend, int T,
    int H) {
    constexpr int NT = kBwdChainThreads;
    constexpr int CB = 16;                  // value columns per workgroup
    constexpr int TPR = NT / D;             // threads per state row
    constexpr int CPT = CB / TPR;           // state columns per thread
    constexpr int FE = kChunk * D / NT;     // factor elements per thread
    constexpr int DP = D + 4;               // padded row (16-byte aligned rows)
    static_assert(CPT >= 1 && FE >= 1, "thread layout");
    constexpr int kAhead = 4;               // chunks of inputs in flight
    __shared__ __attribute__((aligned(16))) float sKd[kChunk][DP];
    __shared__ __attribute__((aligned(16))) float sKt[kChunk][DP];
    __shared__ __attribute__((aligned(16))) float sQt[kChunk][DP];
    __shared__ __attribute__((aligned(16))) float sST[CB][DP];          // dS_end, transposed
    __shared__ __attribute__((aligned(16))) float sdO[kChunk][CB], sY[kChunk][CB];
    __shared__ float sTm[kChunk][17], sAq[kChunk][17], sZ[kChunk][17], sg[D];
    const int tid = (int)threadIdx.x;
    const int nct = D / CB;
    const int ct = (int)(blockIdx.x % nct);
    const size_t u = blockIdx.x / nct;
    const int b = (int)(u / (size_t)H), h = (int)(u % (size_t)H);
    const int NC = (T + kChunk - 1) / kChunk;
    const int c = tid / TPR, j0 = (tid % TPR) * CPT;   // state entries: row c, columns j0 ..
    const bool zt = tid < 256;                         // threads of the 16x16 products
    const int zr = (tid & 255) / CB, zj = tid % CB;
    const size_t col0 = (size_t)ct * CB;
    float dS[CPT];
#pragma unroll
    for (int x = 0; x < CPT; ++x) dS[x] = dST ? dST[(u * D + c) * D + col0 + j0 + x] : 0.f;
    // one chunk's inputs in registers, loaded two chunks ahead of use
    struct In {
        float k[FE], q[FE], g[FE], gm[FE];
        float tm, aq, dO, gg;
    };
    auto load = [&](int n, In& in) {
        const int cs = n * kChunk, L = min(kChunk, T - cs);
        const size_t cidx = u * NC + n;
#pragma unroll
        for (int x = 0; x < FE; ++x) {
            const int e = tid + NT * x, r = e / D, cc = e % D;
            if (r < L) {
                const size_t i = (((size_t)b * T + cs + r) * H + h) * D + cc;
                in.k[x] = to_f32(k[i]);
                in.q[x] = to_f32(q[i]);
                in.g[x] = Gc[i];
            } else {
                in.k[x] = in.q[x] = in.g[x] = 0.f;
            }
            in.gm[x] = gam[cidx * D + cc];
        }
        if (zt) {
            in.tm = Tm[cidx * 256 + tid];
            in.aq = Aqk[cidx * 256 + tid];
            in.dO = zr < L ? to_f32(dO[(((size_t)b * T + cs + zr) * H + h) * D + col0 + zj]) : 0.f;
        }
        in.gg = tid < D ? gam[cidx * D + tid] : 0.f;
    };
    // chunk n from `cur`, whose registers then take chunk n - kAhead's inputs
    auto step = [&](int n, In& cur) {
        const size_t cidx = u * NC + n;
        // the chunk's factors into LDS (rows past its end are zero)
#pragma unroll
        for (int x = 0; x < FE; ++x) {
            const int e = tid + NT * x, r = e / D, cc = e % D;
            const float ex = expf(cur.g[x]);
            sKt[r][cc] = cur.k[x] * ex;
            sQt[r][cc] = cur.q[x] * ex;
            sKd[r][cc] = cur.k[x] * (cur.gm[x] / ex);
        }
        if (zt) {
            sTm[zr][zj] = cur.tm;
            sAq[zr][zj] = cur.aq;
            sdO[zr][zj] = cur.dO;
        }
        if (tid < D) sg[tid] = cur.gg;
#pragma unroll
        for (int x = 0; x < CPT; ++x) {
            sST[j0 + x][c] = dS[x];
            dSend[(cidx * D + c) * D + col0 + j0 + x] = dS[x];
        }
        if (n >= kAhead) load(n - kAhead, cur);
        __syncthreads();
        // Z = Kdec dS_end + Aqk^T dO
        if (zt) {
            float z = 0.f;
#pragma unroll 4
            for (int cc = 0; cc < D; cc += 4) {
                const f32x4 a4 = *reinterpret_cast<const f32x4*>(&sKd[zr][cc]);
                const f32x4 s4 = *reinterpret_cast<const f32x4*>(&sST[zj][cc]);
                z += a4[0] * s4[0] + a4[1] * s4[1] + a4[2] * s4[2] + a4[3] * s4[3];
            }
#pragma unroll
            for (int i = 0; i < kChunk; ++i) z += sAq[i][zr] * sdO[i][zj];
            sZ[zr][zj] = z;
        }
        __syncthreads();
        // Y = Tm^T Z
        if (zt) {
            float y = 0.f;
#pragma unroll
            for (int i = 0; i < kChunk; ++i) y += sTm[i][zr] * sZ[i][zj];
            sY[zr][zj] = y;
        }
        __syncthreads();
        // dS_start = Diag(gamma) dS_end + Q~^T dO - K~^T Y (row c, columns j0 ..)
        const float gc = sg[c];
#pragma unroll
        for (int x = 0; x < CPT; ++x) dS[x] *= gc;
#pragma unroll
        for (int r = 0; r < kChunk; ++r) {
            const float qr = sQt[r][c], kr = sKt[r][c];
#pragma unroll
            for (int x = 0; x < CPT; ++x) dS[x] += qr * sdO[r][j0 + x] - kr * sY[r][j0 + x];
        }
        __syncthreads();   // before the next chunk's factors overwrite LDS
    };
    In r0, r1, r2, r3;   // chunks n, n - 1, n - 2, n - 3 (static register sets)
    load(NC - 1, r0);
    if (NC >= 2) load(NC - 2, r1);
    if (NC >= 3) load(NC - 3, r2);
    if (NC >= 4) load(NC - 4, r3);
    for (int n = NC - 1; n >= 0; n -= kAhead) {
        step(n, r0);
        if (n >= 1) step(n - 1, r1);
        if (n >= 2) step(n - 2, r2);
        if (n >= 3) step(n - 3, r3);
    }
}

// Sums of the column-block partials for tokens [t0, t0 + n_tok) of one
// (b, h) per workgroup row of blocks: dq, dk, dz (through the gate
// derivative), dbeta, and per block of kBwdTokBlock tokens the dA term.
template <typename E, int D>
__global__ __launch_bounds__(D) void bwd_finalize_kernel(
    const E* __restrict__ z, const float* __restrict__ A, float g_min,
    const float* __restrict__ pq, const float* __restrict__ pk, const float* __restrict__ pg,
    const float* __restrict__ pb, E* __restrict__ dq, E* __restrict__ dk, E* __restrict__ dz,
    float* __restrict__ dbeta, float* __restrict__ dA_part, int B, int T, int H, int t0,
    int n_tok, int seg, int nsb, int ntb) {
    using G = BwdGeom<D>;
    __shared__ float red[D];
    const int c = (int)threadIdx.x;
    const int sb = (int)(blockIdx.x % (unsigned)nsb);
    const size_t u = blockIdx.x / (unsigned)nsb;
    const int b = (int)(u / (size_t)H), h = (int)(u % (size_t)H);
    const float eA = expf(A[h]);
    const int r0 = sb * kBwdTokBlock, r1 = min(r0 + kBwdTokBlock, n_tok);
    const size_t cbs = (size_t)B * seg * H;   // stride of one column block
    float acc = 0.f;
    for (int r = r0; r < r1; ++r) {
        const size_t row = ((size_t)b * T + t0 + r) * H + h;
        const size_t prow = ((size_t)b * seg + r) * H + h;
        float sq = 0.f, sk = 0.f, sg = 0.f;
#pragma unroll
        for (int cb = 0; cb < G::NCB; ++cb) {
            const size_t i = (prow + cb * cbs) * D + c;
            sq += pq[i];
            sk += pk[i];
            sg += pg[i];
        }
        const float x = eA * to_f32(z[row * D + c]);
        const float s = 1.0f / (1.0f + expf(-x));
        const float dx = sg * g_min * s * (1.0f - s);
        dq[row * D + c] = from_f32<E>(sq);
        dk[row * D + c] = from_f32<E>(sk);
        dz[row * D + c] = from_f32<E>(dx * eA);
        acc += dx * x;
        if (c == 0) {
            float sbeta = 0.f;
            for (int cb = 0; cb < G::NCB; ++cb) sbeta += pb[prow + cb * cbs];
            dbeta[row] = sbeta;
        }
    }
    red[c] = acc;
    __syncthreads();
    if (c == 0) {
        float s = 0.f;
        for (int i = 0; i < D; ++i) s += red[i];
        dA_part[u * ntb + t0 / kBwdTokBlock + sb] = s;
    }
}

// dA[h] = sum over b and token blocks of the dA terms, in a fixed order.
__global__ __launch_bounds__(256) void bwd_dA_kernel(const float* __restrict__ dA_part,
                                                     float* __restrict__ dA, int B, int H,
                                                     int ntb) {
    __shared__ float red[256];
    const int h = (int)blockIdx.x, tid = (int)threadIdx.x;
    const long n = (long)B * ntb;
    float s = 0.f;
    for (long i = tid; i < n; i += 256) {
        const long b = i / ntb, tb = i % ntb;
        s += dA_part[((size_t)b * H + h) * ntb + tb];
    }
    red[tid] = s;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if (tid < w) red[tid] += red[tid + w];
        __syncthreads();
    }
    if (tid == 0) dA[h] = red[0];
}

// ------------------------------------------------------------------ host

static size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Plan of the reverse sweep: "sweep" (one token-level sweep per (b, h,
// column block) over the whole sequence, the default) or, with
// KDA_BACKWARD_PLAN=chain and more than one chunk, "chain" (the chunk-level
// state-gradient chain, then every chunk's token-level sweep at once; on
// MI355X it is slower for now: its chain kernel runs ~8 us per chunk).
bool bwd_plan_chain(int T) {
    const char* env = std::getenv("KDA_BACKWARD_PLAN");
    return env && std::strcmp(env, "chain") == 0 && T > kChunk;
}

// The chunkwise MFMA plan (kda_bwd_chunk.hip) for bf16 at d = 128 unless a
// token-level plan is forced (KDA_BACKWARD_PLAN = "sweep" or "chain").
bool bwd_plan_chunk(int d, bool is_bf16) {
    const char* env = std::getenv("KDA_BACKWARD_PLAN");
    return bwd_chunk_ok(d, is_bf16) && !env;
}

BwdLayout bwd_layout(int B, int T, int H, int d, bool is_bf16) {
    BwdLayout L;
    // The forward sweep runs as R segments side by side, each from its start
    // state out of a segment scan, when T splits into R whole-chunk segments
    // of at least kBwdSegMin tokens.
    L.R = 1;
    for (int r : {8, 4, 2})
        if (T % (kChunk * r) == 0 && T / r >= kBwdSegMin &&
            (long long)B * r * H <= (1LL << 26)) {   // the inner prefill's unit limit
            L.R = r;
            break;
        }
    const size_t units = (size_t)B * H;
    const int NCB = d / kBwdCols;
    L.NC = (T + kChunk - 1) / kChunk;
    L.chunk = bwd_plan_chunk(d, is_bf16);
    L.ntb = (T + kBwdTokBlock - 1) / kBwdTokBlock;
    // segment length: a multiple of the finalize token block, with the
    // partials of one segment within kBwdPartialBudget bytes
    const size_t per_tok = units * ((size_t)3 * NCB * d + NCB) * sizeof(float);
    size_t seg = kBwdPartialBudget / per_tok;
    seg = seg / kBwdTokBlock * kBwdTokBlock;
    // at least kBwdSegTokensMin tokens per launch, so that many units do not
    // turn the sweep into thousands of short launches (the partials then
    // exceed the budget)
    if (seg < (size_t)kBwdSegTokensMin) seg = kBwdSegTokensMin;
    const size_t Tr = round_up((size_t)T, kBwdTokBlock);
    if (seg > Tr) seg = Tr;
    L.seg = (int)seg;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = round_up(off + bytes, 256);
        return o;
    };
    L.ckpt = take(units * L.NC * (size_t)d * d * sizeof(float));
    L.fac = L.dSend = 0;
    if (L.chunk) {
        // chunkwise plan: checkpoints, the chain's operand blocks, every
        // chunk's end-state gradient and a dA term per chunk
        L.fac = take(units * L.NC * bwd_chunk_fac_bytes());
        L.dSend = take(units * L.NC * (size_t)d * d * sizeof(float));
        L.dA_part = take(units * L.NC * sizeof(float));
        L.carry = L.ucor = L.pq = L.pk = L.pg = L.pb = 0;
        L.chain = false;
        L.Gc = L.Tm = L.Aqk = L.gam = 0;
    } else {
        L.carry = take(units * (size_t)d * d * sizeof(float));
        L.ucor = take(units * (size_t)T * d * sizeof(float));
        const size_t pel = (size_t)NCB * units * seg;   // partial rows
        L.pq = take(pel * d * sizeof(float));
        L.pk = take(pel * d * sizeof(float));
        L.pg = take(pel * d * sizeof(float));
        L.pb = take(pel * sizeof(float));
        L.dA_part = take(units * L.ntb * sizeof(float));
        // chain plan: the gate and intra-chunk exports, and the end-state
        // gradient of every chunk
        L.chain = bwd_plan_chain(T);
        L.Gc = L.Tm = L.Aqk = L.gam = L.dSend = 0;
        if (L.chain) {
            L.Gc = take(units * (size_t)T * d * sizeof(float));
            L.Tm = take(units * L.NC * (size_t)256 * sizeof(float));
            L.Aqk = take(units * L.NC * (size_t)256 * sizeof(float));
            L.gam = take(units * L.NC * (size_t)d * sizeof(float));
            L.dSend = take(units * L.NC * (size_t)d * d * sizeof(float));
        }
    }
    L.segws = L.oscr = 0;
    if (L.R > 1) {
        // the segment scan's passes write no outputs where the plan allows
        // it; otherwise they need a scratch o
        const SegLayout SL = seg_layout(B, T, H, d, is_bf16, L.R);
        L.segws = take(SL.total);
        if (!prefill_state_only_ok(SL.inner, d))
            L.oscr = take((size_t)B * T * H * d * (is_bf16 ? 2 : 4));
    }
    L.total = off;
    return L;
}

template <typename E, int D>
static hipError_t launch_backward_t(const BackwardArgs& a, char* ws, hipStream_t stream) {
    using G = BwdGeom<D>;
    const BwdLayout L = bwd_layout(a.B, a.T, a.H, D, sizeof(E) == 2);
    const size_t units = (size_t)a.B * a.H;
    float* ckpt = (float*)(ws + L.ckpt);
    float* carry = (float*)(ws + L.carry);
    float* ucor = (float*)(ws + L.ucor);
    float* pq = (float*)(ws + L.pq);
    float* pk = (float*)(ws + L.pk);
    float* pg = (float*)(ws + L.pg);
    float* pb = (float*)(ws + L.pb);
    float* dA_part = (float*)(ws + L.dA_part);
    const E* q = (const E*)a.q;
    const E* k = (const E*)a.k;
    const E* v = (const E*)a.v;
    const E* z = (const E*)a.z;
    const dim3 grid((unsigned)(units * G::NCB)), block(G::W);
    hipError_t e = hipSuccess;
    const float* Sseg = nullptr;
    if (L.R > 1) {
        // start states of the R segments by the segment scan of the forward
        const SegLayout SL = seg_layout(a.B, a.T, a.H, D, sizeof(E) == 2, L.R);
        PrefillArgs fa{a.q, a.k, a.v, a.z, a.beta, a.A, a.g_min, dense_state(a.S0, nullptr),
                       ws + L.oscr, a.B, a.T, a.H, D, sizeof(E) == 2};
        if ((e = seg_start_states(fa, L.R, SL, ws + L.segws, stream)) != hipSuccess) return e;
        Sseg = (const float*)(ws + L.segws + SL.Sin);
    }
    if (L.chunk) {
        // chunk-start states by a chunkwise state-only pass, the R segments
        // side by side from their scanned start states
        const PrefillArgs ca{a.q, a.k, a.v, a.z, a.beta, a.A, a.g_min,
                             dense_state(L.R > 1 ? Sseg : a.S0, nullptr), nullptr, a.B * L.R,
                             a.T / L.R, a.H, D, true};
        if ((e = launch_ckpt_pass(ca, CkOut{ckpt, L.R, L.NC}, stream)) != hipSuccess) return e;
        if ((e = launch_bwd_chunk(a, ckpt, ws + L.fac, (float*)(ws + L.dSend), dA_part, stream)) !=
            hipSuccess)
            return e;
        hipLaunchKernelGGL(bwd_dA_kernel, dim3(a.H), dim3(256), 0, stream, dA_part, a.dA, a.B, a.H,
                           L.NC);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((bwd_ckpt_kernel<E, D>), dim3((unsigned)(units * L.R * G::NCB)), block, 0,
                       stream, k, v, z, a.beta, a.A, a.g_min, a.S0, Sseg, L.R, ckpt, ucor, a.B,
                       a.T, a.H);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const float* dSend = nullptr;
    if (L.chain) {
        // chunk factors (the intra-chunk stage's exports) and the chain
        float* Gc = (float*)(ws + L.Gc);
        float* Tm = (float*)(ws + L.Tm);
        float* Aqk = (float*)(ws + L.Aqk);
        float* gam = (float*)(ws + L.gam);
        if ((e = launch_gate_cumsum(a.z, a.A, a.g_min, Gc, a.B, a.T, a.H, D, sizeof(E) == 2,
                                    stream)) != hipSuccess)
            return e;
        if ((e = launch_intra_diag(a.q, a.k, a.z, a.beta, a.A, a.g_min, Tm, Aqk, gam, a.B, a.T, a.H,
                                   D, sizeof(E) == 2, stream)) != hipSuccess)
            return e;
        hipLaunchKernelGGL((bwd_chain_kernel<E, D>), dim3((unsigned)(units * (D / 16))),
                           dim3(kBwdChainThreads),
                           0, stream, q, k, Gc, Tm, Aqk, gam, (const E*)a.dO, a.dST,
                           (float*)(ws + L.dSend), a.T, a.H);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        dSend = (const float*)(ws + L.dSend);
    }
    for (int t1 = a.T; t1 > 0;) {
        const int t0 = ((t1 - 1) / L.seg) * L.seg;
        if (L.chain) {
            const int nch = (t1 - t0 + kChunk - 1) / kChunk;
            hipLaunchKernelGGL((bwd_seg_kernel<E, D, true, kBwdHistPar>),
                               dim3((unsigned)(units * nch * G::NCB)), block, 0, stream, q, k, z,
                               a.beta, a.A, a.g_min, (const E*)a.dO, a.dST, ckpt, ucor, carry,
                               a.dS0, (E*)a.dv, pq, pk, pg, pb, dSend, nch, a.B, a.T, a.H, t0, t1,
                               L.seg);
        } else {
            hipLaunchKernelGGL((bwd_seg_kernel<E, D, false, kChunk>), grid, block, 0, stream, q, k,
                               z, a.beta, a.A, a.g_min, (const E*)a.dO, a.dST, ckpt, ucor, carry,
                               a.dS0, (E*)a.dv, pq, pk, pg, pb, nullptr, 1, a.B, a.T, a.H, t0, t1,
                               L.seg);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int n_tok = t1 - t0;
        const int nsb = (n_tok + kBwdTokBlock - 1) / kBwdTokBlock;
        hipLaunchKernelGGL((bwd_finalize_kernel<E, D>), dim3((unsigned)(units * nsb)), dim3(D), 0,
                           stream, z, a.A, a.g_min, pq, pk, pg, pb, (E*)a.dq, (E*)a.dk, (E*)a.dz,
                           a.dbeta, dA_part, a.B, a.T, a.H, t0, n_tok, L.seg, nsb, L.ntb);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        t1 = t0;
    }
    hipLaunchKernelGGL(bwd_dA_kernel, dim3(a.H), dim3(256), 0, stream, dA_part, a.dA, a.B, a.H,
                       L.ntb);
    return hipGetLastError();
}

hipError_t launch_backward(const BackwardArgs& a, void* ws, hipStream_t stream) {
    char* w = (char*)ws;
    if (a.is_bf16)
        return a.d == 128 ? launch_backward_t<bf16, 128>(a, w, stream)
                          : launch_backward_t<bf16, 32>(a, w, stream);
    return a.d == 128 ? launch_backward_t<float, 128>(a, w, stream)
                      : launch_backward_t<float, 32>(a, w, stream);
}

}  // namespace kda
