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
// summed afterwards in a fixed order.  A workgroup has d_k threads, thread c
// owning key row c of the 8 columns in registers, so every reduction over
// value columns stays in the thread and the one over key rows (S'^T k in the
// forward, dS^T k in the reverse) is a wave reduce-scatter plus an exchange of
// the per-wave sums through LDS: one workgroup barrier per token.
//   bwd_ckpt_kernel   forward over the sequence, storing the state slice at
//                     the start of each 16-token chunk (HBM checkpoints).
//   bwd_seg_kernel    per chunk, last to first: recompute the chunk's states
//                     from its checkpoint into LDS, then sweep it in reverse;
//                     writes dv and per-block partials of dq, dk, dg, dbeta.
//                     Runs over segments of the sequence (last first), the
//                     state gradient carried between launches, so that the
//                     partials occupy a bounded workspace.
//   bwd_finalize_kernel  sums the partials over column blocks, applies the
//                     gate derivative (dz) and forms per-token-block dA terms.
//   bwd_dA_kernel     sums the dA terms of each head in a fixed order.
// The sweep is a serial chain of VALU work and workgroup barriers per token
// (no contraction wide enough for MFMA: per token each thread does O(8) FMAs
// per product); it is bounded by latency, with HBM traffic for inputs, the
// checkpoints and the partials.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <int D>
struct BwdGeom {
    static constexpr int N = kBwdCols;         // value columns per workgroup
    static constexpr int NT = D;               // threads: one per key row
    static constexpr int NCB = D / N;          // column blocks per head
    static constexpr int W = NT < kWave ? NT : kWave;   // lanes of a wave in use
    static constexpr int NW = NT / W;          // waves
    static_assert(N == 8, "row pieces of 8 values");
    static_assert(N <= W, "one reduced column per group of W / N lanes");
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

// Reduce-scatter of N values over the W lanes of a wave: at each step a lane
// keeps half of its values and adds the partner's copy of that half (the
// partner keeps the other half); once one value is left the remaining lane
// masks complete the sum.  Afterwards lane l holds the wave's sum of value
// (l mod W) / (W / N).
template <int W, int N, int M>
__device__ __forceinline__ void wave_rs(float* w, int lane) {
    if constexpr (N > 1) {
        const bool up = (lane & M) != 0;
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            const float send = up ? w[i] : w[i + N / 2];
            const float keep = up ? w[i + N / 2] : w[i];
            w[i] = keep + __shfl_xor(send, M, W);
        }
        wave_rs<W, N / 2, M / 2>(w, lane);
    } else if constexpr (M >= 1) {
        w[0] += __shfl_xor(w[0], M, W);
        wave_rs<W, 1, M / 2>(w, lane);
    }
}

// Sum over the workgroup's key rows (threads) of N per-thread values, result
// in every thread.  wsum is a double buffer of per-wave sums; par alternates
// so that one barrier per call suffices (a buffer is rewritten only after the
// next call's barrier, which every reader of its previous contents has passed).
template <int D>
__device__ __forceinline__ void rows_sum(const float (&part)[kBwdCols], float (&out)[kBwdCols],
                                         float (*wsum)[BwdGeom<D>::NW][kBwdCols], int& par) {
    using G = BwdGeom<D>;
    constexpr int N = G::N, W = G::W, NW = G::NW, GL = W / N;
    float w[N];
#pragma unroll
    for (int i = 0; i < N; ++i) w[i] = part[i];
    const int lane = (int)threadIdx.x & (W - 1), wave = (int)threadIdx.x / W;
    wave_rs<W, N, W / 2>(w, lane);
    if (lane % GL == 0) wsum[par][wave][lane / GL] = w[0];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < N; ++j) {
        float s = wsum[par][0][j];
#pragma unroll
        for (int x = 1; x < NW; ++x) s += wsum[par][x][j];
        out[j] = s;
    }
    par ^= 1;
}

// ------------------------------------------------------------------ kernels

// Forward over the whole sequence; the state slice of each chunk's start goes
// to ckpt[(u * NCB + cb) * NC + n] (D x 8 floats, row-major).
template <typename E, int D>
__global__ __launch_bounds__(D) void bwd_ckpt_kernel(
    const E* __restrict__ k, const E* __restrict__ v, const E* __restrict__ z,
    const float* __restrict__ beta, const float* __restrict__ A, float g_min,
    const float* __restrict__ S0, float* __restrict__ ckpt, int B, int T, int H) {
    using G = BwdGeom<D>;
    constexpr int N = G::N;
    __shared__ float wsum[2][G::NW][N];
    const int c = (int)threadIdx.x;
    const int cb = (int)(blockIdx.x % G::NCB);
    const size_t u = blockIdx.x / G::NCB;
    const int b = (int)(u / (size_t)H), h = (int)(u % (size_t)H);
    const int NC = (T + kChunk - 1) / kChunk;
    const GateConsts gc = make_gate(A[h], g_min);
    float S[N];
    if (S0) load8f(S0 + (u * D + c) * D + cb * N, S);
    else
#pragma unroll
        for (int j = 0; j < N; ++j) S[j] = 0.f;
    float* ck = ckpt + (u * G::NCB + cb) * (size_t)NC * (D * N) + c * N;
    int par = 0;
    for (int t = 0; t < T; ++t) {
        if (t % kChunk == 0) store8f(ck + (size_t)(t / kChunk) * (D * N), S);
        const size_t row = ((size_t)b * T + t) * H + h;
        const float a = gate_alpha(gc, gate_sigmoid(gc, to_f32(z[row * D + c])));
        const float kc = to_f32(k[row * D + c]);
        float Sp[N], part[N], p[N], vv[N];
#pragma unroll
        for (int j = 0; j < N; ++j) {
            Sp[j] = a * S[j];
            part[j] = kc * Sp[j];
        }
        rows_sum<D>(part, p, wsum, par);
        load8(v + row * D + cb * N, vv);
        const float kb = kc * beta[row];
#pragma unroll
        for (int j = 0; j < N; ++j) S[j] = Sp[j] + kb * (vv[j] - p[j]);
    }
}

// Reverse sweep over tokens [t0, t1) (t0 a multiple of the segment length, t1
// = T or the next segment's start).  The state gradient starts from dS_T
// (t1 == T) or the carry of the previous launch, and ends in dS0 (t0 == 0)
// or the carry.  Partials are indexed by the token's place in the segment.
template <typename E, int D>
__global__ __launch_bounds__(D) void bwd_seg_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const E* __restrict__ z, const float* __restrict__ beta, const float* __restrict__ A,
    float g_min, const E* __restrict__ dO, const float* __restrict__ dST,
    const float* __restrict__ ckpt, float* __restrict__ carry, float* __restrict__ dS0,
    E* __restrict__ dv, float* __restrict__ pq, float* __restrict__ pk, float* __restrict__ pg,
    float* __restrict__ pb, int B, int T, int H, int t0, int t1, int seg) {
    using G = BwdGeom<D>;
    constexpr int N = G::N;
    // hist[r][i][c]: the state slice before token r of the chunk, thread c's
    // row, values 4i..4i+3 (each thread reads back only its own row)
    __shared__ f32x4 hist[kChunk][N / 4][D];
    __shared__ float ubuf[kChunk][N];           // u = v - S'^T k per token
    __shared__ float wsum[2][G::NW][N];
    const int c = (int)threadIdx.x;
    const int cb = (int)(blockIdx.x % G::NCB);
    const size_t u = blockIdx.x / G::NCB;
    const int b = (int)(u / (size_t)H), h = (int)(u % (size_t)H);
    const int NC = (T + kChunk - 1) / kChunk;
    const GateConsts gc = make_gate(A[h], g_min);
    const size_t slice = (u * D + c) * D + cb * N;           // [b, h, c, cb * N]
    float dS[N];
    if (t1 == T) {
        if (dST) load8f(dST + slice, dS);
        else
#pragma unroll
            for (int j = 0; j < N; ++j) dS[j] = 0.f;
    } else {
        load8f(carry + slice, dS);
    }
    const float* ck = ckpt + (u * G::NCB + cb) * (size_t)NC * (D * N) + c * N;
    int par = 0;
    for (int n = (t1 - 1) / kChunk; n >= t0 / kChunk; --n) {
        const int cs = n * kChunk;
        const int L = min(kChunk, T - cs);
        float S[N];
        load8f(ck + (size_t)n * (D * N), S);
        // recompute the chunk's states
        for (int r = 0; r < L; ++r) {
#pragma unroll
            for (int i = 0; i < N / 4; ++i)
                hist[r][i][c] = f32x4{S[4 * i], S[4 * i + 1], S[4 * i + 2], S[4 * i + 3]};
            const size_t row = ((size_t)b * T + cs + r) * H + h;
            const float a = gate_alpha(gc, gate_sigmoid(gc, to_f32(z[row * D + c])));
            const float kc = to_f32(k[row * D + c]);
            float Sp[N], part[N], p[N], vv[N];
#pragma unroll
            for (int j = 0; j < N; ++j) {
                Sp[j] = a * S[j];
                part[j] = kc * Sp[j];
            }
            rows_sum<D>(part, p, wsum, par);
            load8(v + row * D + cb * N, vv);
            const float kb = kc * beta[row];
#pragma unroll
            for (int j = 0; j < N; ++j) {
                const float uj = vv[j] - p[j];
                if (c == 0) ubuf[r][j] = uj;
                S[j] = Sp[j] + kb * uj;
            }
        }
        __syncthreads();   // ubuf of the last token
        // reverse sweep
        for (int r = L - 1; r >= 0; --r) {
            const int t = cs + r;
            const size_t row = ((size_t)b * T + t) * H + h;
            const float a = gate_alpha(gc, gate_sigmoid(gc, to_f32(z[row * D + c])));
            const float kc = to_f32(k[row * D + c]);
            const float qc = to_f32(q[row * D + c]);
            const float bt = beta[row];
            float Sprev[N], uu[N], dov[N], Sp[N], part[N], de[N];
#pragma unroll
            for (int i = 0; i < N / 4; ++i) {
                const f32x4 x = hist[r][i][c];
                Sprev[4 * i] = x[0];
                Sprev[4 * i + 1] = x[1];
                Sprev[4 * i + 2] = x[2];
                Sprev[4 * i + 3] = x[3];
            }
#pragma unroll
            for (int j = 0; j < N; ++j) uu[j] = ubuf[r][j];
            load8(dO + row * D + cb * N, dov);
            float dqc = 0.f;
#pragma unroll
            for (int j = 0; j < N; ++j) {
                Sp[j] = a * Sprev[j];
                const float Scur = Sp[j] + kc * bt * uu[j];
                dS[j] += qc * dov[j];
                dqc += Scur * dov[j];
                part[j] = kc * dS[j];
            }
            rows_sum<D>(part, de, wsum, par);
            float dkc = 0.f, dac = 0.f, db = 0.f;
#pragma unroll
            for (int j = 0; j < N; ++j) {
                dkc += bt * (dS[j] * uu[j] - Sp[j] * de[j]);
                const float dSp = dS[j] - kc * bt * de[j];
                dac += dSp * Sprev[j];
                dS[j] = a * dSp;
                db += de[j] * uu[j];
            }
            const size_t prow = (((size_t)cb * B + b) * seg + (t - t0)) * H + h;
            pq[prow * D + c] = dqc;
            pk[prow * D + c] = dkc;
            pg[prow * D + c] = dac * a;
            if (c == 0) {
                pb[prow] = db;
                float dvv[N];
#pragma unroll
                for (int j = 0; j < N; ++j) dvv[j] = bt * de[j];
                store8(dv + row * D + cb * N, dvv);
            }
        }
    }
    if (t0 == 0) {
        if (dS0) store8f(dS0 + slice, dS);
    } else {
        store8f(carry + slice, dS);
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

BwdLayout bwd_layout(int B, int T, int H, int d) {
    BwdLayout L;
    const size_t units = (size_t)B * H;
    const int NCB = d / kBwdCols;
    L.NC = (T + kChunk - 1) / kChunk;
    L.ntb = (T + kBwdTokBlock - 1) / kBwdTokBlock;
    // segment length: a multiple of the finalize token block, with the
    // partials of one segment within kBwdPartialBudget bytes
    const size_t per_tok = units * ((size_t)3 * NCB * d + NCB) * sizeof(float);
    size_t seg = kBwdPartialBudget / per_tok;
    seg = seg / kBwdTokBlock * kBwdTokBlock;
    if (seg < (size_t)kBwdTokBlock) seg = kBwdTokBlock;
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
    L.carry = take(units * (size_t)d * d * sizeof(float));
    const size_t pel = (size_t)NCB * units * seg;   // partial rows
    L.pq = take(pel * d * sizeof(float));
    L.pk = take(pel * d * sizeof(float));
    L.pg = take(pel * d * sizeof(float));
    L.pb = take(pel * sizeof(float));
    L.dA_part = take(units * L.ntb * sizeof(float));
    L.total = off;
    return L;
}

template <typename E, int D>
static hipError_t launch_backward_t(const BackwardArgs& a, char* ws, hipStream_t stream) {
    using G = BwdGeom<D>;
    const BwdLayout L = bwd_layout(a.B, a.T, a.H, D);
    const size_t units = (size_t)a.B * a.H;
    float* ckpt = (float*)(ws + L.ckpt);
    float* carry = (float*)(ws + L.carry);
    float* pq = (float*)(ws + L.pq);
    float* pk = (float*)(ws + L.pk);
    float* pg = (float*)(ws + L.pg);
    float* pb = (float*)(ws + L.pb);
    float* dA_part = (float*)(ws + L.dA_part);
    const E* q = (const E*)a.q;
    const E* k = (const E*)a.k;
    const E* v = (const E*)a.v;
    const E* z = (const E*)a.z;
    const dim3 grid((unsigned)(units * G::NCB)), block(D);
    hipLaunchKernelGGL((bwd_ckpt_kernel<E, D>), grid, block, 0, stream, k, v, z, a.beta, a.A,
                       a.g_min, a.S0, ckpt, a.B, a.T, a.H);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    for (int t1 = a.T; t1 > 0;) {
        const int t0 = ((t1 - 1) / L.seg) * L.seg;
        hipLaunchKernelGGL((bwd_seg_kernel<E, D>), grid, block, 0, stream, q, k, v, z, a.beta,
                           a.A, a.g_min, (const E*)a.dO, a.dST, ckpt, carry, a.dS0, (E*)a.dv, pq,
                           pk, pg, pb, a.B, a.T, a.H, t0, t1, L.seg);
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
