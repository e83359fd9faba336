// kda_decode.hip -- one recurrent KDA decode step, state updated in place.
//
// Per (b, h), with S' = Diag(a) S (a = exp(g_min Sigmoid(e^{A_h} z))):
//   p = S'^T k,  r = S'^T q          (two reductions over key channels)
//   e = beta (v - p)                 (delta-rule correction, d_v values)
//   S <- S' + k e^T                  (= (I - beta k k^T) S' + beta k v^T)
//   o  = S^T q = r + (q . k) e
// (dev.to "Kimi K3 Architecture ...", "The Sequence Bottleneck": state shape,
// retention/delta domains and the gate equation; terrencekim.net "Kimi K3 -
// Sparsity Mechanics ...", section 2: fixed-size state, constant decode
// memory.)
//
// The step is HBM-bound (S is read and written once: 2 * 4 * d_k * d_v bytes
// against ~7 d_k d_v flops), so the kernel is laid out for streaming: one
// workgroup per (b, h); each thread owns 4 adjacent value columns of
// RPT key rows (8 for d = 128, over 512 threads), so every wave instruction
// moves 1 KiB (d = 128) of S with 16-byte accesses.  S is held in registers between the read and the
// write, the two reductions come from the same read, and the update is
// written back with non-temporal stores.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <typename E, int D, int NT>
__global__ __launch_bounds__(NT) void decode_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const E* __restrict__ z, const float* __restrict__ beta, const float* __restrict__ A,
    float g_min, StateIO io, E* __restrict__ o, int H) {
    constexpr int CG = D / 4;          // column groups of 4 (float4)
    constexpr int RG = NT / CG;        // row groups
    constexpr int RPT = D / RG;        // rows per thread
    constexpr int NWAVE = NT / kWave;
    static_assert(NT % CG == 0 && D % RG == 0 && CG <= kWave, "decode layout");

    __shared__ float s_alpha[D], s_k[D], s_q[D], s_v[D];
    __shared__ float s_red[NWAVE][CG][9];

    const int tid = threadIdx.x;
    const size_t unit = blockIdx.x;    // b * H + h
    const int bi = (int)(unit / (size_t)H), h = (int)(unit % (size_t)H);
    const size_t vec = unit * (size_t)D;
    if (io.skip(bi)) return;           // uniform over the workgroup

    const int cg = tid % CG, rg = tid / CG;
    f32x4* Sv = reinterpret_cast<f32x4*>(io.out_at(bi, h, H, D));   // in place: in == out
    const GateConsts gc = make_gate(A[h], g_min);
    for (int c = tid; c < D; c += NT) {
        s_alpha[c] = gate_alpha(gc, gate_sigmoid(gc, to_f32(z[vec + c])));
        s_k[c] = to_f32(k[vec + c]);
        s_q[c] = to_f32(q[vec + c]);
        s_v[c] = to_f32(v[vec + c]);
    }
    __syncthreads();
    f32x4 st[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) st[i] = __builtin_nontemporal_load(&Sv[(rg + RG * i) * CG + cg]);

    float red[9];
#pragma unroll
    for (int x = 0; x < 9; ++x) red[x] = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int c = rg + RG * i;
        const float a = s_alpha[c], kc = s_k[c], qc = s_q[c];
        st[i] *= a;                                  // S' = Diag(a) S
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            red[x] += kc * st[i][x];                 // p = S'^T k
            red[4 + x] += qc * st[i][x];             // r = S'^T q
        }
        red[8] += qc * kc;                           // q . k (same in every column group)
    }
    // reduce over the row groups: first inside the wave (lanes with the same
    // column group), then across waves through LDS, in a fixed order.
#pragma unroll
    for (int off = CG; off < kWave; off <<= 1)
#pragma unroll
        for (int x = 0; x < 9; ++x) red[x] += __shfl_xor(red[x], off);
    const int wave = tid / kWave, lane = tid % kWave;
    if (lane < CG) {
#pragma unroll
        for (int x = 0; x < 9; ++x) s_red[wave][lane][x] = red[x];
    }
    __syncthreads();
    float tot[9];
#pragma unroll
    for (int x = 0; x < 9; ++x) {
        tot[x] = s_red[0][cg][x];
#pragma unroll
        for (int w = 1; w < NWAVE; ++w) tot[x] += s_red[w][cg][x];
    }
    const float b = beta[unit];
    f32x4 e;
#pragma unroll
    for (int x = 0; x < 4; ++x) e[x] = b * (s_v[4 * cg + x] - tot[x]);
    if (rg == 0) {
#pragma unroll
        for (int x = 0; x < 4; ++x)
            o[vec + 4 * cg + x] = from_f32<E>(tot[4 + x] + tot[8] * e[x]);
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int c = rg + RG * i;
        const float kc = s_k[c];
        f32x4 nv = st[i] + kc * e;                   // S = S' + k e^T
        __builtin_nontemporal_store(nv, &Sv[c * CG + cg]);
    }
}

// T consecutive tokens of one sequence per (b, h) from the state io.in; the
// state after the last token goes to io.out (which may be the same state:
// commit in place; or another one: the input stays as the snapshot a
// rejected draft is replayed from).  Same layout and per-token arithmetic as decode_kernel,
// with S kept in registers across the tokens: S is read and written once
// for all T tokens.  Three workgroup barriers per token.
template <typename E, int D, int NT>
__global__ __launch_bounds__(NT) void tokens_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const E* __restrict__ z, const float* __restrict__ beta, const float* __restrict__ A,
    float g_min, StateIO io, E* __restrict__ o, int T, int H) {
    constexpr int CG = D / 4;
    constexpr int RG = NT / CG;
    constexpr int RPT = D / RG;
    constexpr int NWAVE = NT / kWave;
    static_assert(NT % CG == 0 && D % RG == 0 && NT >= D && CG <= kWave, "tokens layout");

    __shared__ float s_alpha[D], s_k[D], s_q[D], s_v[D];
    __shared__ float s_red[NWAVE][CG][9];

    const int tid = threadIdx.x;
    const size_t unit = blockIdx.x;    // b * H + h
    const size_t b = unit / (size_t)H;
    const int h = (int)(unit % (size_t)H);
    if (io.skip((int)b)) return;       // uniform over the workgroup
    const GateConsts gc = make_gate(A[h], g_min);
    const int cg = tid % CG, rg = tid / CG;
    const int wave = tid / kWave, lane = tid % kWave;

    const f32x4* Si = reinterpret_cast<const f32x4*>(io.in_at((int)b, h, H, D));
    f32x4* So = reinterpret_cast<f32x4*>(io.out_at((int)b, h, H, D));
    f32x4 st[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) st[i] = __builtin_nontemporal_load(&Si[(rg + RG * i) * CG + cg]);

    for (int t = 0; t < T; ++t) {
        const size_t tok = (b * (size_t)T + t) * (size_t)H + h;   // (b, t, h)
        const size_t vec = tok * (size_t)D;
        if (t > 0) __syncthreads();   // every thread is done with the previous token's vectors
        if (tid < D) {
            s_alpha[tid] = gate_alpha(gc, gate_sigmoid(gc, to_f32(z[vec + tid])));
            s_k[tid] = to_f32(k[vec + tid]);
            s_q[tid] = to_f32(q[vec + tid]);
            s_v[tid] = to_f32(v[vec + tid]);
        }
        __syncthreads();
        float red[9];
#pragma unroll
        for (int x = 0; x < 9; ++x) red[x] = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int c = rg + RG * i;
            const float a = s_alpha[c], kc = s_k[c], qc = s_q[c];
            st[i] *= a;                                  // S' = Diag(a) S
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                red[x] += kc * st[i][x];                 // p = S'^T k
                red[4 + x] += qc * st[i][x];             // r = S'^T q
            }
            red[8] += qc * kc;                           // q . k
        }
#pragma unroll
        for (int off = CG; off < kWave; off <<= 1)
#pragma unroll
            for (int x = 0; x < 9; ++x) red[x] += __shfl_xor(red[x], off);
        if (lane < CG) {
#pragma unroll
            for (int x = 0; x < 9; ++x) s_red[wave][lane][x] = red[x];
        }
        __syncthreads();
        float tot[9];
#pragma unroll
        for (int x = 0; x < 9; ++x) {
            tot[x] = s_red[0][cg][x];
#pragma unroll
            for (int w = 1; w < NWAVE; ++w) tot[x] += s_red[w][cg][x];
        }
        const float bt = beta[tok];
        f32x4 e;
#pragma unroll
        for (int x = 0; x < 4; ++x) e[x] = bt * (s_v[4 * cg + x] - tot[x]);
        if (rg == 0) {
#pragma unroll
            for (int x = 0; x < 4; ++x) o[vec + 4 * cg + x] = from_f32<E>(tot[4 + x] + tot[8] * e[x]);
        }
#pragma unroll
        for (int i = 0; i < RPT; ++i) st[i] += s_k[rg + RG * i] * e;   // S = S' + k e^T
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) __builtin_nontemporal_store(st[i], &So[(rg + RG * i) * CG + cg]);
}

template <typename E, int D, int NT>
static hipError_t launch_tokens_v(const TokensArgs& a, hipStream_t stream) {
    const size_t units = (size_t)a.B * a.H;
    hipLaunchKernelGGL((tokens_kernel<E, D, NT>), dim3((unsigned)units), dim3(NT), 0, stream,
                       (const E*)a.q, (const E*)a.k, (const E*)a.v, (const E*)a.z, a.beta, a.A,
                       a.g_min, a.S, (E*)a.o, a.T, a.H);
    return hipGetLastError();
}

template <typename E, int D>
static hipError_t launch_tokens_t(const TokensArgs& a, hipStream_t stream) {
    if constexpr (D == 32) {
        return launch_tokens_v<E, D, 2 * D>(a, stream);
    } else {
        // 512 threads (as the single-token step) was 8-10% slower here: the
        // per-token barriers span twice the waves.
        return launch_tokens_v<E, D, 2 * D>(a, stream);
    }
}

hipError_t launch_tokens(const TokensArgs& a, hipStream_t stream) {
    if (a.is_bf16) {
        return a.d == 128 ? launch_tokens_t<bf16, 128>(a, stream) : launch_tokens_t<bf16, 32>(a, stream);
    }
    return a.d == 128 ? launch_tokens_t<float, 128>(a, stream) : launch_tokens_t<float, 32>(a, stream);
}

template <typename E, int D, int NT>
static hipError_t launch_decode_v(const DecodeArgs& a, hipStream_t stream) {
    const size_t units = (size_t)a.B * a.H;
    hipLaunchKernelGGL((decode_kernel<E, D, NT>), dim3((unsigned)units),
                       dim3(NT), 0, stream, (const E*)a.q, (const E*)a.k, (const E*)a.v,
                       (const E*)a.z, a.beta, a.A, a.g_min, a.S, (E*)a.o, a.H);
    return hipGetLastError();
}

// d = 128: 512 threads of 8 rows each (68 VGPRs, seven waves per SIMD);
// d = 32: 64 threads.
template <typename E, int D>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
    if constexpr (D == 32)
        return launch_decode_v<E, D, 2 * D>(a, stream);
    else
        return launch_decode_v<E, D, 4 * D>(a, stream);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    if (a.is_bf16) {
        return a.d == 128 ? launch_decode_t<bf16, 128>(a, stream) : launch_decode_t<bf16, 32>(a, stream);
    }
    return a.d == 128 ? launch_decode_t<float, 128>(a, stream) : launch_decode_t<float, 32>(a, stream);
}

}  // namespace kda
