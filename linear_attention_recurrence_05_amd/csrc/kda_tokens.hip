// kda_tokens.hip -- the multi-token step for gfx950: T consecutive decode
// steps of every (b, h) from one state, S held in registers across the
// tokens, so that S is read and written once for all T tokens.
//
// Per token, the recurrence of one decode step (dev.to "Kimi K3 Architecture
// ...", "The Sequence Bottleneck": state shape, retention/delta domains and
// the gate equation; terrencekim.net "Kimi K3 - Sparsity Mechanics ...",
// section 2: fixed-size state, constant decode memory):
//   S' = Diag(a) S,  e = beta (v - S'^T k),  S <- S' + k e^T,  o = S^T q.
// The state comes from io.in and goes to io.out, which may be the same
// state (commit in place) or another one (the input stays as the snapshot a
// rejected draft is replayed from).  Compiled apart from the single-token
// step: the two kernels want different machine schedulers.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

// T consecutive tokens of one sequence per (b, h) from the state io.in; the
// state after the last token goes to io.out (which may be the same state:
// commit in place; or another one: the input stays as the snapshot a
// rejected draft is replayed from).  Same layout and per-token arithmetic as decode_kernel,
// with S kept in registers across the tokens: S is read and written once
// for all T tokens.  Three workgroup barriers per token.  The d = 32 step
// (64 threads, one unit per workgroup); d = 128 runs tokens_cols_kernel.
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

// The multi-token step at d = 128: U units per workgroup of NT threads, the
// units on separate waves, and within a unit the value columns split over
// its waves: wave w of a unit holds D / (NT / U / 64) columns of all D key
// rows (lane l: 4 columns of D / 8 rows at d = 128, 512 threads, two units),
// so the sums over key rows stay inside the wave (shuffles over its 8 row
// groups) and a token needs no workgroup barrier.  The vectors of TG tokens
// of every unit are staged in LDS at a time, two barriers per group.  At B =
// 256, H = 32, T = 4: 0.188 ms against 0.197-0.200 ms for tokens_kernel
// with 256 threads per unit (whose cross-wave sums cost three barriers per
// token), and 0.190 ms with the units' rows interleaved over all 8 waves as
// in decode_kernel (whose cross-wave sums cost two barriers per token).
template <typename E, int D, int NT, int U>
__global__ __launch_bounds__(NT) void tokens_cols_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const E* __restrict__ z, const float* __restrict__ beta, const float* __restrict__ A,
    float g_min, StateIO io, E* __restrict__ o, int T, int H, int units) {
    constexpr int NTU = NT / U;        // threads of one unit
    constexpr int NWU = NTU / kWave;   // waves of one unit
    constexpr int CW = D / NWU;        // columns of one wave
    constexpr int CGW = CW / 4;        // column groups of one wave
    constexpr int RGW = kWave / CGW;   // row groups of one wave
    constexpr int RPT = D / RGW;
    constexpr int CG = D / 4;
    static_assert(NTU % kWave == 0 && D % NWU == 0 && kWave % CGW == 0 && D % RGW == 0, "tokens layout");
    constexpr int TG = 4;
    constexpr int TD = TG * D;
    __shared__ float s_vec[U * 4 * TD];   // [U][4][TG][D]: alpha, k, q, v

    const int tid = threadIdx.x;
    const int me = tid / NTU;          // this thread's unit (uniform over a wave)
    const int wu = (tid % NTU) / kWave, lane = tid % kWave;
    const int cg = wu * CGW + lane % CGW, rg = lane / CGW;
    size_t unit[U];
    int bb[U], hh[U];
    bool live[U];
    int first = -1;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        unit[u] = (size_t)blockIdx.x * U + u;
        const size_t un = unit[u] < (size_t)units ? unit[u] : 0;
        bb[u] = (int)(un / (size_t)H);
        hh[u] = (int)(un % (size_t)H);
        live[u] = unit[u] < (size_t)units && !io.skip(bb[u]);
        if (live[u] && first < 0) first = u;
    }
    if (first < 0) return;             // uniform over the workgroup
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (!live[u]) { bb[u] = bb[first]; hh[u] = hh[first]; }
    int mb = __builtin_amdgcn_readfirstlane(bb[0]), mh = __builtin_amdgcn_readfirstlane(hh[0]);
    bool mlive = live[0];
#pragma unroll
    for (int u = 1; u < U; ++u)
        if (me == u) { mb = bb[u]; mh = hh[u]; mlive = live[u]; }
    mb = __builtin_amdgcn_readfirstlane(mb);
    mh = __builtin_amdgcn_readfirstlane(mh);
    f32x4 st[RPT];
    for (int t0 = 0; t0 < T; t0 += TG) {
        const int tn = min(TG, T - t0);
        if (t0 > 0) __syncthreads();   // every thread is done with the previous group
        for (int x = tid; x < U * tn * D; x += NT) {
            const int u = x / (tn * D), t = (x / D) % tn, c = x % D;
            int uu = 0;
#pragma unroll
            for (int w = 1; w < U; ++w) uu = u == w ? w : uu;
            const GateConsts gc = make_gate(A[hh[uu]], g_min);
            const size_t vec = (((size_t)bb[uu] * T + t0 + t) * H + hh[uu]) * (size_t)D + c;
            float* sv = s_vec + u * 4 * TD + t * D + c;
            sv[0] = gate_alpha(gc, gate_sigmoid(gc, to_f32(z[vec])));
            sv[TD] = to_f32(k[vec]);
            sv[2 * TD] = to_f32(q[vec]);
            sv[3 * TD] = to_f32(v[vec]);
        }
        __syncthreads();
        if (t0 == 0) {
            const f32x4* Si = reinterpret_cast<const f32x4*>(io.in_at(mb, mh, H, D));
#pragma unroll
            for (int i = 0; i < RPT; ++i) st[i] = __builtin_nontemporal_load(&Si[(rg + RGW * i) * CG + cg]);
        }
        for (int tt = 0; tt < tn; ++tt) {
            const int t = t0 + tt;
            const float* sa = s_vec + me * 4 * TD + tt * D;
            float red[9];
#pragma unroll
            for (int x = 0; x < 9; ++x) red[x] = 0.f;
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int c = rg + RGW * i;
                const float a = sa[c], kc = sa[TD + c], qc = sa[2 * TD + c];
                st[i] *= a;                                  // S' = Diag(a) S
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    red[x] += kc * st[i][x];                 // p = S'^T k
                    red[4 + x] += qc * st[i][x];             // r = S'^T q
                }
                red[8] += qc * kc;                           // q . k
            }
            // over the row groups of the wave (lanes with the same column group)
#pragma unroll
            for (int off = CGW; off < kWave; off <<= 1)
#pragma unroll
                for (int x = 0; x < 9; ++x) red[x] += __shfl_xor(red[x], off);
            const size_t tok = ((size_t)mb * T + t) * H + mh;
            const float bt = beta[tok];
            f32x4 e;
#pragma unroll
            for (int x = 0; x < 4; ++x) e[x] = bt * (sa[3 * TD + 4 * cg + x] - red[x]);
            if (rg == 0 && mlive) {
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    o[tok * D + 4 * cg + x] = from_f32<E>(red[4 + x] + red[8] * e[x]);
            }
#pragma unroll
            for (int i = 0; i < RPT; ++i) st[i] += sa[TD + rg + RGW * i] * e;   // S = S' + k e^T
        }
    }
    if (mlive) {
        f32x4* So = reinterpret_cast<f32x4*>(io.out_at(mb, mh, H, D));
#pragma unroll
        for (int i = 0; i < RPT; ++i) __builtin_nontemporal_store(st[i], &So[(rg + RGW * i) * CG + cg]);
    }
}

template <typename E, int D, int NT, int U>
static hipError_t launch_tokens_cols(const TokensArgs& a, hipStream_t stream) {
    const size_t units = (size_t)a.B * a.H;
    hipLaunchKernelGGL((tokens_cols_kernel<E, D, NT, U>), dim3((unsigned)((units + U - 1) / U)),
                       dim3(NT), 0, stream, (const E*)a.q, (const E*)a.k, (const E*)a.v,
                       (const E*)a.z, a.beta, a.A, a.g_min, a.S, (E*)a.o, a.T, a.H, (int)units);
    return hipGetLastError();
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
    if constexpr (D == 32)
        return launch_tokens_v<E, D, 2 * D>(a, stream);
    else
        return launch_tokens_cols<E, D, 4 * D, 2>(a, stream);
}

hipError_t launch_tokens(const TokensArgs& a, hipStream_t stream) {
    if (a.is_bf16) {
        return a.d == 128 ? launch_tokens_t<bf16, 128>(a, stream) : launch_tokens_t<bf16, 32>(a, stream);
    }
    return a.d == 128 ? launch_tokens_t<float, 128>(a, stream) : launch_tokens_t<float, 32>(a, stream);
}

}  // namespace kda
