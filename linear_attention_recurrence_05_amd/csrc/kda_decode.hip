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
// workgroup per U units (b, h); each thread owns 4 adjacent value columns of
// RPT key rows of every unit (8 for d = 128, over 512 threads), so every wave
// instruction moves 1 KiB (d = 128) of S with 16-byte accesses.  S is held in
// registers between the read and the write, the two reductions come from the
// same read, and the update is written back with non-temporal stores.  At d =
// 128 a workgroup takes two units (104 VGPRs, two workgroups per CU): twice
// the bytes in flight per workgroup of one unit, and 8,192 units make exactly
// eight rounds of 512 workgroup slots -- 0.180 against 0.190 ms per step at
// B = 256, H = 32.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <typename E, int D, int NT, int U>
__global__ __launch_bounds__(NT) void decode_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const E* __restrict__ z, const float* __restrict__ beta, const float* __restrict__ A,
    float g_min, StateIO io, E* __restrict__ o, int H, int units) {
    constexpr int CG = D / 4;          // column groups of 4 (float4)
    constexpr int RG = NT / CG;        // row groups
    constexpr int RPT = D / RG;        // rows per thread
    constexpr int NWAVE = NT / kWave;
    static_assert(NT % CG == 0 && D % RG == 0 && CG <= kWave, "decode layout");

    __shared__ float s_alpha[U][D], s_k[U][D], s_q[U][D], s_v[U][D];
    __shared__ float s_red[U][NWAVE][CG][9];

    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;
    const int wave = tid / kWave, lane = tid % kWave;
    // Unit u of the workgroup and its (b, h); a unit past the last one reads
    // unit 0's vectors (and, below, a live unit's state) and stores nothing.
    size_t unit[U], soff[U];           // soff: element offset of the unit's state in io.out
    int bb[U], hh[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        unit[u] = (size_t)blockIdx.x * U + u;
        const size_t un = unit[u] < (size_t)units ? unit[u] : 0;
        bb[u] = (int)(un / (size_t)H);
        hh[u] = (int)(un % (size_t)H);
        const size_t vec = un * (size_t)D;
        const GateConsts gc = make_gate(A[hh[u]], g_min);
        for (int c = tid; c < D; c += NT) {
            s_alpha[u][c] = gate_alpha(gc, gate_sigmoid(gc, to_f32(z[vec + c])));
            s_k[u][c] = to_f32(k[vec + c]);
            s_q[u][c] = to_f32(q[vec + c]);
            s_v[u][c] = to_f32(v[vec + c]);
        }
    }
    // The unit's state: the slot is read once (for paged states the skip test
    // and the address share it).  Past the last unit, or at a skipped slot,
    // the unit is absent (uniform over the workgroup); an absent unit takes
    // the first live unit's state for its loads, so the loads of all units
    // issue without branches around them.
    bool live[U];
    int first = -1;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int so = io.out_slot ? io.out_slot[bb[u]] : bb[u];
        bool skip = io.ck_out && (unsigned)so >= (unsigned)io.n_slots;
        if (io.ck_in) {
            const int si = io.ck_in == io.out_slot ? so : io.ck_in[bb[u]];
            skip = skip || (unsigned)si >= (unsigned)io.n_slots;
        }
        live[u] = unit[u] < (size_t)units && !skip;
        soff[u] = ((size_t)so * H + hh[u]) * (size_t)D * D;   // in place: in == out
        if (live[u] && first < 0) first = u;
    }
    if (first < 0) return;             // uniform over the workgroup
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (!live[u]) soff[u] = soff[first];
    __syncthreads();
    f32x4 st[U][RPT];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            st[u][i] = __builtin_nontemporal_load(
                &reinterpret_cast<const f32x4*>(io.out + soff[u])[(rg + RG * i) * CG + cg]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float red[9];
#pragma unroll
        for (int x = 0; x < 9; ++x) red[x] = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int c = rg + RG * i;
            const float a = s_alpha[u][c], kc = s_k[u][c], qc = s_q[u][c];
            st[u][i] *= a;                               // S' = Diag(a) S
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                red[x] += kc * st[u][i][x];              // p = S'^T k
                red[4 + x] += qc * st[u][i][x];          // r = S'^T q
            }
            red[8] += qc * kc;                           // q . k (same in every column group)
        }
        // reduce over the row groups: first inside the wave (lanes with the
        // same column group), then across waves through LDS, in a fixed order
#pragma unroll
        for (int off = CG; off < kWave; off <<= 1)
#pragma unroll
            for (int x = 0; x < 9; ++x) red[x] += __shfl_xor(red[x], off);
        if (lane < CG) {
#pragma unroll
            for (int x = 0; x < 9; ++x) s_red[u][wave][lane][x] = red[x];
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (!live[u]) continue;        // uniform over the workgroup
        const size_t vec = unit[u] * (size_t)D;
        float tot[9];
#pragma unroll
        for (int x = 0; x < 9; ++x) {
            tot[x] = s_red[u][0][cg][x];
#pragma unroll
            for (int w = 1; w < NWAVE; ++w) tot[x] += s_red[u][w][cg][x];
        }
        const float b = beta[unit[u]];
        f32x4 e;
#pragma unroll
        for (int x = 0; x < 4; ++x) e[x] = b * (s_v[u][4 * cg + x] - tot[x]);
        if (rg == 0) {
#pragma unroll
            for (int x = 0; x < 4; ++x)
                o[vec + 4 * cg + x] = from_f32<E>(tot[4 + x] + tot[8] * e[x]);
        }
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int c = rg + RG * i;
            const float kc = s_k[u][c];
            f32x4 nv = st[u][i] + kc * e;                // S = S' + k e^T
            __builtin_nontemporal_store(nv, &reinterpret_cast<f32x4*>(io.out + soff[u])[c * CG + cg]);
        }
    }
}

template <typename E, int D, int NT, int U>
static hipError_t launch_decode_v(const DecodeArgs& a, hipStream_t stream) {
    const size_t units = (size_t)a.B * a.H;
    hipLaunchKernelGGL((decode_kernel<E, D, NT, U>), dim3((unsigned)((units + U - 1) / U)),
                       dim3(NT), 0, stream, (const E*)a.q, (const E*)a.k, (const E*)a.v,
                       (const E*)a.z, a.beta, a.A, a.g_min, a.S, (E*)a.o, a.H, (int)units);
    return hipGetLastError();
}

// d = 128: 512 threads of 8 rows each, two units per workgroup; d = 32: 64
// threads, one unit.
template <typename E, int D>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
    if constexpr (D == 32)
        return launch_decode_v<E, D, 2 * D, 1>(a, stream);
    else
        return launch_decode_v<E, D, 4 * D, 2>(a, stream);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    if (a.is_bf16) {
        return a.d == 128 ? launch_decode_t<bf16, 128>(a, stream) : launch_decode_t<bf16, 32>(a, stream);
    }
    return a.d == 128 ? launch_decode_t<float, 128>(a, stream) : launch_decode_t<float, 32>(a, stream);
}

}  // namespace kda
