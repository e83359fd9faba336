// kda_prefill.hip -- chunkwise KDA prefill kernels for gfx950 and the plans
// that compose them (the device building blocks are in kda_chunk.hpp).
//
// Source of the method: dev.to "Kimi K3 Architecture: Scaling 2.8T Parameters
// for Long-Context Multimodal MoE", section "The Sequence Bottleneck: Hybrid
// KDA and Gated MLA": chunkwise parallel execution of the gated delta rule
// over 16-token tiles, with the within-chunk ("diagonal") and state
// ("off-diagonal") parts as dense matrix products.
//
// Kernels:
//   gate_cumsum_kernel / intra_kernel<DIAG>: diagnostic exports of the gate
//       and intra-chunk stages (the same device code the prefill runs).
//   fused_kernel: one workgroup per (b, h, column tile); four producer waves
//       fill one half of a double-buffered LDS ring of factor blocks while
//       the consumer waves run the state chain over the other half.
//   split plan (kda_pair.hip): an intra kernel writes two-chunk factor
//       blocks to a workspace, an inter kernel streams them through an LDS
//       ring to the state chains.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "kda_chunk.hpp"
#include "kda_launch.hpp"

namespace kda {

// --------------------------------------------------------------- kernels

// Gate stage alone (diagnostic): G = chunk-local inclusive cumsum of g.
template <typename E, int D>
__global__ __launch_bounds__(256) void gate_cumsum_kernel(const E* __restrict__ z,
                                                          const float* __restrict__ A, float g_min,
                                                          float* __restrict__ G, int B, int T,
                                                          int H) {
    const int NC = (T + kChunk - 1) / kChunk;
    const size_t total = (size_t)B * NC * H * D;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const int c = (int)(idx % D);
        size_t rest = idx / D;
        const int h = (int)(rest % H);
        rest /= H;
        const int n = (int)(rest % NC);
        const int b = (int)(rest / NC);
        const GateConsts gc = make_gate(A[h], g_min);
        const int t0 = n * kChunk, L = min(kChunk, T - t0);
        float run = 0.f;
        for (int r = 0; r < L; ++r) {
            const size_t i = (((size_t)b * T + t0 + r) * H + h) * D + c;
            run += gc.gmin * gate_sigmoid(gc, to_f32(z[i]));
            G[i] = run;
        }
    }
}

// Intra kernel (split plan and diagnostic export): wave w of workgroup x
// produces chunk 4x + w of the [B*H][n_count] chunk grid starting at chunk
// n_first of every sequence.
template <typename E, int D, bool DIAG>
__global__ __launch_bounds__(256) void intra_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                    const E* __restrict__ z,
                                                    const float* __restrict__ beta,
                                                    const float* __restrict__ A, float g_min,
                                                    char* __restrict__ ws, int B, int T, int H,
                                                    int n_first, int n_count, float* dTm,
                                                    float* dAqk, float* dgam) {
    using Bk = Blk<E, D>;
    __shared__ __attribute__((aligned(16))) char smem[4 * (Bk::BYTES + Bk::SCR_BYTES)];
    const int w = wave_id();
    const size_t id = (size_t)blockIdx.x * 4 + w;
    const size_t total = (size_t)B * H * n_count;
    if (id >= total) return;   // whole wave; no workgroup barrier below
    const int nl = (int)(id % n_count);
    const int u = (int)(id / n_count);
    const int b = u / H, h = u % H;
    const int n = n_first + nl;
    char* blk = smem + w * (Bk::BYTES + Bk::SCR_BYTES);
    char* scr = blk + Bk::BYTES;

    ProdIn<E, D> in;
    prod_load<E, D>(in, q, k, z, beta, chunk_pos<D>(b, h, n, T, H));
    if constexpr (DIAG) {
        const int NC = (T + kChunk - 1) / kChunk;
        const size_t cidx = (size_t)u * NC + n;
        dTm += cidx * 256;
        dAqk += cidx * 256;
        dgam += cidx * D;
    }
    prod_compute<E, D, DIAG>(in, make_gate(A[h], g_min), blk, scr, dTm, dAqk, dgam);
    if (ws) {
        const uint4* src = reinterpret_cast<const uint4*>(blk);
        uint4* dst = reinterpret_cast<uint4*>(ws + id * (size_t)Bk::BYTES);
#pragma unroll 4
        for (int x = lane_id(); x < Bk::BYTES / 16; x += kWave) dst[x] = src[x];
    }
}

// Producer waves per fused workgroup: 4, unless the double-buffered ring of
// 8 factor blocks would not fit the 160 KiB of LDS.
template <typename E, int D>
struct FusedCfg {
    using Bk = Blk<E, D>;
    static constexpr int NPROD = (8 * Bk::BYTES + 4 * Bk::SCR_BYTES <= 160 * 1024) ? 4 : 2;
    static constexpr int RING = 2 * NPROD * Bk::BYTES;
    static constexpr int LDS = RING + NPROD * Bk::SCR_BYTES;
};

// Fused kernel: one workgroup of 8 waves per (b, h, column tile of
// NCW*NB*16 columns).  Waves 0..NPROD-1 produce; waves 4..4+NCW-1 consume.
// Step m: the producers fill ring half (m+1)&1 with the next NPROD chunks
// while the consumers run the state chain over half m&1.  Each role runs its
// own loop (so neither keeps the other's registers live); both execute
// 1 + NM barriers.  WQ = false: only the end state (q and o are not
// touched); VZ: v is taken as zero (v is not read); CK: the state at the
// start of every chunk is stored too (ck, the checkpoints of a backward).
// lim.in limits unit u to its first lim.in[u] chunks.  EX (state-only, v =
// 0): the pass stops after the first step at whose end the state of every
// consumer is exactly zero -- with v = 0 a zero state stays zero, so the end
// state is the same -- and lim.out[u] receives the number of chunks
// processed.
template <typename E, int D, int NB, int NCW, bool WQ = true, bool VZ = false, bool CK = false,
          bool EX = false>
__global__ __launch_bounds__(512) void fused_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                    const E* __restrict__ v, const E* __restrict__ z,
                                                    const float* __restrict__ beta,
                                                    const float* __restrict__ A, float g_min,
                                                    StateIO io, E* __restrict__ o,
                                                    int B, int T, int H, int nct,
                                                    CkOut ck = CkOut{}, ChunkLim lim = ChunkLim{}) {
    using Bk = Blk<E, D>;
    using Cfg = FusedCfg<E, D>;
    constexpr int NPROD = Cfg::NPROD;
    static_assert(!EX || (VZ && !WQ && NCW <= 4), "early exit: state-only passes with v = 0");
    __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS];
    // EX: per consumer wave, whether its state was zero at the end of step m
    // (slot m & 1: a slot is rewritten two steps later, after every wave has
    // passed the barrier between)
    __shared__ int zflag[2][4];
    int u, ct;
    if (!map_unit(nct, B * H, u, ct)) return;   // uniform over the workgroup
    const int b = u / H, h = u % H;
    if (io.skip(b)) return;                      // uniform over the workgroup
    const int w = wave_id();
    const int NCA = (T + kChunk - 1) / kChunk;
    const int NC = lim.in ? max(0, min(NCA, lim.in[u])) : NCA;   // uniform over the workgroup
    const int NM = (NC + NPROD - 1) / NPROD;
    auto all_zero = [&](int m) {
        bool z0 = true;
#pragma unroll
        for (int x = 0; x < NCW; ++x) z0 = z0 && zflag[m & 1][x] != 0;
        return z0;
    };

    if (w < NPROD) {
        // ------------------------------------------------ producer wave
        char* myscr = smem + Cfg::RING + w * Bk::SCR_BYTES;
        const GateConsts gc = make_gate(A[h], g_min);
        ProdIn<E, D> cur, nxt;
        cur.L = 0;
        nxt.L = 0;
        if (w < NC) prod_load<E, D, WQ>(cur, q, k, z, beta, chunk_pos<D>(b, h, w, T, H));
        if (NPROD + w < NC)
            prod_load<E, D, WQ>(nxt, q, k, z, beta, chunk_pos<D>(b, h, NPROD + w, T, H));
        if (cur.L > 0)
            prod_compute<E, D, false, WQ>(cur, gc, smem + w * Bk::BYTES, myscr, nullptr, nullptr,
                                          nullptr);
        wg_barrier();
        for (int m = 0; m < NM; ++m) {
            cur = nxt;
            nxt.L = 0;
            const int n_next = (m + 2) * NPROD + w;
            if (n_next < NC)
                prod_load<E, D, WQ>(nxt, q, k, z, beta, chunk_pos<D>(b, h, n_next, T, H));
            if (cur.L > 0)
                prod_compute<E, D, false, WQ>(cur, gc,
                                              smem + (((m + 1) & 1) * NPROD + w) * Bk::BYTES,
                                              myscr, nullptr, nullptr, nullptr);
            wg_barrier();
            if constexpr (EX) {
                if (all_zero(m)) break;
            }
        }
        return;
    }
    const int cw = w - 4;
    if (cw < 0 || cw >= NCW) {
        // ------------------------------------------------ idle wave
        wg_barrier();
        for (int m = 0; m < NM; ++m) {
            wg_barrier();
            if constexpr (EX) {
                if (all_zero(m)) break;
            }
        }
        return;
    }
    // ---------------------------------------------------- consumer wave
    // bf16, NB = 2: the two blocks interleave (block nb, lane column j =
    // column col0 + 2 j + nb), so V, O and the states move as column pairs.
    // (fp32 keeps separate blocks: built interleaved, its output stores came
    // out wrong -- the compiler stored row 4g's value for all four rows.)
    constexpr bool IL = NB == 2 && std::is_same<E, bf16>::value;
    const int col0 = ct * (NCW * NB * 16) + cw * NB * 16;
    f32x4 S[NB][D / 16];
    constexpr int ES = (int)sizeof(E);
    struct VBlocks {
        u32x4 x[NB];
    };
    using VRaw = typename std::conditional<IL, VPair, VBlocks>::type;
    VRaw Vc[NPROD], Vn[NPROD];
    auto vload = [&](VRaw& V, int n) {
        if constexpr (IL) v_load_il<D>(V, (const bf16*)v, chunk_pos<D>(b, h, n, T, H), col0);
        else v_load<D, NB>(V.x, v, ES, chunk_pos<D>(b, h, n, T, H), col0);
    };
    if constexpr (IL) state_load_il<D>(S, io.in_at(b, h, H, D), col0);
    else state_load<D, NB>(S, io.in_at(b, h, H, D), col0);
    if constexpr (!VZ) {
#pragma unroll
        for (int cc = 0; cc < NPROD; ++cc)
            if (cc < NC) vload(Vc[cc], cc);
    }
    wg_barrier();
    [[maybe_unused]] int done = NC;
    for (int m = 0; m < NM; ++m) {
        if constexpr (!VZ) {
#pragma unroll
            for (int cc = 0; cc < NPROD; ++cc) {
                const int nn = (m + 1) * NPROD + cc;
                if (nn < NC) vload(Vn[cc], nn);
            }
        }
#pragma unroll
        for (int cc = 0; cc < NPROD; ++cc) {
            const int n = m * NPROD + cc;
            if (n < NC) {
                COps<E, D> c;
                cops_load<E, D, LdsSrc, WQ>(c, LdsSrc{smem + ((m & 1) * NPROD + cc) * Bk::BYTES});
                f32x4 O[NB];
                f32x4 Vf[NB];
                if constexpr (VZ) {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) Vf[nb] = zero4();
                } else if constexpr (IL) {
                    v_widen_il(Vc[cc], Vf);
                } else {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) Vf[nb] = v_widen<E>(Vc[cc].x[nb]);
                }
                if constexpr (CK) {
                    // the state entering chunk n, natural [D][D] layout
                    float* cp = ck.at<D>(b, h, n, H);
                    if constexpr (IL) {
                        state_store_il<D>(S, cp, col0);
                    } else {
                        const int lane = lane_id(), j = lane & 15, g = lane >> 4;
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                            for (int mm = 0; mm < D / 16; ++mm)
#pragma unroll
                                for (int p = 0; p < 4; ++p)
                                    cp[(size_t)(16 * mm + 4 * g + p) * D + col0 + 16 * nb + j] =
                                        S[nb][mm][p];
                    }
                }
                chunk_step<E, D, NB, WQ>(c, S, Vf, O);
                if constexpr (WQ) {
                    if constexpr (IL) o_store_il<D>(O, (bf16*)o, chunk_pos<D>(b, h, n, T, H), col0);
                    else o_store<E, D, NB>(O, o, chunk_pos<D>(b, h, n, T, H), col0);
                }
            }
        }
        if constexpr (!VZ) {
#pragma unroll
            for (int cc = 0; cc < NPROD; ++cc) Vc[cc] = Vn[cc];
        }
        if constexpr (EX) {
            // exactly zero: every bit but the sign clear (-0 counts as zero)
            uint32_t bits = 0u;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int mm = 0; mm < D / 16; ++mm)
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        bits |= __builtin_bit_cast(uint32_t, S[nb][mm][p]) & 0x7FFFFFFFu;
            const bool wz = !__any(bits != 0u);
            if (lane_id() == 0) zflag[m & 1][cw] = wz ? 1 : 0;
        }
        wg_barrier();
        if constexpr (EX) {
            if (all_zero(m)) {
                done = min(NC, (m + 1) * NPROD);
                break;
            }
        }
    }
    if constexpr (EX) {
        if (cw == 0 && lane_id() == 0) lim.out[u] = done;
    }
    if (io.out) {
        if constexpr (IL) state_store_il<D>(S, io.out_at(b, h, H, D), col0);
        else state_store<D, NB>(S, io.out_at(b, h, H, D), col0);
    }
}

// --------------------------------------------------------------- plans / launchers


// Plan override for tests and tuning: KDA_PREFILL_PLAN = "fused:<ncol>"
// (ncol in {16, 32, 64, 128}, at most d), "split", "split:<ncol>:<nb>" or
// "ring" (where it runs).  Unset or anything else: chosen from the sizes.
static bool plan_override(int B, int H, int d, bool is_bf16, PlanInfo& p) {
    const char* env = std::getenv("KDA_PREFILL_PLAN");
    if (!env) return false;
    if (std::strcmp(env, "split") == 0) {
        p.plan = Plan::kSplit;
        return true;
    }
    if (std::strcmp(env, "ring") == 0 && ring_ok(B, H, d, is_bf16)) {
        p.plan = Plan::kRing;
        p.ncol = 16;
        p.ws_bytes = ring_ws_bytes(B, H, d, is_bf16);
        return true;
    }
    if (std::strncmp(env, "split:", 6) == 0) {
        int ncol = 0, nb = 0;
        if (std::sscanf(env + 6, "%d:%d", &ncol, &nb) == 2 && pair_variant_ok(d, is_bf16, ncol, nb)) {
            p.plan = Plan::kSplit;
            p.ncol = ncol;
            p.nb = nb;
            return true;
        }
        return false;
    }
    if (std::strncmp(env, "fused:", 6) == 0) {
        const int n = std::atoi(env + 6);
        if ((n == 16 || n == 32 || n == 64 || n == 128) && n <= d) {
            p.plan = Plan::kFused;
            p.ncol = n;
            p.ws_bytes = 0;
            return true;
        }
    }
    return false;
}

PlanInfo choose_plan(int B, int T, int H, int d, bool is_bf16) {
    PlanInfo p;
    const long units = (long)B * H;
    const int NC = (T + kChunk - 1) / kChunk;
    p.plan = Plan::kSplit;
    p.ncol = 0;
    p.nb = 1;
    const bool forced = plan_override(B, H, d, is_bf16, p);
    if (forced && (p.plan == Plan::kFused || p.plan == Plan::kRing)) return p;
    if (!forced && ring_ok(B, H, d, is_bf16)) {
        // few sequence-heads: every unit gets a CU per 16-column tile and
        // its pair blocks pass from producers to chains through L2
        p.plan = Plan::kRing;
        p.ncol = 16;
        p.ws_bytes = ring_ws_bytes(B, H, d, is_bf16);
        return p;
    }
    if (!forced && units >= 128) {
        p.plan = Plan::kFused;
        p.ncol = units >= 256 ? d : (d >= 64 ? 64 : d);
        p.ws_bytes = 0;
        return p;
    }
    p.plan = Plan::kSplit;
    if (p.ncol == 0) {
        // default inter variant: one state chain per workgroup (a CU to
        // itself) while all chains fit on the chip's 256 CUs at once, else
        // four chains (two for fp32) sharing each workgroup's factor stream
        const long chains = units * (d / 16);
        p.ncol = chains <= 256 ? 16 : (is_bf16 && d >= 64 ? 64 : 32);
        p.nb = 1;
    }
    const int seg = NC < kSegChunks ? NC : kSegChunks;
    p.ws_bytes = (size_t)units * ((seg + 1) / 2) * pair_block_bytes(d, is_bf16);
    if (NC > kSegChunks) p.ws_bytes += (size_t)units * d * d * sizeof(float);
    return p;
}

static unsigned grid_units(int units, int nct) {
    return (unsigned)(((units + 7) / 8) * 8 * nct);
}

template <typename E, int D>
static hipError_t launch_prefill_t(const PrefillArgs& a, const PlanInfo& p, void* ws,
                                   hipStream_t stream) {
    const int units = a.B * a.H;
    const int NC = (a.T + kChunk - 1) / kChunk;
    const E* q = (const E*)a.q;
    const E* k = (const E*)a.k;
    const E* v = (const E*)a.v;
    const E* z = (const E*)a.z;
    E* o = (E*)a.o;
    if (p.plan == Plan::kFused) {
        const int nct = D / p.ncol;
        const dim3 grid(grid_units(units, nct)), block(512);
        const CkOut nock{};
        if (!o || !v) {
            // state-only passes (o null; v null = zero), d = 128 with 128 or
            // 64 columns per workgroup (prefill_state_only_ok); a null v
            // with outputs is not a pass any caller makes; the early exit
            // (lim.out) only for v = 0
            if (D != 128 || o != nullptr || (p.ncol != 128 && p.ncol != 64) || (v && a.lim.out))
                return hipErrorInvalidValue;
#define KDA_FUSED_SO(NB, VZ, EX)                                                                  \
    hipLaunchKernelGGL((fused_kernel<E, D, NB, 4, false, VZ, false, EX>), grid, block, 0, stream, q, \
                       k, v, z, a.beta, a.A, a.g_min, a.S, o, a.B, a.T, a.H, nct, nock, a.lim)
            if (p.ncol == 128) {
                if (v) KDA_FUSED_SO(2, false, false);
                else if (a.lim.out) KDA_FUSED_SO(2, true, true);
                else KDA_FUSED_SO(2, true, false);
            } else {
                if (v) KDA_FUSED_SO(1, false, false);
                else if (a.lim.out) KDA_FUSED_SO(1, true, true);
                else KDA_FUSED_SO(1, true, false);
            }
#undef KDA_FUSED_SO
            return hipGetLastError();
        }
        if (a.lim.out) return hipErrorInvalidValue;
#define KDA_FUSED(NB, NCW)                                                                        \
    hipLaunchKernelGGL((fused_kernel<E, D, NB, NCW>), grid, block, 0, stream, q, k, v, z, a.beta,  \
                       a.A, a.g_min, a.S, o, a.B, a.T, a.H, nct, nock, a.lim)
        if (p.ncol == 128 && D == 128) KDA_FUSED(2, 4);
        else if (p.ncol == 64 && D == 128) KDA_FUSED(1, 4);
        else if (p.ncol == 32) KDA_FUSED(1, 2);
        else KDA_FUSED(1, 1);
#undef KDA_FUSED
        return hipGetLastError();
    }
    (void)ws;
    return hipErrorInvalidValue;   // the split plan runs through launch_split
}

hipError_t launch_ckpt_pass(const PrefillArgs& a, const CkOut& ck, hipStream_t stream) {
    if (!a.is_bf16 || a.d != 128) return hipErrorInvalidValue;
    const int units = a.B * a.H;
    hipLaunchKernelGGL((fused_kernel<bf16, 128, 2, 4, false, false, true>),
                       dim3(grid_units(units, 1)), dim3(512), 0, stream, (const bf16*)a.q,
                       (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.z, a.beta, a.A, a.g_min,
                       a.S, (bf16*)nullptr, a.B, a.T, a.H, 1, ck);
    return hipGetLastError();
}

bool prefill_state_only_ok(const PlanInfo& p, int d) {
    return p.plan == Plan::kFused && d == 128 && (p.ncol == 128 || p.ncol == 64);
}

hipError_t launch_prefill(const PrefillArgs& a, const PlanInfo& p, void* ws, hipStream_t stream) {
    if (p.plan == Plan::kSplit) return launch_split(a, p, ws, stream);
    if (p.plan == Plan::kRing) return launch_ring(a, ws, stream);
    if (a.is_bf16)
        return a.d == 128 ? launch_prefill_t<bf16, 128>(a, p, ws, stream)
                          : launch_prefill_t<bf16, 32>(a, p, ws, stream);
    return a.d == 128 ? launch_prefill_t<float, 128>(a, p, ws, stream)
                      : launch_prefill_t<float, 32>(a, p, ws, stream);
}

template <typename E, int D>
static hipError_t launch_gate_t(const void* z, const float* A, float g_min, float* G, int B, int T,
                                int H, hipStream_t stream) {
    const int NC = (T + kChunk - 1) / kChunk;
    const size_t total = (size_t)B * NC * H * D;
    size_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL((gate_cumsum_kernel<E, D>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const E*)z, A, g_min, G, B, T, H);
    return hipGetLastError();
}

hipError_t launch_gate_cumsum(const void* z, const float* A, float g_min, float* G, int B, int T,
                              int H, int d, bool is_bf16, hipStream_t stream) {
    if (is_bf16)
        return d == 128 ? launch_gate_t<bf16, 128>(z, A, g_min, G, B, T, H, stream)
                        : launch_gate_t<bf16, 32>(z, A, g_min, G, B, T, H, stream);
    return d == 128 ? launch_gate_t<float, 128>(z, A, g_min, G, B, T, H, stream)
                    : launch_gate_t<float, 32>(z, A, g_min, G, B, T, H, stream);
}

template <typename E, int D>
static hipError_t launch_intra_diag_t(const void* q, const void* k, const void* z,
                                      const float* beta, const float* A, float g_min, float* Tm,
                                      float* Aqk, float* gamma, int B, int T, int H,
                                      hipStream_t stream) {
    const int NC = (T + kChunk - 1) / kChunk;
    const size_t nchunks = (size_t)B * H * NC;
    hipLaunchKernelGGL((intra_kernel<E, D, true>), dim3((unsigned)((nchunks + 3) / 4)), dim3(256), 0,
                       stream, (const E*)q, (const E*)k, (const E*)z, beta, A, g_min,
                       (char*)nullptr, B, T, H, 0, NC, Tm, Aqk, gamma);
    return hipGetLastError();
}

hipError_t launch_intra_diag(const void* q, const void* k, const void* z, const float* beta,
                             const float* A, float g_min, float* Tm, float* Aqk, float* gamma,
                             int B, int T, int H, int d, bool is_bf16, hipStream_t stream) {
    if (is_bf16)
        return d == 128 ? launch_intra_diag_t<bf16, 128>(q, k, z, beta, A, g_min, Tm, Aqk, gamma, B, T, H, stream)
                        : launch_intra_diag_t<bf16, 32>(q, k, z, beta, A, g_min, Tm, Aqk, gamma, B, T, H, stream);
    return d == 128 ? launch_intra_diag_t<float, 128>(q, k, z, beta, A, g_min, Tm, Aqk, gamma, B, T, H, stream)
                    : launch_intra_diag_t<float, 32>(q, k, z, beta, A, g_min, Tm, Aqk, gamma, B, T, H, stream);
}

}  // namespace kda
