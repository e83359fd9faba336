// kda_pair.hip -- split-plan prefill for gfx950: the state chain advances two
// 16-token chunks per step.
//
// Source of the method: dev.to "Kimi K3 Architecture: Scaling 2.8T Parameters
// for Long-Context Multimodal MoE", section "The Sequence Bottleneck: Hybrid
// KDA and Gated MLA" (lower-bounded gate, 16-token tiles whose cumulative
// log-decay stays inside (-80, 0), chunkwise parallel form).  The two-chunk
// step is an exact regrouping of two single-chunk steps (kda_chunk.hpp); the
// chunks keep their own 16-token factorisation, so every factor stays inside
// the bounds the 16-token tiles guarantee.
//
// For consecutive chunks a, b and the state S at the start of a:
//   x_a = Kt_a S,                      U_a = Tm_a (V_a - x_a)
//   S'  = Diag(gam_a) S + Kd_a^T U_a   (state at the start of b)
//   x_b = Kt_b S' = (Kt_b Diag(gam_a)) S + M_kb U_a,   M_kb = Kt_b Kd_a^T
//   U_b = Tm_b (V_b - x_b)
//   O_a = Qt_a S + Aqk_a U_a
//   O_b = (Qt_b Diag(gam_a)) S + M_qb U_a + Aqk_b U_b, M_qb = Qt_b Kd_a^T
//   S  <- Diag(gam_a gam_b) S + [Kd_a Diag(gam_b); Kd_b]^T [U_a; U_b]
// The cross terms are formed from bounded factors: Kt_b Kd_a^T =
// (Kt_b Diag(gam_a)) Kh_a^T with Kh_a = Kd_a Diag(gam_a)^{-1} = k_a e^{-G}.
// Per pair the chain packs S once, scales it once, and updates it with
// K = 32 products.
#include "kda_chunk.hpp"
#include "kda_launch.hpp"

namespace kda {

// ------------------------------------------------------------ pair block
//
// Operands of one pair in the lane layouts the chain reads (E elements):
//   KA, KB, QA, QB  Kt_a, Kt_b Diag(gam_a), Qt_a, Qt_b Diag(gam_a) in the
//                   A-row layout of Blk (16 rows x D, K = key channels)
//   KD2             S-update A operand, K = 32 tokens: tile m, lane (c, g)
//                   holds [Kd_a[4g+i][16m+c] gam_b[16m+c], Kd_b[4g+i][16m+c]],
//                   i = 0..3 (this K order makes [U_a; U_b] in accumulator
//                   layout its B operand)
//   TMA, TMB, AQA, MKB  16x16 A operands for K = 16: lane (r, c/4) holds
//                   row r, columns 4(c/4) .. 4(c/4)+3
//   OB2             [M_qb | Aqk_b] as a K = 32 A operand: lane (r, g) holds
//                   M_qb[r][4g+i], then Aqk_b[r][4g+i]
//   GAB             gam_a gam_b (fp32, D)
template <typename E, int D>
struct PBlk {
    using B1 = Blk<E, D>;
    static constexpr int ES = (int)sizeof(E);
    static constexpr int NSLOT = B1::NSLOT, MT = B1::MT, OPB = B1::OPB;
    static constexpr int AROW = NSLOT * 1024;
    static constexpr int KA = 0;
    static constexpr int KB = KA + AROW;
    static constexpr int QA = KB + AROW;
    static constexpr int QB = QA + AROW;
    static constexpr int KD2 = QB + AROW;
    static constexpr int TMA = KD2 + MT * kWave * 2 * OPB;
    static constexpr int TMB = TMA + kWave * OPB;
    static constexpr int AQA = TMB + kWave * OPB;
    static constexpr int MKB = AQA + kWave * OPB;
    static constexpr int OB2 = MKB + kWave * OPB;
    static constexpr int GAB = OB2 + kWave * 2 * OPB;
    static constexpr int BYTES = GAB + D * 4;
    static_assert(BYTES % 16 == 0, "pair block must be 16-byte granular");
    // KD2 entry of lane (cl, g) of tile m (swizzled like the single-chunk Kd tile)
    __device__ static __forceinline__ int kd2_offset(int m, int g, int cl) {
        return KD2 + m * kWave * 2 * OPB + (g * 16 + (cl ^ (m & 15))) * 2 * OPB;
    }
    // element (r, c) of a K = 16 A operand at `base`
    __device__ static __forceinline__ int a16_offset(int base, int r, int c) {
        return base + ((c >> 2) * 16 + r) * OPB + (c & 3) * ES;
    }
    // element (r, c) of M_qb (which = 0) or Aqk_b (which = 1) in OB2
    __device__ static __forceinline__ int ob2_offset(int r, int c, int which) {
        return OB2 + ((c >> 2) * 16 + r) * 2 * OPB + (4 * which + (c & 3)) * ES;
    }
};

template <typename E>
using V8 = typename std::conditional<std::is_same<E, bf16>::value, bf16x8,
                                     float __attribute__((ext_vector_type(8)))>::type;

// ------------------------------------------------------------ producer
//
// Per-wave LDS staging of the pair producer: two A-row work areas (R1, R2),
// Kh_a and Kh_b (A-row) and the small operands [TMA, BYTES) of the pair
// block.  The Akk scratch (16x16 fp32) of each solve shares Kh_b's area: the
// solve of chunk a ends before Kh_b is written, and that of chunk b begins
// after Kh_b's last read (the Gram products of chunk b), so 8 producer waves
// fit one CU's LDS at bf16, D = 128.
template <typename E, int D>
struct PStage {
    using P = PBlk<E, D>;
    static constexpr int R1 = 0;
    static constexpr int R2 = R1 + P::AROW;
    static constexpr int KHA = R2 + P::AROW;
    static constexpr int KHB = KHA + P::AROW;
    static constexpr int AKK = KHB;
    static_assert(16 * 16 * 4 <= P::AROW, "Akk scratch must fit in Kh_b's area");
    static constexpr int SMALL = KHB + P::AROW;               // holds P[TMA, BYTES)
    static constexpr int BYTES = SMALL + (P::BYTES - P::TMA);
    __device__ static __forceinline__ int small(int pblk_off) { return SMALL + pblk_off - P::TMA; }
};

// Copies `bytes` (a multiple of 16) from LDS to global memory.
__device__ __forceinline__ void copy_out(char* __restrict__ dst, const char* src, int bytes) {
    const uint4* s = reinterpret_cast<const uint4*>(src);
    uint4* d = reinterpret_cast<uint4*>(dst);
#pragma unroll 4
    for (int x = fresh_lane_id(); x < bytes / 16; x += kWave) d[x] = s[x];
}

// Writes NCL values of one row of the lane's key columns into an A-row area.
template <typename E, int D>
__device__ __forceinline__ void arow_put(char* area, int c0, int r, const float* x) {
    using B = Blk<E, D>;
    const int off = B::arow_offset(c0, r);
    if constexpr (B::NCL == 2 && B::kBF16) {
        *reinterpret_cast<bf16x2*>(area + off) = bf16x2{(bf16)x[0], (bf16)x[1]};
    } else if constexpr (B::NCL == 2) {
        *reinterpret_cast<f32x2*>(area + off) = f32x2{x[0], x[1]};
    } else {
        *reinterpret_cast<E*>(area + off) = from_f32<E>(x[0]);
    }
}

// 16x16 products of two A-row areas (K = D): acc[i][j] = sum_c A[i][c] Bm[j][c].
template <typename E, int D>
__device__ __forceinline__ f32x4 arow_gram(const char* A, const char* Bm) {
    using B = Blk<E, D>;
    const int lane = fresh_lane_id(), ci = lane & 15, g = lane >> 4;
    f32x4 acc = zero4();
#pragma unroll
    for (int s = 0; s < B::NSLOT; ++s) {
        const int off = B::arow_chunk(s, g, ci);
        const V16<E> a = *reinterpret_cast<const V16<E>*>(A + off);
        const V16<E> b = *reinterpret_cast<const V16<E>*>(Bm + off);
        if constexpr (B::kBF16) {
            acc = mma_bf16_k32(a, b, acc);
        } else {
#pragma unroll
            for (int p = 0; p < 4; ++p) acc = mma_f32_k4(a[p], b[p], acc);
        }
    }
    return acc;
}

// Gate of one chunk for the lane's key columns: P_r = e^{G_r} (inclusive
// prefix of the retentions), Qs_r = e^{G_15 - G_r} (exclusive suffix), gam =
// e^{G_15}.  Padded rows (r >= L) have retention 1.
template <typename E, int D>
__device__ __forceinline__ void pair_gate(const ProdIn<E, D>& in, const GateConsts& gc,
                                          float (&P)[16][Blk<E, D>::NCL],
                                          float (&Qs)[16][Blk<E, D>::NCL],
                                          float (&gam)[Blk<E, D>::NCL]) {
    using B = Blk<E, D>;
    constexpr int NCL = B::NCL;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        float zf[NCL];
        unpack_seg<E, NCL, B::NWORD>(in.z[r], zf);
#pragma unroll
        for (int e = 0; e < NCL; ++e) {
            const float a = gate_alpha_row(gc, zf[e], r < in.L ? 1.f : 0.f);
            Qs[r][e] = a;
            P[r][e] = r == 0 ? a : P[r - 1][e] * a;
        }
    }
#pragma unroll
    for (int e = 0; e < NCL; ++e) {
        gam[e] = P[15][e];
        float run = 1.f;
#pragma unroll
        for (int r = 15; r >= 0; --r) {
            const float a = Qs[r][e];
            Qs[r][e] = run;
            run *= a;
        }
    }
}

// Akk (masked, times beta of its row) -> the fp32 scratch; returns nothing.
__device__ __forceinline__ void put_akk(float* akk_s, const f32x4& akk, float bj) {
    const int lane = fresh_lane_id(), ci = lane & 15, g = lane >> 4;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int r = 4 * g + p;
        const float br = __shfl(bj, r);
        akk_s[r * 16 + ci] = ci < r ? br * akk[p] : 0.f;
    }
}

// Tm = (I + Akk)^{-1} Diag(beta) by forward substitution (lane j < 16 solves
// column j), written as a K = 16 A operand at `dst` (LDS).
template <typename E, int D>
__device__ __forceinline__ void put_tm(const float* akk_s, float bj, char* dst) {
    using P = PBlk<E, D>;
    const int lane = fresh_lane_id();
    if (lane < 16) {
        const int j = lane;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = r == j ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) acc -= akk_s[r * 16 + i] * x[i];
            x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
            *reinterpret_cast<E*>(dst + P::a16_offset(0, r, j)) = from_f32<E>(x[r] * bj);
    }
}

// Gate + intra-chunk stage of chunks a, b of one pair (one wave), written to
// the pair block at `out` (global memory) through the wave's staging `st`.
// `next_a()` is called once the inputs in a are no longer needed and
// `next_b()` once those in b are (each may load the next pair's inputs into
// them, so the loads overlap the rest of this pair's work).  They come after
// each chunk's triangular solve, so the solve's registers are never live
// beside both chunks' new inputs.
template <typename E, int D, typename NextA, typename NextB>
__device__ __forceinline__ void pair_produce(ProdIn<E, D>& a, ProdIn<E, D>& b,
                                             const GateConsts& gc, char* __restrict__ st,
                                             char* __restrict__ out, NextA next_a,
                                             NextB next_b) {
    using B = Blk<E, D>;
    using P = PBlk<E, D>;
    using Sg = PStage<E, D>;
    constexpr int NCL = B::NCL;
    const int lane = fresh_lane_id(), ci = lane & 15, g = lane >> 4;
    const bool owner = lane < B::NACT;
    const int c0 = (lane % B::NACT) * NCL;
    float* akk_s = reinterpret_cast<float*>(st + Sg::AKK);

    // ------------------------------------------------ chunk a
    float P_[16][NCL], Qs[16][NCL], gamA[NCL], gamB[NCL];
    float kdA[16][NCL];
    pair_gate<E, D>(a, gc, P_, Qs, gamA);
    {
        float rg[NCL];
#pragma unroll
        for (int e = 0; e < NCL; ++e) rg[e] = fast_rcp(gamA[e]);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float kf[NCL], qf[NCL], kt[NCL], qt[NCL], kh[NCL];
            unpack_seg<E, NCL, B::NWORD>(a.k[r], kf);
            unpack_seg<E, NCL, B::NWORD>(a.q[r], qf);
#pragma unroll
            for (int e = 0; e < NCL; ++e) {
                kt[e] = kf[e] * P_[r][e];
                qt[e] = qf[e] * P_[r][e];
                kdA[r][e] = kf[e] * Qs[r][e];
                kh[e] = kdA[r][e] * rg[e];
            }
            if (owner) {
                arow_put<E, D>(st + Sg::R1, c0, r, kt);
                arow_put<E, D>(st + Sg::R2, c0, r, qt);
                arow_put<E, D>(st + Sg::KHA, c0, r, kh);
            }
        }
    }
    wave_sync_lds();
    {
        const f32x4 akk = arow_gram<E, D>(st + Sg::R1, st + Sg::KHA);
        const f32x4 aqk = arow_gram<E, D>(st + Sg::R2, st + Sg::KHA);
        put_akk(akk_s, akk, a.bj);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int r = 4 * g + p;
            *reinterpret_cast<E*>(st + Sg::small(P::a16_offset(P::AQA, r, ci))) =
                from_f32<E>(ci <= r ? aqk[p] : 0.f);
        }
    }
    wave_sync_lds();
    put_tm<E, D>(akk_s, a.bj, st + Sg::small(P::TMA));
    // a is free from here on; the fence keeps next_a()'s loads after its
    // last reads (hoisted, both pairs' chunk-a inputs would be live at once)
    pin_issued();
    next_a();
    copy_out(out + P::KA, st + Sg::R1, P::AROW);
    copy_out(out + P::QA, st + Sg::R2, P::AROW);
    wave_sync_lds();   // R1, R2 and the Akk scratch are free again

    // ------------------------------------------------ chunk b
    pair_gate<E, D>(b, gc, P_, Qs, gamB);
    {
        float rg[NCL];
#pragma unroll
        for (int e = 0; e < NCL; ++e) rg[e] = fast_rcp(gamB[e]);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float kf[NCL], qf[NCL], kt[NCL], qt[NCL], kh[NCL];
            unpack_seg<E, NCL, B::NWORD>(b.k[r], kf);
            unpack_seg<E, NCL, B::NWORD>(b.q[r], qf);
#pragma unroll
            for (int e = 0; e < NCL; ++e) {
                kt[e] = kf[e] * P_[r][e];
                qt[e] = qf[e] * P_[r][e];
                const float kd = kf[e] * Qs[r][e];
                kh[e] = kd * rg[e];
                Qs[r][e] = kd;                       // Kd_b
            }
            if (owner) {
                arow_put<E, D>(st + Sg::R1, c0, r, kt);   // Kt_b, unscaled
                arow_put<E, D>(st + Sg::R2, c0, r, qt);   // Qt_b, unscaled
                arow_put<E, D>(st + Sg::KHB, c0, r, kh);
            }
        }
    }
    // S-update operand and the pair decay go straight to the block
    if (owner) {
#pragma unroll
        for (int e = 0; e < NCL; ++e) {
            const int col = c0 + e;
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                V8<E> x;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[i] = from_f32<E>(kdA[4 * gg + i][e] * gamB[e]);
                    x[4 + i] = from_f32<E>(Qs[4 * gg + i][e]);
                }
                *reinterpret_cast<V8<E>*>(out + P::kd2_offset(col / 16, gg, col % 16)) = x;
            }
            reinterpret_cast<float*>(st + Sg::small(P::GAB))[col] = gamA[e] * gamB[e];
        }
    }
    wave_sync_lds();
    {
        const f32x4 akk = arow_gram<E, D>(st + Sg::R1, st + Sg::KHB);
        const f32x4 aqk = arow_gram<E, D>(st + Sg::R2, st + Sg::KHB);
        put_akk(akk_s, akk, b.bj);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int r = 4 * g + p;
            *reinterpret_cast<E*>(st + Sg::small(P::ob2_offset(r, ci, 1))) =
                from_f32<E>(ci <= r ? aqk[p] : 0.f);
        }
    }
    wave_sync_lds();   // Kt_b, Qt_b read: replace them by the gam_a-scaled copies
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        float kf[NCL], qf[NCL], kt[NCL], qt[NCL];
        unpack_seg<E, NCL, B::NWORD>(b.k[r], kf);
        unpack_seg<E, NCL, B::NWORD>(b.q[r], qf);
#pragma unroll
        for (int e = 0; e < NCL; ++e) {
            kt[e] = kf[e] * P_[r][e] * gamA[e];
            qt[e] = qf[e] * P_[r][e] * gamA[e];
        }
        if (owner) {
            arow_put<E, D>(st + Sg::R1, c0, r, kt);
            arow_put<E, D>(st + Sg::R2, c0, r, qt);
        }
    }
    const float bjb = b.bj;
    wave_sync_lds();
    {
        // M_kb = (Kt_b Diag(gam_a)) Kh_a^T, M_qb = (Qt_b Diag(gam_a)) Kh_a^T
        const f32x4 mkb = arow_gram<E, D>(st + Sg::R1, st + Sg::KHA);
        const f32x4 mqb = arow_gram<E, D>(st + Sg::R2, st + Sg::KHA);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int r = 4 * g + p;
            *reinterpret_cast<E*>(st + Sg::small(P::a16_offset(P::MKB, r, ci))) = from_f32<E>(mkb[p]);
            *reinterpret_cast<E*>(st + Sg::small(P::ob2_offset(r, ci, 0))) = from_f32<E>(mqb[p]);
        }
    }
    put_tm<E, D>(akk_s, bjb, st + Sg::small(P::TMB));
    pin_issued();
    next_b();
    wave_sync_lds();
    copy_out(out + P::KB, st + Sg::R1, P::AROW);
    copy_out(out + P::QB, st + Sg::R2, P::AROW);
    copy_out(out + P::TMA, st + Sg::SMALL, P::BYTES - P::TMA);
}

// Pair intra kernel over the [B*H][NP] pairs of a segment (chunks
// n_first + 2p, n_first + 2p + 1 of every sequence; a chunk past the
// sequence's end is empty), writing their pair blocks to `ws`.  Each wave
// produces pairs id, id + gridDim.x, ..., and loads the next pair's inputs
// as soon as the current pair's are consumed (same registers), so the loads
// overlap the rest of the pair's work.
template <typename E, int D>
__global__ __launch_bounds__(64, 2) void pair_intra_kernel(const E* __restrict__ q,
                                                        const E* __restrict__ k,
                                                        const E* __restrict__ z,
                                                        const float* __restrict__ beta,
                                                        const float* __restrict__ A, float g_min,
                                                        char* __restrict__ ws, int B, int T, int H,
                                                        int n_first, int NP) {
    using P = PBlk<E, D>;
    __shared__ __attribute__((aligned(16))) char st[PStage<E, D>::BYTES];
    // pair (u, p): unit u = b * H + h, pair p of the segment; the wave's
    // pairs are blockIdx.x, blockIdx.x + gridDim.x, ... in (u, p) order,
    // stepped without a division per pair
    const int units = B * H;
    int u = (int)(blockIdx.x / (unsigned)NP), p = (int)(blockIdx.x % (unsigned)NP);
    if (u >= units) return;
    const int du = (int)(gridDim.x / (unsigned)NP), dp = (int)(gridDim.x % (unsigned)NP);
    // chunk `half` (0: first, 1: second) of pair (pu, pp); with !live an
    // empty chunk (no memory access: its buffers have size 0), so the loads
    // need no branch
    auto load = [&](int pu, int pp, int half, bool live, ProdIn<E, D>& c) {
        ChunkPos cp = chunk_pos<D>(pu / H, pu % H, n_first + 2 * pp + half, T, H);
        cp.L = live ? cp.L : 0;
        prod_load<E, D>(c, q, k, z, beta, cp);
    };
    ProdIn<E, D> ca, cb;
    load(u, p, 0, true, ca);
    load(u, p, 1, true, cb);
    for (;;) {
        int nu = u + du, np = p + dp;
        if (np >= NP) { np -= NP; ++nu; }
        const bool more = nu < units;
        char* out = ws + ((size_t)u * NP + p) * (size_t)P::BYTES;
        pair_produce<E, D>(ca, cb, make_gate(A[u % H], g_min), st, out,
                           [&] { load(nu, np, 0, more, ca); },
                           [&] { load(nu, np, 1, more, cb); });
        if (!more) break;
        u = nu;
        p = np;
    }
}

// Producer waves for `pairs` pairs: as many as are resident at once on the
// 256 CUs (registers and LDS staging decide how many per CU: 8 at bf16,
// D = 128), each producing the same number of pairs.
template <typename E, int D>
static unsigned intra_grid(size_t pairs) {
    static const int per_cu = [] {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, pair_intra_kernel<E, D>, 64, 0) !=
                hipSuccess || n < 1)
            n = 1;
        return n;
    }();
    const size_t slots = 256 * (size_t)per_cu;
    const size_t per = (pairs + slots - 1) / slots;
    return (unsigned)((pairs + per - 1) / per);
}

// ------------------------------------------------------------ chain

// Pair operands in the chain's registers.
template <typename E, int D>
struct POps {
    using P = PBlk<E, D>;
    V16<E> ka[P::NSLOT], kb[P::NSLOT], qa[P::NSLOT], qb[P::NSLOT];
    V8<E> kd2[P::MT];
    V4<E> tma, tmb, aqa, mkb;
    V8<E> ob2;
    f32x2 gv;   // two values of gam_a gam_b per lane (see gab_tile)
};

// gam_a gam_b of rows 16 M + 4 g + p of tile M for lane (j, g) (row_tile).
template <int M>
__device__ __forceinline__ f32x4 gab_tile(const f32x2& gv) {
    return row_tile<M>(gv);
}

// The operands read first (Kt_a, Kt_b Diag(gam_a)): loaded one pair ahead.
template <typename E, int D>
__device__ __forceinline__ void pops_load_k(POps<E, D>& c, const char* blk) {
    using P = PBlk<E, D>;
    const int lane = lane_id(), g = lane >> 4, r = lane & 15;
#pragma unroll
    for (int s = 0; s < P::NSLOT; ++s) {
        const int off = P::B1::arow_chunk(s, g, r);
        c.ka[s] = *reinterpret_cast<const V16<E>*>(blk + P::KA + off);
        c.kb[s] = *reinterpret_cast<const V16<E>*>(blk + P::KB + off);
    }
}

// Operands of U_a, U_b.
template <typename E, int D>
__device__ __forceinline__ void pops_load_u(POps<E, D>& c, const char* blk) {
    using P = PBlk<E, D>;
    const int lane = lane_id();
    c.tma = *reinterpret_cast<const V4<E>*>(blk + P::TMA + lane * P::OPB);
    c.mkb = *reinterpret_cast<const V4<E>*>(blk + P::MKB + lane * P::OPB);
    c.tmb = *reinterpret_cast<const V4<E>*>(blk + P::TMB + lane * P::OPB);
}

// Operands of the state update.
template <typename E, int D>
__device__ __forceinline__ void pops_load_supd(POps<E, D>& c, const char* blk) {
    using P = PBlk<E, D>;
    const int lane = lane_id(), g = lane >> 4, r = lane & 15;
    c.gv = *reinterpret_cast<const f32x2*>(blk + P::GAB + row_vec_offset<D>(g, r));
#pragma unroll
    for (int m = 0; m < P::MT; ++m) {
        c.kd2[m] = *reinterpret_cast<const V8<E>*>(blk + P::kd2_offset(m, g, r));
    }
}

// Operands of the state chain (U and the state update), in the order it uses them.
template <typename E, int D>
__device__ __forceinline__ void pops_load_chain(POps<E, D>& c, const char* blk) {
    pops_load_u<E, D>(c, blk);
    pops_load_supd<E, D>(c, blk);
}

// Operands of the outputs only (used after the state update).
template <typename E, int D>
__device__ __forceinline__ void pops_load_out(POps<E, D>& c, const char* blk) {
    using P = PBlk<E, D>;
    const int lane = lane_id(), g = lane >> 4, r = lane & 15;
#pragma unroll
    for (int s = 0; s < P::NSLOT; ++s) {
        const int off = P::B1::arow_chunk(s, g, r);
        c.qa[s] = *reinterpret_cast<const V16<E>*>(blk + P::QA + off);
        c.qb[s] = *reinterpret_cast<const V16<E>*>(blk + P::QB + off);
    }
    c.aqa = *reinterpret_cast<const V4<E>*>(blk + P::AQA + lane * P::OPB);
    c.ob2 = *reinterpret_cast<const V8<E>*>(blk + P::OB2 + lane * 2 * P::OPB);
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 lo, bf16x4 hi) {
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// The first products of a pair (bf16): S packed once, x_a = Kt_a S and
// x_b = (Kt_b Diag(gam_a)) S.  They need only the operands read one pair
// ahead, so the wave issues them before waiting for this pair's other reads.
template <typename E, int D, int NB>
__device__ __forceinline__ void pair_x(const POps<E, D>& c, const f32x4 (&S)[NB][D / 16],
                                       bf16x8 (&sb)[NB][PBlk<E, D>::NSLOT], f32x4 (&xa)[NB],
                                       f32x4 (&xb)[NB]) {
    using P = PBlk<E, D>;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        xa[nb] = zero4();
        xb[nb] = zero4();
#pragma unroll
        for (int s = 0; s < P::NSLOT; ++s) {
            sb[nb][s] = pack8(S[nb][2 * s], S[nb][2 * s + 1]);
            xa[nb] = mma_bf16_k32(c.ka[s], sb[nb][s], xa[nb]);
            xb[nb] = mma_bf16_k32(c.kb[s], sb[nb][s], xb[nb]);
        }
    }
}

// [U_a; U_b] of a pair (bf16) from x_a, x_b and V (accumulator layout), as
// the B operand of the K = 32 products.  Every 16x16x16 product starts from a
// zero accumulator: an MFMA of one shape must not take as srcC the in-flight
// result of an MFMA of another shape (16x16x32 -> 16x16x16 chains read stale
// srcC on gfx950).
template <typename E, int D>
__device__ __forceinline__ bf16x8 pair_u(const POps<E, D>& c, const f32x4& xa, const f32x4& xb,
                                         const f32x4& Va, const f32x4& Vb) {
    const bf16x4 ua = pack4(mma_bf16_k16(c.tma, pack4(Va - xa), zero4()));
    const f32x4 xbc = mma_bf16_k16(c.mkb, ua, zero4());
    const bf16x4 ub = pack4(mma_bf16_k16(c.tmb, pack4(Vb - xb - xbc), zero4()));
    return cat8(ua, ub);
}

// S <- Diag(gam_a gam_b) S + [Kd_a Diag(gam_b); Kd_b]^T [U_a; U_b] (bf16).
template <typename E, int D>
__device__ __forceinline__ void pair_supdate(const POps<E, D>& c, f32x4 (&S)[D / 16], const bf16x8& u2) {
    static_for<0, PBlk<E, D>::MT>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        S[m] = mma_bf16_k32(c.kd2[m], u2, S[m] * gab_tile<m>(c.gv));
    });
}

// Outputs of a pair (bf16) from the packed state at its start and [U_a; U_b].
template <typename E, int D>
__device__ __forceinline__ void pair_out(const POps<E, D>& c, const bf16x8 (&sb)[PBlk<E, D>::NSLOT],
                                         const bf16x8& u2, f32x4& Oa, f32x4& Ob) {
    f32x4 oa = zero4(), ob = zero4();
#pragma unroll
    for (int s = 0; s < PBlk<E, D>::NSLOT; ++s) {
        oa = mma_bf16_k32(c.qa[s], sb[s], oa);
        ob = mma_bf16_k32(c.qb[s], sb[s], ob);
    }
    const bf16x4 ua = bf16x4{u2[0], u2[1], u2[2], u2[3]};
    Oa = oa + mma_bf16_k16(c.aqa, ua, zero4());
    Ob = ob + mma_bf16_k32(c.ob2, u2, zero4());
}

// The rest of a pair (bf16) after pair_x: U_a, U_b, the state update, then
// the outputs from the packed old state.
template <typename E, int D, int NB>
__device__ __forceinline__ void pair_rest(const POps<E, D>& c, f32x4 (&S)[NB][D / 16],
                                          const bf16x8 (&sb)[NB][PBlk<E, D>::NSLOT],
                                          const f32x4 (&xa)[NB], const f32x4 (&xb)[NB],
                                          const f32x4 (&Va)[NB], const f32x4 (&Vb)[NB],
                                          f32x4 (&Oa)[NB], f32x4 (&Ob)[NB]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const bf16x8 u2 = pair_u<E, D>(c, xa[nb], xb[nb], Va[nb], Vb[nb]);
        pair_supdate<E, D>(c, S[nb], u2);
        pair_out<E, D>(c, sb[nb], u2, Oa[nb], Ob[nb]);
    }
}

// One pair of the state chain for NB 16-column blocks of S.  Va, Vb: V of
// chunks a, b (accumulator layout); Oa, Ob receive the outputs.  The chain
// (x, U, state update) is issued first; the outputs, which read the old
// state, come last so their products fill the MFMA pipe behind the chain.
template <typename E, int D, int NB>
__device__ __forceinline__ void pair_step(const POps<E, D>& c, f32x4 (&S)[NB][D / 16],
                                          const f32x4 (&Va)[NB], const f32x4 (&Vb)[NB],
                                          f32x4 (&Oa)[NB], f32x4 (&Ob)[NB]) {
    using P = PBlk<E, D>;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        if constexpr (P::B1::kBF16) {
            bf16x8 sb[P::NSLOT];
            f32x4 xa = zero4(), xb = zero4();
#pragma unroll
            for (int s = 0; s < P::NSLOT; ++s) {
                sb[s] = pack8(S[nb][2 * s], S[nb][2 * s + 1]);
                xa = mma_bf16_k32(c.ka[s], sb[s], xa);
                xb = mma_bf16_k32(c.kb[s], sb[s], xb);
            }
            // every 16x16x16 product below starts from a zero accumulator: an
            // MFMA of one shape must not take as srcC the in-flight result of
            // an MFMA of another shape (16x16x32 -> 16x16x16 chains read stale
            // srcC on gfx950)
            const bf16x4 ua = pack4(mma_bf16_k16(c.tma, pack4(Va[nb] - xa), zero4()));
            const f32x4 xbc = mma_bf16_k16(c.mkb, ua, zero4());
            const bf16x4 ub = pack4(mma_bf16_k16(c.tmb, pack4(Vb[nb] - xb - xbc), zero4()));
            const bf16x8 u2 = cat8(ua, ub);
            static_for<0, P::MT>([&](auto mc) {
                constexpr int m = decltype(mc)::value;
                S[nb][m] = mma_bf16_k32(c.kd2[m], u2, S[nb][m] * gab_tile<m>(c.gv));
            });
            f32x4 oa = zero4(), ob = zero4();
#pragma unroll
            for (int s = 0; s < P::NSLOT; ++s) {
                oa = mma_bf16_k32(c.qa[s], sb[s], oa);
                ob = mma_bf16_k32(c.qb[s], sb[s], ob);
            }
            Oa[nb] = oa + mma_bf16_k16(c.aqa, ua, zero4());
            Ob[nb] = ob + mma_bf16_k32(c.ob2, u2, zero4());
        } else {
            f32x4 xa = zero4(), xb = zero4(), oa = zero4(), ob = zero4();
#pragma unroll
            for (int m = 0; m < P::MT; ++m)
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    xa = mma_f32_k4(c.ka[m][p], S[nb][m][p], xa);
                    xb = mma_f32_k4(c.kb[m][p], S[nb][m][p], xb);
                    oa = mma_f32_k4(c.qa[m][p], S[nb][m][p], oa);
                    ob = mma_f32_k4(c.qb[m][p], S[nb][m][p], ob);
                }
            const f32x4 ya = Va[nb] - xa;
            f32x4 ua = zero4();
#pragma unroll
            for (int p = 0; p < 4; ++p) ua = mma_f32_k4(c.tma[p], ya[p], ua);
#pragma unroll
            for (int p = 0; p < 4; ++p) xb = mma_f32_k4(c.mkb[p], ua[p], xb);
            const f32x4 yb = Vb[nb] - xb;
            f32x4 ub = zero4();
#pragma unroll
            for (int p = 0; p < 4; ++p) ub = mma_f32_k4(c.tmb[p], yb[p], ub);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                oa = mma_f32_k4(c.aqa[p], ua[p], oa);
                ob = mma_f32_k4(c.ob2[p], ua[p], ob);
                ob = mma_f32_k4(c.ob2[4 + p], ub[p], ob);
            }
            Oa[nb] = oa;
            Ob[nb] = ob;
            static_for<0, P::MT>([&](auto mc) {
                constexpr int m = decltype(mc)::value;
                f32x4 sm = S[nb][m] * gab_tile<m>(c.gv);
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    sm = mma_f32_k4(c.kd2[m][p], ua[p], sm);
                    sm = mma_f32_k4(c.kd2[m][4 + p], ub[p], sm);
                }
                S[nb][m] = sm;
            });
        }
    }
}

// ------------------------------------------------------------ pair inter kernel
//
// One workgroup per (b, h, tile of NCOL = 16 NB NCW value columns) over the
// pairs of chunks [n_first, n_first + n_count).  Waves 0 .. NCW-1 each carry
// the state of NB 16-column blocks; the other NL waves stream the pair blocks
// (and, where the LDS holds them, the V tiles) into an LDS ring of NPAIR
// entries shared by the chains.  A chain reads the pair it computes and the
// first operands of the next pair, so two entries are in use per chain.
//
// Ring entries are handed over by LDS flags, not workgroup barriers, so the
// chains run unaligned and never wait for each other:
//   ready[e]  index of the last pair published in entry e (loader -> chains);
//             a loader stores it after its data stores have completed;
//   done[e][w]  index of the last pair chain w released from entry e
//             (chains -> loaders); stored after the chain's last read of it.
// Pair p goes to entry p mod NPAIR and belongs to loader p mod NL, which
// writes it once every chain has released pair p - NPAIR.
// The slowest chain at pair t waits only for pair t + 1, whose entry was last
// held by pair t + 1 - NPAIR <= t - 1, which every chain has released; so no
// wait closes a cycle.  Every wait is bounded (spin_until_ge).
template <typename E, int D, int NCW_, int NB_>
struct PairCfg {
    static constexpr int ES = (int)sizeof(E);
    static constexpr int NCW = NCW_, NB = NB_;
    static constexpr int NCOL = 16 * NB * NCW;                   // value columns per workgroup
    static constexpr int LDS_MAX = 160 * 1024 - 256;             // room for the flags
    // V tiles of one pair: 32-bit word w of the tile's row r (two bf16 or one
    // fp32 column) at word w * VSTR + r; the padding makes the loaders'
    // word stores conflict-free across the 64 LDS banks
    static constexpr int VSTR = 2 * kChunk + 2;
    static constexpr int VBYTES = NCOL * ES / 4 * VSTR * 4;
    static constexpr int ENT = PBlk<E, D>::BYTES + VBYTES;
    static constexpr int NPAIR = LDS_MAX / ENT < 4 ? LDS_MAX / ENT : 4;
    // loader waves: workgroups of at most four waves keep one wave per SIMD
    // (the chains get the whole register file)
    static constexpr int NL = NCW >= 4 ? 3 : 4 - NCW;
    static constexpr int THREADS = (NCW + NL) * kWave;
    static_assert(NCOL <= D, "column tile wider than the head");
    static_assert(NPAIR >= 2, "the ring needs two pair entries");
    static_assert((2 * kChunk * NCOL * ES / 16) % kWave == 0, "V pieces per loader lane");
    static_assert(VBYTES % 16 == 0, "ring entries stay 16-byte aligned");
};

template <typename E, int D, int NCW, int NB>
__global__ __launch_bounds__((PairCfg<E, D, NCW, NB>::THREADS)) void pair_inter_kernel(
    const char* __restrict__ ws, const E* __restrict__ v, StateIO io, E* __restrict__ o,
    int B, int T, int H, int n_first, int n_count, int nct) {
    using P = PBlk<E, D>;
    using Cfg = PairCfg<E, D, NCW, NB>;
    constexpr int NPAIR = Cfg::NPAIR, NL = Cfg::NL, ENT = Cfg::ENT, ES = Cfg::ES;
    constexpr int NCOL = Cfg::NCOL;
    constexpr int BLK16 = P::BYTES / 16;              // 16-byte pieces of one pair block
    constexpr int PER_LANE = (BLK16 + kWave - 1) / kWave;
    constexpr int RP = NCOL * ES / 16;                // 16-byte pieces per V row of the tile
    constexpr int VPL = 2 * kChunk * RP / kWave;
    constexpr int EPP = 16 / ES;                      // elements per piece
    __shared__ __attribute__((aligned(16))) char ring[NPAIR * ENT];
    __shared__ int ready[NPAIR], done[NPAIR][NCW];
    int u, ct;
    if (!map_unit(nct, B * H, u, ct)) return;   // uniform over the workgroup
    const int b = u / H, h = u % H;
    if (io.skip(b)) return;                      // uniform over the workgroup
    const int w = wave_id();
    const int lane = lane_id();
    const int tile0 = ct * NCOL;
    const int NP = (n_count + 1) / 2;
    const char* blk0 = ws + (size_t)u * NP * P::BYTES;
    const Rsrc rws = make_rsrc(blk0, (uint32_t)((size_t)NP * P::BYTES));
    if (w == 0 && lane < NPAIR) {
        ready[lane] = -1;
#pragma unroll
        for (int c = 0; c < NCW; ++c) done[lane][c] = -1;
    }
    wg_barrier();   // the only barrier: flags initialised

    if (w >= NCW) {
        // ------------------------------------------------ loader waves
        const int L = w - NCW;
        u32x4 buf[PER_LANE];
        u32x4 vbuf[VPL];
        auto issue = [&](int p) {
#pragma unroll
            for (int i = 0; i < PER_LANE; ++i) {
                const int piece = i * kWave + lane;
                buf[i] = buf_load<u32x4>(rws, (p * BLK16 + piece) * 16);   // past the end: 0
            }
            // rows t0 .. t0+31 of the tile's columns; rows past T read 0
            const int t0 = (n_first + 2 * p) * kChunk;
            const int Lr = min(2 * kChunk, T - t0);
            const size_t rs = (size_t)H * D;
            const size_t row0 = ((size_t)b * T + t0) * H + h;
            const Rsrc rv = make_rsrc(v + row0 * D + tile0,
                                      Lr > 0 ? (uint32_t)(((size_t)(Lr - 1) * rs + NCOL) * ES) : 0u);
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int q = i * kWave + lane, r = q / RP, c = q % RP;
                vbuf[i] = buf_load<u32x4>(rv, (int)((r * rs + c * EPP) * ES));
            }
        };
        auto write = [&](int p) {
            char* dst = ring + (p % NPAIR) * ENT;
#pragma unroll
            for (int i = 0; i < PER_LANE; ++i) {
                const int piece = i * kWave + lane;
                if (piece < BLK16) *reinterpret_cast<u32x4*>(dst + piece * 16) = buf[i];
            }
            // V area: word-major (word w of row r at w * VSTR + r), so a
            // chain reads the four rows of its column as 16 bytes
            uint32_t* vd = reinterpret_cast<uint32_t*>(dst + P::BYTES);
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int q = i * kWave + lane, r = q / RP, c = q % RP;
#pragma unroll
                for (int e = 0; e < 4; ++e) vd[(4 * c + e) * Cfg::VSTR + r] = vbuf[i][e];
            }
        };
        // outputs of pair q, left by the chains in its entry's V area (same
        // word-major layout), to o: 16 bytes per lane-piece; rows past T are
        // outside the buffer and dropped
        auto flush = [&](int q, bool ok) {
            const uint32_t* vd = reinterpret_cast<const uint32_t*>(ring + (q % NPAIR) * ENT + P::BYTES);
            const int t0 = (n_first + 2 * q) * kChunk;
            const int Lr = min(2 * kChunk, T - t0);
            const size_t rs = (size_t)H * D;
            const size_t row0 = ((size_t)b * T + t0) * H + h;
            const Rsrc ro = make_rsrc(o + row0 * D + tile0,
                                      Lr > 0 ? (uint32_t)(((size_t)(Lr - 1) * rs + NCOL) * ES) : 0u);
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int q2 = i * kWave + lane, r = q2 / RP, c = q2 % RP;
                u32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = ok ? vd[(4 * c + e) * Cfg::VSTR + r] : kNaNWord;
                buf_store_u32x4(ro, (int)((r * rs + c * EPP) * ES), x);
            }
        };
        auto wait_released = [&](int q) {   // every chain has released pair q
            bool ok = true;
#pragma unroll
            for (int c = 0; c < NCW; ++c) ok = spin_until_ge(&done[q % NPAIR][c], q) && ok;
            return ok;
        };
        if (L < NP) issue(L);
        for (int p = L; p < NP; p += NL) {
            const int e = p % NPAIR;
            if (p >= NPAIR) {   // the entry's previous pair: released, outputs out
                const bool ok = wait_released(p - NPAIR);
                flush(p - NPAIR, ok);
                if (!ok) {   // a chain may still read the entry: poison the V it gets
#pragma unroll
                    for (int i = 0; i < VPL; ++i) vbuf[i] = u32x4{kNaNWord, kNaNWord, kNaNWord, kNaNWord};
                }
            }
            write(p);
            // publish: the data stores complete before the flag store
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
            __hip_atomic_store(&ready[e], p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (p + NL < NP) issue(p + NL);
        }
        // the last pairs' entries are not rewritten: the loader that would
        // have written pair q + NPAIR writes pair q's outputs out
        for (int q = NP - NPAIR > 0 ? NP - NPAIR : 0; q < NP; ++q) {
            if ((q + NPAIR) % NL != L) continue;
            flush(q, wait_released(q));
        }
        return;
    }
    // ---------------------------------------------------- state chains
    const int j = lane & 15, g = lane >> 4;
    const int col0 = tile0 + 16 * NB * w;
    auto entry = [&](int p) { return ring + (p % NPAIR) * ENT; };
    // V of chunk half (0 = a, 1 = b) of the pair in entry `ent`, NB blocks:
    // the raw words (read), then widened to fp32 (widen) once they are needed
    auto v_read = [&](const char* ent, int half, u32x4 (&V)[NB]) {
        const uint32_t* base = reinterpret_cast<const uint32_t*>(ent + P::BYTES) + half * kChunk + 4 * g;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int vcol = 16 * (NB * w + nb) + j;   // column within the tile
            const uint32_t* at = base + (ES == 2 ? vcol >> 1 : vcol) * Cfg::VSTR;
            const u32x2 lo = *reinterpret_cast<const u32x2*>(at);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(at + 2);
            V[nb] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
    };
    auto v_widen2 = [&](const u32x4 (&X)[NB], f32x4 (&V)[NB]) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            u32x4 x = X[nb];
            if constexpr (ES == 2) {
                const int vcol = 16 * (NB * w + nb) + j;
                x <<= 16 * (1 - (vcol & 1));   // bf16 of this column to the high half
                x &= 0xFFFF0000u;
            }
            V[nb] = __builtin_bit_cast(f32x4, x);
        }
    };
    // outputs of a pair into its entry's V area, over the V words of this
    // chain's own columns (read before, by this wave: LDS keeps its order),
    // in the same word-major layout; a loader writes them to o
    auto o_put = [&](const char* ent, const f32x4 (&Oa)[NB], const f32x4 (&Ob)[NB]) {
        char* base = const_cast<char*>(ent) + P::BYTES;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int vcol = 16 * (NB * w + nb) + j;   // column within the tile
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int ra = 4 * g + p, rb = kChunk + 4 * g + p;
                if constexpr (ES == 2) {
                    char* at = base + (vcol & 1) * 2;
                    *reinterpret_cast<bf16*>(at + ((vcol >> 1) * Cfg::VSTR + ra) * 4) = from_f32<E>(Oa[nb][p]);
                    *reinterpret_cast<bf16*>(at + ((vcol >> 1) * Cfg::VSTR + rb) * 4) = from_f32<E>(Ob[nb][p]);
                } else {
                    *reinterpret_cast<float*>(base + (vcol * Cfg::VSTR + ra) * 4) = Oa[nb][p];
                    *reinterpret_cast<float*>(base + (vcol * Cfg::VSTR + rb) * 4) = Ob[nb][p];
                }
            }
        }
    };
    f32x4 S[NB][D / 16];
    state_load<D, NB>(S, io.in_at(b, h, H, D), col0);
    POps<E, D> c;
    // The loop body is one basic block (a branch inside it keeps the
    // scheduler from overlapping a step's tail with what follows): the next
    // pair's first operands are read speculatively at the end of a step,
    // after its ready flag (LDS executes a wave's operations in order, so the
    // data read after a flag that shows the pair published is that pair's);
    // the rare re-read happens at the top of the next step.
    if (!spin_until_ge(&ready[0], 0))
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) poison_state(S[nb]);
    pops_load_k<E, D>(c, entry(0));
    int fl = 0;
    for (int s = 0; s < NP; ++s) {
        const char* ent = entry(s);
        if (fl < s) {
            if (!spin_until_ge(&ready[s % NPAIR], s))
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) poison_state(S[nb]);
            pops_load_k<E, D>(c, ent);
        }
        f32x4 Va[NB], Vb[NB], Oa[NB], Ob[NB];
        u32x4 ra[NB], rb[NB];
        // LDS reads in the order of first use (the wait counter is in order
        // and counts at most 15: a value is usable only once all but 15 of
        // the reads issued after it are done, so the reads come in batches)
        v_read(ent, 0, ra);
        v_read(ent, 1, rb);
        pops_load_chain<E, D>(c, ent);
        if constexpr (ES == 2) {
            // batch 1 (chain operands) issued; x_a, x_b need only operands
            // read a pair ahead; then batch 2 (output operands)
            pin_issued();
            bf16x8 sb[NB][P::NSLOT];
            f32x4 xa[NB], xb[NB];
            pair_x<E, D, NB>(c, S, sb, xa, xb);
            pin_issued();
            pops_load_out<E, D>(c, ent);
            pin_issued();
            v_widen2(ra, Va);
            v_widen2(rb, Vb);
            pair_rest<E, D, NB>(c, S, sb, xa, xb, Va, Vb, Oa, Ob);
        } else {
            pops_load_out<E, D>(c, ent);
            v_widen2(ra, Va);
            v_widen2(rb, Vb);
            pair_step<E, D, NB>(c, S, Va, Vb, Oa, Ob);
        }
        o_put(ent, Oa, Ob);
        // release pair s: its reads and output writes were all issued above
        asm volatile("" ::: "memory");
        __hip_atomic_store(&done[s % NPAIR][w], s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        fl = __hip_atomic_load(&ready[(s + 1) % NPAIR], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        asm volatile("" ::: "memory");
        pops_load_k<E, D>(c, entry(s + 1));   // (past the last pair: stale, unused)
    }
    if (io.out) state_store<D, NB>(S, io.out_at(b, h, H, D), col0);
}

// ------------------------------------------------------------ pair roles kernel
//
// bf16 chains of one 16-column block, with each step split over two waves.
// One wave issues its LDS reads, MFMAs and VALU one after the other, so a
// single chain wave pays for all of a pair's operand reads and products in
// sequence; here the chain wave computes x, U and the state update and leaves
// [U_a; U_b] in the ring entry, and the output wave keeps a replica of the
// state (the same update from the same operands and U, hence bit-identical),
// forms the pair's outputs and stores them.  Loader waves move each pair
// block from the workspace straight into its ring entry (LDS DMA, no VGPRs),
// one pair in flight per loader, and V through VGPRs.
//
// Flags, as in pair_inter_kernel, plus:
//   uready[c]   last pair whose [U_a; U_b] chain c has left in its entry;
//   done[e][r]  readers r = chain waves 0 .. NCW-1, then output waves.
// The output wave of chain c waits only for uready[c]; a chain never waits
// for its output wave except through the ring (a loader refills an entry
// once every reader released it), so no wait closes a cycle.
template <typename E, int D, int NCW_>
struct RoleCfg {
    static constexpr int ES = (int)sizeof(E);
    static constexpr int NCW = NCW_;
    static constexpr int NCOL = 16 * NCW;                        // value columns per workgroup
    static constexpr int LDS_MAX = 160 * 1024 - 512;             // room for the flags
    static constexpr int VSTR = 2 * kChunk + 2;                  // as in PairCfg
    static constexpr int VBYTES = NCOL * ES / 4 * VSTR * 4;
    static constexpr int UBYTES = NCW * kWave * 16;              // one bf16x8 per lane and chain
    static constexpr int ENT = PBlk<E, D>::BYTES + VBYTES + UBYTES;
    static constexpr int NPAIR = LDS_MAX / ENT < 5 ? LDS_MAX / ENT : 5;
    static constexpr int NREAD = 2 * NCW;                        // chain and output waves
    static constexpr int NL = 8 - NREAD;                         // loader waves: two waves per SIMD
    static constexpr int THREADS = (NREAD + NL) * kWave;
    static_assert(ES == 2, "bf16 operands");
    static_assert(NCOL <= D, "column tile wider than the head");
    static_assert(NPAIR >= 2, "the ring needs two pair entries");
    static_assert((2 * kChunk * NCOL * ES / 16) % kWave == 0, "V pieces per loader lane");
    static_assert(VBYTES % 16 == 0 && ENT % 16 == 0, "ring entries stay 16-byte aligned");
};

template <typename E, int D, int NCW>
__global__ __launch_bounds__((RoleCfg<E, D, NCW>::THREADS)) void pair_roles_kernel(
    const char* __restrict__ ws, const E* __restrict__ v, StateIO io, E* __restrict__ o, int B,
    int T, int H, int n_first, int n_count, int nct) {
    using P = PBlk<E, D>;
    using Cfg = RoleCfg<E, D, NCW>;
    constexpr int NPAIR = Cfg::NPAIR, NL = Cfg::NL, ENT = Cfg::ENT, ES = Cfg::ES;
    constexpr int NCOL = Cfg::NCOL, NREAD = Cfg::NREAD;
    constexpr int BLK16 = P::BYTES / 16;              // 16-byte pieces of one pair block
    constexpr int PER_LANE = (BLK16 + kWave - 1) / kWave;
    constexpr int RP = NCOL * ES / 16;                // 16-byte pieces per V row of the tile
    constexpr int VPL = 2 * kChunk * RP / kWave;
    constexpr int EPP = 16 / ES;                      // elements per piece
    constexpr int UOFF = P::BYTES + Cfg::VBYTES;      // [U_a; U_b] of the entry's pair
    __shared__ __attribute__((aligned(16))) char ring[NPAIR * ENT];
    __shared__ int ready[NPAIR], done[NPAIR][NREAD], uready[NCW];
    int u, ct;
    if (!map_unit(nct, B * H, u, ct)) return;   // uniform over the workgroup
    const int b = u / H, h = u % H;
    if (io.skip(b)) return;                      // uniform over the workgroup
    const int w = wave_id();
    const int lane = lane_id();
    const int tile0 = ct * NCOL;
    const int NP = (n_count + 1) / 2;
    const char* blk0 = ws + (size_t)u * NP * P::BYTES;
    const Rsrc rws = make_rsrc(blk0, (uint32_t)((size_t)NP * P::BYTES));
    if (w == 0) {
        if (lane < NPAIR) {
            ready[lane] = -1;
#pragma unroll
            for (int c = 0; c < NREAD; ++c) done[lane][c] = -1;
        }
        if (lane < NCW) uready[lane] = -1;
    }
    // chain wave c and output wave NCW + c start from the initial state of
    // the same 16 columns; both read it before the barrier, so the chain
    // wave's final store (S_T may alias S0) cannot overtake the output wave's
    // read
    f32x4 S[1][D / 16];
    if (w < NREAD) state_load<D, 1>(S, io.in_at(b, h, H, D), tile0 + 16 * (w % NCW));
    wg_barrier();   // the only barrier: flags initialised
    auto entry = [&](int p) { return ring + (p % NPAIR) * ENT; };

    if (w >= NREAD) {
        // ------------------------------------------------ loader waves
        const int L = w - NREAD;
        for (int p = L; p < NP; p += NL) {
            bool ok = true;
            if (p >= NPAIR) {   // every reader has released the entry's previous pair
#pragma unroll
                for (int c = 0; c < NREAD; ++c)
                    ok = spin_until_ge(&done[p % NPAIR][c], p - NPAIR) && ok;
            }
            char* dst = entry(p);
            // V (rows t0 .. t0+31 of the tile's columns; rows past T read 0)
            // into VGPRs, then the pair block into the entry: V comes from
            // memory the producer did not just write, so it is issued first
            // and its latency overlaps the block's
            const int t0 = (n_first + 2 * p) * kChunk;
            const int Lr = min(2 * kChunk, T - t0);
            const size_t rs = (size_t)H * D;
            const size_t row0 = ((size_t)b * T + t0) * H + h;
            const Rsrc rv = make_rsrc(v + row0 * D + tile0,
                                      Lr > 0 ? (uint32_t)(((size_t)(Lr - 1) * rs + NCOL) * ES) : 0u);
            u32x4 vbuf[VPL];
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int q = i * kWave + lane, r = q / RP, c = q % RP;
                vbuf[i] = buf_load<u32x4>(rv, (int)((r * rs + c * EPP) * ES));
            }
#pragma unroll
            for (int i = 0; i < PER_LANE; ++i) {
                const int piece = i * kWave + lane;
                if (i + 1 < PER_LANE || piece < BLK16)
                    buf_load_lds16(rws, (p * BLK16 + piece) * 16, dst + i * kWave * 16);
            }
            vm_wait_all();   // V and every piece of the block have landed
            // V area: word-major (word w of row r at w * VSTR + r); after a
            // wait that gave up, NaN, so the readers still on the entry's
            // previous pair, and this pair's readers, produce NaN
            uint32_t* vd = reinterpret_cast<uint32_t*>(dst + P::BYTES);
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int q = i * kWave + lane, r = q / RP, c = q % RP;
#pragma unroll
                for (int e = 0; e < 4; ++e) vd[(4 * c + e) * Cfg::VSTR + r] = ok ? vbuf[i][e] : kNaNWord;
            }
            // publish: the V stores complete before the flag store
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
            __hip_atomic_store(&ready[p % NPAIR], p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        return;
    }

    const int j = lane & 15, g = lane >> 4;
    if (w < NCW) {
        // ------------------------------------------------ chain waves
        const int col0 = tile0 + 16 * w;
        const int vcol = 16 * w + j;   // column within the tile
        // V of chunk half (0 = a, 1 = b): raw words, widened when needed
        auto v_read = [&](const char* ent, int half) {
            const uint32_t* at = reinterpret_cast<const uint32_t*>(ent + P::BYTES) + half * kChunk +
                                 4 * g + (vcol >> 1) * Cfg::VSTR;
            const u32x2 lo = *reinterpret_cast<const u32x2*>(at);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(at + 2);
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
        };
        auto v_widen = [&](u32x4 x) {
            x <<= 16 * (1 - (vcol & 1));   // bf16 of this column to the high half
            x &= 0xFFFF0000u;
            return __builtin_bit_cast(f32x4, x);
        };
        POps<E, D> c;
        // one basic block per step but for the rare re-read of a pair whose
        // first operands were read ahead of its publication
        if (!spin_until_ge(&ready[0], 0)) poison_state(S[0]);
        pops_load_k<E, D>(c, entry(0));
        int fl = 0;
        for (int s = 0; s < NP; ++s) {
            char* ent = entry(s);
            if (fl < s) {
                if (!spin_until_ge(&ready[s % NPAIR], s)) poison_state(S[0]);
                pops_load_k<E, D>(c, ent);
            }
            const u32x4 ra = v_read(ent, 0), rb = v_read(ent, 1);
            pops_load_chain<E, D>(c, ent);
            pin_issued();
            bf16x8 sb[1][P::NSLOT];
            f32x4 xa[1], xb[1];
            pair_x<E, D, 1>(c, S, sb, xa, xb);
            const bf16x8 u2 = pair_u<E, D>(c, xa[0], xb[0], v_widen(ra), v_widen(rb));
            *reinterpret_cast<bf16x8*>(ent + UOFF + (w * kWave + lane) * 16) = u2;
            asm volatile("" ::: "memory");
            __hip_atomic_store(&uready[w], s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            pair_supdate<E, D>(c, S[0], u2);
            // release pair s: its reads were all issued above
            asm volatile("" ::: "memory");
            __hip_atomic_store(&done[s % NPAIR][w], s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            fl = __hip_atomic_load(&ready[(s + 1) % NPAIR], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            asm volatile("" ::: "memory");
            pops_load_k<E, D>(c, entry(s + 1));   // (past the last pair: stale, unused)
        }
        if (io.out) state_store<D, 1>(S, io.out_at(b, h, H, D), col0);
        return;
    }

    // ---------------------------------------------------- output waves
    const int wc = w - NCW;                 // the chain this wave follows
    const int col0 = tile0 + 16 * wc;
    f32x4 (&Sr)[D / 16] = S[0];             // the replica of chain wc's state
    POps<E, D> c;
    for (int s = 0; s < NP; ++s) {
        char* ent = entry(s);
        if (!spin_until_ge(&uready[wc], s)) poison_state(Sr);
        const bf16x8 u2 = *reinterpret_cast<const bf16x8*>(ent + UOFF + (wc * kWave + lane) * 16);
        pops_load_out<E, D>(c, ent);
        pops_load_supd<E, D>(c, ent);
        pin_issued();
        bf16x8 sb[P::NSLOT];
#pragma unroll
        for (int k = 0; k < P::NSLOT; ++k) sb[k] = pack8(Sr[2 * k], Sr[2 * k + 1]);
        f32x4 Oa, Ob;
        pair_out<E, D>(c, sb, u2, Oa, Ob);
        pair_supdate<E, D>(c, Sr, u2);
        // outputs: rows 4g + (j & 3) of each chunk, columns 4 (j >> 2) .. +3
        // of this block, 8 bytes per lane and chunk; rows past T are dropped
        {
            const int t0 = (n_first + 2 * s) * kChunk;
            const int Lr = min(2 * kChunk, T - t0);
            const size_t rs = (size_t)H * D;
            const size_t row0 = ((size_t)b * T + t0) * H + h;
            const Rsrc ro = make_rsrc(o + row0 * D + col0,
                                      Lr > 0 ? (uint32_t)(((size_t)(Lr - 1) * rs + 16) * ES) : 0u);
            const int r = 4 * g + (j & 3), off = (int)((r * rs + 4 * (j >> 2)) * ES);
            buf_store_u32x2(ro, off, acc_rows_bf16(Oa));
            buf_store_u32x2(ro, off + (int)(kChunk * rs * ES), acc_rows_bf16(Ob));
        }
        asm volatile("" ::: "memory");
        __hip_atomic_store(&done[s % NPAIR][NCW + wc], s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
}

// ------------------------------------------------------------ launch

size_t pair_block_bytes(int d, bool is_bf16) {
    if (is_bf16) return d == 128 ? (size_t)PBlk<bf16, 128>::BYTES : (size_t)PBlk<bf16, 32>::BYTES;
    return d == 128 ? (size_t)PBlk<float, 128>::BYTES : (size_t)PBlk<float, 32>::BYTES;
}

bool pair_variant_ok(int d, bool is_bf16, int ncol, int nb) {
    if (nb != 1 && nb != 2) return false;
    const int ncw = ncol / (16 * nb);
    if (ncw * 16 * nb != ncol || ncol > d) return false;
    // two-block chains: bf16 with d = 128 (their operands and two states fill
    // the register file); four fp32 chains would not fit a shared SIMD
    if (nb == 2) return d == 128 && is_bf16 && (ncw == 1 || ncw == 2);
    return ncw == 1 || ncw == 2 || (ncw == 4 && d == 128 && is_bf16);
}

static unsigned pair_grid(int units, int nct) { return (unsigned)(((units + 7) / 8) * 8 * nct); }

template <typename E, int D, int NCW, int NB>
static hipError_t launch_pair_inter_v(const char* ws, const E* v, const StateIO& io, E* o,
                                      const PrefillArgs& a, int n_first, int n_count,
                                      hipStream_t stream) {
    using Cfg = PairCfg<E, D, NCW, NB>;
    const int nct = D / Cfg::NCOL;
    hipLaunchKernelGGL((pair_inter_kernel<E, D, NCW, NB>), dim3(pair_grid(a.B * a.H, nct)),
                       dim3(Cfg::THREADS), 0, stream, ws, v, io, o, a.B, a.T, a.H, n_first,
                       n_count, nct);
    return hipGetLastError();
}

template <typename E, int D, int NCW>
static hipError_t launch_pair_roles_v(const char* ws, const E* v, const StateIO& io, E* o,
                                      const PrefillArgs& a, int n_first, int n_count,
                                      hipStream_t stream) {
    using Cfg = RoleCfg<E, D, NCW>;
    const int nct = D / Cfg::NCOL;
    hipLaunchKernelGGL((pair_roles_kernel<E, D, NCW>), dim3(pair_grid(a.B * a.H, nct)),
                       dim3(Cfg::THREADS), 0, stream, ws, v, io, o, a.B, a.T, a.H, n_first,
                       n_count, nct);
    return hipGetLastError();
}

template <typename E, int D>
static hipError_t launch_split_t(const PrefillArgs& a, const PlanInfo& p, void* ws,
                                 hipStream_t stream) {
    using P = PBlk<E, D>;
    const int units = a.B * a.H;
    const int NC = (a.T + kChunk - 1) / kChunk;
    const int seg = NC < kSegChunks ? NC : kSegChunks;
    const int NPmax = (seg + 1) / 2;
    char* fws = (char*)ws;
    // the state between segments: the caller's output state (its rows or
    // slots), else a dense buffer after the pair blocks in the workspace
    float* carry = a.S.out;
    const int* carry_slot = a.S.out_slot;
    if (NC > seg && !carry) carry = (float*)(fws + (size_t)units * NPmax * P::BYTES);
    const E* v = (const E*)a.v;
    E* o = (E*)a.o;
    for (int n_first = 0; n_first < NC; n_first += seg) {
        const int n_count = (NC - n_first) < seg ? (NC - n_first) : seg;
        const int NP = (n_count + 1) / 2;
        hipLaunchKernelGGL((pair_intra_kernel<E, D>), dim3(intra_grid<E, D>((size_t)units * NP)), dim3(64),
                           0, stream, (const E*)a.q, (const E*)a.k, (const E*)a.z, a.beta, a.A,
                           a.g_min, fws, a.B, a.T, a.H, n_first, NP);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const bool first = n_first == 0, last = n_first + n_count >= NC;
        StateIO io = a.S;
        if (!first) {
            io.in = carry;
            io.in_slot = carry_slot;
        }
        if (!last) {
            io.out = carry;
            io.out_slot = carry_slot;
        }
#define KDA_PAIR_INTER(NCW, NB) \
    e = launch_pair_inter_v<E, D, NCW, NB>(fws, v, io, o, a, n_first, n_count, stream)
        if constexpr (D == 128 && sizeof(E) == 2) {
            if (p.nb == 2 && p.ncol == 64) KDA_PAIR_INTER(2, 2);
            else if (p.nb == 2) KDA_PAIR_INTER(1, 2);
            else if (p.ncol == 64) KDA_PAIR_INTER(4, 1);
            else if (p.ncol == 32) KDA_PAIR_INTER(2, 1);
            else e = launch_pair_roles_v<E, D, 1>(fws, v, io, o, a, n_first, n_count, stream);
        } else {
            if (p.ncol == 32) KDA_PAIR_INTER(2, 1);
            else KDA_PAIR_INTER(1, 1);
        }
#undef KDA_PAIR_INTER
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_split(const PrefillArgs& a, const PlanInfo& p, void* ws, hipStream_t stream) {
    if (a.lim.in || a.lim.out) return hipErrorInvalidValue;   // per-unit chunk counts: fused plan only
    if (a.is_bf16)
        return a.d == 128 ? launch_split_t<bf16, 128>(a, p, ws, stream)
                          : launch_split_t<bf16, 32>(a, p, ws, stream);
    return a.d == 128 ? launch_split_t<float, 128>(a, p, ws, stream)
                      : launch_split_t<float, 32>(a, p, ws, stream);
}

}  // namespace kda
