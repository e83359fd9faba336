// kda_pair.hpp -- the two-chunk pair step shared by the split plan and the
// ring plan: the pair block, its producer (one wave per pair) and the
// chain's pair step.
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
#pragma once
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
// fit one CU's LDS at bf16, D = 128.  The A-row areas of chunk a (R1A, R2A)
// and chunk b (R1B, R2B) are the same two areas here; the producer copies
// each to the block in global memory once it is final.
template <typename E, int D>
struct PStage {
    using P = PBlk<E, D>;
    static constexpr bool STAGED = false;   // the block is written to global memory
    static constexpr int R1 = 0;
    static constexpr int R2 = R1 + P::AROW;
    static constexpr int R1A = R1, R2A = R2, R1B = R1, R2B = R2;
    static constexpr int KHA = R2 + P::AROW;
    static constexpr int KHB = KHA + P::AROW;
    static constexpr int AKK = KHB;
    static_assert(16 * 16 * 4 <= P::AROW, "Akk scratch must fit in Kh_b's area");
    static constexpr int SMALL = KHB + P::AROW;               // holds P[TMA, BYTES)
    static constexpr int BYTES = SMALL + (P::BYTES - P::TMA);
    __device__ static __forceinline__ int small(int pblk_off) { return SMALL + pblk_off - P::TMA; }
};

// Staging that holds the whole pair block in LDS, in its final layout at
// offset 0, plus Kh_a and Kh_b: the A-row areas of the chunks are the
// block's own Kt/Qt areas (chunk b's are first written unscaled for its
// Gram products, then overwritten by the gam_a-scaled copies), and nothing
// goes to global memory; the caller copies the finished block out in one
// piece.
template <typename E, int D>
struct PStageFull {
    using P = PBlk<E, D>;
    static constexpr bool STAGED = true;
    static constexpr int R1A = P::KA, R2A = P::QA, R1B = P::KB, R2B = P::QB;
    static constexpr int KHA = P::BYTES;
    static constexpr int KHB = KHA + P::AROW;
    static constexpr int AKK = KHB;
    static_assert(16 * 16 * 4 <= P::AROW, "Akk scratch must fit in Kh_b's area");
    static constexpr int BYTES = KHB + P::AROW;
    __device__ static __forceinline__ int small(int pblk_off) { return pblk_off; }
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
template <typename E, int D, typename Sg, typename NextA, typename NextB>
__device__ __forceinline__ void pair_produce(ProdIn<E, D>& a, ProdIn<E, D>& b,
                                             const GateConsts& gc, char* __restrict__ st,
                                             char* __restrict__ out, NextA next_a,
                                             NextB next_b) {
    using B = Blk<E, D>;
    using P = PBlk<E, D>;
    constexpr int NCL = B::NCL;
    const int lane = fresh_lane_id(), ci = lane & 15, g = lane >> 4;
    const bool owner = lane < B::NACT;
    // KD2 and GAB go to the block directly: in global memory, or in the
    // staged block
    char* const kd2_dst = Sg::STAGED ? st : out;
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
                arow_put<E, D>(st + Sg::R1A, c0, r, kt);
                arow_put<E, D>(st + Sg::R2A, c0, r, qt);
                arow_put<E, D>(st + Sg::KHA, c0, r, kh);
            }
        }
    }
    wave_sync_lds();
    {
        const f32x4 akk = arow_gram<E, D>(st + Sg::R1A, st + Sg::KHA);
        const f32x4 aqk = arow_gram<E, D>(st + Sg::R2A, st + Sg::KHA);
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
    if constexpr (!Sg::STAGED) {
        copy_out(out + P::KA, st + Sg::R1A, P::AROW);
        copy_out(out + P::QA, st + Sg::R2A, P::AROW);
    }
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
                arow_put<E, D>(st + Sg::R1B, c0, r, kt);   // Kt_b, unscaled
                arow_put<E, D>(st + Sg::R2B, c0, r, qt);   // Qt_b, unscaled
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
                *reinterpret_cast<V8<E>*>(kd2_dst + P::kd2_offset(col / 16, gg, col % 16)) = x;
            }
            reinterpret_cast<float*>(st + Sg::small(P::GAB))[col] = gamA[e] * gamB[e];
        }
    }
    wave_sync_lds();
    {
        const f32x4 akk = arow_gram<E, D>(st + Sg::R1B, st + Sg::KHB);
        const f32x4 aqk = arow_gram<E, D>(st + Sg::R2B, st + Sg::KHB);
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
            arow_put<E, D>(st + Sg::R1B, c0, r, kt);
            arow_put<E, D>(st + Sg::R2B, c0, r, qt);
        }
    }
    const float bjb = b.bj;
    wave_sync_lds();
    {
        // M_kb = (Kt_b Diag(gam_a)) Kh_a^T, M_qb = (Qt_b Diag(gam_a)) Kh_a^T
        const f32x4 mkb = arow_gram<E, D>(st + Sg::R1B, st + Sg::KHA);
        const f32x4 mqb = arow_gram<E, D>(st + Sg::R2B, st + Sg::KHA);
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
    if constexpr (!Sg::STAGED) {
        copy_out(out + P::KB, st + Sg::R1B, P::AROW);
        copy_out(out + P::QB, st + Sg::R2B, P::AROW);
        copy_out(out + P::TMA, st + Sg::SMALL, P::BYTES - P::TMA);
    }
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

// No work between the products of a step (the default of the hooks below).
struct NoHook {
    __device__ void operator()(int) const {}
};

// The first products of a pair (bf16): S packed once, x_a = Kt_a S and
// x_b = (Kt_b Diag(gam_a)) S.  They need only the operands read one pair
// ahead, so the wave issues them before waiting for this pair's other reads.
// hook(s) runs after the products of A-row slot s (of the last column
// block): a caller can issue other work between them.
template <typename E, int D, int NB, typename Hook = NoHook>
__device__ __forceinline__ void pair_x(const POps<E, D>& c, const f32x4 (&S)[NB][D / 16],
                                       bf16x8 (&sb)[NB][PBlk<E, D>::NSLOT], f32x4 (&xa)[NB],
                                       f32x4 (&xb)[NB], Hook hook = Hook{}) {
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
            if (nb == NB - 1) hook(s);
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
// hook(m) runs after the product of row tile m.
template <typename E, int D, typename Hook = NoHook>
__device__ __forceinline__ void pair_supdate(const POps<E, D>& c, f32x4 (&S)[D / 16], const bf16x8& u2,
                                             Hook hook = Hook{}) {
    static_for<0, PBlk<E, D>::MT>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        S[m] = mma_bf16_k32(c.kd2[m], u2, S[m] * gab_tile<m>(c.gv));
        hook(m);
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

}  // namespace kda
