// kda_chunk.hpp -- device code shared by the chunkwise prefill kernels:
// the single-chunk factor block and its producer (gate + intra-chunk) and
// consumer (one chunk of the state chain), chunk addressing, the state tile
// in registers, and workgroup synchronisation helpers.
//
// Source of the method: dev.to "Kimi K3 Architecture: Scaling 2.8T Parameters
// for Long-Context Multimodal MoE", section "The Sequence Bottleneck: Hybrid
// KDA and Gated MLA" (lower-bounded gate, 16-token tiles, chunkwise parallel
// form).  For a chunk of rows r = 0..15 with G_r the inclusive chunk-local
// cumulative log-decay:
//
//   Kt = k e^{G}, Kh = k e^{-G}, Qt = q e^{G}, Kd = k e^{G_15 - G}, gam = e^{G_15}
//   Akk = tril_{-1}(Diag(beta) Kt Kh^T),   Aqk = tril_0(Qt Kh^T)
//   Tm  = (I + Akk)^{-1} Diag(beta)                    (16x16 forward substitution)
//   U   = Tm (V - Kt S)                                (delta-rule corrections)
//   O   = Qt S + Aqk U
//   S  <- Diag(gam) S + Kd^T U
#pragma once

#include <type_traits>

#include "kda_device.hpp"

namespace kda {

// --------------------------------------------------------------- factor block

template <typename E, int D>
struct Blk {
    static constexpr bool kBF16 = std::is_same<E, bf16>::value;
    static constexpr int ES = (int)sizeof(E);
    static constexpr int KPL = 16 / ES;              // elements per lane per A-row slot
    static constexpr int NSLOT = D / (4 * KPL);      // A-row slots covering the d_k axis
    static constexpr int MT = D / 16;                // 16-row tiles of S
    static constexpr int OPB = 4 * ES;               // bytes per lane: Kd^T tile, Tm, Aqk
    static constexpr int KT = 0;
    static constexpr int QT = KT + NSLOT * 1024;
    static constexpr int KD = QT + NSLOT * 1024;
    static constexpr int TM = KD + MT * kWave * OPB;
    static constexpr int AQ = TM + kWave * OPB;
    static constexpr int GAM = AQ + kWave * OPB;
    static constexpr int BYTES = GAM + D * 4;
    static_assert(BYTES % 16 == 0, "factor block must be 16-byte granular");
    // per-wave producer scratch: Kh in the A-row layout, then Akk (16x16 fp32)
    static constexpr int SCR_KH = 0;
    static constexpr int SCR_AKK = NSLOT * 1024;
    static constexpr int SCR_BYTES = SCR_AKK + 16 * 16 * 4;
    // producer lane ownership: NCL consecutive key columns per lane
    static constexpr int NCL = D >= 64 ? D / 64 : 1;
    static constexpr int NACT = D / NCL;             // lanes that own columns
    static constexpr int NWORD = (NCL * ES + 3) / 4; // 32-bit words per row segment

    // A-row layout: slot s, lane (r, g) = 16g + r holds, as element p, key
    // column 4*KPL*s + 16*(p/4) + 4g + (p%4) of row r; this K order matches
    // S's accumulator rows 16m + 4g + i with m = 2s + p/4 (bf16, 16x16x32) or
    // m = s, i = p (fp32, 16x16x4).  The 16-byte chunk of lane (r, g) is
    // stored at position 16g + (r ^ ((4s + g) & 15)) so that a producer lane
    // writing one row of its columns and a consumer lane reading its whole
    // chunk both spread over the LDS banks.
    __device__ static __forceinline__ int arow_chunk(int s, int g, int r) {
        return s * 1024 + (g * 16 + (r ^ ((4 * s + g) & 15))) * 16;
    }
    __device__ static __forceinline__ int arow_offset(int col, int r) {
        const int s = col / (4 * KPL), w = col % (4 * KPL);
        const int p = 4 * (w / 16) + (w % 4);
        const int g = (w % 16) / 4;
        return arow_chunk(s, g, r) + p * ES;
    }
    // Kd^T tile m, lane (c_l, g) = 16g + c_l holds Kd[4g + 0..3][16m + c_l];
    // stored at entry 16g + (c_l ^ (m & 15)).
    __device__ static __forceinline__ int kd_offset(int m, int g, int cl) {
        return KD + m * kWave * OPB + (g * 16 + (cl ^ (m & 15))) * OPB;
    }
};

template <typename E>
using V16 = typename std::conditional<std::is_same<E, bf16>::value, bf16x8, f32x4>::type;
template <typename E>
using V4 = typename std::conditional<std::is_same<E, bf16>::value, bf16x4, f32x4>::type;

template <typename E>
__device__ __forceinline__ V4<E> cvt4(float a, float b, float c, float d) {
    V4<E> r;
    r[0] = from_f32<E>(a); r[1] = from_f32<E>(b); r[2] = from_f32<E>(c); r[3] = from_f32<E>(d);
    return r;
}

template <typename E>
__device__ __forceinline__ f32x4 widen4(V4<E> x) {
    return f32x4{to_f32(x[0]), to_f32(x[1]), to_f32(x[2]), to_f32(x[3])};
}

// Code-motion fence: memory operations issued before it stay before it (an
// empty asm with a memory clobber stops IR-level sinking; sched_barrier stops
// the machine scheduler).  It does not wait for them to complete.
__device__ __forceinline__ void pin_issued() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// --------------------------------------------------------------- producer

struct ChunkPos {
    size_t row0;     // element offset of (b, t0, h, 0) in q/k/z/v/o
    size_t rstride;  // elements between consecutive tokens: H * D
    size_t brow0;    // offset of (b, t0, h) in beta
    int bstride;     // H
    int L;           // valid rows
};

template <int D>
__device__ __forceinline__ ChunkPos chunk_pos(int b, int h, int n, int T, int H) {
    ChunkPos c;
    const int t0 = n * kChunk;
    c.brow0 = ((size_t)b * T + t0) * H + h;
    c.row0 = c.brow0 * D;
    c.rstride = (size_t)H * D;
    c.bstride = H;
    c.L = min(kChunk, T - t0);
    return c;
}

// Buffer over the chunk's rows of a [.., T, H, D] tensor of element size es:
// from row 0 of the chunk to the end of its last valid row, so every access
// to a row past the chunk's end falls outside and reads 0 / is dropped.  A
// chunk past the end of the sequence (L <= 0) gets an empty buffer.
template <int D>
__device__ __forceinline__ Rsrc chunk_rsrc(const void* base, const ChunkPos& c, int es) {
    // branch-free (a branch here would split the callers' loop bodies): the
    // wrapped value for L <= 0 is multiplied by 0
    const uint32_t valid = c.L > 0 ? 1u : 0u;
    const uint32_t bytes = (uint32_t)(((size_t)(c.L - 1) * c.rstride + D) * es) * valid;
    return make_rsrc((const char*)base + c.row0 * es, bytes);
}

// Raw producer inputs of one chunk, kept in registers so the next chunk's
// loads can be in flight while the current one is computed.  Lane l owns key
// columns (l mod NACT) * NCL + e, all 16 rows.
template <typename E, int D>
struct ProdIn {
    static constexpr int NW = Blk<E, D>::NWORD;
    uint32_t q[16][NW], k[16][NW], z[16][NW];
    float bj;   // beta of chunk row (lane & 15); 0 past the chunk's end
    int L;      // valid rows of the chunk (0 = no chunk)
};

template <typename E, int NCL>
__device__ __forceinline__ void load_seg(Rsrc r, int off, uint32_t* w) {
    constexpr int NB = NCL * (int)sizeof(E);
    if constexpr (NB == 8) {
        const u32x2 a = buf_load<u32x2>(r, off);
        w[0] = a[0]; w[1] = a[1];
    } else if constexpr (NB == 4) {
        w[0] = buf_load<uint32_t>(r, off);
    } else {
        static_assert(NB == 2, "row segment of 2, 4 or 8 bytes");
        w[0] = buf_load<unsigned short>(r, off);
    }
}

template <typename E, int NCL, int NW>
__device__ __forceinline__ void unpack_seg(const uint32_t (&w)[NW], float (&f)[NCL]) {
    if constexpr (std::is_same<E, float>::value) {
#pragma unroll
        for (int i = 0; i < NCL; ++i) f[i] = __builtin_bit_cast(float, w[i]);
    } else {
        f[0] = __builtin_bit_cast(float, w[0] << 16);
        if constexpr (NCL == 2) f[1] = __builtin_bit_cast(float, w[0] & 0xffff0000u);
    }
}

// WQ = false: q is not read (a pass that produces only the end state).
template <typename E, int D, bool WQ = true>
__device__ __forceinline__ void prod_load(ProdIn<E, D>& in, const E* __restrict__ q,
                                          const E* __restrict__ k, const E* __restrict__ z,
                                          const float* __restrict__ beta, const ChunkPos& c) {
    using B = Blk<E, D>;
    constexpr int ES = (int)sizeof(E);
    const int lane = lane_id();
    const int c0 = (lane % B::NACT) * B::NCL;
    in.L = c.L;
    // Rows past the chunk's end lie outside the buffers and read as zero.
    const Rsrc rq = chunk_rsrc<D>(q, c, ES), rk = chunk_rsrc<D>(k, c, ES), rz = chunk_rsrc<D>(z, c, ES);
    // The row stride passes through an empty asm so that the 16 row offsets
    // are formed at each call rather than hoisted out of a producer's loop,
    // where they would hold 16 VGPRs for the whole loop.
    int rowb = (int)(c.rstride * ES);
    asm volatile("" : "+s"(rowb));
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int off = c0 * ES + r * rowb;
        if constexpr (WQ) load_seg<E, B::NCL>(rq, off, in.q[r]);
        load_seg<E, B::NCL>(rk, off, in.k[r]);
        load_seg<E, B::NCL>(rz, off, in.z[r]);
    }
    // beta of rows 0 .. L-1; a chunk past the end of the sequence (L <= 0)
    // gets an empty buffer
    const Rsrc rb = make_rsrc(beta + c.brow0,
                              c.L > 0 ? (uint32_t)(((c.L - 1) * c.bstride + 1) * 4) : 0u);
    in.bj = __builtin_bit_cast(float, buf_load<uint32_t>(rb, (lane & 15) * c.bstride * 4));
}

// Gate + intra-chunk stage of one chunk (one wave).  Writes the factor block
// `blk` (LDS) using the wave-private scratch `scr` (LDS).  With DIAG, fp32
// copies of Tm [16][16], Aqk [16][16] and gam [D] also go to dTm, dAqk, dgam.
// WQ = false: the output factors (Qt, Aqk) are neither formed nor written.
template <typename E, int D, bool DIAG, bool WQ = true>
__device__ __forceinline__ void prod_compute(const ProdIn<E, D>& in, const GateConsts& gc,
                                             char* __restrict__ blk, char* __restrict__ scr,
                                             float* dTm, float* dAqk, float* dgam) {
    using B = Blk<E, D>;
    constexpr int NCL = B::NCL;
    const int lane = lane_id();
    const bool owner = lane < B::NACT;
    const int c0 = (lane % B::NACT) * NCL;
    const int L = in.L;

    // ---- gate: retention a = exp(g_min Sigmoid(e^{A_h} z)) (a = 1 on padded
    // rows), then the chunk's decay products along the rows of each column:
    //   P_r  = e^{G_r}       = a_0 ... a_r        (inclusive prefix)
    //   Qs_r = e^{G_15 - G_r} = a_{r+1} ... a_15  (exclusive suffix)
    float P[16][NCL], Qs[16][NCL], gam[NCL], rgam[NCL];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        float zf[NCL];
        unpack_seg<E, NCL, B::NWORD>(in.z[r], zf);
#pragma unroll
        for (int e = 0; e < NCL; ++e) {
            const float a = gate_alpha_row(gc, zf[e], r < L ? 1.f : 0.f);
            Qs[r][e] = a;                           // holds a_r until the suffix pass
            P[r][e] = r == 0 ? a : P[r - 1][e] * a;
        }
    }
#pragma unroll
    for (int e = 0; e < NCL; ++e) {
        gam[e] = P[15][e];
        rgam[e] = fast_rcp(gam[e]);
        float run = 1.f;
#pragma unroll
        for (int r = 15; r >= 0; --r) {
            const float a = Qs[r][e];
            Qs[r][e] = run;
            run *= a;
        }
    }

    // ---- factors -> LDS in their consumer layouts
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        float kf[NCL], qf[NCL];
        unpack_seg<E, NCL, B::NWORD>(in.k[r], kf);
        if constexpr (WQ) unpack_seg<E, NCL, B::NWORD>(in.q[r], qf);
        float kt[NCL], qt[NCL], kh[NCL];
#pragma unroll
        for (int e = 0; e < NCL; ++e) {
            kt[e] = kf[e] * P[r][e];
            qt[e] = WQ ? qf[e] * P[r][e] : 0.f;
            const float kd = kf[e] * Qs[r][e];
            kh[e] = kd * rgam[e];
            Qs[r][e] = kd;                          // keep Kd for the transposed tile
        }
        if (owner) {
            const int off = B::arow_offset(c0, r);
            if constexpr (NCL == 2 && B::kBF16) {
                bf16x2 a{(bf16)kt[0], (bf16)kt[1]}, b{(bf16)qt[0], (bf16)qt[1]}, c{(bf16)kh[0], (bf16)kh[1]};
                *reinterpret_cast<bf16x2*>(blk + B::KT + off) = a;
                if constexpr (WQ) *reinterpret_cast<bf16x2*>(blk + B::QT + off) = b;
                *reinterpret_cast<bf16x2*>(scr + B::SCR_KH + off) = c;
            } else if constexpr (NCL == 2) {
                *reinterpret_cast<f32x2*>(blk + B::KT + off) = f32x2{kt[0], kt[1]};
                if constexpr (WQ) *reinterpret_cast<f32x2*>(blk + B::QT + off) = f32x2{qt[0], qt[1]};
                *reinterpret_cast<f32x2*>(scr + B::SCR_KH + off) = f32x2{kh[0], kh[1]};
            } else {
                *reinterpret_cast<E*>(blk + B::KT + off) = from_f32<E>(kt[0]);
                if constexpr (WQ) *reinterpret_cast<E*>(blk + B::QT + off) = from_f32<E>(qt[0]);
                *reinterpret_cast<E*>(scr + B::SCR_KH + off) = from_f32<E>(kh[0]);
            }
        }
    }
    if (owner) {
#pragma unroll
        for (int e = 0; e < NCL; ++e) {
            const int col = c0 + e;
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<V4<E>*>(blk + B::kd_offset(col / 16, g, col % 16)) =
                    cvt4<E>(Qs[4 * g][e], Qs[4 * g + 1][e], Qs[4 * g + 2][e], Qs[4 * g + 3][e]);
            reinterpret_cast<float*>(blk + B::GAM)[col] = gam[e];
            if constexpr (DIAG) dgam[col] = gam[e];
        }
    }
    wave_sync_lds();

    // ---- Akk = Kt Kh^T and Aqk = Qt Kh^T on MFMA (K = d_k).  Kh^T as the B
    // operand has the same lane layout as Kh as an A operand.
    const int ci = lane & 15, g = lane >> 4;
    f32x4 akk = zero4(), aqk = zero4();
#pragma unroll
    for (int s = 0; s < B::NSLOT; ++s) {
        const int off = B::arow_chunk(s, g, ci);
        const V16<E> kt = *reinterpret_cast<const V16<E>*>(blk + B::KT + off);
        const V16<E> kh = *reinterpret_cast<const V16<E>*>(scr + B::SCR_KH + off);
        if constexpr (B::kBF16) {
            akk = mma_bf16_k32(kt, kh, akk);
            if constexpr (WQ) {
                const V16<E> qt = *reinterpret_cast<const V16<E>*>(blk + B::QT + off);
                aqk = mma_bf16_k32(qt, kh, aqk);
            }
        } else {
#pragma unroll
            for (int p = 0; p < 4; ++p) akk = mma_f32_k4(kt[p], kh[p], akk);
            if constexpr (WQ) {
                const V16<E> qt = *reinterpret_cast<const V16<E>*>(blk + B::QT + off);
#pragma unroll
                for (int p = 0; p < 4; ++p) aqk = mma_f32_k4(qt[p], kh[p], aqk);
            }
        }
    }
    // accumulator layout: lane (i = lane % 16, g) holds rows 4g + p, column i
    float* akk_s = reinterpret_cast<float*>(scr + B::SCR_AKK);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int r = 4 * g + p;
        const float br = __shfl(in.bj, r);
        akk_s[r * 16 + ci] = ci < r ? br * akk[p] : 0.f;
        if constexpr (WQ) {
            const float aq = ci <= r ? aqk[p] : 0.f;
            // A layout for the 16x16x16 / 16x16x4 consumer: lane (r, ci/4), element ci%4
            *reinterpret_cast<E*>(blk + B::AQ + ((ci >> 2) * 16 + r) * B::OPB + (ci & 3) * B::ES) =
                from_f32<E>(aq);
            if constexpr (DIAG) dAqk[r * 16 + ci] = aq;
        }
    }
    wave_sync_lds();

    // ---- Tm = (I + Akk)^{-1} Diag(beta): lane j < 16 solves column j by
    // forward substitution in fp32.
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
        const float bj = in.bj;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float t = x[r] * bj;
            *reinterpret_cast<E*>(blk + B::TM + ((j >> 2) * 16 + r) * B::OPB + (j & 3) * B::ES) =
                from_f32<E>(t);
            if constexpr (DIAG) dTm[r * 16 + j] = t;
        }
    }
    wave_sync_lds();
}

// --------------------------------------------------------------- consumer

// Factor-block operands of one chunk in the consumer's registers.
template <typename E, int D>
struct COps {
    using B = Blk<E, D>;
    V16<E> kt[B::NSLOT], qt[B::NSLOT];
    V4<E> kd[B::MT];
    V4<E> tm, aq;
    f32x2 gv;   // two values of gam per lane: row_tile<m>(gv) is gam of row tile m
};

// Factor-block sources: LDS (fused kernel) or a buffer over a workspace
// block (inter kernel); both read the same byte offsets.
struct LdsSrc {
    const char* base;
    template <typename T> __device__ __forceinline__ T ld(int off) const {
        return *reinterpret_cast<const T*>(base + off);
    }
};
struct BufSrc {
    Rsrc r;
    template <typename T> __device__ __forceinline__ T ld(int off) const {
        if constexpr (sizeof(T) == 16) return __builtin_bit_cast(T, buf_load<u32x4>(r, off));
        else if constexpr (sizeof(T) == 8) return __builtin_bit_cast(T, buf_load<u32x2>(r, off));
        else return __builtin_bit_cast(T, buf_load<uint32_t>(r, off));
    }
};

// WQ = false: the output factors (Qt, Aqk) are not read.
template <typename E, int D, typename Src, bool WQ = true>
__device__ __forceinline__ void cops_load(COps<E, D>& c, const Src& src) {
    using B = Blk<E, D>;
    const int lane = lane_id(), g = lane >> 4, r = lane & 15;
#pragma unroll
    for (int s = 0; s < B::NSLOT; ++s) {
        const int off = B::arow_chunk(s, g, r);
        c.kt[s] = src.template ld<V16<E>>(B::KT + off);
        if constexpr (WQ) c.qt[s] = src.template ld<V16<E>>(B::QT + off);
    }
#pragma unroll
    for (int m = 0; m < B::MT; ++m) {
        c.kd[m] = src.template ld<V4<E>>(B::kd_offset(m, g, r));
    }
    c.gv = src.template ld<f32x2>(B::GAM + row_vec_offset<D>(g, r));
    c.tm = src.template ld<V4<E>>(B::TM + lane * B::OPB);
    if constexpr (WQ) c.aq = src.template ld<V4<E>>(B::AQ + lane * B::OPB);
}

// V of one chunk for NB 16-column blocks, accumulator layout (rows 4g + p),
// kept as the raw loaded words (a bf16 pattern in the low 16 bits, or fp32
// bits) and widened only when the chunk is consumed, so the loads stay in
// flight across the chunk steps in between; rows past the chunk's end read 0.
template <int D, int NB>
__device__ __forceinline__ void v_load(u32x4 (&V)[NB], const void* __restrict__ v, int es,
                                       const ChunkPos& c, int col0) {
    const int lane = lane_id(), j = lane & 15, g = lane >> 4;
    const Rsrc rv = chunk_rsrc<D>(v, c, es);
    const int rowb = (int)(c.rstride * es);
    const int base = 4 * g * rowb + (col0 + j) * es;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int off = base + p * rowb + 16 * nb * es;
            V[nb][p] = es == 2 ? (uint32_t)buf_load<unsigned short>(rv, off)
                               : buf_load<uint32_t>(rv, off);
        }
}

template <typename E>
__device__ __forceinline__ f32x4 v_widen(u32x4 x) {
    if constexpr (std::is_same<E, bf16>::value) x <<= 16;
    return __builtin_bit_cast(f32x4, x);
}

// O of one chunk; stores to rows past the chunk's end are dropped.
template <typename E, int D, int NB>
__device__ __forceinline__ void o_store(const f32x4 (&O)[NB], E* __restrict__ o, const ChunkPos& c,
                                        int col0) {
    constexpr int ES = (int)sizeof(E);
    const int lane = lane_id(), j = lane & 15, g = lane >> 4;
    const Rsrc ro = chunk_rsrc<D>(o, c, ES);
    const int rowb = (int)(c.rstride * ES);
    const int base = 4 * g * rowb + (col0 + j) * ES;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int off = base + p * rowb + 16 * nb * ES;
            const E x = from_f32<E>(O[nb][p]);
            if constexpr (ES == 2) buf_store_u16(ro, off, __builtin_bit_cast(unsigned short, x));
            else buf_store_u32(ro, off, __builtin_bit_cast(uint32_t, x));
        }
}

// One chunk of the state chain for NB 16-column blocks of S.  WQ = false:
// the state only (O is left unset).
template <typename E, int D, int NB, bool WQ = true>
__device__ __forceinline__ void chunk_step(const COps<E, D>& c, f32x4 (&S)[NB][D / 16],
                                           const f32x4 (&Vf)[NB], f32x4 (&O)[NB]) {
    using B = Blk<E, D>;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        f32x4 x = zero4(), o = zero4();
        const f32x4 V = Vf[nb];
        if constexpr (B::kBF16) {
#pragma unroll
            for (int s = 0; s < B::NSLOT; ++s) {
                const bf16x8 sb = pack8(S[nb][2 * s], S[nb][2 * s + 1]);
                x = mma_bf16_k32(c.kt[s], sb, x);      // Kt S
                if constexpr (WQ) o = mma_bf16_k32(c.qt[s], sb, o);      // Qt S
            }
            const f32x4 y = V - x;
            const f32x4 u = mma_bf16_k16(c.tm, pack4(y), zero4());   // U = Tm (V - Kt S)
            const bf16x4 ub = pack4(u);
            // Aqk U goes to its own accumulator: an MFMA of one shape must not
            // take as srcC the result of an MFMA of another shape still in
            // flight (16x16x32 -> 16x16x16 chains read stale srcC on gfx950).
            if constexpr (WQ) o += mma_bf16_k16(c.aq, ub, zero4());  // + Aqk U
            static_for<0, B::MT>([&](auto mc) {   // Diag(gam) S + Kd^T U
                constexpr int m = decltype(mc)::value;
                // (each column block its own broadcasts: each folds into its multiply)
                const f32x4 gm = nb == 0 ? row_tile<m>(c.gv) : row_tile_mov<m>(c.gv);
                S[nb][m] = mma_bf16_k16(c.kd[m], ub, S[nb][m] * gm);
            });
        } else {
#pragma unroll
            for (int m = 0; m < B::MT; ++m)
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    x = mma_f32_k4(c.kt[m][p], S[nb][m][p], x);
                    if constexpr (WQ) o = mma_f32_k4(c.qt[m][p], S[nb][m][p], o);
                }
            const f32x4 y = V - x;
            f32x4 u = zero4();
#pragma unroll
            for (int p = 0; p < 4; ++p) u = mma_f32_k4(c.tm[p], y[p], u);
            if constexpr (WQ) {
#pragma unroll
                for (int p = 0; p < 4; ++p) o = mma_f32_k4(c.aq[p], u[p], o);
            }
            static_for<0, B::MT>([&](auto mc) {
                constexpr int m = decltype(mc)::value;
                f32x4 s = S[nb][m] * row_tile<m>(c.gv);
#pragma unroll
                for (int p = 0; p < 4; ++p) s = mma_f32_k4(c.kd[m][p], u[p], s);
                S[nb][m] = s;
            });
        }
        if constexpr (WQ) O[nb] = o;
    }
}

// State tile <-> memory (accumulator layout: lane (j, g) holds rows 16m + 4g + p).
template <int D, int NB>
__device__ __forceinline__ void state_load(f32x4 (&S)[NB][D / 16], const float* __restrict__ S0,
                                           int col0) {
    const int lane = lane_id(), j = lane & 15, g = lane >> 4;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int m = 0; m < D / 16; ++m)
#pragma unroll
            for (int p = 0; p < 4; ++p)
                S[nb][m][p] = S0 ? S0[(size_t)(16 * m + 4 * g + p) * D + col0 + 16 * nb + j] : 0.f;
}

template <int D, int NB>
__device__ __forceinline__ void state_store(const f32x4 (&S)[NB][D / 16], float* __restrict__ ST,
                                            int col0) {
    const int lane = lane_id(), j = lane & 15, g = lane >> 4;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int m = 0; m < D / 16; ++m)
#pragma unroll
            for (int p = 0; p < 4; ++p)
                ST[(size_t)(16 * m + 4 * g + p) * D + col0 + 16 * nb + j] = S[nb][m][p];
}

// Interleaved column blocks (fused plan at bf16, two 16-column blocks per
// wave): in a wave's 32 value columns col0 .. col0 + 31, block nb of lane
// column j is column col0 + 2 j + nb.  The value columns evolve
// independently, so any assignment is exact; this one makes the two blocks'
// elements of a row adjacent, so V and O move as 4-byte pairs (one access per
// row and lane instead of two) and states as 8-byte pairs.
template <int D>
__device__ __forceinline__ void state_load_il(f32x4 (&S)[2][D / 16], const float* __restrict__ S0,
                                              int col0) {
    const int lane = lane_id(), j = lane & 15, g = lane >> 4;
#pragma unroll
    for (int m = 0; m < D / 16; ++m)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const f32x2 x = S0 ? *reinterpret_cast<const f32x2*>(
                                     S0 + (size_t)(16 * m + 4 * g + p) * D + col0 + 2 * j)
                               : f32x2{0.f, 0.f};
            S[0][m][p] = x[0];
            S[1][m][p] = x[1];
        }
}

template <int D>
__device__ __forceinline__ void state_store_il(const f32x4 (&S)[2][D / 16], float* __restrict__ ST,
                                               int col0) {
    const int lane = lane_id(), j = lane & 15, g = lane >> 4;
#pragma unroll
    for (int m = 0; m < D / 16; ++m)
#pragma unroll
        for (int p = 0; p < 4; ++p)
            *reinterpret_cast<f32x2*>(ST + (size_t)(16 * m + 4 * g + p) * D + col0 + 2 * j) =
                f32x2{S[0][m][p], S[1][m][p]};
}

// V of one chunk, rows 4g + p of the lane's column pair (bf16): one word per
// row, block 0 in the low half.
struct VPair {
    uint32_t w[4];
};

template <int D>
__device__ __forceinline__ void v_load_il(VPair& V, const bf16* __restrict__ v, const ChunkPos& c,
                                          int col0) {
    const int lane = lane_id(), j = lane & 15, g = lane >> 4;
    const Rsrc rv = chunk_rsrc<D>(v, c, 2);
    const int rowb = (int)(c.rstride * 2);
#pragma unroll
    for (int p = 0; p < 4; ++p) V.w[p] = buf_load<uint32_t>(rv, (4 * g + p) * rowb + (col0 + 2 * j) * 2);
}

__device__ __forceinline__ void v_widen_il(const VPair& V, f32x4 (&Vf)[2]) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        Vf[0][p] = __builtin_bit_cast(float, V.w[p] << 16);
        Vf[1][p] = __builtin_bit_cast(float, V.w[p] & 0xffff0000u);
    }
}

// O of one chunk (both blocks); stores to rows past the chunk's end are dropped.
template <int D>
__device__ __forceinline__ void o_store_il(const f32x4 (&O)[2], bf16* __restrict__ o,
                                           const ChunkPos& c, int col0) {
    const int lane = lane_id(), j = lane & 15, g = lane >> 4;
    const Rsrc ro = chunk_rsrc<D>(o, c, 2);
    const int rowb = (int)(c.rstride * 2);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const bf16x2 x{(bf16)O[0][p], (bf16)O[1][p]};
        buf_store_u32(ro, (4 * g + p) * rowb + (col0 + 2 * j) * 2, __builtin_bit_cast(uint32_t, x));
    }
}

// Workgroup id -> (unit = b*H + h, column tile).  Workgroups are dispatched
// round-robin over the 8 XCDs; all column tiles of one head get the same
// id mod 8 so they share an XCD's L2.
__device__ __forceinline__ bool map_unit(int nct, int units, int& u, int& ct) {
    const int bid = (int)blockIdx.x;
    const int xcd = bid & 7, slot = bid >> 3;
    u = (slot / nct) * 8 + xcd;
    ct = slot % nct;
    return u < units;
}

// Workgroup barrier usable from role-specific code paths: every wave of the
// workgroup executes the same number of these, from whichever branch.
__device__ __forceinline__ void wg_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Bounded poll of an LDS flag: true once *flag >= target, false after
// kSpinLimit polls.  The flag protocols of the split plan never need the
// bound (every wait is released by a wave that does not wait on the waiter;
// tests/test_flag_protocol.py checks this on a model of the protocol); it only
// turns a protocol error into a visible one instead of a hang: a wave that
// gives up poisons what it produces with NaN (poison_state, kNaNWord), so the
// outputs and the final state of its columns come out NaN.
constexpr int kSpinLimit = 1 << 22;

__device__ __forceinline__ bool spin_until_ge(const int* flag, int target) {
    bool ok = false;
    for (int it = 0; it < kSpinLimit; ++it) {
        if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) {
            ok = true;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    // later LDS reads stay after the poll that released them
    asm volatile("" ::: "memory");
    return ok;
}

// A 32-bit word that is NaN read as one fp32 value or as two bf16 values.
constexpr uint32_t kNaNWord = 0x7FC07FC0u;

// Sets a state tile held in registers to NaN (a wave that gave up a wait).
template <int N>
__device__ __forceinline__ void poison_state(f32x4 (&S)[N]) {
    const float nan = __builtin_bit_cast(float, kNaNWord);
#pragma unroll
    for (int m = 0; m < N; ++m) S[m] = f32x4{nan, nan, nan, nan};
}

}  // namespace kda
