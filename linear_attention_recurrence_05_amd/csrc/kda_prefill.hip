// kda_prefill.hip -- chunkwise KDA prefill for gfx950.
//
// Source of the method: dev.to "Kimi K3 Architecture: Scaling 2.8T Parameters
// for Long-Context Multimodal MoE", section "The Sequence Bottleneck: Hybrid
// KDA and Gated MLA": the lower-bounded gate g = g_min Sigmoid(e^{A_h} z),
// 16-token tiles whose cumulative log-decay stays inside (-80, 0), and
// chunkwise parallel execution with the within-chunk ("diagonal") and state
// ("off-diagonal") tiles as dense matrix products.  The chunk equations are
// derived from S_t = (I - b k k^T) Diag(a) S_{t-1} + b k v^T, o_t = S_t^T q_t.
// For a chunk of rows r = 0..15 with G_r the inclusive chunk-local cumulative
// log-decay (e^{G_r} = product of the retentions up to r):
//
//   Kt = k e^{G}, Kh = k e^{-G}, Qt = q e^{G}, Kd = k e^{G_15 - G}, gam = e^{G_15}
//   Akk = tril_{-1}(Diag(beta) Kt Kh^T),   Aqk = tril_0(Qt Kh^T)
//   Tm  = (I + Akk)^{-1} Diag(beta)                    (16x16 forward substitution)
//   U   = Tm (V - Kt S)                                (delta-rule corrections)
//   O   = Qt S + Aqk U
//   S  <- Diag(gam) S + Kd^T U
//
// Stages, written as device functions and composed into kernels:
//   producer (gate + intra-chunk): q, k, z, beta of one chunk -> a "factor
//       block" holding Kt, Qt, Kd^T, Tm, Aqk, gam, each in the lane layout
//       its MFMA consumer reads; one wave per chunk.  Each lane owns whole
//       key columns (all 16 rows), so the decay products are in-lane
//       running products and every row load is one coalesced 256-byte line.
//   consumer (inter-chunk): one wave advances 16*NB value columns of the fp32
//       state by one chunk.  S lives in MFMA accumulator registers for the
//       whole sequence; the K order of every product is chosen so that the
//       accumulator layout of S (and of U) is directly the B operand of the
//       next product, so the serial chain never touches LDS.
//   kernels: "split" = an intra kernel over all chunks writing factor blocks
//       to a workspace + an inter kernel whose loader waves stream them into
//       an LDS ring ahead of the state chain; "fused" = one kernel per
//       (b, h, column tile) with
//       four producer waves filling one half of a double-buffered LDS ring
//       while the consumer waves run the state chain over the other half.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "kda_device.hpp"
#include "kda_launch.hpp"

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
    const size_t bytes = c.L > 0 ? ((size_t)(c.L - 1) * c.rstride + D) * es : 0;
    return make_rsrc((const char*)base + c.row0 * es, (uint32_t)bytes);
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

template <typename E, int D>
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
    const int rowb = (int)(c.rstride * ES);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int off = c0 * ES + r * rowb;
        load_seg<E, B::NCL>(rq, off, in.q[r]);
        load_seg<E, B::NCL>(rk, off, in.k[r]);
        load_seg<E, B::NCL>(rz, off, in.z[r]);
    }
    const Rsrc rb = make_rsrc(beta + c.brow0, (uint32_t)(((c.L - 1) * c.bstride + 1) * 4));
    in.bj = __builtin_bit_cast(float, buf_load<uint32_t>(rb, (lane & 15) * c.bstride * 4));
}

// Gate + intra-chunk stage of one chunk (one wave).  Writes the factor block
// `blk` (LDS) using the wave-private scratch `scr` (LDS).  With DIAG, fp32
// copies of Tm [16][16], Aqk [16][16] and gam [D] also go to dTm, dAqk, dgam.
template <typename E, int D, bool DIAG>
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
            const float a = r < L ? gate_alpha(gc, gate_sigmoid(gc, zf[e])) : 1.f;
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
        unpack_seg<E, NCL, B::NWORD>(in.q[r], qf);
        float kt[NCL], qt[NCL], kh[NCL];
#pragma unroll
        for (int e = 0; e < NCL; ++e) {
            kt[e] = kf[e] * P[r][e];
            qt[e] = qf[e] * P[r][e];
            const float kd = kf[e] * Qs[r][e];
            kh[e] = kd * rgam[e];
            Qs[r][e] = kd;                          // keep Kd for the transposed tile
        }
        if (owner) {
            const int off = B::arow_offset(c0, r);
            if constexpr (NCL == 2 && B::kBF16) {
                bf16x2 a{(bf16)kt[0], (bf16)kt[1]}, b{(bf16)qt[0], (bf16)qt[1]}, c{(bf16)kh[0], (bf16)kh[1]};
                *reinterpret_cast<bf16x2*>(blk + B::KT + off) = a;
                *reinterpret_cast<bf16x2*>(blk + B::QT + off) = b;
                *reinterpret_cast<bf16x2*>(scr + B::SCR_KH + off) = c;
            } else if constexpr (NCL == 2) {
                *reinterpret_cast<f32x2*>(blk + B::KT + off) = f32x2{kt[0], kt[1]};
                *reinterpret_cast<f32x2*>(blk + B::QT + off) = f32x2{qt[0], qt[1]};
                *reinterpret_cast<f32x2*>(scr + B::SCR_KH + off) = f32x2{kh[0], kh[1]};
            } else {
                *reinterpret_cast<E*>(blk + B::KT + off) = from_f32<E>(kt[0]);
                *reinterpret_cast<E*>(blk + B::QT + off) = from_f32<E>(qt[0]);
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
        const V16<E> qt = *reinterpret_cast<const V16<E>*>(blk + B::QT + off);
        const V16<E> kh = *reinterpret_cast<const V16<E>*>(scr + B::SCR_KH + off);
        if constexpr (B::kBF16) {
            akk = mma_bf16_k32(kt, kh, akk);
            aqk = mma_bf16_k32(qt, kh, aqk);
        } else {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                akk = mma_f32_k4(kt[p], kh[p], akk);
                aqk = mma_f32_k4(qt[p], kh[p], aqk);
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
        const float aq = ci <= r ? aqk[p] : 0.f;
        // A layout for the 16x16x16 / 16x16x4 consumer: lane (r, ci/4), element ci%4
        *reinterpret_cast<E*>(blk + B::AQ + ((ci >> 2) * 16 + r) * B::OPB + (ci & 3) * B::ES) =
            from_f32<E>(aq);
        if constexpr (DIAG) dAqk[r * 16 + ci] = aq;
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
    f32x4 gam[B::MT];
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

template <typename E, int D, typename Src>
__device__ __forceinline__ void cops_load(COps<E, D>& c, const Src& src) {
    using B = Blk<E, D>;
    const int lane = lane_id(), g = lane >> 4, r = lane & 15;
#pragma unroll
    for (int s = 0; s < B::NSLOT; ++s) {
        const int off = B::arow_chunk(s, g, r);
        c.kt[s] = src.template ld<V16<E>>(B::KT + off);
        c.qt[s] = src.template ld<V16<E>>(B::QT + off);
    }
#pragma unroll
    for (int m = 0; m < B::MT; ++m) {
        c.kd[m] = src.template ld<V4<E>>(B::kd_offset(m, g, r));
        c.gam[m] = src.template ld<f32x4>(B::GAM + (16 * m + 4 * g) * 4);
    }
    c.tm = src.template ld<V4<E>>(B::TM + lane * B::OPB);
    c.aq = src.template ld<V4<E>>(B::AQ + lane * B::OPB);
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

// One chunk of the state chain for NB 16-column blocks of S.
template <typename E, int D, int NB>
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
                o = mma_bf16_k32(c.qt[s], sb, o);      // Qt S
            }
            const f32x4 y = V - x;
            const f32x4 u = mma_bf16_k16(c.tm, pack4(y), zero4());   // U = Tm (V - Kt S)
            const bf16x4 ub = pack4(u);
            // Aqk U goes to its own accumulator: an MFMA of one shape must not
            // take as srcC the result of an MFMA of another shape still in
            // flight (16x16x32 -> 16x16x16 chains read stale srcC on gfx950).
            o += mma_bf16_k16(c.aq, ub, zero4());                    // + Aqk U
#pragma unroll
            for (int m = 0; m < B::MT; ++m)
                S[nb][m] = mma_bf16_k16(c.kd[m], ub, S[nb][m] * c.gam[m]);  // Diag(gam) S + Kd^T U
        } else {
#pragma unroll
            for (int m = 0; m < B::MT; ++m)
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    x = mma_f32_k4(c.kt[m][p], S[nb][m][p], x);
                    o = mma_f32_k4(c.qt[m][p], S[nb][m][p], o);
                }
            const f32x4 y = V - x;
            f32x4 u = zero4();
#pragma unroll
            for (int p = 0; p < 4; ++p) u = mma_f32_k4(c.tm[p], y[p], u);
#pragma unroll
            for (int p = 0; p < 4; ++p) o = mma_f32_k4(c.aq[p], u[p], o);
#pragma unroll
            for (int m = 0; m < B::MT; ++m) {
                f32x4 s = S[nb][m] * c.gam[m];
#pragma unroll
                for (int p = 0; p < 4; ++p) s = mma_f32_k4(c.kd[m][p], u[p], s);
                S[nb][m] = s;
            }
        }
        O[nb] = o;
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

// Workgroup barrier usable from role-specific code paths: every wave of the
// workgroup executes the same number of these, from whichever branch.
__device__ __forceinline__ void wg_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Inter kernel (split plan): one workgroup per (b, h, tile of NCOL = 16 NB
// NCW value columns) over chunks [n_first, n_first + n_count).  Waves
// 0 .. NCW-1 each carry the state of NB 16-column blocks; the other NL waves
// stream the factor blocks (and, where the LDS holds them, the V tiles) into
// an LDS ring of NPAIR entries of two chunks ("pairs"), shared by the NCW
// chains, which read their operands from LDS one chunk ahead of their use.
// Every chain reads the whole factor block of each chunk, so NB > 1 trades
// MFMA work per wave for less LDS traffic per column.
//
// Synchronisation is by LDS flags, not workgroup barriers, so the chains run
// unaligned (their LDS bursts interleave) and never wait for each other:
//   ready[e]  index of the last pair published in entry e (loader -> chains);
//             a loader stores it after its data stores have completed;
//   done[e]   number of (chain, pair) completions of entry e (chains ->
//             loaders); a chain adds 1 after its last use of the pair.
// Pair p goes to entry p mod NPAIR and belongs to loader p mod NL, which
// writes it once done[e] counts NCW completions of every earlier occupant.
// A chain in pair s also reads the first chunk of pair s + 1; two entries
// suffice for that, so no wait can close a cycle.  Every wait is bounded
// (kSpinLimit polls); a bound that ran out would only corrupt results, the
// kernel still ends.
constexpr int kSpinLimit = 1 << 22;

__device__ __forceinline__ void spin_until_ge(const int* flag, int target) {
    for (int it = 0; it < kSpinLimit; ++it) {
        if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) break;
        __builtin_amdgcn_s_sleep(1);
    }
    // later LDS reads stay after the poll that released them
    asm volatile("" ::: "memory");
}

template <typename E, int D, int NCW_, int NB_>
struct InterCfg {
    static constexpr int ES = (int)sizeof(E);
    static constexpr int NCW = NCW_, NB = NB_;
    static constexpr int NCOL = 16 * NB * NCW;                   // value columns per workgroup
    static constexpr int LDS_MAX = 160 * 1024 - 256;             // room for the flags
    // V tiles of one pair: 32-bit word w of the tile's row r (two bf16 or one
    // fp32 column) at word w * VSTR + r; the padding makes the loaders'
    // word stores conflict-free across the 64 LDS banks
    static constexpr int VSTR = 2 * kChunk + 2;
    static constexpr int VBYTES = NCOL * ES / 4 * VSTR * 4;
    static constexpr int ENT_V = 2 * Blk<E, D>::BYTES + VBYTES;
    static constexpr bool VLDS = LDS_MAX / ENT_V >= 2;           // V staged in the ring
    static constexpr int ENT = VLDS ? ENT_V : 2 * Blk<E, D>::BYTES;
    static constexpr int NPAIR = LDS_MAX / ENT < 4 ? LDS_MAX / ENT : 4;
    // loader waves: workgroups of at most four waves keep one wave per SIMD
    // (the chains get the whole register file)
    static constexpr int NL = NCW >= 4 ? 3 : 4 - NCW;
    static constexpr int THREADS = (NCW + NL) * kWave;
    static_assert(NCOL <= D, "column tile wider than the head");
    static_assert(NPAIR >= 2, "the ring needs two entries of two factor blocks");
    static_assert(!VLDS || (2 * kChunk * NCOL * ES / 16) % kWave == 0, "V pieces per loader lane");
    static_assert(VBYTES % 16 == 0, "ring entries stay 16-byte aligned");
};

template <typename E, int D, int NCW, int NB>
__global__ __launch_bounds__((InterCfg<E, D, NCW, NB>::THREADS)) void inter_kernel(
    const char* __restrict__ ws, const E* __restrict__ v, const float* S0, E* __restrict__ o,
    float* ST, int B, int T, int H, int n_first, int n_count, int nct) {
    using Bk = Blk<E, D>;
    using Cfg = InterCfg<E, D, NCW, NB>;
    constexpr int NPAIR = Cfg::NPAIR, NL = Cfg::NL, ENT = Cfg::ENT, ES = Cfg::ES;
    constexpr int NCOL = Cfg::NCOL;
    constexpr bool VLDS = Cfg::VLDS;
    constexpr int PAIR16 = 2 * Bk::BYTES / 16;        // 16-byte pieces of factor blocks per pair
    constexpr int PER_LANE = (PAIR16 + kWave - 1) / kWave;
    constexpr int RP = NCOL * ES / 16;                // 16-byte pieces per V row of the tile
    constexpr int VPL = VLDS ? 2 * kChunk * RP / kWave : 0;
    constexpr int EPP = 16 / ES;                      // elements per piece
    __shared__ __attribute__((aligned(16))) char ring[NPAIR * ENT];
    __shared__ int ready[NPAIR], done[NPAIR];
    int u, ct;
    if (!map_unit(nct, B * H, u, ct)) return;   // uniform over the workgroup
    const int b = u / H, h = u % H;
    const int w = wave_id();
    const int lane = lane_id();
    const int tile0 = ct * NCOL;
    const int NS = (n_count + 1) / 2;
    const char* blk0 = ws + (size_t)u * n_count * Bk::BYTES;
    const Rsrc rws = make_rsrc(blk0, (uint32_t)((size_t)n_count * Bk::BYTES));
    if (w == 0 && lane < NPAIR) {
        ready[lane] = -1;
        done[lane] = 0;
    }
    wg_barrier();   // the only barrier: flags initialised

    if (w >= NCW) {
        // ------------------------------------------------ loader waves
        const int L = w - NCW;
        u32x4 buf[PER_LANE];
        u32x4 vbuf[VPL > 0 ? VPL : 1];
        auto issue = [&](int p) {
#pragma unroll
            for (int i = 0; i < PER_LANE; ++i) {
                const int piece = i * kWave + lane;
                buf[i] = buf_load<u32x4>(rws, (p * PAIR16 + piece) * 16);   // past the end: 0
            }
            if constexpr (VLDS) {
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
            }
        };
        auto write = [&](int p) {
            char* dst = ring + (p % NPAIR) * ENT;
#pragma unroll
            for (int i = 0; i < PER_LANE; ++i) {
                const int piece = i * kWave + lane;
                if (piece < PAIR16) *reinterpret_cast<u32x4*>(dst + piece * 16) = buf[i];
            }
            if constexpr (VLDS) {
                // V area: word-major (word w of row r at w * VSTR + r), so a
                // chain reads the four rows of its column as 16 bytes
                uint32_t* vd = reinterpret_cast<uint32_t*>(dst + 2 * Bk::BYTES);
#pragma unroll
                for (int i = 0; i < VPL; ++i) {
                    const int q = i * kWave + lane, r = q / RP, c = q % RP;
#pragma unroll
                    for (int e = 0; e < 4; ++e) vd[(4 * c + e) * Cfg::VSTR + r] = vbuf[i][e];
                }
            }
        };
        if (L < NS) issue(L);
        for (int p = L; p < NS; p += NL) {
            const int e = p % NPAIR;
            if (p >= NPAIR) spin_until_ge(&done[e], NCW * (p / NPAIR));
            write(p);
            // publish: the data stores complete before the flag store
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
            __hip_atomic_store(&ready[e], p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (p + NL < NS) issue(p + NL);
        }
        return;
    }
    // ---------------------------------------------------- state chains
    // Straight-line loop body (the odd last chunk runs after the loop), so
    // no load is waited for before its use.
    const int j = lane & 15, g = lane >> 4;
    const int col0 = tile0 + 16 * NB * w;
    auto blk = [&](int nl) { return LdsSrc{ring + ((nl >> 1) % NPAIR) * ENT + (nl & 1) * Bk::BYTES}; };
    // V of chunk nl for the NB blocks: from the ring, or (where it does not
    // fit) the raw words loaded from memory two chunks ahead
    auto v_ring = [&](int nl, f32x4 (&V)[NB]) {
        const uint32_t* base = reinterpret_cast<const uint32_t*>(ring + ((nl >> 1) % NPAIR) * ENT +
                                                                 2 * Bk::BYTES) +
                               (nl & 1) * kChunk + 4 * g;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int vcol = 16 * (NB * w + nb) + j;   // column within the tile
            const uint32_t* at = base + (ES == 2 ? vcol >> 1 : vcol) * Cfg::VSTR;
            const u32x2 lo = *reinterpret_cast<const u32x2*>(at);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(at + 2);
            u32x4 x = {lo[0], lo[1], hi[0], hi[1]};
            if constexpr (ES == 2) {
                x <<= 16 * (1 - (vcol & 1));   // bf16 of this column to the high half
                x &= 0xFFFF0000u;
            }
            V[nb] = __builtin_bit_cast(f32x4, x);
        }
    };
    auto release = [&](int s) {   // this chain is done with pair s
        asm volatile("" ::: "memory");
        if (lane == 0) __hip_atomic_fetch_add(&done[s % NPAIR], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    f32x4 S[NB][D / 16];
    state_load<D, NB>(S, S0 ? S0 + (size_t)u * D * D : nullptr, col0);
    u32x4 vr[2][NB];
    if constexpr (!VLDS) {
        v_load<D, NB>(vr[0], v, ES, chunk_pos<D>(b, h, n_first, T, H), col0);
        v_load<D, NB>(vr[1], v, ES, chunk_pos<D>(b, h, n_first + 1, T, H), col0);
    }
    COps<E, D> ca, cb;
    f32x4 va[NB], vb[NB];
    spin_until_ge(&ready[0], 0);
    cops_load<E, D>(ca, blk(0));
    if constexpr (VLDS) v_ring(0, va);
    const int NFULL = n_count >> 1;
    for (int s = 0; s < NFULL; ++s) {
        const int n0 = n_first + 2 * s;
        f32x4 O[NB];
        cops_load<E, D>(cb, blk(2 * s + 1));
        if constexpr (VLDS) {
            v_ring(2 * s + 1, vb);
        } else {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) va[nb] = v_widen<E>(vr[0][nb]);
        }
        // keep the reads of the next chunk's operands ahead of this chunk's
        // work (IR sinking and the scheduler would otherwise move them to
        // their use); the loads stay in flight until their first use.  The
        // fp32 operands are twice as large: there both sets would not fit
        // the registers, and the reads are left to the scheduler.
        if constexpr (ES == 2) pin_issued();
        chunk_step<E, D, NB>(ca, S, va, O);
        o_store<E, D, NB>(O, o, chunk_pos<D>(b, h, n0, T, H), col0);
        if constexpr (!VLDS) v_load<D, NB>(vr[0], v, ES, chunk_pos<D>(b, h, n0 + 2, T, H), col0);
        if (s + 1 < NS) spin_until_ge(&ready[(s + 1) % NPAIR], s + 1);
        cops_load<E, D>(ca, blk(2 * s + 2));   // pair s + 1 (stale if there is none; unused)
        if constexpr (VLDS) {
            v_ring(2 * s + 2, va);
        } else {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) vb[nb] = v_widen<E>(vr[1][nb]);
        }
        if constexpr (ES == 2) pin_issued();
        chunk_step<E, D, NB>(cb, S, vb, O);
        release(s);
        o_store<E, D, NB>(O, o, chunk_pos<D>(b, h, n0 + 1, T, H), col0);
        if constexpr (!VLDS) v_load<D, NB>(vr[1], v, ES, chunk_pos<D>(b, h, n0 + 3, T, H), col0);
    }
    if (n_count & 1) {
        f32x4 O[NB];
        if constexpr (!VLDS) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) va[nb] = v_widen<E>(vr[0][nb]);
        }
        chunk_step<E, D, NB>(ca, S, va, O);
        o_store<E, D, NB>(O, o, chunk_pos<D>(b, h, n_first + n_count - 1, T, H), col0);
    }
    if (ST) state_store<D, NB>(S, ST + (size_t)u * D * D, col0);
}

// Inter kernel, direct variant (split plan): one wave per (b, h, 16-column
// block) over chunks [n_first, n_first + n_count), no LDS and no barriers.
// The operands of chunk n + PF are loaded from memory (the factor-block
// workspace and V) into a register ring of depth PF while chunk n runs; the
// loop is unrolled by PF so every ring slot is a fixed set of registers and
// every wait for a load is exact.  Blocks past the segment read as zeros and
// are never used.
template <typename E, int D, int PF>
__global__ __launch_bounds__(64) void inter_direct_kernel(const char* __restrict__ ws,
                                                          const E* __restrict__ v,
                                                          const float* S0, E* __restrict__ o,
                                                          float* ST, int B, int T, int H,
                                                          int n_first, int n_count, int nct) {
    using Bk = Blk<E, D>;
    constexpr int ES = (int)sizeof(E);
    int u, ct;
    if (!map_unit(nct, B * H, u, ct)) return;
    const int b = u / H, h = u % H;
    const int col0 = ct * 16;
    const char* blk0 = ws + (size_t)u * n_count * Bk::BYTES;
    auto src = [&](int nl) {
        return BufSrc{make_rsrc(blk0 + (size_t)nl * Bk::BYTES, nl < n_count ? (uint32_t)Bk::BYTES : 0u)};
    };
    f32x4 S[1][D / 16];
    state_load<D, 1>(S, S0 ? S0 + (size_t)u * D * D : nullptr, col0);
    COps<E, D> c[PF];
    u32x4 vr[PF][1];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        cops_load<E, D>(c[i], src(i));
        v_load<D, 1>(vr[i], v, ES, chunk_pos<D>(b, h, n_first + i, T, H), col0);
    }
    int n = 0;
    for (; n + PF <= n_count; n += PF) {
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            f32x4 Vf[1] = {v_widen<E>(vr[i][0])};
            f32x4 O[1];
            chunk_step<E, D, 1>(c[i], S, Vf, O);
            o_store<E, D, 1>(O, o, chunk_pos<D>(b, h, n_first + n + i, T, H), col0);
            cops_load<E, D>(c[i], src(n + i + PF));
            v_load<D, 1>(vr[i], v, ES, chunk_pos<D>(b, h, n_first + n + i + PF, T, H), col0);
        }
    }
#pragma unroll
    for (int i = 0; i < PF - 1; ++i) {
        if (n + i < n_count) {
            f32x4 Vf[1] = {v_widen<E>(vr[i][0])};
            f32x4 O[1];
            chunk_step<E, D, 1>(c[i], S, Vf, O);
            o_store<E, D, 1>(O, o, chunk_pos<D>(b, h, n_first + n + i, T, H), col0);
        }
    }
    if (ST) state_store<D, 1>(S, ST + (size_t)u * D * D, col0);
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
// 1 + NM barriers.
template <typename E, int D, int NB, int NCW>
__global__ __launch_bounds__(512) void fused_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                    const E* __restrict__ v, const E* __restrict__ z,
                                                    const float* __restrict__ beta,
                                                    const float* __restrict__ A, float g_min,
                                                    const float* S0, E* __restrict__ o, float* ST,
                                                    int B, int T, int H, int nct) {
    using Bk = Blk<E, D>;
    using Cfg = FusedCfg<E, D>;
    constexpr int NPROD = Cfg::NPROD;
    __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS];
    int u, ct;
    if (!map_unit(nct, B * H, u, ct)) return;   // uniform over the workgroup
    const int b = u / H, h = u % H;
    const int w = wave_id();
    const int NC = (T + kChunk - 1) / kChunk;
    const int NM = (NC + NPROD - 1) / NPROD;

    if (w < NPROD) {
        // ------------------------------------------------ producer wave
        char* myscr = smem + Cfg::RING + w * Bk::SCR_BYTES;
        const GateConsts gc = make_gate(A[h], g_min);
        ProdIn<E, D> cur, nxt;
        cur.L = 0;
        nxt.L = 0;
        if (w < NC) prod_load<E, D>(cur, q, k, z, beta, chunk_pos<D>(b, h, w, T, H));
        if (NPROD + w < NC) prod_load<E, D>(nxt, q, k, z, beta, chunk_pos<D>(b, h, NPROD + w, T, H));
        if (cur.L > 0)
            prod_compute<E, D, false>(cur, gc, smem + w * Bk::BYTES, myscr, nullptr, nullptr, nullptr);
        wg_barrier();
        for (int m = 0; m < NM; ++m) {
            cur = nxt;
            nxt.L = 0;
            const int n_next = (m + 2) * NPROD + w;
            if (n_next < NC) prod_load<E, D>(nxt, q, k, z, beta, chunk_pos<D>(b, h, n_next, T, H));
            if (cur.L > 0)
                prod_compute<E, D, false>(cur, gc, smem + (((m + 1) & 1) * NPROD + w) * Bk::BYTES,
                                          myscr, nullptr, nullptr, nullptr);
            wg_barrier();
        }
        return;
    }
    const int cw = w - 4;
    if (cw < 0 || cw >= NCW) {
        // ------------------------------------------------ idle wave
        wg_barrier();
        for (int m = 0; m < NM; ++m) wg_barrier();
        return;
    }
    // ---------------------------------------------------- consumer wave
    const int col0 = ct * (NCW * NB * 16) + cw * NB * 16;
    f32x4 S[NB][D / 16];
    constexpr int ES = (int)sizeof(E);
    u32x4 Vc[NPROD][NB], Vn[NPROD][NB];
    state_load<D, NB>(S, S0 ? S0 + (size_t)u * D * D : nullptr, col0);
#pragma unroll
    for (int cc = 0; cc < NPROD; ++cc)
        if (cc < NC) v_load<D, NB>(Vc[cc], v, ES, chunk_pos<D>(b, h, cc, T, H), col0);
    wg_barrier();
    for (int m = 0; m < NM; ++m) {
#pragma unroll
        for (int cc = 0; cc < NPROD; ++cc) {
            const int nn = (m + 1) * NPROD + cc;
            if (nn < NC) v_load<D, NB>(Vn[cc], v, ES, chunk_pos<D>(b, h, nn, T, H), col0);
        }
#pragma unroll
        for (int cc = 0; cc < NPROD; ++cc) {
            const int n = m * NPROD + cc;
            if (n < NC) {
                COps<E, D> c;
                cops_load<E, D>(c, LdsSrc{smem + ((m & 1) * NPROD + cc) * Bk::BYTES});
                f32x4 O[NB];
                f32x4 Vf[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) Vf[nb] = v_widen<E>(Vc[cc][nb]);
                chunk_step<E, D, NB>(c, S, Vf, O);
                o_store<E, D, NB>(O, o, chunk_pos<D>(b, h, n, T, H), col0);
            }
        }
#pragma unroll
        for (int cc = 0; cc < NPROD; ++cc)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) Vc[cc][nb] = Vn[cc][nb];
        wg_barrier();
    }
    if (ST) state_store<D, NB>(S, ST + (size_t)u * D * D, col0);
}

// --------------------------------------------------------------- plans / launchers

size_t factor_block_bytes(int d, bool is_bf16) {
    if (is_bf16) return d == 128 ? (size_t)Blk<bf16, 128>::BYTES : (size_t)Blk<bf16, 32>::BYTES;
    return d == 128 ? (size_t)Blk<float, 128>::BYTES : (size_t)Blk<float, 32>::BYTES;
}

// Chunks per split-plan segment: the workspace holds this many factor blocks
// per head; longer sequences run as consecutive segments carrying the state.
constexpr int kSegChunks = 1024;

// Plan override for tests and tuning: KDA_PREFILL_PLAN = "fused:<ncol>"
// (ncol in {16, 32, 64, 128}, at most d) or "split".  Unset or anything
// else: chosen from the sizes.
// Split-plan inter variants that are compiled: ncol value columns per
// workgroup in 16-column blocks, nb blocks per state chain.
static bool split_variant_ok(int d, bool is_bf16, int ncol, int nb) {
    if (nb == 0) return ncol == 16;   // direct variant
    if (nb != 1 && nb != 2) return false;
    if (nb == 2 && d == 128 && !is_bf16) return false;
    const int ncw = ncol / (16 * nb);
    if (ncw * 16 * nb != ncol || ncol > d) return false;
    return ncw == 1 || ncw == 2 || (ncw == 4 && d == 128 && nb == 1);
}

static bool plan_override(int d, bool is_bf16, PlanInfo& p) {
    const char* env = std::getenv("KDA_PREFILL_PLAN");
    if (!env) return false;
    if (std::strcmp(env, "split") == 0) {
        p.plan = Plan::kSplit;
        return true;
    }
    if (std::strncmp(env, "split:", 6) == 0) {
        int ncol = 0, nb = 0;
        if (std::sscanf(env + 6, "%d:%d", &ncol, &nb) == 2 && split_variant_ok(d, is_bf16, ncol, nb)) {
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
    const bool forced = plan_override(d, is_bf16, p);
    if (forced && p.plan == Plan::kFused) return p;
    if (!forced && units >= 128) {
        p.plan = Plan::kFused;
        p.ncol = units >= 256 ? d : (d >= 64 ? 64 : d);
        p.ws_bytes = 0;
        return p;
    }
    p.plan = Plan::kSplit;
    if (p.ncol == 0) {   // default inter variant
        p.ncol = d >= 64 ? 64 : d;
        p.nb = 1;
    }
    const int seg = NC < kSegChunks ? NC : kSegChunks;
    p.ws_bytes = (size_t)units * seg * factor_block_bytes(d, is_bf16);
    if (NC > kSegChunks) p.ws_bytes += (size_t)units * d * d * sizeof(float);
    return p;
}

static unsigned grid_units(int units, int nct) {
    return (unsigned)(((units + 7) / 8) * 8 * nct);
}

template <typename E, int D, int NCW, int NB>
static hipError_t launch_inter_v(const char* ws, const E* v, const float* s_in, E* o, float* s_out,
                                 const PrefillArgs& a, int n_first, int n_count,
                                 hipStream_t stream) {
    using Cfg = InterCfg<E, D, NCW, NB>;
    const int nct = D / Cfg::NCOL;
    hipLaunchKernelGGL((inter_kernel<E, D, NCW, NB>), dim3(grid_units(a.B * a.H, nct)),
                       dim3(Cfg::THREADS), 0, stream, ws, v, s_in, o, s_out, a.B, a.T, a.H, n_first,
                       n_count, nct);
    return hipGetLastError();
}

// Inter-kernel variant of a split plan: p.ncol value columns per workgroup,
// p.nb 16-column blocks per state chain (see split_variant_ok).
template <typename E, int D>
static hipError_t launch_inter(const PlanInfo& p, const char* ws, const E* v, const float* s_in,
                               E* o, float* s_out, const PrefillArgs& a, int n_first, int n_count,
                               hipStream_t stream) {
    if (p.nb == 0) {   // direct variant: one wave per 16-column block
        hipLaunchKernelGGL((inter_direct_kernel<E, D, 2>), dim3(grid_units(a.B * a.H, D / 16)),
                           dim3(64), 0, stream, ws, v, s_in, o, s_out, a.B, a.T, a.H, n_first,
                           n_count, D / 16);
        return hipGetLastError();
    }
#define KDA_INTER(NCW, NB)                                                                    \
    if (p.ncol == 16 * (NCW) * (NB) && p.nb == (NB))                                           \
        return launch_inter_v<E, D, (NCW), (NB)>(ws, v, s_in, o, s_out, a, n_first, n_count, stream);
    if constexpr (D == 128) {
        KDA_INTER(4, 1)
        KDA_INTER(2, 1)
        KDA_INTER(1, 1)
        if constexpr (sizeof(E) == 2) {
            KDA_INTER(2, 2)
            KDA_INTER(1, 2)
        }
    } else {
        KDA_INTER(2, 1)
        KDA_INTER(1, 1)
        KDA_INTER(1, 2)
    }
#undef KDA_INTER
    return hipErrorInvalidValue;
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
        if (p.ncol == 128 && D == 128)
            hipLaunchKernelGGL((fused_kernel<E, D, 2, 4>), grid, block, 0, stream, q, k, v, z, a.beta,
                               a.A, a.g_min, a.S0, o, a.S_T, a.B, a.T, a.H, nct);
        else if (p.ncol == 64 && D == 128)
            hipLaunchKernelGGL((fused_kernel<E, D, 1, 4>), grid, block, 0, stream, q, k, v, z, a.beta,
                               a.A, a.g_min, a.S0, o, a.S_T, a.B, a.T, a.H, nct);
        else if (p.ncol == 32)
            hipLaunchKernelGGL((fused_kernel<E, D, 1, 2>), grid, block, 0, stream, q, k, v, z, a.beta,
                               a.A, a.g_min, a.S0, o, a.S_T, a.B, a.T, a.H, nct);
        else
            hipLaunchKernelGGL((fused_kernel<E, D, 1, 1>), grid, block, 0, stream, q, k, v, z, a.beta,
                               a.A, a.g_min, a.S0, o, a.S_T, a.B, a.T, a.H, nct);
        return hipGetLastError();
    }
    // split plan, in segments of at most kSegChunks chunks
    const size_t blk_bytes = Blk<E, D>::BYTES;
    char* fws = (char*)ws;
    const int seg = NC < kSegChunks ? NC : kSegChunks;
    float* carry = a.S_T;
    if (NC > seg && !carry) carry = (float*)(fws + (size_t)units * seg * blk_bytes);
    for (int n_first = 0; n_first < NC; n_first += seg) {
        const int n_count = (NC - n_first) < seg ? (NC - n_first) : seg;
        const size_t nchunks = (size_t)units * n_count;
        hipLaunchKernelGGL((intra_kernel<E, D, false>), dim3((unsigned)((nchunks + 3) / 4)), dim3(256), 0,
                           stream, q, k, z, a.beta, a.A, a.g_min, fws, a.B, a.T, a.H, n_first,
                           n_count, (float*)nullptr, (float*)nullptr, (float*)nullptr);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const float* s_in = n_first == 0 ? a.S0 : carry;
        const bool last = n_first + n_count >= NC;
        float* s_out = last ? a.S_T : carry;
        e = launch_inter<E, D>(p, fws, v, s_in, o, s_out, a, n_first, n_count, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_prefill(const PrefillArgs& a, const PlanInfo& p, void* ws, hipStream_t stream) {
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
