// kda_bwd_chunk.hip -- gradients of the KDA prefill in the chunkwise form, on
// MFMA, for bf16 inputs at d_k = d_v = 128.
//
// The pages describe no backward pass (the dev.to page "Kimi K3 Architecture
// ...", section "The Sequence Bottleneck", says chunkwise parallel execution
// runs the within-chunk and state products as dense matrix products, which
// training relies on).  This is the exact gradient of the chunk equations of
// the forward (kda_chunk.hpp), differentiated step by step.  For a chunk with
// start state S, end-state gradient dS (of S' = Diag(gam) S + Kd^T U) and
// output gradient dO:
//   dU  = Kd dS + Aqk^T dO            dW = Tm^T dU         (dv = dW)
//   dS_start = Diag(gam) dS + Qt^T dO - Kt^T dW           (the chain)
//   W   = V - Kt S,   U = Tm W
//   dQt = dO S^T + dAqk Kh            dAqk = tril_0(dO U^T)
//   dKt = -dW S^T + dP Kh             dKh  = dAqk^T Qt + dP^T Kt
//   dKd = U dS^T                      dgam = rowsum(dS o S)
//   dTm = dU W^T,  dbeta_j += sum_r dTm[r][j] Ninv[r][j],  dN = dTm Diag(beta)
//   dM  = -Ninv^T dN Ninv^T,  dA = tril_{-1}(dM),  dbeta_r += sum_j dA[r][j] P[r][j]
//   dP  = Diag(beta) dA                (P = Kt Kh^T, Ninv = (I + Akk)^{-1})
//   dk  = dKt e^G + dKh e^{-G} + dKd gam e^{-G},   dq = dQt e^G
//   dG  = dKt o Kt - dKh o Kh + dQt o Qt - dKd o Kd, plus at the chunk's last
//         row sum_r dKd o Kd + dgam o gam;  dg = reverse cumsum of dG
// and through the gate dz = dg g_min s (1 - s) e^{A_h}, dA_h += dg g_min s (1 - s) x.
//
// Launches (after the forward checkpoints S at every chunk start, natural
// [D][D] layout, which a state-only fused prefill pass writes):
//   bwd_fac_kernel    one workgroup per (b, h, chunk): the chunk's factors,
//                     written as the chain's MFMA operands (13,824 bytes).
//   bwd_dchain_kernel one wave per (b, h, 16 value columns): dS from dS_T back
//                     to dS0 over the chunks, last first (14 MFMAs per chunk),
//                     storing each chunk's end-state gradient.
//   bwd_grad_kernel   one workgroup per (b, h, chunk), all chunks at once:
//                     recomputes the factors and forms every gradient from S
//                     and dS by MFMA products over the 128 key or value
//                     channels; writes dq, dk, dv, dz, dbeta and a dA term.
// Precision: the gradient kernel forms every product from fp32 values split
// into two bf16 parts, x = hi + lo, as hi*hi + hi*lo + lo*hi (three MFMAs;
// inputs that are bf16 already need two), which keeps about 16 bits of each
// operand -- the gate gradient dA sums many terms that largely cancel.  The
// chain uses the factors' leading bf16 part against fp32 state gradients, as
// the forward's state chain does.  Accumulation and the triangular algebra
// are fp32.
#include "kda_chunk.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kD = 128;
constexpr int kRS = kD + 8;      // bf16 row stride of [16][128] tiles in LDS (16 B of padding)
constexpr int kRF = kD + 4;      // fp32 row stride of [16][128] tiles in LDS (16 B of padding)

// Chain operand block of one chunk (lane-major, 16-byte pieces): the layout
// bwd_fac_kernel writes and bwd_dchain_kernel reads.
struct CBlk {
    static constexpr int KD = 0;            // Kd, A-row order: 4 slots x 64 lanes x 16 B
    static constexpr int QK = KD + 4096;    // [Qt^T | -Kt^T] K = 32 A operands: 8 tiles x 64 x 16 B
    static constexpr int AQT = QK + 8192;   // Aqk^T, K = 16 A operand: 64 x 8 B
    static constexpr int TMT = AQT + 512;   // Tm^T, K = 16 A operand: 64 x 8 B
    static constexpr int GAM = TMT + 512;   // gam, fp32 x 128
    static constexpr int BYTES = GAM + 512;
};
static_assert(CBlk::BYTES == 13824, "chain block size");

// Factors of one chunk in LDS, natural layouts (row r = the chunk's token).
struct Fac {
    float G[16][kD];                       // chunk-local cumulative log-decay
    float gam[kD];                         // e^{G_15}
    float beta[16];                        // 0 on padded rows
    float P[16][16];                       // Kt Kh^T
    float Aqk[16][16];                     // tril_0(Qt Kh^T)
    float Ninv[16][16];                    // (I + Akk)^{-1}, Akk = tril_{-1}(Diag(beta) P)
    float Kt[16][kRF], Kh[16][kRF], Qt[16][kRF];   // (Kd = Kh Diag(gam))
};

// The chunk's raw gate inputs z (the finals need the gate's derivative).
struct Raw {
    bf16 z[16][kRS];
};

__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }

// 8 consecutive bf16 of an LDS row as one MFMA operand.
__device__ __forceinline__ bf16x8 ld8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

// An fp32 operand as two bf16 parts, x = hi + lo (lo = the rounding error of hi).
struct B8 {
    bf16x8 hi, lo;
};
struct B4 {
    bf16x4 hi, lo;
};
__device__ __forceinline__ B8 split8(f32x4 a, f32x4 b) {
    B8 r;
    r.hi = pack8(a, b);
    f32x4 ra, rb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        ra[e] = a[e] - (float)r.hi[e];
        rb[e] = b[e] - (float)r.hi[4 + e];
    }
    r.lo = pack8(ra, rb);
    return r;
}
__device__ __forceinline__ B4 split4(f32x4 a) {
    B4 r;
    r.hi = pack4(a);
    f32x4 ra;
#pragma unroll
    for (int e = 0; e < 4; ++e) ra[e] = a[e] - (float)r.hi[e];
    r.lo = pack4(ra);
    return r;
}
// 8 consecutive fp32 of an LDS row (16-byte aligned), split.
__device__ __forceinline__ B8 ld8s(const float* p) {
    return split8(*reinterpret_cast<const f32x4*>(p), *reinterpret_cast<const f32x4*>(p + 4));
}
// acc + a b to about 16 bits of both operands (the lo*lo term is dropped).
__device__ __forceinline__ f32x4 mma3(const B8& a, const B8& b, f32x4 acc) {
    acc = mma_bf16_k32(a.hi, b.hi, acc);
    acc = mma_bf16_k32(a.hi, b.lo, acc);
    return mma_bf16_k32(a.lo, b.hi, acc);
}
// ... with an exact bf16 left operand.
__device__ __forceinline__ f32x4 mma2(bf16x8 a, const B8& b, f32x4 acc) {
    acc = mma_bf16_k32(a, b.hi, acc);
    return mma_bf16_k32(a, b.lo, acc);
}
__device__ __forceinline__ f32x4 mma3(const B4& a, const B4& b, f32x4 acc) {
    acc = mma_bf16_k16(a.hi, b.hi, acc);
    acc = mma_bf16_k16(a.hi, b.lo, acc);
    return mma_bf16_k16(a.lo, b.hi, acc);
}

// Factors of chunk n of (b, h) into F (and, with raw, the raw gate inputs).
// 256 threads; ends with a workgroup barrier after which F is complete.  The
// 16 x 16 matrices P, Aqk and Ninv are computed here (tri == null, with akk as
// scratch) or read from tri (768 floats, as bwd_fac_kernel stores them).
template <bool RAW>
__device__ __forceinline__ void bwd_factors(Fac& F, Raw* raw, const bf16* __restrict__ q,
                                            const bf16* __restrict__ k,
                                            const bf16* __restrict__ z,
                                            const float* __restrict__ beta,
                                            const GateConsts& gc, int b, int h, int n, int T,
                                            int H, const float* __restrict__ tri,
                                            float (*akk)[16]) {
    const int tid = (int)threadIdx.x;
    const ChunkPos cp = chunk_pos<kD>(b, h, n, T, H);
    const int L = cp.L;
    const int rowb = (int)(cp.rstride * 2);
    if (tid < kD) {
        // one key channel per thread, all 16 rows (rows past L read 0 and
        // get retention 1, so G stays at its last value)
        const int c = tid;
        const Rsrc rk = chunk_rsrc<kD>(k, cp, 2), rq = chunk_rsrc<kD>(q, cp, 2),
                   rz = chunk_rsrc<kD>(z, cp, 2);
        float Gacc = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int off = r * rowb + c * 2;
            const uint32_t kb = buf_load<unsigned short>(rk, off);
            const uint32_t qb = buf_load<unsigned short>(rq, off);
            const uint32_t zb = buf_load<unsigned short>(rz, off);
            const float kf = bf16_bits_to_f32(kb), qf = bf16_bits_to_f32(qb);
            const float zf = bf16_bits_to_f32(zb);
            const float keep = r < L ? 1.f : 0.f;
            Gacc += keep * gc.gmin * gate_sigmoid(gc, zf);
            F.G[r][c] = Gacc;
            const float ex = fast_exp2(Gacc * kLog2e), rex = fast_rcp(ex);
            F.Kt[r][c] = kf * ex;
            F.Qt[r][c] = qf * ex;
            F.Kh[r][c] = kf * rex;
            if constexpr (RAW) raw->z[r][c] = __builtin_bit_cast(bf16, (unsigned short)zb);
        }
        F.gam[c] = fast_exp2(Gacc * kLog2e);
    } else {
        const int t = tid - kD;
        if (tri) {
            // P, Aqk, Ninv: 6 floats per thread
#pragma unroll
            for (int x = 0; x < 6; ++x) {
                const int e = t + 128 * x, which = e >> 8, rc = e & 255;
                const float val = tri[e];
                (which == 0 ? &F.P[0][0] : which == 1 ? &F.Aqk[0][0] : &F.Ninv[0][0])[rc] = val;
            }
        }
        if (t < 16) {
            const Rsrc rb = make_rsrc(beta + cp.brow0, L > 0 ? (uint32_t)(((L - 1) * cp.bstride + 1) * 4) : 0u);
            F.beta[t] = __builtin_bit_cast(float, buf_load<uint32_t>(rb, t * cp.bstride * 4));
        }
    }
    __syncthreads();
    if (tri) return;
    if (tid < kWave) {
        // P = Kt Kh^T and Qt Kh^T (K = 128), then Ninv by forward substitution
        const int i = tid & 15, g = tid >> 4;
        f32x4 p = zero4(), a = zero4();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const B8 kh = ld8s(&F.Kh[i][32 * s + 8 * g]);
            p = mma3(ld8s(&F.Kt[i][32 * s + 8 * g]), kh, p);
            a = mma3(ld8s(&F.Qt[i][32 * s + 8 * g]), kh, a);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;   // row r, column i
            F.P[r][i] = p[e];
            F.Aqk[r][i] = r >= i ? a[e] : 0.f;
            akk[r][i] = r > i ? F.beta[r] * p[e] : 0.f;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (tid < 16) {
            const int j = tid;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = r == j ? 1.f : 0.f;
#pragma unroll
                for (int c = 0; c < r; ++c) acc -= akk[r][c] * x[c];
                x[r] = acc;
                F.Ninv[r][j] = acc;
            }
        }
    }
    __syncthreads();
}

}  // namespace

// ------------------------------------------------------------------ kernels

// Chain operands of every chunk: block (u, n) at fac + (u * NC + n) * 13824.
// P, Aqk and Ninv of every chunk, fp32, at tri + (u * NC + n) * 768 (the
// gradient kernel reads them instead of solving again).
__global__ __launch_bounds__(256) void bwd_fac_kernel(const bf16* __restrict__ q,
                                                      const bf16* __restrict__ k,
                                                      const bf16* __restrict__ z,
                                                      const float* __restrict__ beta,
                                                      const float* __restrict__ A, float g_min,
                                                      char* __restrict__ fac,
                                                      float* __restrict__ tri, int B, int T,
                                                      int H) {
    __shared__ Fac F;
    __shared__ float akk[16][16];
    const int NC = (T + kChunk - 1) / kChunk;
    const size_t id = blockIdx.x;
    const int n = (int)(id % NC);
    const size_t u = id / NC;
    const int b = (int)(u / H), h = (int)(u % H);
    bwd_factors<false>(F, nullptr, q, k, z, beta, make_gate(A[h], g_min), b, h, n, T, H, nullptr,
                       akk);
    char* out = fac + id * (size_t)CBlk::BYTES;
    const int tid = (int)threadIdx.x, w = tid >> 6, lane = tid & 63, i = lane & 15, g = lane >> 4;
    {
        float* tr = tri + id * 768;
        tr[tid] = (&F.P[0][0])[tid];
        tr[256 + tid] = (&F.Aqk[0][0])[tid];
        tr[512 + tid] = (&F.Ninv[0][0])[tid];
    }
    if (w == 0) {
        // Kd in the A-row order of the chain's Kd dS product: slot s, lane
        // (i, g), element e <-> key channel 32 s + 16 (e / 4) + 4 g + e % 4,
        // which pairs with dS in its accumulator layout
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int c0 = 32 * s + 4 * g, c1 = c0 + 16;
            const f32x4 lo = *reinterpret_cast<const f32x4*>(&F.Kh[i][c0]) *
                             *reinterpret_cast<const f32x4*>(&F.gam[c0]);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(&F.Kh[i][c1]) *
                             *reinterpret_cast<const f32x4*>(&F.gam[c1]);
            *reinterpret_cast<bf16x8*>(out + CBlk::KD + s * 1024 + lane * 16) = pack8(lo, hi);
        }
    } else if (w <= 2) {
        // tile m of [Qt^T | -Kt^T]: lane (i, g) holds Qt[4g + e][16m + i] and
        // -Kt[4g + e][16m + i], e = 0..3
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
            const int m = 4 * (w - 1) + mm;
            bf16x8 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = (bf16)F.Qt[4 * g + e][16 * m + i];
                x[4 + e] = (bf16)(-F.Kt[4 * g + e][16 * m + i]);
            }
            *reinterpret_cast<bf16x8*>(out + CBlk::QK + m * 1024 + lane * 16) = x;
        }
    } else {
        // Aqk^T and Tm^T = (Ninv Diag(beta))^T as K = 16 A operands: lane
        // (i, g) holds row i, columns 4g .. 4g + 3
        bf16x4 aq, tm;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            aq[e] = (bf16)F.Aqk[4 * g + e][i];
            tm[e] = (bf16)(F.Ninv[4 * g + e][i] * F.beta[i]);
        }
        *reinterpret_cast<bf16x4*>(out + CBlk::AQT + lane * 8) = aq;
        *reinterpret_cast<bf16x4*>(out + CBlk::TMT + lane * 8) = tm;
        reinterpret_cast<float*>(out + CBlk::GAM)[lane] = F.gam[lane];
        reinterpret_cast<float*>(out + CBlk::GAM)[64 + lane] = F.gam[64 + lane];
    }
}

// Workgroup barrier that orders LDS accesses only: this wave's LDS writes
// are done before it, and global stores still in flight stay in flight (a
// workgroup fence would wait for them too).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// The state-gradient chain: one workgroup per (b, h, 16 value columns),
// chunks last to first.  dSend[(u NC + n)] receives the gradient of chunk n's
// end state in 16-column blocks, [D / 16][D][16] (element (k, j) at
// ((j / 16) D + k) 16 + j % 16), so that a chain's share of a chunk is 8 KB
// in one piece; dS0 (if given) the gradient of S0 ([D][D]).  Wave 0 runs the
// chain: the operands of the next three chunks are in flight while a chunk
// computes (a ring of three register sets, the loop unrolled three times),
// and each chunk's dS goes to one of two LDS tiles (eight 16-byte writes per
// lane).  Wave 1 copies the tile to dSend, 1 KB per store instruction, while
// the chain goes on; one workgroup barrier (LDS only) per chunk hands a tile
// over.  Stored by the chain itself into the [D][D] layout, as 32 four-byte
// stores per lane and chunk (64-byte pieces of rows), the state gradients
// took more than half of the chain's time.
__global__ __launch_bounds__(128) void bwd_dchain_kernel(const char* __restrict__ fac,
                                                        const bf16* __restrict__ dO,
                                                        const float* __restrict__ dST,
                                                        float* __restrict__ dSend,
                                                        float* __restrict__ dS0, int B, int T,
                                                        int H) {
    constexpr int NCB = kD / 16;
    const int NC = (T + kChunk - 1) / kChunk;
    // (b, h) of a workgroup id: the 8 column blocks of a head share an XCD
    int u, jb;
    if (!map_unit(NCB, B * H, u, jb)) return;
    const int b = u / H, h = u % H;
    const int lane = lane_id(), i = lane & 15, g = lane >> 4;
    const int j0 = 16 * jb;
    // tile t: row 16 m + r4 (r4 < 16), column c at [t][m][c][r4]
    __shared__ __attribute__((aligned(16))) float tile[2][8 * 256];
    if (wave_id() == 1) {
        // -------------------------------------------- store wave
        for (int n = NC - 1; n >= 0; --n) {
            lds_barrier();   // the chain has written chunk n's tile
            const float* tl = tile[n & 1];
            float* out = dSend + ((size_t)u * NC + n) * kD * kD + (size_t)jb * kD * 16 + 4 * (lane & 3);
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int r4 = lane >> 2;
                f32x4 x;
#pragma unroll
                for (int c = 0; c < 4; ++c) x[c] = tl[m * 256 + (4 * (lane & 3) + c) * 16 + r4];
                *reinterpret_cast<f32x4*>(out + (16 * m + r4) * 16) = x;
            }
        }
        return;
    }
    struct Ops {
        bf16x8 kd[4], qk[8];
        bf16x4 aqt, tmt;
        f32x2 gv;      // gam, two values per lane (row_tile)
        u32x4 dO;
    };
    auto load = [&](Ops& o, int n) {
        if (n < 0) return;
        const Rsrc rf = make_rsrc(fac + ((size_t)u * NC + n) * CBlk::BYTES, CBlk::BYTES);
#pragma unroll
        for (int s = 0; s < 4; ++s)
            o.kd[s] = __builtin_bit_cast(bf16x8, buf_load<u32x4>(rf, CBlk::KD + s * 1024 + lane * 16));
#pragma unroll
        for (int m = 0; m < 8; ++m)
            o.qk[m] = __builtin_bit_cast(bf16x8, buf_load<u32x4>(rf, CBlk::QK + m * 1024 + lane * 16));
        o.aqt = __builtin_bit_cast(bf16x4, buf_load<u32x2>(rf, CBlk::AQT + lane * 8));
        o.tmt = __builtin_bit_cast(bf16x4, buf_load<u32x2>(rf, CBlk::TMT + lane * 8));
        o.gv = __builtin_bit_cast(f32x2, buf_load<u32x2>(rf, CBlk::GAM + row_vec_offset<kD>(g, i)));
        // dO rows 4g .. 4g+3 of column j0 + i (rows past T read 0)
        const ChunkPos cp = chunk_pos<kD>(b, h, n, T, H);
        const Rsrc rd = chunk_rsrc<kD>(dO, cp, 2);
        const int rowb = (int)(cp.rstride * 2);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            o.dO[e] = buf_load<unsigned short>(rd, (4 * g + e) * rowb + (j0 + i) * 2);
    };
    // dS in the accumulator layout: lane (i, g) holds rows 16m + 4g + e of column j0 + i
    f32x4 dS[8];
    const float* st = dST ? dST + (size_t)u * kD * kD : nullptr;
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            dS[m][e] = st ? st[(size_t)(16 * m + 4 * g + e) * kD + j0 + i] : 0.f;
    // chunk n with the operands in c; then chunk n - 3's operands load into c
    auto step = [&](int n, Ops& c) {
        if (n < 0) return;
        // the gradient of this chunk's end state, for the gradient kernel:
        // to tile n & 1, which the store wave copies out after the barrier
        // (it finished the tile's previous chunk, n + 2, before the barrier
        // of chunk n + 1)
        float* tl = tile[n & 1];
#pragma unroll
        for (int m = 0; m < 8; ++m) *reinterpret_cast<f32x4*>(tl + m * 256 + i * 16 + 4 * g) = dS[m];
        lds_barrier();
        // dU = Kd dS + Aqk^T dO (separate accumulators: no 16x16x32 result
        // feeds a 16x16x16 MFMA as its accumulator input)
        f32x4 x = zero4();
#pragma unroll
        for (int s = 0; s < 4; ++s) x = mma_bf16_k32(c.kd[s], pack8(dS[2 * s], dS[2 * s + 1]), x);
        const f32x4 dOf = __builtin_bit_cast(f32x4, c.dO << 16);
        const bf16x4 dOb = pack4(dOf);
        const f32x4 y = mma_bf16_k16(c.aqt, dOb, zero4());
        const f32x4 dU = x + y;
        const f32x4 dW = mma_bf16_k16(c.tmt, pack4(dU), zero4());
        // dS <- Diag(gam) dS + [Qt^T | -Kt^T] [dO; dW]
        const bf16x4 dWb = pack4(dW);
        bf16x8 b2;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            b2[e] = dOb[e];
            b2[4 + e] = dWb[e];
        }
        static_for<0, 8>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            dS[m] = mma_bf16_k32(c.qk[m], b2, dS[m] * row_tile<m>(c.gv));
        });
        load(c, n - 3);
    };
    Ops o0, o1, o2;
    load(o0, NC - 1);
    load(o1, NC - 2);
    load(o2, NC - 3);
    for (int n = NC - 1; n >= 0; n -= 3) {
        step(n, o0);
        step(n - 1, o1);
        step(n - 2, o2);
    }
    if (dS0) {
        float* out = dS0 + (size_t)u * kD * kD + j0 + i;
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) out[(size_t)(16 * m + 4 * g + e) * kD] = dS[m][e];
    }
}

namespace {

// Row stride of the staging tile (64 rows of S or dS, fp32): with 130 floats
// the column reads of the value side (lanes: 16 columns x rows 8 apart) fall
// in distinct banks, and rows stay 8-byte aligned for the row writes.
constexpr int kSS = kD + 2;

// Scratch of the gradient kernel: the 16 x 128 products of the value side and
// the 16 x 16 gradients of the triangular algebra.  Before the products exist
// their space stages half of S or dS at a time for the value side.
struct GradLds {
    Fac F;
    Raw R;
    union {
        struct {
            float W[16][kRF], U[16][kRF], dU[16][kRF], dW[16][kRF];
        };
        float stage[64][kSS];
    };
    float dAqk[16][16], dTm[16][16], dP[16][16], T1[16][16];
    float db2[16];
    float dAred[4];
};
static_assert(sizeof(float) * 64 * kSS <= sizeof(float) * 4 * 16 * kRF, "staging tile fits");

}  // namespace

// Every gradient of chunk n of (b, h), from the chunk's start state (ckpt)
// and the gradient of its end state (dSend, in 16-column blocks as bwd_dchain_kernel stores it), per (b, h, chunk).  One workgroup of four waves; wave w owns value columns and
// key channels 32w .. 32w + 31.
__global__ __launch_bounds__(256) void bwd_grad_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ z, const float* __restrict__ beta, const float* __restrict__ A,
    float g_min, const bf16* __restrict__ dO, const float* __restrict__ ckpt,
    const float* __restrict__ dSend, const float* __restrict__ tri, bf16* __restrict__ dq,
    bf16* __restrict__ dk,
    bf16* __restrict__ dv, bf16* __restrict__ dz, float* __restrict__ dbeta,
    float* __restrict__ dA_part, int B, int T, int H) {
    __shared__ GradLds sm;
    Fac& F = sm.F;
    const int NC = (T + kChunk - 1) / kChunk;
    const size_t id = blockIdx.x;
    const int n = (int)(id % NC);
    const size_t u = id / NC;
    const int b = (int)(u / H), h = (int)(u % H);
    const GateConsts gc = make_gate(A[h], g_min);
    const int tid = (int)threadIdx.x, w = tid >> 6, lane = tid & 63, i = lane & 15, g = lane >> 4;
    const float* sst = ckpt + (u * NC + n) * (size_t)kD * kD;
    const float* dse = dSend + (u * NC + n) * (size_t)kD * kD;
    // S and dS rows 32 w .. 32 w + 31 (the wave's key channels), loaded once
    // while the factors are formed: lane (i, g) holds rows 32 w + 16 kk + i,
    // columns 32 t + 8 g .. + 7 -- the B operands of the key side as they
    // are, and the wave's share of the staging tile for the value side.
    f32x4 rowS[2][4][2], rowD[2][4][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const size_t off = (size_t)(32 * w + 16 * kk + i) * kD + 32 * t + 8 * g;
            rowS[kk][t][0] = *reinterpret_cast<const f32x4*>(sst + off);
            rowS[kk][t][1] = *reinterpret_cast<const f32x4*>(sst + off + 4);
        }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            // dSend in 16-column blocks: columns 32 t + 8 g .. + 7 are in
            // block 2 t + g / 2 at 8 (g % 2)
            const size_t off = ((size_t)(2 * t + (g >> 1)) * kD + 32 * w + 16 * kk + i) * 16 + 8 * (g & 1);
            rowD[kk][t][0] = *reinterpret_cast<const f32x4*>(dse + off);
            rowD[kk][t][1] = *reinterpret_cast<const f32x4*>(dse + off + 4);
        }
    const ChunkPos cp = chunk_pos<kD>(b, h, n, T, H);
    const int L = cp.L;
    const int rowb = (int)(cp.rstride * 2);
    const Rsrc rdo = chunk_rsrc<kD>(dO, cp, 2);
    const Rsrc rv = chunk_rsrc<kD>(v, cp, 2);
    // V and dO of the wave's two 16-column blocks (rows 4g + e, column
    // 32 w + 16 jj + i), issued here so that they arrive while the factors
    // are formed and S, dS pass through the staging tile
    uint32_t vraw[2][4], doraw[2][4];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int jc = 32 * w + 16 * jj + i;
            vraw[jj][e] = buf_load<unsigned short>(rv, (4 * g + e) * rowb + jc * 2);
            doraw[jj][e] = buf_load<unsigned short>(rdo, (4 * g + e) * rowb + jc * 2);
        }
    bwd_factors<true>(F, &sm.R, q, k, z, beta, gc, b, h, n, T, H, tri + id * 768, nullptr);
    // dO row i, columns 32 t + 8 g .. + 7, as an exact bf16 A operand
    auto dO_row = [&](int t) {
        return __builtin_bit_cast(bf16x8, buf_load<u32x4>(rdo, i * rowb + (32 * t + 8 * g) * 2));
    };

    // ---- value side: X = Kt S and Y = Kd dS over the 128 key channels, for
    // the wave's two 16-column blocks.  Half of S (or dS) at a time passes
    // through the staging tile: the two waves that hold rows 64 hf .. 64 hf +
    // 63 write them, then every wave reads its columns of those rows.
    f32x4 Xa[2] = {zero4(), zero4()}, Ya[2] = {zero4(), zero4()};
#pragma unroll
    for (int arr = 0; arr < 2; ++arr) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            if ((w >> 1) == hf) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int t = 0; t < 4; ++t)
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            const f32x4 x = arr == 0 ? rowS[kk][t][hh] : rowD[kk][t][hh];
                            float* dst = &sm.stage[32 * (w & 1) + 16 * kk + i][32 * t + 8 * g + 4 * hh];
                            *reinterpret_cast<f32x2*>(dst) = f32x2{x[0], x[1]};
                            *reinterpret_cast<f32x2*>(dst + 2) = f32x2{x[2], x[3]};
                        }
            }
            __syncthreads();
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                const int s = 2 * hf + sl, c0 = 32 * s + 8 * g;
                B8 a;
                if (arr == 0) {
                    a = ld8s(&F.Kt[i][c0]);
                } else {
                    const f32x4 kd0 = *reinterpret_cast<const f32x4*>(&F.Kh[i][c0]) *
                                      *reinterpret_cast<const f32x4*>(&F.gam[c0]);
                    const f32x4 kd1 = *reinterpret_cast<const f32x4*>(&F.Kh[i][c0 + 4]) *
                                      *reinterpret_cast<const f32x4*>(&F.gam[c0 + 4]);
                    a = split8(kd0, kd1);
                }
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const int jc = 32 * w + 16 * jj + i;
                    f32x4 c_lo, c_hi;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        c_lo[e] = sm.stage[32 * sl + 8 * g + e][jc];
                        c_hi[e] = sm.stage[32 * sl + 8 * g + 4 + e][jc];
                    }
                    if (arr == 0)
                        Xa[jj] = mma3(a, split8(c_lo, c_hi), Xa[jj]);   // Kt S
                    else
                        Ya[jj] = mma3(a, split8(c_lo, c_hi), Ya[jj]);   // Kd dS
                }
            }
            __syncthreads();
        }
    }
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int j0 = 32 * w + 16 * jj, jc = j0 + i;
        const f32x4 X = Xa[jj], Y = Ya[jj];
        // V and dO in the accumulator layout (rows 4g + e, column jc)
        f32x4 Vf, dOf;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            Vf[e] = bf16_bits_to_f32(vraw[jj][e]);
            dOf[e] = bf16_bits_to_f32(doraw[jj][e]);
        }
        // Tm = Ninv Diag(beta) and its transpose, Aqk^T, as K = 16 A operands
        f32x4 tmf, tmtf, aqtf;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            tmf[e] = F.Ninv[i][4 * g + e] * F.beta[4 * g + e];
            tmtf[e] = F.Ninv[4 * g + e][i] * F.beta[i];
            aqtf[e] = F.Aqk[4 * g + e][i];
        }
        const B4 tm = split4(tmf), tmt = split4(tmtf), aqt = split4(aqtf);
        const f32x4 Wv = Vf - X;
        const f32x4 Uv = mma3(tm, split4(Wv), zero4());
        const B4 dOs = {pack4(dOf), pack4(zero4())};   // dO is bf16 already
        const f32x4 dUv = Y + mma3(aqt, dOs, zero4());
        const f32x4 dWv = mma3(tmt, split4(dUv), zero4());
        // dv = dW (rows past the chunk's end are dropped)
        const Rsrc rdv = chunk_rsrc<kD>(dv, cp, 2);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            buf_store_u16(rdv, r * rowb + jc * 2, __builtin_bit_cast(unsigned short, (bf16)dWv[e]));
            sm.W[r][jc] = Wv[e];
            sm.U[r][jc] = Uv[e];
            sm.dU[r][jc] = dUv[e];
            sm.dW[r][jc] = dWv[e];
        }
    }
    __syncthreads();

    // ---- dAqk = tril_0(dO U^T) (wave 0) and dTm = dU W^T (wave 1), K = 128
    if (w < 2) {
        f32x4 c = zero4();
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (w == 0)
                c = mma2(dO_row(t), ld8s(&sm.U[i][32 * t + 8 * g]), c);
            else
                c = mma3(ld8s(&sm.dU[i][32 * t + 8 * g]), ld8s(&sm.W[i][32 * t + 8 * g]), c);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            if (w == 0) sm.dAqk[r][i] = r >= i ? c[e] : 0.f;
            else sm.dTm[r][i] = c[e];
        }
    }
    __syncthreads();

    // ---- the triangular algebra, fp32, one (row r, column j) per thread
    {
        const int r = tid >> 4, j = tid & 15;
        // T1 = dN Ninv^T with dN = dTm Diag(beta)
        float t1 = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2) t1 += sm.dTm[r][s2] * F.beta[s2] * F.Ninv[j][s2];
        sm.T1[r][j] = t1;
        __syncthreads();
        // dM = -Ninv^T T1; dA = tril_{-1}(dM); dP = Diag(beta) dA
        float dm = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2) dm -= F.Ninv[s2][r] * sm.T1[s2][j];
        const float da = r > j ? dm : 0.f;
        sm.dP[r][j] = F.beta[r] * da;
        // dbeta_r += sum_j dA[r][j] P[r][j]: the 16 threads of row r are 16
        // consecutive lanes of one wave
        float t = da * F.P[r][j];
        t += __shfl_xor(t, 1);
        t += __shfl_xor(t, 2);
        t += __shfl_xor(t, 4);
        t += __shfl_xor(t, 8);
        if (j == 0) sm.db2[r] = t;
        __syncthreads();
        if (tid < 16 && tid < L) {
            // plus dbeta_j += sum_r dTm[r][j] Ninv[r][j]
            float dbv = sm.db2[tid];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) dbv += sm.dTm[rr][tid] * F.Ninv[rr][tid];
            dbeta[cp.brow0 + (size_t)tid * cp.bstride] = dbv;
        }
    }
    __syncthreads();

    // ---- key side, two 16-channel blocks per wave
    float dA_acc = 0.f;
    const float eA = __expf(A[h]);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int k0 = 32 * w + 16 * kk, kc = k0 + i;
        f32x4 cQ = zero4(), cK = zero4(), cD = zero4();
        float dgam = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            // S and dS rows kc, value columns 32 t + 8 g .. + 7 (fp32)
            const f32x4 s_lo = rowS[kk][t][0], s_hi = rowS[kk][t][1];
            const f32x4 d_lo = rowD[kk][t][0], d_hi = rowD[kk][t][1];
#pragma unroll
            for (int e = 0; e < 4; ++e) dgam += s_lo[e] * d_lo[e] + s_hi[e] * d_hi[e];
            const B8 sb = split8(s_lo, s_hi), db = split8(d_lo, d_hi);
            cQ = mma2(dO_row(t), sb, cQ);                           // dO S^T
            cK = mma3(ld8s(&sm.dW[i][32 * t + 8 * g]), sb, cK);     // dW S^T
            cD = mma3(ld8s(&sm.U[i][32 * t + 8 * g]), db, cD);      // U dS^T
        }
        dgam += __shfl_xor(dgam, 16);
        dgam += __shfl_xor(dgam, 32);
        // K = 16 products with Kh, Qt, Kt tiles of channels k0 .. k0+15 as B
        f32x4 khf, qtf, ktf, dAqf, dAqTf, dPf, dPTf;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            khf[e] = F.Kh[4 * g + e][kc];
            qtf[e] = F.Qt[4 * g + e][kc];
            ktf[e] = F.Kt[4 * g + e][kc];
            dAqf[e] = sm.dAqk[i][4 * g + e];
            dAqTf[e] = sm.dAqk[4 * g + e][i];
            dPf[e] = sm.dP[i][4 * g + e];
            dPTf[e] = sm.dP[4 * g + e][i];
        }
        const B4 khB = split4(khf), qtB = split4(qtf), ktB = split4(ktf);
        const f32x4 dQt = cQ + mma3(split4(dAqf), khB, zero4());
        const f32x4 dKt = mma3(split4(dPf), khB, zero4()) - cK;
        const f32x4 dKh = mma3(split4(dPTf), ktB, mma3(split4(dAqTf), qtB, zero4()));
        const f32x4 dKd = cD;
        // finals: lane (i, g) holds rows 4g + e of channel kc
        const float gam = F.gam[kc];
        float dG[4], dkv[4], dqv[4], cs = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            const float ex = fast_exp2(F.G[r][kc] * kLog2e), rex = fast_rcp(ex);
            const float kv = F.Kt[r][kc] * rex, qv = F.Qt[r][kc] * rex;
            const float kdv = kv * gam * rex;          // Kd
            dkv[e] = dKt[e] * ex + dKh[e] * rex + dKd[e] * gam * rex;
            dqv[e] = dQt[e] * ex;
            dG[e] = dKt[e] * kv * ex - dKh[e] * kv * rex + dQt[e] * qv * ex - dKd[e] * kdv;
            cs += dKd[e] * kdv;
        }
        cs += __shfl_xor(cs, 16);
        cs += __shfl_xor(cs, 32);
        // dg_r = sum of dG over rows r .. 15, plus the last row's extra terms
        float suf[4];
        suf[3] = dG[3];
        suf[2] = dG[2] + suf[3];
        suf[1] = dG[1] + suf[2];
        suf[0] = dG[0] + suf[1];
        const float t1 = __shfl(suf[0], 16 + i), t2 = __shfl(suf[0], 32 + i),
                    t3 = __shfl(suf[0], 48 + i);
        const float after = (g < 1 ? t1 : 0.f) + (g < 2 ? t2 : 0.f) + (g < 3 ? t3 : 0.f);
        const float extra = cs + dgam * gam;
        const Rsrc rdq = chunk_rsrc<kD>(dq, cp, 2), rdk = chunk_rsrc<kD>(dk, cp, 2),
                   rdz = chunk_rsrc<kD>(dz, cp, 2);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            const float dg = suf[e] + after + extra;
            const float zv = bf2f(sm.R.z[r][kc]);
            const float s = gate_sigmoid(gc, zv);
            const float dx = r < L ? dg * gc.gmin * s * (1.f - s) : 0.f;
            dA_acc += dx * eA * zv;
            const int off = r * rowb + kc * 2;
            buf_store_u16(rdq, off, __builtin_bit_cast(unsigned short, (bf16)dqv[e]));
            buf_store_u16(rdk, off, __builtin_bit_cast(unsigned short, (bf16)dkv[e]));
            buf_store_u16(rdz, off, __builtin_bit_cast(unsigned short, (bf16)(dx * eA)));
        }
    }
    // the chunk's dA term: wave sums, then the four waves in order
#pragma unroll
    for (int x = 1; x < 64; x <<= 1) dA_acc += __shfl_xor(dA_acc, x);
    if (lane == 0) sm.dAred[w] = dA_acc;
    __syncthreads();
    if (tid == 0) dA_part[id] = ((sm.dAred[0] + sm.dAred[1]) + sm.dAred[2]) + sm.dAred[3];
}

// ------------------------------------------------------------------ host

bool bwd_chunk_ok(int d, bool is_bf16) { return d == kD && is_bf16; }

size_t bwd_chunk_fac_bytes() { return CBlk::BYTES + 768 * sizeof(float); }

hipError_t launch_bwd_chunk(const BackwardArgs& a, const float* ckpt, char* fac, float* dSend,
                            float* dA_part, hipStream_t stream) {
    const int NC = (a.T + kChunk - 1) / kChunk;
    const size_t units = (size_t)a.B * a.H;
    const bf16 *q = (const bf16*)a.q, *k = (const bf16*)a.k, *v = (const bf16*)a.v,
               *z = (const bf16*)a.z, *dO = (const bf16*)a.dO;
    float* tri = (float*)(fac + units * NC * (size_t)CBlk::BYTES);
    hipLaunchKernelGGL(bwd_fac_kernel, dim3((unsigned)(units * NC)), dim3(256), 0, stream, q, k, z,
                       a.beta, a.A, a.g_min, fac, tri, a.B, a.T, a.H);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned chains = (unsigned)(((units + 7) / 8) * 8 * (kD / 16));
    hipLaunchKernelGGL(bwd_dchain_kernel, dim3(chains), dim3(128), 0, stream, fac, dO, a.dST, dSend,
                       a.dS0, a.B, a.T, a.H);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_grad_kernel, dim3((unsigned)(units * NC)), dim3(256), 0, stream, q, k, v,
                       z, a.beta, a.A, a.g_min, dO, ckpt, dSend, tri, (bf16*)a.dq, (bf16*)a.dk,
                       (bf16*)a.dv, (bf16*)a.dz, a.dbeta, dA_part, a.B, a.T, a.H);
    return hipGetLastError();
}

}  // namespace kda
