// kda_pair.hip -- split-plan prefill for gfx950: the state chain advances two
// 16-token chunks per step.
//
// The pair block, its producer and the pair step are in kda_pair.hpp.
#include "kda_pair.hpp"

namespace kda {

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
        pair_produce<E, D, PStage<E, D>>(ca, cb, make_gate(A[u % H], g_min), st, out,
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
