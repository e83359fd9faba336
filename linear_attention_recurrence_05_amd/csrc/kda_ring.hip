// kda_ring.hip -- ring-plan prefill for gfx950: the pair producers and the
// state chains of a sequence-head run side by side in one launch, and the
// pair blocks pass between them through the L2 cache of one XCD instead of
// a round trip through HBM.
//
// Source of the method: dev.to "Kimi K3 Architecture: Scaling 2.8T Parameters
// for Long-Context Multimodal MoE", section "The Sequence Bottleneck: Hybrid
// KDA and Gated MLA" (16-token tiles, chunkwise parallel form); the two-chunk
// pair step and its block are those of kda_pair.hpp, unchanged.
//
// For few sequence-heads (B * H <= CUs / 8), every unit u = (b, h) gets
// D / 16 = 8 workgroups, one per 16-column tile of the state, all on the
// XCD u mod 8 (workgroups are dispatched round-robin over the XCDs; each
// workgroup checks the XCD it runs on).  The grid is at most one workgroup
// per CU and every workgroup fits a CU by itself, so the whole grid is
// resident at once, which the waits between workgroups need.  A workgroup:
//   waves 0..2  producers: pairs p = tile + 8 (w + 3 j) of the unit, each
//               built in the wave's LDS as a whole pair block, then copied
//               to ring slot p mod R of the unit (global memory that stays
//               in the XCD's L2) once every tile has taken pair p - R;
//   wave 3      the chain of the tile's 16 columns (x, U, state update),
//               alone on its SIMD;
//   wave 4      the outputs of those columns, from the state at the pair's
//               start (bf16, as the chain packs it for its own products)
//               and [U_a; U_b], both handed over by the chain in LDS;
//   wave 5      the gate: forwards the ring's ready flags to LDS for waves
//               3 and 4, publishes their progress, and passes the slowest
//               tile's progress to this workgroup's producers (only the gate
//               polls flags in L2; every other wait is on LDS).
// The chain and output waves load their operands of a pair from the ring
// straight into registers, one pair ahead, and each releases a pair's slot
// as soon as the operands it still needs have arrived.
//
// Handover through L2 (all parties on one XCD, so one L2 serves them):
//   publish: plain stores of the block, s_waitcnt vmcnt(0) (the stores have
//            reached L2), then the flag by an atomic exchange;
//   observe: flags by atomic adds of zero (atomics execute in L2, never in
//            the CU's vector cache), data by loads with the sc1 bit, which
//            bypass the CU's vector cache and are served by L2.
// Plain loads could hit a stale line in the reading CU's own cache.  The
// flags and counters start from a fill kernel launched just before.  Every
// wait is bounded; a wave that gives up writes NaN where its results go.
#include "kda_pair.hpp"

namespace kda {

template <typename E, int D>
struct RingCfg {
    using P = PBlk<E, D>;
    using Sg = PStageFull<E, D>;
    static constexpr int NCT = D / 16;             // 16-column tiles per unit
    // waves go to the four SIMDs in turn: three producers (SIMDs 0-2), the
    // chain alone on SIMD 3, the output wave and the gate beside producers
    static constexpr int NPW = 3;                  // producer waves
    static constexpr int WCH = NPW, WOUT = NPW + 1, WGATE = NPW + 2;
    static constexpr int THREADS = (NPW + 3) * kWave;
    // ring slots per unit: a consumer waits for pair s + 1 while it holds
    // pair s, and a slot is refilled only after every tile of the unit has
    // released its pair, so the slots beyond two are the slack that hides
    // the hand-off (release, the gates' rounds, the 28 KB publish).  10 are
    // 2-3% faster than 8 at B1 H32 (1.34x against 1.19x the algorithmic
    // bytes at T4096: some blocks are evicted dirty); 12 are slower again,
    // and 16 move 1.9x, as the streaming inputs and outputs evict most
    // blocks from the XCD's 4 MB L2 before their slots are refilled
    static constexpr int R = 10;
    static constexpr int NU = 4;                   // entries chain -> output wave
    // an entry: [U_a; U_b] (bf16x8 per lane), then the packed state (NSLOT
    // bf16x8 per lane)
    static constexpr int UBYTES = kWave * 16 * (1 + P::NSLOT);
    static constexpr int UOFF = NPW * Sg::BYTES;
    static constexpr int LDS = UOFF + NU * UBYTES;
    // flags of a unit (ints): ready[R] (last pair published in each slot),
    // done[NCT] (last pair every consumer of the tile has taken); the gate
    // reads both with one atomic per lane (ready on lanes 0 .. R-1, done on
    // lanes 32 .. 32 + NCT - 1)
    static constexpr int FL_READY = 0, FL_DONE = 32, FL_INTS = 64;
    static_assert(R <= 32 && NCT <= 32, "flag layout");
    static_assert(LDS <= 160 * 1024 - 64, "LDS of one workgroup");
    static_assert(P::BYTES % 16 == 0, "16-byte copies");
};

// The XCD this wave runs on (hardware register XCC_ID, bits 3:0).
__device__ __forceinline__ int xcd_id() {
    return __builtin_amdgcn_s_getreg(20 | (0 << 6) | ((4 - 1) << 11)) & 15;
}

// Zero the optimiser cannot see through, so an atomic add of it stays an
// atomic (an add of a literal zero may become a plain load).
__device__ __forceinline__ int opaque_zero() {
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    return z;
}

// A flag as the XCD's L2 holds it.
__device__ __forceinline__ int l2_read(int* f) {
    return __hip_atomic_fetch_add(f, opaque_zero(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void l2_write(int* f, int x) {
    (void)__hip_atomic_exchange(f, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Every store this wave issued has reached L2.
__device__ __forceinline__ void stores_reached_l2() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    vm_wait_all();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

// Loads served by L2 (sc1: past the CU's vector cache).
template <typename T>
__device__ __forceinline__ T l2_load(Rsrc r, int off);
template <>
__device__ __forceinline__ bf16x8 l2_load<bf16x8>(Rsrc r, int off) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16));
}
template <>
__device__ __forceinline__ bf16x4 l2_load<bf16x4>(Rsrc r, int off) {
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 16));
}
template <>
__device__ __forceinline__ f32x2 l2_load<f32x2>(Rsrc r, int off) {
    return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 16));
}

// Chain operands of the pair block at byte `base` of the ring buffer, in
// two groups issued at different points of the chain's step: the first
// products' operands (Kt_a, Kt_b Diag(gam_a)), and the rest (U and state
// update operands).
template <typename E, int D>
__device__ __forceinline__ void ring_load_chain_k(POps<E, D>& c, Rsrc r, int base) {
    using P = PBlk<E, D>;
    const int lane = lane_id(), g = lane >> 4, rr = lane & 15;
#pragma unroll
    for (int s = 0; s < P::NSLOT; ++s) {
        const int off = P::B1::arow_chunk(s, g, rr);
        c.ka[s] = l2_load<V16<E>>(r, base + P::KA + off);
        c.kb[s] = l2_load<V16<E>>(r, base + P::KB + off);
    }
}
// A-row slot s of Kt_a and Kt_b Diag(gam_a).
template <typename E, int D>
__device__ __forceinline__ void ring_load_k_slot(POps<E, D>& c, Rsrc r, int base, int s) {
    using P = PBlk<E, D>;
    const int lane = lane_id(), g = lane >> 4, rr = lane & 15;
    const int off = P::B1::arow_chunk(s, g, rr);
    c.ka[s] = l2_load<V16<E>>(r, base + P::KA + off);
    c.kb[s] = l2_load<V16<E>>(r, base + P::KB + off);
}
// The 16x16 operands of U_a, U_b and the pair decay.
template <typename E, int D>
__device__ __forceinline__ void ring_load_small(POps<E, D>& c, Rsrc r, int base) {
    using P = PBlk<E, D>;
    const int lane = lane_id(), g = lane >> 4, rr = lane & 15;
    c.tma = l2_load<V4<E>>(r, base + P::TMA + lane * P::OPB);
    c.mkb = l2_load<V4<E>>(r, base + P::MKB + lane * P::OPB);
    c.tmb = l2_load<V4<E>>(r, base + P::TMB + lane * P::OPB);
    c.gv = l2_load<f32x2>(r, base + P::GAB + row_vec_offset<D>(g, rr));
}
// Row tile m of the state-update operand.
template <typename E, int D>
__device__ __forceinline__ void ring_load_kd2(POps<E, D>& c, Rsrc r, int base, int m) {
    using P = PBlk<E, D>;
    const int lane = lane_id(), g = lane >> 4, rr = lane & 15;
    c.kd2[m] = l2_load<V8<E>>(r, base + P::kd2_offset(m, g, rr));
}
template <typename E, int D>
__device__ __forceinline__ void ring_load_chain_rest(POps<E, D>& c, Rsrc r, int base) {
    ring_load_small<E, D>(c, r, base);
#pragma unroll
    for (int m = 0; m < PBlk<E, D>::MT; ++m) ring_load_kd2<E, D>(c, r, base, m);
}

// Output-wave operands.
template <typename E, int D>
__device__ __forceinline__ void ring_load_out(POps<E, D>& c, Rsrc r, int base) {
    using P = PBlk<E, D>;
    const int lane = lane_id(), g = lane >> 4, rr = lane & 15;
#pragma unroll
    for (int s = 0; s < P::NSLOT; ++s) {
        const int off = P::B1::arow_chunk(s, g, rr);
        c.qa[s] = l2_load<V16<E>>(r, base + P::QA + off);
        c.qb[s] = l2_load<V16<E>>(r, base + P::QB + off);
    }
    c.aqa = l2_load<V4<E>>(r, base + P::AQA + lane * P::OPB);
    c.ob2 = l2_load<V8<E>>(r, base + P::OB2 + lane * 2 * P::OPB);
}

// V rows t0 .. t0 + 31 of the tile's 16 columns in the A-operand layout of a
// 16x16x16 product (lane (r, g) holds row r, columns 4g .. 4g + 3, of each
// chunk); rows past T read 0.
template <int D>
__device__ __forceinline__ void ring_load_v(const bf16* v, int b, int h, int T, int H,
                                            int col0, int s, u32x2& va, u32x2& vb) {
    const int t0 = 2 * s * kChunk;
    const int Lr = min(2 * kChunk, T - t0);
    const size_t rs = (size_t)H * D;
    const Rsrc rv = make_rsrc(v + (((size_t)b * T + t0) * H + h) * D + col0,
                              Lr > 0 ? (uint32_t)(((size_t)(Lr - 1) * rs + 16) * 2) : 0u);
    const int lane = lane_id();
    const int off = (int)(((lane & 15) * rs + 4 * (lane >> 4)) * 2);
    va = buf_load<u32x2>(rv, off);
    vb = buf_load<u32x2>(rv, off + (int)(kChunk * rs * 2));
}

// Bounded poll of an LDS flag; `live` false: no wait (a wave that already
// gave up).  Returns whether the wave is still live.
__device__ __forceinline__ bool lds_wait_ge(const int* flag, int target, bool live) {
    if (!live) return false;
    const bool ok = spin_until_ge(flag, target);
    pin_issued();
    return ok;
}

// Mark the gate stores to lready and lfree when it gives up: above every
// pair index, so every wait on them ends, and a consumer that reads it
// poisons its results.
constexpr int kGaveUp = 1 << 30;

// The same with the last value read kept in `seen`: no LDS access while
// seen >= target (flags only grow), and one read per poll otherwise (the
// value that ends the wait is the one kept).  A wait that gives up, or a
// value at kGaveUp, sets `poisoned`.
__device__ __forceinline__ bool lds_wait_seen(const int* flag, int target, int& seen, bool live,
                                              bool& poisoned) {
    if (seen >= target) return live;
    int v = 0x7fffffff;
    if (live) {
        live = false;
        for (int it = 0; it < kSpinLimit; ++it) {
            v = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (v >= target) {
                live = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (!live) v = 0x7fffffff;
    }
    seen = v;
    poisoned = poisoned || !live || v >= kGaveUp;
    // later LDS reads stay after the poll that released them
    asm volatile("" ::: "memory");
    pin_issued();
    return live;
}

// Ties the registers of loaded operands to this point: the compiler waits
// here for the loads that fill them (and only those), so a release of their
// slot after it cannot let a refill overtake them.
template <typename T>
__device__ __forceinline__ void regs_arrived(const T& x) {
    if constexpr (sizeof(T) == 16) asm volatile("" ::"v"(__builtin_bit_cast(u32x4, x)));
    else if constexpr (sizeof(T) == 8) asm volatile("" ::"v"(__builtin_bit_cast(u32x2, x)));
    else asm volatile("" ::"v"(__builtin_bit_cast(uint32_t, x)));
}

// A flag value read ahead of its wait (the read's latency then overlaps other
// work): taken into `seen` as a poll would take it.
__device__ __forceinline__ void lds_note(int v, int& seen, bool& poisoned) {
    seen = max(seen, v);
    poisoned = poisoned || v >= kGaveUp;
}

template <typename E, int D>
__global__ __launch_bounds__((RingCfg<E, D>::THREADS)) void pair_ring_kernel(
    const E* q, const E* k, const E* v, const E* z, const float* beta, const float* A, float g_min,
    StateIO io, E* o, char* ring, int* flags, int B, int T, int H) {
    // (no __restrict__: loads through a restrict pointer may move across the
    // compiler fences that keep each load group in its place in a step, and
    // the waits for a pair's operands count on that order)
    using P = PBlk<E, D>;
    using Cfg = RingCfg<E, D>;
    using Sg = PStageFull<E, D>;
    constexpr int R = Cfg::R, NCT = Cfg::NCT, NPW = Cfg::NPW, NU = Cfg::NU;
    __shared__ __attribute__((aligned(16))) char lds[Cfg::LDS];
    // lready: last pair the gate saw published; lfree: last pair every tile
    // of the unit has taken (its slot may be refilled); ldone[c]: last pair
    // consumer c (0 chain, 1 output) has taken from the ring; uready / udone:
    // the entries between chain and output wave; lbad: the workgroup is not
    // on its unit's XCD (a gate that gives up stores kGaveUp to lready and
    // lfree instead)
    __shared__ int lready, lfree, ldone[2], uready, udone, lbad;
    int u, ct;
    if (!map_unit(NCT, B * H, u, ct)) return;   // uniform over the workgroup
    const int b = u / H, h = u % H;
    if (io.skip(b)) return;                      // uniform over the workgroup
    const int w = wave_id();
    const int lane = lane_id();
    const int NC = (T + kChunk - 1) / kChunk;
    const int NP = (NC + 1) / 2;
    const int col0 = ct * 16;
    int* fl = flags + (size_t)u * Cfg::FL_INTS;
    char* slots = ring + (size_t)u * R * P::BYTES;
    const Rsrc rring = make_rsrc(slots, (uint32_t)(R * P::BYTES));
    if (w == 0 && lane == 0) {
        lready = lfree = -1;
        ldone[0] = ldone[1] = -1;
        uready = udone = -1;
        lbad = xcd_id() != (int)(blockIdx.x & 7);
    }
    // the chain starts from the tile's initial state (read before the
    // barrier: S_T may alias S0)
    f32x4 S[1][D / 16];
    if (w == Cfg::WCH) state_load<D, 1>(S, io.in_at(b, h, H, D), col0);
    wg_barrier();   // the only barrier: flags initialised

    if (w < NPW) {
        // -------------------------------------------------------- producers
        char* st = lds + w * Sg::BYTES;
        const GateConsts gc = make_gate(A[h], g_min);
        const int stride = NCT * NPW;
        int p = ct + NCT * w;
        if (p >= NP) return;
        auto load = [&](int pp, int half, bool live, ProdIn<E, D>& c) {
            ChunkPos cp = chunk_pos<D>(b, h, 2 * pp + half, T, H);
            cp.L = live ? cp.L : 0;
            prod_load<E, D>(c, q, k, z, beta, cp);
        };
        ProdIn<E, D> ca, cb;
        load(p, 0, true, ca);
        load(p, 1, true, cb);
        bool live = true;
        for (;;) {
            const int np = p + stride;
            const bool more = np < NP;
            pair_produce<E, D, Sg>(ca, cb, gc, st, nullptr, [&] { load(np, 0, more, ca); },
                                   [&] { load(np, 1, more, cb); });
            // slot p mod R is free once every tile has taken pair p - R
            live = lds_wait_ge(&lfree, p - R, live);
            pin_issued();
            // the block to its slot (NaN words if the wait gave up): LDS
            // reads into registers, then buffer stores issued back to back
            {
                constexpr int N16 = P::BYTES / 16, NPL = (N16 + kWave - 1) / kWave;
                const Rsrc rs = make_rsrc(slots + (size_t)(p % R) * P::BYTES, (uint32_t)P::BYTES);
#pragma unroll
                for (int i = 0; i < NPL; ++i) {
                    const int x = i * kWave + lane;
                    if (i + 1 < NPL || x < N16) {
                        u32x4 val = *reinterpret_cast<const u32x4*>(st + x * 16);
                        if (!live) val = u32x4{kNaNWord, kNaNWord, kNaNWord, kNaNWord};
                        buf_store_u32x4(rs, x * 16, val);
                    }
                }
            }
            stores_reached_l2();
            if (lane == 0) l2_write(fl + Cfg::FL_READY + p % R, p);
            wave_sync_lds();   // the staging is reused for the next pair
            if (!more) break;
            p = np;
        }
        return;
    }

    if (w == Cfg::WGATE) {
        // -------------------------------------------------------- gate
        // one atomic per lane and round: lanes 0 .. R-1 read the R ready
        // flags, lanes 32 .. 32 + NCT - 1 the tiles' done flags; the run of
        // published pairs from p on is forwarded in one step
        int p = 0, published = -1, freed = -1, idle = 0;
        while (p < NP) {
            const int d = min(__hip_atomic_load(&ldone[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP),
                              __hip_atomic_load(&ldone[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
            if (d > published) {
                if (lane == 0) l2_write(fl + Cfg::FL_DONE + ct, d);
                published = d;
            }
            const bool rl = lane < R, dl = lane >= 32 && lane < 32 + NCT;
            const int want = p + ((lane - p % R + R) % R);   // the pair lane's slot holds next
            const int got = rl ? l2_read(fl + Cfg::FL_READY + lane)
                               : dl ? l2_read(fl + Cfg::FL_DONE + lane - 32) : 0;
            // slowest tile
            int mn = 0x7fffffff;
#pragma unroll
            for (int t = 0; t < NCT; ++t) mn = min(mn, __builtin_amdgcn_readlane(got, 32 + t));
            if (mn > freed) {
                freed = mn;
                if (lane == 0) __hip_atomic_store(&lfree, mn, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
            const uint64_t m = __builtin_amdgcn_ballot_w64(rl && got >= want);
            const int sh = p % R;
            const uint32_t run = (uint32_t)(((m >> sh) | (m << (R - sh))) & ((1u << R) - 1));
            const int n = min(__builtin_ctz(~run), NP - p);
            if (n > 0) {
                p += n;
                asm volatile("" ::: "memory");
                if (lane == 0) __hip_atomic_store(&lready, p - 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                idle = 0;
                continue;
            }
            if (++idle > kSpinLimit) {
                // give up: every wait of the workgroup ends and its results
                // are poisoned
                if (lane == 0) {
                    __hip_atomic_store(&lfree, kGaveUp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    __hip_atomic_store(&lready, kGaveUp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                }
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        return;
    }

    const int j = lane & 15, g = lane >> 4;
    // identity in the B layout of a 16x16x16 product: V rows (A layout) -> V
    // in the accumulator layout, exactly
    bf16x4 ident;
#pragma unroll
    for (int i = 0; i < 4; ++i) ident[i] = (bf16)(4 * g + i == j ? 1.f : 0.f);
    char* uring = lds + Cfg::UOFF;

    if (w == Cfg::WCH) {
        // -------------------------------------------------------- chain
        // A step issues the next pair's loads between its own products: the
        // K rows of the next pair between the x products, the small
        // operands after them, the state-update operand between the
        // update's products.  A CU's vector memory pipeline takes a load
        // every ~20 cycles here, so a burst of them at the top of the step
        // would hold the wave for most of its MFMA time; spread out, they
        // drain while the products run, and each still arrives a whole step
        // before its use (an L2 access takes about as long as a step).  V
        // comes from HBM and goes first.  The last step reloads its own
        // pair, so every step issues the same loads in the same order and a
        // wait for this pair's operands never includes the next pair's.
        POps<E, D> c0, c1;
        u32x2 va0, vb0, va1, vb1;
        int seen_ready = -1, seen_udone = -1, ahead_ready = -1, ahead_udone = -1;
        bool bad = __hip_atomic_load(&lbad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0;
        bool live = lds_wait_seen(&lready, 0, seen_ready, true, bad);
        // (pair 0's loads in the order a step issues them)
        ring_load_v<D>(v, b, h, T, H, col0, 0, va0, vb0);
        ring_load_chain_k<E, D>(c0, rring, 0);
        ring_load_chain_rest<E, D>(c0, rring, 0);
        pin_issued();
        auto step = [&](POps<E, D>& c, const u32x2& va, const u32x2& vb, POps<E, D>& cn, u32x2& van,
                        u32x2& vbn, int s) {
            const int sn = s + 1 < NP ? s + 1 : s;
            const int nbase = (sn % R) * P::BYTES;
            // the next pair is in the ring; the output wave has read entry s - NU
            lds_note(ahead_ready, seen_ready, bad);
            lds_note(ahead_udone, seen_udone, bad);
            live = lds_wait_seen(&lready, sn, seen_ready, live, bad);
            live = lds_wait_seen(&udone, s - NU, seen_udone, live, bad);
            if (bad) poison_state(S[0]);
            pin_issued();
            ring_load_v<D>(v, b, h, T, H, col0, sn, van, vbn);
            pin_issued();
            bf16x8* e = reinterpret_cast<bf16x8*>(uring + (s % NU) * Cfg::UBYTES);
            const f32x4 Va = mma_bf16_k16(__builtin_bit_cast(bf16x4, va), ident, zero4());
            const f32x4 Vb = mma_bf16_k16(__builtin_bit_cast(bf16x4, vb), ident, zero4());
            bf16x8 sb[1][P::NSLOT];
            f32x4 xa[1], xb[1];
            pair_x<E, D, 1>(c, S, sb, xa, xb, [&](int k) {
                ring_load_k_slot<E, D>(cn, rring, nbase, k);
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // the slot's 2 products
                __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);   // then its 2 loads
            });
            ring_load_small<E, D>(cn, rring, nbase);
#pragma unroll
            for (int kk = 0; kk < P::NSLOT; ++kk) e[(1 + kk) * kWave + lane] = sb[0][kk];
            const bf16x8 u2 = pair_u<E, D>(c, xa[0], xb[0], Va, Vb);
            e[lane] = u2;
            asm volatile("" ::: "memory");
            __hip_atomic_store(&uready, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            // both flags of the next step's waits, read while the state
            // update runs
            ahead_ready = __hip_atomic_load(&lready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            ahead_udone = __hip_atomic_load(&udone, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            // the pair's last operands (the update's) have arrived: its slot
            // is released before the update runs (the others were used above)
#pragma unroll
            for (int m = 0; m < P::MT; ++m) regs_arrived(c.kd2[m]);
            regs_arrived(c.gv);
            pin_issued();
            __hip_atomic_store(&ldone[0], s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            pair_supdate<E, D>(c, S[0], u2, [&](int m) {
                ring_load_kd2<E, D>(cn, rring, nbase, m);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);   // the tile's product
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);   // then its load
            });
            pin_issued();
        };
        // whole pairs of steps in the loop, an odd last step after it: every
        // path into the loop head then has the same loads in flight
        int s = 0;
        for (; s + 1 < NP; s += 2) {
            step(c0, va0, vb0, c1, va1, vb1, s);
            step(c1, va1, vb1, c0, va0, vb0, s + 1);
        }
        if (s < NP) step(c0, va0, vb0, c1, va1, vb1, s);
        if (io.out) state_store<D, 1>(S, io.out_at(b, h, H, D), col0);
        return;
    }

    // ------------------------------------------------------------ outputs
    POps<E, D> c0, c1;
    int seen_ready = -1, seen_u = -1;
    bool bad = __hip_atomic_load(&lbad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0;
    bool live = lds_wait_seen(&lready, 0, seen_ready, true, bad);
    ring_load_out<E, D>(c0, rring, 0);
    auto step = [&](POps<E, D>& c, POps<E, D>& cn, int s) {
        const int sn = s + 1 < NP ? s + 1 : s;   // as in the chain
        // The next pair's loads go out once the chain has left its own loads
        // behind, so the two waves' bursts do not meet in the CU's memory
        // pipeline.  The chain stores uready = s only after its wait for
        // pair sn, so pair sn is in the ring by then (a chain whose wait
        // ended in a give-up poisons the state it passes on, and with it
        // these outputs).
        live = lds_wait_seen(&uready, s, seen_u, live, bad);
        ring_load_out<E, D>(cn, rring, (sn % R) * P::BYTES);
        // this pair's operands (loaded a step ago) have arrived: its slot is
        // released now, not after the products
#pragma unroll
        for (int kk = 0; kk < P::NSLOT; ++kk) {
            regs_arrived(c.qa[kk]);
            regs_arrived(c.qb[kk]);
        }
        regs_arrived(c.aqa);
        regs_arrived(c.ob2);
        pin_issued();
        __hip_atomic_store(&ldone[1], s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const bf16x8* e = reinterpret_cast<const bf16x8*>(uring + (s % NU) * Cfg::UBYTES);
        const bf16x8 u2 = e[lane];
        bf16x8 sb[P::NSLOT];
#pragma unroll
        for (int kk = 0; kk < P::NSLOT; ++kk) sb[kk] = e[(1 + kk) * kWave + lane];
        f32x4 Oa, Ob;
        pair_out<E, D>(c, sb, u2, Oa, Ob);
        if (bad) {
            const float nan = __builtin_bit_cast(float, kNaNWord);
            Oa = Ob = f32x4{nan, nan, nan, nan};
        }
        // the entry is in registers (its last use waited for it): release it
        pin_issued();
        __hip_atomic_store(&udone, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        // outputs: rows 4g + (j & 3) of each chunk, columns 4 (j >> 2) .. +3
        // of the tile, 8 bytes per lane and chunk; rows past T are dropped
        const int t0 = 2 * s * kChunk;
        const int Lr = min(2 * kChunk, T - t0);
        const size_t rs = (size_t)H * D;
        const Rsrc ro = make_rsrc(o + (((size_t)b * T + t0) * H + h) * D + col0,
                                  Lr > 0 ? (uint32_t)(((size_t)(Lr - 1) * rs + 16) * 2) : 0u);
        const int r = 4 * g + (j & 3), off = (int)((r * rs + 4 * (j >> 2)) * 2);
        buf_store_u32x2(ro, off, acc_rows_bf16(Oa));
        buf_store_u32x2(ro, off + (int)(kChunk * rs * 2), acc_rows_bf16(Ob));
    };
    int s = 0;
    for (; s + 1 < NP; s += 2) {   // as in the chain
        step(c0, c1, s);
        step(c1, c0, s + 1);
    }
    if (s < NP) step(c0, c1, s);
}

// Flags of every unit to -1 (nothing published, nothing taken).
__global__ void ring_flags_init(int* __restrict__ flags, int n) {
    for (int i = (int)(blockIdx.x * blockDim.x + threadIdx.x); i < n; i += (int)(gridDim.x * blockDim.x))
        flags[i] = -1;
}

// ------------------------------------------------------------ launch

// CUs of the current device (read once per device).
static int device_cus() {
    static int cus[64];   // 0: not read yet
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev >= 64) {
        int n = 0;
        return hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? n : 0;
    }
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cus[dev] = n;
    }
    return cus[dev];
}

bool ring_ok(int B, int H, int d, bool is_bf16) {
    if (!is_bf16 || d != 128) return false;
    const long units = (long)B * H;
    const long wgs = ((units + 7) / 8) * 8 * RingCfg<bf16, 128>::NCT;
    return units >= 1 && wgs <= device_cus();
}

size_t ring_ws_bytes(int B, int H, int d, bool is_bf16) {
    (void)d;
    (void)is_bf16;
    using Cfg = RingCfg<bf16, 128>;
    const size_t units = (size_t)B * H;
    const size_t flag_bytes = (units * Cfg::FL_INTS * sizeof(int) + 255) / 256 * 256;
    return flag_bytes + units * Cfg::R * PBlk<bf16, 128>::BYTES;
}

hipError_t launch_ring(const PrefillArgs& a, void* ws, hipStream_t stream) {
    if (!ring_ok(a.B, a.H, a.d, a.is_bf16) || a.lim.in || a.lim.out || !a.o || !a.v || !ws)
        return hipErrorInvalidValue;
    using Cfg = RingCfg<bf16, 128>;
    const int units = a.B * a.H;
    const size_t flag_bytes = ((size_t)units * Cfg::FL_INTS * sizeof(int) + 255) / 256 * 256;
    int* flags = (int*)ws;
    char* ring = (char*)ws + flag_bytes;
    const int nflags = units * Cfg::FL_INTS;
    hipLaunchKernelGGL(ring_flags_init, dim3((unsigned)((nflags + 255) / 256)), dim3(256), 0, stream,
                       flags, nflags);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned grid = (unsigned)(((units + 7) / 8) * 8 * Cfg::NCT);
    hipLaunchKernelGGL((pair_ring_kernel<bf16, 128>), dim3(grid), dim3(Cfg::THREADS), 0, stream,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.z,
                       a.beta, a.A, a.g_min, a.S, (bf16*)a.o, ring, flags, a.B, a.T, a.H);
    return hipGetLastError();
}

}  // namespace kda
