// kda_device.hpp -- device-side building blocks for the gfx950 KDA kernels:
// element types, bf16 conversion, MFMA wrappers, lane-layout helpers and the
// gate arithmetic.
//
// Lane layouts (wave64).  A 16x16 fp32 MFMA result ("acc layout") puts in
// lane l the column j = l % 16 and rows 4*(l/16) + {0,1,2,3}.  Throughout,
// g = l / 16 is the lane group and the MFMA K index held by a lane is chosen
// so that the acc layout of one product can feed the next product as its B
// operand without moving data between lanes (the K order of a contraction is
// free as long as both operands use the same one).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace kda {

constexpr int kChunk = 16;     // tokens per chunk (the pages' 16-token tiles)
constexpr int kWave = 64;

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ scalars

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __builtin_bit_cast(float, bits16 << 16);
}

// Element <-> fp32.  bf16 is stored as its 16-bit pattern.
template <typename E> __device__ __forceinline__ float to_f32(E x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16>(bf16 x) { return (float)x; }

template <typename E> __device__ __forceinline__ E from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// Round to nearest even (the hardware conversion on gfx950).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

constexpr float kLog2e = 1.4426950408889634f;

// Gate constants of one head: x = e^{A_h} z, g = g_min Sigmoid(x), a = e^g.
struct GateConsts {
    float neg_ea_log2e;    // -e^{A_h} log2(e): exp2(z * this) = e^{-x}
    float gmin_log2e;      // g_min log2(e):    exp2(s * this) = e^{g}
    float gmin;
};

__device__ __forceinline__ GateConsts make_gate(float A_h, float g_min) {
    GateConsts c;
    c.neg_ea_log2e = -__expf(A_h) * kLog2e;
    c.gmin_log2e = g_min * kLog2e;
    c.gmin = g_min;
    return c;
}

// Sigmoid(e^{A_h} z) = 1 / (1 + e^{-x}); overflow of e^{-x} gives 0 and
// underflow gives 1, which are the limits.
__device__ __forceinline__ float gate_sigmoid(const GateConsts& c, float z) {
    return fast_rcp(1.0f + fast_exp2(z * c.neg_ea_log2e));
}

// Retention a = exp(g_min * s) for a sigmoid value s.
__device__ __forceinline__ float gate_alpha(const GateConsts& c, float s) {
    return fast_exp2(s * c.gmin_log2e);
}

// Retention of gate input z in a row that may be padding: keep = 1 for a real
// row (the same value as gate_alpha(c, gate_sigmoid(c, z))), keep = 0 for
// padding, whose retention is then exactly e^0 = 1.  A multiply instead of a
// select keeps the code branch-free: the compiler turns a select between e^g
// and 1 on the uniform row count into a branch around the exponentials,
// which splits an unrolled loop over rows into one scheduling region per row.
__device__ __forceinline__ float gate_alpha_row(const GateConsts& c, float z, float keep) {
    return fast_exp2(gate_sigmoid(c, z) * keep * c.gmin_log2e);
}

// ------------------------------------------------------------------ buffers

// Raw buffer resource over [base, base + bytes): loads past the end return 0
// and stores past it are dropped (hardware range check on the VGPR offset),
// which is how short chunks and padded rows are handled without branches.
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// 16 bytes per lane from the buffer straight into LDS: lane l's bytes land at
// lds + 16 l (lds wave-uniform), without VGPRs.  Completion is counted like a
// load's (in order with the wave's other loads); past the buffer's end the
// bytes are zero.
__device__ __forceinline__ void buf_load_lds16(Rsrc r, int off, void* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 0);
}
// Wait until every buffer load this wave issued has completed (vmcnt = 0;
// expcnt and lgkmcnt left at their maximum, i.e. not waited for).
__device__ __forceinline__ void vm_wait_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
template <typename T> __device__ __forceinline__ T buf_load(Rsrc r, int off);
template <> __device__ __forceinline__ uint32_t buf_load<uint32_t>(Rsrc r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
template <> __device__ __forceinline__ u32x2 buf_load<u32x2>(Rsrc r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
template <> __device__ __forceinline__ u32x4 buf_load<u32x4>(Rsrc r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
template <> __device__ __forceinline__ unsigned short buf_load<unsigned short>(Rsrc r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ void buf_store_u16(Rsrc r, int off, unsigned short x) {
    __builtin_amdgcn_raw_buffer_store_b16(x, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store_u32x4(Rsrc r, int off, u32x4 x) {
    __builtin_amdgcn_raw_buffer_store_b128(x, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store_u32x2(Rsrc r, int off, u32x2 x) {
    __builtin_amdgcn_raw_buffer_store_b64(x, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store_u32(Rsrc r, int off, uint32_t x) {
    __builtin_amdgcn_raw_buffer_store_b32(x, r, off, 0, 0);
}

// ------------------------------------------------------------------ lanes

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// x of lane L of each row of 16 lanes, for every lane of the row (a DPP
// row broadcast: a VALU operand modifier, no LDS traffic)
template <int L>
__device__ __forceinline__ float row_bcast(float x) {
    static_assert(L >= 0 && L < 16, "row lane");
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 0x150 + L, 0xF, 0xF, false));
}

// The same broadcast written as a DPP move: a second use of one broadcast
// value then stays a separate instruction that can fold into its own VALU
// operation (one broadcast with two uses becomes a move plus two operations).
template <int L>
__device__ __forceinline__ float row_bcast_mov(float x) {
    static_assert(L >= 0 && L < 16, "row lane");
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + L,
                                                              0xF, 0xF, true));
}

// Values of rows 16 M + 4 g + p (p = 0..3) of a length-D vector for lane
// (j, g) = 16 g + j, when lane (k, g) holds rows 16 (k/2) + 4 g + 2 (k%2) +
// {0, 1} (row_vec_offset): DPP row broadcasts deliver them, so a lane reads
// and holds 8 bytes of the vector instead of 16 per 16-row tile.
template <int M>
__device__ __forceinline__ f32x4 row_tile(const f32x2& gv) {
    return f32x4{row_bcast<2 * M>(gv[0]), row_bcast<2 * M>(gv[1]),
                 row_bcast<2 * M + 1>(gv[0]), row_bcast<2 * M + 1>(gv[1])};
}
template <int M>
__device__ __forceinline__ f32x4 row_tile_mov(const f32x2& gv) {
    return f32x4{row_bcast_mov<2 * M>(gv[0]), row_bcast_mov<2 * M>(gv[1]),
                 row_bcast_mov<2 * M + 1>(gv[0]), row_bcast_mov<2 * M + 1>(gv[1])};
}

// Byte offset (from the start of the fp32 vector) of the two values lane
// (r, g) holds for row_tile; lanes past the last tile read a valid word.
template <int D>
__device__ __forceinline__ int row_vec_offset(int g, int r) {
    const int mm = min(r >> 1, D / 16 - 1);
    return (16 * mm + 4 * g + 2 * (r & 1)) * 4;
}

// f(integral_constant<int, I>) for I = B .. E-1, each with a compile-time index
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}
// The same value, recomputed at every call: values derived from it are not
// hoisted out of a persistent loop and kept live across its iterations
// (which costs registers when the loop body already needs nearly all).
__device__ __forceinline__ int fresh_lane_id() {
    int t = (int)threadIdx.x;
    asm volatile("" : "+v"(t));
    return t & (kWave - 1);   // the mask after the asm keeps the range known
}
// Index of this wave in its workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
}

// Value of lane `src` (0..3) of this lane's quad (DPP quad_perm broadcast).
template <int src>
__device__ __forceinline__ float quad_bcast(float x) {
    constexpr int ctrl = src | (src << 2) | (src << 4) | (src << 6);
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), ctrl,
                                                              0xF, 0xF, true));
}

// ------------------------------------------------------------------ MFMA

// 16x16x32 bf16 -> fp32.  A: lane l holds row l%16, eight K values of group
// l/16; B: lane l holds column l%16, the same eight K values.
__device__ __forceinline__ f32x4 mma_bf16_k32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 16x16x16 bf16 -> fp32 (four K values per lane).
__device__ __forceinline__ f32x4 mma_bf16_k16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                     __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}
// 16x16x4 fp32 (one K value per lane).
__device__ __forceinline__ f32x4 mma_f32_k4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x2 pack2(float a, float b) {
    bf16x2 r;
    r[0] = (bf16)a; r[1] = (bf16)b;
    return r;
}
// Built from two 2-element conversions (one v_cvt_pk_bf16_f32 each).
__device__ __forceinline__ bf16x4 pack4(f32x4 x) {
    const u32x2 w = {__builtin_bit_cast(uint32_t, pack2(x[0], x[1])),
                     __builtin_bit_cast(uint32_t, pack2(x[2], x[3]))};
    return __builtin_bit_cast(bf16x4, w);
}
__device__ __forceinline__ bf16x8 pack8(f32x4 lo, f32x4 hi) {
    bf16x8 r;
    r[0] = (bf16)lo[0]; r[1] = (bf16)lo[1]; r[2] = (bf16)lo[2]; r[3] = (bf16)lo[3];
    r[4] = (bf16)hi[0]; r[5] = (bf16)hi[1]; r[6] = (bf16)hi[2]; r[7] = (bf16)hi[3];
    return r;
}

// 32-bit word of lane (this lane xor X) of the quad, X = 1 or 2.
template <int X>
__device__ __forceinline__ uint32_t quad_xor(uint32_t x) {
    static_assert(X == 1 || X == 2, "quad xor");
    constexpr int ctrl = X == 1 ? 0xB1 : 0x4E;   // quad_perm [1,0,3,2] / [2,3,0,1]
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, ctrl, 0xF, 0xF, false);
}

// Rows of an accumulator tile as bf16, in registers.  Lane (j, g) holds
// column j, rows 4g .. 4g+3 of a 16x16 fp32 tile; on return lane
// (4a + q, g) holds row 4g + q, columns 4a .. 4a+3, as four bf16 (8 bytes,
// column order).  A 4x4 transpose inside each quad of lanes: 16-bit halves
// across lane pairs (xor 1), then 32-bit words across pair pairs (xor 2).
__device__ __forceinline__ u32x2 acc_rows_bf16(f32x4 x) {
    const int q = (int)(threadIdx.x & 3);
    const uint32_t w0 = __builtin_bit_cast(uint32_t, pack2(x[0], x[1]));   // rows 0, 1 of this column
    const uint32_t w1 = __builtin_bit_cast(uint32_t, pack2(x[2], x[3]));   // rows 2, 3
    // lanes (2c, 2c+1): the even lane keeps the low halves (rows 0 and 2) of
    // both columns, the odd lane the high halves (rows 1 and 3)
    const uint32_t sel = (q & 1) ? 0x03020706u : 0x05040100u;
    const uint32_t a0 = __builtin_amdgcn_perm(quad_xor<1>(w0), w0, sel);
    const uint32_t a1 = __builtin_amdgcn_perm(quad_xor<1>(w1), w1, sel);
    // now lane q holds row (q & 1) in a0 and row (q & 1) + 2 in a1, for
    // columns 2 (q >> 1) and 2 (q >> 1) + 1; lanes q and q ^ 2 swap one word
    const bool hi = (q & 2) != 0;
    const uint32_t r = quad_xor<2>(hi ? a0 : a1);
    return hi ? u32x2{r, a1} : u32x2{a0, r};
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace kda
