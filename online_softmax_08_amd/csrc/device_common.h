// device_common.h -- small gfx950 (CDNA4) device helpers shared by the kernels
// of this library: vector types, wave64 reductions built from DPP and the
// gfx950 permlane swaps, and exp2 on the hardware transcendental unit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace osm {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();

// 2^x on the transcendental unit (v_exp_f32).  exp2(-inf) = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) on the transcendental unit (v_log_f32).
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// DPP lane moves inside 16-lane rows.  Control codes follow the GFX9 DPP
// encoding: quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E, row_half_mirror =
// 0x141, row_mirror = 0x140.
template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF,
                                                      false));
}

// Value of lane ^ 32 (gfx950 v_permlane32_swap with both operands = v).
__device__ __forceinline__ float lane_xor32(float v)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                              false);
    // r[0]: lanes 0-31 keep v, lanes 32-63 receive v of lanes 0-31;
    // r[1]: lanes 0-31 receive v of lanes 32-63, lanes 32-63 keep v.
    return __uint_as_float(__lane_id() < 32 ? r[1] : r[0]);
}

// Value of lane ^ 16 (gfx950 v_permlane16_swap with both operands = v).
__device__ __forceinline__ float lane_xor16(float v)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                              false);
    return __uint_as_float((__lane_id() & 16) ? r[0] : r[1]);
}

// op(v, v of lane ^ 32) without a lane select: the swap hands every lane
// both halves' values.
template <class Op>
__device__ __forceinline__ float combine_xor32(float v, Op op)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                              false);
    return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// op(v, v of lane ^ 16), likewise.
template <class Op>
__device__ __forceinline__ float combine_xor16(float v, Op op)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                              false);
    return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

struct MaxOp {
    __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct SumOp {
    __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};

// Butterfly reduction over all 64 lanes; every lane ends with the same value
// (each step combines a lane with its partner, and the operation is
// commutative, so partners compute identical results).
template <class Op>
__device__ __forceinline__ float wave_reduce(float v, Op op)
{
    v = op(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
    v = op(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
    v = op(v, dpp<0x141>(v));  // row_half_mirror: combine the two quads of a half-row
    v = op(v, dpp<0x140>(v));  // row_mirror: combine the two half-rows
    v = combine_xor16(v, op);  // combine 16-lane rows pairwise
    v = combine_xor32(v, op);  // combine the two 32-lane halves
    return v;
}

// Output tile of one wave, 32 rows x D, from transposed MFMA accumulators
// acc[D / 32] (lane j owns output row row0 + j, and its lane half h owns
// columns 32 dt + 8 g + 4 h .. + 3 in registers 4 g .. 4 g + 3 of acc[dt]),
// times mul, rounded to bf16 and stored to the [rows][D] tensor of buffer
// resource ors.  Direct stores would write 16-byte pieces of 32 different
// rows per instruction; instead the wave writes its rows into the LDS region
// ost (32 rows of pitch D + 8 elements, 2-way bank conflicts at most) and
// then stores whole rows, 64 lanes x 16 bytes = 64 / (D / 8) rows per
// instruction.  Rows past the resource's range are dropped.  Only the
// calling wave touches ost, so a wave-local wait orders the two halves; a
// second call may reuse the same region.
template <int D>
__device__ __forceinline__ void store_tile_rows(const f32x16 (&acc)[D / 32], float mul, char* ost,
                                                __amdgpu_buffer_rsrc_t ors, int row0, int lane)
{
    const int j = lane & 31, h = lane >> 5;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 o4 = {acc[dt][4 * g] * mul, acc[dt][4 * g + 1] * mul,
                              acc[dt][4 * g + 2] * mul, acc[dt][4 * g + 3] * mul};
            *reinterpret_cast<bf16x4*>(ost + (j * (D + 8) + dt * 32 + 8 * g + 4 * h) * 2) =
                __builtin_convertvector(o4, bf16x4);
        }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes have landed
    __builtin_amdgcn_wave_barrier();
    constexpr int CPR = D / 8, RPI = 64 / CPR;
#pragma unroll
    for (int u = 0; u < 32 / RPI; ++u) {
        const int row = u * RPI + lane / CPR, ch = lane % CPR;
        const u32x4 v4 = *reinterpret_cast<const u32x4*>(ost + (row * (D + 8) + ch * 8) * 2);
        __builtin_amdgcn_raw_buffer_store_b128(v4, ors, (uint32_t)((row0 + row) * D + ch * 8) * 2, 0, 0);
    }
}

}  // namespace osm
