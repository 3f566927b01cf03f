// fp8_quant.hip -- block quantization of bf16 tensors to FP8 (OCP E4M3) with
// one power-of-two scale per block of 32 elements, optionally after the
// random-sign Hadamard rotation, on gfx950.  These are the two accuracy
// devices of the FP8 section of "Moving less: four generations of
// FlashAttention" (4.6): block quantization (a scale per block instead of
// per tensor) and incoherent processing (Q and K multiplied by one random
// orthogonal matrix M = diag(s) H / sqrt(d) before quantization; M M^T = I
// keeps Q K^T, and the rotation spreads a few large components over all of
// them).
//
// Blocks run along the axis the attention contracts, which is the axis the
// fp8 matrix cores apply a block scale on (32 elements per scale, E8M0
// bytes, value 2^(byte - 127)):
//  * rows (Q, K): 32 consecutive head columns of one row;
//  * columns (V): 32 consecutive rows (keys) of one column of a [n][d] slice.
// A block's scale is 2^e with e the smallest integer for which its largest
// magnitude fits, amax <= 448 * 2^e (e = 0 for an all-zero block); each
// element is the E4M3 code of x / 2^e, rounded to nearest with ties to the
// even code by v_cvt_pk_fp8_f32 (measured on every midpoint of the format).
//
// Both kernels move 2 bytes in and 1 + 1/32 out per element (HBM bound),
// and keep each block in one thread so that its maximum needs no exchange:
//  * fp8_quant_rows_kernel: d / 32 lanes per row, one block of 32 elements
//    per lane.  The rotation is the fast Walsh-Hadamard transform in fp32:
//    five butterfly stages inside the lane and log2(d / 32) across the lanes
//    of the row by DPP swaps, after the sign flips and before 1 / sqrt(d).
//  * fp8_quant_cols_kernel: a quad of threads per 8 columns of a 32-row
//    block, 8 rows per thread held in registers, the column maxima combined
//    by DPP swaps inside the quad.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "kernels.h"

namespace osm {
namespace {

// e of the block scale 2^e: the smallest integer with amax <= 448 * 2^e.
// With amax = f 2^ex, f in [0.5, 1): 448 * 2^(ex - 8) = 1.75 * 2^ex fits,
// and 448 * 2^(ex - 9) = 0.875 * 2^ex fits exactly when f <= 0.875; e - 2
// never does.  Exact in fp32 (frexp, a compare with a power-of-two multiple
// of 448).
__device__ __forceinline__ int block_exponent(float amax)
{
    if (amax == 0.f) return 0;
    int ex;
    (void)frexpf(amax, &ex);
    int e = ex - 8;
    if (amax <= ldexpf(448.0f, e - 1)) e -= 1;
    return max(-127, min(127, e));
}

// Four fp32 values to four E4M3 codes (bytes 0..3 in order).
__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Lane swaps inside quads (DPP quad_perm): the value of lane ^ 1 or lane ^ 2.
template <int M>
__device__ __forceinline__ float quad_xor(float v)
{
    static_assert(M == 1 || M == 2, "quad_perm swaps");
    constexpr int ctrl = M == 1 ? 0xB1 : 0x4E;  // [1,0,3,2] / [2,3,0,1]
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, false));
}

// Rows: D / 32 lanes per row (a quad or half a quad), each holding one block
// of 32 consecutive elements (four 16-byte loads), so a block's maximum is
// in-lane.  The rotation: sign flips, the five butterfly stages of the
// element bits inside the lane, the one or two of the lane bits by DPP lane
// swaps, then 1 / sqrt(D).
template <int D, bool ROT>
__global__ void __launch_bounds__(256)
fp8_quant_rows_kernel(const __bf16* __restrict__ X, uint8_t* __restrict__ codes,
                      uint8_t* __restrict__ scales, long long rows, uint64_t neg_lo,
                      uint64_t neg_hi)
{
    constexpr int LPR = D / 32, RPB = 256 / LPR;
    const int l = threadIdx.x % LPR;  // this lane holds elements 32 l .. 32 l + 31 of its row
    // bit u set: element 32 l + u is negated (s_t = -1)
    const uint32_t neg = l == 0 ? (uint32_t)neg_lo : l == 1 ? (uint32_t)(neg_lo >> 32)
                       : l == 2 ? (uint32_t)neg_hi : (uint32_t)(neg_hi >> 32);
    for (long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR; row < rows;
         row += (long long)gridDim.x * RPB) {
        float v[32];
        const __bf16* src = X + row * D + 32 * l;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const bf16x8 xv = *reinterpret_cast<const bf16x8*>(src + 8 * k);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[8 * k + e] = (float)xv[e];
        }
        if constexpr (ROT) {
#pragma unroll
            for (int u = 0; u < 32; ++u)
                v[u] = __int_as_float(__float_as_int(v[u]) ^ (int)((neg >> u) << 31));
            // y = x H (Sylvester order): one butterfly stage per bit of the
            // element index, (a, b) -> (a + b, a - b) for the pair whose
            // index differs in that bit.
#pragma unroll
            for (int st = 1; st < 32; st <<= 1)
#pragma unroll
                for (int u = 0; u < 32; ++u)
                    if (!(u & st)) {
                        const float a = v[u], b = v[u + st];
                        v[u] = a + b;
                        v[u + st] = a - b;
                    }
            // lane bits: own + partner where the bit is clear, partner - own
            // where it is set
            const float s1 = (l & 1) ? -1.f : 1.f;
#pragma unroll
            for (int u = 0; u < 32; ++u) v[u] = fmaf(v[u], s1, quad_xor<1>(v[u]));
            if constexpr (LPR == 4) {
                const float s2 = (l & 2) ? -1.f : 1.f;
#pragma unroll
                for (int u = 0; u < 32; ++u) v[u] = fmaf(v[u], s2, quad_xor<2>(v[u]));
            }
            const float norm = D == 64 ? 0.125f : 0.0883883476483184406f;  // 1 / sqrt(D)
#pragma unroll
            for (int u = 0; u < 32; ++u) v[u] *= norm;
        }
        float am = 0.f;
#pragma unroll
        for (int u = 0; u < 32; ++u) am = fmaxf(am, fabsf(v[u]));
        const int ex = block_exponent(am);
        u32x4 c[2];
#pragma unroll
        for (int w = 0; w < 8; ++w)
            c[w >> 2][w & 3] = pack4(ldexpf(v[4 * w], -ex), ldexpf(v[4 * w + 1], -ex),
                                     ldexpf(v[4 * w + 2], -ex), ldexpf(v[4 * w + 3], -ex));
        uint8_t* dst = codes + row * D + 32 * l;
        *reinterpret_cast<u32x4*>(dst) = c[0];
        *reinterpret_cast<u32x4*>(dst + 16) = c[1];
        scales[row * (D / 32) + l] = (uint8_t)(ex + 127);
    }
}

// Columns: a quad of threads owns 8 adjacent columns of one block (32 rows
// of one slice), each thread 8 of its rows (one 16-byte load per row; the
// D / 2 threads of a block read each row whole); the column maxima are
// combined over the quad by two DPP swaps.
template <int D>
__global__ void __launch_bounds__(256)
fp8_quant_cols_kernel(const __bf16* __restrict__ X, uint8_t* __restrict__ codes,
                      uint8_t* __restrict__ scales, long long nblocks, int n)
{
    constexpr int TPB = D / 2, BPW = 256 / TPB;  // threads per block, blocks per workgroup
    const int nb = (n + 31) / 32;
    const int rq = threadIdx.x & 3, c8 = (threadIdx.x % TPB) >> 2;
    for (long long blk = (long long)blockIdx.x * BPW + threadIdx.x / TPB; blk < nblocks;
         blk += (long long)gridDim.x * BPW) {
        const long long sl = blk / nb;
        const int r0 = (int)(blk - sl * nb) * 32;
        const int nr = min(32, n - r0);
        const __bf16* xs = X + ((size_t)sl * n + r0) * D + 8 * c8;
        u32x4 raw[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int r = 8 * rq + k;
            raw[k] = r < nr ? *reinterpret_cast<const u32x4*>(xs + (size_t)r * D) : u32x4{0, 0, 0, 0};
        }
        float am[8] = {};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const bf16x8 xv = __builtin_bit_cast(bf16x8, raw[k]);
#pragma unroll
            for (int e = 0; e < 8; ++e) am[e] = fmaxf(am[e], fabsf((float)xv[e]));
        }
        int ex[8];
        uint32_t sb[2] = {0, 0};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            am[e] = fmaxf(am[e], quad_xor<1>(am[e]));
            am[e] = fmaxf(am[e], quad_xor<2>(am[e]));
            ex[e] = block_exponent(am[e]);
            sb[e >> 2] |= (uint32_t)(ex[e] + 127) << (8 * (e & 3));
        }
        if (rq == 0)
            *reinterpret_cast<uint2*>(scales + ((size_t)sl * nb + r0 / 32) * D + 8 * c8) =
                uint2{sb[0], sb[1]};
        uint8_t* dst = codes + ((size_t)sl * n + r0) * D + 8 * c8;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int r = 8 * rq + k;
            if (r >= nr) break;
            const bf16x8 xv = __builtin_bit_cast(bf16x8, raw[k]);
            float w[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = ldexpf((float)xv[e], -ex[e]);
            *reinterpret_cast<uint2*>(dst + (size_t)r * D) =
                uint2{pack4(w[0], w[1], w[2], w[3]), pack4(w[4], w[5], w[6], w[7])};
        }
    }
}

template <int D>
hipError_t rows_launch(const void* X, void* codes, void* scales, long long rows, bool rot,
                       uint64_t neg_lo, uint64_t neg_hi, hipStream_t stream)
{
    constexpr int RPB = 256 / (D / 32);
    const long long need = (rows + RPB - 1) / RPB;
    const unsigned grid = (unsigned)(need < 65536 ? need : 65536);
    const auto* x = static_cast<const __bf16*>(X);
    auto* c = static_cast<uint8_t*>(codes);
    auto* s = static_cast<uint8_t*>(scales);
    if (rot)
        fp8_quant_rows_kernel<D, true><<<grid, 256, 0, stream>>>(x, c, s, rows, neg_lo, neg_hi);
    else
        fp8_quant_rows_kernel<D, false><<<grid, 256, 0, stream>>>(x, c, s, rows, 0, 0);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8_quant_rows(const void* X, void* codes, void* scales, long long rows, int d,
                                 bool rot, uint64_t neg_lo, uint64_t neg_hi, hipStream_t stream)
{
    return d == 64 ? rows_launch<64>(X, codes, scales, rows, rot, neg_lo, neg_hi, stream)
                   : rows_launch<128>(X, codes, scales, rows, rot, neg_lo, neg_hi, stream);
}

hipError_t launch_fp8_quant_cols(const void* X, void* codes, void* scales, long long slices,
                                 int n, int d, hipStream_t stream)
{
    const long long nblocks = slices * ((n + 31) / 32);
    const long long need = (nblocks + 256 / (d / 2) - 1) / (256 / (d / 2));
    const unsigned grid = (unsigned)(need < 65536 ? need : 65536);
    const auto* x = static_cast<const __bf16*>(X);
    auto* c = static_cast<uint8_t*>(codes);
    auto* s = static_cast<uint8_t*>(scales);
    if (d == 64)
        fp8_quant_cols_kernel<64><<<grid, 256, 0, stream>>>(x, c, s, nblocks, n);
    else
        fp8_quant_cols_kernel<128><<<grid, 256, 0, stream>>>(x, c, s, nblocks, n);
    return hipGetLastError();
}

}  // namespace osm
