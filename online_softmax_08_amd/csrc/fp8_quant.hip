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
// Both kernels are HBM bound: 2 bytes read and 1 + 1/32 written per element.
//  * fp8_quant_rows_kernel: d / 8 lanes per row, 8 elements per lane (one
//    16-byte load).  The rotation: sign flips, the fast Walsh-Hadamard
//    transform in fp32 (three butterfly stages inside the lane, log2(d / 8)
//    across lanes by lane swaps), then 1 / sqrt(d).  A block is 4 lanes; its
//    maximum takes two lane swaps.
//  * fp8_quant_cols_kernel: one workgroup per block row (32 rows x d) of a
//    slice, coalesced row loads, the column maxima through LDS.
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

template <int D, bool ROT>
__global__ void __launch_bounds__(256)
fp8_quant_rows_kernel(const __bf16* __restrict__ X, uint8_t* __restrict__ codes,
                      uint8_t* __restrict__ scales, long long rows, uint64_t neg_lo,
                      uint64_t neg_hi)
{
    constexpr int LPR = D / 8, RPB = 256 / LPR;
    const int l = threadIdx.x % LPR;  // this lane holds elements 8 l .. 8 l + 7 of its row
    for (long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR; row < rows;
         row += (long long)gridDim.x * RPB) {
        const bf16x8 xv = *reinterpret_cast<const bf16x8*>(X + row * D + 8 * l);
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (float)xv[e];
        if constexpr (ROT) {
            // x diag(s): bit t of (neg_hi:neg_lo) set means s_t = -1.
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int t = 8 * l + e;
                const uint64_t bit = t < 64 ? (neg_lo >> t) & 1u : (neg_hi >> (t - 64)) & 1u;
                if (bit) v[e] = -v[e];
            }
            // y = x H (Sylvester order, y_k = sum_t x_t (-1)^popcount(t & k)):
            // one butterfly stage per bit of the element index, (a, b) ->
            // (a + b, a - b) for the pair whose index differs in that bit.
#pragma unroll
            for (int st = 1; st < 8; st <<= 1)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (!(e & st)) {
                        const float a = v[e], b = v[e + st];
                        v[e] = a + b;
                        v[e + st] = a - b;
                    }
#pragma unroll
            for (int m = 1; m < LPR; m <<= 1)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float p = __shfl_xor(v[e], m);
                    v[e] = (l & m) ? p - v[e] : v[e] + p;
                }
            const float norm = D == 64 ? 0.125f : 0.0883883476483184406f;  // 1 / sqrt(D)
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] *= norm;
        }
        float am = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(v[e]));
        am = fmaxf(am, __shfl_xor(am, 1));
        am = fmaxf(am, __shfl_xor(am, 2));
        const int ex = block_exponent(am);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = ldexpf(v[e], -ex);
        const uint2 c8 = {pack4(v[0], v[1], v[2], v[3]), pack4(v[4], v[5], v[6], v[7])};
        *reinterpret_cast<uint2*>(codes + row * D + 8 * l) = c8;
        if ((l & 3) == 0) scales[row * (D / 32) + l / 4] = (uint8_t)(ex + 127);
    }
}

template <int D>
__global__ void __launch_bounds__(256)
fp8_quant_cols_kernel(const __bf16* __restrict__ X, uint8_t* __restrict__ codes,
                      uint8_t* __restrict__ scales, long long nblocks, int n)
{
    constexpr int LPR = D / 8, RPT = 256 / LPR, TRIPS = 32 / RPT;
    __shared__ float mag[32][D];
    __shared__ int ecol[D];
    const int nb = (n + 31) / 32;
    const int c8 = threadIdx.x % LPR;
    for (long long blk = blockIdx.x; blk < nblocks; blk += gridDim.x) {
        const long long sl = blk / nb;
        const int r0 = (int)(blk - sl * nb) * 32;
        const __bf16* xs = X + (size_t)sl * n * D;
        float v[TRIPS][8];
#pragma unroll
        for (int it = 0; it < TRIPS; ++it) {
            const int r = it * RPT + threadIdx.x / LPR;
            bf16x8 xv = {};
            if (r0 + r < n) xv = *reinterpret_cast<const bf16x8*>(xs + (size_t)(r0 + r) * D + 8 * c8);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                v[it][e] = (float)xv[e];
                mag[r][8 * c8 + e] = fabsf(v[it][e]);
            }
        }
        __syncthreads();
        if (threadIdx.x < D) {
            float am = 0.f;
#pragma unroll 8
            for (int r = 0; r < 32; ++r) am = fmaxf(am, mag[r][threadIdx.x]);
            const int ex = block_exponent(am);
            ecol[threadIdx.x] = ex;
            scales[((size_t)sl * nb + r0 / 32) * D + threadIdx.x] = (uint8_t)(ex + 127);
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < TRIPS; ++it) {
            const int r = it * RPT + threadIdx.x / LPR;
            if (r0 + r >= n) continue;
            float w[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = ldexpf(v[it][e], -ecol[8 * c8 + e]);
            const uint2 c = {pack4(w[0], w[1], w[2], w[3]), pack4(w[4], w[5], w[6], w[7])};
            *reinterpret_cast<uint2*>(codes + ((size_t)sl * n + r0 + r) * D + 8 * c8) = c;
        }
        __syncthreads();  // mag and ecol are rewritten by the next block
    }
}

template <int D>
hipError_t rows_launch(const void* X, void* codes, void* scales, long long rows, bool rot,
                       uint64_t neg_lo, uint64_t neg_hi, hipStream_t stream)
{
    constexpr int RPB = 256 / (D / 8);
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
    const unsigned grid = (unsigned)(nblocks < 65536 ? nblocks : 65536);
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
