// row_softmax.hip -- numerically stable softmax of every row of x [B, N]
// (fp32), y[b, j] = exp(x[b, j] - m_b) / sum_t exp(x[b, t] - m_b) with
// m_b = max_t x[b, t].
//
// Follows "Lesson 22: why softmax is hard to make efficient, and how
// FlashAttention reduces memory traffic", sections 2-11: the row maximum is
// subtracted so every exponent is <= 0 (section 2); rows are independent and
// map to one wave or one workgroup depending on N (section 5); a row that fits
// the registers is read from HBM exactly once (section 11), so the traffic is
// the 4N bytes read plus 4N written of section 4.
//
// Three kernels:
//   * wave-per-row    N <= 1024: one 64-lane wave per row, four rows per
//                     workgroup, all reductions inside the wave (DPP + permlane);
//   * block-per-row   1024 < N <= 32768: one workgroup per row held in
//                     registers, reductions wave-then-LDS;
//   * online, 2 reads N > 32768: one workgroup per row, a first streaming
//                     pass keeps a running (max, sum) per lane and merges them
//                     with the two-block rule of sections 18-19; a second
//                     pass rescales.
// Each has a float4 variant (N % 4 == 0 and 16-byte aligned rows) and a
// scalar one.  x and y may be the same buffer: every lane reads all of its
// elements before writing any of them, and only its own.

#include "device_common.h"
#include "kernels.h"

namespace osm {
namespace {

// Rows are read once and written once, so both sides are streamed with
// nontemporal accesses (no cache allocation for data that is not reused);
// on the [32768, 8192] workload this moves the kernel from 5.4 to 5.85 TB/s.
__device__ __forceinline__ float4 ld4(const float* p)
{
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st4(float* p, float4 v)
{
    const f32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<f32x4*>(p));
}

__device__ __forceinline__ float max4(float4 v) { return fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)); }

// e = exp(x - m) evaluated as 2^((x - m) log2 e); x - m is formed first so a
// large common offset (rows like 1000 - j) cancels exactly before scaling.
__device__ __forceinline__ float expm(float x, float m) { return exp2_hw((x - m) * kLog2e); }

// Block-wide reduction: wave butterfly, then one LDS slot per wave.
template <int NW, class Op>
__device__ __forceinline__ float block_reduce(float v, Op op, float* slots)
{
    v = wave_reduce(v, op);
    if (NW == 1) return v;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) slots[wave] = v;
    __syncthreads();
    float r = slots[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = op(r, slots[w]);
    return r;
}

// ---------------------------------------------------------------- wave/row --
// E4 float4 chunks per lane: chunk c = lane + 64 i covers x[4c .. 4c+3].
template <int E4>
__global__ void __launch_bounds__(256)
softmax_wave_vec4(const float* x, float* y, int B, int N)
{
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= B) return;
    const int lane = threadIdx.x & 63;
    const int n4 = N >> 2;
    const float* xr = x + (size_t)row * N;
    float* yr = y + (size_t)row * N;
    float4 v[E4];
    float m = kNegInf;
#pragma unroll
    for (int i = 0; i < E4; ++i) {
        const int c = lane + 64 * i;
        if (c < n4) {
            v[i] = ld4(xr + 4 * c);
            m = fmaxf(m, max4(v[i]));
        }
    }
    m = wave_reduce(m, MaxOp());
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < E4; ++i) {
        const int c = lane + 64 * i;
        if (c < n4) {
            v[i].x = expm(v[i].x, m);
            v[i].y = expm(v[i].y, m);
            v[i].z = expm(v[i].z, m);
            v[i].w = expm(v[i].w, m);
            s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
        }
    }
    s = wave_reduce(s, SumOp());
    const float inv = 1.0f / s;
#pragma unroll
    for (int i = 0; i < E4; ++i) {
        const int c = lane + 64 * i;
        if (c < n4)
            st4(yr + 4 * c, make_float4(v[i].x * inv, v[i].y * inv, v[i].z * inv, v[i].w * inv));
    }
}

// E scalars per lane: element j = lane + 64 i.
template <int E>
__global__ void __launch_bounds__(256)
softmax_wave_scalar(const float* x, float* y, int B, int N)
{
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= B) return;
    const int lane = threadIdx.x & 63;
    const float* xr = x + (size_t)row * N;
    float* yr = y + (size_t)row * N;
    float v[E];
    float m = kNegInf;
#pragma unroll
    for (int i = 0; i < E; ++i) {
        const int j = lane + 64 * i;
        v[i] = j < N ? xr[j] : kNegInf;
        m = fmaxf(m, v[i]);
    }
    m = wave_reduce(m, MaxOp());
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) {
        v[i] = expm(v[i], m);  // padding lanes: exp2(-inf) = 0
        s += v[i];
    }
    s = wave_reduce(s, SumOp());
    const float inv = 1.0f / s;
#pragma unroll
    for (int i = 0; i < E; ++i) {
        const int j = lane + 64 * i;
        if (j < N) yr[j] = v[i] * inv;
    }
}

// --------------------------------------------------------------- block/row --
// T threads, E4 float4 chunks per thread: chunk c = tid + T i.
template <int T, int E4>
__global__ void __launch_bounds__(T)
softmax_block_vec4(const float* x, float* y, int N)
{
    constexpr int NW = T / 64;
    __shared__ float red_max[NW], red_sum[NW];
    const int tid = threadIdx.x;
    const int n4 = N >> 2;
    const float* xr = x + (size_t)blockIdx.x * N;
    float* yr = y + (size_t)blockIdx.x * N;
    float4 v[E4];
#pragma unroll
    for (int i = 0; i < E4; ++i) {
        const int c = tid + T * i;
        v[i] = c < n4 ? ld4(xr + 4 * c) : make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
    }
    float m = kNegInf;
#pragma unroll
    for (int i = 0; i < E4; ++i) m = fmaxf(m, max4(v[i]));
    m = block_reduce<NW>(m, MaxOp(), red_max);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < E4; ++i) {
        v[i].x = expm(v[i].x, m);
        v[i].y = expm(v[i].y, m);
        v[i].z = expm(v[i].z, m);
        v[i].w = expm(v[i].w, m);
        s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    }
    s = block_reduce<NW>(s, SumOp(), red_sum);
    const float inv = 1.0f / s;
#pragma unroll
    for (int i = 0; i < E4; ++i) {
        const int c = tid + T * i;
        if (c < n4)
            st4(yr + 4 * c, make_float4(v[i].x * inv, v[i].y * inv, v[i].z * inv, v[i].w * inv));
    }
}

template <int T, int E>
__global__ void __launch_bounds__(T)
softmax_block_scalar(const float* x, float* y, int N)
{
    constexpr int NW = T / 64;
    __shared__ float red_max[NW], red_sum[NW];
    const int tid = threadIdx.x;
    const float* xr = x + (size_t)blockIdx.x * N;
    float* yr = y + (size_t)blockIdx.x * N;
    float v[E];
    float m = kNegInf;
#pragma unroll
    for (int i = 0; i < E; ++i) {
        const int j = tid + T * i;
        v[i] = j < N ? xr[j] : kNegInf;
        m = fmaxf(m, v[i]);
    }
    m = block_reduce<NW>(m, MaxOp(), red_max);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) {
        v[i] = expm(v[i], m);
        s += v[i];
    }
    s = block_reduce<NW>(s, SumOp(), red_sum);
    const float inv = 1.0f / s;
#pragma unroll
    for (int i = 0; i < E; ++i) {
        const int j = tid + T * i;
        if (j < N) yr[j] = v[i] * inv;
    }
}

// ------------------------------------------------------------ online/row --
// (m, l) pairs merge by the two-block rule: m = max(mA, mB),
// l = lA e^(mA - m) + lB e^(mB - m).  An empty side has m = -inf, l = 0.
struct MaxSum {
    float m, l;
};

__device__ __forceinline__ MaxSum merge(MaxSum a, MaxSum b)
{
    const float m = fmaxf(a.m, b.m);
    if (m == kNegInf) return {m, 0.f};
    return {m, a.l * expm(a.m, m) + b.l * expm(b.m, m)};
}

template <int CTRL>
__device__ __forceinline__ MaxSum dpp_pair(MaxSum v)
{
    return {dpp<CTRL>(v.m), dpp<CTRL>(v.l)};
}

__device__ __forceinline__ MaxSum permlane_pair(MaxSum v, bool x32)
{
    if (x32) {
        auto rm = __builtin_amdgcn_permlane32_swap(__float_as_uint(v.m), __float_as_uint(v.m), false, false);
        auto rl = __builtin_amdgcn_permlane32_swap(__float_as_uint(v.l), __float_as_uint(v.l), false, false);
        return merge({__uint_as_float(rm[0]), __uint_as_float(rl[0])},
                     {__uint_as_float(rm[1]), __uint_as_float(rl[1])});
    }
    auto rm = __builtin_amdgcn_permlane16_swap(__float_as_uint(v.m), __float_as_uint(v.m), false, false);
    auto rl = __builtin_amdgcn_permlane16_swap(__float_as_uint(v.l), __float_as_uint(v.l), false, false);
    return merge({__uint_as_float(rm[0]), __uint_as_float(rl[0])},
                 {__uint_as_float(rm[1]), __uint_as_float(rl[1])});
}

__device__ __forceinline__ MaxSum wave_merge(MaxSum v)
{
    v = merge(v, dpp_pair<0xB1>(v));
    v = merge(v, dpp_pair<0x4E>(v));
    v = merge(v, dpp_pair<0x141>(v));
    v = merge(v, dpp_pair<0x140>(v));
    v = permlane_pair(v, false);
    v = permlane_pair(v, true);
    return v;
}

// Running state update for a group of values already in registers.
__device__ __forceinline__ MaxSum absorb(MaxSum st, const float* vals, int n)
{
    float bm = kNegInf;
    for (int k = 0; k < n; ++k) bm = fmaxf(bm, vals[k]);
    const float m = fmaxf(st.m, bm);
    if (m == kNegInf) return st;
    float s = 0.f;
    for (int k = 0; k < n; ++k) s += expm(vals[k], m);
    return {m, st.l * expm(st.m, m) + s};
}

template <int T, bool VEC>
__global__ void __launch_bounds__(T)
softmax_online(const float* x, float* y, int N)
{
    constexpr int NW = T / 64;
    __shared__ float red_m[NW], red_l[NW];
    const int tid = threadIdx.x;
    const float* xr = x + (size_t)blockIdx.x * N;
    float* yr = y + (size_t)blockIdx.x * N;
    MaxSum st = {kNegInf, 0.f};
    if (VEC) {
        const int n4 = N >> 2;
        for (int c = tid; c < n4; c += T) {
            const float4 v = ld4(xr + 4 * c);
            const float vals[4] = {v.x, v.y, v.z, v.w};
            st = absorb(st, vals, 4);
        }
    } else {
        for (int j = tid; j < N; j += T) {
            const float v = xr[j];
            st = absorb(st, &v, 1);
        }
    }
    st = wave_merge(st);
    const int lane = tid & 63, wave = tid >> 6;
    if (lane == 0) {
        red_m[wave] = st.m;
        red_l[wave] = st.l;
    }
    __syncthreads();
    MaxSum tot = {red_m[0], red_l[0]};
    for (int w = 1; w < NW; ++w) tot = merge(tot, {red_m[w], red_l[w]});
    const float inv = 1.0f / tot.l;
    if (VEC) {
        const int n4 = N >> 2;
        for (int c = tid; c < n4; c += T) {
            const float4 v = ld4(xr + 4 * c);
            st4(yr + 4 * c, make_float4(expm(v.x, tot.m) * inv, expm(v.y, tot.m) * inv,
                                        expm(v.z, tot.m) * inv, expm(v.w, tot.m) * inv));
        }
    } else {
        for (int j = tid; j < N; j += T) yr[j] = expm(xr[j], tot.m) * inv;
    }
}

}  // namespace

namespace {

// One dispatch over rows 0 .. B - 1 of x and y.
hipError_t launch_rows(const float* x, float* y, int B, int N, bool vec, hipStream_t stream)
{
    if (N <= kSoftmaxWaveMaxN) {
        const dim3 grid((B + 3) / 4), block(256);
        if (vec) {
            const int e4 = (N / 4 + 63) / 64;  // float4 chunks per lane, <= 4
            if (e4 <= 1) softmax_wave_vec4<1><<<grid, block, 0, stream>>>(x, y, B, N);
            else if (e4 <= 2) softmax_wave_vec4<2><<<grid, block, 0, stream>>>(x, y, B, N);
            else softmax_wave_vec4<4><<<grid, block, 0, stream>>>(x, y, B, N);
        } else {
            const int e = (N + 63) / 64;  // scalars per lane, <= 16
            if (e <= 1) softmax_wave_scalar<1><<<grid, block, 0, stream>>>(x, y, B, N);
            else if (e <= 2) softmax_wave_scalar<2><<<grid, block, 0, stream>>>(x, y, B, N);
            else if (e <= 4) softmax_wave_scalar<4><<<grid, block, 0, stream>>>(x, y, B, N);
            else if (e <= 8) softmax_wave_scalar<8><<<grid, block, 0, stream>>>(x, y, B, N);
            else softmax_wave_scalar<16><<<grid, block, 0, stream>>>(x, y, B, N);
        }
    } else if (N <= kSoftmaxBlockMaxN) {
        const dim3 grid(B);
        if (vec) {
            // Two waves per row with up to 16 float4 per lane measured
            // fastest at N = 8192 (more resident rows per CU, one LDS
            // exchange per reduction).
            if (N <= 2048) softmax_block_vec4<128, 4><<<grid, 128, 0, stream>>>(x, y, N);
            else if (N <= 4096) softmax_block_vec4<128, 8><<<grid, 128, 0, stream>>>(x, y, N);
            else if (N <= 8192) softmax_block_vec4<128, 16><<<grid, 128, 0, stream>>>(x, y, N);
            else if (N <= 16384) softmax_block_vec4<256, 16><<<grid, 256, 0, stream>>>(x, y, N);
            else softmax_block_vec4<512, 16><<<grid, 512, 0, stream>>>(x, y, N);
        } else {
            if (N <= 2048) softmax_block_scalar<256, 8><<<grid, 256, 0, stream>>>(x, y, N);
            else if (N <= 4096) softmax_block_scalar<256, 16><<<grid, 256, 0, stream>>>(x, y, N);
            else if (N <= 8192) softmax_block_scalar<256, 32><<<grid, 256, 0, stream>>>(x, y, N);
            else if (N <= 16384) softmax_block_scalar<1024, 16><<<grid, 1024, 0, stream>>>(x, y, N);
            else softmax_block_scalar<1024, 32><<<grid, 1024, 0, stream>>>(x, y, N);
        }
    } else {
        const dim3 grid(B);
        if (vec) softmax_online<1024, true><<<grid, 1024, 0, stream>>>(x, y, N);
        else softmax_online<1024, false><<<grid, 1024, 0, stream>>>(x, y, N);
    }
    return hipGetLastError();
}

}  // namespace

// Host-side dispatch.  Sizes were validated by the caller (B >= 1, N >= 1).
// A dispatch counts at most 2^32 - 1 work-items and the kernels use up to
// 1024 per row, so rows go out in chunks of 2^21 (2^31 work-items at most).
hipError_t launch_row_softmax(const float* x, float* y, int B, int N, hipStream_t stream)
{
    const bool vec = (N % 4 == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0) &&
                     ((reinterpret_cast<uintptr_t>(y) & 15) == 0);
    constexpr int kChunk = 1 << 21;
    for (int r0 = 0; r0 < B; r0 += kChunk) {
        const int rows = B - r0 < kChunk ? B - r0 : kChunk;
        const hipError_t e = launch_rows(x + (size_t)r0 * N, y + (size_t)r0 * N, rows, N, vec, stream);
        if (e != hipSuccess) return e;
        if (B - r0 <= kChunk) break;
    }
    return hipSuccess;
}

}  // namespace osm
