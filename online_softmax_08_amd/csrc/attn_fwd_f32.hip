// attn_fwd_f32.hip -- exact attention forward in fp32 on the fp32 matrix
// cores (v_mfma_f32_32x32x2_f32): O = softmax(scale Q K^T) V and the per-row
// natural-log logsumexp, for inputs whose outputs must stay within fp32
// rounding of the exact result.
//
// The algorithm is the tiled online softmax of "Lesson 22: why softmax is hard
// to make efficient, and how FlashAttention reduces memory traffic", sections
// 21-24 and 32: a block of query rows stays on chip while key/value tiles
// stream past; each row keeps a running maximum m, denominator l and an
// unnormalised output a, rescaled by exp(m_old - m_new) whenever the maximum
// grows, and divided by l once at the end ("Moving less: four generations of
// FlashAttention", section 3.2).  Causal masking sets keys j > i to -inf and
// never visits tiles that lie wholly above the diagonal (Lesson 22, section 34).
//
// Mapping: one workgroup = 4 waves x 32 query rows; keys in tiles of 32.
// S^T = K Q^T is formed so that each lane owns one query row (lane % 32) and
// 16 of the tile's keys, which makes the row max/sum one in-lane pass plus one
// exchange with lane ^ 32.  The probabilities then feed O^T += V^T P^T
// straight from the accumulator registers.  Tiles are single-buffered in LDS
// with two barriers per tile; the next tile's K and V rows are fetched into
// registers (16-byte loads) while the current one is computed, so global
// latency overlaps the products.

#include "device_common.h"
#include "kernels.h"

namespace osm {
namespace {

constexpr int F32_BR = 128;  // query rows per workgroup
constexpr int F32_BC = 32;   // keys per tile

// Key (within a 32-row MFMA tile) held by accumulator register r of a lane in
// half h: the 32x32 accumulator layout puts row 8*(r/4) + 4*h + r%4 there.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256)
attn_fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                    const float* __restrict__ V, float* __restrict__ O,
                    float* __restrict__ lse, int N, int BH, int nqt, float scale)
{
    constexpr int BC = F32_BC, KP = D + 1;
    __shared__ float Ks[BC * KP];
    __shared__ __attribute__((aligned(16))) float Vs[BC * D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 31, h = lane >> 5;
    const int t = blockIdx.x / BH, bh = blockIdx.x - t * BH;
    const int qt = CAUSAL ? nqt - 1 - t : t;  // causal: longest rows first
    const int q0 = qt * F32_BR;
    const size_t base = (size_t)bh * N * D;
    const int qw0 = q0 + wave * 32;
    const int q = qw0 + j;

    // B operand of S^T = K Q^T for k-step kk: lane (j, h) holds Q[q][2 kk + h].
    float qv[D / 2];
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) qv[kk] = q < N ? Q[base + (size_t)q * D + 2 * kk + h] : 0.f;

    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
    float m = kNegInf, l = 0.f;
    const float c = scale * kLog2e;

    const int kv_end = CAUSAL ? min(N, q0 + F32_BR) : N;
    const int ntiles = (kv_end + BC - 1) / BC;
    // Thread tid fetches 4-float pieces tid + 256 u (u < NF) of the tile's
    // K and V rows: piece p is row 4 p / D, columns 4 p % D .. + 3 (zero
    // for rows past N).
    constexpr int NF = BC * D / 4 / 256;
    static_assert(NF * 256 * 4 == BC * D, "whole pieces per thread");
    f32x4 kreg[NF], vreg[NF];
    auto fetch = [&](int kt) {
#pragma unroll
        for (int u = 0; u < NF; ++u) {
            const int e = 4 * (tid + 256 * u), r = e / D, col = e - r * D, key = kt * BC + r;
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            kreg[u] = key < N ? *reinterpret_cast<const f32x4*>(K + base + (size_t)key * D + col) : z;
            vreg[u] = key < N ? *reinterpret_cast<const f32x4*>(V + base + (size_t)key * D + col) : z;
        }
    };
    if (ntiles > 0) fetch(0);
    for (int kt = 0; kt < ntiles; ++kt) {
        const int kv0 = kt * BC;
        __syncthreads();  // the previous tile is no longer read
#pragma unroll
        for (int u = 0; u < NF; ++u) {
            const int e = 4 * (tid + 256 * u), r = e / D, col = e - r * D;
#pragma unroll
            for (int x = 0; x < 4; ++x) Ks[r * KP + col + x] = kreg[u][x];  // odd pitch: 4-byte stores
            *reinterpret_cast<f32x4*>(&Vs[r * D + col]) = vreg[u];
        }
        __syncthreads();
        if (kt + 1 < ntiles) fetch(kt + 1);      // lands while this tile is computed
        if (CAUSAL && kv0 > qw0 + 31) continue;  // every key of the tile is in this wave's future

        f32x16 s = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 2; ++kk)
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[j * KP + 2 * kk + h], qv[kk], s, 0, 0, 0);

        float mx = kNegInf;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = kv0 + acc_row(r, h);
            if (key >= N || (CAUSAL && key > q)) s[r] = kNegInf;
            mx = fmaxf(mx, s[r]);
        }
        mx = combine_xor32(mx, MaxOp());
        const float m_new = fmaxf(m, mx);
        // Correction of the history; an empty history (m = -inf) contributes 0.
        const float alpha = (m == kNegInf) ? 0.f : exp2_hw((m - m_new) * c);
        const float m_ref = (m_new == kNegInf) ? 0.f : m_new;
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s[r] = exp2_hw((s[r] - m_ref) * c);
            psum += s[r];
        }
        l = alpha * l + psum;  // this lane's share; the halves are added at the end
        m = m_new;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) acc[dt] *= alpha;
        // O^T += V^T P^T, one key per k-step: B = P[q][key], A = V[key][d].
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = acc_row(r, h);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * D + dt * 32 + j], s[r],
                                                               acc[dt], 0, 0, 0);
        }
    }

    const float l_tot = combine_xor32(l, SumOp());
    if (q < N) {
        const float inv = 1.0f / l_tot;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                O[base + (size_t)q * D + dt * 32 + acc_row(r, h)] = acc[dt][r] * inv;
        if (h == 0) lse[(size_t)bh * N + q] = m * scale + logf(l_tot);
    }
}

template <int D, bool CAUSAL>
hipError_t launch(const float* Q, const float* K, const float* V, float* O, float* lse, int BH,
                  int N, float scale, hipStream_t stream)
{
    const int nqt = (N + F32_BR - 1) / F32_BR;
    const dim3 grid((unsigned)(nqt * BH)), block(256);
    attn_fwd_f32_kernel<D, CAUSAL><<<grid, block, 0, stream>>>(Q, K, V, O, lse, N, BH, nqt, scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_f32(const float* Q, const float* K, const float* V, float* O,
                               float* lse, int BH, int N, int d, float scale, bool causal,
                               hipStream_t stream)
{
    if (d == 64)
        return causal ? launch<64, true>(Q, K, V, O, lse, BH, N, scale, stream)
                      : launch<64, false>(Q, K, V, O, lse, BH, N, scale, stream);
    return causal ? launch<128, true>(Q, K, V, O, lse, BH, N, scale, stream)
                  : launch<128, false>(Q, K, V, O, lse, BH, N, scale, stream);
}

}  // namespace osm
