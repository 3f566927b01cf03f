// attn_fwd_bf16.hip -- fused exact attention forward for bf16 Q, K, V on the
// gfx950 bf16 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation):
// O = softmax(scale Q K^T) V written as bf16, plus the per-row natural-log
// logsumexp in fp32.  The N x N score and probability matrices exist only as
// register tiles and never reach HBM.
//
// Method: the tiled online softmax of "Lesson 22: why softmax is hard to make
// efficient, and how FlashAttention reduces memory traffic", sections 21-24
// and 32 (the update rule of section 22, the causal tile skipping of section
// 34), with the refinements of "Moving less: four generations of
// FlashAttention", chapter 3: the output stays unnormalised until the end
// (3.2), the grid runs over query-row blocks (3.3), and query rows are split
// across waves so waves never exchange partial outputs (3.4).  lse = m + ln l
// is the statistic of section 2.4 of the same page.
//
// gfx950 design:
//  * Work: one workgroup per (batch*head, block of BR query rows); a wave owns
//    QT x 32 query rows.  Under the causal mask workgroups are issued longest
//    first.  Consecutive workgroup ids walk the batch*head index, so when
//    batch*head is a multiple of 8 every query block of one head lands on the
//    same XCD (ids are dealt round-robin over the 8 XCDs) and shares its L2.
//  * Q stays in VGPRs as the B operand of S^T = K Q^T for the whole kernel.
//  * K and V tiles of 64 keys are staged through LDS, double-buffered: the
//    global loads of tile j+1 are issued before tile j is computed and written
//    to the other LDS buffer after it, with one barrier per tile.  K rows are
//    stored with an XOR swizzle of their 16-byte chunks; V is stored
//    transposed (V^T, keys contiguous) with its own swizzle, so both MFMA A
//    operands are single 16-byte LDS reads.
//  * S^T puts one query per lane (lane % 32) and 16 keys per lane in each
//    32x32 accumulator, so the row max and row sum are in-lane reductions plus
//    one v_permlane32_swap; the row sum is kept per lane and the two halves
//    are added once at the end.  The K rows are permuted inside each 32-row
//    MFMA tile so that every accumulator register group of 8 holds 8
//    consecutive keys: the bf16 probabilities then are, register for
//    register, the B operand of O^T += V^T P^T -- no shuffles.
//  * p = 2^(s c - m c) with c = scale log2(e): one FMA and one v_exp_f32.
//    The accumulator rescale by exp(m_old - m_new) is skipped when no row of
//    the wave changed its maximum (the factor is then exactly 1).

#include "device_common.h"
#include "kernels.h"

namespace osm {
namespace {

constexpr int BC = 64;  // keys per tile

typedef __attribute__((ext_vector_type(8))) float f32x8;

// Key row (inside a 32-row MFMA tile) that A-operand row i reads, chosen so
// that accumulator register r of lane half h ends up holding key
// 16*(r/8) + 8*h + r%8.  With i = 8g + 4h + t the 32x32 accumulator layout
// places row i in register 4g + t of half h.
__device__ __forceinline__ int key_of_row(int i)
{
    return 16 * (i >> 4) + 8 * ((i >> 2) & 1) + 4 * ((i >> 3) & 1) + (i & 3);
}
// Swizzle (XOR on 16-byte chunks) of K row r: the 8 lanes that read one
// column of chunks together see 8 different chunk positions.
__device__ __forceinline__ int kswz(int r) { return (r & 3) | (((r >> 3) & 1) << 2); }
// Swizzle of V^T row d (chunks of 8 keys): consecutive rows, and rows 8 apart,
// fall on different chunk positions.
__device__ __forceinline__ int vswz(int d) { return (d + (d >> 3)) & 7; }

template <int D, int QT, int NW>
struct Cfg {
    static constexpr int T = NW * 64;           // threads per workgroup
    static constexpr int BR = NW * QT * 32;     // query rows per workgroup
    static constexpr int KCH = D / 8;           // 16-byte chunks per K row
    static constexpr int KPT = BC * KCH / T;    // K chunks staged per thread
    static constexpr int NVB = (BC / 4) * KCH;  // V blocks of 4 keys x 8 columns
    static constexpr int VPT = (NVB + T - 1) / T;
    static constexpr int TILE = BC * D;         // elements of one K (or V) tile
    static_assert(BC * KCH % T == 0, "K staging must divide evenly");
};

template <int D, int QT, int NW, bool CAUSAL>
__global__ void __launch_bounds__(NW * 64)
attn_fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                     const __bf16* __restrict__ V, __bf16* __restrict__ O,
                     float* __restrict__ lse, int N, int BH, int nqt, float scale)
{
    using C = Cfg<D, QT, NW>;
    __shared__ __attribute__((aligned(16))) __bf16 Ks[2][C::TILE];
    __shared__ __attribute__((aligned(16))) __bf16 Vt[2][C::TILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int j = lane & 31, h = lane >> 5;
    const int t = blockIdx.x / BH, bh = blockIdx.x - t * BH;
    const int qt = CAUSAL ? nqt - 1 - t : t;
    const int q0 = qt * C::BR;
    const size_t base = (size_t)bh * N * D;
    const __bf16* Qb = Q + base;
    const __bf16* Kb = K + base;
    const __bf16* Vb = V + base;
    const int qw0 = q0 + wave * QT * 32;  // first query row of this wave

    // Q as the B operand of S^T = K Q^T: lane (j, h), k-step kk holds
    // Q[row][16 kk + 8 h .. +7] of row qw0 + 32 nt + j.
    bf16x8 qf[QT][D / 16];
#pragma unroll
    for (int nt = 0; nt < QT; ++nt) {
        const int q = qw0 + nt * 32 + j;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            qf[nt][kk] = q < N ? *reinterpret_cast<const bf16x8*>(Qb + (size_t)q * D + kk * 16 + 8 * h)
                               : bf16x8{};
    }

    f32x16 acc[QT][D / 32];
#pragma unroll
    for (int nt = 0; nt < QT; ++nt)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) acc[nt][dt] = f32x16{};
    float m[QT], l[QT];
#pragma unroll
    for (int nt = 0; nt < QT; ++nt) {
        m[nt] = kNegInf;
        l[nt] = 0.f;
    }
    const float c = scale * kLog2e;

    // ---- staging of one K/V tile: global -> registers -> LDS ----
    u32x4 kreg[C::KPT];
    u32x4 vreg[C::VPT][4];
    auto gload = [&](int kt) {
        const int kv0 = kt * BC;
#pragma unroll
        for (int i = 0; i < C::KPT; ++i) {
            const int cidx = tid + i * C::T, row = cidx / C::KCH, ch = cidx % C::KCH;
            const int key = kv0 + row;
            kreg[i] = key < N ? *reinterpret_cast<const u32x4*>(Kb + (size_t)key * D + ch * 8)
                              : u32x4{};
        }
#pragma unroll
        for (int b = 0; b < C::VPT; ++b) {
            const int blk = tid + b * C::T;
            if (blk < C::NVB) {
                const int kg = blk / C::KCH, dc = blk % C::KCH;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int key = kv0 + 4 * kg + e;
                    vreg[b][e] = key < N ? *reinterpret_cast<const u32x4*>(Vb + (size_t)key * D + dc * 8)
                                         : u32x4{};
                }
            }
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < C::KPT; ++i) {
            const int cidx = tid + i * C::T, row = cidx / C::KCH, ch = cidx % C::KCH;
            *reinterpret_cast<u32x4*>(&Ks[buf][row * D + ((ch ^ kswz(row)) * 8)]) = kreg[i];
        }
#pragma unroll
        for (int b = 0; b < C::VPT; ++b) {
            const int blk = tid + b * C::T;
            if (blk < C::NVB) {
                const int kg = blk / C::KCH, dc = blk % C::KCH;
                // vreg[b][e] holds columns 8 dc .. 8 dc + 7 of key 4 kg + e; dword w
                // packs columns 2w (low half) and 2w + 1 (high half).  Gather the
                // four keys of one column into 8 bytes of the V^T row.
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t lo01 = __builtin_amdgcn_perm(vreg[b][1][w], vreg[b][0][w], 0x05040100u);
                    const uint32_t lo23 = __builtin_amdgcn_perm(vreg[b][3][w], vreg[b][2][w], 0x05040100u);
                    const uint32_t hi01 = __builtin_amdgcn_perm(vreg[b][1][w], vreg[b][0][w], 0x07060302u);
                    const uint32_t hi23 = __builtin_amdgcn_perm(vreg[b][3][w], vreg[b][2][w], 0x07060302u);
                    const int d0 = dc * 8 + 2 * w, d1 = d0 + 1;
                    *reinterpret_cast<u32x2*>(&Vt[buf][d0 * BC + (((kg >> 1) ^ vswz(d0)) * 8) + (kg & 1) * 4]) =
                        u32x2{lo01, lo23};
                    *reinterpret_cast<u32x2*>(&Vt[buf][d1 * BC + (((kg >> 1) ^ vswz(d1)) * 8) + (kg & 1) * 4]) =
                        u32x2{hi01, hi23};
                }
            }
        }
    };

    const int kv_end = CAUSAL ? min(N, q0 + C::BR) : N;
    const int ntiles = (kv_end + BC - 1) / BC;

    gload(0);
    lstore(0);
    __syncthreads();

    for (int kt = 0; kt < ntiles; ++kt) {
        const int buf = kt & 1;
        const int kv0 = kt * BC;
        const bool more = kt + 1 < ntiles;
        if (more) gload(kt + 1);

        // A wave whose rows all precede the tile's first key sees nothing in it.
        const bool active = !CAUSAL || kv0 <= qw0 + QT * 32 - 1;
        if (active) {
            // ---- S^T = K Q^T for two 32-key MFMA tiles ----
            f32x16 s[2][QT];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < QT; ++nt) s[mt][nt] = f32x16{};
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    const int row = mt * 32 + key_of_row(j);
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                        &Ks[buf][row * D + (((2 * kk + h) ^ kswz(row)) * 8)]);
#pragma unroll
                    for (int nt = 0; nt < QT; ++nt)
                        s[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[nt][kk], s[mt][nt], 0, 0, 0);
                }
            }

            // ---- mask, online softmax statistics, probabilities ----
            const bool need_mask = (kv0 + BC > N) || (CAUSAL && kv0 + BC - 1 > qw0);
            float alpha[QT];
#pragma unroll
            for (int nt = 0; nt < QT; ++nt) {
                const int q = qw0 + nt * 32 + j;
                if (need_mask) {
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = kv0 + mt * 32 + 16 * (r >> 3) + 8 * h + (r & 7);
                            if (key >= N || (CAUSAL && key > q)) s[mt][nt][r] = kNegInf;
                        }
                }
                float mx = kNegInf;
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][nt][r]);
                mx = combine_xor32(mx, MaxOp());
                const float m_new = fmaxf(m[nt], mx);
                // Tile 0 holds key 0, visible to every row, so m_new is finite from
                // the first tile on; the guards only keep -inf - -inf out of exp2.
                // alpha is exactly 1 when the maximum did not move and 0 for an
                // empty history (m = -inf).
                const float mc = (m_new == kNegInf) ? 0.f : m_new * c;
                alpha[nt] = (m_new == kNegInf) ? 1.f : exp2_hw((m[nt] - m_new) * c);
                float psum = 0.f;
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float p = exp2_hw(fmaf(s[mt][nt][r], c, -mc));
                        s[mt][nt][r] = p;
                        psum += p;
                    }
                l[nt] = alpha[nt] * l[nt] + psum;
                m[nt] = m_new;
            }
            bool rescale = false;
#pragma unroll
            for (int nt = 0; nt < QT; ++nt) rescale |= alpha[nt] != 1.0f;
            if (__builtin_amdgcn_ballot_w64(rescale) != 0) {
#pragma unroll
                for (int nt = 0; nt < QT; ++nt)
#pragma unroll
                    for (int dt = 0; dt < D / 32; ++dt) acc[nt][dt] *= alpha[nt];
            }

            // ---- O^T += V^T P^T over four 16-key steps ----
#pragma unroll
            for (int ks = 0; ks < BC / 16; ++ks) {
                bf16x8 pf[QT];
#pragma unroll
                for (int nt = 0; nt < QT; ++nt) {
                    const f32x16& sv = s[ks >> 1][nt];
                    const f32x8 p8 = (ks & 1) ? __builtin_shufflevector(sv, sv, 8, 9, 10, 11, 12, 13, 14, 15)
                                              : __builtin_shufflevector(sv, sv, 0, 1, 2, 3, 4, 5, 6, 7);
                    pf[nt] = __builtin_convertvector(p8, bf16x8);
                }
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) {
                    const int d = dt * 32 + j;
                    const bf16x8 va = *reinterpret_cast<const bf16x8*>(
                        &Vt[buf][d * BC + (((2 * ks + h) ^ vswz(d)) * 8)]);
#pragma unroll
                    for (int nt = 0; nt < QT; ++nt)
                        acc[nt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[nt], acc[nt][dt], 0, 0, 0);
                }
            }
        }

        if (more) lstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = acc / l in bf16, lse = m scale + ln l ----
#pragma unroll
    for (int nt = 0; nt < QT; ++nt) {
        const int q = qw0 + nt * 32 + j;
        const float l_tot = combine_xor32(l[nt], SumOp());
        if (q < N) {
            const float inv = 1.0f / l_tot;
            __bf16* orow = O + base + (size_t)q * D;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 o4 = {acc[nt][dt][4 * g] * inv, acc[nt][dt][4 * g + 1] * inv,
                                      acc[nt][dt][4 * g + 2] * inv, acc[nt][dt][4 * g + 3] * inv};
                    *reinterpret_cast<bf16x4*>(orow + dt * 32 + 8 * g + 4 * h) =
                        __builtin_convertvector(o4, bf16x4);
                }
            if (h == 0) lse[(size_t)bh * N + q] = m[nt] * scale + logf(l_tot);
        }
    }
}

template <int D, int QT, int NW, bool CAUSAL>
hipError_t launch(const void* Q, const void* K, const void* V, void* O, float* lse, int BH,
                  int N, float scale, hipStream_t stream)
{
    using C = Cfg<D, QT, NW>;
    const int nqt = (N + C::BR - 1) / C::BR;
    const dim3 grid((unsigned)(nqt * BH)), block(C::T);
    attn_fwd_bf16_kernel<D, QT, NW, CAUSAL><<<grid, block, 0, stream>>>(
        static_cast<const __bf16*>(Q), static_cast<const __bf16*>(K), static_cast<const __bf16*>(V),
        static_cast<__bf16*>(O), lse, N, BH, nqt, scale);
    return hipGetLastError();
}

// d = 64: 4 waves x 64 query rows (one wave per SIMD, Q and the output
// accumulators of 64 rows fit the registers).  d = 128: 8 waves x 32 rows
// (two waves per SIMD) -- 64 rows per wave would exceed the register file.
template <int D, bool CAUSAL>
hipError_t dispatch(const void* Q, const void* K, const void* V, void* O, float* lse, int BH,
                    int N, float scale, hipStream_t stream)
{
    if (D == 64) return launch<D, 2, 4, CAUSAL>(Q, K, V, O, lse, BH, N, scale, stream);
    return launch<D, 1, 8, CAUSAL>(Q, K, V, O, lse, BH, N, scale, stream);
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const void* Q, const void* K, const void* V, void* O,
                                float* lse, int BH, int N, int d, float scale, bool causal,
                                hipStream_t stream)
{
    if (d == 64)
        return causal ? dispatch<64, true>(Q, K, V, O, lse, BH, N, scale, stream)
                      : dispatch<64, false>(Q, K, V, O, lse, BH, N, scale, stream);
    return causal ? dispatch<128, true>(Q, K, V, O, lse, BH, N, scale, stream)
                  : dispatch<128, false>(Q, K, V, O, lse, BH, N, scale, stream);
}

}  // namespace osm
