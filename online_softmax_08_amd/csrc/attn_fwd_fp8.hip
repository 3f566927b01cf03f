// attn_fwd_fp8.hip -- the attention forward pass with fp8 (OCP E4M3) inputs on
// gfx950, the FP8 variant of "Moving less: four generations of FlashAttention"
// (section 4.6): both products on the fp8 matrix cores
// (v_mfma_*_32x32x64_f8f6f4, twice the bf16 rate), the softmax in fp32.
//
// Inputs are Q, K, V in fp8 with one scale per tensor (a stored byte x
// stands for decode(x) * q_scale, and so on), or block-quantized (the
// section's block quantization: one power-of-two scale per 32 elements along
// each contracted axis, applied by the matrix cores, see MX below); O is
// written in bf16 and lse in fp32.  The arithmetic:
//  * S = (Q K^T) * q_scale * k_scale * scale on the matrix cores, which form
//    the fp8 products exactly and sum each 64-term block at reduced
//    precision (measured: errors up to ~2e-5 of the block's sum of
//    |products| on Gaussian data), the blocks in fp32 (with block scales:
//    each 32-term block sum times its two scales);
//  * the online softmax of attn_fwd_bf16_pp_kernel (running reference, fp32
//    row sums), with the probabilities formed as p' = 2^(S log2 e - r) against
//    a reference r kept 4 (log2 units) below the row's running maximum, so the
//    largest p' of a tile that moved the reference is 16;
//  * p' is rounded to fp8 and multiplied with V on the matrix cores: the
//    reference moves whenever some lane's partial row sum of a tile exceeds
//    448, the largest finite E4M3 value, so no p' overflows (each is at most
//    its lane's sum), and probabilities down to 2^-13 of the row maximum keep
//    a representable (subnormal) code;
//  * O = (sum_j p'_j v_j) * v_scale / sum_j p'_j, lse = ln sum_j e^(S_j).
//
// The schedule is the phase-staggered one of attn_fwd_bf16_pp_kernel: 8 waves
// of 32 query rows, waves w and w + 4 on one SIMD half a tile step apart (one
// runs its products while the other runs the softmax), 64-key tiles through
// LDS by buffer-to-LDS loads, one barrier per step.  What differs is the
// operand layout of the fp8 products:
//  * S^T = K Q^T: lane (i, h) of the A operand holds 32 bytes of key row i,
//    the B operand 32 bytes of query row j; byte b of half h is the same
//    reduction index in both (measured), and the product's two scale blocks
//    are bytes 0-15 and 16-31 of both halves (measured): half h takes head
//    columns 64 kk + 16 h .. + 15 and 64 kk + 32 + 16 h .. + 15, so that scale
//    block kb is the quantization block of columns 64 kk + 32 kb .. + 31.
//  * O^T += V^T P^T: the B operand is the tile's p' in fp8 straight from the
//    S^T accumulators of the lane, in register order (32 bytes: both 32-key
//    score tiles' 16 values, so scale block kb is keys 32 kb .. + 31 of the
//    tile); the A operand gathers the same keys in the same
//    order from the row-major V tile with four ds_read_b64_tr_b8, which hand
//    lane q of each 16 lanes byte q % 8 of the 8 bytes addressed by lanes
//    q / 8, q / 8 + 2, .., q / 8 + 14 (measured).  Each addressing lane names
//    the key row that belongs in its byte position, so the transposing read
//    also performs the key permutation.
//  * K and V tiles sit in LDS unpadded with their 16-byte chunks XOR-permuted
//    by a few bits of the row index (different bits for K and V, matched to
//    the row sets each read serves per cycle), so both reads are bank
//    conflict free.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace osm {
namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2_t;

constexpr float kFp8Max = 448.0f;   // largest finite E4M3 value
constexpr float kRefOffset = 4.0f;  // reference 4 log2 units below the maximum

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    // Raw buffer (stride 0): loads at offsets >= bytes return 0, stores there
    // are dropped.
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// 16 bytes per lane from a buffer into LDS (lane L writes dst + OFF + 16 L from
// buffer offset voff + OFF; the range check applies to voff + OFF).
template <int OFF = 0>
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, lds_void_t* dst, uint32_t voff)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff, 0, OFF, 0);
#endif
}

// One 32x32x64 fp8 x fp8 product (both operands E4M3) with E8M0 block
// scales: the 64-element reduction is two blocks of 32, block kb being bytes
// 16 kb .. 16 kb + 15 of both lane halves of a row (measured), and the scale
// of row i's block kb is byte OPA (OPB) of the scale operand of lane
// i + 32 kb of A (B).  Scale byte 127 is 2^0.  The byte selects must be
// constants: the switch folds once the callers' loops are unrolled.
template <int OPB>
__device__ __forceinline__ f32x16 mfma8s_b(i32x8 a, i32x8 b, f32x16 c, int sa, int opa, int sb)
{
    switch (opa) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, OPB, sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 1, sa, OPB, sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 2, sa, OPB, sb);
    default: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 3, sa, OPB, sb);
    }
}
__device__ __forceinline__ f32x16 mfma8s(i32x8 a, i32x8 b, f32x16 c, int sa, int opa, int sb, int opb)
{
    return opb == 0 ? mfma8s_b<0>(a, b, c, sa, opa, sb) : mfma8s_b<1>(a, b, c, sa, opa, sb);
}

// With MX (block-quantized inputs) a stored byte x of Q or K stands for
// decode(x) * 2^(s - 127) with s the scale byte of its row's 32-column block
// (Qs, Ks: [slice][N][D / 32]), a byte of V for decode(x) * 2^(s - 127) with
// s the byte of its column's 32-key block (Vs: [slice][ceil(N / 32)][D]);
// the matrix cores apply every block scale, so qk_scale is the softmax
// scale alone and v_scale is 1.  Without MX the scale pointers are unused.
template <int D, bool CAUSAL, bool MX>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_fp8_pp_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
                       const uint8_t* __restrict__ V, const uint8_t* __restrict__ Qs,
                       const uint8_t* __restrict__ Ks, const uint8_t* __restrict__ Vs,
                       __bf16* __restrict__ O, float* __restrict__ lse, int N, int BH, int nqt,
                       float qk_scale, float v_scale, int H, int Hkv)
{
    constexpr int NW = 8, BC = 64, BR = 256;
    constexpr int TB = BC * D;                         // tile bytes (unpadded rows of D bytes)
    constexpr int STAGE = 2 * 32 * (D + 8) * 2;        // output staging per buffer (two waves)
    constexpr int BUF = TB > STAGE ? TB : STAGE;
    __shared__ __attribute__((aligned(1024))) char kbuf0[BUF];
    __shared__ __attribute__((aligned(1024))) char kbuf1[BUF];
    __shared__ __attribute__((aligned(1024))) char vbuf0[BUF];
    __shared__ __attribute__((aligned(1024))) char vbuf1[BUF];
    auto kbuf = [&](auto bufc) -> char* { if constexpr (decltype(bufc)::value == 0) return kbuf0; else return kbuf1; };
    auto vbuf = [&](auto bufc) -> char* { if constexpr (decltype(bufc)::value == 0) return vbuf0; else return vbuf1; };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool late = wave >= NW / 2;  // runs each phase one step after its SIMD partner
    const int j = lane & 31, h = lane >> 5;
    const int t = blockIdx.x / BH, bh = blockIdx.x - t * BH;
    const int qt = CAUSAL ? nqt - 1 - t : t;
    const int q0 = qt * BR;
    const int b = bh / H, hh = bh - b * H;
    const size_t base = (size_t)bh * N * D;
    const size_t kvs = (size_t)b * Hkv + hh / (H / Hkv);  // key/value slice
    const size_t kvbase = kvs * N * D;
    const uint32_t slice_b = (uint32_t)N * D;
    const int qw0 = q0 + wave * 32;
    const int qrow = qw0 + j;

    // Q rows as B operands: qf[kk] holds head columns 64 kk + 16 h .. + 15
    // in bytes 0-15 and 64 kk + 32 + 16 h .. + 15 in bytes 16-31, so that the
    // product's reduction block kb is head columns 64 kk + 32 kb .. + 31: one
    // quantization block of 32 columns.
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + base, slice_b);
    i32x8 qf[D / 64];
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk) {
        const uint32_t off = (uint32_t)(qrow * D + 64 * kk + 16 * h);
        const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0);
        const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(qrs, off + 32, 0, 0);
        qf[kk] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                       (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    // Block scales (MX).  Lane (i, h) supplies the scale of block h of its
    // row in each product: for Q, byte kk of qsc is block 2 kk + h of query
    // row qrow.  Rows past N read as zero (and their codes are zero).
    constexpr int SPR = D / 32;  // scale bytes per row (Q, K)
    const int nkb = (N + 31) / 32;
    // Without MX every byte of every scale operand is 127 (2^0).
    constexpr int kUnitScales = 0x7F7F7F7F;
    int qsc = kUnitScales;
    const __amdgpu_buffer_rsrc_t ksrs = make_rsrc(MX ? Ks + kvs * N * SPR : K, MX ? (uint32_t)N * SPR : 0u);
    const __amdgpu_buffer_rsrc_t vsrs = make_rsrc(MX ? Vs + kvs * nkb * D : V, MX ? (uint32_t)nkb * D : 0u);
    if constexpr (MX) {
        const __amdgpu_buffer_rsrc_t qsrs = make_rsrc(Qs + (size_t)bh * N * SPR, (uint32_t)N * SPR);
        qsc = 0;
#pragma unroll
        for (int kk = 0; kk < D / 64; ++kk)
            qsc |= (int)__builtin_amdgcn_raw_buffer_load_b8(qsrs, (uint32_t)(qrow * SPR + 2 * kk + h), 0, 0)
                   << (8 * kk);
    }
    // K scales of tile kt: byte mt * D / 64 + kk is block 2 kk + h of key row
    // 64 kt + 32 mt + j.  V scales of tile kt: byte dt is the block of keys
    // 64 kt + 32 h .. + 31 of head column 32 dt + j.
    auto load_ksc = [&](int kt) __attribute__((always_inline)) -> int {
        if constexpr (D == 128) {
            // the two rows' four scale bytes each, then bytes h and 2 + h of
            // row 32 mt + j into bytes 2 mt and 2 mt + 1 (v_perm_b32: selector
            // values 0-3 pick bytes of the second operand, 4-7 of the first)
            const uint32_t r0 = __builtin_amdgcn_raw_buffer_load_b32(
                ksrs, (uint32_t)((64 * kt + j) * SPR), 0, 0);
            const uint32_t r1 = __builtin_amdgcn_raw_buffer_load_b32(
                ksrs, (uint32_t)((64 * kt + 32 + j) * SPR), 0, 0);
            return (int)__builtin_amdgcn_perm(r1, r0, 0x06040200u + 0x01010101u * (uint32_t)h);
        } else {
            int w = 0;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                w |= (int)__builtin_amdgcn_raw_buffer_load_b8(
                         ksrs, (uint32_t)((64 * kt + 32 * mt + j) * SPR + h), 0, 0)
                     << (8 * mt);
            return w;
        }
    };
    auto load_vsc = [&](int kt) __attribute__((always_inline)) -> int {
        int w = 0;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
            w |= (int)__builtin_amdgcn_raw_buffer_load_b8(
                     vsrs, (uint32_t)((2 * kt + h) * D + 32 * dt + j), 0, 0)
                 << (8 * dt);
        return w;
    };
    int ksc = kUnitScales, vsc = kUnitScales;  // scales of the next S^T and P V products
    if constexpr (MX) ksc = load_ksc(0);

    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
    float m = kNegInf, l = 0.f;  // reference (raw score units) and this lane's row sum
    const float c = qk_scale * kLog2e;

    const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
    const int ntiles = (kv_end + BC - 1) / BC;
    const int T = CAUSAL ? min(ntiles, qw0 / BC + 1) : ntiles;
    const int kvm = (T - 1) * BC;
    const bool mask_last = (kvm + BC > N) || (CAUSAL && kvm + BC - 1 > qw0);

    // Tile layout: row r (key) of D bytes, 16-byte chunk c at slot c ^ key(r).
    //   K: key(r) = (r / RPQ) & (CPR - 1): the 16 key rows a ds_read_b128
    //      serves per cycle then fall in 16 different 16-byte bank groups.
    //   V: key(r) = 2 ((r >> 1) & 1 | ((r >> 3) & 1) << 1) at D = 128 and
    //      2 ((r >> 3) & 1) at D = 64: the 8 key rows x 32 bytes that 32 lanes
    //      of a ds_read_b64_tr_b8 take per cycle fall in 16 different groups.
    constexpr int CPR = D / 16, RPQ = 256 / D;
    constexpr int NG = NW / 2;
    constexpr int LPW = (TB / 1024) / NG;  // 1 KiB loads per wave and tile part
    static_assert(LPW >= 1 && LPW <= 2 && (TB / 1024) % NG == 0, "tile parts split evenly");
    auto kkey = [](int r) { return (r / RPQ) & (CPR - 1); };
    auto vkey = [](int r) {
        if constexpr (D == 128) return 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1));
        else return 2 * ((r >> 3) & 1);
    };
    const int g = wave % NG;
    uint32_t src[LPW];
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
        const int p = (g * LPW + u) * 64 + lane;
        const int r = p / CPR, slot = p % CPR;
        const int cc = slot ^ (late ? vkey(r) : kkey(r));
        src[u] = (uint32_t)(r * D + 16 * cc) - 1024u * u;
    }
    // This wave's share of tile kt of X (K for waves 0-3, V for 4-7) into dst;
    // a tile past the last one gets an empty range (its loads fill dst with
    // zeros, which no later step reads).
    auto load_part = [&](const uint8_t* X, char* dst, int kt) __attribute__((always_inline)) {
        // kt and the range are wave-uniform; said explicitly, because the
        // compiler otherwise keeps the late group's range in a vector
        // register and wraps each load in a loop over its distinct values.
        kt = __builtin_amdgcn_readfirstlane(kt);
        const int kv0 = kt * BC;
        const uint32_t range = (uint32_t)__builtin_amdgcn_readfirstlane(
            kt < ntiles ? (int)((uint32_t)(N - kv0) * D) : 0);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(X + kvbase + (size_t)kv0 * D, range);
        lds_void_t* const d = (lds_void_t*)(dst + g * LPW * 1024);
        lds_dma16<0>(rs, d, src[0]);
        if constexpr (LPW > 1) lds_dma16<1024>(rs, d, src[1]);
    };

    // Operand read addresses.  K (S^T A operand): lane (i, h) reads key row
    // 32 mt + i, chunks 4 kk + h and 4 kk + 2 + h (the arrangement of qf):
    // kb ^ (64 kk) and kb ^ (64 kk + 32).
    const int kb = j * D + 16 * (kkey(j) ^ h);
    // V (P V A operand, d-tile dt, read rr): lane l of 16-lane group gq
    // addresses key row 32 (rr >> 1) + 16 (rr & 1) + 8 (b2 >> 2) + 4 h + (b2 & 3)
    // (b2 = (l % 16) / 2: the key of byte b2 of the receiving lanes), bytes
    // 32 dt + 16 (gq & 1) + 8 (l & 1) .. + 7.
    const int gq = lane >> 4, b2 = (lane & 15) >> 1;
    const int vrow = 8 * (b2 >> 2) + 4 * h + (b2 & 3);
    const int vb = vrow * D + 8 * (lane & 1) + 16 * (gq & 1) + 16 * vkey(vrow);

    f32x16 s[2];  // scores of the current tile, 32 keys each
    i32x8 pf;     // its probabilities p' in fp8, the B operand of P V
    pf = i32x8{};

    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    auto kread = [&](auto kbc, int mt, int kk) __attribute__((always_inline)) -> i32x8 {
        const char* p0 = kbuf(kbc) + mt * 32 * D + (kb ^ (64 * kk));
        const char* p1 = kbuf(kbc) + mt * 32 * D + (kb ^ (64 * kk + 32));
        const u32x4 lo = *reinterpret_cast<const u32x4*>(p0);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(p1);
        return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    auto qk = [&](auto kbc) __attribute__((always_inline)) {
        s[0] = f32x16{};
        s[1] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 64; ++kk)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                s[mt] = mfma8s(kread(kbc, mt, kk), qf[kk], s[mt], ksc, mt * (D / 64) + kk, qsc, kk);
    };
    auto pv = [&](auto vbc) __attribute__((always_inline)) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            i32x8 va;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const char* vp = vbuf(vbc) + (32 * (rr >> 1) + 16 * (rr & 1)) * D + (vb ^ (32 * dt));
                const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)vp);
                va[2 * rr] = w[0];
                va[2 * rr + 1] = w[1];
            }
            acc[dt] = mfma8s(va, pf, acc[dt], vsc, dt, 127, 0);
        }
    };

    // Matrix phase of step i (1 <= i <= T): the wave's tile loads, P V of tile
    // i - 1, then S^T of tile i (skipped at step T).  A wave past its last tile
    // only loads.
    auto matrix_phase = [&](auto kbc, auto vbc, auto ldc, const uint8_t* X, char* ldst, int kt,
                            int i) __attribute__((always_inline)) {
        constexpr bool LD = decltype(ldc)::value;
        if (CAUSAL && i > T) {
            if constexpr (LD) load_part(X, ldst, kt);
            return;
        }
        if constexpr (LD) {
            load_part(X, ldst, kt);
            __builtin_amdgcn_sched_barrier(0);
        }
        pv(vbc);
        if (i < T) {
            qk(kbc);
            if constexpr (MX) {  // scales of P V (tile i) and S^T (tile i + 1), next phase
                vsc = load_vsc(i);
                ksc = load_ksc(i + 1);
            }
        }
    };
    // Vector phase of step i: mask (last tile only), p' and row sums, fp8
    // conversion, and the rare move of the reference.
    auto vector_phase = [&](int i) __attribute__((always_inline)) {
        if (i < 0 || i >= T) return;
        if (i == T - 1 && mask_last) {
            // Key kvm + 32 mt + 8 (r / 4) + 4 h + r % 4 of register r is hidden
            // when it is past N or (under the mask) after this lane's query.
            int thr = (CAUSAL ? min(N, qrow + 1) : N) - kvm - 4 * h;
            asm volatile("" : "+v"(thr));
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (32 * mt + 8 * (r >> 2) + (r & 3) >= thr) s[mt][r] = kNegInf;
        }
        // p' = 2^(s c - mc) for the current reference (one FMA and one
        // v_exp_f32 each), this lane's partial row sum, and the fp8 codes in
        // register order (byte 4 w + e of pf = register 4 (w % 4) + e of
        // tile w / 4).
        auto probs = [&](float mc) __attribute__((always_inline)) {
            float ps[4];
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                float p4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    p4[e] = exp2_hw(fmaf(s[w >> 2][4 * (w & 3) + e], c, -mc));
                    if (w == 0)
                        ps[e] = p4[e];
                    else
                        ps[e] += p4[e];
                }
                int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p4[0], p4[1], 0, false);
                wd = __builtin_amdgcn_cvt_pk_fp8_f32(p4[2], p4[3], wd, true);
                pf[w] = wd;
            }
            return (ps[0] + ps[1]) + (ps[2] + ps[3]);
        };
        float lsum = i == 0 ? 0.f : probs(m * c - kRefOffset);
        // While every lane's sum stays within the largest E4M3 value, so does
        // every p' of the tile.  Otherwise, and on tile 0, the reference moves
        // to the row maximum (less the offset): l and the accumulators are
        // rescaled by 2^(c (m_old - m_new)) and p' is recomputed.
        if (i == 0 || __builtin_amdgcn_ballot_w64(lsum > kFp8Max) != 0) {
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = fmaxf(s[0][u], s[0][u + 4]);
#pragma unroll
            for (int r = 8; r < 16; ++r) v[r & 3] = fmaxf(v[r & 3], s[0][r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) v[r & 3] = fmaxf(v[r & 3], s[1][r]);
            const float mx = combine_xor32(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])), MaxOp());
            const float m_new = fmaxf(m, mx);
            const float alpha = (m_new == kNegInf) ? 1.f : exp2_hw((m - m_new) * c);
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) acc[dt] *= alpha;
            m = m_new;
            lsum = probs(m * c - kRefOffset);
        }
        l += lsum;
    };

    // Prologue: K(0) (waves 0-3).
    if (!late) load_part(K, kbuf0, 0);
    __syncthreads();
    // Steps i = 0 .. ntiles as in attn_fwd_bf16_pp_kernel: step 0 (S^T of
    // tile 0) peeled, two steps per loop trip (K(i) in kbuf[i % 2], V(i) in
    // vbuf[i % 2]), one barrier per step.  Waves 4-7 load V(i) at the start of
    // their vector phase 2i (the fp8 matrix phase is too short to cover a load
    // issued at its start).
    auto steps = [&](auto latec) __attribute__((always_inline)) {
        constexpr bool LATE = decltype(latec)::value;
        if constexpr (!LATE) {
            if (1 < ntiles) load_part(K, kbuf1, 1);
            qk(B0{});
            if constexpr (MX) {
                vsc = load_vsc(0);
                ksc = load_ksc(1);
            }
            vector_phase(0);
        } else {
            load_part(V, vbuf0, 0);
            qk(B0{});
            if constexpr (MX) {
                vsc = load_vsc(0);
                ksc = load_ksc(1);
            }
        }
        __syncthreads();  // K(1) and V(0) have landed
        for (int i = 1; i <= ntiles; i += 2) {
            if constexpr (!LATE) {
                matrix_phase(B1{}, B0{}, std::true_type{}, K, kbuf0, i + 1, i);
                vector_phase(i);
            } else {
                load_part(V, vbuf1, i);
                vector_phase(i - 1);
                matrix_phase(B1{}, B0{}, std::false_type{}, V, vbuf1, i, i);
            }
            if (i + 1 > ntiles) break;
            __syncthreads();  // K(i + 1) and V(i) have landed
            if constexpr (!LATE) {
                matrix_phase(B0{}, B1{}, std::true_type{}, K, kbuf1, i + 2, i + 1);
                vector_phase(i + 1);
            } else {
                load_part(V, vbuf0, i + 1);
                vector_phase(i);
                matrix_phase(B0{}, B1{}, std::false_type{}, V, vbuf0, i + 1, i + 1);
            }
            __syncthreads();  // K(i + 2) and V(i + 1) have landed
        }
    };
    if (late)
        steps(std::true_type{});
    else
        steps(std::false_type{});

    const __amdgpu_buffer_rsrc_t ors = make_rsrc(O + base, slice_b * 2);
    const __amdgpu_buffer_rsrc_t lrs = make_rsrc(lse + (size_t)bh * N, (uint32_t)N * 4);
    const float l_tot = combine_xor32(l, SumOp());
    __syncthreads();  // every wave is done with the tile buffers
    char* const stage = (wave < 2 ? kbuf0 : wave < 4 ? kbuf1 : wave < 6 ? vbuf0 : vbuf1) +
                        (wave & 1) * (32 * (D + 8) * 2);
    store_tile_rows<D>(acc, v_scale / l_tot, stage, ors, qw0, lane);
    if (h == 0)
        __builtin_amdgcn_raw_buffer_store_b32(
            __float_as_uint(m * qk_scale + (log2_hw(l_tot) - kRefOffset) * kLn2), lrs,
            (uint32_t)qrow * 4, 0, 0);
}

struct Fp8Args {
    const void *Q, *K, *V, *Qs, *Ks, *Vs;
    void* O;
    float* lse;
    int BH, N, H, Hkv;
    float qk_scale, v_scale;
};

template <int D, bool CAUSAL, bool MX>
hipError_t launch_fp8(const Fp8Args& a, hipStream_t stream)
{
    const int nqt = (a.N + 255) / 256;
    attn_fwd_fp8_pp_kernel<D, CAUSAL, MX><<<dim3((unsigned)(nqt * a.BH)), dim3(512), 0, stream>>>(
        static_cast<const uint8_t*>(a.Q), static_cast<const uint8_t*>(a.K),
        static_cast<const uint8_t*>(a.V), static_cast<const uint8_t*>(a.Qs),
        static_cast<const uint8_t*>(a.Ks), static_cast<const uint8_t*>(a.Vs),
        static_cast<__bf16*>(a.O), a.lse, a.N, a.BH, nqt, a.qk_scale, a.v_scale, a.H, a.Hkv);
    return hipGetLastError();
}

template <bool MX>
hipError_t dispatch_fp8(const Fp8Args& a, int d, bool causal, hipStream_t stream)
{
    if (d == 64)
        return causal ? launch_fp8<64, true, MX>(a, stream) : launch_fp8<64, false, MX>(a, stream);
    return causal ? launch_fp8<128, true, MX>(a, stream) : launch_fp8<128, false, MX>(a, stream);
}

}  // namespace

hipError_t launch_attn_fwd_fp8(const void* Q, const void* K, const void* V, void* O, float* lse,
                               int B, int H, int Hkv, int N, int d, float qk_scale, float v_scale,
                               bool causal, hipStream_t stream)
{
    const Fp8Args a{Q, K, V, nullptr, nullptr, nullptr, O, lse, B * H, N, H, Hkv, qk_scale, v_scale};
    return dispatch_fp8<false>(a, d, causal, stream);
}

hipError_t launch_attn_fwd_fp8_mx(const void* Q, const void* Qs, const void* K, const void* Ks,
                                  const void* V, const void* Vs, void* O, float* lse, int B, int H,
                                  int Hkv, int N, int d, float scale, bool causal, hipStream_t stream)
{
    const Fp8Args a{Q, K, V, Qs, Ks, Vs, O, lse, B * H, N, H, Hkv, scale, 1.0f};
    return dispatch_fp8<true>(a, d, causal, stream);
}

}  // namespace osm
