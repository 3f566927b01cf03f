// attn_bwd_bf16.hip -- backward pass of the bf16 attention forward on the
// gfx950 bf16 matrix cores: dQ, dK, dV of L = sum(dO * O), written as bf16.
//
// Method: recompute instead of store ("Lesson 22: why softmax is hard to make
// efficient, and how FlashAttention reduces memory traffic", sections 30-31;
// "Moving less: four generations of FlashAttention", 2.4): every probability
// tile is rebuilt from Q, K and the forward's row statistic,
// P_ij = exp(S_ij - L_i) with L = lse, so no N x N matrix is read or written.
// The gradients are the chain rule through O = P V and the row softmax:
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  D_i = sum_t dO_it O_it,
//   dQ = scale dS K,  dK = scale dS^T Q
// (D_i equals sum_j P_ij dP_ij because O_i = sum_j P_ij V_j).
//
// gfx950 design -- two kernels, no atomics, bitwise deterministic:
//  * row statistics D and L log2(e): formed by the dQ kernel (below), which
//    holds each row's dO in VGPRs anyway and loads its O row next to it; it
//    runs first and stores them for the dK/dV kernel.  The split backward
//    takes them from attn_bwd_delta_kernel (HBM bound, reads O, dO), since
//    its dQ workgroups cover a query block several times.
//  * attn_bwd_dkdv_kernel: one workgroup per (batch*key/value head, 256 keys),
//    summing over the query heads that share the key/value head, a wave
//    per 32 keys (two per SIMD), the keys' K rows held in VGPRs and their V
//    rows in LDS for the whole kernel as the B operands of S = Q K^T and
//    dP = dO V^T (one key per lane, the queries of a 32-query step in the
//    accumulator registers).  Query tiles
//    of 64 rows of Q and dO stream through LDS, double-buffered.  P and dS,
//    rounded to bf16, are register for register the B operands of
//    dV^T += dO^T P and dK^T += Q^T dS, whose A operands come from the same
//    tiles through the transposing LDS read.  The column-block split is the
//    one of the four-generations page, 3.3; unlike there, dQ is not summed
//    across these workgroups with atomic adds.
//  * attn_bwd_dq_kernel: one workgroup per (batch*head, 256 queries), a wave
//    per 32 queries with Q and dO in VGPRs, K and V tiles of 64 keys through
//    LDS: S^T = K Q^T and dP^T = V dO^T (one query per lane, as in the
//    forward), then dQ^T += K^T dS^T.  Recomputing S and dP here costs two
//    more products than accumulating dQ with atomics, and keeps dQ exact to
//    the summation order and reproducible.
//  * Q/dO (dK/dV kernel) and K (dQ kernel) tiles are read both row-wise
//    (ds_read_b128, rows permuted at read time so that each 8-register group
//    of an accumulator holds 8 consecutive tile rows) and transposed
//    (ds_read_b64_tr_b16).  No row pitch is free of bank conflicts for both:
//    a b128 read serves 16 lanes (16 rows) per cycle and wants rows 16 bytes
//    apart modulo 256, the transposed read serves 32 lanes (64 bytes of each
//    of 4 rows) and wants them 64 bytes apart.  So tiles keep pitch d + 8 and
//    store the rows of each 16-row group in the order that swaps the two
//    2-bit halves of the row index: the 4 rows of a transposed read then
//    lie 4 physical rows (64 bytes modulo 256) apart, while the 16 rows of a
//    row-wise read are still 16 distinct rows of one group.  The permutation
//    is its own inverse and costs nothing: the DMA source offsets and the
//    lanes' LDS addresses are computed once.

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace osm {
namespace {

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

__device__ __forceinline__ int swap_bits23(int i)
{
    return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// Physical LDS row of tile row r: bits 0-1 and 2-3 of r swapped.
__device__ __forceinline__ int lds_row(int r)
{
    return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, lds_void_t* dst, uint32_t voff)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff, 0, 0, 0);
#endif
}

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Tile of R rows x D bf16 in LDS with row pitch D + 8 elements, filled by
// 1 KiB wave loads: load i writes chunk positions 64 i .. 64 i + 63; chunk
// position p holds tile row lds_row(p / (D/8 + 1)), column chunk
// p % (D/8 + 1) (the last chunk of a row is padding and re-fetches the row's
// last real chunk).
template <int D, int R>
struct Tile {
    static constexpr int P = D + 8;          // row pitch (elements)
    static constexpr int CPR = P / 8;        // 16-byte chunks per row
    static constexpr int BYTES = R * P * 2;
    static constexpr int INST = BYTES / 1024;
    static_assert(BYTES % 1024 == 0, "tile is whole wave loads");
    static_assert(R % 16 == 0, "rows are permuted in groups of 16");
    __device__ static uint32_t src_offset(int p)
    {
        const int row = lds_row(p / CPR), ch = min(p % CPR, D / 8 - 1);
        return (uint32_t)(row * D + ch * 8) * 2;
    }
};

// A operand of a 32x32x16 product from a row-major LDS tile, row-wise: lane
// (i, h) supplies tile row row0 + swap_bits23(i), columns col0 + 8 h .. + 7
// (row0 a multiple of 16).
template <int PITCH>
__device__ __forceinline__ bf16x8 rows_a(const char* tile, int row0, int col0, int i, int h)
{
    return *reinterpret_cast<const bf16x8*>(
        tile + ((row0 + lds_row(swap_bits23(i))) * PITCH + col0 + 8 * h) * 2);
}

// A operand from a row-major LDS tile, transposed: operand row i is tile
// column col0 + i, operand column k (= 8 h + e) is tile row row0 + k, via
// two ds_read_b64_tr_b16 (lane 16 g + 4 e + a reads 4 columns
// 16 (g % 2) + 4 a of tile row 8 (g / 2) + e, and of the row 4 further,
// which are physical rows 4 e + 2 (g / 2) and the next one; row0 a multiple
// of 16).
template <int PITCH>
__device__ __forceinline__ bf16x8 cols_a(const char* tile, int row0, int col0, int lane)
{
    const int g16 = lane >> 4, e4 = (lane >> 2) & 3, a4 = lane & 3;
    const char* p = tile + ((row0 + 4 * e4 + 2 * (g16 >> 1)) * PITCH + col0 + 16 * (g16 & 1) + 4 * a4) * 2;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p + PITCH * 2));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Rows of one (sequence, head) slice.  Dense tensors [B][Hx][N][D] (Hx = H
// for Q, O, dO and the row statistics, Hkv for K and V): the slice of
// (b, hx) starts at row (b Hx + hx) N and has N rows.  Packed sequences
// [Hx][total][D]: it starts at row hx total + cu[b] and has cu[b+1] - cu[b]
// rows, clamped to [0, Nmax] and to the packed extent.
template <bool VARLEN>
struct Seq {
    int b, start, n, total;
    __device__ Seq(int b_, int Nmax, const int* cu, int total_) : b(b_), total(total_)
    {
        if constexpr (VARLEN) {
            start = min(max(__builtin_amdgcn_readfirstlane(cu[b]), 0), total);
            const int end = min(max(__builtin_amdgcn_readfirstlane(cu[b + 1]), start), total);
            n = min(end - start, Nmax);
        } else {
            start = 0;
            n = Nmax;
        }
    }
    // First row of head hx of a tensor with Hx heads (dense stride: n rows).
    __device__ size_t row0(int hx, int Hx) const
    {
        if constexpr (VARLEN) return (size_t)hx * total + start;
        else return ((size_t)b * Hx + hx) * n;
    }
};

// bf16 of registers 8 G .. 8 G + 7 of an accumulator.
__device__ __forceinline__ bf16x8 half_bf16(const f32x16& v, int G)
{
    const f32x8 p8 = G ? __builtin_shufflevector(v, v, 8, 9, 10, 11, 12, 13, 14, 15)
                       : __builtin_shufflevector(v, v, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_convertvector(p8, bf16x8);
}

// fp32 rows of a wave's 32-row accumulator tile (lane (j, h) holds row
// row0 + j, columns 32 dt + 8 g + 4 h .. + 3 in registers 4 g .. 4 g + 3 of
// acc[dt]), stored straight from the registers: 16 bytes per lane and
// instruction.  Rows past the buffer's range are dropped.
template <int D>
__device__ __forceinline__ void store_rows_f32(const f32x16 (&acc)[D / 32],
                                               __amdgpu_buffer_rsrc_t rs, int row0, int lane)
{
    const int j = lane & 31, h = lane >> 5;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 o4 = {acc[dt][4 * g], acc[dt][4 * g + 1], acc[dt][4 * g + 2], acc[dt][4 * g + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o4), rs,
                                                   (uint32_t)((row0 + j) * D + dt * 32 + 8 * g + 4 * h) * 4, 0, 0);
        }
}

// ---------------------------------------------------------------- delta ----
// D[r] = sum_t dO[r][t] O[r][t] (bf16 products, fp32 sums) and
// Lc[r] = lse[r] log2(e), for rows r of [rows][D]; D / 8 lanes per row.
template <int D>
__global__ void __launch_bounds__(256)
attn_bwd_delta_kernel(const __bf16* __restrict__ O, const __bf16* __restrict__ dO,
                      const float* __restrict__ lse, float* __restrict__ Dl,
                      float* __restrict__ Lc, long long rows)
{
    constexpr int LPR = D / 8, RPB = 256 / LPR;
    const int c8 = threadIdx.x % LPR;
    for (long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR; row < rows;
         row += (long long)gridDim.x * RPB) {
        // all three loads first (every lane of the row reads its lse, one
        // cache line), so that a row costs one memory round trip
        const bf16x8 o = *reinterpret_cast<const bf16x8*>(O + row * D + 8 * c8);
        const bf16x8 g = *reinterpret_cast<const bf16x8*>(dO + row * D + 8 * c8);
        float L = lse[row];
        asm volatile("" : "+v"(L));  // keeps the load here instead of sunk into the branch
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf((float)o[e], (float)g[e], s);
        // sum over the row's LPR lanes (a 16- or 8-lane group) by DPP:
        // quads, then the two quads of a half-row, then the two half-rows
        s += dpp<0xB1>(s);   // quad_perm [1,0,3,2]
        s += dpp<0x4E>(s);   // quad_perm [2,3,0,1]
        s += dpp<0x141>(s);  // row_half_mirror
        if constexpr (LPR == 16) s += dpp<0x140>(s);  // row_mirror
        if (c8 == 0) {
            Dl[row] = s;
            Lc[row] = L * kLog2e;
        }
    }
}

// ------------------------------------------------------------ dK and dV ----
template <int D, int NW, bool CAUSAL, bool VARLEN, bool SPLIT = false>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dkdv_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                     const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                     const float* __restrict__ Lc, const float* __restrict__ Dl,
                     __bf16* __restrict__ dK, __bf16* __restrict__ dV, int Nmax, int BHkv, int H,
                     int Hkv, float scale, const int* __restrict__ cu, int total,
                     float* __restrict__ part, int nsplit)
{
    constexpr int BK = NW * 32, BQ = 64;
    using TQ = Tile<D, BQ>;
    using TV = Tile<D, BK>;
    constexpr int LPW = (TQ::INST + NW - 1) / NW;  // loads per wave per tile
    constexpr int VPW = (TV::INST + NW - 1) / NW;  // loads per wave of the V block
    // The V block of 8-wave workgroups sits in dynamic LDS (the launch passes
    // its size), the smaller workgroups' in a static array.  The compiler
    // schedules for the static footprint it sees: with all 137 KiB static at
    // D = 128 (one workgroup per CU) it schedules the 8-wave kernel's loop
    // looser and the call runs 2-3% slower; the 4-wave kernel, which does run
    // one workgroup per CU with more than 256 registers, loses 3% the other
    // way round.  Same instructions, bitwise-equal gradients.
    extern __shared__ __attribute__((aligned(1024))) char vdyn[];
    __shared__ __attribute__((aligned(1024))) char vsta[NW == 8 ? 16 : TV::BYTES];
    char* const vblk = NW == 8 ? vdyn : vsta;
    __shared__ __attribute__((aligned(1024))) char qb0[TQ::BYTES];
    __shared__ __attribute__((aligned(1024))) char qb1[TQ::BYTES];
    __shared__ __attribute__((aligned(1024))) char ob0[TQ::BYTES];
    __shared__ __attribute__((aligned(1024))) char ob1[TQ::BYTES];
    __shared__ __attribute__((aligned(16))) float lb[2][BQ];
    __shared__ __attribute__((aligned(16))) float db[2][BQ];
    auto qbuf = [&](auto bc) -> char* { if constexpr (decltype(bc)::value == 0) return qb0; else return qb1; };
    auto obuf = [&](auto bc) -> char* { if constexpr (decltype(bc)::value == 0) return ob0; else return ob1; };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31, h = lane >> 5;
    // Key blocks in natural order: under the mask the first ones see the
    // most queries, so the longest workgroups start first.  The workgroup's
    // key/value head kvbh serves the query heads b H + hkv G .. + G - 1
    // (G = H / Hkv), whose contributions it sums.
    // With SPLIT (dense only) the query tiles of a key block are divided
    // into nsplit contiguous ranges, one workgroup per (key block, range);
    // each writes its partial dK^T and dV^T sums in fp32 to part.
    const int tt = blockIdx.x / BHkv, kvbh = blockIdx.x - tt * BHkv;
    const int t = SPLIT ? tt / nsplit : tt;
    const int sp = SPLIT ? tt - t * nsplit : 0;
    const int k0 = t * BK, kw0 = k0 + wave * 32;
    const int G = H / Hkv, hkv = kvbh % Hkv;
    const Seq<VARLEN> sq(kvbh / Hkv, Nmax, cu, total);
    const int N = sq.n;
    if (VARLEN && k0 >= N) return;  // key block past this sequence (whole workgroup)
    const size_t base = sq.row0(hkv, Hkv) * D;
    const uint32_t slice_b = (uint32_t)N * D * 2;
    const float c = scale * kLog2e;

    // K rows of this wave's keys as B operands in VGPRs: lane (j, h), step
    // kk holds row kw0 + j, columns 16 kk + 8 h .. + 7 (zero past N).  The
    // workgroup's V rows wait in LDS (registers would not leave room for two
    // waves per SIMD); lane (j, h) reads the same part of V row kw0 + j.
    bf16x8 kf[D / 16];
    {
        const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + base, slice_b);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            const uint32_t off = (uint32_t)((kw0 + j) * D + kk * 16 + 8 * h) * 2;
            kf[kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0));
        }
        const uint32_t vleft = (uint32_t)(N - k0) * D * 2;
        const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + base + (size_t)k0 * D, vleft);
#pragma unroll
        for (int u = 0; u < VPW; ++u) {
            const int i = wave + u * NW;
            if (TV::INST % NW == 0 || i < TV::INST)
                lds_dma16(vrs, (lds_void_t*)(vblk + i * 1024), TV::src_offset(i * 64 + lane));
        }
    }
    const char* vrow = vblk + ((wave * 32 + lds_row(j)) * TV::P + 8 * h) * 2;
    f32x16 dvt[D / 32], dkt[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
        dvt[dt] = f32x16{};
        dkt[dt] = f32x16{};
    }

    uint32_t src[LPW];
#pragma unroll
    for (int u = 0; u < LPW; ++u) src[u] = TQ::src_offset((wave + u * NW) * 64 + lane);
    // Steps it = 0 .. G * nq - 1 walk query head g = it / nq of the group and
    // its query tile qt0 + it % nq.
    const int nqt = (N + BQ - 1) / BQ;
    const int qt0 = CAUSAL ? k0 / BQ : 0;     // first query tile with a visible pair
    const int nq = nqt - qt0;
    auto tile_of = [&](int it) { return qt0 + it % nq; };
    auto qbase_of = [&](int it) { return sq.row0(hkv * G + it / nq, H); };  // row 0 of the query head
    auto issue = [&](auto bc, int it) {
        const int r0 = tile_of(it) * BQ;
        const size_t qb = (qbase_of(it) + r0) * D;
        const uint32_t left = (uint32_t)(N - r0) * D * 2;
        const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + qb, left);
        const __amdgpu_buffer_rsrc_t ors = make_rsrc(dO + qb, left);
#pragma unroll
        for (int u = 0; u < LPW; ++u) {
            const int i = wave + u * NW;
            if (TQ::INST % NW == 0 || i < TQ::INST) {
                lds_dma16(qrs, (lds_void_t*)(qbuf(bc) + i * 1024), src[u]);
                lds_dma16(ors, (lds_void_t*)(obuf(bc) + i * 1024), src[u]);
            }
        }
    };
    // Row statistics of a query tile: threads 0-63 fetch L log2(e), 64-127
    // fetch D (zero past N); written to LDS before the tile's barrier.
    auto stat_load = [&](int it) -> float {
        const int q = tile_of(it) * BQ + (tid & 63);
        if (tid < 2 * BQ && q < N) return (tid < BQ ? Lc : Dl)[qbase_of(it) + q];
        return 0.f;
    };
    auto stat_store = [&](auto bc, float v) {
        if (tid < BQ) lb[decltype(bc)::value][tid] = v;
        else if (tid < 2 * BQ) db[decltype(bc)::value][tid - BQ] = v;
    };

    const int key = kw0 + j;                  // this lane's key

    auto compute = [&](auto bc, int it) {
        const int qt = tile_of(it);
        if (CAUSAL && qt * BQ + BQ - 1 < kw0) return;  // every query precedes every key
        const char* qt_l = qbuf(bc);
        const char* ot_l = obuf(bc);
        const float* lbv = lb[decltype(bc)::value];
        const float* dbv = db[decltype(bc)::value];
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
            const int qr0 = qt * BQ + 32 * qs;       // first query of the step
            if (qr0 >= N) continue;                  // past the last query
            // S = Q K^T for the 32 queries and this wave's 32 keys; register
            // r of half h holds query qr0 + 16 (r / 8) + 8 h + r % 8.
            f32x16 s = f32x16{};
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
                s = mfma(rows_a<TQ::P>(qt_l, 32 * qs, 16 * kk, j, h), kf[kk], s);
            // P = exp(S scale - L), in place; masked pairs (query past N, or
            // key after query) are exactly 0.
#pragma unroll
            for (int G = 0; G < 2; ++G) {
                const int qi0 = 32 * qs + 16 * G + 8 * h;  // tile row of register 8 G
                const f32x4 l0 = *reinterpret_cast<const f32x4*>(lbv + qi0);
                const f32x4 l1 = *reinterpret_cast<const f32x4*>(lbv + qi0 + 4);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    s[8 * G + e] = exp2_hw(fmaf(s[8 * G + e], c, -(e < 4 ? l0[e] : l1[e - 4])));
            }
            if ((qr0 + 32 > N) || (CAUSAL && qr0 < kw0 + 31)) {
                // Offsets of N and of this lane's key from the first query of
                // the lane's registers; kept opaque so that the compares
                // below are not hoisted out of the query loop as 16
                // loop-invariant thresholds.
                int nq = N - qr0 - 8 * h, kq = key - qr0 - 8 * h;
                asm volatile("" : "+v"(nq), "+v"(kq));
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int o = 16 * (r >> 3) + (r & 7);
                    if (o >= nq || (CAUSAL && kq > o)) s[r] = 0.f;
                }
            }
            // dV^T += dO^T P
            const bf16x8 pb0 = half_bf16(s, 0), pb1 = half_bf16(s, 1);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                dvt[dt] = mfma(cols_a<TQ::P>(ot_l, 32 * qs, 32 * dt, lane), pb0, dvt[dt]);
                dvt[dt] = mfma(cols_a<TQ::P>(ot_l, 32 * qs + 16, 32 * dt, lane), pb1, dvt[dt]);
            }
            // dP = dO V^T, then dS = P (dP - D) in place
            f32x16 dp = f32x16{};
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
                dp = mfma(rows_a<TQ::P>(ot_l, 32 * qs, 16 * kk, j, h),
                          *reinterpret_cast<const bf16x8*>(vrow + kk * 32), dp);
#pragma unroll
            for (int G = 0; G < 2; ++G) {
                const int qi0 = 32 * qs + 16 * G + 8 * h;
                const f32x4 d0 = *reinterpret_cast<const f32x4*>(dbv + qi0);
                const f32x4 d1 = *reinterpret_cast<const f32x4*>(dbv + qi0 + 4);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    dp[8 * G + e] = s[8 * G + e] * (dp[8 * G + e] - (e < 4 ? d0[e] : d1[e - 4]));
            }
            // dK^T += Q^T dS
            const bf16x8 sb0 = half_bf16(dp, 0), sb1 = half_bf16(dp, 1);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                dkt[dt] = mfma(cols_a<TQ::P>(qt_l, 32 * qs, 32 * dt, lane), sb0, dkt[dt]);
                dkt[dt] = mfma(cols_a<TQ::P>(qt_l, 32 * qs + 16, 32 * dt, lane), sb1, dkt[dt]);
            }
        }
    };

    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    const int nit = G * nq;
    int it0 = 0, it1 = nit;  // this workgroup's steps
    if constexpr (SPLIT) {
        const int per = (nit + nsplit - 1) / nsplit;
        it0 = min(nit, sp * per);
        it1 = min(nit, it0 + per);
    }
    if (it1 > it0) {
        issue(B0{}, it0);
        stat_store(B0{}, stat_load(it0));
        __syncthreads();
        for (int it = it0; it < it1; it += 2) {
            float st = 0.f;
            if (it + 1 < it1) {
                issue(B1{}, it + 1);
                st = stat_load(it + 1);
            }
            compute(B0{}, it);
            stat_store(B1{}, st);
            __syncthreads();
            if (it + 1 >= it1) break;
            if (it + 2 < it1) {
                issue(B0{}, it + 2);
                st = stat_load(it + 2);
            }
            compute(B1{}, it + 1);
            stat_store(B0{}, st);
            __syncthreads();
        }
    }
    if constexpr (SPLIT) {
        // Partials [2][nsplit][BHkv][N][D]: dK^T (scale not applied), then
        // dV^T; an empty range writes zeros.
        const size_t slice = (size_t)N * D;
        float* const pk = part + ((size_t)sp * BHkv + kvbh) * slice;
        float* const pv = pk + (size_t)nsplit * BHkv * slice;
        store_rows_f32<D>(dkt, make_rsrc(pk, (uint32_t)slice * 4), kw0, lane);
        store_rows_f32<D>(dvt, make_rsrc(pv, (uint32_t)slice * 4), kw0, lane);
        return;
    }
    // Both gradients leave through the wave's 32-row slice of the V block
    // (BK x (D + 8) elements, 32 rows per wave), which no wave reads any more.
    __syncthreads();
    char* const ost = vblk + wave * 32 * (D + 8) * 2;
    store_tile_rows<D>(dkt, scale, ost, make_rsrc(dK + base, slice_b), key - j, lane);
    store_tile_rows<D>(dvt, 1.0f, ost, make_rsrc(dV + base, slice_b), key - j, lane);
}

// ------------------------------------------------------ split reduction ----
// out[e] = bf16(mul * sum_{s < S} part[s * stride + e]) for the n8 * 8
// elements of one gradient; the sum runs in s order, so the result does not
// depend on the launch shape.  Three gradients per launch (dK, dV, dQ), eight
// elements per thread per trip, grid-stride.
struct SumSeg {
    const float* part;
    __bf16* out;
    long long n8, stride;
    float mul;
};

__global__ void __launch_bounds__(256)
attn_bwd_sum_kernel(SumSeg a, SumSeg b, SumSeg c, int S)
{
    const long long total = a.n8 + b.n8 + c.n8;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (long long)gridDim.x * 256) {
        const float* p;
        __bf16* o;
        long long stride;
        float mul;
        if (i < a.n8) {
            p = a.part + 8 * i; o = a.out + 8 * i; stride = a.stride; mul = a.mul;
        } else if (i < a.n8 + b.n8) {
            const long long k = i - a.n8;
            p = b.part + 8 * k; o = b.out + 8 * k; stride = b.stride; mul = b.mul;
        } else {
            const long long k = i - a.n8 - b.n8;
            p = c.part + 8 * k; o = c.out + 8 * k; stride = c.stride; mul = c.mul;
        }
        f32x4 x0 = *reinterpret_cast<const f32x4*>(p), x1 = *reinterpret_cast<const f32x4*>(p + 4);
        for (int sp = 1; sp < S; ++sp) {
            p += stride;
            x0 += *reinterpret_cast<const f32x4*>(p);
            x1 += *reinterpret_cast<const f32x4*>(p + 4);
        }
        const f32x8 y = {x0[0] * mul, x0[1] * mul, x0[2] * mul, x0[3] * mul,
                         x1[0] * mul, x1[1] * mul, x1[2] * mul, x1[3] * mul};
        *reinterpret_cast<bf16x8*>(o) = __builtin_convertvector(y, bf16x8);
    }
}

// ------------------------------------------------------------------- dQ ----
template <int D, int NW, bool CAUSAL, bool VARLEN, bool SPLIT = false>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dq_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                   const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                   const __bf16* __restrict__ O, const float* __restrict__ lse,
                   float* __restrict__ Lc, float* __restrict__ Dl,
                   __bf16* __restrict__ dQ, int Nmax, int BH, int nqb, int H, int Hkv,
                   float scale, const int* __restrict__ cu, int total,
                   float* __restrict__ part, int nsplit)
{
    constexpr int BR = NW * 32, BC = 64;
    using TK = Tile<D, BC>;
    static_assert(NW <= 8 && TK::BYTES >= 2 * 32 * (D + 8) * 2, "dQ staging fits the tile buffers");
    constexpr int LPW = (TK::INST + NW - 1) / NW;
    __shared__ __attribute__((aligned(1024))) char kb0[TK::BYTES];
    __shared__ __attribute__((aligned(1024))) char kb1[TK::BYTES];
    __shared__ __attribute__((aligned(1024))) char vb0[TK::BYTES];
    __shared__ __attribute__((aligned(1024))) char vb1[TK::BYTES];
    auto kbuf = [&](auto bc) -> char* { if constexpr (decltype(bc)::value == 0) return kb0; else return kb1; };
    auto vbuf = [&](auto bc) -> char* { if constexpr (decltype(bc)::value == 0) return vb0; else return vb1; };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31, h = lane >> 5;
    // With SPLIT (dense only) the key tiles of a query block are divided into
    // nsplit contiguous ranges, one workgroup per (query block, range); each
    // writes its partial dQ^T sum in fp32 to part.
    const int tt = blockIdx.x / BH, bh = blockIdx.x - tt * BH;
    const int t = SPLIT ? tt / nsplit : tt;
    const int sp = SPLIT ? tt - t * nsplit : 0;
    const int qb = CAUSAL ? nqb - 1 - t : t;  // longest first under the mask
    const int q0 = qb * BR, qw0 = q0 + wave * 32, q = qw0 + j;
    const int hq = bh % H;
    const Seq<VARLEN> sq(bh / H, Nmax, cu, total);
    const int N = sq.n;
    if (VARLEN && q0 >= N) return;  // query block past this sequence (whole workgroup)
    const size_t qrow0 = sq.row0(hq, H);
    const size_t base = qrow0 * D;
    const size_t kvbase = sq.row0(hq / (H / Hkv), Hkv) * D;
    const uint32_t slice_b = (uint32_t)N * D * 2;
    const float c = scale * kLog2e;

    // Q and dO rows of this lane's query as B operands (zero past N).
    bf16x8 qf[D / 16], gf[D / 16];
    {
        const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + base, slice_b);
        const __amdgpu_buffer_rsrc_t grs = make_rsrc(dO + base, slice_b);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            const uint32_t off = (uint32_t)(q * D + kk * 16 + 8 * h) * 2;
            qf[kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0));
            gf[kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(grs, off, 0, 0));
        }
    }
    // Row statistics of this lane's query.  With SPLIT they come from
    // attn_bwd_delta_kernel.  Otherwise this kernel forms them (it runs
    // before the dK/dV kernel, which reads them): D = sum_t dO_t O_t in fp32
    // over the lane's 64 elements of the row (chunks 2 kk + h, as Q and dO
    // above) plus the other lane half's, and L log2(e) from lse.
    float lq, dq;
    if constexpr (SPLIT) {
        lq = q < N ? Lc[qrow0 + q] : 0.f;
        dq = q < N ? Dl[qrow0 + q] : 0.f;
    } else {
        const __amdgpu_buffer_rsrc_t ors = make_rsrc(O + base, slice_b);
        float sd = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            const bf16x8 o = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                ors, (uint32_t)(q * D + kk * 16 + 8 * h) * 2, 0, 0));
#pragma unroll
            for (int e = 0; e < 8; ++e) sd = fmaf((float)o[e], (float)gf[kk][e], sd);
        }
        dq = combine_xor32(sd, SumOp());  // rows past N: zeros, never stored
        lq = q < N ? lse[qrow0 + q] * kLog2e : 0.f;
        if (h == 0 && q < N) {
            Lc[qrow0 + q] = lq;
            Dl[qrow0 + q] = dq;
        }
    }
    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};

    uint32_t src[LPW];
#pragma unroll
    for (int u = 0; u < LPW; ++u) src[u] = TK::src_offset((wave + u * NW) * 64 + lane);
    auto issue = [&](auto bc, int kt) {
        const int kv0 = kt * BC;
        const uint32_t left = (uint32_t)(N - kv0) * D * 2;
        const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + kvbase + (size_t)kv0 * D, left);
        const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + kvbase + (size_t)kv0 * D, left);
#pragma unroll
        for (int u = 0; u < LPW; ++u) {
            const int i = wave + u * NW;
            if (TK::INST % NW == 0 || i < TK::INST) {
                lds_dma16(krs, (lds_void_t*)(kbuf(bc) + i * 1024), src[u]);
                lds_dma16(vrs, (lds_void_t*)(vbuf(bc) + i * 1024), src[u]);
            }
        }
    };

    const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
    const int ntiles = (kv_end + BC - 1) / BC;
    const int wt = CAUSAL ? min(ntiles, (qw0 + 31) / BC + 1) : ntiles;

    auto compute = [&](auto bc, int kt) {
        if (kt >= wt) return;
        const char* kt_l = kbuf(bc);
        const char* vt_l = vbuf(bc);
        const int kv0 = kt * BC;
        f32x16 s[2], dp[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            s[mt] = f32x16{};
            dp[mt] = f32x16{};
        }
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                s[mt] = mfma(rows_a<TK::P>(kt_l, 32 * mt, 16 * kk, j, h), qf[kk], s[mt]);
                dp[mt] = mfma(rows_a<TK::P>(vt_l, 32 * mt, 16 * kk, j, h), gf[kk], dp[mt]);
            }
        // Scheduling pipelines for this block and for dQ below keep the LDS
        // operand reads four products ahead (+2% on the backward).
        {
            constexpr int NM = 4 * (D / 16);  // products, one LDS read each
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int u = 0; u < NM - 4; ++u) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
        // Register r of half h of tile mt holds key kv0 + 32 mt + 16 (r / 8) + 8 h + r % 8.
        const bool need_mask = (kv0 + BC > N) || (CAUSAL && kv0 + BC - 1 > qw0);
        bf16x8 sb[BC / 16];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            f32x16 ds;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float pv = exp2_hw(fmaf(s[mt][r], c, -lq));
                if (need_mask) {
                    const int kidx = kv0 + 32 * mt + 16 * (r >> 3) + 8 * h + (r & 7);
                    if (kidx >= N || (CAUSAL && kidx > q)) pv = 0.f;
                }
                ds[r] = pv * (dp[mt][r] - dq);
            }
            sb[2 * mt] = half_bf16(ds, 0);
            sb[2 * mt + 1] = half_bf16(ds, 1);
        }
#pragma unroll
        for (int ks = 0; ks < BC / 16; ++ks)
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                acc[dt] = mfma(cols_a<TK::P>(kt_l, 16 * ks, 32 * dt, lane), sb[ks], acc[dt]);
        {
            constexpr int NM = (BC / 16) * (D / 32);  // products, two LDS reads each
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
            for (int u = 0; u < NM - 4; ++u) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
    };

    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    int kt0 = 0, kt1 = ntiles;  // this workgroup's key tiles
    if constexpr (SPLIT) {
        const int per = (ntiles + nsplit - 1) / nsplit;
        kt0 = min(ntiles, sp * per);
        kt1 = min(ntiles, kt0 + per);
    }
    if (kt1 > kt0) {
        issue(B0{}, kt0);
        __syncthreads();
        for (int kt = kt0; kt < kt1; kt += 2) {
            if (kt + 1 < kt1) issue(B1{}, kt + 1);
            compute(B0{}, kt);
            __syncthreads();
            if (kt + 1 >= kt1) break;
            if (kt + 2 < kt1) issue(B0{}, kt + 2);
            compute(B1{}, kt + 1);
            __syncthreads();
        }
    }
    if constexpr (SPLIT) {
        // Partials [nsplit][BH][N][D] of dQ^T (scale not applied); an empty
        // range writes zeros.
        const size_t slice = (size_t)N * D;
        store_rows_f32<D>(acc, make_rsrc(part + ((size_t)sp * BH + bh) * slice, (uint32_t)slice * 4),
                          qw0, lane);
        return;
    }
    // dQ leaves through LDS: the wave's half of one of the four K/V tile
    // buffers (waves 2b, 2b + 1 share buffer b; each holds 2 x 32 rows of
    // pitch D + 8), which no wave reads any more.
    __syncthreads();
    char* const ost = (wave < 2 ? kb0 : wave < 4 ? kb1 : wave < 6 ? vb0 : vb1) + (wave & 1) * (32 * (D + 8) * 2);
    store_tile_rows<D>(acc, scale, ost, make_rsrc(dQ + base, slice_b), qw0, lane);
}

// Workgroups of 8 waves (256 keys or queries) while that still gives one per
// CU (256) or more; smaller problems take workgroups of 4 or 2 waves so that
// the grid covers more of the chip.
constexpr long long kCUs = 256;

// N is the sequence length, or with cu (packed sequences) the longest one.
// Dynamic LDS of attn_bwd_dkdv_kernel<D, NW>: the V block for 8 waves.
template <int D, int NW>
constexpr unsigned dkdv_dynamic_lds() { return NW == 8 ? (unsigned)Tile<D, NW * 32>::BYTES : 0u; }

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_dkdv(const __bf16* q, const __bf16* k, const __bf16* v, const __bf16* g,
                       const float* Lc, const float* Dl, void* dK, void* dV, int B, int H,
                       int Hkv, int N, float scale, const int* cu, int total, hipStream_t stream)
{
    const int BHkv = B * Hkv;
    auto go = [&](auto nwc) {
        constexpr int NW = decltype(nwc)::value;
        const int nkb = (N + NW * 32 - 1) / (NW * 32);
        attn_bwd_dkdv_kernel<D, NW, CAUSAL, VARLEN><<<dim3((unsigned)(nkb * BHkv)), dim3(NW * 64),
                                                      dkdv_dynamic_lds<D, NW>(), stream>>>(
            q, k, v, g, Lc, Dl, static_cast<__bf16*>(dK), static_cast<__bf16*>(dV), N, BHkv, H, Hkv,
            scale, cu, total, nullptr, 1);
        return hipGetLastError();
    };
    if ((long long)((N + 255) / 256) * BHkv >= kCUs) return go(std::integral_constant<int, 8>{});
    if ((long long)((N + 127) / 128) * BHkv >= kCUs) return go(std::integral_constant<int, 4>{});
    return go(std::integral_constant<int, 2>{});
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_dq(const __bf16* q, const __bf16* k, const __bf16* v, const __bf16* g,
                     const __bf16* o, const float* lse, float* Lc, float* Dl, void* dQ, int B,
                     int H, int Hkv, int N, float scale, const int* cu, int total,
                     hipStream_t stream)
{
    const int BH = B * H;
    auto go = [&](auto nwc) {
        constexpr int NW = decltype(nwc)::value;
        const int nqb = (N + NW * 32 - 1) / (NW * 32);
        attn_bwd_dq_kernel<D, NW, CAUSAL, VARLEN><<<dim3((unsigned)(nqb * BH)), dim3(NW * 64), 0, stream>>>(
            q, k, v, g, o, lse, Lc, Dl, static_cast<__bf16*>(dQ), N, BH, nqb, H, Hkv, scale, cu,
            total, nullptr, 1);
        return hipGetLastError();
    };
    if ((long long)((N + 255) / 256) * BH >= kCUs) return go(std::integral_constant<int, 8>{});
    if ((long long)((N + 127) / 128) * BH >= kCUs) return go(std::integral_constant<int, 4>{});
    return go(std::integral_constant<int, 2>{});
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                      const float* lse, void* dQ, void* dK, void* dV, int B, int H, int Hkv, int N,
                      float scale, float* Dl, float* Lc, const int* cu, int total,
                      hipStream_t stream)
{
    const __bf16* q = static_cast<const __bf16*>(Q);
    const __bf16* k = static_cast<const __bf16*>(K);
    const __bf16* v = static_cast<const __bf16*>(V);
    const __bf16* g = static_cast<const __bf16*>(dO);
    // dQ first: its workgroups also form the row statistics (D and L log2 e
    // of every query row of a sequence), which the dK/dV kernel reads.
    if (const hipError_t e = launch_dq<D, CAUSAL, VARLEN>(q, k, v, g, static_cast<const __bf16*>(O),
                                                          lse, Lc, Dl, dQ, B, H, Hkv, N, scale, cu,
                                                          total, stream);
        e != hipSuccess)
        return e;
    return launch_dkdv<D, CAUSAL, VARLEN>(q, k, v, g, Lc, Dl, dK, dV, B, H, Hkv, N, scale, cu, total,
                                          stream);
}

// Split backward (dense): the dK/dV workgroups divide their query tiles, the
// dQ workgroups their key tiles, into nsplit ranges; fp32 partials in part
// ([2][nsplit][B Hkv][N][D] for dK and dV, then [nsplit][B H][N][D] for dQ),
// summed by attn_bwd_sum_kernel.  8-wave workgroups throughout.
template <int D, bool CAUSAL>
hipError_t launch_bwd_split(const void* Q, const void* K, const void* V, const void* O,
                            const void* dO, const float* lse, void* dQ, void* dK, void* dV, int B,
                            int H, int Hkv, int N, float scale, int nsplit, float* Dl, float* Lc,
                            float* part, hipStream_t stream)
{
    const int BH = B * H, BHkv = B * Hkv;
    const __bf16* q = static_cast<const __bf16*>(Q);
    const __bf16* k = static_cast<const __bf16*>(K);
    const __bf16* v = static_cast<const __bf16*>(V);
    const __bf16* g = static_cast<const __bf16*>(dO);
    const long long rows = (long long)BH * N;
    {
        constexpr int RPB = 256 / (D / 8);
        const long long need = (rows + RPB - 1) / RPB;
        attn_bwd_delta_kernel<D><<<dim3((unsigned)(need < 65536 ? need : 65536)), dim3(256), 0, stream>>>(
            static_cast<const __bf16*>(O), g, lse, Dl, Lc, rows);
        if (const hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    const int nb = (N + 255) / 256;
    float* const pkv = part;
    float* const pq = part + (size_t)2 * nsplit * BHkv * N * D;
    attn_bwd_dkdv_kernel<D, 8, CAUSAL, false, true><<<dim3((unsigned)(nb * nsplit * BHkv)), dim3(512),
                                                      dkdv_dynamic_lds<D, 8>(), stream>>>(
        q, k, v, g, Lc, Dl, nullptr, nullptr, N, BHkv, H, Hkv, scale, nullptr, 0, pkv, nsplit);
    if (const hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    attn_bwd_dq_kernel<D, 8, CAUSAL, false, true><<<dim3((unsigned)(nb * nsplit * BH)), dim3(512), 0, stream>>>(
        q, k, v, g, nullptr, nullptr, Lc, Dl, nullptr, N, BH, nb, H, Hkv, scale, nullptr, 0, pq, nsplit);
    if (const hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    const long long kv8 = (long long)BHkv * N * D / 8, q8 = rows * D / 8;
    const long long kvs = (long long)BHkv * N * D, qs = rows * D;
    const SumSeg sk{pkv, static_cast<__bf16*>(dK), kv8, kvs, scale};
    const SumSeg sv{pkv + (size_t)nsplit * kvs, static_cast<__bf16*>(dV), kv8, kvs, 1.0f};
    const SumSeg sq{pq, static_cast<__bf16*>(dQ), q8, qs, scale};
    const long long blocks = (2 * kv8 + q8 + 255) / 256;
    attn_bwd_sum_kernel<<<dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, stream>>>(sk, sv, sq, nsplit);
    return hipGetLastError();
}

}  // namespace

int attn_bwd_split_auto(int BH, int N, int d, bool causal)
{
    // BH counts (batch, key/value head) slices: the dK/dV grid's.  Measured
    // over [1..2, 1..16, 2048..32768, d] (both masks, Hkv = H): no split
    // while 8-wave workgroups of 256 rows cover the 256 compute units, nor
    // for rows of 2048 or fewer once the unsplit launch's 4-wave workgroups
    // do; otherwise enough ranges for about one 8-wave workgroup per CU,
    // twice that under the mask (its ranges are unequal), while each range
    // keeps at least 512 rows of the loop it divides (256 at d = 64, whose
    // partials cost half the bytes), and at most 16.  With grouped queries
    // (measured on [2, 16/4, 2048, 128], [1, 32/1..8, 4096, 128],
    // [2, 16/2, 4096, 64], [1, 32/4, 8192, 128]) this count is the best of
    // the sweep or within 6% of it, and 1.3-4x the unsplit call.
    const long long w = (long long)((N + 255) / 256) * BH;
    if (w >= kCUs || N <= 256) return 1;
    if (N <= 2048 && (long long)((N + 127) / 128) * BH >= kCUs) return 1;
    long long n = (kCUs + w - 1) / w;
    if (causal) n *= 2;
    long long cap = N / (d == 64 ? 256 : 512);
    if (cap > 16) cap = 16;
    if (n > cap) n = cap;
    return n < 2 ? 1 : (int)n;
}

hipError_t launch_attn_bwd_bf16_split(const void* Q, const void* K, const void* V, const void* O,
                                      const void* dO, const float* lse, void* dQ, void* dK,
                                      void* dV, int B, int H, int Hkv, int N, int d, float scale,
                                      bool causal, int nsplit, float* Dl, float* Lc, float* part,
                                      hipStream_t stream)
{
    if (d == 64)
        return causal ? launch_bwd_split<64, true>(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Hkv, N, scale, nsplit, Dl, Lc, part, stream)
                      : launch_bwd_split<64, false>(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Hkv, N, scale, nsplit, Dl, Lc, part, stream);
    return causal ? launch_bwd_split<128, true>(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Hkv, N, scale, nsplit, Dl, Lc, part, stream)
                  : launch_bwd_split<128, false>(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Hkv, N, scale, nsplit, Dl, Lc, part, stream);
}

hipError_t launch_attn_bwd_bf16(const void* Q, const void* K, const void* V, const void* O,
                                const void* dO, const float* lse, void* dQ, void* dK, void* dV,
                                int B, int H, int Hkv, int N, int d, float scale, bool causal,
                                float* Dl, float* Lc, hipStream_t stream)
{
    if (d == 64)
        return causal ? launch_bwd<64, true, false>(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Hkv, N, scale, Dl, Lc, nullptr, 0, stream)
                      : launch_bwd<64, false, false>(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Hkv, N, scale, Dl, Lc, nullptr, 0, stream);
    return causal ? launch_bwd<128, true, false>(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Hkv, N, scale, Dl, Lc, nullptr, 0, stream)
                  : launch_bwd<128, false, false>(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Hkv, N, scale, Dl, Lc, nullptr, 0, stream);
}

hipError_t launch_attn_bwd_bf16_varlen(const void* Q, const void* K, const void* V, const void* O,
                                       const void* dO, const float* lse, void* dQ, void* dK,
                                       void* dV, const int* cu, int B, int H, int Hkv, int total,
                                       int max_seqlen, int d, float scale, bool causal, float* Dl,
                                       float* Lc, hipStream_t stream)
{
    if (d == 64)
        return causal ? launch_bwd<64, true, true>(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Hkv, max_seqlen, scale, Dl, Lc, cu, total, stream)
                      : launch_bwd<64, false, true>(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Hkv, max_seqlen, scale, Dl, Lc, cu, total, stream);
    return causal ? launch_bwd<128, true, true>(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Hkv, max_seqlen, scale, Dl, Lc, cu, total, stream)
                  : launch_bwd<128, false, true>(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Hkv, max_seqlen, scale, Dl, Lc, cu, total, stream);
}

}  // namespace osm
