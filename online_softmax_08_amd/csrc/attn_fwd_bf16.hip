// attn_fwd_bf16.hip -- fused exact attention forward for bf16 Q, K, V on the
// gfx950 bf16 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation):
// O = softmax(scale Q K^T) V written as bf16, plus the per-row natural-log
// logsumexp in fp32.  The N x N score and probability matrices exist only as
// register tiles and never reach HBM.
//
// Method: the tiled online softmax of "Lesson 22: why softmax is hard to make
// efficient, and how FlashAttention reduces memory traffic", sections 21-24
// and 32 (the merge rule of section 22, the causal tile skipping of section
// 34), with the refinements of "Moving less: four generations of
// FlashAttention": the output stays unnormalised until the end (3.2), the
// grid runs over query-row blocks (3.3), query rows are split across waves so
// waves never exchange partial outputs (3.4), and the running maximum used as
// the exponent reference is only moved when it has grown by more than a fixed
// margin (5.4).  lse = m + ln l is the statistic of section 2.4.
//
// gfx950 design:
//  * Work: one workgroup per (batch*head, block of BR query rows); a wave owns
//    QT x 32 query rows.  Under the causal mask workgroups are issued longest
//    first.  Consecutive workgroup ids walk the batch*head index, so when
//    batch*head is a multiple of 8 all query blocks of one head land on the
//    same XCD (ids are dealt round-robin over the 8 XCDs) and share its L2.
//  * Global memory goes through buffer resources: rows past N read as zero
//    and stores past N are dropped by the hardware range check, so ragged
//    tails need no branches.
//  * Q stays in VGPRs as the B operand of S^T = K Q^T for the whole kernel.
//  * K and V tiles of 64 keys move HBM -> LDS by buffer loads that write LDS
//    directly (no VGPR staging), double-buffered: tile j+1 is in flight while
//    tile j is computed, one barrier per tile.  Both tiles stay row-major;
//    each wave load instruction fills 1 KiB of LDS, and every lane picks the
//    global 16 bytes that belong at its LDS position (in the padded layout,
//    lanes landing on row padding fetch a harmless duplicate).  The tile loop
//    is unrolled by two, so every LDS read address is a loop-invariant
//    register plus an immediate.
//  * S^T puts one query per lane (lane % 32) and 16 keys per lane in each
//    32x32 accumulator, so the row max and row sum are in-lane reductions plus
//    one v_permlane32_swap; the row sum is kept per lane and the halves are
//    added once at the end.  Lane i reads K row swap_bits23(i) of each
//    32-key group (attn_fwd_bf16_kernel stores the rows in that order,
//    attn_fwd_bf16_pp_kernel permutes the read address), so that each group
//    of 8 accumulator registers holds 8 consecutive keys: the bf16
//    probabilities are, register for register, the B operand of
//    O^T += V^T P^T.
//  * The V^T A operand (8 consecutive keys of one column per lane) comes from
//    the row-major V tile through ds_read_b64_tr_b16, the gfx950 transposing
//    LDS read: in each group of 16 lanes, lane 4a + b receives element b of
//    the 8-byte reads of lanes a, a + 4, a + 8 and a + 12.
//  * In attn_fwd_bf16_kernel, row pitches (K: d + 8, V: d + 32 elements)
//    make both LDS read patterns bank-conflict free; attn_fwd_bf16_pp_kernel
//    keeps the tiles unpadded and permutes 16-byte chunks (K) or 64-byte
//    blocks (V) inside each row by an XOR with row bits instead, which needs
//    no padding chunks and so five fewer tile loads per step.  Either way:
//    a 16-byte row read serves 16 lanes per cycle, so its 16 rows must hit
//    16 different 16-byte bank groups (pitch d + 8 puts rows 16 bytes apart
//    modulo 256; the XOR sends chunk c of row r to slot c ^ r); the 8-byte
//    transposed read serves 32 lanes per cycle, which take 64 contiguous
//    bytes from each of 4 rows, so those rows must start 64 bytes apart
//    modulo 256, which a pitch of d + 32 gives (d + 16 leaves 2-way
//    conflicts), or sit in different 64-byte block slots, which the XOR of
//    the row's low bits into the block index gives.
//  * p = 2^(s c - m c) with c = scale log2(e): one FMA and one v_exp_f32 per
//    score.  The reference m is not moved on every new maximum: in
//    attn_fwd_bf16_kernel it moves when some row of the wave has a tile
//    maximum more than 8 (in log2 units) above it, so every p <= 2^8; in
//    attn_fwd_bf16_pp_kernel the tile's probabilities are computed first and
//    the reference moves only when some lane's partial row sum exceeds 2^16
//    (which bounds every p), so the common tile needs no row maximum.  Either
//    way the result is the same exact quantity: l and the accumulators share
//    the reference.
//  * Two schedules share these pieces.  attn_fwd_bf16_kernel runs each tile
//    as S^T, softmax, P V in every wave; the two waves of a SIMD then mostly
//    use the matrix core and the vector unit at the same time and wait for
//    each other.  It serves the smaller grids (128- and 64-row workgroups
//    whose key loop is split over two wave groups).
//    attn_fwd_bf16_pp_kernel (8-wave workgroups of 256 rows, both masks, and
//    the split-KV partial pass) staggers the two waves of each SIMD by half
//    a tile step, so that one issues only MFMAs while the other runs the
//    softmax.
//  * The output tile of each wave leaves through LDS as whole rows
//    (store_tile_rows): the accumulators hold O^T, whose direct stores would
//    write 16-byte pieces of 32 rows per instruction.

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace osm {
namespace {

constexpr float kRescaleLog2 = 8.0f;  // move the reference beyond 2^8 growth
// Phase-staggered kernel: keep the reference while every lane's partial row
// sum of a tile stays within 2^16 (so every p <= 2^16, far inside bf16 and
// fp32 range).
constexpr float kSumLimit = 65536.0f;

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// Inside a 32-key MFMA tile, A-operand row i (read by lane i) is key
// swap_bits23(i) (bits 2 and 3 exchanged; the map is its own inverse): the
// plain kernel stores the keys in that order in LDS, the phase-staggered kernel
// stores them in key order and lets lane i read row swap_bits23(i).  The 32x32
// accumulator layout (row 8g + 4h + t lands in register 4g + t of lane half h)
// then leaves key 16*(r/8) + 8*h + r%8 in register r of half h.
__device__ __forceinline__ int swap_bits23(int i)
{
    return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    // Raw buffer (stride 0): loads at offsets >= bytes return 0, stores there
    // are dropped.  0x00020000 selects 32-bit data format for untyped access.
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// 16 bytes per lane from a buffer straight into LDS: lane L of the wave reads
// buffer offset voff + OFF and writes dst + OFF + 16 L.  The instruction's
// immediate offset OFF moves both addresses, and the range check applies to
// voff + OFF (measured: lanes whose sum passes the range read zero), so loads
// that share one LDS base (M0) can still fill different LDS blocks.  The
// builtin sits in a device-only body because clang's host pass otherwise drops
// the launch stubs of kernels that contain it.
template <int OFF = 0>
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, lds_void_t* dst, uint32_t voff)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff, 0, OFF, 0);
#endif
}

// Where the (batch, head) slice of a workgroup lives: dense tensors
// [B*H][N][D] (lse [B*H][N]), or packed variable-length sequences
// [H][total][D] (lse [H][total]) whose batch b holds rows cu[b] .. cu[b+1]-1
// of every head.  K and V have Hkv heads (Hkv divides H; query head h reads
// key/value head h / (H / Hkv)).  Packed lengths are clamped to [0, Nmax]
// and to the packed extent, so a malformed cu cannot move an access outside
// the tensors.
struct Slice {
    size_t base;    // element offset of row 0 of the slice in Q and O
    size_t kvbase;  // element offset of row 0 of its key/value slice in K and V
    size_t lbase;   // element offset of row 0 in lse
    int n;          // rows (queries = keys) of the slice
};

template <int D, bool VARLEN>
__device__ __forceinline__ Slice slice_of(int bh, int Nmax, int H, int Hkv, const int* cu, int total)
{
    const int b = bh / H, hh = bh - b * H;
    const int hkv = hh / (H / Hkv);
    if constexpr (!VARLEN) {
        const size_t kvbh = (size_t)b * Hkv + hkv;
        return {(size_t)bh * Nmax * D, kvbh * Nmax * D, (size_t)bh * Nmax, Nmax};
    } else {
        const int start = min(max(__builtin_amdgcn_readfirstlane(cu[b]), 0), total);
        const int end = min(max(__builtin_amdgcn_readfirstlane(cu[b + 1]), start), total);
        const size_t row0 = (size_t)hh * total + start;
        return {row0 * D, ((size_t)hkv * total + start) * D, row0, min(end - start, Nmax)};
    }
}

// LDS staging region of a wave's output tile (store_tile_rows): the wave's
// half of one of the four key/value tile buffers (waves 2b, 2b + 1 share
// buffer b), each of which holds at least 2 x 32 x (D + 8) x 2 bytes.  The
// caller makes sure no wave still reads the tiles.
template <int D>
__device__ __forceinline__ char* out_stage(int wave, char* k0, char* k1, char* v0, char* v1)
{
    char* const b = wave < 2 ? k0 : wave < 4 ? k1 : wave < 6 ? v0 : v1;
    return b + (wave & 1) * (32 * (D + 8) * 2);
}

// KS > 1 splits the key tiles of a workgroup over KS groups of NW / KS waves
// that share the same query rows (see attn_fwd_bf16_kernel).
template <int D, int QT, int NW, int BC_, int KS_ = 1>
struct Cfg {
    static constexpr int BC = BC_;            // keys per tile
    static constexpr int KS = KS_;            // key groups
    static constexpr int NWR = NW / KS;       // waves per key group
    static constexpr int T = NW * 64;         // threads per workgroup
    static constexpr int BR = NWR * QT * 32;  // query rows per workgroup
    static constexpr int KP = D + 8;          // K row pitch in LDS (elements)
    static constexpr int VP = D + 32;         // V row pitch in LDS (elements)
    static constexpr int KCPR = KP / 8;       // 16-byte chunks per K row (last is padding)
    static constexpr int VCPR = VP / 8;       // 16-byte chunks per V row (last four padding)
    static constexpr int KTILE_B = BC * KP * 2;
    static constexpr int VTILE_B = BC * VP * 2;
    static constexpr int KINST = KTILE_B / 1024;  // 1 KiB wave loads per K tile
    static constexpr int VINST = VTILE_B / 1024;
    static constexpr int KBUF_INST = KS * KINST;      // loads per K buffer (KS tiles)
    static constexpr int VBUF_INST = KS * VINST;
    static constexpr int KPW = (KBUF_INST + NW - 1) / NW;  // K loads issued per wave
    static constexpr int VPW = (VBUF_INST + NW - 1) / NW;
    static constexpr int LDS_B2 = 2 * KS * (KTILE_B + VTILE_B);  // 2 K + 2 V buffers
    static_assert(KTILE_B % 1024 == 0 && VTILE_B % 1024 == 0, "tiles are whole wave loads");
    static_assert(NW % KS == 0, "key groups of equal size");
};

// With KS = 2 the workgroup's waves form two key groups over the same query
// rows: wave w (group w / (NW / 2)) computes the even key tiles, wave
// w + NW / 2 the odd ones, from one LDS buffer that holds both tiles of a
// pair.  At the end the odd group hands its reference, row sums and output
// accumulators to the even group through LDS, which merges them by the rule
// of Lesson 22, section 22 (rescale both to the larger reference and add)
// and writes O and lse.  A small grid then keeps twice as many waves busy,
// each with half of the key loop, and needs no workspace.
template <int D, int QT, int NW, int WPE, int BC, bool CAUSAL, bool VARLEN, int KS = 1>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
attn_fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                     const __bf16* __restrict__ V, __bf16* __restrict__ O,
                     float* __restrict__ lse, int Nmax, int BH, int nqt, float scale,
                     const int* __restrict__ cu, int H, int Hkv, int total)
{
    static_assert(KS == 1 || KS == 2, "one or two key groups");
    using C = Cfg<D, QT, NW, BC, KS>;
    static_assert(NW <= 8 && C::KTILE_B >= 2 * 32 * (D + 8) * 2, "output staging fits the tile buffers");
    constexpr int NMT = BC / 32;  // 32-key MFMA tiles per key tile
    // Separate LDS objects (not slices of one array): the compiler can then
    // prove that the DMA filling one buffer does not alias reads of the
    // other, and does not stall those reads on the DMA's completion.  (Below,
    // two buffers may share the dynamic array only when they are filled
    // together and read together.)
    __shared__ __attribute__((aligned(1024))) char kbuf0[KS * C::KTILE_B];
    __shared__ __attribute__((aligned(1024))) char ksta1[(D == 128 && KS == 2) ? 16 : KS * C::KTILE_B];
    __shared__ __attribute__((aligned(1024))) char vbuf0[KS * C::VTILE_B];
    // With two key groups the four buffers take 84 KiB at D = 64 and 148 KiB
    // at D = 128, and the compiler, which schedules for the static LDS it
    // sees, then plans for one workgroup per CU: the 4-wave kernels got 176
    // and 292 registers and slower loops.  So part of the buffers lives in
    // dynamic LDS (passed at launch): at D = 64 the second V buffer, at
    // D = 128 the second K and V buffers together (always filled together
    // and read together, so no load into one part of that object is in
    // flight while the other part is read).  Static LDS 60 and
    // 74 KiB, 135 and 219 registers, same output bit for bit: +12-15% on
    // [2, 8, 1024, 64] (both masks) and [1, 8, 2048, 64], +11-13% on
    // [1, 8, 2048, 128] causal, [2, 4, 1000, 128] and [1, 2, 8192, 128]
    // causal; the 8-wave workgroups unchanged.
    constexpr bool VDYN = D == 64 && KS == 2, KVDYN = D == 128 && KS == 2;
    extern __shared__ __attribute__((aligned(1024))) char vdyn[];
    __shared__ __attribute__((aligned(1024))) char vsta1[(VDYN || KVDYN) ? 16 : KS * C::VTILE_B];
    char* const kbuf1 = KVDYN ? vdyn : ksta1;
    char* const vbuf1 = VDYN ? vdyn : KVDYN ? vdyn + KS * C::KTILE_B : vsta1;
    auto kbuf = [&](auto bufc) -> char* { if constexpr (decltype(bufc)::value == 0) return kbuf0; else return kbuf1; };
    auto vbuf = [&](auto bufc) -> char* { if constexpr (decltype(bufc)::value == 0) return vbuf0; else return vbuf1; };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int rw = wave % C::NWR, kg = wave / C::NWR;            // row wave, key group
    const int j = lane & 31, h = lane >> 5;
    const int t = blockIdx.x / BH, bh = blockIdx.x - t * BH;
    const int qt = CAUSAL ? nqt - 1 - t : t;
    const int q0 = qt * C::BR;
    const Slice sl = slice_of<D, VARLEN>(bh, Nmax, H, Hkv, cu, total);
    const int N = sl.n;
    if (VARLEN && q0 >= N) return;  // query block past this sequence (whole workgroup)
    const size_t base = sl.base;
    const uint32_t slice_b = (uint32_t)N * D * 2;
    const int qw0 = q0 + rw * QT * 32;  // first query row of this wave

    // Q as the B operand of S^T = K Q^T: lane (j, h), k-step kk holds
    // Q[row][16 kk + 8 h .. +7] of row qw0 + 32 nt + j (zero past N).
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + base, slice_b);
    bf16x8 qf[QT][D / 16];
#pragma unroll
    for (int nt = 0; nt < QT; ++nt) {
        const int q = qw0 + nt * 32 + j;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            const u32x4 raw = __builtin_amdgcn_raw_buffer_load_b128(
                qrs, (uint32_t)(q * D + kk * 16 + 8 * h) * 2, 0, 0);
            qf[nt][kk] = __builtin_bit_cast(bf16x8, raw);
        }
    }

    f32x16 acc[QT][D / 32];
#pragma unroll
    for (int nt = 0; nt < QT; ++nt)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) acc[nt][dt] = f32x16{};
    float m[QT], l[QT];  // exponent reference (raw score units) and lane's share of the sum
#pragma unroll
    for (int nt = 0; nt < QT; ++nt) {
        m[nt] = kNegInf;
        l[nt] = 0.f;
    }
    const float c = scale * kLog2e;

    // ---- HBM -> LDS tile loads (loop-invariant per-lane source offsets) ----
    // A buffer holds KS consecutive tiles, tile g at byte g * TILE_B.  Wave
    // load i writes LDS chunk positions 64 i .. 64 i + 63 of the buffer; the
    // lane at position p of tile g fetches row p / CPR, column chunk p % CPR
    // (padding chunks re-fetch the row's last real chunk) of that tile.  K
    // rows are permuted inside each 32-row group (swap_bits23); V rows keep
    // key order.
    uint32_t ksrc[C::KPW], vsrc[C::VPW];
#pragma unroll
    for (int u = 0; u < C::KPW; ++u) {
        const int i = wave + u * NW, g = i / C::KINST;
        const int p = (i - g * C::KINST) * 64 + lane;
        const int lrow = p / C::KCPR, ch = min(p % C::KCPR, D / 8 - 1);
        const int row = g * BC + ((lrow & ~31) | swap_bits23(lrow & 31));
        ksrc[u] = (uint32_t)(row * D + ch * 8) * 2;
    }
#pragma unroll
    for (int u = 0; u < C::VPW; ++u) {
        const int i = wave + u * NW, g = i / C::VINST;
        const int p = (i - g * C::VINST) * 64 + lane;
        const int row = g * BC + p / C::VCPR, ch = min(p % C::VCPR, D / 8 - 1);
        vsrc[u] = (uint32_t)(row * D + ch * 8) * 2;
    }
    const __bf16* Kb = K + sl.kvbase;
    const __bf16* Vb = V + sl.kvbase;
    auto issue_k = [&](auto bufc, int kt) {
        const int kv0 = kt * BC;
        const uint32_t left = (uint32_t)(N - kv0) * D * 2;  // bytes of this slice from kv0 on
        const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kb + (size_t)kv0 * D, left);
#pragma unroll
        for (int u = 0; u < C::KPW; ++u) {
            const int i = wave + u * NW;
            if (C::KBUF_INST % NW == 0 || i < C::KBUF_INST)
                lds_dma16(krs, (lds_void_t*)(kbuf(bufc) + i * 1024), ksrc[u]);
        }
    };
    auto issue_v = [&](auto bufc, int kt) {
        const int kv0 = kt * BC;
        const uint32_t left = (uint32_t)(N - kv0) * D * 2;
        const __amdgpu_buffer_rsrc_t vrs = make_rsrc(Vb + (size_t)kv0 * D, left);
#pragma unroll
        for (int u = 0; u < C::VPW; ++u) {
            const int i = wave + u * NW;
            if (C::VBUF_INST % NW == 0 || i < C::VBUF_INST)
                lds_dma16(vrs, (lds_void_t*)(vbuf(bufc) + i * 1024), vsrc[u]);
        }
    };
    auto issue = [&](auto bufc, int kt) {
        issue_k(bufc, kt);
        issue_v(bufc, kt);
    };


    // Per-lane LDS read bases.  K A operand: row j of each 32-row group, half
    // h of each 16-column step.  V^T A operand via the transposing read: in
    // lane group g = lane / 16 the lane 16 g + 4 e + a reads 4 columns
    // (16 (g % 2) + 4 a ..) of key row 8 (g / 2) + e (+ 4 for the second
    // read); lane i of the group then holds column 16 (g % 2) + i for 4 keys.
    // Key group kg reads tile kg of each buffer.
    const int kread = kg * C::KTILE_B + (j * C::KP + 8 * h) * 2;
    const int g16 = lane >> 4, e4 = (lane >> 2) & 3, a4 = lane & 3;
    const int vread = kg * C::VTILE_B + ((8 * (g16 >> 1) + e4) * C::VP + 16 * (g16 & 1) + 4 * a4) * 2;

    // S^T = K Q^T of the K tile in LDS buffer KB, two 32-key MFMA tiles.
    auto qk = [&](auto kbc, f32x16 (&s)[NMT][QT]) {
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
            for (int nt = 0; nt < QT; ++nt) s[mt][nt] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                    kbuf(kbc) + kread + (mt * 32 * C::KP + kk * 16) * 2);
#pragma unroll
                for (int nt = 0; nt < QT; ++nt)
                    s[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[nt][kk], s[mt][nt], 0, 0, 0);
            }
        }
    };

    // Mask (diagonal / tail tiles only), tile row maxima, and the rare move of
    // the exponent reference.
    auto stats = [&](f32x16 (&s)[NMT][QT], int kv0) {
        const bool need_mask = (kv0 + BC > N) || (CAUSAL && kv0 + BC - 1 > qw0);
        float mx[QT];
#pragma unroll
        for (int nt = 0; nt < QT; ++nt) {
            if (need_mask) {
                const int q = qw0 + nt * 32 + j;
                // Keys visible to query q in this tile: kv0 .. lim - 1.
                const int lim = CAUSAL ? min(N, q + 1) : N;
#pragma unroll
                for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kv0 + mt * 32 + 16 * (r >> 3) + 8 * h + (r & 7);
                        if (key >= lim) s[mt][nt][r] = kNegInf;
                    }
            }
            float v = kNegInf;
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
                for (int r = 0; r < 16; r += 2) v = fmaxf(v, fmaxf(s[mt][nt][r], s[mt][nt][r + 1]));
            mx[nt] = combine_xor32(v, MaxOp());
        }
        bool grow = false;
#pragma unroll
        for (int nt = 0; nt < QT; ++nt) grow |= (mx[nt] - m[nt]) * c > kRescaleLog2;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
            for (int nt = 0; nt < QT; ++nt) {
                const float m_new = fmaxf(m[nt], mx[nt]);
                // Tile 0 holds key 0, visible to every row, so m_new is finite;
                // an empty history (m = -inf, l = acc = 0) gets factor 0.  The
                // guard keeps -inf - -inf out of exp2 all the same.
                const float alpha = (m_new == kNegInf) ? 1.f : exp2_hw((m[nt] - m_new) * c);
                l[nt] *= alpha;
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) acc[nt][dt] *= alpha;
                m[nt] = m_new;
            }
        }
    };

    // Probabilities of the scores in s (bf16 B fragments, row sums into l).
    auto probs = [&](f32x16 (&s)[NMT][QT], bf16x8 (&pf)[BC / 16][QT]) {
#pragma unroll
        for (int nt = 0; nt < QT; ++nt) {
            // The tiles of the odd key group can lie wholly in a row's
            // future; that row keeps m = -inf and all its p must come out 0,
            // not NaN.
            const float mc = (KS > 1 && m[nt] == kNegInf) ? 0.f : m[nt] * c;
            float ps[4];  // four partial sums, seeded by the first four p
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = exp2_hw(fmaf(s[mt][nt][r], c, -mc));
                    s[mt][nt][r] = p;
                    if (mt == 0 && r < 4)
                        ps[r] = p;
                    else
                        ps[r & 3] += p;
                }
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const f32x16& sv = s[mt][nt];
                    const f32x8 p8 = half ? __builtin_shufflevector(sv, sv, 8, 9, 10, 11, 12, 13, 14, 15)
                                          : __builtin_shufflevector(sv, sv, 0, 1, 2, 3, 4, 5, 6, 7);
                    pf[2 * mt + half][nt] = __builtin_convertvector(p8, bf16x8);
                }
            }
            l[nt] += (ps[0] + ps[1]) + (ps[2] + ps[3]);
        }
    };

    // O^T += V^T P^T over four 16-key steps, V from LDS buffer VB.
    auto pv = [&](auto vbc, bf16x8 (&pf)[BC / 16][QT]) {
#pragma unroll
        for (int ks = 0; ks < BC / 16; ++ks) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                const char* vp = vbuf(vbc) + vread + (16 * ks * C::VP + 32 * dt) * 2;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)vp);
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vp + 4 * C::VP * 2));
                const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                for (int nt = 0; nt < QT; ++nt)
                    acc[nt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[ks][nt], acc[nt][dt], 0, 0, 0);
            }
        }
    };

    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    const int kv_end = CAUSAL ? min(N, q0 + C::BR) : N;
    const int ntiles = (kv_end + BC - 1) / BC;
    // Key tiles of this workgroup: t_lo .. t_hi - 1.
    const int t_lo = 0, t_hi = ntiles;
    // Tiles this wave computes: t_lo .. wt - 1 (under the causal mask the
    // later tiles of the workgroup lie wholly in this wave's future).
    const int wt = CAUSAL ? min(t_hi, (qw0 + QT * 32 - 1) / BC + 1) : t_hi;

    // One tile: S^T, statistics and probabilities, P V.  The two products
    // get scheduling pipelines that keep their LDS operand reads four
    // products ahead (neutral to +4% on the grids this kernel serves).
    auto compute = [&](auto bufc, int kt) {
        if (kt >= wt) return;
        f32x16 s[NMT][QT];
        qk(bufc, s);
        {
            constexpr int NR = (D / 16) * NMT;  // K reads, QT products each
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // LDS reads
#pragma unroll
            for (int u = 0; u < NR - 4; ++u) {
                __builtin_amdgcn_sched_group_barrier(0x008, QT, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4 * QT, 0);
        }
        stats(s, kt * BC);
        bf16x8 pf[BC / 16][QT];
        probs(s, pf);
        pv(bufc, pf);
        {
            constexpr int NV = (BC / 16) * (D / 32);  // V operands, 2 reads each
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
            for (int u = 0; u < NV - 4; ++u) {
                __builtin_amdgcn_sched_group_barrier(0x008, QT, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4 * QT, 0);
        }
    };
    // A buffer holds tiles kt .. kt + KS - 1; key group kg computes kt + kg.
    issue(B0{}, t_lo);
    __syncthreads();  // waits for the tile loads (vmcnt) before publishing
    for (int kt = t_lo; kt < t_hi; kt += 2 * KS) {
        // compute buffer 0 while tiles kt + KS .. stream into buffer 1
        if (kt + KS < t_hi) issue(B1{}, kt + KS);
        compute(B0{}, kt + kg);
        __syncthreads();
        if (kt + KS >= t_hi) break;
        // compute buffer 1 while tiles kt + 2 KS .. stream into buffer 0
        if (kt + 2 * KS < t_hi) issue(B0{}, kt + 2 * KS);
        compute(B1{}, kt + KS + kg);
        __syncthreads();
    }

    // ---- epilogue: O = acc / l in bf16 (rows past N dropped), lse = m scale + ln l ----
    const __amdgpu_buffer_rsrc_t ors = make_rsrc(O + base, slice_b);
    const __amdgpu_buffer_rsrc_t lrs = make_rsrc(lse + sl.lbase, (uint32_t)N * 4);
    __syncthreads();  // every wave is done with the tile buffers
    if constexpr (KS > 1) {
        // The odd group's (m, l, acc), lane by lane, through the V buffers:
        // row waves 0-1 use vbuf0, 2-3 vbuf1, element e of lane L of the
        // buffer's row wave r at float (r E + e) 64 + L.  The even group
        // includes tile 0, whose key 0 every row sees, so its m is finite;
        // an odd group that saw no key has m = -inf and weight 0.
        constexpr int E = QT * (2 + 16 * (D / 32));
        static_assert(C::NWR <= 4 && 2 * E * 64 * 4 <= KS * C::VTILE_B, "exchange fits the V buffers");
        float* const xch = reinterpret_cast<float*>(rw < 2 ? vbuf0 : vbuf1) + (rw & 1) * E * 64 + lane;
        if (kg == 1) {
#pragma unroll
            for (int nt = 0; nt < QT; ++nt) {
                float* const x = xch + nt * (2 + 16 * (D / 32)) * 64;
                x[0] = m[nt];
                x[64] = l[nt];
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) x[(2 + 16 * dt + r) * 64] = acc[nt][dt][r];
            }
        }
        __syncthreads();
        if (kg == 0) {
#pragma unroll
            for (int nt = 0; nt < QT; ++nt) {
                const float* const x = xch + nt * (2 + 16 * (D / 32)) * 64;
                const float m1 = x[0];
                const float m_new = fmaxf(m[nt], m1);
                const float a0 = exp2_hw((m[nt] - m_new) * c);
                const float a1 = exp2_hw((m1 - m_new) * c);  // 0 for m1 = -inf
                l[nt] = a0 * l[nt] + a1 * x[64];
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[nt][dt][r] = a0 * acc[nt][dt][r] + a1 * x[(2 + 16 * dt + r) * 64];
                m[nt] = m_new;
            }
        }
        __syncthreads();  // the exchange area is read before the output staging
    }
    if (kg == 0) {
        char* const ost = out_stage<D>(rw, kbuf0, kbuf1, vbuf0, vbuf1);
#pragma unroll
        for (int nt = 0; nt < QT; ++nt) {
            const float l_tot = combine_xor32(l[nt], SumOp());
            const float inv = 1.0f / l_tot;
            store_tile_rows<D>(acc[nt], inv, ost, ors, qw0 + nt * 32, lane);
            if (h == 0)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m[nt] * scale + logf(l_tot)), lrs,
                                                      (uint32_t)(qw0 + nt * 32 + j) * 4, 0, 0);
        }
    }
}

// Phase-staggered variant: 8 waves of 32 query rows, two per SIMD (waves w
// and w + 4 share one).  Each tile step of a wave is split into a matrix
// phase, P V of the previous tile and S^T = K Q^T of this one, and a vector
// phase, the tile's mask, maxima, reference move and exponentials.  Waves
// 0-3 run their matrix phase while waves 4-7 run their vector phase and vice
// versa: the matrix core of every SIMD is fed by one wave while the vector
// unit serves the other.  One workgroup barrier per tile step (after the
// odd phase) keeps the groups half a step apart; it is also the only one
// the LDS buffers need.  Tile i is read in phases 2i (waves 0-3) and 2i + 1
// (waves 4-7); the loads of K(i + 1) start in phase 2i, those of V(i) in
// phase 2i + 1 (phase 2i at D = 64), and both are waited for before the
// barrier that ends phase 2i + 1.
//
// Merge of the S split partials of one row, four fp32 columns (4 c4 ..
// 4 c4 + 3) per lane, by the merge rule of Lesson 22, section 22: keep the
// largest partial logsumexp M seen so far, scale what was accumulated by
// e^(M_old - M_new) when it grows, and add each partial output with weight
// e^(lse_s - M).  At the end O = sum_s e^(lse_s - M) O_s / sum_s e^(lse_s - M)
// and lse = M + ln sum_s e^(lse_s - M).  Partials with lse_s = -inf are empty
// and skipped without reading their O_s; a row with no non-empty partial
// gets O = 0 and lse = -inf.  Partial s of row `row` sits at s rows + row.
template <int D, class PT>
__device__ __forceinline__ void merge_row(const PT* __restrict__ opart,
                                          const float* __restrict__ lpart, __bf16* __restrict__ O,
                                          float* __restrict__ lse, int S, long long rows,
                                          long long row, int c4)
{
    float M = kNegInf, l = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < S; ++s) {
        const size_t pr = (size_t)s * rows + row;
        const float ls = lpart[pr];
        if (ls == kNegInf) continue;
        f32x4 o;
        if constexpr (std::is_same_v<PT, float>)
            o = *reinterpret_cast<const f32x4*>(opart + pr * D + 4 * c4);
        else
            o = __builtin_convertvector(*reinterpret_cast<const bf16x4*>(opart + pr * D + 4 * c4), f32x4);
        if (ls > M) {
            const float a = exp2_hw((M - ls) * kLog2e);  // M = -inf gives 0
            acc *= a;
            l *= a;
            M = ls;
        }
        const float w = exp2_hw((ls - M) * kLog2e);
        acc += w * o;
        l += w;
    }
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    const bf16x4 ob = __builtin_convertvector(acc * inv, bf16x4);
    *reinterpret_cast<bf16x4*>(O + (size_t)row * D + 4 * c4) = ob;
    if (c4 == 0) lse[row] = l > 0.f ? M + logf(l) : kNegInf;
}

// With SPLIT (dense only) the workgroup computes one of nsplit contiguous
// ranges of its query block's key tiles and writes the normalised partial
// output in bf16 (through LDS as whole rows, like O) and the partial
// logsumexp in fp32 (-inf for a row that sees no key of the range) to opart
// [nsplit][BH][N][D] and lpart [nsplit][BH][N]; attn_combine_kernel merges
// them in fp32.
template <int D, bool CAUSAL, bool VARLEN, bool SPLIT = false>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_bf16_pp_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                        const __bf16* __restrict__ V, __bf16* __restrict__ O,
                        float* __restrict__ lse, int Nmax, int BH, int nqt, float scale,
                        const int* __restrict__ cu, int H, int Hkv, int total,
                        __bf16* __restrict__ opart, float* __restrict__ lpart, int nsplit)
{
    static_assert(!(SPLIT && VARLEN), "split-KV runs on dense tensors");
    // Keys per step: 128 at D = 64 (its 64-key steps are half as long as at
    // D = 128, so the per-step costs weigh twice as much), 64 at D = 128
    // (128-key steps there need more than 256 registers).
    constexpr int NW = 8, BC = D == 64 ? 128 : 64;
    using C = Cfg<D, 1, NW, 64>;
    // Unpadded tiles; at least the padded 64-key size, which the output
    // staging (store_tile_rows) needs.
    constexpr int KT_B = BC * D * 2 > C::KTILE_B ? BC * D * 2 : C::KTILE_B;
    constexpr int VT_B = BC * D * 2 > C::VTILE_B ? BC * D * 2 : C::VTILE_B;
    __shared__ __attribute__((aligned(1024))) char kbuf0[KT_B];
    __shared__ __attribute__((aligned(1024))) char kbuf1[KT_B];
    __shared__ __attribute__((aligned(1024))) char vbuf0[VT_B];
    __shared__ __attribute__((aligned(1024))) char vbuf1[VT_B];
    auto kbuf = [&](auto bufc) -> char* { if constexpr (decltype(bufc)::value == 0) return kbuf0; else return kbuf1; };
    auto vbuf = [&](auto bufc) -> char* { if constexpr (decltype(bufc)::value == 0) return vbuf0; else return vbuf1; };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool late = wave >= NW / 2;  // runs each phase one step after its SIMD partner
    const int j = lane & 31, h = lane >> 5;
    // Workgroup id = t * BH + bh, or with SPLIT (t * nsplit + split) * BH + bh.
    const int tt = blockIdx.x / BH, bh = blockIdx.x - tt * BH;
    const int t = SPLIT ? tt / nsplit : tt;
    const int split = SPLIT ? tt - t * nsplit : 0;
    const int qt = CAUSAL ? nqt - 1 - t : t;
    const int q0 = qt * C::BR;
    const Slice sl = slice_of<D, VARLEN>(bh, Nmax, H, Hkv, cu, total);
    const int N = sl.n;
    if (VARLEN && q0 >= N) return;  // query block past this sequence (whole workgroup)
    const size_t base = sl.base;
    const uint32_t slice_b = (uint32_t)N * D * 2;
    const int qw0 = q0 + wave * 32;
    const int qrow = qw0 + j;

    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + base, slice_b);
    bf16x8 qf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
        qf[kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
            qrs, (uint32_t)(qrow * D + kk * 16 + 8 * h) * 2, 0, 0));

    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
    float m = kNegInf, l = 0.f;
    const float c = scale * kLog2e;

    const int kv_end = CAUSAL ? min(N, q0 + C::BR) : N;
    const int nvis = (kv_end + BC - 1) / BC;  // key tiles the block sees
    // The workgroup's tiles are kt0 .. kt0 + ntiles - 1 (all nvis without
    // SPLIT); the steps below count tiles from kt0.
    int kt0 = 0, ntiles = nvis;
    if constexpr (SPLIT) {
        const int per = (nvis + nsplit - 1) / nsplit;
        kt0 = min(nvis, split * per);
        ntiles = min(nvis, kt0 + per) - kt0;
    }
    // This wave computes tiles 0 .. T - 1 (of the workgroup's); only tile
    // T - 1 can need a mask.  Under SPLIT the first of a wave's tiles holds a
    // key every row of the wave sees (its first key precedes the wave's rows),
    // so its reference becomes finite there.
    const int T = !CAUSAL ? ntiles
                : SPLIT  ? max(0, min(ntiles, qw0 / BC + 1 - kt0))
                         : min(ntiles, qw0 / BC + 1);
    const int kvm = (kt0 + T - 1) * BC;
    const bool mask_last = (kvm + BC > N) || (CAUSAL && kvm + BC - 1 > qw0);

    // Tile loads.  The four waves that are about to run their matrix phase
    // load one part of a tile right before it: waves 0-3 load K(i + 1) at
    // the start of phase 2i, waves 4-7 load V(i) at the start of phase
    // 2i + 1 (at D = 64 at the start of their vector phase 2i instead, see
    // steps below).  Tiles sit in LDS unpadded (row pitch D elements) with their
    // 16-byte chunks permuted inside each row by an XOR with a few bits of
    // the row index, so that every LDS read below is conflict-free and a
    // part is exactly D / 8 wave loads of 1 KiB (four per wave at D = 128).
    // Load n of a part fills LDS positions 64 n .. 64 n + 63; the lane at
    // position p holds LDS row p / CPR (key order, for K and V), slot
    // p % CPR, and fetches the global chunk that belongs there.  Wave g of
    // the group issues loads n = g LPW .. g LPW + LPW - 1: one LDS base for
    // all of them, load u placed by the immediate offset u KiB, which
    // src[u] has subtracted (it stays >= 0: the block starts at byte
    // n KiB of the tile).
    //   K: chunk c of row r sits in slot c ^ kkey(r), kkey(r) = (r / RPQ) &
    //      (CPR - 1), RPQ = rows per 256 bytes: the 16 rows a ds_read_b128
    //      serves per cycle then hit 16 different 16-byte bank groups.
    //   V: 64-byte block b of row r sits in block slot b ^ vkey(r), vkey(r) =
    //      (r / RPQ) & (D / 32 - 1): the 4 rows x 64 bytes that 32 lanes of a
    //      ds_read_b64_tr_b16 take per cycle then hit all 64 banks once.
    constexpr int NG = NW / 2;  // waves per group
    constexpr int CPR = D / 8, RPQ = 256 / (2 * D), NB = D / 32;
    constexpr int LPW = (BC * D * 2 / 1024) / NG;
    static_assert((BC * D * 2 / 1024) % NG == 0, "tile parts split evenly over the group");
    const int g = wave % NG;
    uint32_t src[LPW];
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
        const int p = (g * LPW + u) * 64 + lane;
        const int r = p / CPR, slot = p % CPR;
        if (!late) {
            const int c = slot ^ ((r / RPQ) & (CPR - 1));
            src[u] = (uint32_t)(r * D + c * 8) * 2 - 1024u * u;
        } else {
            const int blk = (slot / 4) ^ ((r / RPQ) & (NB - 1));
            src[u] = (uint32_t)(r * D + blk * 32 + (slot % 4) * 8) * 2 - 1024u * u;
        }
    }
    // This wave's share of tile kt of X (K or V) into the LDS buffer dst.
    // Both are named at each call site, so the compiler sees which LDS
    // object every load writes.  A tile past the last one (kt >= ntiles)
    // gets an empty range: its loads read nothing and fill dst with zeros,
    // which no later step reads, so the loads need no branch.
    static_assert(LPW >= 1 && LPW <= 4, "one to four loads per wave");
    auto load_part = [&](const __bf16* X, char* dst, int kt) __attribute__((always_inline)) {
        const int kv0 = (kt0 + kt) * BC;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(
            X + sl.kvbase + (size_t)kv0 * D, kt < ntiles ? (uint32_t)(N - kv0) * D * 2 : 0u);
        lds_void_t* const d = (lds_void_t*)(dst + g * LPW * 1024);
        lds_dma16<0>(rs, d, src[0]);
        if constexpr (LPW > 1) lds_dma16<1024>(rs, d, src[1]);
        if constexpr (LPW > 2) lds_dma16<2048>(rs, d, src[2]);
        if constexpr (LPW > 3) lds_dma16<3072>(rs, d, src[3]);
    };

    // Lane addresses of the operand reads.  K: row jr = swap_bits23(j)
    // (+ 32 mt), chunk 2 kk + h at slot (2 kk + h) ^ kkey(jr): kbase ^
    // (kk << 5).  V (the
    // transposing read): row 16 ks + 8 (g16 >> 1) + e4 (+ 4 for the upper
    // half), 8 bytes at column 32 dt + 16 (g16 & 1) + 4 a4 of block dt, which
    // sits in block slot dt ^ vkey: vbase ^ (dt << 6).
    const int jr = swap_bits23(j);
    const int kj = (jr / RPQ) & (CPR - 1);
    const int kbase = jr * D * 2 + (h ^ (kj & 1)) * 16 + ((kj >> 1) << 5);
    const int g16 = lane >> 4, e4 = (lane >> 2) & 3, a4 = lane & 3;
    const int vrow = 8 * (g16 >> 1) + e4;
    const int vbase = vrow * D * 2 + (16 * (g16 & 1) + 4 * a4) * 2 + (((vrow / RPQ) & (NB - 1)) << 6);

    f32x16 s[BC / 32];   // scores of the current tile, 32 keys each
    bf16x8 pf[BC / 16];  // its probabilities, bf16, 16 keys each
#pragma unroll
    for (int ks = 0; ks < BC / 16; ++ks) pf[ks] = bf16x8{};

    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    auto qk = [&](auto kbc) __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < BC / 32; ++mt) s[mt] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int mt = 0; mt < BC / 32; ++mt) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                    kbuf(kbc) + mt * 64 * D + (kbase ^ (kk << 5)));
                s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[mt], 0, 0, 0);
            }
    };
    auto pv = [&](auto vbc) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < BC / 16; ++ks)
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                const char* vp = vbuf(vbc) + 16 * ks * D * 2 + (vbase ^ (dt << 6));
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)vp);
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vp + 4 * D * 2));
                const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[ks], acc[dt], 0, 0, 0);
            }
    };


    // Matrix phase of step i (1 <= i <= T): the wave's tile loads (tile kt
    // of X into ldst), P V of tile i - 1, then S^T of tile i (skipped at
    // step T), with the LDS reads of each scheduled several MFMAs ahead of
    // their use.  A wave past its last tile (i > T) only loads.  One code
    // path for steps 1 .. T keeps the accumulators in fixed registers.
    auto matrix_phase = [&](auto kbc, auto vbc, auto ldc, const __bf16* X, char* ldst, int kt,
                            int i) __attribute__((always_inline)) {
        constexpr bool LD = decltype(ldc)::value;  // this phase issues the loads
        if (CAUSAL && i > T) {  // without the mask every wave computes every step
            if constexpr (LD) load_part(X, ldst, kt);
            return;
        }
        if constexpr (LD) {
            load_part(X, ldst, kt);
            // Keep the loads first: issued at the end of the block they would
            // leave no time before the barrier that waits for them.
            __builtin_amdgcn_sched_barrier(0);
        }
        // P V, then S^T unless this is step T, whose scores are never used.
        // Each block gets its own pipeline: a few LDS reads ahead, then one
        // MFMA per one or two reads (P V: 2 reads per product, S^T: 1).
        constexpr int NPV = (BC / 16) * (D / 32), NQK = (BC / 32) * (D / 16);
        pv(vbc);
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // LDS reads
#pragma unroll
        for (int u = 0; u < NPV - 4; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        if (i < T) {
            qk(kbc);
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int u = 0; u < NQK - 4; ++u) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
    };
    // Step 0 has no probabilities yet: its matrix phase is S^T of tile 0.
    auto first_matrix_phase = [&]() __attribute__((always_inline)) {
        qk(B0{});
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int u = 0; u < (BC / 32) * (D / 16) - 4; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    };
    // Vector phase of step i: mask (last tile only), probabilities and row
    // sums, and the rare move of the exponent reference.
    auto vector_phase = [&](int i) __attribute__((always_inline)) {
        if (i < 0 || i >= T) return;
        if (i == T - 1 && mask_last) {
            // Key kvm + o of register r (o below) is hidden when o >= thr.
            // The empty asm keeps the 32 comparisons inside this rarely
            // taken branch instead of letting them be hoisted out of the loop.
            int thr = (CAUSAL ? min(N, qrow + 1) : N) - kvm - 8 * h;
            asm volatile("" : "+v"(thr));
#pragma unroll
            for (int mt = 0; mt < BC / 32; ++mt) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (mt * 32 + 16 * (r >> 3) + (r & 7) >= thr) s[mt][r] = kNegInf;
                // one 32-key group at a time: bounds the live compare masks
                if constexpr (BC > 64) __builtin_amdgcn_sched_barrier(0);
            }
        }
        // Probabilities against the current reference m (one FMA and one
        // v_exp_f32 each), their bf16 copies (the B operand of P V) and this
        // lane's partial row sum.  s keeps the scores for a recomputation.
        auto probs = [&](float mc) __attribute__((always_inline)) {
            float ps[4];  // four partial sums, seeded by the first four p
#pragma unroll
            for (int mt = 0; mt < BC / 32; ++mt)
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    f32x8 p8;
#pragma unroll
                    for (int r8 = 0; r8 < 8; ++r8) {
                        p8[r8] = exp2_hw(fmaf(s[mt][8 * half + r8], c, -mc));
                        if (mt == 0 && half == 0 && r8 < 4)
                            ps[r8] = p8[r8];
                        else
                            ps[r8 & 3] += p8[r8];
                    }
                    pf[2 * mt + half] = __builtin_convertvector(p8, bf16x8);
                }
            return (ps[0] + ps[1]) + (ps[2] + ps[3]);
        };
        // Every row of the wave starts at tile 0 with m = -inf: there the
        // probabilities against m would be inf or NaN, so tile 0 goes
        // straight to the reference move below.
        float lsum = i == 0 ? 0.f : probs(m * c);
        // No p exceeds its lane's sum, so while every lane's sum stays within
        // kSumLimit the reference can stay where it is: the tile needs no row
        // maximum at all.  Otherwise, and on tile 0, the reference moves to
        // the row maximum, l and the accumulators are rescaled by
        // 2^((m_old - m_new) c) (0 for an empty history), and the tile's
        // probabilities are (re)computed.  Tile 0 holds key 0, visible to
        // every row, so the new reference is finite.
        if (i == 0 || __builtin_amdgcn_ballot_w64(lsum > kSumLimit) != 0) {
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = fmaxf(s[0][u], s[0][u + 4]);
#pragma unroll
            for (int r = 8; r < 16; ++r) v[r & 3] = fmaxf(v[r & 3], s[0][r]);
#pragma unroll
            for (int mt = 1; mt < BC / 32; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) v[r & 3] = fmaxf(v[r & 3], s[mt][r]);
            const float mx = combine_xor32(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])), MaxOp());
            const float m_new = fmaxf(m, mx);
            const float alpha = (m_new == kNegInf) ? 1.f : exp2_hw((m - m_new) * c);
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) acc[dt] *= alpha;
            m = m_new;
            lsum = probs(m * c);
        }
        l += lsum;
    };

    // Prologue: K(0) (waves 0-3).
    if (!late) load_part(K, kbuf0, 0);
    __syncthreads();
    // Steps i = 0 .. ntiles (step ntiles only finishes P V); step 0 (S^T of
    // tile 0 alone) is peeled, then two steps per loop trip so that every
    // LDS buffer is a compile-time choice: K(i) sits in
    // kbuf[i % 2], V(i) in vbuf[i % 2].  K(i + 1) (loaded at the start of
    // phase 2i) and V(i) (start of phase 2i + 1, or of 2i) are waited for at
    // the barrier that ends phase 2i + 1.  No barrier separates phase 2i from
    // 2i + 1: each buffer a phase fills was last read before the previous
    // barrier, and each buffer it reads was filled before it (measured 1-2%
    // faster than a barrier between every two phases).  The two wave groups
    // run separate copies of the loop (same barriers, phases swapped), which
    // keeps each copy's live registers to those of one phase order.
    // Where waves 4-7 load V(i): at D = 128 at the start of their matrix
    // phase 2i + 1; at D = 64, whose matrix phase is half as long, a load
    // issued there has not landed by the barrier that ends the phase, so it
    // moves to the start of their vector phase 2i (V(i)'s buffer was last
    // read in phase 2i - 1).  Measured: +6% at D = 64 (both masks), -4% for
    // causal D = 128.
    using VEarly = std::integral_constant<bool, D == 64>;
    using VInMatrix = std::integral_constant<bool, D != 64>;
    auto steps = [&](auto latec) __attribute__((always_inline)) {
        constexpr bool LATE = decltype(latec)::value;
        // step 0
        // (under SPLIT a wave may have no tile of the range: T = 0)
        if constexpr (!LATE) {
            if (1 < ntiles) load_part(K, kbuf1, 1);
            if (!SPLIT || T > 0) first_matrix_phase();
            vector_phase(0);
        } else {
            load_part(V, vbuf0, 0);
            if (!SPLIT || T > 0) first_matrix_phase();
        }
        __syncthreads();  // K(1) and V(0) have landed
        for (int i = 1; i <= ntiles; i += 2) {
            if constexpr (!LATE) {
                matrix_phase(B1{}, B0{}, std::true_type{}, K, kbuf0, i + 1, i);
            } else {
                if constexpr (VEarly::value) load_part(V, vbuf1, i);
                vector_phase(i - 1);
            }
            if constexpr (!LATE) {
                vector_phase(i);
            } else {
                matrix_phase(B1{}, B0{}, VInMatrix{}, V, vbuf1, i, i);
            }
            if (i + 1 > ntiles) break;
            __syncthreads();  // K(i + 1) and V(i) have landed
            if constexpr (!LATE) {
                matrix_phase(B0{}, B1{}, std::true_type{}, K, kbuf1, i + 2, i + 1);
            } else {
                if constexpr (VEarly::value) load_part(V, vbuf0, i + 1);
                vector_phase(i);
            }
            if constexpr (!LATE) {
                vector_phase(i + 1);
            } else {
                matrix_phase(B0{}, B1{}, VInMatrix{}, V, vbuf0, i + 1, i + 1);
            }
            __syncthreads();  // K(i + 2) and V(i + 1) have landed
        }
    };
    if (late)
        steps(std::true_type{});
    else
        steps(std::false_type{});

    const float l_tot = combine_xor32(l, SumOp());
    if constexpr (SPLIT) {
        // Partial of this key range: O_s = acc / l rounded to bf16 and
        // stored as whole rows through LDS, lse_s = m scale + ln l, or O_s = 0
        // and -inf for a row that saw no key of the range.  bf16 partials
        // halve the bytes the partial pass writes and the merge reads; fp32
        // ones measured 6-17% slower for the whole call ([1, 2, 8192, 128],
        // [1, 4, 4096, 128], [1, 1, 16384, 128], both masks), with the same
        // lse and an output within one bf16 rounding.
        const size_t pslice = (size_t)split * BH + bh;
        const __amdgpu_buffer_rsrc_t prs = make_rsrc(opart + pslice * N * D, (uint32_t)N * D * 2);
        const __amdgpu_buffer_rsrc_t plrs = make_rsrc(lpart + pslice * N, (uint32_t)N * 4);
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
        __syncthreads();  // every wave is done with the tile buffers
        store_tile_rows<D>(acc, inv, out_stage<D>(wave, kbuf0, kbuf1, vbuf0, vbuf1), prs, qw0, lane);
        if (h == 0) {
            const float ls = l_tot > 0.f ? m * scale + logf(l_tot) : kNegInf;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ls), plrs, (uint32_t)qrow * 4, 0, 0);
        }
        return;
    }
    const __amdgpu_buffer_rsrc_t ors = make_rsrc(O + base, slice_b);
    const __amdgpu_buffer_rsrc_t lrs = make_rsrc(lse + sl.lbase, (uint32_t)N * 4);
    __syncthreads();  // every wave is done with the tile buffers
    store_tile_rows<D>(acc, 1.0f / l_tot, out_stage<D>(wave, kbuf0, kbuf1, vbuf0, vbuf1), ors, qw0, lane);
    if (h == 0)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m * scale + logf(l_tot)), lrs,
                                              (uint32_t)qrow * 4, 0, 0);
}

// N is the sequence length, or with cu (packed sequences) the longest
// sequence; H and total describe the packed layout (unused when dense).
template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_pp(const void* Q, const void* K, const void* V, void* O, float* lse, int BH,
                     int N, float scale, const int* cu, int H, int Hkv, int total,
                     hipStream_t stream)
{
    constexpr int BR = 256;
    const int nqt = (N + BR - 1) / BR;
    const dim3 grid((unsigned)(nqt * BH)), block(512);
    attn_fwd_bf16_pp_kernel<D, CAUSAL, VARLEN><<<grid, block, 0, stream>>>(
        static_cast<const __bf16*>(Q), static_cast<const __bf16*>(K), static_cast<const __bf16*>(V),
        static_cast<__bf16*>(O), lse, N, BH, nqt, scale, cu, H, Hkv, total, nullptr, nullptr, 1);
    return hipGetLastError();
}

template <int D, int QT, int NW, int WPE, int BC, bool CAUSAL, bool VARLEN, int KS = 1>
hipError_t launch(const void* Q, const void* K, const void* V, void* O, float* lse, int BH,
                  int N, float scale, const int* cu, int H, int Hkv, int total,
                  hipStream_t stream)
{
    using C = Cfg<D, QT, NW, BC, KS>;
    const int nqt = (N + C::BR - 1) / C::BR;
    const dim3 grid((unsigned)(nqt * BH)), block(C::T);
    // the part of the tile buffers in dynamic LDS (VDYN / KVDYN in the kernel)
    constexpr unsigned dyn = (D == 64 && KS == 2) ? (unsigned)(KS * C::VTILE_B)
                           : (D == 128 && KS == 2) ? (unsigned)(KS * (C::KTILE_B + C::VTILE_B)) : 0u;
    attn_fwd_bf16_kernel<D, QT, NW, WPE, BC, CAUSAL, VARLEN, KS><<<grid, block, dyn, stream>>>(
        static_cast<const __bf16*>(Q), static_cast<const __bf16*>(K), static_cast<const __bf16*>(V),
        static_cast<__bf16*>(O), lse, N, BH, nqt, scale, cu, H, Hkv, total);
    return hipGetLastError();
}

// Launch shape, from the number of 256-row (W256) and 128-row (W128) query
// blocks against the 256 CUs (measured over [1..2, 6..32, 1024..4096, d]):
//  * the phase-staggered kernel (8 waves x 32 rows, one workgroup per CU at
//    a time) when W256 > 256, and without the mask already when W128 > 256:
//    unmasked, it beats the plain kernel even with 160-192 workgroups (+11%
//    to +15% on [1, 10..24, 2048..4096, 128]), while under the causal mask
//    one round of unequal blocks leaves CUs idle ([1, 32, 2048, 64] causal:
//    396 against 468 TFLOPS with key groups);
//  * otherwise the plain kernel with 128-row workgroups of 8 waves in two
//    key groups, as long as that fills the CUs (W128 >= 256 under the causal
//    mask, W128 > 128 without it: +4-10% over 4 waves with the whole key
//    loop, +6-20% causal);
//  * below that 64-row workgroups of 4 waves in two key groups (+21-47%
//    over 2 waves with the whole key loop on [2, 8, 1024, 64],
//    [1, 8, 2048, 128] and [1, 2, 8192, 128]).
template <int D, bool CAUSAL, bool VARLEN = false>
hipError_t dispatch(const void* Q, const void* K, const void* V, void* O, float* lse, int BH,
                    int N, float scale, hipStream_t stream, int H = 1, int Hkv = 1,
                    const int* cu = nullptr, int total = 0)
{
    constexpr long long kCUs = 256;
    const long long w256 = (long long)((N + 255) / 256) * BH;
    const long long w128 = (long long)((N + 127) / 128) * BH;
    if (w256 > kCUs || (!CAUSAL && w128 > kCUs))
        return launch_pp<D, CAUSAL, VARLEN>(Q, K, V, O, lse, BH, N, scale, cu, H, Hkv, total, stream);
    if (CAUSAL ? w128 >= kCUs : w128 > kCUs / 2)
        return launch<D, 1, 8, 2, 64, CAUSAL, VARLEN, 2>(Q, K, V, O, lse, BH, N, scale, cu, H, Hkv, total, stream);
    return launch<D, 1, 4, 2, 64, CAUSAL, VARLEN, 2>(Q, K, V, O, lse, BH, N, scale, cu, H, Hkv, total, stream);
}

// Merge of split partials (attn_combine): merge_row for every row, D / 4
// lanes per row, rows walked grid-stride.
template <int D, class PT>
__global__ void __launch_bounds__(256)
attn_combine_kernel(const PT* __restrict__ opart, const float* __restrict__ lpart,
                    __bf16* __restrict__ O, float* __restrict__ lse, int S, long long rows)
{
    constexpr int LPR = D / 4;         // lanes per row
    constexpr int RPB = 256 / LPR;     // rows per workgroup and pass
    const int c4 = threadIdx.x % LPR;  // column group of this lane
    for (long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR; row < rows;
         row += (long long)gridDim.x * RPB)
        merge_row<D, PT>(opart, lpart, O, lse, S, rows, row, c4);
}

// Split-KV forward: 8-wave workgroups (256 query rows) over nsplit key ranges
// each, then the merge.
template <int D, bool CAUSAL>
hipError_t launch_split(const void* Q, const void* K, const void* V, void* O, float* lse, int BH,
                        int N, float scale, int nsplit, __bf16* opart, float* lpart, int H, int Hkv,
                        hipStream_t stream)
{
    // Partial pass: the phase-staggered kernel over (256-row query block,
    // key range) workgroups, longest blocks first under the mask; then the
    // merge over all rows.  (Merging each block in the last of its
    // workgroups to finish, behind a per-block counter, was measured 1.7-6x
    // slower, with fp32 partials: one workgroup's serial loads cannot move a
    // block's nsplit partials, ~1 MiB at d = 128, in the time the whole-chip
    // merge takes.)
    constexpr int BR = 256;
    const int nqt = (N + BR - 1) / BR;
    attn_fwd_bf16_pp_kernel<D, CAUSAL, false, true>
        <<<dim3((unsigned)(nqt * nsplit * BH)), dim3(512), 0, stream>>>(
            static_cast<const __bf16*>(Q), static_cast<const __bf16*>(K),
            static_cast<const __bf16*>(V), nullptr, nullptr, N, BH, nqt, scale, nullptr, H, Hkv, 0,
            opart, lpart, nsplit);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long rows = (long long)BH * N;
    const int rpb = 256 / (D / 4);
    const long long need = (rows + rpb - 1) / rpb;
    attn_combine_kernel<D, __bf16><<<dim3((unsigned)(need < 65536 ? need : 65536)), dim3(256), 0, stream>>>(
        opart, lpart, static_cast<__bf16*>(O), lse, nsplit, rows);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_combine(const float* opart, const float* lpart, void* O, float* lse, int S,
                               long long rows, int d, hipStream_t stream)
{
    // Enough workgroups for several per CU; larger problems loop.
    const int rpb = 256 / (d / 4);
    const long long need = (rows + rpb - 1) / rpb;
    const dim3 grid((unsigned)(need < 65536 ? need : 65536)), block(256);
    if (d == 64)
        attn_combine_kernel<64, float><<<grid, block, 0, stream>>>(opart, lpart, static_cast<__bf16*>(O),
                                                            lse, S, rows);
    else
        attn_combine_kernel<128, float><<<grid, block, 0, stream>>>(opart, lpart, static_cast<__bf16*>(O),
                                                             lse, S, rows);
    return hipGetLastError();
}

int attn_splitkv_auto(int BH, int N, int d, bool causal)
{
    // Every wave of the single pass owns 32 query rows; 2048 waves (two per
    // SIMD on 256 CUs) keep both the matrix core and the vector unit of every
    // SIMD busy.  Below that, split the keys so that the partial pass reaches
    // 2048 waves, twice that under the causal mask (its query blocks differ
    // in length, and more, shorter ranges even them out), with at least 512
    // keys per range.  Rows of 1024 keys or fewer are not split, nor rows of
    // 2048 or fewer without the mask or with more than 16384 rows in all
    // (8192 at d = 64): there the partials cost as much HBM time as the
    // occupancy gains (and the single pass already splits the key loop over
    // two wave groups).  Measured with bf16 partials: [1, 4, 2048, 128]
    // causal gains 14% from 4 ranges, [1, 8, 2048, 128] and [1, 4, 2048, 64]
    // 3-4%; [1, 8, 2048, 64] and [1, 16..24, 2048, d] causal and
    // [1, 8, 2048, 128] unmasked lose.
    const long long rows = (long long)BH * N;
    // Unmasked grids of 256-row blocks just past one round of the CUs (the
    // second round nearly empty): two ranges fill the rounds better.
    // Measured: [1, 24, 3000, 128] +5%, [1, 17, 4096, 128] and
    // [2, 9, 3600, 128] +8%, [1, 20, 4096, 64] +15%; [1, 12, 8192, 128] (a
    // half-full second round) +1%, and longer grids gain less than the
    // partials cost.
    const long long w256 = (long long)BH * ((N + 255) / 256);
    if (!causal && N > 2048 && w256 > 256 && w256 < 512 && w256 % 256 <= 96) return 2;
    if (N <= 1024 || rows >= 65536) return 1;
    if (N <= 2048 && (!causal || rows > (d == 64 ? 8192 : 16384))) return 1;
    long long s = (65536 * (causal ? 2 : 1) + rows - 1) / rows;
    const long long cap = N / 512;
    if (s > cap) s = cap;
    if (s > 16) s = 16;
    return s < 1 ? 1 : (int)s;
}

hipError_t launch_attn_fwd_bf16_split(const void* Q, const void* K, const void* V, void* O,
                                      float* lse, int B, int H, int Hkv, int N, int d, float scale,
                                      bool causal, int nsplit, __bf16* opart, float* lpart,
                                      hipStream_t stream)
{
    const int BH = B * H;
    if (d == 64)
        return causal ? launch_split<64, true>(Q, K, V, O, lse, BH, N, scale, nsplit, opart, lpart, H, Hkv, stream)
                      : launch_split<64, false>(Q, K, V, O, lse, BH, N, scale, nsplit, opart, lpart, H, Hkv, stream);
    return causal ? launch_split<128, true>(Q, K, V, O, lse, BH, N, scale, nsplit, opart, lpart, H, Hkv, stream)
                  : launch_split<128, false>(Q, K, V, O, lse, BH, N, scale, nsplit, opart, lpart, H, Hkv, stream);
}

hipError_t launch_attn_fwd_bf16_varlen(const void* Q, const void* K, const void* V, void* O,
                                       float* lse, const int* cu, int B, int H, int Hkv, int total,
                                       int max_seqlen, int d, float scale, bool causal,
                                       hipStream_t stream)
{
    const int BH = B * H;
    if (d == 64)
        return causal ? dispatch<64, true, true>(Q, K, V, O, lse, BH, max_seqlen, scale, stream, H, Hkv, cu, total)
                      : dispatch<64, false, true>(Q, K, V, O, lse, BH, max_seqlen, scale, stream, H, Hkv, cu, total);
    return causal ? dispatch<128, true, true>(Q, K, V, O, lse, BH, max_seqlen, scale, stream, H, Hkv, cu, total)
                  : dispatch<128, false, true>(Q, K, V, O, lse, BH, max_seqlen, scale, stream, H, Hkv, cu, total);
}

hipError_t launch_attn_fwd_bf16(const void* Q, const void* K, const void* V, void* O,
                                float* lse, int B, int H, int Hkv, int N, int d, float scale,
                                bool causal, hipStream_t stream)
{
    const int BH = B * H;
    if (d == 64)
        return causal ? dispatch<64, true>(Q, K, V, O, lse, BH, N, scale, stream, H, Hkv)
                      : dispatch<64, false>(Q, K, V, O, lse, BH, N, scale, stream, H, Hkv);
    return causal ? dispatch<128, true>(Q, K, V, O, lse, BH, N, scale, stream, H, Hkv)
                  : dispatch<128, false>(Q, K, V, O, lse, BH, N, scale, stream, H, Hkv);
}

}  // namespace osm
