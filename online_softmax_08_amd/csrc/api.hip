// api.hip -- the C ABI (include/osm.h): host-side argument validation, the
// gfx950 device check and dispatch to the kernels.  Validation runs before any
// HIP call, so a rejected call touches neither the device nor the stream.

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "kernels.h"
#include "osm.h"

namespace {

bool overlaps(const void* a, size_t abytes, const void* b, size_t bbytes)
{
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return abytes && bbytes && a0 < b0 + bbytes && b0 < a0 + abytes;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Per-device result of the architecture check: 0 unknown, 1 gfx950, 2 other.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

int check_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return OSM_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return OSM_ERR_DEVICE;
    int state = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return OSM_ERR_HIP;
        state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_arch_ok[dev].store(state, std::memory_order_relaxed);
    }
    return state == 1 ? OSM_OK : OSM_ERR_DEVICE;
}

int finish(hipError_t e) { return e == hipSuccess ? OSM_OK : OSM_ERR_HIP; }

// Device scratch of attn_bwd_noalloc: the two fp32 row statistics of the
// backward (D and L log2 e, OSM_NOALLOC_BWD_MAX_ROWS rows each), one copy per
// GPU, held from the library's first use on that GPU until the process ends.
// On the host, `scratch` names a host-side stand-in, not device memory: host
// code only ever uses the per-device address hipGetSymbolAddress returns.
static __device__ __align__(256) float scratch[2 * (size_t)OSM_NOALLOC_BWD_MAX_ROWS];

std::atomic<void*> g_scratch[kMaxDevices];

// Device address of this GPU's scratch array, looked up once per device with
// that device current (the caller has run check_device, so the current
// device index is valid).  Concurrent first calls look up the same address.
int scratch_address(float** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return OSM_ERR_HIP;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return OSM_ERR_HIP;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = static_cast<float*>(p);
    return OSM_OK;
}

// Shape and scale checks shared by the attention entry points.
int check_attn_shape(int B, int H, int N, int d, float scale, size_t elem)
{
    if (B < 0 || H < 0 || N < 0) return OSM_ERR_SIZE;
    if (d != 64 && d != 128) return OSM_ERR_HEAD_DIM;
    if (!(std::isfinite(scale) && scale > 0.f)) return OSM_ERR_SCALE;
    if (B == 0 || H == 0 || N == 0) return OSM_OK;
    const long long bh = (long long)B * H;
    // Work-group ids (bh * query blocks of at least 128 rows) and row indices
    // must fit in 32 bits, a dispatch counts at most 2^32 - 1 work-items (the
    // launch of every grid above 65,536 rows has two per row, rounded up to
    // 256-row blocks; the smaller grids, with up to four per row in 64- or
    // 128-row blocks, stay far below), and the bytes of one (b, h) slice are
    // a 32-bit buffer offset.
    if (bh > INT_MAX || bh * ((N + 127) / 128) > INT_MAX) return OSM_ERR_SIZE;
    if (bh * ((N + 255) / 256) * 512 > UINT32_MAX || (long long)N * d * (long long)elem > UINT32_MAX)
        return OSM_ERR_SIZE;
    return OSM_OK;
}

// Key/value heads: 1 <= Hkv <= H and Hkv divides H (checked once H > 0).
int check_heads(int H, int Hkv)
{
    return (Hkv >= 1 && Hkv <= H && H % Hkv == 0) ? OSM_OK : OSM_ERR_HEADS;
}

// Shared validation of the dense forward calls (K and V with Hkv heads).
// *work is set to false for an empty problem (valid, nothing to launch).
int validate_attn(const void* Q, const void* K, const void* V, const void* O, const float* lse,
                  int B, int H, int Hkv, int N, int d, float scale, size_t elem, bool* work)
{
    *work = false;
    int st = check_attn_shape(B, H, N, d, scale, elem);
    if (st != OSM_OK || B == 0 || H == 0 || N == 0) return st;
    if ((st = check_heads(H, Hkv)) != OSM_OK) return st;
    const long long bh = (long long)B * H;
    if (!Q || !K || !V || !O || !lse) return OSM_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(lse, 4))
        return OSM_ERR_ALIGN;
    const size_t tbytes = (size_t)bh * N * d * elem, lbytes = (size_t)bh * N * sizeof(float);
    const size_t kvbytes = (size_t)B * Hkv * N * d * elem;
    if (overlaps(O, tbytes, Q, tbytes) || overlaps(O, tbytes, K, kvbytes) ||
        overlaps(O, tbytes, V, kvbytes) || overlaps(lse, lbytes, Q, tbytes) ||
        overlaps(lse, lbytes, K, kvbytes) || overlaps(lse, lbytes, V, kvbytes) ||
        overlaps(lse, lbytes, O, tbytes))
        return OSM_ERR_ALIAS;
    *work = true;
    return OSM_OK;
}

// Bytes of the split-KV workspace: bf16 partial outputs [nsplit][bh][N][d],
// then the fp32 partial logsumexps [nsplit][bh][N].
size_t splitkv_workspace(int nsplit, long long bh, int N, int d)
{
    return (size_t)nsplit * bh * N * ((size_t)d * 2 + sizeof(float));
}

}  // namespace

extern "C" {

int attn_fwd(const void* Q, const void* K, const void* V, void* O, float* lse, int B, int H,
             int N, int d, float scale, int causal, void* stream)
{
    bool work = false;
    int st = validate_attn(Q, K, V, O, lse, B, H, H, N, d, scale, 2, &work);
    if (st != OSM_OK || !work) return st;
    if ((st = check_device()) != OSM_OK) return st;
    return finish(osm::launch_attn_fwd_bf16(Q, K, V, O, lse, B, H, H, N, d, scale, causal != 0,
                                            static_cast<hipStream_t>(stream)));
}

int attn_fwd_gqa(const void* Q, const void* K, const void* V, void* O, float* lse, int B, int H,
                 int Hkv, int N, int d, float scale, int causal, void* stream)
{
    bool work = false;
    int st = validate_attn(Q, K, V, O, lse, B, H, Hkv, N, d, scale, 2, &work);
    if (st != OSM_OK || !work) return st;
    if ((st = check_device()) != OSM_OK) return st;
    return finish(osm::launch_attn_fwd_bf16(Q, K, V, O, lse, B, H, Hkv, N, d, scale, causal != 0,
                                            static_cast<hipStream_t>(stream)));
}

int attn_fwd_fp8(const void* Q, const void* K, const void* V, float q_scale, float k_scale,
                 float v_scale, void* O, float* lse, int B, int H, int Hkv, int N, int d,
                 float scale, int causal, void* stream)
{
    // Sizes as for the bf16 call (the bf16 output's slice bytes bound the
    // 32-bit offsets); one byte per input element.
    int st = check_attn_shape(B, H, N, d, scale, 2);
    if (st != OSM_OK || B == 0 || H == 0 || N == 0) return st;
    if (!(std::isfinite(q_scale) && q_scale > 0.f && std::isfinite(k_scale) && k_scale > 0.f &&
          std::isfinite(v_scale) && v_scale > 0.f))
        return OSM_ERR_SCALE;
    if (!(std::isfinite(scale * q_scale * k_scale) && scale * q_scale * k_scale > 0.f))
        return OSM_ERR_SCALE;
    if ((st = check_heads(H, Hkv)) != OSM_OK) return st;
    if (!Q || !K || !V || !O || !lse) return OSM_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(lse, 4))
        return OSM_ERR_ALIGN;
    const long long bh = (long long)B * H;
    const size_t qbytes = (size_t)bh * N * d, kvbytes = (size_t)B * Hkv * N * d;
    const size_t obytes = (size_t)bh * N * d * 2, lbytes = (size_t)bh * N * sizeof(float);
    if (overlaps(O, obytes, Q, qbytes) || overlaps(O, obytes, K, kvbytes) ||
        overlaps(O, obytes, V, kvbytes) || overlaps(lse, lbytes, Q, qbytes) ||
        overlaps(lse, lbytes, K, kvbytes) || overlaps(lse, lbytes, V, kvbytes) ||
        overlaps(lse, lbytes, O, obytes))
        return OSM_ERR_ALIAS;
    if ((st = check_device()) != OSM_OK) return st;
    return finish(osm::launch_attn_fwd_fp8(Q, K, V, O, lse, B, H, Hkv, N, d,
                                           scale * q_scale * k_scale, v_scale, causal != 0,
                                           static_cast<hipStream_t>(stream)));
}

int attn_fwd_fp8_mx(const void* Q, const void* q_scales, const void* K, const void* k_scales,
                    const void* V, const void* v_scales, void* O, float* lse, int B, int H,
                    int Hkv, int N, int d, float scale, int causal, void* stream)
{
    int st = check_attn_shape(B, H, N, d, scale, 2);
    if (st != OSM_OK || B == 0 || H == 0 || N == 0) return st;
    if ((st = check_heads(H, Hkv)) != OSM_OK) return st;
    if (!Q || !K || !V || !q_scales || !k_scales || !v_scales || !O || !lse) return OSM_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(lse, 4))
        return OSM_ERR_ALIGN;
    const long long bh = (long long)B * H, bhkv = (long long)B * Hkv;
    const size_t qbytes = (size_t)bh * N * d, kvbytes = (size_t)bhkv * N * d;
    const size_t qsb = (size_t)bh * N * (d / 32), ksb = (size_t)bhkv * N * (d / 32);
    const size_t vsb = (size_t)bhkv * ((N + 31) / 32) * d;
    const size_t obytes = (size_t)bh * N * d * 2, lbytes = (size_t)bh * N * sizeof(float);
    const void* in[6] = {Q, K, V, q_scales, k_scales, v_scales};
    const size_t inb[6] = {qbytes, kvbytes, kvbytes, qsb, ksb, vsb};
    for (int i = 0; i < 6; ++i)
        if (overlaps(O, obytes, in[i], inb[i]) || overlaps(lse, lbytes, in[i], inb[i]))
            return OSM_ERR_ALIAS;
    if (overlaps(lse, lbytes, O, obytes)) return OSM_ERR_ALIAS;
    if ((st = check_device()) != OSM_OK) return st;
    return finish(osm::launch_attn_fwd_fp8_mx(Q, q_scales, K, k_scales, V, v_scales, O, lse, B, H,
                                              Hkv, N, d, scale, causal != 0,
                                              static_cast<hipStream_t>(stream)));
}

int fp8_quantize_rows(const void* X, const signed char* signs, void* codes, void* scales,
                      long long rows, int d, void* stream)
{
    if (rows < 0) return OSM_ERR_SIZE;
    if (d != 64 && d != 128) return OSM_ERR_HEAD_DIM;
    uint64_t neg[2] = {0, 0};
    if (signs) {
        for (int t = 0; t < d; ++t) {
            if (signs[t] != 1 && signs[t] != -1) return OSM_ERR_SIGNS;
            if (signs[t] == -1) neg[t / 64] |= 1ull << (t % 64);
        }
    }
    if (rows == 0) return OSM_OK;
    if (!X || !codes || !scales) return OSM_ERR_NULL;
    if (!aligned(X, 16) || !aligned(codes, 8)) return OSM_ERR_ALIGN;
    const size_t xb = (size_t)rows * d * 2, cb = (size_t)rows * d, sb = (size_t)rows * (d / 32);
    if (overlaps(codes, cb, X, xb) || overlaps(scales, sb, X, xb) || overlaps(scales, sb, codes, cb))
        return OSM_ERR_ALIAS;
    int st = check_device();
    if (st != OSM_OK) return st;
    return finish(osm::launch_fp8_quant_rows(X, codes, scales, rows, d, signs != nullptr, neg[0],
                                             neg[1], static_cast<hipStream_t>(stream)));
}

int fp8_quantize_cols(const void* X, void* codes, void* scales, long long slices, int n, int d,
                      void* stream)
{
    if (slices < 0 || n < 0) return OSM_ERR_SIZE;
    if (d != 64 && d != 128) return OSM_ERR_HEAD_DIM;
    if (slices == 0 || n == 0) return OSM_OK;
    if (!X || !codes || !scales) return OSM_ERR_NULL;
    if (!aligned(X, 16) || !aligned(codes, 8)) return OSM_ERR_ALIGN;
    const size_t xb = (size_t)slices * n * d * 2, cb = (size_t)slices * n * d;
    const size_t sb = (size_t)slices * ((n + 31) / 32) * d;
    if (overlaps(codes, cb, X, xb) || overlaps(scales, sb, X, xb) || overlaps(scales, sb, codes, cb))
        return OSM_ERR_ALIAS;
    int st = check_device();
    if (st != OSM_OK) return st;
    return finish(osm::launch_fp8_quant_cols(X, codes, scales, slices, n, d,
                                             static_cast<hipStream_t>(stream)));
}

int attn_fwd_f32(const float* Q, const float* K, const float* V, float* O, float* lse, int B,
                 int H, int N, int d, float scale, int causal, void* stream)
{
    bool work = false;
    int st = validate_attn(Q, K, V, O, lse, B, H, H, N, d, scale, 4, &work);
    if (st != OSM_OK || !work) return st;
    if ((st = check_device()) != OSM_OK) return st;
    return finish(osm::launch_attn_fwd_f32(Q, K, V, O, lse, B * H, N, d, scale, causal != 0,
                                           static_cast<hipStream_t>(stream)));
}

int row_softmax(const float* x, float* y, int B, int N, void* stream)
{
    if (B < 0 || N < 0) return OSM_ERR_SIZE;
    if (B == 0 || N == 0) return OSM_OK;
    if (!x || !y) return OSM_ERR_NULL;
    if (!aligned(x, 4) || !aligned(y, 4)) return OSM_ERR_ALIGN;
    const size_t bytes = (size_t)B * N * sizeof(float);
    if (x != y && overlaps(x, bytes, y, bytes)) return OSM_ERR_ALIAS;
    int st = check_device();
    if (st != OSM_OK) return st;
    return finish(osm::launch_row_softmax(x, y, B, N, static_cast<hipStream_t>(stream)));
}

int attn_fwd_varlen(const void* Q, const void* K, const void* V, void* O, float* lse,
                    const int* cu_seqlens, int B, int H, int Hkv, int total, int max_seqlen,
                    int d, float scale, int causal, void* stream)
{
    if (B < 0 || H < 0 || total < 0 || max_seqlen < 0) return OSM_ERR_SIZE;
    if (d != 64 && d != 128) return OSM_ERR_HEAD_DIM;
    if (!(std::isfinite(scale) && scale > 0.f)) return OSM_ERR_SCALE;
    if (B == 0 || H == 0 || total == 0 || max_seqlen == 0) return OSM_OK;
    // Per-workgroup limits are those of a dense call with N = max_seqlen.
    int st = check_attn_shape(B, H, max_seqlen, d, scale, 2);
    if (st != OSM_OK) return st;
    if ((st = check_heads(H, Hkv)) != OSM_OK) return st;
    if (!Q || !K || !V || !O || !lse || !cu_seqlens) return OSM_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) ||
        !aligned(lse, 4) || !aligned(cu_seqlens, 4))
        return OSM_ERR_ALIGN;
    const size_t tb = (size_t)H * total * d * 2, lb = (size_t)H * total * sizeof(float);
    const size_t kvb = (size_t)Hkv * total * d * 2, cb = (size_t)(B + 1) * sizeof(int);
    if (overlaps(O, tb, Q, tb) || overlaps(O, tb, K, kvb) || overlaps(O, tb, V, kvb) ||
        overlaps(O, tb, cu_seqlens, cb) || overlaps(lse, lb, Q, tb) ||
        overlaps(lse, lb, K, kvb) || overlaps(lse, lb, V, kvb) || overlaps(lse, lb, O, tb) ||
        overlaps(lse, lb, cu_seqlens, cb))
        return OSM_ERR_ALIAS;
    if ((st = check_device()) != OSM_OK) return st;
    return finish(osm::launch_attn_fwd_bf16_varlen(Q, K, V, O, lse, cu_seqlens, B, H, Hkv, total,
                                                   max_seqlen, d, scale, causal != 0,
                                                   static_cast<hipStream_t>(stream)));
}

int attn_fwd_splitkv_plan(int B, int H, int N, int d, int causal, int nsplit, int* nsplit_out,
                          size_t* workspace_bytes)
{
    if (!nsplit_out || !workspace_bytes) return OSM_ERR_NULL;
    if (B < 0 || H < 0 || N < 0) return OSM_ERR_SIZE;
    if (d != 64 && d != 128) return OSM_ERR_HEAD_DIM;
    if (nsplit < 0 || nsplit > osm::kMaxSplits) return OSM_ERR_SPLITS;
    const long long bh = (long long)B * H;
    if (bh > INT_MAX) return OSM_ERR_SIZE;
    if (nsplit == 0) nsplit = (bh == 0 || N == 0) ? 1 : osm::attn_splitkv_auto((int)bh, N, d, causal != 0);
    *nsplit_out = nsplit;
    *workspace_bytes = nsplit == 1 ? 0 : splitkv_workspace(nsplit, bh, N, d);
    return OSM_OK;
}

int attn_fwd_splitkv(const void* Q, const void* K, const void* V, void* O, float* lse, int B,
                     int H, int Hkv, int N, int d, float scale, int causal, int nsplit,
                     void* workspace, size_t workspace_bytes, void* stream)
{
    bool work = false;
    int st = validate_attn(Q, K, V, O, lse, B, H, Hkv, N, d, scale, 2, &work);
    if (st != OSM_OK) return st;
    if (nsplit < 0 || nsplit > osm::kMaxSplits) return OSM_ERR_SPLITS;
    if (!work) return OSM_OK;
    const long long bh = (long long)B * H;
    if (nsplit == 0) nsplit = osm::attn_splitkv_auto((int)bh, N, d, causal != 0);
    if (nsplit == 1) {
        if ((st = check_device()) != OSM_OK) return st;
        return finish(osm::launch_attn_fwd_bf16(Q, K, V, O, lse, B, H, Hkv, N, d, scale, causal != 0,
                                                static_cast<hipStream_t>(stream)));
    }
    // The partial pass launches bh * ceil(N / 256) * nsplit workgroups of 512
    // work-items, and a dispatch counts at most 2^32 - 1 work-items; offsets
    // into one bf16 partial slice are 32-bit.
    if (bh * ((N + 255) / 256) * nsplit * 512 > UINT32_MAX || (long long)N * d * 2 > UINT32_MAX)
        return OSM_ERR_SIZE;
    const size_t need = splitkv_workspace(nsplit, bh, N, d);
    if (!workspace) return OSM_ERR_NULL;
    if (workspace_bytes < need) return OSM_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return OSM_ERR_ALIGN;
    const size_t tbytes = (size_t)bh * N * d * 2, lbytes = (size_t)bh * N * sizeof(float);
    const size_t kvbytes = (size_t)B * Hkv * N * d * 2;
    if (overlaps(workspace, need, Q, tbytes) || overlaps(workspace, need, K, kvbytes) ||
        overlaps(workspace, need, V, kvbytes) || overlaps(workspace, need, O, tbytes) ||
        overlaps(workspace, need, lse, lbytes))
        return OSM_ERR_ALIAS;
    if ((st = check_device()) != OSM_OK) return st;
    __bf16* opart = static_cast<__bf16*>(workspace);
    float* lpart = reinterpret_cast<float*>(opart + (size_t)nsplit * bh * N * d);
    return finish(osm::launch_attn_fwd_bf16_split(Q, K, V, O, lse, B, H, Hkv, N, d, scale,
                                                  causal != 0, nsplit, opart, lpart,
                                                  static_cast<hipStream_t>(stream)));
}

int attn_combine(const float* O_part, const float* lse_part, void* O, float* lse, int S, int B,
                 int H, int N, int d, void* stream)
{
    if (B < 0 || H < 0 || N < 0) return OSM_ERR_SIZE;
    if (d != 64 && d != 128) return OSM_ERR_HEAD_DIM;
    if (S < 1 || S > osm::kMaxSplits) return OSM_ERR_SPLITS;
    if (B == 0 || H == 0 || N == 0) return OSM_OK;
    const long long rows = (long long)B * H * N;
    if ((long long)B * H > INT_MAX) return OSM_ERR_SIZE;
    if (!O_part || !lse_part || !O || !lse) return OSM_ERR_NULL;
    if (!aligned(O_part, 16) || !aligned(lse_part, 4) || !aligned(O, 8) || !aligned(lse, 4))
        return OSM_ERR_ALIGN;
    const size_t pbytes = (size_t)S * rows * d * 4, plbytes = (size_t)S * rows * 4;
    const size_t obytes = (size_t)rows * d * 2, lbytes = (size_t)rows * 4;
    if (overlaps(O, obytes, O_part, pbytes) || overlaps(O, obytes, lse_part, plbytes) ||
        overlaps(lse, lbytes, O_part, pbytes) || overlaps(lse, lbytes, lse_part, plbytes) ||
        overlaps(lse, lbytes, O, obytes))
        return OSM_ERR_ALIAS;
    int st = check_device();
    if (st != OSM_OK) return st;
    return finish(osm::launch_attn_combine(O_part, lse_part, O, lse, S, rows, d,
                                           static_cast<hipStream_t>(stream)));
}

size_t attn_bwd_workspace_bytes(int B, int H, int N)
{
    if (B <= 0 || H <= 0 || N <= 0) return 0;
    return (size_t)2 * B * H * N * sizeof(float);
}

}  // extern "C"

namespace {

// Validation of attn_bwd's tensors and, with use_ws, of its workspace
// (attn_bwd_noalloc has none).  *work is set to false for an empty problem
// (valid, nothing to launch).
int validate_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                 const float* lse, void* dQ, void* dK, void* dV, int B, int H, int Hkv, int N,
                 int d, float scale, bool use_ws, size_t need, const void* workspace,
                 size_t workspace_bytes, bool* work)
{
    *work = false;
    int st = check_attn_shape(B, H, N, d, scale, 2);
    if (st != OSM_OK || B == 0 || H == 0 || N == 0) return st;
    if ((st = check_heads(H, Hkv)) != OSM_OK) return st;
    if (!Q || !K || !V || !O || !dO || !lse || !dQ || !dK || !dV || (use_ws && !workspace))
        return OSM_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) ||
        !aligned(dO, 16) || !aligned(lse, 4) || !aligned(dQ, 16) || !aligned(dK, 16) ||
        !aligned(dV, 16) || (workspace && !aligned(workspace, 16)))
        return OSM_ERR_ALIGN;
    const long long bh = (long long)B * H;
    if (!use_ws) need = 0;
    if (workspace_bytes < need) return OSM_ERR_WORKSPACE;
    const size_t tb = (size_t)bh * N * d * 2, lb = (size_t)bh * N * sizeof(float);
    const size_t kvb = (size_t)B * Hkv * N * d * 2;
    const void* outs[3] = {dQ, dK, dV};
    const size_t out_bytes[3] = {tb, kvb, kvb};
    const void* ins[6] = {Q, K, V, O, dO, lse};
    const size_t in_bytes[6] = {tb, kvb, kvb, tb, tb, lb};
    for (int a = 0; a < 3; ++a) {
        for (int b = 0; b < 6; ++b)
            if (overlaps(outs[a], out_bytes[a], ins[b], in_bytes[b])) return OSM_ERR_ALIAS;
        for (int b = a + 1; b < 3; ++b)
            if (overlaps(outs[a], out_bytes[a], outs[b], out_bytes[b])) return OSM_ERR_ALIAS;
        if (overlaps(outs[a], out_bytes[a], workspace, need)) return OSM_ERR_ALIAS;
    }
    for (int b = 0; b < 6; ++b)
        if (overlaps(workspace, need, ins[b], in_bytes[b])) return OSM_ERR_ALIAS;
    *work = true;
    return OSM_OK;
}

}  // namespace

extern "C" {

int attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
             const float* lse, void* dQ, void* dK, void* dV, int B, int H, int Hkv, int N, int d,
             float scale, int causal, void* workspace, size_t workspace_bytes, void* stream)
{
    bool work = false;
    int st = validate_bwd(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Hkv, N, d, scale, true,
                          attn_bwd_workspace_bytes(B, H, N), workspace, workspace_bytes, &work);
    if (st != OSM_OK || !work) return st;
    if ((st = check_device()) != OSM_OK) return st;
    const long long bh = (long long)B * H;
    float* Dl = static_cast<float*>(workspace);
    float* Lc = Dl + (size_t)bh * N;
    return finish(osm::launch_attn_bwd_bf16(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Hkv, N, d, scale,
                                            causal != 0, Dl, Lc, static_cast<hipStream_t>(stream)));
}

int attn_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                     const float* lse, void* dQ, void* dK, void* dV, int B, int H, int Hkv, int N,
                     int d, float scale, int causal, void* stream)
{
    bool work = false;
    int st = validate_bwd(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Hkv, N, d, scale, false, 0,
                          nullptr, 0, &work);
    if (st != OSM_OK || !work) return st;
    const long long rows = (long long)B * H * N;
    if (rows > OSM_NOALLOC_BWD_MAX_ROWS) return OSM_ERR_SCRATCH;
    if ((st = check_device()) != OSM_OK) return st;
    float* Dl = nullptr;
    if ((st = scratch_address(&Dl)) != OSM_OK) return st;
    // Same kernels as attn_bwd, with the row statistics in the static scratch
    // (D in rows 0 .. rows - 1, L log2 e after them).  The delta kernel writes
    // every value the later kernels read, so nothing needs clearing.
    float* Lc = Dl + rows;
    return finish(osm::launch_attn_bwd_bf16(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Hkv, N, d, scale,
                                            causal != 0, Dl, Lc, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Workspace of the split backward: the row statistics (2 B H N fp32, padded
// to 256 bytes), then the fp32 partials of dK and dV ([2][nsplit][B Hkv][N][d])
// and of dQ ([nsplit][B H][N][d]).
size_t bwd_stats_bytes(long long bh, int N)
{
    return ((size_t)2 * bh * N * sizeof(float) + 255) & ~(size_t)255;
}

size_t bwd_split_workspace(int nsplit, long long bh, long long bhkv, int N, int d)
{
    return bwd_stats_bytes(bh, N) + (size_t)nsplit * (2 * bhkv + bh) * N * d * sizeof(float);
}

}  // namespace

extern "C" {

int attn_bwd_split_plan(int B, int H, int Hkv, int N, int d, int causal, int nsplit,
                        int* nsplit_out, size_t* workspace_bytes)
{
    if (!nsplit_out || !workspace_bytes) return OSM_ERR_NULL;
    if (B < 0 || H < 0 || N < 0) return OSM_ERR_SIZE;
    if (d != 64 && d != 128) return OSM_ERR_HEAD_DIM;
    if (nsplit < 0 || nsplit > osm::kMaxSplits) return OSM_ERR_SPLITS;
    const long long bh = (long long)B * H;
    if (bh > INT_MAX) return OSM_ERR_SIZE;
    if (bh > 0 && N > 0) {
        const int st = check_heads(H, Hkv);
        if (st != OSM_OK) return st;
    }
    // The count follows the key/value heads: the dK/dV grid has B Hkv key
    // blocks per row of blocks, and with grouped queries it is the one that
    // leaves compute units idle.
    if (nsplit == 0)
        nsplit = (bh == 0 || N == 0) ? 1 : osm::attn_bwd_split_auto((int)((long long)B * Hkv), N, d, causal != 0);
    *nsplit_out = nsplit;
    *workspace_bytes = (bh == 0 || N == 0) ? 0
                       : nsplit == 1       ? attn_bwd_workspace_bytes(B, H, N)
                                           : bwd_split_workspace(nsplit, bh, (long long)B * Hkv, N, d);
    return OSM_OK;
}

int attn_bwd_split(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                   const float* lse, void* dQ, void* dK, void* dV, int B, int H, int Hkv, int N,
                   int d, float scale, int causal, int nsplit, void* workspace,
                   size_t workspace_bytes, void* stream)
{
    if (nsplit < 0 || nsplit > osm::kMaxSplits) return OSM_ERR_SPLITS;
    const long long bh = (long long)B * H;
    if (B > 0 && H > 0 && N > 0 && bh <= INT_MAX && nsplit == 0 && check_heads(H, Hkv) == OSM_OK)
        nsplit = osm::attn_bwd_split_auto((int)((long long)B * Hkv), N, d, causal != 0);
    if (nsplit <= 1)
        return attn_bwd(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Hkv, N, d, scale, causal, workspace,
                        workspace_bytes, stream);
    // Sizes are checked by validate_bwd first; the workspace size formula
    // needs them non-negative.
    int st = check_attn_shape(B, H, N, d, scale, 2);
    if (st != OSM_OK || B == 0 || H == 0 || N == 0) return st;
    if ((st = check_heads(H, Hkv)) != OSM_OK) return st;
    const size_t need = bwd_split_workspace(nsplit, bh, (long long)B * Hkv, N, d);
    bool work = false;
    st = validate_bwd(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Hkv, N, d, scale, true, need,
                      workspace, workspace_bytes, &work);
    if (st != OSM_OK || !work) return st;
    // The split kernels launch ceil(N / 256) * nsplit * B * H workgroups of
    // 512 work-items, and a dispatch counts at most 2^32 - 1 work-items;
    // offsets into one fp32 partial slice are 32-bit.
    if (bh * ((N + 255) / 256) * nsplit * 512 > UINT32_MAX || (long long)N * d * 4 > UINT32_MAX)
        return OSM_ERR_SIZE;
    if ((st = check_device()) != OSM_OK) return st;
    float* Dl = static_cast<float*>(workspace);
    float* Lc = Dl + (size_t)bh * N;
    float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + bwd_stats_bytes(bh, N));
    return finish(osm::launch_attn_bwd_bf16_split(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Hkv, N, d,
                                                  scale, causal != 0, nsplit, Dl, Lc, part,
                                                  static_cast<hipStream_t>(stream)));
}

int attn_bwd_varlen(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                    const float* lse, void* dQ, void* dK, void* dV, const int* cu_seqlens, int B,
                    int H, int Hkv, int total, int max_seqlen, int d, float scale, int causal,
                    void* workspace, size_t workspace_bytes, void* stream)
{
    if (B < 0 || H < 0 || total < 0 || max_seqlen < 0) return OSM_ERR_SIZE;
    if (d != 64 && d != 128) return OSM_ERR_HEAD_DIM;
    if (!(std::isfinite(scale) && scale > 0.f)) return OSM_ERR_SCALE;
    if (B == 0 || H == 0 || total == 0 || max_seqlen == 0) return OSM_OK;
    int st = check_attn_shape(B, H, max_seqlen, d, scale, 2);
    if (st != OSM_OK) return st;
    if ((st = check_heads(H, Hkv)) != OSM_OK) return st;
    if (!Q || !K || !V || !O || !dO || !lse || !dQ || !dK || !dV || !cu_seqlens || !workspace)
        return OSM_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) ||
        !aligned(dO, 16) || !aligned(lse, 4) || !aligned(dQ, 16) || !aligned(dK, 16) ||
        !aligned(dV, 16) || !aligned(cu_seqlens, 4) || !aligned(workspace, 16))
        return OSM_ERR_ALIGN;
    const size_t need = attn_bwd_workspace_bytes(1, H, total);
    if (workspace_bytes < need) return OSM_ERR_WORKSPACE;
    const size_t tb = (size_t)H * total * d * 2, kvb = (size_t)Hkv * total * d * 2;
    const size_t lb = (size_t)H * total * sizeof(float), cb = (size_t)(B + 1) * sizeof(int);
    const void* outs[3] = {dQ, dK, dV};
    const size_t out_bytes[3] = {tb, kvb, kvb};
    const void* ins[7] = {Q, K, V, O, dO, lse, cu_seqlens};
    const size_t in_bytes[7] = {tb, kvb, kvb, tb, tb, lb, cb};
    for (int a = 0; a < 3; ++a) {
        for (int b = 0; b < 7; ++b)
            if (overlaps(outs[a], out_bytes[a], ins[b], in_bytes[b])) return OSM_ERR_ALIAS;
        for (int b = a + 1; b < 3; ++b)
            if (overlaps(outs[a], out_bytes[a], outs[b], out_bytes[b])) return OSM_ERR_ALIAS;
        if (overlaps(outs[a], out_bytes[a], workspace, need)) return OSM_ERR_ALIAS;
    }
    for (int b = 0; b < 7; ++b)
        if (overlaps(workspace, need, ins[b], in_bytes[b])) return OSM_ERR_ALIAS;
    if ((st = check_device()) != OSM_OK) return st;
    float* Dl = static_cast<float*>(workspace);
    float* Lc = Dl + (size_t)H * total;
    return finish(osm::launch_attn_bwd_bf16_varlen(Q, K, V, O, dO, lse, dQ, dK, dV, cu_seqlens, B,
                                                   H, Hkv, total, max_seqlen, d, scale,
                                                   causal != 0, Dl, Lc,
                                                   static_cast<hipStream_t>(stream)));
}

const char* osm_status_str(int status)
{
    switch (status) {
    case OSM_OK: return "ok";
    case OSM_ERR_NULL: return "a required pointer is NULL";
    case OSM_ERR_SIZE: return "a size is negative or the problem is too large";
    case OSM_ERR_HEAD_DIM: return "head dimension d must be 64 or 128";
    case OSM_ERR_SCALE: return "scale must be finite and > 0";
    case OSM_ERR_ALIAS: return "an output buffer overlaps another buffer";
    case OSM_ERR_ALIGN: return "a pointer is not aligned as required";
    case OSM_ERR_DEVICE: return "the current device is not a gfx950 (MI355X) GPU";
    case OSM_ERR_HIP: return "the HIP runtime reported an error";
    case OSM_ERR_SPLITS: return "the number of key splits is out of range";
    case OSM_ERR_WORKSPACE: return "the workspace is smaller than the call requires";
    case OSM_ERR_HEADS: return "key/value heads must divide the query heads (1 <= Hkv <= H)";
    case OSM_ERR_SCRATCH: return "the problem needs more than the library's static scratch";
    case OSM_ERR_SIGNS: return "every rotation sign must be +1 or -1";
    default: return "unknown status";
    }
}

}  // extern "C"
