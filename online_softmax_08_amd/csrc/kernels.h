// kernels.h -- internal launch entry points of the HIP kernels (host side).
// Arguments are validated by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>

namespace osm {

// Row softmax dispatch thresholds: wave-per-row up to this N, then one
// workgroup per register-resident row, then the two-read online kernel.
constexpr int kSoftmaxWaveMaxN = 1024;
constexpr int kSoftmaxBlockMaxN = 32768;

hipError_t launch_row_softmax(const float* x, float* y, int B, int N, hipStream_t stream);

// Q, O: [B*H][N][d] row-major; K, V: [B*Hkv][N][d] (Hkv divides H; query
// head h reads key/value head h / (H / Hkv)); lse: [B*H][N].  d is 64 or 128.
hipError_t launch_attn_fwd_bf16(const void* Q, const void* K, const void* V, void* O,
                                float* lse, int B, int H, int Hkv, int N, int d, float scale,
                                bool causal, hipStream_t stream);
// Packed variable-length sequences: Q, K, V, O [H][total][d], lse [H][total],
// cu: device int32 [B + 1] row offsets, sequences no longer than max_seqlen.
hipError_t launch_attn_fwd_bf16_varlen(const void* Q, const void* K, const void* V, void* O,
                                       float* lse, const int* cu, int B, int H, int Hkv, int total,
                                       int max_seqlen, int d, float scale, bool causal,
                                       hipStream_t stream);
// Split-KV forward.  opart: bf16 [nsplit][B*H][N][d], lpart: fp32
// [nsplit][B*H][N] (workspace); 1 <= nsplit <= kMaxSplits.
constexpr int kMaxSplits = 64;
hipError_t launch_attn_fwd_bf16_split(const void* Q, const void* K, const void* V, void* O,
                                      float* lse, int B, int H, int Hkv, int N, int d, float scale,
                                      bool causal, int nsplit, __bf16* opart, float* lpart,
                                      hipStream_t stream);
// The number of key ranges the split-KV forward picks when asked to choose.
int attn_splitkv_auto(int BH, int N, int d, bool causal);
// Merge of S partials (opart [S][rows][d] fp32, lpart [S][rows]) into O (bf16
// [rows][d]) and lse ([rows]).
hipError_t launch_attn_combine(const float* opart, const float* lpart, void* O, float* lse, int S,
                               long long rows, int d, hipStream_t stream);
// Backward: dQ (bf16 [B*H][N][d]), dK, dV (bf16 [B*Hkv][N][d]) from Q, O, dO
// ([B*H][N][d]), K, V ([B*Hkv][N][d]) and the forward's lse; Dl and Lc are
// fp32 [B*H][N] workspace rows.
hipError_t launch_attn_bwd_bf16(const void* Q, const void* K, const void* V, const void* O,
                                const void* dO, const float* lse, void* dQ, void* dK, void* dV,
                                int B, int H, int Hkv, int N, int d, float scale, bool causal,
                                float* Dl, float* Lc, hipStream_t stream);
// Split backward (dense): part is fp32 workspace of
// (2 nsplit B Hkv + nsplit B H) N d values; 1 <= nsplit <= kMaxSplits.
hipError_t launch_attn_bwd_bf16_split(const void* Q, const void* K, const void* V, const void* O,
                                      const void* dO, const float* lse, void* dQ, void* dK,
                                      void* dV, int B, int H, int Hkv, int N, int d, float scale,
                                      bool causal, int nsplit, float* Dl, float* Lc, float* part,
                                      hipStream_t stream);
// The number of ranges the split backward picks when asked to choose.
int attn_bwd_split_auto(int BH, int N, int d, bool causal);
// Backward over packed sequences: Q, O, dO, dQ [H][total][d], K, V, dK, dV
// [Hkv][total][d], lse, Dl, Lc [H][total].
hipError_t launch_attn_bwd_bf16_varlen(const void* Q, const void* K, const void* V, const void* O,
                                       const void* dO, const float* lse, void* dQ, void* dK,
                                       void* dV, const int* cu, int B, int H, int Hkv, int total,
                                       int max_seqlen, int d, float scale, bool causal, float* Dl,
                                       float* Lc, hipStream_t stream);
// fp8 forward: Q [B*H][N][d], K, V [B*Hkv][N][d] as OCP FP8 E4M3 bytes, O
// bf16 and lse fp32 as for the bf16 call; qk_scale = scale * q_scale *
// k_scale multiplies the raw fp8 dot products, v_scale the output.
hipError_t launch_attn_fwd_fp8(const void* Q, const void* K, const void* V, void* O, float* lse,
                               int B, int H, int Hkv, int N, int d, float qk_scale, float v_scale,
                               bool causal, hipStream_t stream);
// Block-quantized fp8 forward: Q, K, V codes as above; Qs [B*H][N][d/32] and
// Ks [B*Hkv][N][d/32] hold one E8M0 scale byte per 32 head columns of a row,
// Vs [B*Hkv][ceil(N/32)][d] one per 32 keys of a column; scale is the softmax
// scale.
hipError_t launch_attn_fwd_fp8_mx(const void* Q, const void* Qs, const void* K, const void* Ks,
                                  const void* V, const void* Vs, void* O, float* lse, int B, int H,
                                  int Hkv, int N, int d, float scale, bool causal, hipStream_t stream);
// Block quantization of bf16 [rows][d] (d = 64 or 128) to E4M3 codes with one
// E8M0 scale per 32 columns of a row ([rows][d/32]), after the random-sign
// Hadamard rotation when rot (bit t of neg_hi:neg_lo set: column t negated).
hipError_t launch_fp8_quant_rows(const void* X, void* codes, void* scales, long long rows, int d,
                                 bool rot, uint64_t neg_lo, uint64_t neg_hi, hipStream_t stream);
// Block quantization of bf16 [slices][n][d] with one scale per 32 rows of a
// column of each slice ([slices][ceil(n/32)][d]).
hipError_t launch_fp8_quant_cols(const void* X, void* codes, void* scales, long long slices,
                                 int n, int d, hipStream_t stream);
hipError_t launch_attn_fwd_f32(const float* Q, const float* K, const float* V, float* O,
                               float* lse, int BH, int N, int d, float scale, bool causal,
                               hipStream_t stream);

}  // namespace osm
