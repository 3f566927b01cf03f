/*
 * osm.h -- C ABI of the MI355X (gfx950) online-softmax attention library.
 *
 * The operations, all defined on the source pages:
 *
 *  attn_fwd / attn_fwd_f32
 *    Exact attention forward O = softmax(scale * Q K^T) V for every
 *    (batch, head), with an optional causal mask, plus the per-row
 *    logsumexp.  Definition: "Lesson 22: why softmax is hard to make
 *    efficient, and how FlashAttention reduces memory traffic", sections 12-13
 *    (the attention product) and 34 (causal mask: key j is hidden from query
 *    i when j > i); "Moving less: four generations of FlashAttention",
 *    section 1.2 (S = QK^T / sqrt(d), P = softmax(S), O = PV) and section 2.4
 *    (the row statistic L = m + log l, natural log, of the scaled scores).
 *    The computation is the fused, tiled online softmax of Lesson 22,
 *    sections 21-24 and 32: S and P are never written to memory.
 *
 *  attn_fwd_gqa
 *    The same attention with fewer key/value heads than query heads
 *    (grouped- and multi-query attention, among the variants a production
 *    kernel must serve in "Operator fusion seen through FlashAttention",
 *    the list of interface semantics): query head h attends with key/value
 *    head h / (H / Hkv).  Every key/value-head argument below has this
 *    meaning; Hkv = H is attn_fwd.
 *
 *  attn_fwd_fp8
 *    The same attention with Q, K and V stored as 8-bit floats (OCP FP8
 *    E4M3) and one scale per tensor, both products on the fp8 matrix cores:
 *    the FP8 variant of "Moving less: four generations of FlashAttention",
 *    section 4.6.  Its own tolerance, from the rounding of the
 *    probabilities to fp8, is stated with the function below.
 *
 *  fp8_quantize_rows / fp8_quantize_cols / attn_fwd_fp8_mx
 *    The two accuracy devices of the same FP8 section: block quantization
 *    (one scale per block of elements instead of one per tensor) and
 *    incoherent processing (Q and K multiplied by one random orthogonal
 *    matrix, random signs times a Hadamard matrix, before quantizing; the
 *    product Q K^T is unchanged because the matrix times its transpose is
 *    the identity).  The blocks are 32 elements along each contracted axis
 *    with power-of-two scales, the block format the gfx950 fp8 matrix cores
 *    apply themselves; attn_fwd_fp8_mx is the attention on such inputs.
 *
 *  attn_fwd_varlen
 *    The same attention over a batch of sequences of different lengths
 *    packed end to end with no padding: the padding mask of Lesson 22,
 *    section 35 (keys past a sequence's length get weight 0) realised as the
 *    packed, variable-length layout that section recommends.
 *
 *  attn_fwd_splitkv / attn_combine
 *    The same attention with the keys of each query block divided into
 *    several ranges computed in parallel, each yielding a normalised partial
 *    output and a partial logsumexp, which a second kernel merges.  The
 *    split is the occupancy device of "Operator fusion seen through
 *    FlashAttention", the list of risks, item 6 (split-KV with accumulated
 *    lse and output partials, then a combine); the merge is the rule for
 *    joining two partial softmax states of Lesson 22, section 22.
 *
 *  attn_bwd
 *    The gradients dQ, dK, dV of the scalar sum(dO * O) for attn_fwd's
 *    output O.  The probabilities are recomputed from Q, K and the forward's
 *    lse instead of being stored (Lesson 22, sections 30-31; "Moving less",
 *    section 2.4, P_ij = exp(S_ij - L_i)); the gradient formulas themselves
 *    are the chain rule through O = P V and the row softmax.
 *
 *  row_softmax
 *    Numerically stable softmax of each row of x [B][N]:
 *    y[b][j] = exp(x[b][j] - m_b) / sum_t exp(x[b][t] - m_b),
 *    m_b = max_t x[b][t].  Definition: Lesson 22, sections 2-3.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers (HIP device memory), owned by the
 *    caller; the library never allocates, frees or retains them.
 *  - Layouts are contiguous row-major: Q, K, V, O are [B][H][N][d]
 *    (d fastest), lse is [B][H][N]; x and y are [B][N].
 *  - Q, K, V, O must be 16-byte aligned (for bf16 also implied by d being 64
 *    or 128 once the base is aligned).  lse needs 4-byte alignment.
 *  - `stream` is a hipStream_t passed as void*; NULL means the default
 *    stream.  Every call only enqueues work and returns without
 *    synchronising; results are ready when the stream reaches that point.
 *  - Arguments are validated on the host before any HIP call; an invalid call
 *    enqueues nothing and returns a nonzero osm_status.  A launch failure
 *    returns OSM_ERR_HIP.  The library keeps no mutable global state except a
 *    per-device cache of the architecture check, so calls are thread-safe.
 *  - Empty problems (B, H or N equal to 0) return OSM_OK and enqueue nothing;
 *    their pointers may then be NULL.
 */
#ifndef OSM_H
#define OSM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    OSM_OK = 0,
    OSM_ERR_NULL = 1,     /* a required pointer is NULL                        */
    OSM_ERR_SIZE = 2,     /* a size is negative or the problem is too large    */
    OSM_ERR_HEAD_DIM = 3, /* d is not 64 or 128                                */
    OSM_ERR_SCALE = 4,    /* scale is not finite and > 0                       */
    OSM_ERR_ALIAS = 5,    /* an output overlaps an input or the other output   */
    OSM_ERR_HIP = 6,      /* the HIP runtime reported an error at launch       */
    /* Codes added after the first seven for the checks the later entry points
     * and the device guard make: */
    OSM_ERR_ALIGN = 7,    /* a pointer is not aligned as required              */
    OSM_ERR_DEVICE = 8,   /* the current device is not a gfx950 GPU            */
    OSM_ERR_SPLITS = 9,   /* a split count is outside its documented range     */
    OSM_ERR_WORKSPACE = 10, /* workspace_bytes is below what the call requires */
    OSM_ERR_HEADS = 11,    /* Hkv is not a divisor of H in 1 .. H               */
    OSM_ERR_SCRATCH = 12,  /* the problem exceeds the static scratch's limit    */
    OSM_ERR_SIGNS = 13     /* a rotation sign is neither +1 nor -1              */
} osm_status;

/*
 * attn_fwd -- bf16 inputs, fp32 accumulation.
 *   Q, K, V : const bf16 [B][H][N][d]   (bf16 = IEEE binary32 upper half)
 *   O       : bf16 [B][H][N][d], written with round-to-nearest-even
 *   lse     : fp32 [B][H][N], lse[i] = max_j s_ij + ln(sum_j exp(s_ij - max_j s_ij))
 *             over the visible keys j, with s_ij = scale * q_i . k_j
 *   B, H, N : batch, heads, sequence length (queries = keys = N), >= 0
 *   d       : head dimension, 64 or 128
 *   scale   : score scale, finite and > 0 (usually 1/sqrt(d))
 *   causal  : nonzero hides key j from query i when j > i
 *   stream  : hipStream_t or NULL
 * The probabilities are rounded to bf16 before they multiply V (the row sums
 * use the unrounded fp32 values).  Returns an osm_status.
 */
int attn_fwd(const void* Q, const void* K, const void* V, void* O, float* lse,
             int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * attn_fwd_f32 -- the same operation with fp32 Q, K, V and O (fp32 matrix
 * cores, fp32 probabilities).  Same arguments and errors as attn_fwd.
 */
int attn_fwd_f32(const float* Q, const float* K, const float* V, float* O, float* lse,
                 int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * attn_fwd_gqa -- attn_fwd with Hkv key/value heads.
 *   Q, O : bf16 [B][H][N][d];  K, V : bf16 [B][Hkv][N][d];  lse : fp32 [B][H][N]
 *   Hkv  : 1 <= Hkv <= H, H % Hkv == 0 (else OSM_ERR_HEADS); query head h
 *          reads key/value head h / (H / Hkv)
 * Other arguments, alignment and errors as for attn_fwd.  With Hkv = H the
 * result is bitwise that of attn_fwd.
 */
int attn_fwd_gqa(const void* Q, const void* K, const void* V, void* O, float* lse,
                 int B, int H, int Hkv, int N, int d, float scale, int causal, void* stream);

/*
 * attn_fwd_fp8 -- attention forward on fp8 inputs.
 *   Q : uint8 [B][H][N][d], K, V : uint8 [B][Hkv][N][d], each byte an OCP
 *       FP8 E4M3 code (sign, 4 exponent bits with bias 7, 3 mantissa bits;
 *       subnormals below exponent 1; S.1111.111 is NaN, no infinities; the
 *       largest finite magnitude is 448).  Element x of Q stands for
 *       decode(x) * q_scale, of K for decode(x) * k_scale, of V for
 *       decode(x) * v_scale.  NaN codes give undefined results.
 *   q_scale, k_scale, v_scale : finite and > 0 (else OSM_ERR_SCALE), as is
 *       scale * q_scale * k_scale
 *   O   : bf16 [B][H][N][d], lse : fp32 [B][H][N]: the attention of attn_fwd
 *       (with the same scale and mask) on the decoded, scaled inputs.
 *   Hkv, B, H, N, d, scale, causal, stream : as for attn_fwd_gqa.
 * The matrix cores form the fp8 products exactly and sum each 64-term block
 * at reduced precision (measured on gfx950: up to ~2e-5 of the block's sum
 * of |products| on Gaussian data, 1e-4 on arbitrary codes), so a score
 * errs by up to ~1e-4 * scale * sum_d |q_d k_d| and lse by as much.  The
 * probabilities enter the P V product rounded to fp8 (E4M3, relative error
 * up to 2^-4; each is kept at or below 28 times its row's running maximum,
 * and values below 2^-13 of it may round to zero), and the row sums use them
 * unrounded, so each element of O carries an error of about
 * 2^-4 sqrt(sum_j (P_ij V_jt)^2 / 3) (a sum of independent roundings)
 * besides the score error's share and its bf16 rounding.
 * Q, K, V, O need 16-byte alignment, lse 4; O and lse may not overlap the
 * inputs or each other.  Returns an osm_status.
 */
int attn_fwd_fp8(const void* Q, const void* K, const void* V, float q_scale, float k_scale,
                 float v_scale, void* O, float* lse, int B, int H, int Hkv, int N, int d,
                 float scale, int causal, void* stream);

/*
 * Block-quantized FP8 ("Moving less: four generations of FlashAttention",
 * section 4.6, block quantization and incoherent processing).
 *
 * A block is 32 consecutive elements along the axis the attention contracts:
 * 32 head columns of one row (Q, K), or 32 consecutive rows of one column of
 * a [N][d] slice (V; the last block of a slice may be shorter).  Its scale
 * is a power of two 2^e stored as the byte e + 127 (E8M0): e is the smallest
 * integer with amax <= 448 * 2^e, amax the block's largest magnitude (e = 0
 * for an all-zero block), and each element is stored as the E4M3 code of
 * x / 2^e, rounded to nearest with ties to the even code.  A code x with
 * scale byte s stands for decode(x) * 2^(s - 127).  Scale byte 255 is NaN.
 */

/*
 * fp8_quantize_rows -- block quantization along rows, optionally after the
 * random-sign Hadamard rotation.
 *   X      : bf16 [rows][d] (device), d = 64 or 128 (else OSM_ERR_HEAD_DIM);
 *            finite values.
 *   signs  : NULL (no rotation), or a HOST array of d values, each +1 or -1
 *            (else OSM_ERR_SIGNS): the rows are first replaced by
 *            x diag(signs) H / sqrt(d), H the d x d Hadamard matrix of
 *            Sylvester's doubling construction (entry (t, k) =
 *            (-1)^popcount(t & k)), computed in fp32 by the fast
 *            Walsh-Hadamard transform.  Use the same signs for Q and K.
 *   codes  : uint8 [rows][d] (device, 8-byte aligned), the E4M3 codes.
 *   scales : uint8 [rows][d / 32] (device), the block scale bytes.
 *   rows >= 0 (else OSM_ERR_SIZE); rows = 0 enqueues nothing.
 * X must be 16-byte aligned; no two buffers may overlap (OSM_ERR_ALIAS).
 * Returns an osm_status.
 */
int fp8_quantize_rows(const void* X, const signed char* signs, void* codes, void* scales,
                      long long rows, int d, void* stream);

/*
 * fp8_quantize_cols -- block quantization along the rows of each column, the
 * layout attn_fwd_fp8_mx takes for V.
 *   X      : bf16 [slices][n][d] (device, 16-byte aligned), d = 64 or 128.
 *   codes  : uint8 [slices][n][d] (device, 8-byte aligned).
 *   scales : uint8 [slices][ceil(n / 32)][d] (device): byte (s, i, t) is the
 *            scale of rows 32 i .. min(32 i + 31, n - 1) of column t of
 *            slice s.
 *   slices, n >= 0 (else OSM_ERR_SIZE).  No two buffers may overlap.
 * Returns an osm_status.
 */
int fp8_quantize_cols(const void* X, void* codes, void* scales, long long slices, int n, int d,
                      void* stream);

/*
 * attn_fwd_fp8_mx -- attention forward on block-quantized fp8 inputs.
 *   Q : uint8 [B][H][N][d] codes, q_scales : uint8 [B][H][N][d / 32]
 *   K : uint8 [B][Hkv][N][d] codes, k_scales : uint8 [B][Hkv][N][d / 32]
 *   V : uint8 [B][Hkv][N][d] codes, v_scales : uint8 [B][Hkv][ceil(N/32)][d]
 *       (the layouts fp8_quantize_rows and fp8_quantize_cols write).
 *   O, lse, B, H, Hkv, N, d, scale, causal, stream : as for attn_fwd_fp8,
 *       with the values the codes and scales stand for as its inputs.
 * The matrix cores apply every block scale (exact: powers of two); the
 * rounding and summation error of attn_fwd_fp8 applies unchanged, with
 * sum_d |q_d k_d| taken over the decoded values.  When Q and K were rotated
 * with the same signs, O and lse are those of the unrotated attention (the
 * rotation is orthogonal) up to that error.  Q, K, V, O need 16-byte
 * alignment, lse 4; O and lse may not overlap any input or each other.
 * Returns an osm_status.
 */
int attn_fwd_fp8_mx(const void* Q, const void* q_scales, const void* K, const void* k_scales,
                    const void* V, const void* v_scales, void* O, float* lse, int B, int H,
                    int Hkv, int N, int d, float scale, int causal, void* stream);

/*
 * attn_fwd_varlen -- attn_fwd over packed variable-length sequences.
 *   Q, O       : bf16 [H][total][d]: head h's rows of every sequence, the
 *                sequences end to end (sequence b is rows cu_seqlens[b] ..
 *                cu_seqlens[b+1] - 1 of each head)
 *   K, V       : bf16 [Hkv][total][d], the same packing (Hkv as for
 *                attn_fwd_gqa)
 *   lse        : fp32 [H][total]
 *   cu_seqlens : DEVICE int32 [B + 1], cu_seqlens[0] = 0, nondecreasing,
 *                cu_seqlens[B] = total; read by the kernels, so the host
 *                cannot check it: the caller guarantees it.  Entries outside
 *                [0, total] are clamped and a sequence is cut at max_seqlen,
 *                so a malformed array gives wrong results but no access
 *                outside the tensors.
 *   B, H, total : sequences, heads, packed rows (all >= 0)
 *   max_seqlen : an upper bound of every sequence length (sets the grid)
 *   d, scale, causal, stream : as for attn_fwd; queries and keys of one
 *                sequence only see each other, causal counts positions
 *                within the sequence
 * Alignment: Q, K, V, O 16 bytes; lse and cu_seqlens 4.  O and lse may not
 * overlap the inputs, cu_seqlens or each other.  Empty problems (B, H,
 * total or max_seqlen 0) are a no-op.  With equal lengths the result is
 * bitwise that of attn_fwd on the same rows.  Returns an osm_status.
 */
int attn_fwd_varlen(const void* Q, const void* K, const void* V, void* O, float* lse,
                    const int* cu_seqlens, int B, int H, int Hkv, int total, int max_seqlen,
                    int d, float scale, int causal, void* stream);

/*
 * attn_fwd_splitkv_plan -- resolve a split count and size its workspace.
 *   B, H, N, d, causal : as for attn_fwd (d must be 64 or 128)
 *   nsplit             : 1 .. 64 key ranges, or 0 to let the library choose
 *                        (it splits only when 256-row query blocks alone
 *                        would leave compute units idle)
 *   *nsplit_out        : the count attn_fwd_splitkv will use for nsplit
 *   *workspace_bytes   : device bytes attn_fwd_splitkv needs for it:
 *                        nsplit * B * H * N * (2 * d + 4), or 0 when the
 *                        count is 1 (then the call is exactly attn_fwd)
 * Host only; touches no device.  Returns OSM_ERR_NULL for NULL out pointers,
 * OSM_ERR_SIZE, OSM_ERR_HEAD_DIM or OSM_ERR_SPLITS for bad sizes.
 */
int attn_fwd_splitkv_plan(int B, int H, int N, int d, int causal, int nsplit,
                          int* nsplit_out, size_t* workspace_bytes);

/*
 * attn_fwd_splitkv -- attn_fwd computed as nsplit parallel key ranges plus a
 * merge.  Q, K, V, O, lse, B, H, Hkv, N, d, scale, causal, stream as for
 * attn_fwd_gqa (Hkv = H for plain multi-head attention).
 *   nsplit          : 0 (library's choice) or 1 .. 64.  Each 256-row query
 *                     block divides its visible key tiles (64 keys each at
 *                     d = 128, 128 at d = 64) into nsplit near-equal
 *                     contiguous ranges; ranges past the last visible tile
 *                     are empty.
 *   workspace       : device memory of at least workspace_bytes as returned
 *                     by attn_fwd_splitkv_plan for the same arguments,
 *                     16-byte aligned, not overlapping any other argument;
 *                     may be NULL when the resolved count is 1.  The caller
 *                     owns it; its contents on entry do not matter and on
 *                     return are unspecified.  Calls that share a workspace
 *                     must be ordered on one stream.
 * O and lse satisfy attn_fwd's tolerance against the exact result; they are
 * not bitwise equal to attn_fwd's (each range's normalised output is kept in
 * bf16 in the workspace, its logsumexp in fp32, and the merge is computed in
 * fp32).  Returns an osm_status (OSM_ERR_WORKSPACE if workspace_bytes is too
 * small, OSM_ERR_SIZE if N * d * 2 does not fit in 32 bits).
 */
int attn_fwd_splitkv(const void* Q, const void* K, const void* V, void* O, float* lse,
                     int B, int H, int Hkv, int N, int d, float scale, int causal, int nsplit,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_combine -- merge S partial attention results over disjoint key sets.
 *   O_part   : const fp32 [S][B][H][N][d], partial s normalised over its keys
 *   lse_part : const fp32 [S][B][H][N], the partial logsumexps (finite, or -inf
 *              for a row of a partial that saw no key: its O_part row is then
 *              not read)
 *   O        : bf16 [B][H][N][d] = sum_s e^(lse_s - lse) O_s
 *   lse      : fp32 [B][H][N] = ln sum_s e^(lse_s); -inf (and O = 0) for a
 *              row whose every partial is -inf
 *   S        : 1 .. 64
 * Alignment: O_part 16 bytes, O 8, lse_part and lse 4.  Outputs may not
 * overlap the inputs or each other.  This is the merge step of attn_fwd_splitkv
 * and of attention whose keys are held in shards.  Returns an osm_status.
 */
int attn_combine(const float* O_part, const float* lse_part, void* O, float* lse, int S,
                 int B, int H, int N, int d, void* stream);

/*
 * attn_bwd_workspace_bytes -- device bytes attn_bwd needs as workspace:
 *   2 * B * H * N * 4 (two fp32 values per query row), 0 for an empty problem.
 */
size_t attn_bwd_workspace_bytes(int B, int H, int N);

/*
 * attn_bwd -- backward pass of attn_fwd (bf16 inputs, fp32 accumulation).
 *   Q       : const bf16 [B][H][N][d], K, V : const bf16 [B][Hkv][N][d], the
 *             forward's inputs (Hkv as for attn_fwd_gqa; Hkv = H for
 *             attn_fwd)
 *   O       : const bf16 [B][H][N][d], the forward's output
 *   dO      : const bf16 [B][H][N][d], the gradient of the loss w.r.t. O
 *   lse     : const fp32 [B][H][N], the forward's logsumexp
 *   dQ      : bf16 [B][H][N][d];  dK, dV : bf16 [B][Hkv][N][d], written
 *             (round-to-nearest-even): dV = P^T dO, dQ = scale dS K,
 *             dK = scale dS^T Q with P_ij = exp(scale q_i.k_j - lse_i) over
 *             the visible keys and dS_ij = P_ij (dO_i.v_j - sum_t dO_it O_it);
 *             a key/value head's dK and dV sum over the query heads that
 *             read it
 *   B, H, Hkv, N, d, scale, causal : as for the forward call
 *   workspace : device memory of at least attn_bwd_workspace_bytes(B, H, N),
 *             16-byte aligned, caller-owned, contents irrelevant on entry
 *   stream  : hipStream_t or NULL
 * The probabilities and dS are rounded to bf16 before they enter the dV, dK
 * and dQ products.  Q, K, V, O, dO, dQ, dK, dV need 16-byte alignment, lse 4.
 * dQ, dK, dV may overlap neither each other, nor any input, nor the
 * workspace.  The result is deterministic (no atomic accumulation).  Returns
 * an osm_status (OSM_ERR_WORKSPACE if workspace_bytes is too small).
 */
int attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
             const float* lse, void* dQ, void* dK, void* dV, int B, int H, int Hkv, int N, int d,
             float scale, int causal, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_bwd_split_plan -- resolve a split count for attn_bwd_split and size its
 * workspace.
 *   B, H, Hkv, N, d, causal : as for attn_bwd (d must be 64 or 128)
 *   nsplit             : 1 .. 64 ranges, or 0 to let the library choose (it
 *                        splits only when 256-row blocks of the B Hkv
 *                        key/value slices would leave compute units idle, so
 *                        grouped queries split sooner)
 *   *nsplit_out        : the count attn_bwd_split will use for nsplit
 *   *workspace_bytes   : device bytes attn_bwd_split needs for it: for a
 *                        count of 1 attn_bwd_workspace_bytes(B, H, N) (the
 *                        call is then exactly attn_bwd), otherwise
 *                        round_up(2 B H N 4, 256) + nsplit (2 B Hkv + B H) N d 4
 * Host only; touches no device.  Returns OSM_ERR_NULL for NULL out pointers,
 * OSM_ERR_SIZE, OSM_ERR_HEAD_DIM, OSM_ERR_HEADS or OSM_ERR_SPLITS for bad
 * sizes.
 */
int attn_bwd_split_plan(int B, int H, int Hkv, int N, int d, int causal, int nsplit,
                        int* nsplit_out, size_t* workspace_bytes);

/*
 * attn_bwd_split -- attn_bwd for problems with few (batch, head) slices, the
 * backward counterpart of attn_fwd_splitkv (Lesson 22, sections 30-31, and
 * "Fast, memory-efficient and exact attention", section 3.3: the gradient
 * is a sum over key blocks for dQ and over query blocks for dK and dV, so
 * either sum can be cut into parts computed in parallel and added).  The
 * dK/dV workgroup of each 256-key block divides its query tiles (64 rows;
 * with Hkv < H those of all query heads of the group, head by head) into
 * nsplit near-equal contiguous ranges; the dQ workgroup of each 256-query
 * block divides its visible key tiles (64 keys) likewise.  Each range writes
 * its partial sums in fp32 to the workspace, and a last kernel adds the
 * nsplit partials of every element in range order and rounds to bf16.
 *   Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Hkv, N, d, scale, causal, stream :
 *             as for attn_bwd
 *   nsplit  : 0 (library's choice) or 1 .. 64; a count of 1 runs attn_bwd
 *   workspace : device memory of at least workspace_bytes as returned by
 *             attn_bwd_split_plan for the same arguments, 16-byte aligned,
 *             caller-owned, not overlapping any other argument; its contents
 *             on entry do not matter and on return are unspecified.  Calls
 *             that share a workspace must be ordered on one stream.
 * The gradients satisfy attn_bwd's tolerance against the exact result and
 * are deterministic for a given nsplit; they are not bitwise equal to
 * attn_bwd's (the products are summed in another order).  Returns an
 * osm_status (OSM_ERR_WORKSPACE if workspace_bytes is too small, OSM_ERR_SIZE
 * if N * d * 4 does not fit in 32 bits).
 */
int attn_bwd_split(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                   const float* lse, void* dQ, void* dK, void* dV, int B, int H, int Hkv, int N,
                   int d, float scale, int causal, int nsplit, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Query rows B * H * N up to which attn_bwd_noalloc runs (its scratch holds
 * two fp32 values per row: 32 MiB per GPU). */
#define OSM_NOALLOC_BWD_MAX_ROWS (1 << 22)

/*
 * attn_bwd_noalloc -- attn_bwd for callers that cannot allocate device
 * memory: code under HIP graph capture, tight training loops, harnesses that
 * forbid hipMalloc.  Same arguments, gradients, rounding, alignment and
 * overlap rules as attn_bwd, without the workspace: the row statistics live
 * in a static device array of the library (one per GPU, 32 MiB, held from the
 * library's first use on that GPU until the process ends).  The call
 * allocates nothing and calls no allocating routine.
 *   B * H * N must not exceed OSM_NOALLOC_BWD_MAX_ROWS (else
 *   OSM_ERR_SCRATCH, before any HIP call).
 * Every call on one GPU uses that GPU's single array: calls that overlap in
 * time on one GPU (different streams or host threads without ordering) race
 * and may return wrong gradients; calls ordered on one stream are safe.
 * Nothing in the array needs clearing between calls: each call writes every
 * value it reads.  Returns an osm_status.
 */
int attn_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                     const float* lse, void* dQ, void* dK, void* dV, int B, int H, int Hkv, int N,
                     int d, float scale, int causal, void* stream);

/*
 * attn_bwd_varlen -- attn_bwd for attn_fwd_varlen: packed sequences.
 *   Q, O, dO, dQ : bf16 [H][total][d];  K, V, dK, dV : bf16 [Hkv][total][d];
 *   lse : fp32 [H][total]; cu_seqlens, B, H, Hkv, total, max_seqlen, d,
 *   scale, causal : as for the attn_fwd_varlen call that produced O and lse
 *   workspace : at least attn_bwd_workspace_bytes(1, H, total) bytes,
 *              16-byte aligned, caller-owned
 * Gradients, rounding, alignment (cu_seqlens 4 bytes) and overlap rules as
 * for attn_bwd; a sequence's gradients depend on its own rows only.
 * Returns an osm_status.
 */
int attn_bwd_varlen(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                    const float* lse, void* dQ, void* dK, void* dV, const int* cu_seqlens,
                    int B, int H, int Hkv, int total, int max_seqlen, int d, float scale,
                    int causal, void* workspace, size_t workspace_bytes, void* stream);

/*
 * row_softmax -- stable softmax of each fp32 row.
 *   x : const fp32 [B][N];  y : fp32 [B][N]
 *   y may be exactly x (in place); any other overlap is OSM_ERR_ALIAS.
 *   Rows must hold finite values.  Any N >= 1 is accepted: rows up to 1024
 *   elements use one wave per row, up to 32768 one workgroup per
 *   register-resident row (one read, one write of each element), longer rows
 *   a two-read online kernel.
 */
int row_softmax(const float* x, float* y, int B, int N, void* stream);

/* Static, human-readable text for an osm_status value. */
const char* osm_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* OSM_H */
