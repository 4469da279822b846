/*
 * q3.h -- C ABI of the 3-bit FP8-codebook decode linear layer for MI355X (gfx950).
 *
 * The method (Hibana: Fast Agentic Inference on Unified-Memory Devices, section
 * "Model surgery", subsection "Three-bit weights"): every group of 32 consecutive
 * weights of a row is stored as 3-bit indices into an 8-entry FP8 codebook plus
 * one 8-bit scale per group, 3 + 8/32 = 3.25 bits per weight.  A decode or
 * speculative-verify step multiplies the dequantised matrix by a few token
 * activations:
 *
 *     w[n][k] = E4M3FN(codebook[n][code[n][k]]) * 2^(scale[n][k/32] - 127)
 *     y[m][n] = sum_k x[m][k] * w[n][k]          (x bf16, y fp32)
 *
 * Readings of the page used here: one codebook per output row (8 bytes, outside
 * the 3.25 bits/weight count); FP8 = OCP E4M3FN; scale = OCP-MX E8M0.
 *
 * ---- Packed format ------------------------------------------------------------
 *   groups G = k/32, padded to Gp = 4*ceil(k/128) (padding groups are zero);
 *   rows padded to a multiple of 16 (padding rows are zero).  Both planes are
 *   cut into tiles of 16 rows stored one after the other; inside a tile a row's
 *   groups form steps of 16 groups (512 weights); the last step holds
 *   p = 4, 8, 12 or 16 groups, i.e. q = p/4 quads of 4 groups.
 *   Row r is row i = r%16 of tile T = r/16; group g is slot t = g%4 of quad
 *   kb = (g%16)/4 of step s = g/16.
 *   code plane : a group's 96 code bits are 3 little-endian words.  Byte b
 *                (0..3) of word j (0..2) of a group with codes c[0..31]:
 *                  bits 0..2 = c[8j+b], bits 3..5 = c[8j+4+b],
 *                  bits 6..7 = bits 2j..2j+1 of (c[24+b] | c[28+b] << 3).
 *                Word j of (r, g) sits at byte
 *                  T*192*Gp + 3072*s + 16*(16*(q*j + kb) + i) + 4*t,
 *                so a tile is 192*Gp bytes, a full step 3072, and word j of a
 *                step is one contiguous run over (quad, row) in 16-byte pieces.
 *   scale plane: one E8M0 byte per group; the scale of (r, g) sits at byte
 *                  T*16*Gp + 256*s + 4*(16*kb + i) + t.
 *   codebook   : uint8 [n][8], E4M3FN bytes, entry j is what code j selects.
 *   x          : bf16 bit patterns, [m][ldx] (ldx >= k elements).
 *   y          : fp32, [m][ldy] (ldy >= n elements).
 *
 * ---- Conventions ----------------------------------------------------------------
 *   * Every pointer argument except the descriptor structs is a DEVICE pointer.
 *     Descriptor structs are host memory, read during the call only.
 *   * The caller owns all buffers; compute calls never allocate or free.
 *   * Every call is asynchronous on `stream` (a hipStream_t; NULL = the legacy
 *     default stream) and returns after launching.  Calls on different streams
 *     may run concurrently; the library keeps no mutable global state besides a
 *     once-per-device capability check.
 *   * Arguments are validated on the host before any HIP call; a rejected call
 *     launches nothing.  Launch failures are reported as Q3_ERR_HIP.
 *   * Size limits: each plane (q3_layout's plane bytes) and the activation block
 *     ((m-1)*ldx*2 + k*2 bytes) must stay below 2 GiB - 16 MiB
 *     (Q3_ERR_UNSUPPORTED_SHAPE otherwise); the code plane needs 16-byte
 *     alignment, the scale plane 4-byte, the codebook 8-byte; x needs
 *     ldx % 8 == 0 and 16-byte alignment, y 4-byte alignment
 *     (Q3_ERR_MISALIGNED).
 *   * Numerics: products are formed exactly and accumulated in fp32, so every
 *     output satisfies |y - y_exact| <= 1e-3 * sum_k |x_k w_k| for k <= 8192.
 *     Preconditions (not checked on the device): scale bytes in [16, 240],
 *     codebook bytes not NaN (0x7F/0xFF), x finite (bf16 subnormals are kept,
 *     not flushed).  The bound also takes the fp32 products and partial sums
 *     to stay inside fp32's range: no overflow, and none below its normal
 *     range (2^-126), where fp32 cannot keep the relative precision.  Code bits
 *     above bit 2 of q3_pack's input are ignored.
 */
#ifndef Q3_H
#define Q3_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q3_API __attribute__((visibility("default")))

typedef enum q3_status {
  Q3_OK = 0,
  Q3_ERR_INVALID_ARG = 1,        /* null pointer, negative size, bad mode          */
  Q3_ERR_UNSUPPORTED_SHAPE = 2,  /* k not a multiple of 32, m out of range, ...    */
  Q3_ERR_MISALIGNED = 3,         /* pointer or stride not aligned as required      */
  Q3_ERR_UNSUPPORTED_DEVICE = 4, /* current device is not gfx950                   */
  Q3_ERR_HIP = 5                 /* a HIP runtime call or kernel launch failed     */
} q3_status;

/* Sizes of the packed planes for an n x k matrix (host-only, no HIP call). */
typedef struct q3_layout_info {
  int64_t n, k;
  int64_t groups;            /* k/32                                          */
  int64_t padded_groups;     /* Gp = 4*ceil(k/128)                            */
  int64_t tiles;             /* ceil(n/16)                                    */
  int64_t code_tile_bytes;   /* 192*Gp: 16 rows x 12 bytes per group          */
  int64_t scale_tile_bytes;  /* 16*Gp                                         */
  int64_t code_plane_bytes;  /* tiles*code_tile_bytes                         */
  int64_t scale_plane_bytes; /* tiles*scale_tile_bytes                        */
  int64_t codebook_bytes;    /* 8*n                                           */
  int64_t payload_bytes;     /* n*k*13/32: codes + scales, 3.25 bits/weight   */
} q3_layout_info;

/* A packed matrix.  Pointers are device pointers to planes of q3_layout's
 * sizes; the code plane must be 16-byte aligned, the scale plane 4-byte
 * aligned, the codebook 8-byte aligned. */
typedef struct q3_matrix {
  int64_t n, k;
  const void* code_plane;
  const void* scale_plane;
  const void* codebook;
} q3_matrix;

/* A stack of E experts with one shape; expert e's planes start at
 * base + e*stride (bytes).  Strides keep the alignments of q3_matrix and are
 * at least the plane sizes. */
typedef struct q3_expert_stack {
  int64_t num_experts, n, k;
  const void* code_plane;
  int64_t code_expert_stride;
  const void* scale_plane;
  int64_t scale_expert_stride;
  const void* codebook;
  int64_t codebook_expert_stride;
} q3_expert_stack;

/* Human-readable name of a status code (static string). */
Q3_API const char* q3_status_string(q3_status s);

/* Packed-plane sizes for an n x k matrix (the 3.25 bits/weight format of
 * "Three-bit weights").  Q3_ERR_UNSUPPORTED_SHAPE unless k > 0, k % 32 == 0,
 * n >= 0.  Host only. */
Q3_API q3_status q3_layout(int64_t n, int64_t k, q3_layout_info* out);

/* Quantize fp32 weights under given per-row codebooks (the step before
 * q3_pack; "Model surgery" brings a model's weights to this format, the rule
 * is this library's reading):
 *   scale_bytes[r][g] = the smallest s in 0..254 with
 *       max_{k in group g} |w[r][k]| <= max_j |E4M3(codebook[r][j])| * 2^(s-127)
 *     (254 when none fits, i.e. an all-zero codebook; 0 for an all-zero group);
 *   codes[r][k] = argmin_j |w[r][k] - E4M3(codebook[r][j]) * 2^(s-127)|, equal
 *     distances (and repeated entries) to the lower index j.
 * Exact (bit-identical to exact rational arithmetic).
 *   w           [n][ldw] fp32, finite, |w| <= 2^64 (not checked); 16-byte
 *               aligned, ldw % 4 == 0, ldw >= k
 *   codebook    [n][8] E4M3FN bytes without NaN entries (not checked), 8-byte aligned
 *   codes       [n][ldc] uint8 out, 8-byte aligned, ldc % 8 == 0, ldc >= k
 *   scale_bytes [n][lds] uint8 out, lds >= k/32
 * k > 0, k % 32 == 0.  One launch; the codebooks may come from q3_fit_codebook.
 * A group whose largest magnitude is below max|codebook| * 2^-111 (an all-zero
 * group included) or above max|codebook| * 2^113 gets a scale byte outside
 * [16, 240], the range in which the products below dequantise exactly; their
 * outputs for rows with such groups are then not covered by the 1e-3 bound. */
Q3_API q3_status q3_quantize(const float* w, int64_t ldw, const uint8_t* codebook, int64_t n, int64_t k,
                             uint8_t* codes, int64_t ldc, uint8_t* scale_bytes, int64_t lds, void* stream);

/* Fit each row's codebook to its weights (the step before q3_quantize; the
 * page's "Three-bit weights" illustration fits the 8-entry FP8 codebook to the
 * weights it serves; the procedure is this library's reading, every decision
 * exact, so results are bit-identical to exact arithmetic):
 *   1. per group of 32: e = the smallest integer with max|w| <= 2^e (0 for an
 *      all-zero group);
 *   2. q = round(w * 2^(12 - e)), ties to even (integers in [-4096, 4096]);
 *   3. 1-D k-means (Lloyd) with 8 centroids on the row's q: start at the
 *      values of ranks floor((2i+1)K/16) of the sorted q; each q joins its
 *      nearest centroid (equal distances: lower index); a centroid with
 *      points becomes their exact mean, one without keeps its value; the
 *      centroids are re-sorted by value (stable); stop when no centroid
 *      changes or after 64 updates;
 *   4. codebook[r][i] = centroid i / 2^12 rounded to the nearest E4M3FN value,
 *      ties to the even significand (-0 for a negative centroid rounding to 0).
 * Entries come out in ascending order.
 *   w        [n][ldw] fp32, finite (not checked); 16-byte aligned, ldw % 4 == 0,
 *            ldw >= k; 0 < k <= 262144, k % 32 == 0
 *   codebook [n][8] uint8 out (E4M3FN), 8-byte aligned
 * One launch, one block per row. */
Q3_API q3_status q3_fit_codebook(const float* w, int64_t ldw, int64_t n, int64_t k, uint8_t* codebook,
                                 void* stream);

/* Pack unpacked codes and scales into the planes ("Three-bit weights": a
 * 3-bit index per weight, one 8-bit scale per group of 32).
 *   codes       [n][ldc] uint8, entries 0..7 (higher bits ignored), ldc >= k
 *   scale_bytes [n][lds] uint8 E8M0, lds >= k/32
 *   code_plane / scale_plane: outputs of q3_layout's plane sizes, aligned as
 *   in q3_matrix; every byte is written (padding as zero).
 * Bit-exact; one launch per plane. */
Q3_API q3_status q3_pack(const uint8_t* codes, int64_t ldc, const uint8_t* scale_bytes, int64_t lds,
                         int64_t n, int64_t k, void* code_plane, void* scale_plane, void* stream);

/* Inverse of q3_pack: codes_out [n][k] (values 0..7), scale_out [n][k/32]. */
Q3_API q3_status q3_unpack(const q3_matrix* w, uint8_t* codes_out, uint8_t* scale_out, void* stream);

/* y[m][n] = x[m][:] . w[n][:] for 1 <= m <= 8 tokens (decode and short
 * speculative-verify rounds), on the vector ALUs: the packed codes are streamed
 * once, looked up in the row's codebook with byte permutes, widened exactly to
 * bf16 with the group scale folded in, and dotted with x in fp32.  x is bf16
 * [m][ldx], y fp32 [m][ldy]; ldx, ldy in elements. */
Q3_API q3_status q3_gemv(const q3_matrix* w, const uint16_t* x, int64_t m, int64_t ldx,
                         float* y, int64_t ldy, void* stream);

/* Same product for 1 <= m <= 64 on the matrix cores: each 16-row tile of
 * codes is dequantised exactly to bf16 in registers and multiplied by the
 * activations with bf16 MFMA, fp32 accumulation.  m > 64 is rejected
 * (Q3_ERR_UNSUPPORTED_SHAPE); call again per 64-token slice. */
Q3_API q3_status q3_gemm_small_m(const q3_matrix* w, const uint16_t* x, int64_t m, int64_t ldx,
                                 float* y, int64_t ldy, void* stream);

/* Device workspace bytes q3_gemm_small_m_ws can use for an n x k matrix and m
 * tokens (host only, no device call); 0 when the product runs in one pass. */
Q3_API int64_t q3_gemm_small_m_workspace_bytes(int64_t n, int64_t k, int64_t m);

/* q3_gemm_small_m with a caller-owned workspace.  When the activations are too
 * large to be staged in LDS whole (m * k above about 68K elements) and the
 * matrix has few 16-row tiles, K is split over blocks: each split writes an
 * fp32 partial plane into the workspace and a second launch adds the planes
 * in split order, so results are run-to-run identical.  workspace: device
 * memory, 16-byte aligned, of at least q3_gemm_small_m_workspace_bytes(n, k, m)
 * bytes; NULL or a smaller workspace_bytes gives the one-pass product (never an
 * error).  Calls that overlap in time must not share a workspace.  Same
 * arguments, result tolerance and errors as q3_gemm_small_m otherwise. */
Q3_API q3_status q3_gemm_small_m_ws(const q3_matrix* w, const uint16_t* x, int64_t m, int64_t ldx, float* y,
                                    int64_t ldy, void* workspace, int64_t workspace_bytes, void* stream);

/* Router of an MoE verify round (Hibana page, "Adaptive speculation",
 * "Expert sharing": a verify round reads the weights of each expert chosen by
 * at least one of its drafted tokens).  logits fp32 [t][num_experts] (row pitch num_experts) ->
 * topk_ids int32 [t][topk], highest logit first, ties to the lower expert
 * index.  1 <= topk <= num_experts <= 1024, t >= 1; logits must not be NaN
 * (not checked).  One block per token ranks all experts at once. */
Q3_API q3_status q3_moe_topk(const float* logits, int32_t t, int32_t num_experts, int32_t topk,
                             int32_t* topk_ids, void* stream);

/* Router of a verify round with a shared expert budget ("Expert sharing": the
 * round gets a budget of experts and choices outside it are replaced by
 * choices inside it).  Reading of the policy: keep the `budget` experts with
 * the largest routing mass (sum over the t tokens of softmax(logits[i])[e];
 * equal mass: lower index), then give each token its top-k experts inside that
 * set by logit (highest first; equal logits: lower index).  topk_ids int32
 * [t][topk]; experts (may be NULL) int32 [budget], the kept set ascending.
 * 1 <= topk <= budget <= num_experts <= 1024, 1 <= t <= 1024; logits finite (not
 * checked).  Masses are fp32 sums in a fixed order (run-to-run identical).
 * One block per token; each block recomputes the round's masses. */
Q3_API q3_status q3_moe_budget_topk(const float* logits, int32_t t, int32_t num_experts, int32_t topk,
                                    int32_t budget, int32_t* topk_ids, int32_t* experts, void* stream);

/* Expert-grouped product of one verify round.  Only experts that appear in
 * topk_ids are read from memory, each once, and each is applied only to the
 * (token, slot) pairs routed to it:
 *     y[i][j][:] = W[topk_ids[i][j]] . xin(i, j)
 * where xin(i, j) = x[i][:] when x_by_slot == 0 (gate/up projection) or
 * x[i*topk + j][:] when x_by_slot == 1 (down projection, one activation per
 * pair).  x bf16 with row pitch ldx elements; y fp32 [t*topk][ldy].
 * topk_ids is a device int32 [t][topk] array (e.g. from q3_moe_topk); ids
 * outside [0, num_experts) are skipped (their rows of y are not written).
 * t*topk <= 64. */
Q3_API q3_status q3_grouped_expert_gemv(const q3_expert_stack* w, const uint16_t* x, int64_t ldx,
                                        int32_t x_by_slot, const int32_t* topk_ids, int32_t t,
                                        int32_t topk, float* y, int64_t ldy, void* stream);

/* Fused expert MLP of one verify round (Hibana page, "Adaptive speculation",
 * "Expert sharing": the experts a round reads, each run as its MLP on the
 * tokens routed to it).  Readings of the page, which gives no MLP detail:
 *   gate_up: per expert [gate rows 0..I-1; up rows I..2I-1] x K_in (n = 2I);
 *   down:    per expert H x I (k = I);
 *   h[i][j]  = silu(gate . x[i]) * (up . x[i]), silu(z) = z / (1 + e^-z), for
 *              expert e = topk_ids[i][j]; carried into the down product as two
 *              bf16 terms (|h - hi - lo| <= 2^-17 |h|), not rounded to bf16;
 *   out[i][:] = sum_j p[i][j] * (down_e . h[i][j]), p[i] = softmax over token
 *              i's routed logits logits[i][topk_ids[i][j]] (its top-k
 *              probabilities renormalised to sum 1).
 * x bf16 [t][ldx]; logits fp32 [t][ld_logits] (the router's, e.g. the input of
 * q3_moe_topk or q3_moe_budget_topk); out fp32 [t][ldo].  Ids outside
 * [0, num_experts) are skipped (weight 0, excluded from the softmax); a token
 * with none in range gets a row of zeros (every row of out is written).
 * Three launches (gate/up with the SwiGLU, down, combine), no host
 * synchronisation; only experts that appear in topk_ids are read, each once
 * per matrix.  Deterministic: the combine adds slots in slot order.
 * Shapes: gate_up.n % 64 == 0, down.k == gate_up.n / 2, same num_experts,
 * 1 <= t*topk <= 64.
 * workspace: device memory of at least q3_moe_mlp_workspace_bytes(...) bytes,
 * 256-byte aligned, any contents (it holds h and the per-pair outputs); calls
 * that overlap in time must not share a workspace. */
Q3_API int64_t q3_moe_mlp_workspace_bytes(int64_t n_gu, int64_t n_dn, int32_t t, int32_t topk);
Q3_API q3_status q3_moe_mlp(const q3_expert_stack* gate_up, const q3_expert_stack* down, const uint16_t* x,
                            int64_t ldx, const int32_t* topk_ids, int32_t t, int32_t topk, const float* logits,
                            int64_t ld_logits, void* workspace, int64_t workspace_bytes, float* out, int64_t ldo,
                            void* stream);

/* q3_moe_mlp without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): h and the per-pair outputs live in scratch memory the
 * library owns, q3_moe_mlp_noalloc_max_bytes() bytes per GPU (4 MiB, allocated
 * with the library's code object on each GPU it runs on and held until the
 * process ends).  The call allocates and frees nothing.  Same arguments,
 * results and errors as q3_moe_mlp without workspace / workspace_bytes, and
 * bitwise the same outputs; a round whose q3_moe_mlp_workspace_bytes(...)
 * exceeds the scratch size is rejected with Q3_ERR_UNSUPPORTED_SHAPE before
 * any launch (e.g. 64 pairs allow I + ceil(n_down/4)*4 <= 16384).  Every call
 * on one GPU uses that GPU's one scratch array: calls that overlap in time on
 * the same GPU (different streams, or different host threads without
 * ordering) race and must not be issued; calls in one stream's order are
 * safe.  The scratch keeps the last call's contents; nothing in it needs to
 * start at zero. */
Q3_API int64_t q3_moe_mlp_noalloc_max_bytes(void);
Q3_API q3_status q3_moe_mlp_noalloc(const q3_expert_stack* gate_up, const q3_expert_stack* down,
                                    const uint16_t* x, int64_t ldx, const int32_t* topk_ids, int32_t t,
                                    int32_t topk, const float* logits, int64_t ld_logits, float* out,
                                    int64_t ldo, void* stream);

/* ---- Two-bit draft head ------------------------------------------------------
 * (Hibana page, "Model surgery" / "Two-bit draft head": the drafter's
 * vocabulary projection is first evaluated on a 2-bit copy to pick a handful
 * of candidate tokens, and only those candidates are evaluated again with the
 * FP8 weights, which make the choice.)  Readings of the page:
 *   2-bit copy : 2-bit codes into a 4-entry E4M3FN codebook per row and one
 *                E8M0 scale per group of 32, 2 + 8/32 = 2.25 bits per weight:
 *                  w2[n][k] = E4M3FN(cb4[n][code]) * 2^(scale[n][k/32] - 127).
 *                Planes as above with two code words per group: byte b of
 *                word j (0..1) holds code 16j+4q+b in bits 2q..2q+1; word j of
 *                (r, g) sits at T*128*Gp + 2048*s + 16*(16*(q*j + kb) + i) + 4*t;
 *                the scale plane is laid out exactly as the 3-bit one; the
 *                codebook is uint8 [n][4].  q3_matrix describes such a head
 *                with `codebook` pointing at [n][4] (4-byte aligned).
 *   FP8 head   : OCP MXFP8, row-major: elements uint8 [n][ld_elements]
 *                E4M3FN, scales uint8 [n][ld_scales] E8M0, one per 32
 *                consecutive elements of a row:
 *                  w8[n][k] = E4M3FN(e8[n][k]) * 2^(s8[n][k/32] - 127).
 *   Ranking    : larger score first, equal scores to the lower row index.
 * Scores are exact products accumulated in fp32, as above. */

typedef struct q3_mxfp8_matrix {
  int64_t n, k;
  const void* elements;    /* [n][ld_elements] E4M3FN, 16-byte aligned, ld % 16 == 0 */
  int64_t ld_elements;
  const void* scales;      /* [n][ld_scales] E8M0 (ld_scales >= k/32)                */
  int64_t ld_scales;
} q3_mxfp8_matrix;

/* Plane sizes of an n x k 2-bit head: code_tile_bytes = 128*Gp, codebook_bytes
 * = 4*n, payload_bytes = n*k*9/32 (2.25 bits per weight).  Host only. */
Q3_API q3_status q3_layout2(int64_t n, int64_t k, q3_layout_info* out);

/* Pack / unpack the 2-bit copy: codes [n][ldc] uint8 0..3 (higher bits
 * ignored), scale_bytes [n][lds]; same conventions as q3_pack / q3_unpack. */
Q3_API q3_status q3_pack2(const uint8_t* codes, int64_t ldc, const uint8_t* scale_bytes, int64_t lds,
                          int64_t n, int64_t k, void* code_plane, void* scale_plane, void* stream);
Q3_API q3_status q3_unpack2(const q3_matrix* w, uint8_t* codes_out, uint8_t* scale_out, void* stream);

/* 2-bit scores of every row for 1 <= m <= 16 queries:
 * y[m][n] = x[m] . w2[n] (x bf16 [m][ldx], y fp32 [m][ldy]), on the matrix
 * cores like q3_gemm_small_m. */
Q3_API q3_status q3_head2_scores(const q3_matrix* w2, const uint16_t* x, int64_t m, int64_t ldx,
                                 float* y, int64_t ldy, void* stream);

/* Device workspace bytes q3_shortlist needs for m queries (host only). */
Q3_API int64_t q3_shortlist_workspace_bytes(int64_t m);

/* Shortlist: per query i the `size` rows with the largest scores[i][0..n),
 * larger first, equal scores to the lower row: ids int32 [m][size] and, if
 * vals is not NULL, their scores fp32 [m][size].  1 <= size <= 16,
 * size <= n, 1 <= m <= 65535; scores fp32 [m][ld], finite (not checked);
 * workspace: device memory of workspace_bytes bytes, at least
 * q3_shortlist_workspace_bytes(m) (Q3_ERR_INVALID_ARG otherwise), 8-byte
 * aligned, owned by the caller (its contents are scratch; calls that overlap
 * in time must not share it).  Two launches. */
Q3_API q3_status q3_shortlist(const float* scores, int64_t m, int64_t n, int64_t ld, int32_t size,
                              void* workspace, int64_t workspace_bytes, int32_t* ids, float* vals, void* stream);

/* FP8 rescoring of listed rows: y[i][j] = x[i] . w8[ids[i][j]] (fp32 [m][size])
 * and best[i] = the listed row with the largest y[i][.] (equal: lower row).
 * Ids outside [0, n) score 0.  1 <= size <= 16, 1 <= m <= 65535; x bf16
 * [m][ldx] as above.  One block per query. */
Q3_API q3_status q3_rescore_fp8(const q3_mxfp8_matrix* w8, const uint16_t* x, int64_t m, int64_t ldx,
                                const int32_t* ids, int32_t size, float* y, int32_t* best, void* stream);

/* The whole draft-head decision for 1 <= m <= 16 queries: 2-bit scores of all
 * rows, shortlist of `size`, FP8 rescoring and the decision, in four launches.
 * w2 and w8 must have the same n and k.  workspace: device memory of
 * workspace_bytes bytes, at least q3_draft_head_workspace_bytes(m, n)
 * (Q3_ERR_INVALID_ARG otherwise), 8-byte aligned, any contents (the 2-bit
 * scores [m][n] then the shortlist scratch; calls that overlap in time must
 * not share it).  Outputs: ids [m][size] (the list), y8 [m][size] (FP8
 * scores), best [m]. */
Q3_API int64_t q3_draft_head_workspace_bytes(int64_t m, int64_t n);
Q3_API q3_status q3_draft_head(const q3_matrix* w2, const q3_mxfp8_matrix* w8, const uint16_t* x, int64_t m,
                               int64_t ldx, int32_t size, void* workspace, int64_t workspace_bytes, int32_t* ids,
                               float* y8, int32_t* best, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q3_H */
