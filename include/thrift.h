/*
 * thrift.h - C ABI of the ThriftAttention forward pass on AMD MI355X (gfx950).
 *
 * ThriftAttention ("ThriftAttention: Selective Mixed Precision for
 * Long-Context FP4 Attention"; summaries at gist.science, Dutch section
 * "Methodologie", French section "Methodologie") computes softmax attention
 * in two precisions at once: a cheap score per (query block, key block) pair,
 * the dot product of the two blocks' token means, picks the top-k pairs of
 * every query block; those pairs run in FP16 and every other pair runs in
 * 4-bit E2M1 with micro-scaling; one online softmax merges both.
 *
 * Three calls make up the path, in this order:
 *   thrift_select_blocks  - block means, pair scores and per-query-block top-k
 *   thrift_quantize_fp4   - FP16 -> E2M1 codes + block scales (Q, K and V)
 *   thrift_attention_fwd  - the mixed FP4/FP16 forward pass
 * Further sections declare the fused and cache-side variants of the first
 * two, the decode-shaped forward, the middle-tier (MXFP8) variant and the
 * Attn-QAT backward.
 *
 * Conventions (all calls):
 *   - Tensors are contiguous, row-major, [batch, head, seq, dim] unless stated.
 *   - Every pointer is a DEVICE pointer except where marked "host".
 *   - The caller owns and allocates every buffer, workspace included; the
 *     library never allocates, frees or synchronises; its only state is a
 *     per-device flag that its kernels' LDS limits have been raised.
 *   - Every call is asynchronous on `stream`; calls on different streams
 *     may run concurrently when they share no output buffer.
 *   - Arguments are validated before anything is launched; on failure the
 *     call returns a non-zero thrift_status and launches nothing.  A launch
 *     failure reported by the HIP runtime returns THRIFT_EHIP.  No exception
 *     or signal crosses the ABI.
 *   - Results are deterministic: the kernels use no floating-point atomics,
 *     so two calls on the same inputs give identical bits.
 *   - Supported shapes: D in {64, 128}; block_q in {64, 128}; block_k = 64;
 *     1 <= S <= 262144; Hq a multiple of Hkv; B, Hq >= 1.
 */
#ifndef THRIFT_H
#define THRIFT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  THRIFT_OK = 0,
  THRIFT_EINVAL = 1,       /* a size, flag or pointer argument is invalid */
  THRIFT_EUNSUPPORTED = 2, /* a shape outside the supported set above */
  THRIFT_EALIGN = 3,       /* a pointer is not 16-byte aligned */
  THRIFT_EWORKSPACE = 4,   /* workspace missing or smaller than required */
  THRIFT_EHIP = 5          /* the HIP runtime reported a launch error */
} thrift_status;

/* FP4 micro-scaling formats.  Both store E2M1 elements (1 sign, 2 exponent,
 * 1 mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6), two per byte with the even
 * element in the low nibble.
 *   THRIFT_NVFP4: the format the pages name for the FP4 path: one E4M3 block
 *     scale per 16 elements, plus one fp32 scale per (batch, head) slice,
 *     sg = amax / (6 * 448) of the slice (1 for an all-zero slice); block byte
 *     = E4M3(amax_block / (6 sg)), element = E2M1(x / (block * sg)).
 *   THRIFT_MXFP4: one E8M0 scale per 32 elements (OCP MX): exponent
 *     floor(log2 amax_block) - 2, element = E2M1(x / 2^exponent); this is the
 *     layout gfx950's block-scaled FP4 matrix instructions consume.
 * All roundings are to nearest, ties to even, saturating (E2M1 at 6, E4M3 at
 * 448); the sign of a value that rounds to zero is kept.
 *   THRIFT_NVFP4_MXP: thrift_attention_fwd only, a variant of the FP4 path:
 *     Q, K and V as THRIFT_NVFP4 tensors, but the probabilities quantised
 *     MX-style (level 1 the tile maximum, E8M0 per 32 keys) instead of
 *     NVFP4's two levels.  Every other call rejects it (THRIFT_EINVAL). */
typedef enum { THRIFT_NVFP4 = 0, THRIFT_MXFP4 = 1, THRIFT_NVFP4_MXP = 2 } thrift_format;

/* Grouping axis of a quantised tensor.
 *   THRIFT_GROUP_D (Q, K): groups run along dim; codes [B,H,S,D/2] u8,
 *     scales [B,H,S,D/g] u8 (g = 16 NVFP4, 32 MXFP4).
 *   THRIFT_GROUP_S (V): groups run along the sequence and the tensor is
 *     stored transposed in 64-token blocks, so that one key block of V^T is
 *     contiguous: codes [B,H,Sp/64,D,32] u8 (byte i of row d of block jb
 *     holds tokens jb*64 + 2i, +2i+1, low nibble first), scales
 *     [B,H,Sp/64,D,64/g] u8, with Sp = S rounded up to a multiple of 64 and
 *     the padding tokens zero. */
typedef enum { THRIFT_GROUP_D = 0, THRIFT_GROUP_S = 1 } thrift_group_axis;

/* ---------------------------------------------------------------------- */
/* Block selection ("Heuristische Blokkenselectie" on the Dutch page)       */
/* ---------------------------------------------------------------------- */

/* Host helper: the largest per-query-block budget k_i, i.e. the minimum
 * `kmax` that thrift_select_blocks accepts.  Query block i covers rows
 * [i*block_q, min(S,(i+1)*block_q)); its valid key blocks are all key
 * blocks, or (causal, query and key sequences aligned at their starts) the
 * blocks j with j*block_k <= min(S,(i+1)*block_q) - 1; n_i is their count and
 * k_i = min(n_i, topk_count) if topk_count >= 0, else
 * min(n_i, ceil(n_i * topk_bp / 10000)).  Returns -1 on invalid arguments. */
int thrift_select_kmax(int S, int block_q, int block_k, int causal, int topk_count, int topk_bp);

/* Workspace bytes thrift_select_blocks needs (the fp32 block means). */
size_t thrift_select_workspace_bytes(int B, int Hq, int Hkv, int S, int D, int block_q,
                                     int block_k);

/* Importance scores and top-k (pages: S^_ij = qbar_i . kbar_j, the top-k
 * highest-scoring pairs go to FP16).
 *   q16 [B,Hq,S,D] fp16, k16 [B,Hkv,S,D] fp16: inputs (read only).
 *   qbar_i, kbar_j: the arithmetic mean of the block's valid rows, summed in
 *     fp64 (exact) and rounded once to fp32.
 *   score: fp32, one fused multiply-add per channel in ascending order.
 *   Query head hq reads key head hq / (Hq / Hkv).
 *   The k_i best valid key blocks of each query block are kept (ties: the
 *   lower block index wins; -0 == +0; inputs must be finite).
 *   idx [B,Hq,nQ,kmax] int32 (out): the kept block indices, ascending,
 *     padded with -1; cnt [B,Hq,nQ] int32 (out): k_i.  nQ = ceil(S/block_q).
 *   kmax: row length of idx, >= thrift_select_kmax(...).
 *   workspace: device buffer of at least thrift_select_workspace_bytes. */
thrift_status thrift_select_blocks(const void* q16, const void* k16, int B, int Hq, int Hkv, int S,
                                   int D, int block_q, int block_k, int causal, int topk_count,
                                   int topk_bp, int32_t* idx, int32_t* cnt, int kmax,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Selection for Sq queries that are the last Sq positions of an Sk-key
 * sequence (Sq <= Sk; decode: new tokens against the KV cache).  Everything
 * as thrift_select_blocks with q16 [B,Hq,Sq,D] and k16 [B,Hkv,Sk,D]; nQ =
 * ceil(Sq/block_q); under causal masking query block i may see key block j
 * when j*block_k <= Sk - Sq + min(Sq,(i+1)*block_q) - 1.  The three calls
 * above are the Sq = Sk case of these. */
int thrift_select_kmax_kv(int Sq, int Sk, int block_q, int block_k, int causal, int topk_count,
                          int topk_bp);
size_t thrift_select_workspace_bytes_kv(int B, int Hq, int Hkv, int Sq, int Sk, int D, int block_q,
                                        int block_k);
thrift_status thrift_select_blocks_kv(const void* q16, const void* k16, int B, int Hq, int Hkv,
                                      int Sq, int Sk, int D, int block_q, int block_k, int causal,
                                      int topk_count, int topk_bp, int32_t* idx, int32_t* cnt,
                                      int kmax, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* Key-block means kept beside a KV cache (the cache holds FP16 and FP4
 * copies of K/V, summaries "Betekenis en Beweringen"), so that a decode step
 * recomputes only the block its new keys land in.
 *   x16 [B,H,S,D] fp16 (read only).
 *   means [B,H,ceil(S/blk),D] fp32 (in/out): blocks j0 <= j < j1 of every
 *     (batch, head) slice are written - the mean of the block's rows that lie
 *     below S, summed in fp64 and rounded once to fp32, bit-identical to the
 *     kbar thrift_select_blocks computes; every other block is left as is.
 *   0 <= j0 < j1 <= ceil(S/blk), else THRIFT_EINVAL. */
thrift_status thrift_block_means(const void* x16, int B, int H, int S, int D, int blk, int j0, int j1,
                                 float* means, hipStream_t stream);

/* thrift_select_blocks_kv with the key-block means given instead of the fp16
 * keys: kbar [B,Hkv,ceil(Sk/block_k),D] fp32 as thrift_block_means writes
 * them with blk = block_k (read only).  Same idx and cnt.  workspace: at
 * least B*Hq*ceil(Sq/block_q)*D*4 bytes (the query means;
 * thrift_select_workspace_bytes_kv is always enough). */
thrift_status thrift_select_blocks_kbar(const void* q16, const float* kbar, int B, int Hq, int Hkv,
                                        int Sq, int Sk, int D, int block_q, int block_k, int causal,
                                        int topk_count, int topk_bp, int32_t* idx, int32_t* cnt,
                                        int kmax, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream);

/* Selection from query and key block means computed beforehand: qbar
 * [B,Hq,ceil(Sq/block_q),D] fp32 (blk = block_q) and kbar
 * [B,Hkv,ceil(Sk/block_k),D] fp32 (blk = block_k), as thrift_block_means or
 * thrift_quantize_fp4_means write them (read only).  Same idx and cnt as
 * thrift_select_blocks_kv on the tensors they came from; no workspace. */
thrift_status thrift_select_blocks_means(const float* qbar, const float* kbar, int B, int Hq, int Hkv,
                                         int Sq, int Sk, int D, int block_q, int block_k, int causal,
                                         int topk_count, int topk_bp, int32_t* idx, int32_t* cnt,
                                         int kmax, hipStream_t stream);

/* Per-head budget: the other reading of the pages' top-k over the best-scoring
 * block pairs (summaries "Heuristische Blokkenselectie"): one budget over all
 * valid pairs of a query head, K = min(P, topk_count) or
 * ceil(P * topk_bp / 10^4) of its P valid pairs, the K best-scoring pairs
 * kept (ties: lower query block, then lower key block).  Scores as
 * thrift_select_blocks; means as thrift_select_blocks_means takes them.
 *   idx [B,Hq,nQ,kmax] (out): each query block's kept key blocks ascending,
 *     padded with -1; cnt [B,Hq,nQ] (out): their number (0 .. n_i);
 *   kmax >= thrift_select_head_kmax(...) (the largest n_i), else EINVAL;
 *   workspace: thrift_select_head_workspace_bytes (every pair's score, the
 *     per-head threshold and the per-query-block tie offsets).
 * The idx/cnt it writes drive thrift_attention_fwd unchanged. */
int thrift_select_head_kmax(int Sq, int Sk, int block_q, int block_k, int causal);
size_t thrift_select_head_workspace_bytes(int B, int Hq, int Sq, int Sk, int block_q, int block_k);
thrift_status thrift_select_blocks_head(const float* qbar, const float* kbar, int B, int Hq, int Hkv, int Sq,
                                        int Sk, int D, int block_q, int block_k, int causal, int topk_count,
                                        int topk_bp, int32_t* idx, int32_t* cnt, int kmax, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* FP4 quantisation (the FP4 path's NVFP4 micro-scaling)                    */
/* ---------------------------------------------------------------------- */

/* Workspace bytes thrift_quantize_fp4 needs (per-slice maxima, NVFP4 only;
 * 0 for MXFP4). */
size_t thrift_quantize_workspace_bytes(int B, int H, int S, int D, int fmt);

/* Quantise x16 [B,H,S,D] fp16 to FP4 along `axis` (layouts above).
 *   codes, scales (out): as laid out for the axis;
 *   tensor_scale [B,H] fp32 (out): the per-slice scale, NVFP4 only (may be
 *     NULL for MXFP4).
 * Every code and scale byte equals the exact round-to-nearest-even result of
 * the rule stated with thrift_format, whatever the hardware's own
 * conversion instructions do. */
thrift_status thrift_quantize_fp4(const void* x16, int B, int H, int S, int D,
                                  int axis, int fmt, uint8_t* codes,
                                  uint8_t* scales, float* tensor_scale, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* Block means and FP4 codes along D (Q or K) from one read of x16: the
 * selection's block means and the FP4 path's operand in a single pass
 * (summaries "Methodologie": both come from the same fp16 Q and K).
 *   means [B,H,ceil(S/blk),D] fp32 (out): as thrift_block_means over all
 *     blocks, bit for bit;
 *   codes, scales, tensor_scale (out): as thrift_quantize_fp4 with
 *     THRIFT_GROUP_D, byte for byte.
 * NVFP4 reads x16 twice (its slice scale must precede the codes) and needs
 * thrift_quantize_means_workspace_bytes of workspace; MXFP4 reads it once
 * and needs none. */
size_t thrift_quantize_means_workspace_bytes(int B, int H, int S, int D, int fmt, int blk);
thrift_status thrift_quantize_fp4_means(const void* x16, int B, int H, int S, int D, int fmt,
                                        int blk, uint8_t* codes, uint8_t* scales, float* tensor_scale,
                                        float* means, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream);

/* Re-encode part of a KV-cache FP4 copy after new tokens were written to
 * positions s0 <= s < s1 of x16 [B,H,S,D] (the FP4 copy of the cache,
 * summaries "Betekenis en Beweringen").  Along THRIFT_GROUP_D the rows
 * s0..s1-1 are re-encoded; along THRIFT_GROUP_S every 128-position tile that
 * holds one of them.  Bytes outside those rows or tiles are not touched.
 *   MXFP4: each byte written equals the byte thrift_quantize_fp4 writes for
 *     the tensor as it is now (MX groups depend on nothing else);
 *   NVFP4: tensor_scale [B,H] (in, required) is the slice scale the copy was
 *     encoded with and is kept, so the bytes equal a whole-tensor encode as
 *     long as the new positions do not raise the slice's maximum (a caller
 *     whose new tokens do re-encodes the slice with thrift_quantize_fp4).
 * 0 <= s0 < s1 <= S, else THRIFT_EINVAL. */
thrift_status thrift_quantize_fp4_range(const void* x16, int B, int H, int S, int D,
                                        int axis, int fmt, int s0, int s1,
                                        uint8_t* codes, uint8_t* scales, const float* tensor_scale,
                                        hipStream_t stream);

/* The same cache maintenance in one launch: after new tokens were written to
 * positions s0 <= s < s1 of the cache's fp16 k16 and v16 [B,H,S,D], the
 * means of the key blocks (block_k rows) that hold them into kbar
 * [B,H,ceil(S/block_k),D] (as thrift_block_means), K's FP4 rows (as
 * thrift_quantize_fp4_range along THRIFT_GROUP_D) and V's FP4 tiles (along
 * THRIFT_GROUP_S).  Byte for byte the results of those three calls; the
 * NVFP4 slice scales k4_tscale, v4_tscale are read, not changed. */
thrift_status thrift_cache_update(const void* k16, const void* v16, int B, int H, int S, int D, int block_k,
                                  int s0, int s1, int fmt, float* kbar, uint8_t* k4_codes,
                                  uint8_t* k4_scales, const float* k4_tscale, uint8_t* v4_codes,
                                  uint8_t* v4_scales, const float* v4_tscale, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Mixed FP4/FP16 attention ("Gemengd-Precisie Berekening & Samenvoeging")  */
/* ---------------------------------------------------------------------- */

/* Forward pass.  For every query row r of query block i (head hq, key head
 * hk = hq / (Hq/Hkv)), with t = sm_scale * q.k in log2 units:
 *  1. FP4 path, over every valid key block of i that idx does not list,
 *     ascending: scores from the FP4 Q and K; causal mask (key > r) and keys
 *     past S get probability 0; the tile's probabilities are quantised in two
 *     levels (level 1 per row and tile, level 2 per key group aligned with V's
 *     groups):
 *       NVFP4: v = 2688 * 2^(t - tile max), per-16 E4M3 scale E4M3(max v / 6),
 *              E2M1 codes of v / scale;
 *       MXFP4: v = 2^(t - tile max), per-32 E8M0 scale 2^(floor(log2 max v)
 *              - 2), E2M1 codes of v / scale;
 *     then multiplied with the FP4 V.
 *  2. FP16 path, over the promoted blocks idx[.., :cnt] ascending (FP16 Q is
 *     read only for query blocks with cnt > 0, FP16 K/V only for promoted
 *     blocks): scores from fp16 Q and K, probabilities relative to the
 *     tile maximum (2^(t - tile max)) rounded to fp16, times fp16 V.
 *  3. Both paths feed one online softmax (running max, running sum of the
 *     unquantised probabilities, fp32 accumulator); O = acc / sum.
 * Arguments:
 *   q16 [B,Hq,S,D], k16/v16 [B,Hkv,S,D] fp16: may be NULL only if every cnt is 0.
 *   q4_codes/q4_scales/q4_tscale, k4_*: Q and K from thrift_quantize_fp4 along
 *     THRIFT_GROUP_D; v4_*: V along THRIFT_GROUP_S; *_tscale NULL for MXFP4.
 *   idx, cnt, kmax: from thrift_select_blocks (or any ascending, -1 padded
 *     list of valid blocks per query block).
 *   sm_scale: softmax scale (1/sqrt(D) is customary).
 *   o [B,Hq,S,D] (out): fp16 if o_is_fp32 == 0, fp32 otherwise.
 *   lse [B,Hq,S] fp32 (out, may be NULL): natural-log log-sum-exp of the
 *     scores with the unquantised probabilities. */
thrift_status thrift_attention_fwd(const void* q16, const void* k16, const void* v16,
                                   const uint8_t* q4_codes, const uint8_t* q4_scales,
                                   const float* q4_tscale, const uint8_t* k4_codes,
                                   const uint8_t* k4_scales, const float* k4_tscale,
                                   const uint8_t* v4_codes, const uint8_t* v4_scales,
                                   const float* v4_tscale, int fmt, const int32_t* idx,
                                   const int32_t* cnt, int kmax, int B, int Hq, int Hkv, int S,
                                   int D, int block_q, int block_k, int causal, float sm_scale,
                                   void* o, int o_is_fp32, float* lse, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Middle precision tier (a variant): FP4, FP8 and FP16 in one kernel       */
/* ---------------------------------------------------------------------- */
/* The hyperion-consulting.io article on the method ("ThriftAttention:
 * Selective Mixed Precision for Long-Context FP4 Attention", in German;
 * sections "Einführung" and "COMPUTE-Schicht") names three precision levels,
 * FP4, FP8 and BF16,
 * switched inside one kernel; the method's other pages choose between two by
 * block-mean scores.  This variant keeps their selection and inserts MXFP8
 * between them: the blocks of the selection under budget bp16 run in FP16,
 * the blocks the selection under bp16 + bp8 adds run in FP8, the rest in
 * FP4 (MX format).
 *
 * MXFP8 quantisation of x16 [B,H,S,D] fp16 along `axis`: E4M3 elements
 * (bias 7, largest 448, subnormals m 2^-9, no infinity) under one E8M0 scale
 * per 32 elements, exponent floor(log2 amax) - 8 (so the group maximum lands
 * in [256, 512)), element code = E4M3 of x / 2^exponent rounded to nearest
 * even, saturating at 448, sign kept (-0 gives 0x80); an all-zero group has
 * exponent -127.
 *   THRIFT_GROUP_D (Q, K): codes [B,H,S,D] u8, scales [B,H,S,D/32] u8;
 *   THRIFT_GROUP_S (V): codes [B,H,D,Sp] u8 (V transposed, Sp = S rounded up
 *     to 64, padding tokens zero), scales [B,H,D,Sp/32] u8.
 * codes 16-byte aligned; no workspace. */
thrift_status thrift_quantize_fp8(const void* x16, int B, int H, int S, int D, int axis,
                                  uint8_t* codes, uint8_t* scales, hipStream_t stream);

/* Three-tier forward (MX format).  As thrift_attention_fwd with
 * fmt = THRIFT_MXFP4, plus a middle tier between its two paths: every valid
 * block that idx2[.., :cnt2] lists and idx[.., :cnt] does not runs, after the
 * FP4 path and before the FP16 path, ascending, with scores from the MXFP8 Q
 * and K, the probabilities quantised in two levels as on the MXFP4 path but
 * with E4M3 elements (v = 2^(t - tile max), E8M0 exponent
 * floor(log2 max v) - 8 per 32 keys, E4M3 codes of v / 2^exponent), times the
 * MXFP8 V.  FP4 runs on every valid block neither list holds.  The
 * unquantised probabilities feed the row sum on all three tiers.
 *   q8_*, k8_*: thrift_quantize_fp8 along THRIFT_GROUP_D; v8_*: along
 *     THRIFT_GROUP_S; scales 4-byte aligned.
 *   idx2, cnt2, kmax2: the FP16 and FP8 tiers' blocks together, e.g. from
 *     thrift_select_blocks under the two budgets' sum (its top-k list then
 *     contains idx's, as both come from one ranking); a block both lists
 *     hold stays on the FP16 path.
 * Everything else (layouts, o, lse, errors) as thrift_attention_fwd. */
thrift_status thrift_attention_fwd_tiered(
    const void* q16, const void* k16, const void* v16, const uint8_t* q4_codes, const uint8_t* q4_scales,
    const uint8_t* k4_codes, const uint8_t* k4_scales, const uint8_t* v4_codes, const uint8_t* v4_scales,
    const uint8_t* q8_codes, const uint8_t* q8_scales, const uint8_t* k8_codes, const uint8_t* k8_scales,
    const uint8_t* v8_codes, const uint8_t* v8_scales, const int32_t* idx, const int32_t* cnt, int kmax,
    const int32_t* idx2, const int32_t* cnt2, int kmax2, int B, int Hq, int Hkv, int S, int D, int block_q,
    int block_k, int causal, float sm_scale, void* o, int o_is_fp32, float* lse, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Decode-shaped forward (new tokens against the dual FP16/FP4 KV cache;    */
/* decode results in "Resultaten", the cache in "Betekenis en Beweringen")  */
/* ---------------------------------------------------------------------- */

/* Workspace bytes thrift_attention_decode needs (per-split partial results). */
size_t thrift_attention_decode_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D,
                                               int kmax);

/* The forward pass of thrift_attention_fwd for Sq new queries that are the
 * last Sq positions of an Sk-key sequence (causal masks aligned at the
 * ends: query row r sees keys <= Sk - Sq + r), computed split over the keys
 * and merged by log-sum-exp.  Same per-row arithmetic, so the same result up
 * to fp32 rounding order.
 *   q16 [B,Hq,Sq,D], k16/v16 [B,Hkv,Sk,D] fp16 (required);
 *   q4_*: Q along THRIFT_GROUP_D (S = Sq); k4_*, v4_*: the cache's K and V
 *     along THRIFT_GROUP_D / THRIFT_GROUP_S (S = Sk);
 *   idx [B,Hq,1,kmax], cnt [B,Hq,1]: thrift_select_blocks_kv with one query
 *     block (block_q >= Sq);
 *   o [B,Hq,Sq,D] (fp16 or fp32), lse [B,Hq,Sq] (may be NULL);
 *   workspace: device buffer of at least
 *     thrift_attention_decode_workspace_bytes(...), caller-owned, 16-byte
 *     aligned; its contents are scratch.
 *   q4_tscale, k4_tscale, v4_tscale: the slice scales, required for
 *     THRIFT_NVFP4 (EINVAL if NULL), ignored for THRIFT_MXFP4.
 * Supported: both formats, D 64 or 128, block_k 64, Sq <= 32 and
 * (Hq/Hkv)*Sq <= 128 (the query heads of a key head and their rows are the
 * columns of 32-column tiles; the key head's K/V are read once per 32
 * columns), Sk <= 262144, and the promoted-block table of a key head's
 * query heads (Hq/Hkv words per 32 valid key blocks) beside the split
 * kernel's stages in 160 KB of LDS, which limits only THRIFT_NVFP4 at D 128:
 * Hq/Hkv * ceil(ceil(Sk/64)/32) <= 5120.  Other shapes return
 * THRIFT_EUNSUPPORTED and launch nothing. */
thrift_status thrift_attention_decode(const void* q16, const void* k16, const void* v16,
                                      const uint8_t* q4_codes, const uint8_t* q4_scales,
                                      const float* q4_tscale, const uint8_t* k4_codes,
                                      const uint8_t* k4_scales, const float* k4_tscale,
                                      const uint8_t* v4_codes, const uint8_t* v4_scales,
                                      const float* v4_tscale, int fmt,
                                      const int32_t* idx, const int32_t* cnt, int kmax, int B,
                                      int Hq, int Hkv, int Sq, int Sk, int D, int block_k,
                                      int causal, float sm_scale, void* o, int o_is_fp32,
                                      float* lse, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * thrift_attention_decode with the split partials in the library's own
 * static device array of THRIFT_DECODE_SCRATCH_BYTES per GPU (held until the
 * process ends) instead of a caller workspace.  Same arguments, results and
 * validation as thrift_attention_decode, minus workspace and
 * workspace_bytes; returns THRIFT_EWORKSPACE when the shape's partials
 * (thrift_attention_decode_workspace_bytes) exceed the array, THRIFT_EHIP
 * when the array's device address cannot be taken.  Allocates nothing.
 * Every call on one GPU shares the array: calls that overlap on one GPU (on
 * different streams, or from different threads) race. */
#define THRIFT_DECODE_SCRATCH_BYTES ((size_t)16 << 20)
thrift_status thrift_attention_decode_noalloc(const void* q16, const void* k16, const void* v16,
                                              const uint8_t* q4_codes, const uint8_t* q4_scales,
                                              const float* q4_tscale, const uint8_t* k4_codes,
                                              const uint8_t* k4_scales, const float* k4_tscale,
                                              const uint8_t* v4_codes, const uint8_t* v4_scales,
                                              const float* v4_tscale, int fmt,
                                              const int32_t* idx, const int32_t* cnt, int kmax, int B,
                                              int Hq, int Hkv, int Sq, int Sk, int D, int block_k,
                                              int causal, float sm_scale, void* o, int o_is_fp32,
                                              float* lse, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Backward pass for quantisation-aware training ("Attn-QAT: 4-Bit         */
/* Attention With Quantization-Aware Training"; gist.science summary in     */
/* German, section 2 "Methodik", and the paper's abstract)                  */
/* ---------------------------------------------------------------------- */

/* The gradient of thrift_attention_fwd with the selection (idx, cnt) held
 * fixed and every quantiser taken as the identity in the backward pass
 * (straight-through), as quantisation-aware training differentiates through
 * fake quantisation.  The two Attn-QAT rules:
 *   - the backward recomputes each probability from the forward's
 *     log-sum-exp in the precision the forward used for it: on FP4 pairs the
 *     two-level quantised value (its codes are relative to the tile, so they
 *     do not depend on the LSE), on FP16 pairs p rounded to fp16;
 *   - the row term of the softmax gradient is dO . O', where O' is the
 *     output with the exact (unquantised) probabilities, which the forward
 *     stores besides O; dO . O (the FP4 output) would be wrong.
 * For row r and key c of a valid pair (operands in the pair's path's
 * precision): p = exp(sm_scale q.k - lse), dV[c] += pt dO[r],
 * dS = p (dO[r].v[c] - dO[r].O'[r]), dQ[r] += sm_scale dS k[c],
 * dK[c] += sm_scale dS q[r].  Training shape only: Sq = Sk = S.
 * Both formats; *_tscale are the NVFP4 slice scales (required for
 * THRIFT_NVFP4, EINVAL if NULL; ignored for THRIFT_MXFP4).  Supported:
 * D 64 or 128, block_q 64 or 128, block_k 64, S <= 262144. */

/* Workspace bytes both calls below need: FP4-decoded fp16 copies of Q (and
 * of Q times its NVFP4 slice scale), K and V (V in rows and in its stored
 * transposed order), the promoted-block bit table, the row terms and the
 * rows' log-sum-exp in log2 units (about 2 Q-sized and 3 K-sized fp16
 * tensors). */
size_t thrift_attention_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int D, int block_q);

/* O' of the forward: ohp [B,Hq,S,D] fp32 (out) from the same inputs as
 * thrift_attention_fwd (FP4 tensors as written by thrift_quantize_fp4:
 * Q and K along THRIFT_GROUP_D, V along THRIFT_GROUP_S) and its lse
 * [B,Hq,S] (in, natural log, 16-byte aligned).  Rows past S are not
 * written.  The workspace contents are scratch. */
thrift_status thrift_attention_fwd_hp(const void* q16, const void* k16, const void* v16,
                                      const uint8_t* q4_codes, const uint8_t* q4_scales,
                                      const float* q4_tscale, const uint8_t* k4_codes,
                                      const uint8_t* k4_scales, const float* k4_tscale,
                                      const uint8_t* v4_codes, const uint8_t* v4_scales,
                                      const float* v4_tscale, int fmt, const int32_t* idx, const int32_t* cnt,
                                      int kmax, int B, int Hq, int Hkv, int S, int D, int block_q,
                                      int block_k, int causal, float sm_scale, const float* lse,
                                      float* ohp, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* Gradients: do16 [B,Hq,S,D] fp16 (in), lse and ohp from the forward (in);
 * dq [B,Hq,S,D], dk and dv [B,Hkv,S,D] fp32 (out, overwritten; query heads
 * sharing a key head are summed into it).  Deterministic: no atomics. */
thrift_status thrift_attention_bwd(const void* q16, const void* k16, const void* v16,
                                   const uint8_t* q4_codes, const uint8_t* q4_scales,
                                   const float* q4_tscale, const uint8_t* k4_codes,
                                   const uint8_t* k4_scales, const float* k4_tscale,
                                   const uint8_t* v4_codes, const uint8_t* v4_scales,
                                   const float* v4_tscale, int fmt, const int32_t* idx, const int32_t* cnt, int kmax,
                                   int B, int Hq, int Hkv, int S, int D, int block_q, int block_k,
                                   int causal, float sm_scale, const float* lse, const float* ohp,
                                   const void* do16, float* dq, float* dk, float* dv, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/* Static string for a status code (host): s is a thrift_status value;
 * any other value gives "unknown status". */
const char* thrift_status_string(int s);

#ifdef __cplusplus
}
#endif
#endif /* THRIFT_H */
