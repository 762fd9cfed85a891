/*
 * tilemix.h -- C ABI of the MI355X (gfx950) TileMix library.
 *
 * TileMix is causal dense prefill attention in one fused streaming kernel in
 * which every hardware-aligned score-tile group computes Q.K^T either in FP16
 * or in blockwise INT8, and all groups share one online-softmax state.  Besides
 * that path the library offers one decode step against an INT8 key/value
 * cache, content-dependent routing words, an FP8 (E4M3) third score path and
 * the layers of a synthetic attention stack that carries the deviation from
 * layer to layer.  The prefill (two- or three-path) comes in two forms with
 * bit-identical output: reading Q's codes from the quantisers, or making them
 * in its prologue (one work unit is exactly one Q block), which leaves only
 * K to quantise beforehand.
 *
 * Sources (web pages about TileMix), cited by title and section:
 *   [Digest]    "TileMix: Tile-Centric Mixed-Precision Attention for LLM
 *               Inference Acceleration" (paper digest), method and setup.
 *   [Explainer] "TileMix：给AI大模型的“注意力”做一次精准的精度分配手术"
 *               (popular explainer), sections 第一步 / 第二步 / 第三步 / 支持的场景 /
 *               数字精度混用到底靠不靠谱 / 写在后面.
 *   [Routes]    "TileMix Routes Attention Precision at the Hardware-Tile
 *               Level", section "Precision routing over score tiles".
 *   [Map]       "Precision Has a Map: TileMix Routes INT8 Inside Dense
 *               Attention", section "The routing mechanism is designed to stay
 *               inside the hot loop".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are token-major and contiguous: Q, O are [T, Hq, d], K, V are
 *    [T, Hkv, d]; sequences are packed back to back (cu_seqlens: B+1 int32
 *    prefix sums, cu_seqlens[0] = 0, non-decreasing).  FP16 is IEEE binary16.
 *  - Score tiles are TILEMIX_BLOCK_M query rows x TILEMIX_BLOCK_N keys,
 *    counted from each sequence's first token.  Per sequence of length L:
 *    Tm = ceil(L/128) query tiles, Tn = ceil(L/64) key tiles, grouping factor
 *    g = max(1, ceil(Tn/64)); routing group G of a row holds key tiles
 *    G*g .. G*g+g-1.  Global tile indices concatenate the sequences' tiles in
 *    batch order (sequence s starts at sum of Tm / Tn of sequences < s).
 *  - Head dims supported: 64 and 128.  Query head h reads KV head
 *    h / (Hq/Hkv) (GQA with contiguous groups).
 *  - The caller owns every buffer.  Entry points taking device pointers only
 *    enqueue work on `hip_stream` (a hipStream_t; NULL = the null stream) and
 *    never synchronise; they allocate no device memory.
 *  - Every pointer must be non-NULL (unless its count is 0) and 16-byte
 *    aligned.  All validation happens on the host before any launch.
 *  - Return value: TILEMIX_OK (0) or a negative TILEMIX_E* code; then
 *    tilemix_last_error() describes the failure.  No C++ exception crosses
 *    the ABI.
 */
#ifndef TILEMIX_H
#define TILEMIX_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TILEMIX_BLOCK_M 128   /* query rows per score tile and per Q quant block */
#define TILEMIX_BLOCK_N 64    /* keys per score tile and per K quant block      */
#define TILEMIX_WORD_BITS 64  /* routing groups per query-tile row, at most     */
/* Scratch bytes the allocation-free decode step holds per GPU (32 MiB). */
#define TILEMIX_DECODE_SCRATCH_BYTES (32ll * 1024 * 1024)

enum tilemix_status {
  TILEMIX_OK = 0,
  TILEMIX_EINVAL = -1,       /* bad argument (null/misaligned pointer, range)  */
  TILEMIX_EUNSUPPORTED = -2, /* head_dim not in {64, 128}, plan version, ...   */
  TILEMIX_EHIP = -3          /* a HIP runtime call or launch failed             */
};

/* Static routing templates ([Digest, method]: Band keeps the diagonal-local
 * region in FP16, Global keeps designated positions, Row-Random keeps a random
 * FP16 subset per row, Aligned-Sparse extends right-aligned, BigBird is the
 * union of the first three, SpTrans is stride plus tail). */
enum tilemix_template {
  TILEMIX_BAND = 0,
  TILEMIX_GLOBAL = 1,
  TILEMIX_ROWRANDOM = 2,
  TILEMIX_ALIGNEDSPARSE = 3,
  TILEMIX_BIGBIRD = 4,
  TILEMIX_SPTRANS = 5
};

/* Message of the last failure on the calling thread ("" if none).  The string
 * stays valid until the next call of a tilemix function on this thread. */
const char* tilemix_last_error(void);

/* Sizes of a packed batch (host only).
 * cu_seqlens_h: host int32[batch+1].  Outputs (host, any may be NULL):
 * total tokens T, total query tiles sum(Tm), total key tiles sum(Tn). */
int tilemix_query_sizes(const int32_t* cu_seqlens_h, int32_t batch, int64_t* total_tokens,
                        int64_t* total_q_tiles, int64_t* total_k_tiles);

/* Routing words (host only) -- [Digest, method]: one bit per routing group
 * (1 = INT8, 0 = FP16), one 64-bit word per (KV head, query-tile row), looked
 * up with a shift and a mask ([Map, hot loop]); coverage is the INT8 share of
 * legal tile groups; a static template is reused across layers, batch entries
 * and KV heads.
 *
 * A group (r, G) is legal when it holds a pair with key <= query inside the
 * sequence.  The template orders a sequence's legal groups; the first
 * N_legal - N8 stay FP16 and the last N8 = floor((coverage_bp * N_legal +
 * 5000) / 10000) go INT8.  Bit G of a word is group G (LSB = group 0); bits of
 * illegal groups are 0.  `seed` feeds Row-Random (and BigBird) only.
 *
 * Outputs (host buffers owned by the caller):
 *   words_h        uint64[num_kv_heads][total_q_tiles] (same for every head)
 *   g_h            int32[batch]     grouping factor per sequence (may be NULL)
 *   int8_groups_h  int64[batch]     N8 per sequence (may be NULL)
 *   legal_groups_h int64[batch]     N_legal per sequence (may be NULL)
 * Errors: EINVAL for coverage outside [0, 10000], unknown template, bad
 * cu_seqlens or null words_h with a non-empty batch. */
int tilemix_build_routing(const int32_t* cu_seqlens_h, int32_t batch, int32_t num_kv_heads,
                          int32_t tmpl, int32_t coverage_bp, uint64_t seed, uint64_t* words_h,
                          int32_t* g_h, int64_t* int8_groups_h, int64_t* legal_groups_h);

/* Three-class routing (host) -- a third precision, FP8 (OCP E4M3), for the
 * open question of [Digest, setup] / [Explainer, 写在后面] (moving to FP8
 * needs scales and schedule redone).  The template's order keeps its first
 * groups FP16, the next FP8, the last INT8: N8 = floor((int8_bp * N_legal +
 * 5000) / 10000) and N8 + Nf8 = the same with int8_bp + fp8_bp, so the INT8
 * word equals tilemix_build_routing's at int8_bp and INT8 | FP8 equals it at
 * int8_bp + fp8_bp.  words_f8_h marks FP8 groups (disjoint from INT8).
 * Errors: EINVAL when int8_bp + fp8_bp > 10000, else as
 * tilemix_build_routing. */
int tilemix_build_routing3(const int32_t* cu_seqlens_h, int32_t batch, int32_t num_kv_heads, int32_t tmpl,
                           int32_t int8_bp, int32_t fp8_bp, uint64_t seed, uint64_t* words_i8_h,
                           uint64_t* words_f8_h, int32_t* g_h, int64_t* int8_groups_h, int64_t* fp8_groups_h,
                           int64_t* legal_groups_h);

/* Adaptive routing words (host) -- [Digest, setup]: the evaluated routing is
 * static, and the interface accepts adaptive policies; [Map, "Placement
 * can matter more than the nominal percentage"].  Given the importance of
 * every legal group (from tilemix_routing_importance, copied to the host),
 * the legal groups of each (sequence, KV head) are ordered by (importance,
 * r, G) ascending and the first N8 -- the same count as a template at
 * coverage_bp -- get bit 1 (INT8).  Words may differ between KV heads.
 * importance_h: float[num_kv_heads][total_q_tiles][64] (slots of illegal
 * groups are ignored).  Outputs as tilemix_build_routing.
 * Errors: EINVAL for bad cu_seqlens or coverage, NULL buffers, or a NaN
 * importance. */
int tilemix_build_routing_adaptive(const int32_t* cu_seqlens_h, int32_t batch, int32_t num_kv_heads,
                                   const float* importance_h, int32_t coverage_bp, uint64_t* words_h,
                                   int32_t* g_h, int64_t* int8_groups_h, int64_t* legal_groups_h);

/* Work plan (host only) -- the geometry and schedule of one packed batch:
 * per-sequence tile offsets and grouping factors, plus the ordered list of
 * (sequence, query head, query-tile row) work units the fused kernel runs,
 * longest rows first and grouped so that units sharing a KV head run on the
 * same accelerator complex die.  The plan is an opaque array of int32; the
 * caller keeps a host copy and uploads an identical device copy (both are
 * passed to the device entry points).  It depends only on (cu_seqlens, Hq,
 * Hkv, head_dim) and can be reused across layers and calls.
 * tilemix_plan_size returns its length in int32 elements in *plan_len.
 *
 * The plan is how the device entry points receive the problem statement of
 * [Digest, method]: cu_seqlens (host and device), the batch size, Hq, Hkv,
 * head_dim and each sequence's grouping factor g are all in it, in place of
 * separate arguments (the caller-owned planner workspace of the interface).
 * plan_d must hold exactly plan_h's int32 values: the kernels read work
 * units and sequence records from plan_d while the grid comes from plan_h.
 * Every entry point verifies plan_h's checksum (a modified or truncated host
 * plan is refused with EINVAL); plan_d against plan_h is verified only in the
 * debug build (python -m mixed_precision_attention_amd.build --debug), since
 * reading it back costs a synchronous copy -- otherwise it is the caller's
 * duty, which the Python binding's bundles meet by uploading plan_d from
 * plan_h themselves. */
int tilemix_plan_size(const int32_t* cu_seqlens_h, int32_t batch, int32_t hq, int32_t hkv,
                      int32_t head_dim, int64_t* plan_len);
int tilemix_build_plan(const int32_t* cu_seqlens_h, int32_t batch, int32_t hq, int32_t hkv,
                       int32_t head_dim, int32_t* plan_h, int64_t plan_len);

/* Blockwise symmetric quantiser (device) -- [Digest, method]: the problem
 * statement's cu_seqlens, batch, Hq, Hkv and head_dim come in through
 * plan_h / plan_d (see the work plan above).  Only Q and K are
 * quantised, in blocks of 128 x d (Q) and 64 x d (K), symmetric with scale =
 * absmax / 127.  Per (head, block): a = max|x|, s = a / 127 and q =
 * round-half-even(x / s) clamped to [-127, 127], both divisions IEEE binary32;
 * a = 0 gives s = 0 and q = 0.  A block at a sequence end holds only that
 * sequence's rows.
 * Inputs:  q_f16 [T, Hq, d], k_f16 [T, Hkv, d] (device).
 * Outputs: q_i8 [T, Hq, d], k_i8 [T, Hkv, d] (device int8),
 *          q_scale float[Hq][total_q_tiles], k_scale float[Hkv][total_k_tiles]. */
int tilemix_quantize_qk(const int32_t* plan_h, const int32_t* plan_d, const void* q_f16,
                        const void* k_f16, int8_t* q_i8, int8_t* k_i8, float* q_scale,
                        float* k_scale, void* hip_stream);

/* Fused mixed-precision causal prefill (device) -- [Digest, method]; [Routes,
 * precision routing]; [Map, hot loop].  cu_seqlens, batch, Hq, Hkv, head_dim
 * and the grouping factors g come in through plan_h / plan_d (the work plan
 * above); words_d is the routing words' device copy.  For every legal key
 * tile t of query tile row r, bit = (word >> (t / g)) & 1 selects the score
 * path:
 *   bit 1: S = float(int32 sum of q_i8 * k_i8) * (s_q * s_k / sqrt(d))
 *   bit 0: S = (fp16 Q . fp16 K, fp32 accumulation) / sqrt(d)
 * then the causal / sequence-end mask (independent of the bit), one shared
 * online softmax (running max, normaliser, output accumulator in fp32), and
 * P.V with P rounded to fp16 and V fp16 (fp32 accumulation).  O = acc / l is
 * written as fp16 (round-to-nearest-even).
 * words_d: device uint64[Hkv][total_q_tiles] from tilemix_build_routing (bits
 * of illegal groups are never read).  q_i8/k_i8/q_scale/k_scale from
 * tilemix_quantize_qk.  out_f16: device [T, Hq, d]. */
int tilemix_prefill_varlen(const int32_t* plan_h, const int32_t* plan_d, const void* q_f16,
                           const void* k_f16, const void* v_f16, const int8_t* q_i8,
                           const int8_t* k_i8, const float* q_scale, const float* k_scale,
                           const uint64_t* words_d, void* out_f16, void* hip_stream);

/* Key half of tilemix_quantize_qk (device): the same K blocks, scales and
 * codes, for use with tilemix_prefill_varlen_qinline.
 * Inputs:  k_f16 [T, Hkv, d] (device).
 * Outputs: k_i8 [T, Hkv, d] (device int8), k_scale float[Hkv][total_k_tiles].
 * Errors: EINVAL for a missing or misaligned pointer, more than 65,535
 * sequences, or Hkv * d * 2 * 64 above 2^31 - 1 bytes. */
int tilemix_quantize_k(const int32_t* plan_h, const int32_t* plan_d, const void* k_f16, int8_t* k_i8,
                       float* k_scale, void* hip_stream);

/* tilemix_prefill_varlen with the Q quantisation done inside the kernel
 * (device) -- [Digest, method]: each work unit covers exactly one Q block
 * (128 rows of one query head), so it reduces that block's absmax across its
 * waves and forms s_q = a / 127 and the INT8 codes in registers with the
 * arithmetic of tilemix_quantize_qk.  The output equals, bit for bit, that of
 * tilemix_quantize_qk followed by tilemix_prefill_varlen on the same inputs;
 * Q's INT8 codes and scales are never written.  k_i8/k_scale from
 * tilemix_quantize_k (or tilemix_quantize_qk).  Other arguments, layouts and
 * errors as tilemix_prefill_varlen. */
int tilemix_prefill_varlen_qinline(const int32_t* plan_h, const int32_t* plan_d, const void* q_f16,
                                   const void* k_f16, const void* v_f16, const int8_t* k_i8,
                                   const float* k_scale, const uint64_t* words_d, void* out_f16,
                                   void* hip_stream);

/* INT8 key/value cache quantiser (device) -- [Explainer, 支持的场景]; [Digest,
 * setup]: the decode side keeps the cache in INT8.  Both K and V use the
 * prefill quantiser's key blocks: per (head, 64-row block of one sequence),
 * a = max|x|, s = a / 127, q = round-half-even(x / s) clamped to [-127, 127],
 * both divisions IEEE binary32, a = 0 gives s = 0 and q = 0.  The plan is the
 * one of the cache lengths.
 * Inputs:  k_f16, v_f16 [T, Hkv, d] (device).
 * Outputs: k_i8, v_i8 [T, Hkv, d] (device int8); k_scale, v_scale
 *          float[Hkv][total_k_tiles] (device). */
int tilemix_quantize_kv(const int32_t* plan_h, const int32_t* plan_d, const void* k_f16,
                        const void* v_f16, int8_t* k_i8, int8_t* v_i8, float* k_scale,
                        float* v_scale, void* hip_stream);

/* FP8 (E4M3) blockwise quantiser (device): the blocks of tilemix_quantize_qk,
 * s = fl32(absmax / 448), code = E4M3 round-half-even of fl32(x / s) (IEEE
 * division); a = 0 gives s = 0 and codes 0.
 * Outputs: q_f8 [T, Hq, d], k_f8 [T, Hkv, d] (device bytes), q_scale_f8
 * float[Hq][total_q_tiles], k_scale_f8 float[Hkv][total_k_tiles]. */
int tilemix_quantize_qk_fp8(const int32_t* plan_h, const int32_t* plan_d, const void* q_f16,
                            const void* k_f16, uint8_t* q_f8, uint8_t* k_f8, float* q_scale_f8,
                            float* k_scale_f8, void* hip_stream);

/* Three-path fused prefill (device): as tilemix_prefill_varlen, and a group
 * whose bit is set in words_f8_d (and not in words_i8_d) computes
 * S = (sum over d of q_f8 * k_f8) * (s_q8 * s_k8 / sqrt(d)) on the FP8 matrix
 * cores.  The E4M3 products are exact, but the matrix instruction does not
 * sum them in full binary32: each 64-product step may be off by up to about
 * 2^-11.5 of its largest product (measured), which matters only for blocks
 * dominated by a few large products. */
int tilemix_prefill_varlen3(const int32_t* plan_h, const int32_t* plan_d, const void* q_f16,
                            const void* k_f16, const void* v_f16, const int8_t* q_i8, const int8_t* k_i8,
                            const float* q_scale, const float* k_scale, const uint8_t* q_f8,
                            const uint8_t* k_f8, const float* q_scale_f8, const float* k_scale_f8,
                            const uint64_t* words_i8_d, const uint64_t* words_f8_d, void* out_f16,
                            void* hip_stream);

/* Key half of tilemix_quantize_qk_fp8 (device): the same K blocks, scales
 * and codes, for use with tilemix_prefill_varlen3_qinline.
 * Outputs: k_f8 [T, Hkv, d] (device bytes), k_scale_f8 float[Hkv][total_k_tiles]. */
int tilemix_quantize_k_fp8(const int32_t* plan_h, const int32_t* plan_d, const void* k_f16, uint8_t* k_f8,
                           float* k_scale_f8, void* hip_stream);

/* Both key quantisers in one pass over K (device): the codes and scales of
 * tilemix_quantize_k and tilemix_quantize_k_fp8, bit for bit, from a single
 * read of each key block.  Outputs as those two calls. */
int tilemix_quantize_k_i8_fp8(const int32_t* plan_h, const int32_t* plan_d, const void* k_f16, int8_t* k_i8,
                              float* k_scale, uint8_t* k_f8, float* k_scale_f8, void* hip_stream);

/* tilemix_prefill_varlen3 with Q's INT8 and FP8 codes made inside the kernel
 * (device), one Q block per work unit as in tilemix_prefill_varlen_qinline:
 * the INT8 codes with the arithmetic of tilemix_quantize_qk and the E4M3 codes
 * with that of tilemix_quantize_qk_fp8, from the one block absmax.  The
 * output equals, bit for bit, that of the two quantisers followed by
 * tilemix_prefill_varlen3.  K's codes from tilemix_quantize_k and
 * tilemix_quantize_k_fp8 (or the Q/K quantisers).  Other arguments, layouts
 * and errors as tilemix_prefill_varlen3. */
int tilemix_prefill_varlen3_qinline(const int32_t* plan_h, const int32_t* plan_d, const void* q_f16,
                                    const void* k_f16, const void* v_f16, const int8_t* k_i8,
                                    const float* k_scale, const uint8_t* k_f8, const float* k_scale_f8,
                                    const uint64_t* words_i8_d, const uint64_t* words_f8_d, void* out_f16,
                                    void* hip_stream);

/* Bytes of device workspace tilemix_decode_varlen needs for this plan:
 * B * Hq * ceil(max L / 256) * (d + 2) * 4. */
int tilemix_decode_workspace_size(const int32_t* plan_h, int64_t* bytes);

/* One decode step against the INT8 cache (device).  The plan and routing
 * words are those of the cache lengths L_s (cu_seqlens of the cache, which
 * already holds the new tokens).  Each sequence's new query is the token at
 * position L_s - 1; it attends to all L_s cached positions.  Key tile t of
 * sequence s is routed by bit t / g of the word of the query-tile row holding
 * L_s - 1 ([Map, hot loop]):
 *   bit 1: S = float(int32 sum of q_i8 * k_i8) * (s_q * s_k / sqrt(d)), with
 *          q_i8, s_q the query quantised on its own (a block of one row);
 *   bit 0: S = (fp16 q . (k_i8 * s_k)) / sqrt(d);
 * then softmax over the L_s keys with P rounded to fp16 and
 * O = sum P (v_i8 * s_v) / sum P, written as fp16.
 * q_f16: device [B, Hq, d]; k_i8, v_i8, k_scale, v_scale from
 * tilemix_quantize_kv; words_d from tilemix_build_routing; workspace: device
 * scratch of at least tilemix_decode_workspace_size bytes (its contents are
 * overwritten); out_f16: device [B, Hq, d] (zeros for an empty sequence).
 * Errors: EINVAL for a missing or misaligned pointer, a small workspace, more
 * than 65,535 sequences, a sequence of more than 65,535 * 256 keys, or
 * Hkv * d * 256 above 2^31 - 1 bytes. */
int tilemix_decode_varlen(const int32_t* plan_h, const int32_t* plan_d, const void* q_f16,
                          const int8_t* k_i8, const int8_t* v_i8, const float* k_scale,
                          const float* v_scale, const uint64_t* words_d, void* workspace,
                          int64_t workspace_bytes, void* out_f16, void* hip_stream);

/* tilemix_decode_varlen without the workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The partial-softmax records live
 * in a static device array of TILEMIX_DECODE_SCRATCH_BYTES per GPU, owned by
 * the library and held until the process ends; its address is looked up once
 * per device, on the first call with that device current.  Same arguments,
 * kernels and output as tilemix_decode_varlen; nothing is allocated.  Every
 * call on a GPU shares that GPU's array (each record is written before it is
 * read, so nothing needs clearing between calls): calls that overlap on one
 * GPU (other streams, other threads) race.  Errors: as tilemix_decode_varlen,
 * plus EINVAL when tilemix_decode_workspace_size exceeds
 * TILEMIX_DECODE_SCRATCH_BYTES (use tilemix_decode_varlen then). */
int tilemix_decode_varlen_noalloc(const int32_t* plan_h, const int32_t* plan_d, const void* q_f16,
                                  const int8_t* k_i8, const int8_t* v_i8, const float* k_scale,
                                  const float* v_scale, const uint64_t* words_d, void* out_f16,
                                  void* hip_stream);

/* Bytes of device workspace tilemix_routing_importance needs:
 * (Hq * total_q_tiles + Hkv * total_k_tiles) * d * 4. */
int tilemix_importance_workspace_size(const int32_t* plan_h, int64_t* bytes);

/* Group importance for adaptive routing (device), a cheap statistic of the
 * quantiser's output:
 *   colsum of each int8 block (Q 128-row blocks per query head, K 64-row
 *   tiles per KV head);
 *   z(h, r, t) = fl32(dot) * fl32(fl32(s_q * s_k) / (n_q * n_k)), dot the
 *   exact integer dot product of the Q block's and K tile's colsums, n_q and
 *   n_k their rows;
 *   Z(kv, r, t) = max over the KV head's query heads;
 *   importance(kv, r, G) = max of Z over the group's legal tiles - max of Z
 *   over the row's legal tiles (binary32), +inf for illegal slots.
 * Inputs from tilemix_quantize_qk; workspace: device scratch of
 * tilemix_importance_workspace_size bytes (overwritten); importance_d:
 * device float[Hkv][total_q_tiles][64].  Sequences of more than 262144
 * tokens are EUNSUPPORTED. */
int tilemix_routing_importance(const int32_t* plan_h, const int32_t* plan_d, const int8_t* q_i8,
                               const int8_t* k_i8, const float* q_scale, const float* k_scale,
                               void* workspace, int64_t workspace_bytes, float* importance_d,
                               void* hip_stream);

/* Adaptive routing words selected on the device (same policy and result,
 * bit for bit, as tilemix_build_routing_adaptive, without the round trip of
 * the importances through the host) -- [Digest, setup]: the interface
 * accepts adaptive policies; [Map, "Placement can matter more than the
 * nominal percentage"].  For each (sequence, KV head) the legal groups are
 * ordered by (importance, r, G) ascending and the first
 * N8 = round-half-up(coverage_bp * N_legal / 10000) get bit 1 (INT8); -0
 * and +0 tie, a NaN importance ranks after +inf (the host builder rejects
 * NaN instead).  importance_d: device float[Hkv][total_q_tiles][64] from
 * tilemix_routing_importance (slots of illegal groups ignored); words_d:
 * device uint64[Hkv][total_q_tiles], every word of every sequence written
 * (illegal groups' bits 0).  int8_groups_h, legal_groups_h (host, [batch],
 * may be NULL): N8 and N_legal per sequence, filled once the plan and
 * coverage are accepted (before the pointer checks and the launch).
 * One workgroup per (sequence, KV head), enqueued on hip_stream.
 * Errors: EINVAL for bad plans or coverage, or a missing or misaligned
 * pointer. */
int tilemix_select_routing_adaptive(const int32_t* plan_h, const int32_t* plan_d, const float* importance_d,
                                    int32_t coverage_bp, uint64_t* words_d, int64_t* int8_groups_h,
                                    int64_t* legal_groups_h, void* hip_stream);

/* ---- Synthetic multi-layer stack ------------------------------------------
 * [Explainer, 数字精度混用到底靠不靠谱]: deeper models pile up more deviation,
 * the error of one layer being carried into the next.  The pages give no
 * layer beyond attention; the stack below keeps attention whose Q, K, V come
 * from the running hidden state, plus a residual connection.  The hidden
 * state x [T, Hq*d] (fp32) is Hkv independent streams of width
 * W = (Hq/Hkv)*d: stream g is channels g*W .. g*W+W-1, owned by KV head g
 * and its query heads g*Hq/Hkv .. (g+1)*Hq/Hkv - 1.  d is 64 or 128 and W at
 * most 1024.  All pointers are device pointers, 16-byte aligned; nothing is
 * allocated; kernels run on hip_stream.  Errors: EINVAL (NULL or misaligned
 * pointer, negative size, Hq not a multiple of Hkv, small workspace),
 * EUNSUPPORTED (d, W). */

/* u = fl16(x * 1/sqrt(mean(x^2) + eps)) per (token, stream), sum of squares
 * and the factor in binary32.  x: float [T, Hq*d]; u_f16: [T, Hq*d]. */
int tilemix_stack_rms_norm(const float* x, void* u_f16, int64_t tokens, int32_t hq, int32_t hkv,
                           int32_t head_dim, float eps, void* hip_stream);

/* [q | k | v] = u_g . Wqkv_g^T per stream (f16 matrix cores, fp32
 * accumulation, one rounding to fp16).  wqkv_f16: [Hkv][W + 2d][W], row n of
 * stream g = the weights of output n: n < W feeds q head g*Hq/Hkv + n/d,
 * channel n % d; n in [W, W+d) feeds k head g, channel n - W; the last d rows
 * feed v head g.  Outputs q_f16 [T, Hq, d], k_f16 and v_f16 [T, Hkv, d]. */
int tilemix_stack_qkv(const void* u_f16, const void* wqkv_f16, void* q_f16, void* k_f16, void* v_f16,
                      int64_t tokens, int32_t hq, int32_t hkv, int32_t head_dim, void* hip_stream);

/* x_g += o_g . Wo_g^T per stream (fp32 accumulation, then one fp32 add).
 * o_f16: [T, Hq, d] (query head g*Hq/Hkv + j fills stream channels
 * j*d .. j*d+d-1); wo_f16: [Hkv][W][W], row n = output channel n. */
int tilemix_stack_out_residual(const void* o_f16, const void* wo_f16, float* x, int64_t tokens,
                               int32_t hq, int32_t hkv, int32_t head_dim, void* hip_stream);

/* Bytes of device workspace one tilemix_stack_layer call needs for this
 * plan (normalised input / attention output, Q, K, V, K's int8 codes and
 * scales). */
int tilemix_stack_workspace_size(const int32_t* plan_h, int64_t* bytes);

/* One layer in place on x (device float [T, Hq*d], T = the plan's tokens):
 * tilemix_stack_rms_norm, tilemix_stack_qkv, tilemix_quantize_k,
 * tilemix_prefill_varlen_qinline with words_d ([Digest, method]: the same template
 * words serve every layer), tilemix_stack_out_residual.  The workspace's
 * contents are overwritten; calls that share a workspace must not overlap. */
int tilemix_stack_layer(const int32_t* plan_h, const int32_t* plan_d, const uint64_t* words_d, float* x,
                        const void* wqkv_f16, const void* wo_f16, float eps, void* workspace,
                        int64_t workspace_bytes, void* hip_stream);

/* Test hook (device): the int32 accumulator of one 128 x 64 INT8 score tile
 * (sequence seq, query head, query-tile row r, key tile t), computed by the
 * same device routine the fused kernel uses ([Digest, method]: INT8 MMA with
 * INT32 accumulation).  Entries whose query or key lies outside the sequence
 * are 0.  acc_d: device int32[128][64]. */
int tilemix_debug_qk_i32_tile(const int32_t* plan_h, const int32_t* plan_d, const int8_t* q_i8,
                              const int8_t* k_i8, int32_t seq, int32_t head, int32_t r,
                              int32_t t, int32_t* acc_d, void* hip_stream);

/* Test hook (device): the fp32 accumulator of one 128 x 64 FP8 (E4M3) score
 * tile -- the sum over d of q_f8 * k_f8 products of E4M3 values, no scale
 * applied -- computed by the routine the three-path kernel uses for FP8
 * groups (the open FP8 question of [Digest, setup]; [Explainer, 写在后面]), so
 * the accumulation of the FP8 matrix instruction can be compared with exact
 * sums.  q_f8/k_f8 from tilemix_quantize_qk_fp8.  Entries whose query or key
 * lies outside the sequence are 0.  acc_d: device float[128][64]. */
int tilemix_debug_qk_f8_tile(const int32_t* plan_h, const int32_t* plan_d, const uint8_t* q_f8,
                             const uint8_t* k_f8, int32_t seq, int32_t head, int32_t r, int32_t t,
                             float* acc_d, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* TILEMIX_H */
