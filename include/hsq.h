/*
 * hsq.h -- C ABI of libhsq: the HSQ decode step and its TurboQuant codec on
 * AMD Instinct MI355X (gfx950).
 *
 * Method sources (web pages):
 *  [HSQ]  "Tamarin (HSQ) - reversible hierarchical KV-cache compression",
 *         technical summary, section 2 "Methodology": "Three-tier
 *         architecture", "Decode process", "Key technical components".
 *  [ABL]  "Ablation, Statistical Inference, and Validation for KV-Cache
 *         Compression", technical summary, "Experimental setup" (TurboQuant =
 *         random Walsh-Hadamard transform + data-oblivious Beta Lloyd-Max
 *         codebook).
 *
 * Conventions shared by every call
 *  - Return value: HSQ_OK (0) or a negative HSQ_ERR_* code.  Arguments are
 *    validated on the host before anything is launched; an argument error
 *    launches nothing.  hsq_last_error() returns a thread-local message for
 *    the last failing call on the calling thread.
 *  - Device calls are asynchronous on `stream` (a hipStream_t passed as
 *    void*; NULL = the null stream).  They never allocate, never free and
 *    never synchronise the host.  The caller owns every buffer and keeps it
 *    alive until the stream work completes.  Pointers are device pointers
 *    (hipMalloc'd, or the device alias of pinned mapped host memory where a
 *    call says "device-visible").
 *  - Shapes: d (head dim) in {64, 128}; 4-bit and 3-bit codes; group size
 *    N in {8, 16}; Hq % Hkv == 0 with G = Hq / Hkv in 1..8.  Query head h
 *    belongs to kv-head h / G.
 *  - Rotation: R = H_d D / sqrt(d).  D = diag(+-1) from a sign mask of d/32
 *    uint32 words, bit i of word i/32 set meaning coordinate i is negated;
 *    H_d is the Sylvester Hadamard matrix, H_ij = (-1)^popcount(i & j).
 *    One mask per (layer, kv-head, K|V) [HSQ, quantisation item: fixed random
 *    orthonormal rotation; ABL: random Walsh-Hadamard transform].
 *  - Vector record: r = ||x||_2 as fp32 plus codes of y = R x / r,
 *    code_i = #{j : t_j < y_i} against the ascending fp32 thresholds.
 *    4-bit packing: byte k = code[2k] | code[2k+1] << 4 (d/2 bytes).
 *    3-bit packing: LSB-first bit stream, code i in bits [3i, 3i+3)
 *    (3d/8 bytes).  Dequantisation: x_hat = r R^T c[code].
 *  - Tier layouts (unit u = b * Hkv + kvh):
 *      L1  codes [B][Hkv][n1][d/2] u8, norms [B][Hkv][n1] f32   (4-bit)
 *      L2  codes [B][Hkv][ng][3d/8] u8, norms [B][Hkv][ng] f32  (3-bit)
 *      L3  records [B][Hkv][ng], one record per group of N tokens:
 *          [K codes N*d/2][K norms N*4][V codes N*d/2][V norms N*4] bytes,
 *          i.e. N*(d+8) bytes.
 *    L1 and L2 have separate K and V arrays.
 */
#ifndef HSQ_H
#define HSQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  HSQ_OK = 0,
  HSQ_ERR_ARG = -1,         /* invalid argument (null pointer, bad size) */
  HSQ_ERR_UNSUPPORTED = -2, /* valid but unsupported shape (d, bits, N, G) */
  HSQ_ERR_HIP = -3,         /* a HIP runtime call or launch failed */
  HSQ_ERR_WORKSPACE = -4    /* workspace missing or smaller than required */
};

enum { HSQ_F32 = 0, HSQ_BF16 = 1 };
enum { HSQ_AGG_MAX = 0, HSQ_AGG_MEAN = 1 };

/* Library version string (static storage). */
const char* hsq_version(void);

/* Message of the last failing call on this thread ("" if none). */
const char* hsq_last_error(void);

/* ---------------------------------------------------------------- host ---- */

/*
 * hsq_codebook -- Beta Lloyd-Max codebook for (d, bits) [ABL, "Experimental
 * setup": data-oblivious Beta Lloyd-Max codebook].  The quantised variable
 * is one coordinate of a uniformly random unit vector in R^d, density
 * proportional to (1 - y^2)^((d-3)/2) on [-1, 1].  Computed on the host in
 * double precision by Lloyd iteration to its fixed point (centroid =
 * conditional mean of its cell, threshold = midpoint of neighbouring
 * centroids), made exactly odd-symmetric.  Stored tables: the fixed
 * point's centroids and its thresholds (midpoints formed in double
 * precision), each rounded to the nearest fp32 value, so the tables satisfy
 * both Lloyd conditions to fp32 rounding.
 *   d           3..4096 (any integer; the codec itself needs d in {64,128})
 *   bits        1..4
 *   centroids   host out, [2^bits] ascending
 *   thresholds  host out, [2^bits - 1] ascending (middle one exactly 0)
 * Errors: HSQ_ERR_ARG for null pointers or d/bits out of range.
 */
int hsq_codebook(int d, int bits, float* centroids, float* thresholds);

/*
 * hsq_tier_plan -- split the T positions of one sequence into L1 and groups
 * [HSQ, "Three-tier architecture": L1 = attention sinks + recent window +
 * reader-marked tokens; the rest in groups of N].  L1 = positions
 * [0, n_sink) + [T - n_recent, T) + marked + the trailing remainder of fewer
 * than N non-L1 positions, ascending.  Groups = the other positions in
 * ascending order, cut into consecutive runs of N.
 *   marked      host in, [n_marked] positions in [0, T) (duplicates allowed)
 *   l1_pos      host out [T] capacity, or NULL to query only n1
 *   group_pos   host out [T] capacity, or NULL; group g = entries
 *               [g*N, (g+1)*N)
 *   n1, n_groups  host out
 * Errors: HSQ_ERR_ARG for T < 1, negative counts, N < 1, marks out of range.
 */
int hsq_tier_plan(int T, int n_sink, int n_recent, const int32_t* marked, int n_marked,
                  int group_n, int32_t* l1_pos, int* n1, int32_t* group_pos, int* n_groups);

/*
 * hsq_workspace_bytes -- device workspace needed by hsq_route_topk,
 * hsq_decode_attn and hsq_decode_step for these sizes (one number covers
 * all three).  Returns 0 on invalid sizes.
 */
size_t hsq_workspace_bytes(int B, int Hq, int Hkv, int d, int n_l1, int n_groups, int beta,
                           int group_n);

/* -------------------------------------------------------------- device ---- */

/*
 * hsq_encode -- TurboQuant encode of n_vec vectors [HSQ quantisation item;
 * ABL "Experimental setup"]: norm, sign flip, Walsh-Hadamard transform,
 * threshold count, bit packing.  Variants [ABL "Key contributions" item 1,
 * "Results and recommendations"]: signs == NULL is Plain-KV (rotation off:
 * the unit vector x / r is quantised as it is); bits == 2 is the 2-bit budget.
 *   x           [rows][d] in x_dtype (HSQ_F32 or HSQ_BF16)
 *   row_idx     NULL: vector i reads rows [i*group_n, (i+1)*group_n);
 *               else int64 [n_vec*group_n] row numbers
 *   group_n     1 = encode each row; N > 1 = encode the mean of N rows
 *   signs       uint32 [n_rot][d/32]; vector i uses mask
 *               (i / vecs_per_rot) % n_rot; NULL = no rotation
 *               (vecs_per_rot and n_rot are then not used, but must be >= 1)
 *   bits        2, 3 or 4
 *   thresholds  fp32 [2^bits - 1] ascending and symmetric about 0 (the
 *               middle one 0, t[2^bits - 2 - k] = -t[k]), as hsq_codebook
 *               gives (device)
 *   codes       out [n_vec][bits*d/8]: 4-bit, byte k = code[2k] |
 *               code[2k+1] << 4; 2- and 3-bit, an LSB-first bit stream
 *               with code i in bits [bits*i, bits*i + bits)
 *   norms       out [n_vec] fp32
 * Errors: HSQ_ERR_ARG (null x, thresholds, codes or norms, n_vec < 0,
 * vecs_per_rot < 1, n_rot < 1, group_n < 1), HSQ_ERR_UNSUPPORTED (d, bits,
 * dtype, n_vec >= 2^32), HSQ_ERR_HIP.
 * n_vec == 0 is a no-op.
 */
int hsq_encode(const void* x, int x_dtype, int64_t n_vec, int d, int bits,
               const int64_t* row_idx, int group_n, const uint32_t* signs,
               int64_t vecs_per_rot, int n_rot, const float* thresholds, uint8_t* codes,
               float* norms, void* stream);

/*
 * hsq_decode -- dequantise n_vec vectors: x_hat = r R^T c[code]
 * [HSQ "Decode process" step 2: dequantise and rotate back].
 *   codes/norms as written by hsq_encode; centroids fp32 [2^bits] (device);
 *   signs as for hsq_encode (NULL: R = I, x_hat = r c[code]);
 *   out [n_vec][d] in out_dtype (HSQ_F32 or HSQ_BF16).
 * Errors as hsq_encode.
 */
int hsq_decode(const uint8_t* codes, const float* norms, int64_t n_vec, int d, int bits,
               const uint32_t* signs, int64_t vecs_per_rot, int n_rot, const float* centroids,
               void* out, int out_dtype, void* stream);

/*
 * hsq_decode_rope -- the fetch of a pre-RoPE archive: dequantise n_vec
 * vectors as hsq_decode does, then rotate vector i to position positions[i]
 * with the rotary position embedding
 * [HSQ "Decode process" step 2: dequantise, then rotate to the semantic
 * positions; RoPE as in Su et al., RoFormer (2021)].
 *   Coordinate f < d/2 pairs with f + d/2 and turns by the angle
 *   positions[i] * rope_base^(-2f/d):
 *     (a, b) -> (a cos - b sin, b cos + a sin).
 *   The angle's fraction of a turn comes from a 64-bit fixed-point product
 *   (within 2e-7 rad at any int32 position); sine, cosine and the rotation
 *   are fp32.
 *   positions   int32 [n_vec] (device), any value (negative turns backwards)
 *   rope_base   the rotary base (1e6 for the Qwen3 models), finite, > 0
 *   everything else as for hsq_decode.
 * Errors as hsq_decode, plus HSQ_ERR_ARG for a null positions or a bad
 * rope_base.
 */
int hsq_decode_rope(const uint8_t* codes, const float* norms, int64_t n_vec, int d, int bits,
                    const uint32_t* signs, int64_t vecs_per_rot, int n_rot,
                    const float* centroids, const int32_t* positions, double rope_base,
                    void* out, int out_dtype, void* stream);

/*
 * hsq_build_tiers -- build L1, L2 and L3 of one layer from raw K and V
 * [HSQ "Three-tier architecture"; L2 summary = 3-bit code of the mean of the
 * group's raw vectors, standing in for the trained compressor].
 *   k, v        [B][Hkv][T][d] in dtype
 *   l1_pos      int32 [B][n1] positions (device), as hsq_tier_plan gives
 *   group_pos   int32 [B][n_groups*group_n] positions (device)
 *   k_signs, v_signs  uint32 [Hkv][d/32]
 *   thr4, thr3  fp32 thresholds for 4 and 3 bits (device)
 *   outputs     tier arrays in the layouts above
 * n1 == 0 or n_groups == 0 skip the matching tiers.
 * Errors: HSQ_ERR_ARG (null pointers, bad sizes, n1 + n_groups*group_n > T),
 * HSQ_ERR_UNSUPPORTED (d, dtype, B*Hkv*T >= 2^32), HSQ_ERR_HIP.
 */
int hsq_build_tiers(const void* k, const void* v, int dtype, int B, int Hkv, int T, int d,
                    const int32_t* l1_pos, int n1, const int32_t* group_pos, int n_groups,
                    int group_n, const uint32_t* k_signs, const uint32_t* v_signs,
                    const float* thr4, const float* thr3, uint8_t* l1k, float* l1k_n,
                    uint8_t* l1v, float* l1v_n, uint8_t* l2k, float* l2k_n, uint8_t* l2v,
                    float* l2v_n, uint8_t* l3, void* stream);

/*
 * hsq_route_topk -- router + top-beta [HSQ "Decode process" steps 1-2].
 * For every unit (b, kvh) and group g: s_g = agg over the G query heads h of
 * kvh of scale * q_h . k_hat_g, with k_hat_g the dequantised 3-bit summary
 * key; then the beta largest s_g, ties to the lower g, written ascending.
 *   q           fp32 [B][Hq][d]
 *   l2k/l2k_n   3-bit summary keys / norms
 *   k_signs     uint32 [Hkv][d/32];  cb3 fp32 [8] centroids (device)
 *   agg         HSQ_AGG_MAX or HSQ_AGG_MEAN
 *   beta        >= 0, clamped to n_groups
 *   topk_idx    out int32 [B][Hkv][min(beta, n_groups)]
 *   scores      optional out fp32 [B][Hkv][n_groups] (NULL = not written).
 *               When asked for, the router adds the centroids' low parts and
 *               the scores are fp32-accurate; otherwise the selection is
 *               still exact: groups whose computed score lies within the
 *               computed scores' error bound of the beta-th are re-scored with
 *               the fp32 centroids before the tie-break.
 *   workspace   device, >= hsq_workspace_bytes(...) bytes, 256-byte aligned;
 *               holds the selection and the summary-attention partials
 *               between the launches of one call.  No initial contents are
 *               needed.  Calls that share a workspace must be ordered on one
 *               stream.
 * When G * n_groups exceeds 12288 (more router logits than one work-group
 * holds on chip) the scores go through the workspace (two launches).
 * Errors: HSQ_ERR_ARG (null pointers, negative sizes, bad agg),
 * HSQ_ERR_UNSUPPORTED (d, G > 8, n_groups > 16384), HSQ_ERR_WORKSPACE,
 * HSQ_ERR_HIP.
 */
int hsq_route_topk(const float* q, int B, int Hq, int Hkv, int d, const uint8_t* l2k,
                   const float* l2k_n, int n_groups, const uint32_t* k_signs, const float* cb3,
                   float scale, int agg, int beta, int32_t* topk_idx, float* scores,
                   void* workspace, size_t ws_bytes, void* stream);

/*
 * hsq_decode_attn -- fused union-set attention given the fetched groups
 * [HSQ "Decode process" step 3].  For query head h of unit (b, kvh):
 *   out = sum_e softmax_e(scale * q_h . k_e + bias_e) v_e
 * over e in L1 tokens, summaries of groups NOT in topk_idx (bias =
 * summary_bias) and the N tokens of every group in topk_idx (dequantised
 * 4-bit originals).  Summaries of fetched groups are excluded.
 *   topk_idx    int32 [B][Hkv][beta] distinct group ids in [0, n_groups)
 *   l3          device-visible L3 base.  l3_staged == 0: records
 *               [B][Hkv][n_groups] (HBM-resident, or the device alias of a
 *               pinned mapped host archive); l3_staged == 1: records
 *               [B][Hkv][beta] in topk_idx order (hsq_gather_l3 output)
 *   cb4, cb3    fp32 centroids [16], [8] (device)
 *   out         fp32 [B][Hq][d]; a unit with no entries at all gets zeros
 * Errors: as hsq_route_topk; HSQ_ERR_UNSUPPORTED also when G * n_groups
 * exceeds 12288 (hsq_decode_step serves such shapes).
 */
int hsq_decode_attn(const float* q, int B, int Hq, int Hkv, int d, const uint8_t* l1k,
                    const float* l1k_n, const uint8_t* l1v, const float* l1v_n, int n_l1,
                    const uint8_t* l2k, const float* l2k_n, const uint8_t* l2v,
                    const float* l2v_n, int n_groups, const uint8_t* l3, int group_n,
                    int l3_staged, const int32_t* topk_idx, int beta, const uint32_t* k_signs,
                    const uint32_t* v_signs, const float* cb4, const float* cb3, float scale,
                    float summary_bias, void* workspace, size_t ws_bytes, float* out,
                    void* stream);

/*
 * hsq_decode_step -- the whole decode step of one layer: route, top-beta and
 * attention [HSQ "Decode process" steps 1-3]: hsq_route_topk followed by
 * hsq_decode_attn with l3_staged == 0 (the same selection; the output to
 * fp32 rounding of the order in which the partials merge).  With
 * 1 <= n_groups <= 2048 it runs as one launch, one work-group per unit (b,
 * kvh), for any number of units: one stream over the summaries (router
 * scores and the summary attention together), the selection on chip, then
 * the fetched summaries taken out again and the tokens attended.  With more
 * than 2048 groups it runs as the split step when there are fewer than 128
 * units or G * n_groups > 12288: four launches that spread each unit over
 * many work-groups (router logits and keys, the selection, summary-value and
 * token chunks as partials, a log-sum-exp merge), with the hand-overs in the
 * workspace; a unit's result depends only on its own inputs, not on the
 * batch.  Otherwise (more than 2048 groups, 128 or more units,
 * G * n_groups <= 12288), and with n_groups == 0, it runs as the two
 * launches of hsq_route_topk and hsq_decode_attn.
 *   topk_idx    optional out int32 [B][Hkv][min(beta, n_groups)] (NULL = not
 *               returned)
 *   other arguments as in hsq_route_topk / hsq_decode_attn
 */
int hsq_decode_step(const float* q, int B, int Hq, int Hkv, int d, const uint8_t* l1k,
                    const float* l1k_n, const uint8_t* l1v, const float* l1v_n, int n_l1,
                    const uint8_t* l2k, const float* l2k_n, const uint8_t* l2v,
                    const float* l2v_n, int n_groups, const uint8_t* l3, int group_n, int beta,
                    int agg, const uint32_t* k_signs, const uint32_t* v_signs, const float* cb4,
                    const float* cb3, float scale, float summary_bias, int32_t* topk_idx,
                    void* workspace, size_t ws_bytes, float* out, void* stream);

/*
 * hsq_prerope_workspace_bytes / hsq_decode_step_prerope -- the decode step
 * over a pre-RoPE archive [HSQ "Decode process" step 2: the originals of the
 * fetched groups are dequantised and rotated to their semantic positions
 * before they are attended; RoPE as in Su et al., RoFormer (2021), pairing
 * coordinate f < d/2 with f + d/2 as hsq_decode_rope does].  L1 and L2 hold
 * keys with RoPE applied, as for hsq_decode_step; the L3 records hold the
 * keys without it (values are never rotated).  The route, the selection, the
 * summaries and L1 are as in hsq_decode_step (hsq_step_route, then
 * hsq_step_attend_prerope over the archive in place); between them a
 * third launch takes every fetched record's 4-bit key codes back to the
 * model's domain and rotates each token to its position, into fp16 rows in
 * the workspace, and the attention multiplies those rows against the
 * unrotated query where it would look the codes up (the norms, the values
 * and everything else unchanged).
 *   group_pos   int32 [B][n_groups*group_n] (device): position of token t of
 *               group g of sequence b at [b][g*group_n + t], any value
 *   rope_base   the rotary base (1e6 for the Qwen3 models), finite, > 0
 *   workspace   hsq_prerope_workspace_bytes(...) bytes, 256-byte aligned:
 *               hsq_workspace_bytes' plus B*Hkv*min(beta, n_groups)*group_n*d
 *               fp16 rows
 *   other arguments as in hsq_decode_step
 * With G * n_groups > 12288 (router logits beyond the chip's LDS) the route
 * and the attend are the split step's two halves, the RoPE pass between.
 * Errors: as hsq_decode_step, plus HSQ_ERR_ARG for a null group_pos (with
 * n_groups > 0) or a bad rope_base.
 * hsq_prerope_workspace_bytes returns 0 for sizes hsq_workspace_bytes
 * rejects.
 */
size_t hsq_prerope_workspace_bytes(int B, int Hq, int Hkv, int d, int n_l1, int n_groups,
                                   int beta, int group_n);
/*
 * hsq_step_attend_prerope -- the second half of the pre-RoPE step, after
 * hsq_step_route on the same workspace (hsq_prerope_workspace_bytes bytes):
 * the fetched keys rotated to their positions, then the attend.  With
 * l3_staged != 0, l3 holds the fetched records gathered by hsq_gather_l3
 * ([B][Hkv][beta] records, the CPU-RAM archive of the pages read over
 * PCIe); else the whole archive in device memory.  The positions come from
 * the selection hsq_step_route left in the workspace.  Arguments and errors
 * as hsq_step_attend plus group_pos and rope_base as below.
 */
int hsq_step_attend_prerope(const float* q, int B, int Hq, int Hkv, int d, const uint8_t* l1k,
                            const float* l1k_n, const uint8_t* l1v, const float* l1v_n, int n_l1,
                            int n_groups, const uint8_t* l3, int group_n, int l3_staged, int beta,
                            const uint32_t* k_signs, const uint32_t* v_signs, const float* cb4,
                            float scale, const int32_t* group_pos, double rope_base,
                            void* workspace, size_t ws_bytes, float* out, void* stream);
int hsq_decode_step_prerope(const float* q, int B, int Hq, int Hkv, int d, const uint8_t* l1k,
                            const float* l1k_n, const uint8_t* l1v, const float* l1v_n, int n_l1,
                            const uint8_t* l2k, const float* l2k_n, const uint8_t* l2v,
                            const float* l2v_n, int n_groups, const uint8_t* l3, int group_n,
                            int beta, int agg, const uint32_t* k_signs, const uint32_t* v_signs,
                            const float* cb4, const float* cb3, float scale, float summary_bias,
                            const int32_t* group_pos, double rope_base, int32_t* topk_idx,
                            void* workspace, size_t ws_bytes, float* out, void* stream);

/*
 * hsq_decode_step_qjl -- the decode step over TQ-QKV token keys [ABL "Key
 * contributions" 1: TQ-QKV = TurboQuant plus a 1-bit QJL sketch of the key
 * residual; estimator as hsq_qjl_logits].  Every 4-bit token key (L1 and the
 * archive) carries its sketch and gamma, as hsq_encode_qjl writes them for
 * that key (same signs, the 4-bit codebook, one S per kv-head); the L2
 * summaries do not.  The route, the selection and the summaries are as in
 * hsq_decode_step (two launches); the logit of every L1 token and every
 * fetched token is
 *   scale * (r <R q, c[code]> + sqrt(pi/2)/d * gamma * <S R q, 1 - 2 bits>),
 * the correction formed on MFMA from the sketch bits (fp16 S R q operands).
 *   l1_sketch   uint8 [B][Hkv][n_l1][d/8], l1_gamma fp32 [B][Hkv][n_l1]
 *               (the L1 keys in L1 order)
 *   l3_sketch   uint8 [B][Hkv][n_groups][group_n][d/8], l3_gamma fp32
 *               [B][Hkv][n_groups][group_n] (the grouped keys in group order)
 *   S           fp32 [Hkv][d][d], row j = sketch direction j of kv-head h,
 *               16-byte aligned (sketch arrays and gammas 4-byte aligned)
 *   workspace   hsq_workspace_bytes(...) bytes, as hsq_decode_step
 *   other arguments as in hsq_decode_step
 * With G * n_groups > 12288 it runs as the split step's two halves, the
 * token chunks with the sketch correction.
 * Errors: as hsq_decode_step, plus HSQ_ERR_ARG for a null or misaligned S,
 * null or misaligned sketches or gammas of a tier that has entries.
 */
int hsq_decode_step_qjl(const float* q, int B, int Hq, int Hkv, int d, const uint8_t* l1k,
                        const float* l1k_n, const uint8_t* l1v, const float* l1v_n, int n_l1,
                        const uint8_t* l2k, const float* l2k_n, const uint8_t* l2v,
                        const float* l2v_n, int n_groups, const uint8_t* l3, int group_n,
                        int beta, int agg, const uint32_t* k_signs, const uint32_t* v_signs,
                        const float* cb4, const float* cb3, float scale, float summary_bias,
                        const uint8_t* l1_sketch, const float* l1_gamma,
                        const uint8_t* l3_sketch, const float* l3_gamma, const float* S,
                        int32_t* topk_idx, void* workspace, size_t ws_bytes, float* out,
                        void* stream);

/*
 * hsq_decode_step_static -- hsq_decode_step without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * workspace is a file-scope device array of 8 MiB per GPU, kept until the
 * process ends; the call allocates nothing and calls no allocating routine.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (other streams, other host threads) race; calls on one stream are
 * ordered and safe.  The array needs no initial contents (each call writes
 * what it later reads).
 * Errors: as hsq_decode_step; HSQ_ERR_UNSUPPORTED when the sizes need more
 * than 8 MiB of workspace (hsq_workspace_bytes) or the device ordinal is
 * above 63; HSQ_ERR_HIP when the array's address cannot be looked up.
 */
int hsq_decode_step_static(const float* q, int B, int Hq, int Hkv, int d, const uint8_t* l1k,
                           const float* l1k_n, const uint8_t* l1v, const float* l1v_n, int n_l1,
                           const uint8_t* l2k, const float* l2k_n, const uint8_t* l2v,
                           const float* l2v_n, int n_groups, const uint8_t* l3, int group_n,
                           int beta, int agg, const uint32_t* k_signs, const uint32_t* v_signs,
                           const float* cb4, const float* cb3, float scale, float summary_bias,
                           int32_t* topk_idx, float* out, void* stream);

/*
 * hsq_step_route / hsq_step_attend -- the two launches of hsq_decode_step,
 * exposed so a caller can put work between them: the host-archive path runs
 * hsq_step_route, then hsq_gather_l3 (PCIe, side stream), then
 * hsq_step_attend with l3_staged = 1 [HSQ "Decode process": routing, then
 * fetching from the CPU archive, then attention].
 *   hsq_step_route   router scores, top-beta and the summary-attention
 *                    partials (all summaries, then the fetched ones removed)
 *                    into the workspace.  The selection stays at the start
 *                    of the workspace, int32 [B*Hkv][min(beta, n_groups)]
 *                    ascending per unit, where a device-side consumer such
 *                    as hsq_gather_l3 can read it in place; topk_idx
 *                    (optional) receives a copy.
 *   hsq_step_attend  L1 and fetched-token attention, merge with the summary
 *                    partials, inverse V rotation, out.  Reads the selection
 *                    from the workspace written by the preceding
 *                    hsq_step_route with the same sizes and workspace.
 * Both take n_l1 and n_groups so they size the workspace identically.
 * Shapes with G * n_groups above 12288 (more router logits than these
 * launches hold on chip) run as the two halves of the split decode step (see
 * hsq_decode_step): hsq_step_route launches the score chunks, the selection
 * and the summary-value chunks, hsq_step_attend the token chunks (L1 and the
 * fetched records, staged ones read by slot) and the merge.
 * Errors: as hsq_decode_attn, without its G * n_groups limit.
 */
int hsq_step_route(const float* q, int B, int Hq, int Hkv, int d, int n_l1, const uint8_t* l2k,
                   const float* l2k_n, const uint8_t* l2v, const float* l2v_n, int n_groups,
                   int group_n, int beta, int agg, const uint32_t* k_signs, const float* cb3,
                   float scale, float summary_bias, int32_t* topk_idx, void* workspace,
                   size_t ws_bytes, void* stream);
int hsq_step_attend(const float* q, int B, int Hq, int Hkv, int d, const uint8_t* l1k,
                    const float* l1k_n, const uint8_t* l1v, const float* l1v_n, int n_l1,
                    int n_groups, const uint8_t* l3, int group_n, int l3_staged, int beta,
                    const uint32_t* k_signs, const uint32_t* v_signs, const float* cb4,
                    float scale, void* workspace, size_t ws_bytes, float* out, void* stream);

/*
 * hsq_gather_l3 -- copy the fetched L3 records into a staging buffer
 * [HSQ "Decode process" step 2: fetch the originals of the chosen groups
 * from the CPU archive].  Reads device-visible `l3_src` (typically the
 * device alias of pinned mapped host memory, so the copy crosses PCIe with
 * indices that never leave the device) and writes
 * staging[u][i] = l3_src[u][topk_idx[u][i]] for units u < B*Hkv, i < beta.
 *   rec_bytes   bytes per record, N*(d+8); a multiple of 16, at most 1 MiB
 * A selection index outside [0, n_groups) leaves its staging record as it
 * was.  The launch uses few work-groups (128 records each), so that route
 * and attend launches of other micro-batches keep most CUs to themselves.
 * Errors: HSQ_ERR_ARG (null, sizes), HSQ_ERR_UNSUPPORTED (rec_bytes above
 * 1 MiB, B*Hkv*beta >= 2^32), HSQ_ERR_HIP.
 */
int hsq_gather_l3(const uint8_t* l3_src, size_t rec_bytes, int B, int Hkv, int n_groups,
                  const int32_t* topk_idx, int beta, uint8_t* staging, void* stream);

/*
 * hsq_gather_l3_ordered -- hsq_gather_l3 that takes its turn on the PCIe
 * link after other gathers, for callers that split a batch into
 * micro-batches on several streams [HSQ "Decode process" step 2; the
 * pages put long-context decode time on the fetch from CPU memory, HSQ
 * section 4 "Results"].  Before copying, the call's work-groups wait on the
 * device until *turn >= after (compared modulo 2^32), for at most about
 * 2 ms, and then copy regardless: the wait orders use of the link and never
 * the data, so a wrong `after` costs time, not correctness.  Each
 * work-group adds its records to *turn when its reads are done: once the
 * call completes, *turn has grown by B*Hkv*beta.  A chain of gathers on
 * any streams passes after = the running total of B*Hkv*beta of the gathers
 * before it, with *turn zeroed (on the device, before the first) by the
 * caller; the gathers then run one after the other without host-side
 * events between the streams.
 *   turn        device uint32, 4-byte aligned, owned by the caller
 * Errors: as hsq_gather_l3; HSQ_ERR_ARG for a null or misaligned turn;
 * HSQ_ERR_UNSUPPORTED when B*Hkv*beta >= 2^32.
 */
int hsq_gather_l3_ordered(const uint8_t* l3_src, size_t rec_bytes, int B, int Hkv, int n_groups,
                          const int32_t* topk_idx, int beta, uint8_t* staging, uint32_t* turn,
                          uint32_t after, void* stream);

/* ------------------------------------------ decode-time tier maintenance -- */

/*
 * Cache layout.  The tiers of a layer that grows during decoding, with room
 * reserved per unit u = b * Hkv + kvh (capacities l1_cap rows, ng_cap groups):
 *   L1   codes [B][Hkv][l1_cap][d/2] u8, norms [B][Hkv][l1_cap] f32 (K and V).
 *        Rows [0, n_fix): sinks and reader-marked tokens; rows
 *        [n_fix, n_fix + W): the recent window, position p in row
 *        n_fix + p % W; rows [n_fix + W, n_fix + W + n_pending): the pending
 *        tokens (left the window, not yet grouped) in position order.
 *        n_l1 = n_fix + W + n_pending.
 *   raw  K and V [B][Hkv][W + N][d] in the append dtype: row p % W holds the
 *        raw vector of window position p, row W + j that of pending token j
 *        (a group summary is the mean of raw vectors).
 *   L2   codes [B][Hkv][ng_cap][3d/8] u8, norms [B][Hkv][ng_cap] f32.
 *   L3   records [B][Hkv][ng_cap], N*(d+8) bytes each (layout above).
 * A compress-time build (hsq_build_tiers with l1_pos listing the L1 rows in
 * this order) placed into these arrays gives the starting cache.
 */

/*
 * hsq_cache_append -- append one token per unit at position t (the context
 * held t tokens) [HSQ "Three-tier architecture": the tiers after the call
 * are those the compress-time build gives for the t + 1 tokens with the same
 * reader marks; new tokens are not marked].  Steps, in stream order:
 *   1. position t - W leaves the window: its L1 row and raw row move to
 *      pending slot n_pending;
 *   2. the new token is encoded at 4 bits into the window row of slot t % W
 *      and its raw vector stored in raw row t % W;
 *   3. if n_pending + 1 == group_n, the N pending tokens are sealed as group
 *      n_groups: their codes and norms form its L3 record, and the 3-bit
 *      code of the mean of their raw vectors its K and V summaries in L2.
 * After the call the caller's counts are n_pending + 1 (or 0 after a seal,
 * with n_groups + 1).  Requires every position of the window to be bound for
 * a group (the window past the sinks and holding no marked position), which
 * a cache built from a prefix of at least n_sink + W tokens satisfies.
 *   k_new, v_new  [B][Hkv][d] in dtype (HSQ_F32 or HSQ_BF16), the raw dtype
 *   t             >= n_recent;  0 <= n_pending < group_n
 *   l1_cap        >= n_fix + n_recent + group_n;  ng_cap > n_groups on a seal
 *   k_signs, v_signs, thr4, thr3  as for hsq_build_tiers
 * Errors: HSQ_ERR_ARG (null pointers, sizes, a full group capacity),
 * HSQ_ERR_UNSUPPORTED (d, group_n, dtype, B*Hkv*capacity >= 2^32),
 * HSQ_ERR_HIP.  Calls on one cache must be ordered on one stream.
 */
int hsq_cache_append(const void* k_new, const void* v_new, int dtype, int B, int Hkv, int d,
                     int group_n, int n_fix, int n_recent, int64_t t, int n_pending,
                     int n_groups, int l1_cap, int ng_cap, const uint32_t* k_signs,
                     const uint32_t* v_signs, const float* thr4, const float* thr3,
                     uint8_t* l1k, float* l1k_n, uint8_t* l1v, float* l1v_n, void* raw_k,
                     void* raw_v, uint8_t* l2k, float* l2k_n, uint8_t* l2v, float* l2v_n,
                     uint8_t* l3, void* stream);

/*
 * hsq_cache_decode_step -- hsq_decode_step over a cache laid out with
 * capacities: unit u's L1 rows start at row u * l1_cap and its groups at
 * group u * ng_cap; n_l1 rows and n_groups groups of each unit are used.
 * Archive in device memory (one launch, or two through the workspace as
 * hsq_decode_step).  Workspace sized by hsq_workspace_bytes with the counts.
 * Errors as hsq_decode_step, and HSQ_ERR_ARG for capacities below the counts.
 */
int hsq_cache_decode_step(const float* q, int B, int Hq, int Hkv, int d, const uint8_t* l1k,
                          const float* l1k_n, const uint8_t* l1v, const float* l1v_n, int n_l1,
                          int l1_cap, const uint8_t* l2k, const float* l2k_n,
                          const uint8_t* l2v, const float* l2v_n, int n_groups, int ng_cap,
                          const uint8_t* l3, int group_n, int beta, int agg,
                          const uint32_t* k_signs, const uint32_t* v_signs, const float* cb4,
                          const float* cb3, float scale, float summary_bias, int32_t* topk_idx,
                          void* workspace, size_t ws_bytes, float* out, void* stream);

/* ---------------------------------------------------- TQ-QKV key path --- */

/*
 * hsq_encode_qjl -- TurboQuant key codes plus a 1-bit QJL sketch of the key's
 * residual [ABL "Experimental setup": an optional 1-bit Johnson-Lindenstrauss
 * residual sketch on the K or V path; "Key contributions" 1: TQ-QKV adds it on
 * the key path].  Estimator: the published QJL one (Zandieh, Daliri and Han,
 * 2024).  For each row: codes and norm exactly as hsq_encode (rotation on,
 * one mask for all rows); u = y - c[code], the TurboQuant error in the rotated
 * unit domain (y = R x / r); sketch bit j set when (S u)_j < 0 (LSB-first, bit
 * j in byte j / 8, d bits per row); gamma = r * ||u||_2.
 *   x           [n_vec][d] in x_dtype (HSQ_F32 or HSQ_BF16)
 *   bits        3 or 4;  signs uint32 [d/32];  thresholds fp32 [2^bits - 1]
 *   centroids   fp32 [2^bits] (the thresholds' codebook)
 *   S           fp32 [d][d], row j the j-th sketch direction (i.i.d. N(0,1)
 *               data, one per (layer, kv-head))
 *   codes       out [n_vec][bits*d/8];  norms out fp32 [n_vec]
 *   sketch      out [n_vec][d/8];  gamma out fp32 [n_vec]
 * Errors: HSQ_ERR_ARG (null pointers, n_vec < 0), HSQ_ERR_UNSUPPORTED (d,
 * bits, dtype), HSQ_ERR_HIP.  n_vec == 0 is a no-op.
 */
int hsq_encode_qjl(const void* x, int x_dtype, int64_t n_vec, int d, int bits,
                   const uint32_t* signs, const float* thresholds, const float* centroids,
                   const float* S, uint8_t* codes, float* norms, uint8_t* sketch, float* gamma,
                   void* stream);

/*
 * hsq_build_sketches -- the QJL sketches and gammas of a layer's 4-bit token
 * keys, for hsq_decode_step_qjl [ABL "Key contributions" 1: TQ-QKV adds the
 * sketch on the key path].  Each key is encoded as hsq_encode_qjl encodes it
 * (4 bits, its kv-head's signs and S), read straight from k at the tier
 * plan's rows; the codes themselves are hsq_build_tiers' and are not
 * written again.
 *   k           [B][Hkv][T][d] in dtype (HSQ_F32 or HSQ_BF16)
 *   l1_pos      int32 [B][n1], group_pos int32 [B][n_groups*group_n]
 *               (device; the rows hsq_build_tiers was given)
 *   k_signs     uint32 [Hkv][d/32];  thr4, cb4  4-bit codebook (device)
 *   S           fp32 [Hkv][d][d]
 *   outputs     l1_sketch [B][Hkv][n1][d/8], l1_gamma [B][Hkv][n1],
 *               l3_sketch [B][Hkv][n_groups][group_n][d/8],
 *               l3_gamma [B][Hkv][n_groups][group_n]
 * Two launches per kv-head.  n1 == 0 or n_groups == 0 skip that tier.
 * The sketch arrays are written 2 bytes at a time (2-byte aligned).
 * Errors: HSQ_ERR_ARG (null pointers, bad sizes, n1 + n_groups*group_n > T,
 * misaligned sketch arrays),
 * HSQ_ERR_UNSUPPORTED (d, dtype, B*Hkv*T >= 2^32), HSQ_ERR_HIP.
 */
int hsq_build_sketches(const void* k, int dtype, int B, int Hkv, int T, int d,
                       const int32_t* l1_pos, int n1, const int32_t* group_pos, int n_groups,
                       int group_n, const uint32_t* k_signs, const float* thr4, const float* cb4,
                       const float* S, uint8_t* l1_sketch, float* l1_gamma, uint8_t* l3_sketch,
                       float* l3_gamma, void* stream);

/*
 * hsq_qjl_logits -- TQ-QKV logits of n_q query rows against n_keys keys
 * encoded by hsq_encode_qjl (same signs, centroids and S):
 *   out[h][k] = scale * (r_k <R q_h, c[code_k]> +
 *               sqrt(pi/2) / d * gamma_k * sum_j (S R q_h)_j (1 - 2 bit_kj))
 * i.e. the TurboQuant logit plus the unbiased QJL estimate of the residual's
 * share [ABL "Key contributions" 2: this correction is zero-mean but its
 * variance inflates softmax weights by about exp(sigma^2 / 2)].
 *   q    fp32 [n_q][d], 1 <= n_q <= 8;  out fp32 [n_q][n_keys]
 * Errors: HSQ_ERR_ARG, HSQ_ERR_UNSUPPORTED (d, bits), HSQ_ERR_HIP.
 */
int hsq_qjl_logits(const float* q, int n_q, int d, int bits, const uint8_t* codes,
                   const float* norms, const uint8_t* sketch, const float* gamma, int64_t n_keys,
                   const uint32_t* signs, const float* centroids, const float* S, float scale,
                   float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HSQ_H */
