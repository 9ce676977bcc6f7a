/*
 * joint_attn -- joint multi-stream attention for AMD Instinct MI355X (gfx950).
 *
 * The operation.  In FLUX 3 Image Klein's diffusion transformer the text tokens, the
 * noisy target-image tokens and zero or more reference-image tokens are kept in
 * separate streams and meet only in one joint self-attention over their concatenation
 * (VisualGen FLUX 3 article, everytik.com translation, section
 * 使用 TensorRT LLM VisualGen 进行 FLUX 3 推理; several reference images may be passed,
 * section 离线推理).  The article's section 量化注意力与稀疏注意力 names that attention as
 * the main cost at 2048x2048 and offers bf16 and fp8 (qk_dtype / v_dtype) variants.
 * This library computes it as unmasked scaled-dot-product attention,
 *     O = softmax(Q K^T * softmax_scale) V        (per batch b and head h),
 * in four calls: pack the streams, then either the bf16 forward, or the fp8 quantiser
 * followed by the fp8 forward; joint_attn_fwd_bf16_streams (and its split-KV form) does
 * pack and bf16 forward in one call, reading the streams in place.
 *
 * Conventions for every call.
 *   - Tensor pointers are DEVICE pointers (HBM) owned by the caller; the library never
 *     allocates, frees or keeps them.  "Host" marks the few host pointers.  bf16 and
 *     e4m3 tensors must be 16-byte aligned, fp32 and int32 arrays 4-byte aligned
 *     (JA_EUNSUPPORTED otherwise).
 *   - Each call validates its arguments first; on any error nothing is launched and
 *     nothing is written.  Otherwise it enqueues its kernels on `stream` (a hipStream_t
 *     passed as void*; NULL = the default stream) and returns without synchronising.
 *   - Return value: JA_OK (0) or an error code below; joint_attn_strerror() names it.
 *     No C++ exception crosses this interface and the library never aborts.
 *   - Calls keep no state between them and may be issued from several host threads.
 *   - bf16 is IEEE binary32's top 16 bits; e4m3 is the OCP FP8 E4M3 format (bias 7,
 *     3 mantissa bits, max finite 448, no infinities).
 *   - Layouts (all dense, row-major, innermost last):
 *       BNHD  [B][N][H][D]   token-major, what a per-stream projection produces
 *       BHND  [B][H][N][D]   head-major, packed Q and K
 *       BHDN  [B][H][D][ld]  channel-major with row pitch ld >= N, ld % 16 == 0, used for
 *                            V (columns N..ld-1 are padding that pack writes as zero)
 *   - Supported head sizes D: 64 and 128.  N may be any positive length (no multiple
 *     required); N == 0 is accepted and does nothing.  The longest sequence is set by
 *     one head's BHDN V tensor, D * ld <= JA_MAX_HEAD_ELEMS elements (N <= 8,388,608 at
 *     D = 128, 16,777,216 at D = 64), which keeps every in-kernel offset inside that
 *     tensor in 32 bits; longer sequences return JA_EINVAL.
 */
#ifndef JOINT_ATTN_H
#define JOINT_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define JA_OK 0
#define JA_EINVAL 1        /* NULL pointer, non-positive size, inconsistent sizes, overflow */
#define JA_EUNSUPPORTED 2  /* head size not 64/128, misaligned pointer, too many streams */
#define JA_EHIP 3          /* the HIP runtime refused a launch; see joint_attn_last_hip_error */
#define JA_ESCRATCH 4      /* more scratch than JA_SCRATCH_BYTES (joint_attn_fwd_bf16_splitkv_noalloc) */

#define JA_LAYOUT_BHND 0
#define JA_LAYOUT_BHDN 1

#define JA_MAX_STREAMS 16   /* text + target + up to 14 reference images */
#define JA_MAX_HEAD_ELEMS (1 << 30)   /* D * ld of one (b, h) of a BHDN tensor, at most */
#define JA_QK_BLOCK 128     /* tokens per fp8 scale block of Q and K */
#define JA_HI_CHANNELS 16   /* Q/K channels per (b, h) kept out of e4m3 in fp8 mode 1 */

#define JA_SPARSE_BLOCK 128       /* query rows and keys per block of the sparse mask */
#define JA_SPARSE_MAX_N 131072    /* longest sequence of joint_attn_fwd_bf16_sparse */
#define JA_SPARSE_PLAN_MAX 2097152 /* B * H * ceil(N / JA_SPARSE_BLOCK) limit of a sparse plan */

#define JA_FP8_PLAIN 0      /* fp8 mode 0: every Q/K channel in e4m3 */
#define JA_FP8_SPLIT 1      /* fp8 mode 1: JA_HI_CHANNELS outlier channels in bf16 */
#define JA_FP8_REPAIR 2     /* fp8 token repair: the *_repair entry points below */

#define JA_REPAIR_MAX_N 131072    /* longest sequence of joint_attn_fwd_fp8_repair */
#define JA_REPAIR_TILE 64         /* v8t_sel row pitch: n_repair rounded up to this */

#define JA_SCRATCH_BYTES (64 << 20)  /* static scratch of joint_attn_fwd_bf16_splitkv_noalloc, per device */

/* Human-readable name of a status code (static string). */
const char *joint_attn_strerror(int status);

/* hipError_t of the last failed launch on the calling thread (0 if none). */
int joint_attn_last_hip_error(void);

/* Smallest legal BHDN pitch for N tokens: N rounded up to a multiple of 16. */
int64_t joint_attn_vt_ld(int64_t N);

/*
 * joint_attn_pack -- concatenate token streams along the token axis (the joint
 * sequence of the VisualGen FLUX 3 article's joint attention; stream order text,
 * noisy target, then reference images in the order they were given).
 *
 *   n_streams  1..JA_MAX_STREAMS
 *   src        host array of n_streams device pointers; stream s is bf16 BNHD
 *              [B][lens[s]][H][D] (a zero-length stream may pass NULL)
 *   lens       host array of n_streams token counts (>= 0)
 *   layout     JA_LAYOUT_BHND: dst is bf16 [B][H][N][D] (use for Q and K)
 *              JA_LAYOUT_BHDN: dst is bf16 [B][H][D][ld] (use for V); padding zeroed
 *   ld         row pitch for BHDN (ignored for BHND)
 *   offsets    host output, n_streams + 1 entries: offsets[0] = 0,
 *              offsets[s + 1] = offsets[s] + lens[s]; N = offsets[n_streams].
 *              Written even when N == 0.
 * Every element is copied bit for bit.  Source and destination must not overlap.
 * Pointers must be 16-byte aligned.
 */
int joint_attn_pack(int n_streams, const void *const *src, const int64_t *lens,
                    int B, int H, int D, int layout, int64_t ld,
                    void *dst, int64_t *offsets, void *stream);

/*
 * joint_attn_fwd_bf16 -- O = softmax(Q K^T * softmax_scale) V over all N packed
 * tokens, per (b, h), bf16 operands with fp32 accumulation and an online softmax.
 *
 *   q, k           bf16 BHND [B][H][N][D]
 *   vt             bf16 BHDN [B][H][D][ldv] (only columns < N are read)
 *   softmax_scale  usually 1/sqrt(D); must be finite and > 0
 *   o              bf16 BNHD [B][N][H][D] (stream s's output is rows
 *                  offsets[s] .. offsets[s+1]-1 of every batch)
 *   lse            fp32 [B][H][N], natural-log log-sum-exp of each query row's logits,
 *                  or NULL
 * Results are deterministic (fixed reduction order, no atomics).
 */
int joint_attn_fwd_bf16(const void *q, const void *k, const void *vt,
                        int B, int H, int64_t N, int D, int64_t ldv, float softmax_scale,
                        void *o, float *lse, void *stream);

/*
 * joint_attn_fwd_bf16_sparse -- block-sparse variant of joint_attn_fwd_bf16: the sparse
 * attention option of the VisualGen FLUX 3 article (section 量化注意力与稀疏注意力), which
 * runs on a general block-sparse attention kernel; the rule that picks the blocks is not
 * part of this library, the mask is an input.  Query row i of (b, h) attends key j only if
 *     block_mask[b][h][i / JA_SPARSE_BLOCK][j / JA_SPARSE_BLOCK] != 0;
 * a row that attends no key gets O = 0 and lse = -inf.  Each 128-row query block visits
 * only the key blocks its mask row allows (the work saved scales with the zero blocks).
 *
 *   q, k, vt, o, lse  as for joint_attn_fwd_bf16
 *   block_mask        device uint8 [B][H][nb][nb], nb = ceil(N / JA_SPARSE_BLOCK)
 *   N                 at most JA_SPARSE_MAX_N
 */
int joint_attn_fwd_bf16_sparse(const void *q, const void *k, const void *vt,
                               int B, int H, int64_t N, int D, int64_t ldv,
                               const uint8_t *block_mask, float softmax_scale,
                               void *o, float *lse, void *stream);

/*
 * joint_attn_sparse_plan -- the order in which joint_attn_fwd_bf16_sparse_planned starts
 * the workgroups of a block mask (one per 128-row query block; the operation is that of
 * joint_attn_fwd_bf16_sparse, which this only schedules).  The workgroups are dealt to
 * the GPU's eight XCDs in eight contiguous shares; within each share the query blocks
 * whose mask row allows more than twice the share's mean number of key blocks (in a
 * joint sequence, the text rows, which see every block) are moved to the front, the
 * others keep their order.  Long workgroups then start first instead of trailing the
 * share, while consecutive short ones still share one (b, h)'s keys in L2.
 *
 *   block_mask   device uint8 [B][H][nb][nb] as for joint_attn_fwd_bf16_sparse
 *   plan         device int32 buffer of at least joint_attn_sparse_plan_bytes() bytes,
 *                owned by the caller, 4-byte aligned; receives a permutation of
 *                0 .. B*H*nb - 1 (entry p = the query block, b*H*nb + h*nb + i, that
 *                workgroup position p runs).  Its contents on entry do not matter.
 *   B*H*nb       at most JA_SPARSE_PLAN_MAX (JA_EUNSUPPORTED otherwise); N at most
 *                JA_SPARSE_MAX_N
 * Two kernels on `stream`; a plan stays valid for as long as the mask and B, H, N do not
 * change, so one plan can serve every forward over that mask.
 */
int64_t joint_attn_sparse_plan_bytes(int B, int H, int64_t N);
int joint_attn_sparse_plan(const uint8_t *block_mask, int B, int H, int64_t N,
                           int32_t *plan, int64_t plan_bytes, void *stream);

/*
 * joint_attn_fwd_bf16_sparse_planned -- joint_attn_fwd_bf16_sparse with its workgroups
 * started in the order of a plan from joint_attn_sparse_plan for the same block_mask,
 * B, H and N.  Same arguments, plus:
 *   plan         device int32 [B*H*nb], read only.  Each workgroup computes its query
 *                block exactly as the unplanned call does, so the results are bit for bit
 *                those of joint_attn_fwd_bf16_sparse.  A buffer that is not such a
 *                permutation is not detected: entries are clamped to the valid range, so
 *                reads and writes stay inside the tensors, but rows of query blocks it
 *                omits are left unwritten.
 */
int joint_attn_fwd_bf16_sparse_planned(const void *q, const void *k, const void *vt,
                                       int B, int H, int64_t N, int D, int64_t ldv,
                                       const uint8_t *block_mask, const int32_t *plan,
                                       float softmax_scale, void *o, float *lse, void *stream);

/*
 * joint_attn_fwd_bf16_splitkv -- joint_attn_fwd_bf16 with the query tiles of the last,
 * partial round of workgroups split into n_split key ranges (one workgroup per (tile,
 * range)), so that the CUs left idle by that round get work: a grid of B*H*ceil(N/256)
 * workgroups (128-row tiles at D = 64) rarely fills whole rounds (2048x2048 T2I: 3168
 * tiles for 256 CUs; a 1024x1024 image; one GPU's share of a head split).  The tiles
 * that fill whole rounds run over all keys.  The split tiles' partial results are
 * merged with the log-sum-exp rule: for key sets S_1 .. S_n,
 *     O = sum_s exp(lse_s - lse) O_s,   lse = ln sum_s exp(lse_s).
 * Same operation, layouts and arguments as joint_attn_fwd_bf16, plus:
 *   n_split          1 .. 64 (clamped to the number of 32-key tiles; 1, or a grid of
 *                    whole rounds, is the plain forward);
 *                    joint_attn_fwd_bf16_splitkv_suggest() gives one from a model of
 *                    the rounds saved against the partial results' cost (1 = none)
 *   workspace        device scratch owned by the caller, 16-byte aligned, at least
 *                    joint_attn_fwd_bf16_splitkv_workspace() bytes, asked on the device
 *                    the call runs on (fp32 partial outputs and log-sum-exps of at most
 *                    one round of split tiles); its contents on entry do not matter
 * Results are deterministic but, in the split tiles, not bit-identical to
 * joint_attn_fwd_bf16 (the sums are split differently).  Calls that share a workspace
 * must not overlap.
 */
int64_t joint_attn_fwd_bf16_splitkv_workspace(int B, int H, int64_t N, int D, int n_split);
int joint_attn_fwd_bf16_splitkv_suggest(int B, int H, int64_t N, int D);
int joint_attn_fwd_bf16_splitkv(const void *q, const void *k, const void *vt,
                                int B, int H, int64_t N, int D, int64_t ldv,
                                float softmax_scale, int n_split,
                                void *workspace, int64_t workspace_bytes,
                                void *o, float *lse, void *stream);

/*
 * joint_attn_fwd_bf16_splitkv_noalloc -- joint_attn_fwd_bf16_splitkv without a workspace
 * argument and without any allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The partial results go to a static scratch array of JA_SCRATCH_BYTES inside the
 * library instead: each GPU the library runs on holds one (until the process ends),
 * looked up on the first call on that GPU.  Same operation, layouts, arguments, results
 * (bit for bit) and errors as joint_attn_fwd_bf16_splitkv, plus:
 *   JA_ESCRATCH  the split tiles' partials do not fit: tail * min(n_split, ceil(N/32))
 *                * rows * (D + 1) * 4 bytes > JA_SCRATCH_BYTES, where tail = the query
 *                tiles of the last, partial round (B*H*ceil(N/rows) modulo the
 *                workgroups resident at once, rows = 256 at D = 128, 128 at D = 64).
 *                2048x2048 T2I at the suggested split (5) needs 63.4 MB.  Nothing is
 *                launched; the workspace variant takes any size.
 * Every call on one GPU shares that GPU's scratch array: calls that overlap on one GPU
 * (on different streams, or from several host threads) race and must not be issued;
 * calls ordered on one stream are safe.  No state needs clearing between calls (every
 * partial a call reads was written by that call).
 */
int joint_attn_fwd_bf16_splitkv_noalloc(const void *q, const void *k, const void *vt,
                                        int B, int H, int64_t N, int D, int64_t ldv,
                                        float softmax_scale, int n_split,
                                        void *o, float *lse, void *stream);

/*
 * joint_attn_fwd_bf16_streams -- the same attention as joint_attn_fwd_bf16, reading Q, K
 * and V in place from the per-stream tensors instead of packed copies: the joint
 * sequence of the VisualGen FLUX 3 article (everytik.com translation, section
 * 使用 TensorRT LLM VisualGen 进行 FLUX 3 推理: text, noisy target and reference streams
 * processed apart and joined only in attention) is formed by the kernel's own loads, so
 * no pack step is needed.  Results are bit-identical to joint_attn_pack (x3) followed
 * by joint_attn_fwd_bf16 on the same streams.
 *
 *   n_streams   1..JA_MAX_STREAMS, in joint-sequence order (text, target, references)
 *   q, k, v     host arrays of n_streams device pointers; stream s is bf16 BNHD
 *               [B][lens[s]][H][D] (a zero-length stream may pass NULL); 16-byte aligned
 *   lens        host array of n_streams token counts (>= 0); N = sum of lens
 *   o           bf16 BNHD [B][N][H][D] (stream s's output is rows offsets[s] ..
 *               offsets[s+1]-1 of every batch)
 *   lse         fp32 [B][H][N] natural-log log-sum-exp per query row, or NULL
 *   offsets     host output, n_streams + 1 entries as in joint_attn_pack, or NULL;
 *               written whenever the arguments are valid, also for N == 0
 */
int joint_attn_fwd_bf16_streams(int n_streams, const void *const *q, const void *const *k,
                                const void *const *v, const int64_t *lens,
                                int B, int H, int D, float softmax_scale,
                                void *o, float *lse, int64_t *offsets, void *stream);

/*
 * joint_attn_fwd_bf16_streams_splitkv -- joint_attn_fwd_bf16_streams with the query tiles
 * of the last, partial round split into key ranges and merged, as joint_attn_fwd_bf16_splitkv
 * does for packed operands (the log-sum-exp merge of the split-KV comment above).  Q and K
 * are always read in place from the streams (the joint sequence of the VisualGen FLUX 3
 * article, everytik.com translation, section 使用 TensorRT LLM VisualGen 进行 FLUX 3 推理).
 *   n_streams .. offsets   as for joint_attn_fwd_bf16_streams
 *   n_split           as for joint_attn_fwd_bf16_splitkv (the same suggestion applies)
 *   pack_v            0: V is read in place too and transposed in LDS (no copy of V);
 *                     1: V is first transposed into the workspace (BHDN, pitch
 *                     joint_attn_vt_ld(N)) by the pack kernel, and the forward loads
 *                     its V^T tiles from there (faster forward, B*H*D*ld*2 more bytes)
 *   workspace         device scratch owned by the caller, 16-byte aligned, at least
 *                     joint_attn_fwd_bf16_streams_splitkv_workspace() bytes (asked on the
 *                     device the call runs on): the V^T copy (pack_v = 1), then the split
 *                     tiles' fp32 partials; its contents on entry do not matter
 * Results are bit-identical to joint_attn_pack (x3) followed by joint_attn_fwd_bf16_splitkv
 * with the same n_split, for either pack_v.  Errors as joint_attn_fwd_bf16_streams and
 * joint_attn_fwd_bf16_splitkv (JA_EINVAL also for pack_v not 0 or 1).  Calls that share a
 * workspace must not overlap.
 */
int64_t joint_attn_fwd_bf16_streams_splitkv_workspace(int B, int H, int64_t N, int D,
                                                      int n_split, int pack_v);
int joint_attn_fwd_bf16_streams_splitkv(int n_streams, const void *const *q,
                                        const void *const *k, const void *const *v,
                                        const int64_t *lens, int B, int H, int D,
                                        float softmax_scale, int n_split, int pack_v,
                                        void *workspace, int64_t workspace_bytes,
                                        void *o, float *lse, int64_t *offsets,
                                        void *stream);

/*
 * joint_attn_quant_fp8 -- quantise packed bf16 Q, K, V to e4m3 with dequantisation
 * scales (x ~= decode(code) * scale).  The article's fp8 attention setting
 * (section 量化注意力与稀疏注意力) fixes only that Q, K and V are fp8; the scaling
 * granularity follows the block-wise-scale advice of the kongchang.com English page
 * (section "Reducing Numerical Precision"):
 *   Q, K: one scale per (b, h, block of JA_QK_BLOCK consecutive packed tokens; the last
 *         block may be shorter);
 *   V:    one scale per (b, h, channel) over all N tokens;
 *   every scale is a power of two, as in the OCP Microscaling formats: the smallest
 *   s = 2^k (k >= -126) with amax <= 448 s (s = 1 when amax == 0), so x / s is exact and
 *   code = e4m3(x / s), rounded to nearest even; the sign of a zero result is kept.
 *   Inputs must be finite.
 *
 *   mode JA_FP8_PLAIN (0): the above.
 *   mode JA_FP8_SPLIT (1): additionally, per (b, h), the JA_HI_CHANNELS channels with the
 *     largest amax|q_c| * amax|k_c| over all tokens (ties to the lower index) are kept
 *     out of e4m3 -- the article's VC-Attention remark (same section) gives the part of
 *     the input with the largest quantisation error a residual correction; activation
 *     outliers sit in whole channels.  Their codes are written as 0 and their exact
 *     values divided by the block scale go to q_hi / k_hi.
 *
 *   q, k       bf16 BHND [B][H][N][D]      -> q8, k8   e4m3 BHND [B][H][N][D]
 *   vt         bf16 BHDN [B][H][D][ldv]    -> v8t      e4m3 BHDN [B][H][D][ldv],
 *                                                     padding columns written as 0
 *   q_scale, k_scale  fp32 [B][H][ceil(N / JA_QK_BLOCK)]
 *   v_scale           fp32 [B][H][D]
 *   mode 1 only (ignored, may be NULL, in mode 0):
 *   q_hi, k_hi  bf16 [B][H][N][JA_HI_CHANNELS]  kept channels / block scale
 *   hi_idx      int32 [B][H][JA_HI_CHANNELS]    kept channel indices, ascending
 *   ch_amax     fp32 [B][H][2][D]               per-channel amax of Q (0) and K (1)
 * Codes, scales, q_hi/k_hi and hi_idx are bit-exact functions of the inputs.
 */
int joint_attn_quant_fp8(const void *q, const void *k, const void *vt,
                         int B, int H, int64_t N, int D, int64_t ldv, int mode,
                         void *q8, void *k8, void *v8t,
                         float *q_scale, float *k_scale, float *v_scale,
                         void *q_hi, void *k_hi, int32_t *hi_idx, float *ch_amax,
                         void *stream);

/*
 * joint_attn_quant_fp8_streams -- joint_attn_quant_fp8 reading Q, K and V in place from
 * the per-stream tensors (laid out and passed as for joint_attn_fwd_bf16_streams), so the
 * fp8 path needs no bf16 pack step either.  The outputs (packed e4m3 codes, V^T codes with
 * pitch ldv, scales, and in mode 1 the kept channels) are bit-identical to those of
 * joint_attn_pack followed by joint_attn_quant_fp8 on the same streams.  `offsets` (host,
 * n_streams + 1 entries, or NULL) receives the stream offsets as in joint_attn_pack.
 */
int joint_attn_quant_fp8_streams(int n_streams, const void *const *q, const void *const *k,
                                 const void *const *v, const int64_t *lens,
                                 int B, int H, int D, int64_t ldv, int mode,
                                 void *q8, void *k8, void *v8t,
                                 float *q_scale, float *k_scale, float *v_scale,
                                 void *q_hi, void *k_hi, int32_t *hi_idx, float *ch_amax,
                                 int64_t *offsets, void *stream);

/*
 * joint_attn_fwd_fp8 -- attention on the e4m3 operands of joint_attn_quant_fp8.
 *   QK^T on fp8 matrix cores with fp32 accumulation (mode 1 adds the kept channels on a
 *   bf16 MFMA into the same accumulator); per-block Q/K scales and softmax_scale are
 *   folded into the base-2 exponent; the softmax numerators, taken relative to an
 *   integer row maximum M (base 2) and multiplied by 2^8, are rounded to e4m3 for the
 *   fp8 P.V product; the row sum uses the unrounded numerators; the per-channel V scale
 *   is applied in the epilogue:
 *     t_j = (q8_i . k8_j + q_hi_i . k_hi_j) * qs * ks * softmax_scale * log2(e),
 *     p_j = 2^(t_j - M),  O[c] = vs[c] * sum_j e4m3(2^8 p_j) v8_j[c] / (2^8 sum_j p_j).
 *   The fp8 matrix cores sum each group of 8 products at reduced precision (relative to
 *   the group's largest product), so on inputs with large-magnitude channels mode 0
 *   differs from exact fp8 arithmetic by up to ~2e-2 (relative Frobenius).
 *
 *   q8, k8            e4m3 BHND [B][H][N][D]
 *   v8t               e4m3 BHDN [B][H][D][ldv]
 *   q_scale, k_scale  fp32 [B][H][ceil(N / JA_QK_BLOCK)];  v_scale fp32 [B][H][D]
 *   mode              JA_FP8_PLAIN or JA_FP8_SPLIT (then q_hi, k_hi as written by the
 *                     quantiser; NULL in mode 0)
 *   o                 bf16 BNHD [B][N][H][D];  lse fp32 [B][H][N] or NULL
 */
int joint_attn_fwd_fp8(const void *q8, const void *k8, const void *v8t,
                       const float *q_scale, const float *k_scale, const float *v_scale,
                       int B, int H, int64_t N, int D, int64_t ldv, float softmax_scale,
                       int mode, const void *q_hi, const void *k_hi,
                       void *o, float *lse, void *stream);

/*
 * joint_attn_fwd_fp8_splitkv -- joint_attn_fwd_fp8 (either mode) with the query tiles of
 * the last, partial round of workgroups split into n_split ranges of 64-key tiles, merged
 * with the log-sum-exp rule, as joint_attn_fwd_bf16_splitkv does for the bf16 forward
 * (same motivation: 2048x2048 T2I has 3168 workgroups for 256 CUs).  Same operation,
 * layouts and arguments as joint_attn_fwd_fp8, plus:
 *   n_split          1 .. 64 (clamped to the number of 64-key tiles; 1, or a grid of
 *                    whole rounds, is the plain forward);
 *                    joint_attn_fwd_fp8_splitkv_suggest() gives one for the mode
 *   workspace        device scratch owned by the caller, 16-byte aligned, at least
 *                    joint_attn_fwd_fp8_splitkv_workspace() bytes, asked on the device
 *                    the call runs on; its contents on entry do not matter
 * The split tiles' partial outputs carry the V scale; results are deterministic, not
 * bit-identical to joint_attn_fwd_fp8 in the split tiles.  Calls that share a workspace
 * must not overlap.
 */
int64_t joint_attn_fwd_fp8_splitkv_workspace(int B, int H, int64_t N, int D, int n_split);
int joint_attn_fwd_fp8_splitkv_suggest(int B, int H, int64_t N, int D, int mode);
int joint_attn_fwd_fp8_splitkv(const void *q8, const void *k8, const void *v8t,
                               const float *q_scale, const float *k_scale, const float *v_scale,
                               int B, int H, int64_t N, int D, int64_t ldv, float softmax_scale,
                               int mode, const void *q_hi, const void *k_hi, int n_split,
                               void *workspace, int64_t workspace_bytes,
                               void *o, float *lse, void *stream);

/*
 * Token repair of fp8 attention: the repair budget rho of VC-Attention FP8 (VisualGen
 * FLUX 3 article, everytik.com translation, section 量化注意力与稀疏注意力: the share
 * rho of tokens with the highest quantisation error gets a residual correction).  Per
 * (b, h), separately for Q and K, n = ceil(rho N) tokens are repaired: those with the
 * largest max_c |x_c - decode(code_c) * scale| (exact in fp32; ties to the lower token
 * index).  Their residual is added back, i.e. they enter Q K^T with their exact bf16
 * values; P and V are as in mode JA_FP8_PLAIN.
 *
 * joint_attn_repair_count -- n = ceil(rho * N) evaluated in double, for N >= 0 and
 *   0 <= rho <= 1; -1 otherwise.
 */
int64_t joint_attn_repair_count(int64_t N, double rho);

/*
 * joint_attn_quant_fp8_repair -- the JA_FP8_PLAIN quantisation of joint_attn_quant_fp8
 * (same codes and scales, same layouts), plus the repair selection.
 *   n_repair          0 <= n_repair <= N (normally joint_attn_repair_count(N, rho))
 *   q_err, k_err      fp32 [B][H][N] out: each token's largest absolute residual
 *   q_sel, k_sel      int32 [B][H][n_repair] out: the repaired tokens, ascending
 *   v8t_sel           e4m3 [B][H][D][ldr] out, ldr = n_repair rounded up to
 *                     JA_REPAIR_TILE: the V^T codes of the repaired keys (columns k_sel
 *                     of v8t), zero padded, for the forward's key correction
 *                     (q_sel, k_sel, v8t_sel may be NULL when n_repair == 0)
 * Errors: JA_EINVAL for a NULL output or n_repair outside [0, N]; otherwise as
 * joint_attn_quant_fp8.
 */
int joint_attn_quant_fp8_repair(const void *q, const void *k, const void *vt, int B, int H,
                                int64_t N, int D, int64_t ldv, int64_t n_repair,
                                void *q8, void *k8, void *v8t,
                                float *q_scale, float *k_scale, float *v_scale,
                                float *q_err, float *k_err, int32_t *q_sel, int32_t *k_sel,
                                void *v8t_sel, void *stream);

/*
 * joint_attn_fwd_fp8_repair -- joint_attn_fwd_fp8 (mode JA_FP8_PLAIN) with the listed
 * tokens repaired:
 *     t_ij = q~_i . k~_j * softmax_scale * log2(e),  q~ = q for listed queries, else
 *     decode(q8) * qs (likewise k~), P and O as in joint_attn_fwd_fp8.
 * Two launches on `stream`, in this order: the plain forward on the codes (writing O
 * and lse) with, appended to its grid, a recomputation of the listed query rows from
 * their exact values; then a correction of every other row that replaces each listed
 * key's code term by its exact-value term (rebuilding the row's state from O and lse).
 *   q8 ... v_scale    as written by joint_attn_quant_fp8_repair
 *   q, k              bf16 BHND [B][H][N][D]: the unquantised inputs of the quantiser
 *   q_sel, k_sel, v8t_sel   as written by joint_attn_quant_fp8_repair with the same
 *                     n_repair: ascending distinct token indices in [0, N).  The kernels
 *                     clamp every entry they load into [0, N) (a negative key entry is
 *                     skipped), so lists of other contents give wrong results in O and
 *                     lse but no access outside the arguments' extents.
 *   N                 at most JA_REPAIR_MAX_N
 *   o                 bf16 BNHD [B][N][H][D];  lse fp32 [B][H][N], required (the key
 *                     correction reads and rewrites it)
 * Errors: as joint_attn_fwd_fp8, plus JA_EINVAL for NULL q / k / lse / lists or n_repair
 * outside [0, N], JA_EUNSUPPORTED for N > JA_REPAIR_MAX_N.
 */
int joint_attn_fwd_fp8_repair(const void *q8, const void *k8, const void *v8t,
                              const float *q_scale, const float *k_scale, const float *v_scale,
                              const void *q, const void *k, const int32_t *q_sel,
                              const int32_t *k_sel, const void *v8t_sel, int64_t n_repair,
                              int B, int H, int64_t N, int D, int64_t ldv, float softmax_scale,
                              void *o, float *lse, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* JOINT_ATTN_H */
