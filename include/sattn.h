/*
 * sattn.h - C ABI of the fine-grained (Mx1-slice / column-sparse) self-attention library
 * for AMD Instinct MI355X (gfx950).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are dense, row-major and head-major: Q is [B,H,Nq,D], K and V are [B,H,Nk,D],
 *    bf16 (IEEE bfloat16 bit patterns, 2 bytes each).  One K or V row is D*2 bytes.
 *  - Every data pointer is a DEVICE pointer owned by the caller.  The library never allocates,
 *    frees or keeps device memory; it only launches kernels on `stream` (a hipStream_t; NULL is
 *    the default stream) and never synchronises.  Calls are asynchronous: device-side results
 *    are ready when the stream reaches them.
 *  - D must be 64 or 128.  Queries are split into G = ceil(Nq / group) groups of `group`
 *    contiguous tokens; the last group may be partial.  group is a multiple of 16 in [16, 256].
 *  - scale multiplies q.k before the softmax; pass 1/sqrt(D) for standard attention.
 *  - Return value: SATTN_OK (0) or a sattn_status code.  Arguments are validated on the host
 *    before any HIP call; on a validation error nothing is launched and no output is touched.
 *    A failed launch returns SATTN_ERR_HIP.  Faults inside a kernel surface at the caller's
 *    next synchronisation.  sattn_last_error() returns a thread-local detail string.
 *  - Thread safety: every entry point may be called from several host threads at once.  In
 *    validation mode (SATTN_VALIDATE=1) the device check of the index lists is serialised across
 *    threads (one check word per device); calls that validate wait for each other.
 *  - Environment: SATTN_VALIDATE=1 checks index lists on the device before sattn_forward,
 *    sattn_forward_split, sattn_delta_forward, sattn_fp8_forward and sattn_fp4_forward; SATTN_LOG=1
 *    prints one line per launch decision (entry point, sizes, kernel variant, workgroups) to stderr;
 *    SATTN_SERIAL_GATHER=1 runs sattn_forward, sattn_forward_split, sattn_delta_forward and
 *    attn_forward at pipeline depth 1 (every key block's
 *    gather completes before the block before it computes), a slower order whose results must equal
 *    the default double-buffered ones bit for bit (a check for races in the buffering).
 */
#ifndef SATTN_H
#define SATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SATTN_OK = 0,
  SATTN_ERR_NULL = 1,         /* a required pointer is NULL */
  SATTN_ERR_SHAPE = 2,        /* a size is < 1, or sizes overflow the supported index range */
  SATTN_ERR_UNSUPPORTED = 3,  /* D not in {64,128}; group not a multiple of 16 in [16,256]; Nk too large */
  SATTN_ERR_ARG = 4,          /* bad mode / dtype / topk / thresh / cap */
  SATTN_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than sattn_mask_workspace_bytes() */
  SATTN_ERR_HIP = 6,          /* a HIP launch or runtime call failed */
  SATTN_ERR_INDEX = 7         /* validation mode: an index list breaks the sattn_forward preconditions */
} sattn_status;

enum { SATTN_TOPK = 0, SATTN_THRESH = 1 };   /* sattn_mask mode */
enum { SATTN_BF16 = 0, SATTN_F32 = 1 };      /* output dtype */

/* Largest supported key count for sattn_mask (the per-group scores are held on chip). */
#define SATTN_MASK_MAX_NK 131072

/*
 * sattn_mask_workspace_bytes - device workspace that sattn_mask needs for these sizes.
 * Returns 0 if the sizes are invalid.  The workspace holds the group means and the fp32
 * mean-query scores of as many heads as fit in about 2 GB (at least one head), plus a
 * 1/16 sample of those scores.
 */
size_t sattn_mask_workspace_bytes(int B, int H, int Nq, int Nk, int D, int group);

/*
 * sattn_mask - per-group key lists from the group-mean query (the pooling mask).
 *
 * FG-Attn review (pith.science/paper/2509.16518), "The pith" and Referee major comment 2:
 * the queries of a group are averaged into q_avg, every key is scored against it, and slices
 * whose pooled score is small are skipped.  The threshold there is garbled; it is read as the
 * pooled softmax probability p_j = exp(s_j) / sum_i exp(s_i), s_j = scale * (q_avg . k_j).
 * Chipmunk review (pith.science/paper/CJ4ETNKV), "What carries the argument": a top-k index mask.
 *
 *   q      bf16 [B,H,Nq,D]            k  bf16 [B,H,Nk,D]
 *   mode   SATTN_TOPK:   keep the `topk` (1..Nk) highest s_j; ties go to the lower key index.
 *          SATTN_THRESH: keep j iff p_j >= thresh (thresh in [0,1]; 0 keeps all);
 *                        if no key qualifies the arg-max key (lowest index on ties) is kept.
 *   idx    int32 [B,H,G,cap]  out: idx[b,h,g,0:counts[b,h,g]] = kept key indices, strictly
 *                             ascending; entries past counts are left untouched.
 *   counts int32 [B,H,G]      out: number kept (= topk in TOPK mode, >= 1 in THRESH mode).
 *   cap    row length of idx: >= topk (TOPK) or >= Nk (THRESH).
 *   workspace / ws_bytes: device scratch of at least sattn_mask_workspace_bytes() bytes.
 * Scores are computed in fp32 (q_avg is split into two bf16 terms for the matrix cores), so a
 * key whose score lies within ~1e-5 of the cut may land on either side of it.
 * Errors: SATTN_ERR_NULL, _SHAPE, _UNSUPPORTED (also Nk > SATTN_MASK_MAX_NK), _ARG, _WORKSPACE, _HIP.
 */
int sattn_mask(const void* q, const void* k, int B, int H, int Nq, int Nk, int D, int group,
               int mode, int topk, float thresh, float scale,
               int32_t* idx, int32_t* counts, int cap,
               void* workspace, size_t ws_bytes, void* stream);

/*
 * sattn_mask_noalloc - sattn_mask without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid it).
 *
 * Same arguments (minus workspace / ws_bytes), modes, outputs and errors as sattn_mask, and the same
 * kernels, so the key lists equal sattn_mask's bit for bit.  The workspace is a fixed device array of
 * SATTN_MASK_SCRATCH_BYTES inside the library: every GPU the library runs on holds one until the
 * process ends, and the call itself allocates nothing.  The heads run in ranges whose workspace fits
 * that array; a shape for which one head's workspace does not fit (about 4.3 * G * Nk bytes: 549
 * groups of 70,200 keys need about 164 MB and fit, 1024 groups of 131,072 keys need about 570 MB and
 * do not) returns SATTN_ERR_UNSUPPORTED before any HIP call.  All calls on one GPU share its array: calls that overlap
 * on one GPU (other streams or host threads) race and must be serialised by the caller.
 */
#define SATTN_MASK_SCRATCH_BYTES (192u << 20)
int sattn_mask_noalloc(const void* q, const void* k, int B, int H, int Nq, int Nk, int D, int group,
                       int mode, int topk, float thresh, float scale,
                       int32_t* idx, int32_t* counts, int cap, void* stream);

/*
 * sattn_colsum_mask - Chipmunk's selection: per group, the topk keys with the largest column sums
 * of attention probabilities.
 *
 * Chipmunk review, Referee major comment 2 (Alg. 4 and Appendix B.2): a chunk's columns are
 * ranked by the summed attention probabilities of its queries, computed with the softmax
 * normalisation constants of an earlier step, and the top-k indices are cached for the sparse
 * steps.  With lse the natural-log row log-sum-exp of that step (attn_forward's lse):
 *     c[g][j] = sum_{i in group g} exp(scale * Q[i].K[j] - lse[i]),   keep the topk largest
 * (ties to the lowest key index; lists ascending, counts = topk).  bf16 inputs, fp32 sums.
 *
 *   q, k, group, topk, scale, idx, counts, cap, workspace, ws_bytes: as sattn_mask in top-k mode
 *   (the workspace size is sattn_mask_workspace_bytes()).  lse fp32 [B,H,Nq] (device).
 * Errors: as sattn_mask.
 */
int sattn_colsum_mask(const void* q, const void* k, const float* lse,
                      int B, int H, int Nq, int Nk, int D, int group, int topk, float scale,
                      int32_t* idx, int32_t* counts, int cap,
                      void* workspace, size_t ws_bytes, void* stream);

/*
 * sattn_cached_mask - the full-attention slice mask that a dense iteration leaves for later ones.
 *
 * FG-Attn review, Figure 10 and its list of free parameters: every M x 1 slice (the `group`
 * queries of a group against one key) that holds at least one full-attention softmax
 * probability above tau_cached = 0.5 / N is kept, and the mask is reused by later iterations.
 * With lse the natural-log row log-sum-exp of the dense pass (attn_forward's lse output):
 *     keep (g, j)  <=>  max_{i in group g} exp(scale * Q[i].K[j] - lse[i]) >= tau
 * (tau <= 0 keeps every key; a group may keep none).  Scores are bf16 x bf16 with fp32
 * accumulation; the comparison is made in fp32.
 *
 *   q bf16 [B,H,Nq,D]; k bf16 [B,H,Nk,D]; lse fp32 [B,H,Nq] (caller-owned, device).
 *   group: multiple of 16 in [16, 256]; D in {64, 128}; Nk <= SATTN_MASK_MAX_NK.
 *   Outputs as sattn_mask: idx int32 [B,H,G,cap] ascending (entries past counts untouched),
 *   counts int32 [B,H,G] = min(kept, cap); a list longer than cap keeps its first cap keys.
 *   No workspace; nothing is allocated.
 * Errors: SATTN_ERR_NULL, _SHAPE, _UNSUPPORTED, _ARG (cap < 1, scale, NaN tau, alignment), _HIP.
 */
int sattn_cached_mask(const void* q, const void* k, const float* lse,
                      int B, int H, int Nq, int Nk, int D, int group, float tau, float scale,
                      int32_t* idx, int32_t* counts, int cap, void* stream);

/*
 * sattn_forward - fine-grained sparse attention forward over per-group key lists.
 *
 * FG-Attn review, "What carries the argument" and Fig. 6 / Fig. 7 captions: each group of
 * `group` contiguous queries computes scores only against its relevant keys, which are
 * gathered into dense tiles for the matrix units.  Chipmunk review, Referee major comment 1
 * (Alg. 3): the softmax is normalised over the selected keys only.  So for group rows R and
 * kept keys J = idx[b,h,g,0:c], c = counts[b,h,g]:
 *     out[R] = softmax_J(scale * Q[R] K[J]^T) V[J],   lse[R] = ln sum_{j in J} exp(scale * Q[R].K[j])
 * computed with bf16 inputs, fp32 accumulation and an fp32 online softmax (LongLive DiT blog,
 * "Online Softmax").  The probabilities enter P.V rounded to bf16 and the normaliser sums those
 * same rounded values, so out is exactly their weighted mean of V (error within the stated
 * 1e-2 max-abs / 5e-3 rel-L2 of the exact result; lse within -ln(1 - 2^-8) = 3.9e-3, the bf16
 * rounding of the summed probabilities).  A group with c = 0
 * gets out = 0 and lse = -inf.
 *
 *   q bf16 [B,H,Nq,D]; k, v bf16 [B,H,Nk,D]
 *   idx int32 [B,H,G,cap], counts int32 [B,H,G], 0 <= counts <= cap.
 *   Preconditions: idx[b,h,g,0:counts] unique, ascending, in [0,Nk).  Entries past counts
 *   are never read.  With the environment variable SATTN_VALIDATE=1 the lists are checked on
 *   the device first (the call then synchronises the stream) and a violation returns
 *   SATTN_ERR_INDEX; otherwise a violation is undefined behaviour (out-of-range indices are
 *   read as zero rows, never out of bounds).
 *   out  [B,H,Nq,D], bf16 (round to nearest even) or fp32 per out_dtype.
 *   lse  fp32 [B,H,Nq] or NULL.
 */
int sattn_forward(const void* q, const void* k, const void* v,
                  const int32_t* idx, const int32_t* counts, int cap,
                  int B, int H, int Nq, int Nk, int D, int group, float scale,
                  void* out, int out_dtype, float* lse, void* stream);

/*
 * sattn_forward_split_workspace_bytes - device workspace that sattn_forward_split needs: per query
 * row and part, D fp32 partial outputs and a (max, normaliser) float pair.  0 for invalid sizes.
 */
size_t sattn_forward_split_workspace_bytes(int B, int H, int Nq, int D, int splits);

/*
 * sattn_forward_split - sattn_forward with each group's key list cut into `splits` parts that run
 * as separate workgroups, then merged.
 *
 * The same result as sattn_forward (same definition, inputs, preconditions, out and lse; FG-Attn
 * review, "What carries the argument"; Chipmunk review, Referee major comment 1), reached for lists
 * too few or too unequal to fill the GPU in one pass: part p takes whole 32-key blocks
 * [p n / splits, (p+1) n / splits) of the group's n blocks and leaves its unnormalised output and its
 * online-softmax state (running max m_p, normaliser l_p) in the workspace; a merge pass forms
 * out = sum_p 2^(m_p - m) O_p / sum_p 2^(m_p - m) l_p with m = max_p m_p (LongLive DiT blog,
 * "Online Softmax": the rescale that combines partial softmax states).  The result differs from
 * sattn_forward's only in fp32 rounding order, within the same error bounds.
 *   splits: 1 .. 32.
 *   workspace / ws_bytes: device memory of at least sattn_forward_split_workspace_bytes() bytes,
 *   16-byte aligned; its contents are overwritten.  Calls sharing a workspace must not overlap.
 *   Errors as sattn_forward, plus SATTN_ERR_WORKSPACE for a NULL or short workspace and
 *   SATTN_ERR_ARG for splits outside 1 .. 32.
 */
int sattn_forward_split(const void* q, const void* k, const void* v,
                        const int32_t* idx, const int32_t* counts, int cap,
                        int B, int H, int Nq, int Nk, int D, int group, float scale, int splits,
                        void* workspace, size_t ws_bytes,
                        void* out, int out_dtype, float* lse, void* stream);

/*
 * sattn_delta_forward - Chipmunk sparse-delta step: refresh only the listed keys' part of a
 * cached attention output.
 *
 * Chipmunk review, "What carries the argument" and Referee major comments 1-2: the output of
 * a step is the cached output plus a sparse correction recomputed for the selected columns of
 * K^T and rows of V, with the softmax normalisation constants of an earlier step reused.  In
 * the full-softmax form the review asks for, with a stale lse and kept keys J of group g:
 *     fresh_new[i] = sum_{j in J} exp(scale * Q[i].K[j] - lse[i]) V[j]     (no renormalisation)
 *     out[i]       = out_prev[i] - fresh[i] + fresh_new[i],   then fresh[i] <- fresh_new[i].
 * At a dense step the caller keeps the dense output as out_prev and obtains the first fresh
 * part by one call with out_prev = fresh = 0.
 *
 *   q, k, v, idx, counts, cap, group, scale: as sattn_forward (same list preconditions).
 *   lse      fp32 [B,H,Nq], natural log (e.g. attn_forward's lse of the dense step).
 *   out_prev fp32 [B,H,Nq,D] cached output; fresh fp32 [B,H,Nq,D] in: previous part, out: new part.
 *   out      [B,H,Nq,D] bf16 or fp32 per out_dtype; may be out_prev itself when fp32 (in place).
 * Errors: as sattn_forward.
 */
int sattn_delta_forward(const void* q, const void* k, const void* v,
                        const int32_t* idx, const int32_t* counts, int cap,
                        int B, int H, int Nq, int Nk, int D, int group, float scale,
                        const float* lse, const float* out_prev, float* fresh,
                        void* out, int out_dtype, void* stream);

/*
 * attn_forward - dense control path: every query attends to every key.
 * LongLive DiT blog, "Self Attention" and "Online Softmax": per-head softmax(Q K^T * scale) V,
 * tiled so the score matrix is never materialised.  Same layouts, precision and lse definition
 * as sattn_forward, with no index lists.
 */
int attn_forward(const void* q, const void* k, const void* v,
                 int B, int H, int Nq, int Nk, int D, float scale,
                 void* out, int out_dtype, float* lse, void* stream);

/*
 * FP8 value path (V-Smart/ExpCast summary, its V-Smooth and ExpCast-FP8 paragraphs).
 *
 * sattn_vsmooth_quantize - V-Smooth quantisation of V for sattn_fp8_forward.  Per block of 128
 * tokens (the last block may be shorter) and channel, the exact mean of the bf16 tokens is
 * rounded to bf16 (nearest even); the fp32 residual v - mean is divided by the channel scale
 * s = 2^e, the smallest power of two with 448 * s >= max |residual| over the head (1 when the
 * residual is 0), and rounded to E4M3 (OCP "fn" encoding, nearest even).
 *   v       bf16 [B,H,Nk,D], 16-byte aligned.
 *   codes   out: uint8 [B,H,Nk,D] E4M3 codes, 16-byte aligned.
 *   vscale  out: fp32 [B,H,D] channel scales (powers of two), 16-byte aligned.
 *   vmean   out: bf16 [B,H,D,S] with S = sattn_vsmooth_mean_stride(Nk), 16-byte aligned:
 *           entry [b,h,d,blk] = mean of block blk / vscale[b,h,d] (exact); entries past the last
 *           block are 0.  Channel-major so that the forward reads a window of 32 blocks per channel.
 *   workspace device scratch of sattn_vsmooth_workspace_bytes(B,H,Nk,D) bytes, 256-byte aligned.
 * The block mean equals the rounded exact mean when the tokens of a block span fewer than 2^45
 * in magnitude (the fp64 sum is then exact).  Errors: NULL pointers, D not 64/128, bad sizes or
 * alignment, workspace too small.
 */
size_t sattn_vsmooth_workspace_bytes(int B, int H, int Nk, int D);
int sattn_vsmooth_mean_stride(int Nk);   /* 4 * ceil(ceil(Nk / 128) / 4); 0 if Nk < 1 */
int sattn_vsmooth_quantize(const void* v, int B, int H, int Nk, int D, uint8_t* codes, float* vscale,
                           void* vmean, void* workspace, size_t ws_bytes, void* stream);

/*
 * sattn_fp8_forward - sparse forward over per-group key lists with ExpCast probability bytes and
 * an E4M3 P.V product, on V quantised by sattn_vsmooth_quantize.
 *
 * For query row i of group g with listed keys J (list order, blocks of 64): s = scale q_i.k_j in
 * log2 units; the row's reference point m (a multiple of 1/8) is ceil8 of the first block's max
 * and moves only when a later block's max exceeds m + 13/16 (a byte would pass 126), then by the
 * smallest whole number of log2 units that brings that max to or below m (earlier sums are scaled
 * by the exact power of two 2^(m_old - m_new)); the probability is the E4M3 byte
 * round-half-even(8 (s - m) + 120) clamped to [0, 126] (the summary's 8 log2 v + 56 with the
 * probability scaled by 2^8).  While every byte is a normal code this equals ExpCast in one pass at
 * the final m: the result does not depend on the block size or on where the moves fall;
 *     out[i] = sum_j p_j (vscale * E4M3(codes[j]) + mean_block(j)) / sum_j p_j,
 *     lse[i] = ln(sum_j p_j) + (m - 8) ln 2.
 *   q, k, idx, counts, cap, group, scale, out, out_dtype, lse: as sattn_forward (same list
 *   preconditions); codes, vscale, vmean: the outputs of sattn_vsmooth_quantize for V.
 * Range: the sums are kept in the frame of the row's first reference point, each later block scaled
 * by 2^(m - m_first) with that factor capped at 2^90 so the fp32 sums stay finite.  A row whose
 * largest listed score exceeds m_first by more than 90 log2 units (62.38 in units of scale q.k)
 * would weigh its later keys wrongly, so its out and lse are written as NaN (the call still returns
 * SATTN_OK).  Rows within that range get the result above.
 * Errors: as sattn_forward; codes, vscale and vmean must be 16-byte aligned.
 */
int sattn_fp8_forward(const void* q, const void* k, const uint8_t* codes, const float* vscale,
                      const void* vmean, const int32_t* idx, const int32_t* counts, int cap,
                      int B, int H, int Nq, int Nk, int D, int group, float scale,
                      void* out, int out_dtype, float* lse, void* stream);

/*
 * 4-bit QK^T (LongLive DiT blog, section "1. NVFP4": E2M1 codes with a shared scale per block,
 * applied inside the block-scaled matrix product).  On gfx950 the format is MXFP4 (OCP microscaling):
 * blocks of 32 elements along the head dimension with power-of-two (E8M0) scales.
 *
 * sattn_mx4_quantize - per row of x and block of 32: scale 2^e with the smallest e such that
 * 6 * 2^e >= max |x| (e >= -127; e = 0 for a zero block), codes = nearest E2M1 of x / 2^e (ties to
 * the even code).  (FourOverSix's max-to-4 alternative never has the smaller error with power-of-two
 * scales, so max-to-6 is the rule.)
 *   x       bf16 [B,H,N,D], 16-byte aligned (queries or keys).
 *   codes   out: uint8 [B,H,N,D/2], two codes a byte (even element in the low nibble), 16-byte aligned.
 *   scales  out: uint8 [B,H,N,4], byte b = e + 127 of block b (D/32 blocks; at D = 64 bytes 2 and 3 are
 *           127), 4-byte aligned.
 * Errors: NULL pointers, D not 64/128, bad sizes or alignment.
 */
int sattn_mx4_quantize(const void* x, int B, int H, int N, int D, uint8_t* codes, uint8_t* scales, void* stream);

/*
 * sattn_fp4_forward - sattn_fp8_forward with the scores from the MXFP4 queries and keys:
 * s = scale * sum_b 2^(eq_b + ek_b) E2M1(q_b) . E2M1(k_b), on v_mfma_scale_f32_32x32x64_f8f6f4 in
 * FP4 x FP4.  q4, q_scales, k4, k_scales: sattn_mx4_quantize of Q and K; everything else as
 * sattn_fp8_forward (its range limit included).  Errors: as sattn_fp8_forward; q4 and k4 16-byte, the
 * scales 4-byte aligned.
 */
int sattn_fp4_forward(const uint8_t* q4, const uint8_t* q_scales, const uint8_t* k4, const uint8_t* k_scales,
                      const uint8_t* codes, const float* vscale, const void* vmean,
                      const int32_t* idx, const int32_t* counts, int cap,
                      int B, int H, int Nq, int Nk, int D, int group, float scale,
                      void* out, int out_dtype, float* lse, void* stream);

/*
 * sattn_voxel_permutation - host-side token order that makes every run of vt*vy*vx tokens one
 * spatio-temporal voxel of a (T, Hg, Wg) raster grid.
 * Chipmunk review, "What carries the argument" and Fig. 2 caption (voxel reordering so that
 * column-sparse chunks are 3D cubes; voxel (4,6,8) in "Assumptions & free parameters").
 * Tokens are ordered by (t/vt, y/vy, x/vx, t%vt, y%vy, x%vx).  perm is a HOST int32 array of
 * T*Hg*Wg entries: permuted[i] = original[perm[i]].
 */
int sattn_voxel_permutation(int T, int Hg, int Wg, int vt, int vy, int vx, int32_t* perm);

/*
 * sattn_permute_tokens - dst[b,h,i,:] = src[b,h,perm[i],:] (inverse = 0) or
 * dst[b,h,perm[i],:] = src[b,h,i,:] (inverse = 1) for bf16 [B,H,N,D] tensors; perm is a
 * DEVICE int32 permutation of [0,N).  Applies and undoes the voxel order on the device.
 * perm is not checked: an entry outside [0,N) leaves its destination row unwritten, and a
 * repeated entry leaves some destination row unwritten (or, with inverse = 1, written twice).
 */
int sattn_permute_tokens(const void* src, void* dst, const int32_t* perm, int B, int H, int N, int D,
                         int inverse, void* stream);

const char* sattn_strerror(int status);   /* static description of a status code */
const char* sattn_last_error(void);       /* thread-local detail of the last failed call */

#ifdef __cplusplus
}
#endif
#endif /* SATTN_H */
