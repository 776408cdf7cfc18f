/*
 * drafthead.h -- C ABI of the 2-bit speculative-draft LM head for MI355X (gfx950).
 *
 * The head scores x[M, K] against one tensor-parallel rank's vocabulary shard
 * W[N, K] (row n = vocabulary token n) with 2-bit weights, keeps the best
 * KCAND columns of every 64-column block, rescoring the best R of those
 * exactly against the bf16 weight, and returns each row's argmax token.
 * The method is the one the page "radiance_drafthead.py" (a vLLM plug-in
 * module) describes in its module docstring and implements in
 * `_quantize_head_now` (load time) and `_apply_head_int2` (per call).
 *
 * Call sequence:
 *   load time (host):  draft_head_quantize_pack -> draft_head_tile -> copy to device
 *   per call (device): draft_head_coarse -> draft_head_rerank -> draft_head_argmax,
 *                      or the three in one host call: draft_head_forward
 *                      (rerank from e4m3 rows: the *_e4m3 variants); for a top-k
 *                      caller, draft_head_forward_row (the call and the row
 *                      together) or draft_head_logits_row after a call
 *
 * Conventions for every function:
 *   - Return value: DH_OK (0) or a negative DH_E* code; never throws.  The
 *     message of the last error on the calling thread is draft_head_last_error().
 *   - All argument validation happens before any HIP call, so every error
 *     except DH_EHIP can be provoked without a GPU.
 *   - The caller owns every buffer.  The library allocates no device memory
 *     and keeps no state between calls; the scratch memory the coarse pass
 *     and the one-call path need (hand-off words, and for more than 8 rows x laid
 *     out for the many-row kernel) is the caller's workspace of
 *     draft_head_workspace_bytes() bytes.
 *   - Device functions enqueue work asynchronously on `stream` (a hipStream_t
 *     passed as void*, NULL = the null stream) and return once it is enqueued;
 *     launch errors are reported by the call that launched (DH_EHIP).  Calls on
 *     one stream see each other's results in order.
 *   - bf16 values are passed as their 16-bit patterns (uint16_t) or as void*.
 */
#ifndef DRAFTHEAD_H
#define DRAFTHEAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DH_OK 0
#define DH_EINVAL (-1)  /* null or misaligned pointer, argument out of range */
#define DH_ESHAPE (-2)  /* K not a positive multiple of 512 (or > DH_MAX_K), N < 1 */
#define DH_EUNSUP (-3)  /* M > DH_MAX_M, kcand outside 1..DH_MAX_KCAND, R outside 1..min(ncand, DH_MAX_R) */
#define DH_EHIP (-4)    /* HIP runtime or kernel launch error */

#define DH_GROUP 128        /* quantisation group along K (the page's GROUP) */
#define DH_BLOCK_N 64       /* selection block width (the page's BLOCK_N) */
#define DH_MAX_M 128
#define DH_MAX_K 65536
#define DH_MAX_KCAND 64
#define DH_MAX_R 1024
#define DH_NOALLOC_SCRATCH_BYTES (4u << 20)   /* draft_head_forward_noalloc's static scratch per GPU */

/* Message describing the last error returned on the calling thread ("" if none). */
const char* draft_head_last_error(void);

/*
 * Buffer sizes for an N x K head (K a multiple of 512).
 *   packed_bytes   N * K/4        canonical quarter-split codes (draft_head_quantize_pack)
 *   scale_elems    N * K/128      entries of S and of ZS each (bf16)
 *   tiled_bytes    NBLK*64 * K/4  device-layout codes (draft_head_tile), NBLK = ceil(N/64)
 *   tiled_pairs    NBLK*64 * K/128  device-layout (S, ZS) pairs, one uint32 each
 * Any output pointer may be NULL.  Errors: DH_ESHAPE.
 */
int draft_head_sizes(int64_t N, int64_t K, size_t* packed_bytes, size_t* scale_elems,
                     size_t* tiled_bytes, size_t* tiled_pairs);

/*
 * HOST.  Quantise a bf16 weight to asymmetric min/max int2 and pack it, as
 * the radiance_drafthead.py page's load-time quantiser does: each group of
 * 128 consecutive k of a row gets a grid of four levels spanning the group's
 * range, with step max((hi - lo)/3, 1e-8) and zero level -lo/step rounded to
 * nearest even and clamped to 0..3; a weight's code is w/step + zero rounded
 * to nearest even and clamped; the group stores S = bf16(4 step) and
 * ZS = bf16(4 step + zero step).  Every step is one float32 operation rounded
 * on its own, as the page's tensor operations are, so the bytes match its
 * quantiser exactly.  Packing (the module docstring's "Quarter-split
 * packing"): byte j of a row holds the codes of k = j, K/4+j, K/2+j, 3K/4+j in
 * bits 0-1, 2-3, 4-5, 6-7.
 *   w        bf16 bits, row-major [N][ldw], ldw >= K (read only)
 *   packed   out, uint8 [N][K/4]
 *   S, ZS    out, bf16 bits [N][K/128] each
 *   nthreads host threads to use (0 = all hardware threads)
 * The effective weight of code v is (S/4) v - (ZS - S).
 * Errors: DH_EINVAL (null pointer, ldw < K, nthreads < 0), DH_ESHAPE.
 */
int draft_head_quantize_pack(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                             uint8_t* packed, uint16_t* S, uint16_t* ZS, int nthreads);

/*
 * HOST.  Rearrange the canonical arrays into the device layout the coarse
 * kernel streams (a pure permutation; the last block is padded with zero
 * codes and zero scales).  With b = n/64, t = (n%64)/16, c = n%16 and, for
 * code byte j, G = j/128, h = (j%128)/64, s = (j%64)/16, w = j%16:
 *   tiled[((((b*NG4 + G)*2 + h)*4 + t)*64 + s*16 + c)*16 + w] = packed[n][j]
 *   pairs[((b*NG4 + G)*4 + t)*64 + c*4 + q] = S[n][q*NG4 + G] | ZS[n][q*NG4 + G] << 16
 * where NG4 = K/512 and q = 0..3 is the quarter.  Each 64-column block is one
 * contiguous span of K/4*64 code bytes and K/128*64 pairs.
 *   packed, S, ZS  canonical arrays (read only);  tiled, pairs  out
 * Limits: every |S| <= 255 (the fp16 many-row kernel forms each weight
 * (S/4) v as an exact fp16 value; the quantiser's S = bf16(4 (hi - lo) / 3)
 * stays below it for any group whose range is under about 191), and every
 * S - ZS a bf16 value (the many-row kernels take the zero-point term as that
 * one weight; the quantiser's ZS lies within a factor 1.75 of S).
 * Errors: DH_EINVAL (null pointer), DH_ESHAPE, DH_EUNSUP (a pair beyond the
 * limits, or not finite).
 */
int draft_head_tile(const uint8_t* packed, const uint16_t* S, const uint16_t* ZS,
                    int64_t N, int64_t K, uint8_t* tiled, uint32_t* pairs);

/*
 * HOST.  The 4-bit head of the page (`_quantize_head_now` at BITS = 4): the
 * quantiser of draft_head_quantize_pack with 15 levels and the premultiplier
 * 16, per (row n, group g of 128 consecutive k), each float32 operation
 * rounded on its own:
 *   sc = max((hi - lo) / 15, 1e-8);  zp = clamp(rne(-lo / sc), 0, 15)
 *   q = clamp(rne(w / sc + zp), 0, 15);  S = bf16(16 sc);  ZS = bf16(16 sc + zp sc)
 * and half-split packing: byte j of a row holds the codes of k = j (bits 0-3)
 * and K/2 + j (bits 4-7).  The effective weight of code v is (S/16) v - (ZS - S).
 *   w        bf16 bits [N][ldw], ldw >= K;  packed4  out, uint8 [N][K/2]
 *   S, ZS    out, bf16 bits [N][K/128] each
 * Limits: K a positive multiple of 256 with 2K <= DH_MAX_K.
 * Errors: DH_EINVAL (null pointer, ldw < K, nthreads < 0), DH_ESHAPE.
 */
int draft_head_quantize_pack_int4(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* packed4,
                                  uint16_t* S, uint16_t* ZS, int nthreads);

/*
 * HOST.  A 4-bit head as a 2-bit head of length 2K, the form the device path
 * runs: with v = 4 vh + vl, the weight (S/16) v - (ZS - S) of k equals the
 * 2-bit weight of k' = k (code vh, pair S, ZS) plus that of k' = K + k (code
 * vl, pair S/4, S/4, exact in bf16), so for x' = (x, x) the 2-bit scores of
 * the 2K-long head are the 4-bit scores.  The output is in the canonical
 * 2-bit form (quarter-split over 2K; pairs of groups K/128 .. 2K/128 - 1 are
 * the S/4 ones); tile it with draft_head_tile(N, 2K).
 *   packed4, S, ZS   draft_head_quantize_pack_int4's arrays
 *   packed2   out, uint8 [N][K/2] (2K/4 bytes a row);  S2, ZS2  out, bf16 bits [N][2K/128]
 * Errors: DH_EINVAL (null pointer), DH_ESHAPE (as draft_head_quantize_pack_int4).
 */
int draft_head_int4_as_int2(const uint8_t* packed4, const uint16_t* S, const uint16_t* ZS, int64_t N, int64_t K,
                            uint8_t* packed2, uint16_t* S2, uint16_t* ZS2);

/*
 * HOST.  The device form of a 4-bit head, which draft_head_coarse_int4 and
 * draft_head_forward_int4 take: the page's own code bytes (byte j: the code
 * of k = j in bits 0-3, of K/2 + j in bits 4-7), placed as draft_head_tile
 * places a 2-bit head of length 2K, whose bytes have the same count
 * (tiled = draft_head_tile(packed4 as [N][2K/4], N, 2K)'s codes, NBLK*64 *
 * K/2 bytes); quarter q < 2 of that form covers the k of nibble q.  pairs
 * holds the head's own (S, ZS), NBLK*64 * K/128 entries, in the slots of
 * quarters 0 and 1 of each byte group of that form:
 *   pairs[((b*NG4 + G)*4 + t)*32 + c*2 + q] = S | ZS << 16 of column
 *   64b + 16t + c, group q*NG4 + G   (NG4 = K/256, q = 0, 1)
 * A call streams N*K/2 code bytes and N*K/128 pairs, the 4-bit head's size.
 *   packed4, S, ZS  draft_head_quantize_pack_int4's arrays;  tiled, pairs  out
 * Limits and errors: as draft_head_quantize_pack_int4 and draft_head_tile.
 */
int draft_head_tile_int4(const uint8_t* packed4, const uint16_t* S, const uint16_t* ZS, int64_t N, int64_t K,
                         uint8_t* tiled, uint32_t* pairs);

/*
 * Bytes of device workspace draft_head_coarse / draft_head_forward need for M
 * rows of length K: 1,024 bytes of per-row hand-off words for the one-call
 * path's rerank (a row's exact logits may be split over several workgroups),
 * plus, where M <= 8 and the resident kernel holds all of x in LDS (any K at
 * M = 1; K <= 39424, 19456, 8704 at M = 2, 3..4, 5..8), 65,536 bytes in which
 * the one-call path's coarse kernel writes each block's maximum once more,
 * contiguously, for its rerank (66,560 bytes in all); otherwise the x of one
 * launch of up to 80 rows laid out for the many-row kernel, (K/128) * 4096 *
 * MT + (K/512) * 4096 + 512 bytes with MT = min(ceil(M/16), 5), and the block
 * maxima of the M rows, 8,192 * M bytes (1,451,520 bytes in all at M = 72,
 * K = 5120).
 * Errors: DH_EINVAL (null pointer, M < 1), DH_EUNSUP (M > DH_MAX_M), DH_ESHAPE.
 */
int draft_head_workspace_bytes(int M, int K, size_t* bytes);

/*
 * DEVICE.  Coarse scores and block top-KCAND candidates.
 * Follows `_draft_head_int2` and `_emit` on the radiance_drafthead.py page:
 * for every row m and column n, c[m][n] = sum over groups g of
 * S * sum_k x (1 + v/4) - ZS * sum_k x  (fp32 accumulation), which equals
 * sum_k x[m][k] * ((S/4) v - (ZS - S)); then, per 64-column block, the KCAND
 * largest c ordered by (value desc, column asc).
 *   x          device, bf16 [M][K] row-major, 16-byte aligned
 *   tiled, pairs  device, draft_head_tile layout, 16-byte aligned
 *   cand_val   out, fp32 [M][NBLK*kcand]; slot b*kcand + i = i-th best of block b
 *   cand_id    out, int32, same shape: global column id, or -1 (value -inf)
 *              when block b has fewer than kcand columns (n >= N)
 *   coarse_out optional out (NULL = not written), fp32 [M][N] coarse scores
 *   workspace  device scratch of at least draft_head_workspace_bytes(M, K)
 *              bytes, 16-byte aligned; its contents are overwritten, so calls
 *              that share one workspace must be ordered (e.g. on one stream)
 * x values must be finite with |x| < 2^63 (x is scaled by 2^64 on chip).
 * Limits: 1 <= M <= DH_MAX_M, K % 512 == 0, N >= 1, 1 <= kcand <= DH_MAX_KCAND.
 * Errors: DH_EINVAL (also: workspace missing, misaligned or too small),
 *         DH_ESHAPE, DH_EUNSUP, DH_EHIP.
 */
int draft_head_coarse(const void* x, int M, int K, int N, const uint8_t* tiled,
                      const uint32_t* pairs, int kcand, float* cand_val, int32_t* cand_id,
                      float* coarse_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * DEVICE.  Row top-R of the candidates and their exact logits.
 * Follows `bm.topk(RERANK)` + `bi.gather` and `_rerank_exact` (bf16 branch) on
 * the radiance_drafthead.py page: per row, the R best (value desc, id asc)
 * candidates with id >= 0, then e = sum_k x[m][k] * W[id][k] in fp32.
 *   x          device, bf16 [M][K], 16-byte aligned
 *   w          device, bf16 [N][ldw] (the head's own weight), 16-byte aligned,
 *              ldw >= K and ldw % 8 == 0
 *   cand_val, cand_id  device, [M][ncand] as written by draft_head_coarse
 *   rr_id      out, int32 [M][R], ordered (coarse value desc, id asc); -1 pads
 *              a row with fewer than R valid candidates
 *   rr_val     out, fp32 [M][R] exact logit of rr_id (-inf where rr_id = -1)
 * Limits: 1 <= M <= DH_MAX_M, K % 256 == 0, 1 <= R <= min(ncand, DH_MAX_R).
 * Errors: DH_EINVAL, DH_ESHAPE, DH_EUNSUP, DH_EHIP.
 */
int draft_head_rerank(const void* x, const void* w, int64_t ldw, int M, int K, int N,
                      const float* cand_val, const int32_t* cand_id, int ncand, int R,
                      int32_t* rr_id, float* rr_val, void* stream);

/*
 * DEVICE.  draft_head_rerank with the head's rows stored as e4m3 bytes and a
 * per-row fp32 scale (the FP8 branch of `_rerank_exact` on the
 * radiance_drafthead.py page: a per-channel FP8 lm_head).  Each byte b is
 * decoded by the page's bit arithmetic: e = (b >> 3) & 15, mant = b & 7,
 * magnitude mant * 2^-9 if e == 0 else (1 + mant/8) * 2^(e-7), bit 7 the sign
 * (so 0x7F / 0xFF read as +-480, not NaN); the weight is that value times
 * wscale[id] in fp32, and e = sum_k x * weight in fp32.
 *   w8       device, e4m3 bytes [N][ldw], 16-byte aligned, ldw >= K, ldw % 16 == 0
 *   wscale   device, fp32 [N]
 * Everything else as draft_head_rerank.  Errors: as draft_head_rerank.
 */
int draft_head_rerank_e4m3(const void* x, const uint8_t* w8, const float* wscale, int64_t ldw, int M, int K,
                           int N, const float* cand_val, const int32_t* cand_id, int ncand, int R,
                           int32_t* rr_id, float* rr_val, void* stream);

/*
 * DEVICE.  draft_head_rerank with the head's rows in NVFP4 (the gathered
 * projection `_nvfp4_gathered_bias_kernel` on the page for vLLM pull request
 * 55713): per row, K/2 bytes of e2m1 codes, byte j holding element 2j in its
 * low nibble and element 2j+1 in its high nibble; an e4m3 scale byte per 16
 * elements (the format's own decode: 0x7F / 0xFF are NaN); one global fp32
 * scale.  An e2m1 nibble has sign bit 3, exponent bits 2-1 with bias 1 and
 * mantissa bit 0 (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).  The weight is
 * bf16(fp32(fp32(value * block scale) * global scale)), rounded to nearest
 * even, and e = sum_k x * weight in fp32.
 *   w4       device, uint8 [N][ldw], 16-byte aligned, ldw >= K/2, ldw % 16 == 0
 *   bscale   device, e4m3 bytes [N][lds], 2-byte aligned, lds >= K/16, lds even
 *   gscale   device, one fp32
 * Everything else as draft_head_rerank.  Errors: as draft_head_rerank.
 */
int draft_head_rerank_nvfp4(const void* x, const uint8_t* w4, int64_t ldw, const uint8_t* bscale, int64_t lds,
                            const float* gscale, int M, int K, int N, const float* cand_val, const int32_t* cand_id,
                            int ncand, int R, int32_t* rr_id, float* rr_val, void* stream);

/*
 * DEVICE.  Final token per row: the rr_id whose exact value is largest, ties
 * to the lower id, entries with id -1 ignored (the page leaves the argmax of
 * the written-back row to the caller's sampler).
 *   rr_id, rr_val  device, [M][R]
 *   out_id     out, int32 [M] (-1 if a row has no valid entry)
 *   out_val    out, fp32 [M] its exact logit (-inf if none)
 * Errors: DH_EINVAL, DH_EUNSUP, DH_EHIP.
 */
int draft_head_argmax(const int32_t* rr_id, const float* rr_val, int M, int R,
                      int32_t* out_id, float* out_val, void* stream);

/*
 * DEVICE.  One full call of the head: draft_head_coarse, draft_head_rerank
 * (ncand = NBLK*kcand) and draft_head_argmax enqueued back to back on
 * `stream` with one host call (the page's `_draft_head_int2` from x to the
 * written-back candidates, plus the final argmax).  Every argument is
 * validated before the first launch; the arguments mean what they mean in
 * the three calls above.
 *   coarse_start_event, coarse_stop_event  optional hipEvent_t (as void*,
 *              created by the caller, NULL = none): they take the start and
 *              end timestamps of the coarse kernel's own dispatch
 *              (hipExtLaunchKernel), so hipEventElapsedTime gives that
 *              kernel's duration (for M > 8, the many-row kernel's, without
 *              the small kernel that lays x out in the workspace before it);
 *              where M > 80 needs several coarse launches, the first one's
 *              start and the last one's end.
 * Errors: as the three calls.
 */
int draft_head_forward(const void* x, int M, int K, int N, const uint8_t* tiled,
                       const uint32_t* pairs, const void* w, int64_t ldw, int kcand, int R,
                       float* cand_val, int32_t* cand_id, int32_t* rr_id, float* rr_val,
                       int32_t* out_id, float* out_val, float* coarse_out, void* workspace,
                       size_t workspace_bytes, void* stream, void* coarse_start_event,
                       void* coarse_stop_event);

/*
 * DEVICE.  draft_head_forward without a workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc.  The scratch the call needs lives in a
 * static device array of DH_NOALLOC_SCRATCH_BYTES (4 MiB) that the library
 * holds on every GPU it runs on until the process ends; the call itself
 * makes no hipMalloc, hipFree or other allocating call.  The caller still
 * passes every input and output, as for draft_head_forward.
 * Limit: draft_head_workspace_bytes(M, K) <= DH_NOALLOC_SCRATCH_BYTES (any M
 * up to DH_MAX_M at K <= 18,432; M <= 8 wherever the resident kernel holds
 * x).  Every call on one GPU shares that GPU's array and overwrites it:
 * calls that overlap on one GPU race, so order them (one stream).  The
 * stream must belong to the current device.
 * Errors: as draft_head_forward; DH_EUNSUP when the call needs more scratch
 * than the array holds (before any HIP call); DH_EINVAL when the stream's
 * device is not the current one; DH_EHIP when the array's address cannot
 * be obtained.
 */
int draft_head_forward_noalloc(const void* x, int M, int K, int N, const uint8_t* tiled,
                               const uint32_t* pairs, const void* w, int64_t ldw, int kcand, int R,
                               float* cand_val, int32_t* cand_id, int32_t* rr_id, float* rr_val,
                               int32_t* out_id, float* out_val, float* coarse_out, void* stream,
                               void* coarse_start_event, void* coarse_stop_event);

/*
 * DEVICE.  draft_head_forward with the e4m3 rerank source of
 * draft_head_rerank_e4m3 (w8, wscale, ldw in bytes) in place of the bf16 rows.
 */
int draft_head_forward_e4m3(const void* x, int M, int K, int N, const uint8_t* tiled, const uint32_t* pairs,
                            const uint8_t* w8, const float* wscale, int64_t ldw, int kcand, int R,
                            float* cand_val, int32_t* cand_id, int32_t* rr_id, float* rr_val, int32_t* out_id,
                            float* out_val, float* coarse_out, void* workspace, size_t workspace_bytes,
                            void* stream, void* coarse_start_event, void* coarse_stop_event);

/*
 * DEVICE.  draft_head_forward with the NVFP4 rerank source of
 * draft_head_rerank_nvfp4 (w4, ldw and lds in bytes, bscale, gscale) in place
 * of the bf16 rows.
 */
int draft_head_forward_nvfp4(const void* x, int M, int K, int N, const uint8_t* tiled, const uint32_t* pairs,
                             const uint8_t* w4, int64_t ldw, const uint8_t* bscale, int64_t lds, const float* gscale,
                             int kcand, int R, float* cand_val, int32_t* cand_id, int32_t* rr_id, float* rr_val,
                             int32_t* out_id, float* out_val, float* coarse_out, void* workspace,
                             size_t workspace_bytes, void* stream, void* coarse_start_event,
                             void* coarse_stop_event);

/*
 * DEVICE.  draft_head_coarse and draft_head_forward for a 4-bit head (the
 * page's BITS = 4 configuration, KCAND = 1 in its measurements): tiled and
 * pairs are draft_head_tile_int4's, which the coarse kernels run in the
 * tiles of a 2-bit head of length 2K, each byte's two codes decoded whole;
 * x, w and everything else are as for the 2-bit calls with K the head's own
 * length.  The workspace is draft_head_workspace_bytes(M, 2K).
 * Limits: K a positive multiple of 256 with 2K <= DH_MAX_K.
 * Errors: as draft_head_coarse / draft_head_forward.
 */
int draft_head_coarse_int4(const void* x, int M, int K, int N, const uint8_t* tiled, const uint32_t* pairs,
                           int kcand, float* cand_val, int32_t* cand_id, float* coarse_out, void* workspace,
                           size_t workspace_bytes, void* stream);
int draft_head_forward_int4(const void* x, int M, int K, int N, const uint8_t* tiled, const uint32_t* pairs,
                            const void* w, int64_t ldw, int kcand, int R, float* cand_val, int32_t* cand_id,
                            int32_t* rr_id, float* rr_val, int32_t* out_id, float* out_val, float* coarse_out,
                            void* workspace, size_t workspace_bytes, void* stream, void* coarse_start_event,
                            void* coarse_stop_event);

/*
 * DEVICE.  The bf16 row the page's `_apply_head_int2` hands to its caller
 * after the rerank: y[m][n] = bf16(coarse[m][n]) (round to nearest even), or
 * -inf for a top-k caller (`_radiance_topk_only`, topk_only != 0: only the
 * reranked ids stay eligible); then, for every r with rr_id[m][r] >= 0,
 * y[m][rr_id[m][r]] = bf16(rr_val[m][r]) (`y.scatter_(1, idx, ex)`).  Ids of
 * -1 write nothing; the ids of a row must be distinct (as draft_head_rerank
 * writes them).
 *   coarse     device, fp32 [M][N] (coarse_out of draft_head_coarse or
 *              draft_head_forward); may be NULL when topk_only
 *   rr_id, rr_val  device, [M][R] as written by draft_head_rerank / forward
 *   row_out    out, bf16 bits [M][N]
 * Limits: 1 <= M <= DH_MAX_M, N >= 1, 1 <= R <= DH_MAX_R.
 * Errors: DH_EINVAL (null pointer, coarse NULL without topk_only),
 *         DH_ESHAPE, DH_EUNSUP, DH_EHIP.
 */
int draft_head_logits_row(const float* coarse, const int32_t* rr_id, const float* rr_val, int M, int N,
                          int R, int topk_only, uint16_t* row_out, void* stream);

/*
 * DEVICE.  draft_head_forward plus the bf16 row for the caller, with no fp32
 * row in between (the page's `_draft_head_int2` stores Y as bf16 from its
 * accumulator; `_apply_head_int2` then scatters the exact values over it):
 * the coarse kernel writes row_out[m][n] = bf16(coarse score) (round to
 * nearest even), or -inf when topk_only != 0 (`_radiance_topk_only`), in its
 * epilogue, and the rerank writes bf16(rr_val[m][r]) at every reranked id.
 * The result equals draft_head_logits_row applied to this call's own coarse
 * scores and reranked values.
 *   row_out    out, bf16 bits [M][N]
 *   the other arguments as draft_head_forward (bf16 rerank rows; no fp32
 *   coarse row and no timing events)
 * Errors: as draft_head_forward; DH_EINVAL for a null row_out.
 */
int draft_head_forward_row(const void* x, int M, int K, int N, const uint8_t* tiled,
                           const uint32_t* pairs, const void* w, int64_t ldw, int kcand, int R,
                           float* cand_val, int32_t* cand_id, int32_t* rr_id, float* rr_val,
                           int32_t* out_id, float* out_val, uint16_t* row_out, int topk_only,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * DEVICE.  Measurement reference, not part of the head: reads `bytes` bytes at
 * p once, with the coarse kernel's kind of loads (16-byte nontemporal loads,
 * each of DH_READ_BLOCKS workgroups streaming one contiguous span), so that
 * its duration gives the read rate the device achieves.  out[b] = XOR of the
 * 32-bit words of workgroup b's span (span b = words [b*S, (b+1)*S) of the
 * 16-byte words, S = ceil(bytes/16 / DH_READ_BLOCKS), cut at the end).
 *   p    device, 16-byte aligned, bytes a positive multiple of 16
 *   out  device, uint32 [DH_READ_BLOCKS]
 * Errors: DH_EINVAL, DH_EHIP.
 */
#define DH_READ_BLOCKS 2048
int draft_head_stream_read(const void* p, size_t bytes, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DRAFTHEAD_H */
