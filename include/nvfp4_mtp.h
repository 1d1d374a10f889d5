/*
 * nvfp4_mtp.h -- C ABI of the NVFP4 W4A16 MTP draft-head library (AMD gfx950).
 *
 * The library runs the hot path of a multi-token-prediction draft head whose
 * projection, expert and LM-head weights are NVFP4: a quantizer, a W4A16
 * decode GEMV, a W4A16 GEMM for prompt-sized row counts, an LM-head GEMV fused
 * with argmax, and a top-k MoE expert FFN.  The operations are the ones the
 * following pages describe (cited by page and item):
 *   [new.rs]      spark_model/layers/mtp_head/new.rs -- `MtpHead::new`
 *   [mtp_head.rs] metrale_model_layers/layers/mtp_head.rs -- module doc,
 *                 `MtpHead` fields, `MtpHead::gemv`, `quantize_proj`
 *   [v4_mtp.rs]   spark_model/layers/deepseek_v4_mtp.rs -- `forward_one`,
 *                 `argmax_grammar_masked`
 *   [prefill.rs]  spark_model/layers/qwen3_attention/prefill_weights.rs --
 *                 `w4a16_gemm_m128_dispatch`
 *
 * Conventions shared by every entry point:
 *  - All data pointers are DEVICE pointers unless a comment says "host".
 *    The caller owns every buffer; the library allocates nothing, keeps no
 *    state between calls and is safe to call from several host threads.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on it and returns; it never synchronizes or reads back
 *    (moe_workspace_status, a host query, is the one exception).
 *  - Return value: NVFP4_OK (0) or a negative status.  Arguments are checked
 *    on the host before anything is enqueued; on failure nothing is enqueued
 *    and nvfp4_mtp_last_error() describes the problem.
 *  - bf16 data are passed as uint16_t bit patterns.
 *
 * NVFP4 weight layout (the pages show only the packed [N, K/2] code array;
 * the rest is the public NVFP4 format): a weight W[N][K] (out = in @ W^T, the
 * convention of [mtp_head.rs] `MtpHead::gemv` and [prefill.rs]) is stored as
 *   codes [N][K/2]  u8, two E2M1 codes per byte, even k in the low nibble;
 *   scales[N][K/16] u8, one E4M3FN scale per 16 consecutive k of a row,
 *                   row-major, no swizzle (bytes 0x7F/0xFF are invalid);
 *   global          one nvfp4_global, dequantized value
 *                   W^[n][k] = e2m1(code) * e4m3(scale) * global.dec.
 */
#ifndef NVFP4_MTP_H
#define NVFP4_MTP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Per-matrix global scale, 16 bytes, device resident.  Written by
 * nvfp4_quantize: amax = max |W|, enc = 2688 / amax (0 if amax == 0, at most
 * FLT_MAX), dec = amax / 2688 (2688 = 6 * 448, the largest E2M1 value times
 * the largest E4M3 value).  flags is reserved (written 0). */
typedef struct nvfp4_global {
    float dec;
    float enc;
    float amax;
    uint32_t flags;
} nvfp4_global;

/* Host-side descriptor of one NVFP4 matrix W[n][k] (device pointers inside).
 * codes must be 16-byte aligned, scales 2-byte aligned, global 4-byte
 * aligned; k % 32 == 0; n >= 0. */
typedef struct nvfp4_weight {
    const uint8_t *codes;         /* [n][k/2]  */
    const uint8_t *scales;        /* [n][k/16] */
    const nvfp4_global *global;   /* one struct */
    int32_t n;
    int32_t k;
} nvfp4_weight;

/* Host-side descriptor of a stack of NVFP4 routed experts (the NVFP4 MoE of
 * [new.rs] `MtpHead::new`: per expert a gate and an up projection
 * [inter][hidden] and a down projection [hidden][inter]).  Expert e's gate
 * codes start at gate_codes + e * inter * hidden / 2, its scales at
 * gate_scales + e * inter * hidden / 16, its global at gate_global[e]; the
 * same for up; down uses [hidden][inter] per expert. */
typedef struct nvfp4_moe_weights {
    int32_t num_experts;   /* E, 1..1024            */
    int32_t hidden;        /* H, % 32 == 0          */
    int32_t inter;         /* I, % 32 == 0          */
    const uint8_t *gate_codes, *gate_scales;
    const nvfp4_global *gate_global;
    const uint8_t *up_codes, *up_scales;
    const nvfp4_global *up_global;
    const uint8_t *down_codes, *down_scales;
    const nvfp4_global *down_global;
} nvfp4_moe_weights;

enum {
    NVFP4_OK = 0,
    NVFP4_ERR_ARG = -1,         /* null pointer or out-of-range scalar    */
    NVFP4_ERR_SHAPE = -2,       /* k % 32 != 0, m out of range, ...       */
    NVFP4_ERR_ALIGN = -3,       /* a pointer misses its alignment         */
    NVFP4_ERR_WORKSPACE = -4,   /* workspace missing or too small         */
    NVFP4_ERR_UNSUPPORTED = -5, /* shape the kernels do not handle        */
    NVFP4_ERR_HIP = -6,         /* kernel launch failed (message has why) */
    NVFP4_ERR_DEVICE = -7       /* a kernel reported a failure (workspace status) */
};

enum { NVFP4_OUT_F32 = 0, NVFP4_OUT_BF16 = 1 };

/* Bit 0 of lmhead_gemv_argmax's flags: compare bf16-rounded logits. */
#define NVFP4_ARGMAX_BF16_KEYS 1u

/*
 * nvfp4_quantize -- the two quantizer passes [new.rs] resolves in
 * `MtpHead::new` as `nvfp4_global_absmax` and `quantize_bf16_to_nvfp4` and
 * applies to every projection, router and expert matrix (`quantize_proj` in
 * [mtp_head.rs]).
 *   w_bf16  [n][k] bf16, row-major, 16-byte aligned; finite values (with a
 *           NaN or Inf the outputs are unspecified, nothing faults).
 *   codes   out [n][k/2] (16-byte aligned); scales out [n][k/16] (2-byte
 *           aligned); global out (one struct, 16-byte aligned).
 * Pass 1: amax = max |w|.  Pass 2, per 16-element block of a row:
 *   scale = E4M3_rne_sat(fl(fl(bmax * enc) / 6)), sf = its value;
 *   inv = sf > 0 ? min(fl(enc / sf), FLT_MAX) : 0;
 *   code = E2M1 nearest to fl(w * inv), ties to the even code, saturating
 *   at 6, sign = sign of the product.
 * Requires n >= 1, k >= 32, k % 32 == 0, n * k < 2^40.  Three launches
 * (clear, absmax, encode); no workspace.
 */
int nvfp4_quantize(const uint16_t *w_bf16, int32_t n, int32_t k, uint8_t *codes,
                   uint8_t *scales, nvfp4_global *global, void *stream);

/*
 * w4a16_gemv -- decode-row W4A16 GEMV, y[m][n] = sum_k x[m][k] * W^[n][k]
 * ([mtp_head.rs] `MtpHead::gemv` -> `w4a16_decode_gemv`; its doc of the
 * batched-M tiers: one pass over the weight serves all M rows).
 *   x_bf16  [m][w->k] bf16, 16-byte aligned; m in 1..8.
 *   y       [m][w->n], fp32 (y_dtype NVFP4_OUT_F32) or bf16 rounded to
 *           nearest-even from the fp32 sum (NVFP4_OUT_BF16); 4-byte aligned.
 * fp32 accumulation; one pass over codes and scales; one launch.  The
 * activations are staged in LDS: when round_up_pow2(m) * k * 2 exceeds
 * 155648 bytes the rows go in groups of the most that fit, one pass and
 * one launch per group (k * 2 <= 155648 is required).  Large weights
 * (enough 4-, 8- or 16-row units for every wavefront of the device) run on
 * the persistent streaming grid of lmhead_gemv_argmax with plain outputs;
 * either way each output is one fp32 sum.
 */
int w4a16_gemv(const uint16_t *x_bf16, int32_t m, const nvfp4_weight *w, void *y,
               int32_t y_dtype, void *stream);

/*
 * w4a16_gemv_grouped -- the same GEMV for `count` weights that share K and
 * the activations, in one launch: y[i][m][w[i]->n] = x * W^_i transposed,
 * for i < count.  The head's q, k and v projections read one normed hidden
 * state, as do an FFN's gate and up ([new.rs] `MtpHead::new` resolves the
 * `w4a16_gemv_qg` and dual `w4a16_gemv_fused` kernels next to the plain
 * GEMV; [prefill_weights.rs] installs a fused [q|k|v] weight for prefill).
 *   w       host array of `count` descriptors (1 <= count <= 8), all with the
 *           same k; a descriptor with n == 0 contributes nothing and its
 *           output pointer is not read.
 *   y       host array of `count` device pointers, each [m][w[i]->n] of
 *           y_dtype, 4-byte aligned.
 * Each output is the fp32-accumulated product of w4a16_gemv; the order of
 * the fp32 partial sums can differ from a call for that weight alone (the
 * tile shape is chosen for the summed row count).  Outputs must not
 * overlap.  Errors as w4a16_gemv, plus NVFP4_ERR_ARG for a bad
 * count or NULL arrays and NVFP4_ERR_SHAPE for mismatched k.
 */
int w4a16_gemv_grouped(const uint16_t *x_bf16, int32_t m, const nvfp4_weight *const *w,
                       void *const *y, int32_t count, int32_t y_dtype, void *stream);

/*
 * w4a16_gemm_m128 -- W4A16 GEMM for prompt-sized row counts, the
 * `w4a16_gemm_m128_dispatch` of [prefill.rs] in its lossless form (NVFP4 ->
 * bf16 dequantization, bf16 matrix products, fp32 accumulation; activations
 * are never quantized).  y[m][n] = sum_k x[m][k] * W^[n][k].
 *   x_bf16     [m][w->k] bf16, 16-byte aligned; m >= 1 (any m; work is tiled
 *              in 128- or 256-row blocks, a ragged last block is masked).
 *   y          [m][w->n] fp32 or bf16 (y_dtype), 4-byte aligned.
 *   workspace  NULL, or 16-byte aligned device scratch of at least
 *              w4a16_gemm_m128_workspace_bytes(m, w->n, w->k) bytes.  When
 *              the output tiles are too few to fill the device, or a last
 *              round of them would leave most of it idle, K of those tiles
 *              is cut into slices whose fp32 partial sums go to the
 *              workspace and are added in slice order by a second kernel
 *              (the same order on every call).  NULL: one pass over K.
 *              Nothing needs to be initialised; calls that overlap on one
 *              workspace race.
 * Any n >= 0; rows and columns outside the tiles are masked.  Errors:
 * NVFP4_ERR_WORKSPACE for a non-NULL workspace below the size needed, and
 * those of w4a16_gemv.
 */
size_t w4a16_gemm_m128_workspace_bytes(int32_t m, int32_t n, int32_t k);
int w4a16_gemm_m128(const uint16_t *x_bf16, int32_t m, const nvfp4_weight *w, void *y,
                    int32_t y_dtype, void *workspace, size_t ws_bytes, void *stream);

/*
 * lmhead_gemv_argmax -- LM-head GEMV over the first V vocabulary rows fused
 * with argmax: the draft-token selection of [v4_mtp.rs] `forward_one` (LM
 * head, then argmax) and of the NVFP4 LM head of [new.rs], with the reduced
 * vocabulary of [new.rs] / [v4_mtp.rs] (V = min(vocab_rows, w->n), 0 = all).
 * No logits tensor is written.
 *   h_bf16   [m][w->k] bf16, 16-byte aligned; m in 1..8.
 *   out_idx  [m] int32: the lowest index i < V whose key is the maximum,
 *            where key = logit (fp32), or the logit rounded to bf16 when
 *            flags & NVFP4_ARGMAX_BF16_KEYS.  The selection follows the
 *            ascending strict-greater scan of [v4_mtp.rs]
 *            `argmax_grammar_masked`: NaN never wins, -0 == +0, and if no
 *            key exceeds -inf the index is 0.
 *   out_max  [m] fp32: the fp32 logit of the selected row.
 *   workspace device scratch of at least
 *            lmhead_gemv_argmax_workspace_bytes(m, V) bytes (V = the number
 *            of rows scored), 256-byte aligned.  It holds a ticket counter
 *            and per-row packed maxima that must be zero before the first
 *            call (zero-fill the buffer once); each call returns them to
 *            zero (and lmhead_gemv_argmax_fc's call count, which only
 *            advances).  A workspace serves one call at a time: calls that
 *            overlap on one workspace race, and can leave the ticket off
 *            zero, which makes later calls wrong; zero-fill it again after
 *            such an overlap.
 * Rows with equal codes and scales produce bit-identical logits.  One launch.
 */
size_t lmhead_gemv_argmax_workspace_bytes(int32_t m, int32_t vocab_rows);
int lmhead_gemv_argmax(const uint16_t *h_bf16, int32_t m, const nvfp4_weight *w,
                       int32_t vocab_rows, int32_t *out_idx, float *out_max, void *workspace,
                       size_t ws_bytes, uint32_t flags, void *stream);

/*
 * lmhead_gemv_argmax_noalloc -- lmhead_gemv_argmax for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation): the same kernels and results, with the
 * workspace in a static array of the library, one copy of
 * NVFP4_NOALLOC_SCRATCH_BYTES per device, held until the process ends.  The
 * first call on a device looks the array up and clears its counters (a
 * kernel on `stream`); every call returns them to zero.  All calls on one
 * device share the array: calls that overlap on a device race (one at a
 * time per device, as with one workspace).  The grid is the device's
 * resident LM-head workgroups, each with m partials of 32 bytes; a grid
 * whose 512 + 32 * round_up(m) * workgroups bytes exceed the array is
 * refused with NVFP4_ERR_WORKSPACE (256 CUs need at most 131,584 bytes).
 * Allocates nothing (no hipMalloc, no allocating library routine).
 * Arguments, outputs and the other errors as lmhead_gemv_argmax.
 */
#define NVFP4_NOALLOC_SCRATCH_BYTES (1u << 20)
int lmhead_gemv_argmax_noalloc(const uint16_t *h_bf16, int32_t m, const nvfp4_weight *w,
                               int32_t vocab_rows, int32_t *out_idx, float *out_max, uint32_t flags,
                               void *stream);

/*
 * lmhead_gemv_argmax_logprob -- lmhead_gemv_argmax that also returns, per
 * activation row, the top-1 log-probability of the selected token: the
 * batched argmax of [mtp_head.rs] (`MtpHead` fields) that writes each row's
 * top-1 log-probability for the draft confidence stop.  In the same pass over
 * the weights (no extra bytes read) each slot keeps an online log-sum-exp of
 * the keys, merged with the argmax partials:
 *   out_logprob[i] = key[out_idx[i]] - log(sum over r < V of exp(key[r]))
 * in fp32, with the keys of lmhead_gemv_argmax (fp32 logits, or their bf16
 * rounding with NVFP4_ARGMAX_BF16_KEYS).  A NaN or +inf key, or a vocabulary
 * whose keys are all -inf, gives NaN.  All other arguments, the workspace
 * (the same size) and the errors as lmhead_gemv_argmax; out_logprob [m] fp32,
 * 4-byte aligned, must not be NULL.  One launch.
 */
int lmhead_gemv_argmax_logprob(const uint16_t *h_bf16, int32_t m, const nvfp4_weight *w,
                               int32_t vocab_rows, int32_t *out_idx, float *out_max,
                               float *out_logprob, void *workspace, size_t ws_bytes,
                               uint32_t flags, void *stream);

/*
 * lmhead_gemv_argmax_masked -- lmhead_gemv_argmax restricted to the tokens a
 * grammar allows: the device-side form of the masked argmax of [v4_mtp.rs]
 * `argmax_grammar_masked`, which needs no logits readback.
 *   allow_mask    device uint32 [m][mask_words]: token r is allowed for
 *                 activation row i when bit r % 32 of word r / 32 of row i is
 *                 set; tokens past the mask are not allowed.  4-byte aligned.
 *   out_logprob   NULL, or [m] fp32: the top-1 log-probability over the
 *                 allowed tokens (key[idx] minus the log-sum-exp of the
 *                 allowed keys); NaN when no allowed key has finite mass.
 * A disallowed token is scored as a -inf key, so the scan of
 * lmhead_gemv_argmax applies: the lowest-index maximum among the allowed
 * tokens, and index 0 (with row 0's logit in out_max) when nothing allowed
 * exceeds -inf, including an empty allowed set -- the pad draft of the scan.
 * Workspace, errors and the other arguments as lmhead_gemv_argmax.  One
 * launch; the mask word of each 32-row tile is loaded with its weights.
 */
int lmhead_gemv_argmax_masked(const uint16_t *h_bf16, int32_t m, const nvfp4_weight *w,
                              int32_t vocab_rows, const uint32_t *allow_mask, int32_t mask_words,
                              int32_t *out_idx, float *out_max, float *out_logprob,
                              void *workspace, size_t ws_bytes, uint32_t flags, void *stream);

/*
 * lmhead_gemv_argmax_fc -- the end of one draft step and the start of the
 * next: lmhead_gemv_argmax, then the next step's fc over the chosen
 * tokens' embedding rows, y = w4a16_gemv_embed(out_idx, table, x_rest, fc)
 * ([v4_mtp.rs] `propose` feeds each draft into the next step's input;
 * [mtp_head.rs] `MtpHead` fields: `embed_from_argmax`, the fc).
 *   h_bf16 ... flags          as lmhead_gemv_argmax (out_idx, out_max are
 *                             its outputs, bit for bit).
 *   table_bf16, table_vocab, hidden, x_rest_bf16, fc, y, y_dtype
 *                             as w4a16_gemv_embed with idx = out_idx.
 * At one row with K = 2048 and an fc of k = 2048 or 4096, and when the LM
 * head's grid can take every fc row (wavefronts 1..7 of each workgroup, two
 * rows each: 14 rows a workgroup, 3584 on 256 CUs), one launch: the
 * LM head's workgroups load their fc rows while its end chain runs, wait
 * (bounded, about a second) for the last workgroup to publish the id in the
 * workspace, gather its embedding row and finish the fc.  y then sums each
 * row in another order than w4a16_gemv_embed (equal up to fp32 rounding;
 * bit for bit on exactly representable sums), and is NaN if that wait gave
 * up.  The whole grid must be resident at once (the persistent LM-head grid
 * is sized so).  Otherwise the two calls, in order.  The workspace is
 * lmhead_gemv_argmax's; every call advances a count in it.
 */
int lmhead_gemv_argmax_fc(const uint16_t *h_bf16, int32_t m, const nvfp4_weight *w, int32_t vocab_rows,
                          int32_t *out_idx, float *out_max, void *workspace, size_t ws_bytes, uint32_t flags,
                          const uint16_t *table_bf16, int32_t table_vocab, int32_t hidden,
                          const uint16_t *x_rest_bf16, const nvfp4_weight *fc, void *y, int32_t y_dtype,
                          void *stream);

/*
 * embed_from_argmax -- the draft tokens' embedding rows, gathered on the
 * device: the `embed_from_argmax` step of [mtp_head.rs] (`MtpHead` fields),
 * which feeds the next draft step and stores the draft id in device memory
 * for deferred readback, so that a chain of draft steps needs no host round
 * trip ([v4_mtp.rs] `propose` feeds each draft into the next step).
 *   idx         device int32 [m] (e.g. out_idx of lmhead_gemv_argmax).
 *   table_bf16  device bf16 [vocab][hidden], 16-byte aligned; hidden % 8 == 0.
 *   out_bf16    device bf16, row i at out_bf16 + i * out_stride (elements;
 *               out_stride >= hidden, a multiple of 8), 16-byte aligned --
 *               e.g. the first half of the next step's fc input row.
 *   id_log      NULL, or device int32 [m]: receives idx (the chain's record).
 * An index outside [0, vocab) gives a zero row (id_log still records it).
 * m == 0 does nothing.  One launch.
 */
int embed_from_argmax(const int32_t *idx, int32_t m, const uint16_t *table_bf16, int32_t vocab,
                      int32_t hidden, uint16_t *out_bf16, int64_t out_stride, int32_t *id_log,
                      void *stream);

/*
 * lmhead_gemv_argmax_embed -- the LM head's argmax with the embedding gather
 * of the selected tokens done by its last workgroup: one launch for the tail
 * of a draft step and the head of the next (the gather of embed_from_argmax
 * without a kernel boundary or a second read of the index).
 *   allow_mask, mask_words   as lmhead_gemv_argmax_masked, or NULL / 0.
 *   out_logprob              NULL, or as lmhead_gemv_argmax_logprob.
 *   table_bf16, table_vocab, hidden, out_embed, out_stride, id_log
 *                            as embed_from_argmax (table_vocab may differ
 *                            from the head's rows; hidden % 8 == 0).
 * out_idx, out_max, the workspace and the errors as lmhead_gemv_argmax.
 */
int lmhead_gemv_argmax_embed(const uint16_t *h_bf16, int32_t m, const nvfp4_weight *w,
                             int32_t vocab_rows, const uint32_t *allow_mask, int32_t mask_words,
                             int32_t *out_idx, float *out_max, float *out_logprob,
                             const uint16_t *table_bf16, int32_t table_vocab, int32_t hidden,
                             uint16_t *out_embed, int64_t out_stride, int32_t *id_log,
                             void *workspace, size_t ws_bytes, uint32_t flags, void *stream);

/*
 * w4a16_gemv_embed -- w4a16_gemv whose activation rows begin with the
 * embedding rows of the tokens in idx, read by the GEMV itself: the next
 * draft step's fc over [embed(draft token) | hidden state] with the gather of
 * embed_from_argmax ([mtp_head.rs] `MtpHead` fields; [v4_mtp.rs] `propose`
 * feeds each draft into the next step) folded into its activation loads, so
 * the embedding row is fetched while the weights stream and no kernel
 * writes it.  Activation row i, element kk: table[idx[i]][kk] for kk <
 * hidden (a zero row for an id outside [0, table_vocab)), x_rest[i][kk -
 * hidden] for kk >= hidden.
 *   idx          device int32 [m] (e.g. out_idx of lmhead_gemv_argmax).
 *   table_bf16   device bf16 [table_vocab][hidden], 16-byte aligned;
 *                hidden a positive multiple of 32, at most w->k.
 *   x_rest_bf16  device bf16 [m][w->k - hidden], 16-byte aligned (NULL
 *                when hidden == w->k).
 *   m, w, y, y_dtype, stream, the kernels and the other errors as
 *                w4a16_gemv; the result equals w4a16_gemv of the
 *                concatenated rows bit for bit.
 */
int w4a16_gemv_embed(const int32_t *idx, const uint16_t *table_bf16, int32_t table_vocab,
                     int32_t hidden, const uint16_t *x_rest_bf16, int32_t m, const nvfp4_weight *w,
                     void *y, int32_t y_dtype, void *stream);

/*
 * moe_w4a16_gemv -- routed-expert MoE FFN for decode rows: the
 * `moe_topk_softmax` -> `moe_silu_mul` -> weighted-sum chain named in
 * [new.rs] `MtpHead::new`, on NVFP4 experts.
 *   x_bf16         [m][H] bf16, 16-byte aligned; m in 1..8.
 *   router_logits  [m][E] fp32 (the router projection's output).
 *   top_k          1..min(E, 16).
 *   y              out [m][H] fp32: sum_j w[j] * down_e(j)(a_j), summed
 *                  in fp32 in an order fixed by the routing (the same
 *                  inputs give the same bits).
 *   topk_ids       out [m][top_k] int32: experts by descending logit, the
 *                  lower id first among equal logits.
 *   topk_w         out [m][top_k] fp32: softmax over the selected logits.
 *   workspace      at least moe_w4a16_gemv_workspace_bytes(m, top_k, e),
 *                  256-byte aligned, zero-filled before its first use (it
 *                  holds ticket and column counters, which every call
 *                  returns to zero, per-call tagged hand-off words and a
 *                  sticky status word: see moe_workspace_status).  One
 *                  call at a time per workspace.
 * Per selected expert: g = gate x, u = up x (fp32),
 * a = bf16_rne(silu(g) * u), d = down a (fp32).  The gate/up weights are
 * read once per (row, slot) pair, the down weights once per distinct expert.
 * Requires H, I % 32 == 0
 * and round_up(m, 1|2|4|8) * max(H, I) * 2 <= 159744 bytes of LDS (H up to
 * 9984 at m = 8); NVFP4_ERR_UNSUPPORTED otherwise.  One launch at one
 * token when the down pass's activation rows fit in LDS and the whole grid
 * is resident at once (decode at the usual shapes); else gate/up (with the
 * routing), then the down pass with the combine.
 */
size_t moe_w4a16_gemv_workspace_bytes(int32_t m, int32_t top_k, const nvfp4_moe_weights *e);
int moe_w4a16_gemv(const uint16_t *x_bf16, int32_t m, const float *router_logits,
                   int32_t top_k, const nvfp4_moe_weights *e, float *y, int32_t *topk_ids,
                   float *topk_w, void *workspace, size_t ws_bytes, void *stream);

/*
 * moe_w4a16_gemv_trace -- moe_w4a16_gemv in its one-launch form with phase
 * timestamps, for profiling the one-token latency chain; the outputs are
 * those of moe_w4a16_gemv bit for bit.  Not a second computation: the same
 * kernel, given a trace buffer.
 *   m              1 (NVFP4_ERR_UNSUPPORTED otherwise, and when the call
 *                  would not take the one-launch form).
 *   trace          device uint64[trace_words], 8-byte aligned, at least
 *                  moe_w4a16_gemv_trace_words(m, top_k, e) words (0 when m
 *                  != 1); out: event ev of workgroup b at trace[ev * G + b],
 *                  G = ceil(I / 16) * top_k gate/up workgroups followed by
 *                  ceil(H / 8) down workgroups, each the GPU's 100 MHz
 *                  constant clock (s_memrealtime) read by the workgroup's
 *                  first thread.  Gate/up events: 0 start, 1 routing done,
 *                  2 activations stored, 3 counted in its column (the last
 *                  of a column: after issuing the release).  Down events:
 *                  0 start, 1 weight loads issued, 2 go word seen,
 *                  3 activations staged, 4 sums done, 5 output written.
 *                  Unused slots are left as they were.
 *   the other arguments and errors as moe_w4a16_gemv.
 */
size_t moe_w4a16_gemv_trace_words(int32_t m, int32_t top_k, const nvfp4_moe_weights *e);
int moe_w4a16_gemv_trace(const uint16_t *x_bf16, int32_t m, const float *router_logits,
                         int32_t top_k, const nvfp4_moe_weights *e, float *y, int32_t *topk_ids,
                         float *topk_w, void *workspace, size_t ws_bytes, uint64_t *trace,
                         size_t trace_words, void *stream);

/*
 * moe_layer_w4a16 -- the complete MoE layer of the draft head: the NVFP4
 * router (`moe_gate`, quantized next to the experts in [new.rs]
 * `MtpHead::new`), the routed experts of moe_w4a16_gemv and the shared
 * expert with its sigmoid `shared_expert_gate`, blended as the pages'
 * `moe_weighted_sum_blend`:
 *   router_logits = router x  (fp32 out [m][E]),
 *   y = sum_j w[j] * down_e(j)(a_j) + sigmoid(g . x) * down_s(a_s),
 *   a_s = bf16(silu(gate_s x) * up_s x),
 * with g = shared_gate_w_bf16 ([H] bf16) or, when it is NULL, a factor 1.
 *   router        [E][H] NVFP4 (n = num_experts, k = hidden).
 *   shared_gate, shared_up   [I][H] NVFP4; shared_down [H][I] NVFP4 (the
 *                 routed experts' width I).
 *   y, topk_ids, topk_w      as moe_w4a16_gemv.
 *   workspace     at least moe_layer_w4a16_workspace_bytes(m, top_k, e),
 *                 256-byte aligned, zero-filled before its first use.
 * Three launches: one grouped GEMV (router, shared gate, shared up), the
 * routing with the routed gate/up and the shared activations, and the down
 * pass over the routed experts and the shared one.  Requires, besides the
 * limits of moe_w4a16_gemv, (m * top_k + m) * I * 2 <= 153600 bytes (the
 * activation rows the down pass keeps in LDS); NVFP4_ERR_UNSUPPORTED
 * otherwise.
 */
size_t moe_layer_w4a16_workspace_bytes(int32_t m, int32_t top_k, const nvfp4_moe_weights *e);
int moe_layer_w4a16(const uint16_t *x_bf16, int32_t m, const nvfp4_weight *router, int32_t top_k,
                    const nvfp4_moe_weights *e, const nvfp4_weight *shared_gate,
                    const nvfp4_weight *shared_up, const nvfp4_weight *shared_down,
                    const uint16_t *shared_gate_w_bf16, float *y, int32_t *topk_ids, float *topk_w,
                    float *router_logits, void *workspace, size_t ws_bytes, void *stream);

/*
 * moe_workspace_status -- reads and clears the sticky status word of a
 * moe_w4a16_gemv / moe_layer_w4a16 workspace.  In the one-launch path the
 * down workgroups wait (bounded, about a second) for the gate/up workgroups
 * of the same launch, released through per-workgroup go words that carry
 * a per-call tag (a release left over from an earlier call never satisfies
 * a later wait).  If a wait gives up, or a go word holds a value no call
 * writes (the workspace was overwritten), that down workgroup writes NaN
 * rows into y and sets bit 0 (timeout) or bit 1 (overwritten) of this
 * word; the call itself has already returned NVFP4_OK.
 *   workspace  the MoE workspace (device), ws_bytes its size.
 *   status     host uint32: receives the bits (0 after clean calls).
 * Synchronizes `stream` (not allowed during graph capture:
 * NVFP4_ERR_UNSUPPORTED).  Returns NVFP4_OK when no bit was set, else
 * NVFP4_ERR_DEVICE with the reason in nvfp4_mtp_last_error(); an
 * overwritten workspace must be zero-filled again before its next use.
 */
int moe_workspace_status(void *workspace, size_t ws_bytes, uint32_t *status, void *stream);

/* Message of the last failing call on this host thread ("" if none); the
 * pointer stays valid until the next call on the same thread. */
const char *nvfp4_mtp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_MTP_H */
