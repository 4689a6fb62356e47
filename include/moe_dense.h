/*
 * moe_dense.h -- C ABI of the decoder's two dense ends in libmoe.so, for a
 * few tokens at a time (decode): the lm_head projection with greedy token
 * selection, and the dense SwiGLU MLP of layer 0.
 *
 * Sources: browser demo page "A 3-billion-parameter OCR model. In this tab.",
 * "One forward pass, left to right": step 6 (layer 0 of the DeepSeek-V2
 * decoder is a dense SwiGLU MLP; layers 1-11 are the MoE layers of moe.h) and
 * step 7 (the final RMSNorm feeds an lm_head GEMV from 1,280 to 129,280
 * logits; decoding is greedy).  franken_ocr README, "Architecture" (the same
 * structure, vocabulary 129280) and "CPU Backend and Optimizations"
 * (quantisation policy: the dense layer-0 MLP is quantised with the expert
 * matrices; lm_head stays at source precision unless the experimental int8
 * gate is armed, see the environment-variable table).
 *
 * Readings where the pages are silent: the dense MLP's intermediate size is
 * 6848 (the pages' model-specific K = 6848 int8 GEMM case is the reduction
 * length of its down projection); its codes use the experts' format (int8 or
 * int4 two's complement, one f32 scale per group along K); greedy decoding
 * returns the lowest token id among equal largest logits.
 *
 * Conventions are those of moe.h (status codes, stream order, caller-owned
 * buffers, validation before anything is enqueued).  Weights here are plain
 * row-major matrices, no repacking:
 *   - lm_head: [vocab][1280] bf16 (16-bit patterns) or int8 codes, with
 *     [vocab][1280 / group] f32 scales for int8;
 *   - dense MLP codes, one buffer: gate [inter][1280] | up [inter][1280] |
 *     down [1280][inter]; int8 one code per byte, int4 two codes per byte
 *     (element 2j in the low nibble); scales, one buffer:
 *     gate [inter][1280 / group] | up [inter][1280 / group] |
 *     down [1280][inter / group] f32.
 * These GEMV paths take at most MOE_DENSE_MAX_TOKENS tokens per call.
 */
#ifndef MOE_DENSE_H
#define MOE_DENSE_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_VOCAB 129280
#define MOE_DENSE_INTER 6848
#define MOE_DENSE_MAX_TOKENS 4
#define MOE_DENSE_MAX_INTER 8192
#define MOE_HEAD_MAX_VOCAB 1048576

/* lm_head weight storage (the w_bits argument) */
enum { MOE_HEAD_INT8 = 8, MOE_HEAD_BF16 = 16 };

/* Workspace bytes of moe_lm_head_argmax for n_tokens tokens and a vocabulary
   of `vocab` rows (0 for arguments out of range). */
size_t moe_lm_head_workspace_bytes(int32_t n_tokens, int32_t vocab);

/*
 * lm_head + greedy token (demo page step 7).
 *   h           [n_tokens][1280] f32 device: final residual stream rows.
 *   flags       MOE_NORM_INPUT: the logits use z = RMSNorm(h) (eps 1e-6, no
 *               gain: the decoder's final norm); 0: z = h.
 *   w, w_bits   lm_head weights, MOE_HEAD_BF16 or MOE_HEAD_INT8 (16-byte aligned).
 *   w_scales    int8 only: [vocab][1280 / group] f32; group in {32, 64, 128}.
 *   logits      optional [n_tokens][vocab] f32 output (NULL: not stored).
 *   token       [n_tokens] int32 output: argmax over the vocabulary of
 *               sum_k W[v][k] z[k], the lowest id among equal maxima.
 *   token_logit [n_tokens] f32 output: that largest logit.
 * Arithmetic: f32 products and sums in a fixed order (bitwise reproducible).
 * n_tokens in [0, MOE_DENSE_MAX_TOKENS] (0 enqueues nothing); vocab in
 * [1, MOE_HEAD_MAX_VOCAB].
 */
moe_status_t moe_lm_head_argmax(const float* h, int32_t n_tokens, uint32_t flags,
                                const void* w, int32_t w_bits, const float* w_scales, int32_t group,
                                int32_t vocab, float* logits, int32_t* token, float* token_logit,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the dense MLP's code buffer for (bits, inter): 3 * inter * 1280 *
   bits / 8 (0 for arguments out of range). */
size_t moe_dense_ffn_code_bytes(int32_t bits, int32_t inter);

/*
 * Dense MLP weight codes into the one code buffer moe_dense_ffn_forward takes
 * (host memory in, host memory out; no GPU involved).
 *   gate, up    [inter][1280] int8, one signed code per byte, row-major;
 *   down        [1280][inter] int8, likewise;
 *   bits        8: the codes are copied as bytes; 4: codes must lie in
 *               [-8, 7] and two consecutive codes of a row share a byte,
 *               element 2j in the low nibble (two's complement);
 *   codes_out   moe_dense_ffn_code_bytes(bits, inter) bytes, gate | up | down.
 * Returns MOE_E_NULLPTR for a missing pointer, MOE_E_SHAPE for an inter the
 * forward call rejects, MOE_E_FORMAT for bits not in {4, 8} or an int4 code
 * out of range (nothing is written then).  The scales need no packing: they
 * are the plain concatenation gate | up | down of [rows][K / group] f32.
 */
moe_status_t moe_pack_dense_ffn(const int8_t* gate, const int8_t* up, const int8_t* down, int32_t bits,
                                int32_t inter, void* codes_out);

/* Workspace bytes of moe_dense_ffn_forward (0 for arguments out of range). */
size_t moe_dense_ffn_workspace_bytes(int32_t n_tokens, int32_t inter);

/*
 * Dense SwiGLU MLP (layer 0 of the decoder, demo page step 6):
 *   y (+)= W_d (SiLU(W_g z) * (W_u z)),  z = RMSNorm(x) with MOE_NORM_INPUT, else x.
 *   x       [n_tokens][1280] f32 device.
 *   codes, scales, bits, group, inter: the layout in the header comment;
 *           bits in {4, 8}, group in {32, 64, 128} dividing inter, inter a
 *           multiple of 64 in [64, MOE_DENSE_MAX_INTER] (the decoder: 6848).
 *   y       [n_tokens][1280] f32 device; with MOE_ACCUMULATE it is added to
 *           (x may then be y: the in-place residual stream).
 * Flags: MOE_NORM_INPUT, MOE_ACCUMULATE (moe.h).  n_tokens in
 * [0, MOE_DENSE_MAX_TOKENS].
 */
moe_status_t moe_dense_ffn_forward(const float* x, int32_t n_tokens, const void* codes, const float* scales,
                                   int32_t bits, int32_t group, int32_t inter, float* y, uint32_t flags,
                                   void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DENSE_H */
