/*
 * moe_attn.h -- C ABI of one R-SWA attention decode step in libmoe.so.
 *
 * R-SWA (Reference Sliding Window Attention) is the decoder's attention: a
 * generated token attends, per head, to every reference token (the visual
 * prefill plus the prompt prefix, a frozen global KV that is never evicted)
 * and to the newest generated tokens through a ring-buffer KV of 128 slots,
 * so the generated-token KV stays constant in size.  Sources: franken_ocr
 * README, "Design Philosophy" ("Bounded generated-token KV") and the
 * "Bounded long-doc memory" row of the table under "Why focr?"; browser demo
 * page "A 3-billion-parameter OCR model. In this tab.", "One forward pass,
 * left to right", step 6 (ten attention heads of dimension 128).  Attention
 * stays at source precision (bf16) in the conservative recipe (README, "CPU
 * Backend and Optimizations", quantisation policy).
 *
 * Readings where the pages are silent: the new token's key and value are
 * written to ring slot n_gen mod 128 (n_gen = tokens generated before it)
 * before it attends, so it sees min(n_gen + 1, 128) generated tokens, itself
 * included; scores are q.k / sqrt(128) under a plain softmax over the
 * reference keys and the live ring slots; q, k and v arrive after any
 * positional transform (the pages describe none, and none is applied); the
 * KV is bf16 (the new key and value are rounded to nearest, ties to even).
 *
 * Conventions are those of moe.h.  Streams are independent (the continuous
 * batch spine); all streams of one call share the reference length n_ref.
 */
#ifndef MOE_ATTN_H
#define MOE_ATTN_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_HEADS 10
#define MOE_HEAD_DIM 128
#define MOE_RSWA_WINDOW 128
#define MOE_RSWA_MAX_STREAMS 4096
#define MOE_RSWA_MAX_REF 65536

/* Workspace bytes of moe_rswa_decode (0 for arguments out of range). */
size_t moe_rswa_workspace_bytes(int32_t n_streams, int32_t n_ref);

/*
 * One decode step of n_streams streams, all device pointers:
 *   q, k_new, v_new  [S][10][128] f32: the new token's query, key and value.
 *   ref_k, ref_v     [S][10][n_ref][128] bf16 bit patterns: the frozen block.
 *   ring_k, ring_v   [S][10][128][128] bf16 bit patterns, updated in place:
 *                    slot n_gen[s] mod 128 receives the new key and value.
 *   n_gen            [S] int32: tokens each stream generated before this one
 *                    (slots 0 .. min(n_gen, 127) are live; negative reads as 0).
 *   out              [S][10][128] f32: softmax(q k / sqrt(128)) v per head.
 * Arithmetic in f32 with a fixed order (bitwise reproducible).
 * n_streams in [0, MOE_RSWA_MAX_STREAMS] (0 enqueues nothing), n_ref in
 * [0, MOE_RSWA_MAX_REF].  Pointers 16-byte aligned (n_gen 4-byte).
 */
moe_status_t moe_rswa_decode(int32_t n_streams, int32_t n_ref, const float* q, const float* k_new,
                             const float* v_new, const void* ref_k, const void* ref_v, void* ring_k, void* ring_v,
                             const int32_t* n_gen, float* out, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * The attention half of a decoder layer for n_streams streams (the layer's
 * MoE half is moe_layer_forward with MOE_NORM_INPUT | MOE_ACCUMULATE, or
 * moe_decode_forward): browser demo page "One forward pass, left to right",
 * step 6 (R-SWA attention of ten heads of 128, then the MoE FFN); model card
 * "The rest of the pipeline" (plain multi-head attention).
 *   z = RMSNorm(h) (no gain, eps 1e-6 inside the root)
 *   q = W_q z, k = W_k z, v = W_v z        (1280 -> 1280 each)
 *   a = the R-SWA step of moe_rswa_decode on q, k, v (ring updated in place)
 *   h = h + W_o a                          (in place)
 * h        [S][1280] f32, device, read and updated in place.
 * w_qkv    [3840][1280] bf16 bit patterns, device: rows 0..1279 W_q,
 *          1280..2559 W_k, 2560..3839 W_v (y = W x: row n gives output n).
 * w_o      [1280][1280] bf16 bit patterns, device.
 * ref_k, ref_v, ring_k, ring_v, n_gen: as for moe_rswa_decode.
 * workspace >= moe_attn_block_workspace_bytes(n_streams, n_ref) bytes,
 *          16-byte aligned; garbage before and after the call.
 * No bias and no positional transform (the pages name none).  Projections
 * multiply bf16 weights with the f32 activations split into two bf16 halves
 * (16 significant bits) on the matrix cores, fp32 accumulation.
 * n_streams in [0, MOE_RSWA_MAX_STREAMS] (0 enqueues nothing, and h, the KV
 * and n_gen may then be NULL); errors as for moe_rswa_decode.  Stream ordered; the persistent decode step
 * (moe_decode_forward) takes every compute unit, so the two are enqueued one
 * after the other on one stream, never concurrently.
 */
size_t moe_attn_block_workspace_bytes(int32_t n_streams, int32_t n_ref);
moe_status_t moe_attn_block_forward(int32_t n_streams, int32_t n_ref, float* h, const void* w_qkv, const void* w_o,
                                    const void* ref_k, const void* ref_v, void* ring_k, void* ring_v,
                                    const int32_t* n_gen, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ATTN_H */
