/*
 * moe.h -- C ABI of the quantized expert-FFN MoE layer library (libmoe.so).
 *
 * The layer is the mixture-of-experts FFN of the Unlimited-OCR DeepSeek-V2
 * decoder: hidden 1280, a softmax router over 64 routed experts, the top 6
 * picked greedily with no renormalisation, SiLU-gated (SwiGLU) experts of
 * intermediate 896, and two always-on shared experts fused into one SwiGLU of
 * intermediate 1792, all combined with the router weights.  Sources: browser
 * demo page "A 3-billion-parameter OCR model. In this tab.", section "One
 * forward pass, left to right", step 6; franken_ocr README, sections
 * "Architecture" and "Design Philosophy" (fixed dimensions: 64 experts, top-6,
 * MoE intermediate 896, hidden 1280).  Expert weights are integer codes, int4
 * two's-complement nibbles or int8, with one f32 scale per group of
 * consecutive weights along the reduction axis (demo page, section "Four bits,
 * one shared scale"; README "CPU Backend and Optimizations", quantisation
 * policy: router and norms stay high precision, so the router is f32 here).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Shapes are fixed (the MOE_* constants below); other shapes are rejected.
 * - Device pointers are plain device addresses (e.g. torch.Tensor.data_ptr()).
 *   The caller owns every buffer; the library never allocates, frees or keeps
 *   a pointer after the call returns.
 * - GPU entry points are stream ordered: they validate on the host, enqueue
 *   kernels on `stream` (a hipStream_t; NULL = the default stream) and return
 *   without synchronising.  Launch errors are reported as MOE_E_HIP.
 * - Errors are status codes, never exceptions or aborts.  All argument checks
 *   happen before anything is enqueued, so a non-OK status means nothing ran.
 * - Calls are re-entrant; concurrent calls need distinct workspaces.
 * - Activation, weight-code, router-weight and workspace pointers must be
 *   16-byte aligned; scales, bias, ids and weights 4-byte aligned
 *   (MOE_E_ALIGN otherwise).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_HIDDEN 1280
#define MOE_EXPERTS 64
#define MOE_TOPK 6
#define MOE_INTER 896
#define MOE_SHARED_INTER 1792
#define MOE_MAX_TOKENS 8192
/* Group value that, with 4-bit codes, selects the two-level (Q4_K-style)
   expert format; see moe_pack_expert_q4k. */
#define MOE_Q4K 256

typedef enum {
  MOE_OK = 0,
  MOE_E_NULLPTR = 1,   /* a required pointer is NULL */
  MOE_E_SHAPE = 2,     /* token count or intermediate size out of range */
  MOE_E_FORMAT = 3,    /* bits not in {4, 8}, group not in {32, 64, 128} (or MOE_Q4K with 4 bits),
                          or a code out of range */
  MOE_E_ALIGN = 4,     /* a device pointer is not 16-byte aligned */
  MOE_E_WORKSPACE = 5, /* workspace smaller than moe_workspace_bytes() */
  MOE_E_HIP = 6,       /* the HIP runtime reported an error while enqueueing */
  MOE_E_ARG = 7        /* any other invalid argument (dtype, flags, aliasing) */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

/* moe_layer_forward flags */
enum {
  /* y += layer(x) instead of y = layer(x): the residual add of a chained
     decoder.  x may then be the same buffer as y (in-place residual stream). */
  MOE_ACCUMULATE = 1u,
  /* The layer input is RMSNorm(x) = x / sqrt(mean(x^2) + eps) with eps =
     1e-6 and no learned gain, computed inside the call (the decoder's RMSNorm;
     demo page step 7).  Requires x in f32. */
  MOE_NORM_INPUT = 2u,
  /* With MOE_NORM_INPUT: round the normalised input to bf16 (nearest, ties to
     even) before it reaches the router and the experts. */
  MOE_NORM_BF16 = 4u,
  /* Force the per-token GEMV path (at most 64 tokens) / the grouped MFMA
     path regardless of the token count (both give the same result up to fp32
     rounding order).  Without either flag a call takes the per-token path up
     to a token count that depends on the routed format and the input type,
     the measured crossover of the two paths: 6 for 32-column groups, 12 for
     int8 codes, 16 for the two-level format, 13 for int4 G64 / G128 with a
     bf16 expert input and 18 with an f32 one; the grouped path beyond. */
  MOE_FORCE_DECODE = 8u,
  MOE_FORCE_GROUPED = 16u
};

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_str(int32_t status);

/* ------------------------------------------------------------------------
 * Weight packing (host memory in, host memory out; no GPU involved).
 *
 * Canonical input layout of one expert (routed: inter = 896; the fused
 * shared expert: inter = 1792):
 *   gate codes [inter][1280], up codes [inter][1280], down codes [1280][inter],
 *   one signed code per int8 byte, row-major, K (the reduction axis) last;
 *   scales gate [inter][1280/G], up [inter][1280/G], down [1280][inter/G] f32,
 *   scale (r, g) applying to codes (r, g*G .. g*G+G-1)  (W = scale * code,
 *   no zero point).
 * int4 codes must lie in [-8, 7]; int8 codes in [-128, 127].
 *
 * Packed layout written to codes_out (moe_expert_code_bytes() bytes):
 *   [gate | up | down]; every matrix is a sequence of 1 KiB tiles, and inside
 *   a tile lane l = 0..63 owns bytes 16l..16l+15, i.e. four 32-bit words
 *   w0..w3, with r = l % 16 and q = l / 16.  Codes are stored as two's
 *   complement (int4: one nibble; int8: one byte).
 *   gate and up ([N = inter rows][K = 1280]): tiles of 16 rows x KB columns,
 *     KB = 128 (int4) or 64 (int8), tile (nt, kb) at byte 1024*(nt*(K/KB) + kb);
 *     row 16nt + r;
 *       int4: word j = codes k = 128kb + 32j + 8q + i (i = 0..7) in nibble i;
 *       int8: word j = codes k = 64kb + 32(j/2) + 8q + 4(j%2) + i (i = 0..3)
 *             in byte i.
 *   down ([N = 1280 rows][K = inter]): tiles of DR rows x 32 columns, DR = 64
 *     (int4) or 32 (int8), tile (kc, rt) at byte 1024*(kc*(1280/DR) + rt);
 *       int4: word j = row DR*rt + 16j + r, codes k = 32kc + 8q + i in nibble i;
 *       int8: word j = row DR*rt + 16(j/2) + r, codes k = 32kc + 8q + 4(j%2) + i
 *             in byte i.
 *   (A 32-column slab of the down matrix, which is what one slice of the
 *   intermediate dimension multiplies, is contiguous.)
 * Packed scales written to scales_out (moe_expert_scale_count() floats):
 *   [gate | up | down]; gate and up keep the canonical row-major [N][K/G];
 *   down is [K/G][1280/DR][16][DR/16] with entry (g, rt, r, j) = scale of row
 *   DR*rt + 16j + r, group g.
 * Experts of a layer are concatenated: expert e at byte e * code_bytes and
 * float e * scale_count.
 * ------------------------------------------------------------------------ */
size_t moe_expert_code_bytes(int32_t bits, int32_t inter);
/* floats of packed scales per expert (group MOE_Q4K: 4-byte words of metadata) */
size_t moe_expert_scale_count(int32_t group_size, int32_t inter);
moe_status_t moe_pack_expert(const int8_t* gate, const int8_t* up, const int8_t* down,
                             const float* gate_scales, const float* up_scales,
                             const float* down_scales, int32_t inter, int32_t bits,
                             int32_t group_size, void* codes_out, float* scales_out);

/* ------------------------------------------------------------------------
 * Two-level 4-bit expert format (Q4_K-style).  The Unlimited-OCR DeepEncoder
 * ONNX model card ("The rest of the pipeline") pairs the pipeline with a
 * community K-quant GGUF of the decoder, read by the WebGPU engine's q4k
 * storage; the pages define no layout, so the K-quant definition is taken:
 * along K, super-blocks of 256 columns with f16 factors d and dmin, split
 * into 8 sub-blocks of 32 columns with 6-bit unsigned sc and m, unsigned
 * 4-bit codes q, and
 *     W[r][k] = d[r][k/256] * sc[r][k/32] * q[r][k] - dmin[r][k/256] * m[r][k/32].
 * A row whose length is not a multiple of 256 (the routed down projection,
 * K = 896) ends in a partial super-block of 4 sub-blocks.
 *
 * Canonical input of one matrix [N rows][K] (moe_q4k_matrix_t, host memory):
 *   q [N][K] codes 0..15, one per byte; d, dmin [N][ceil(K/256)] f16 bit
 *   patterns (finite); sc, m [N][K/32] values 0..63, one per byte.
 * moe_pack_expert_q4k writes:
 *   codes_out: moe_expert_code_bytes(4, inter) bytes, the int4 tile layout
 *     above holding q - 8 (so W = s (q - 8) + beta with s = d sc and
 *     beta = 8 s - dmin m per sub-block);
 *   meta_out: 4 * moe_expert_scale_count(MOE_Q4K, inter) bytes, 4-byte aligned:
 *     gate records [inter][5] then up records [inter][5], 16 bytes each (row,
 *     super-block): w0 = d | dmin << 16; byte j (j < 4) of w1 = sc_j |
 *     (m_j >> 4) << 6, of w2 = sc_{4+j} | (m_{4+j} >> 4) << 6, of w3 =
 *     (m_j & 15) | (m_{4+j} & 15) << 4;
 *     then the down matrix in its tiles' row order, slot (rt, r, j) =
 *     rt * 64 + r * 4 + j holding row 64 rt + 16 j + r (rt < 20, r < 16,
 *     j < 4): uint32 d | dmin << 16 [ceil(inter/256)][1280 slots], then
 *     uint16 sc | m << 8 [inter/32][1280 slots] (one 32-column slice of the
 *     down matrix reads 6 bytes per row).
 *   Metadata bits per weight: 0.5 for gate and up, 0.625 for down (0.64 for
 *   the routed down, whose last super-block is half full).
 * Experts are concatenated as for moe_pack_expert.  The metadata travels in
 * the expert_scales / shared_scales arguments with group = MOE_Q4K and
 * bits = 4.
 * Every path takes this format: moe_decode_forward, and moe_layer_forward
 * on the per-token path and on the grouped path (there a call with a
 * two-level expert set runs the small 16- or 32-row tiles at every token
 * count).
 * Returns MOE_E_NULLPTR for a missing pointer, MOE_E_SHAPE for an
 * intermediate size other than 896 or 1792, MOE_E_ALIGN for a meta_out not
 * 4-byte aligned, MOE_E_FORMAT for a field out of range (nothing is written
 * then).
 * ------------------------------------------------------------------------ */
typedef struct {
  const uint8_t* q;      /* [N][K] codes 0..15 */
  const uint16_t* d;     /* [N][ceil(K/256)] f16 */
  const uint16_t* dmin;  /* [N][ceil(K/256)] f16 */
  const uint8_t* sc;     /* [N][K/32] 0..63 */
  const uint8_t* m;      /* [N][K/32] 0..63 */
} moe_q4k_matrix_t;
moe_status_t moe_pack_expert_q4k(const moe_q4k_matrix_t* gate, const moe_q4k_matrix_t* up,
                                 const moe_q4k_matrix_t* down, int32_t inter, void* codes_out,
                                 void* meta_out);

/* Bytes of device workspace moe_layer_forward needs for n_tokens tokens. */
size_t moe_workspace_bytes(int32_t n_tokens);

/* ------------------------------------------------------------------------
 * One MoE layer over n_tokens tokens (0 <= n_tokens <= MOE_MAX_TOKENS).
 * With n_tokens == 0 nothing is enqueued and x, y, topk_ids and topk_w may be
 * NULL; the other arguments are still validated.
 *
 *   y[t] (+)= FFN_shared(x'[t]) + sum_{i<6} w[t,i] * FFN_{ids[t,i]}(x'[t])
 *
 * x'           = x, or RMSNorm(x) with MOE_NORM_INPUT (see the flags).
 * x            [n_tokens][1280], dtype x_dtype (MOE_F32 or MOE_BF16).
 * router_w     [64][1280] f32.  router_b: [64] f32 added to the logits, or NULL.
 * expert_q     64 packed experts (moe_pack_expert, inter = 896), format
 *              (expert_bits, expert_group).  expert_scales: their packed scales.
 * shared_q     the packed fused shared expert (inter = 1792), format
 *              (shared_bits, shared_group).  shared_scales: its packed scales.
 * y            [n_tokens][1280] f32 output (read too with MOE_ACCUMULATE).
 * topk_ids     [n_tokens][6] int32 out: expert ids in pick order (descending
 *              probability; equal probabilities go to the lower index).
 * topk_w       [n_tokens][6] f32 out: the picked softmax probabilities (over
 *              all 64 experts, not renormalised; they sum to at most 1).
 * workspace    device scratch of at least moe_workspace_bytes(n_tokens)
 *              bytes; its contents need no initialisation and are garbage
 *              after the call.
 * Routing is computed in f32.  Expert arithmetic: the grouped (MFMA) path
 * multiplies exact integer codes by f16 inputs (f32 inputs split into two f16
 * halves) with fp32 accumulation; the per-token path writes each input block
 * in block floating point (19-bit mantissa for int4 weights, 23-bit for int8,
 * one shared power of two per scale group) and forms exact integer dot
 * products.  Both apply each group scale to the partial sum of its group.
 * Domain of the grouped path: every input element (after the optional
 * RMSNorm, which bounds it by sqrt(1280)) and every element of the SwiGLU
 * intermediate h = SiLU(gate) * up (the down projection's input, split into
 * f16 halves the same way) must be below 65504 in magnitude, the f16 range;
 * beyond it the grouped path gives non-finite outputs for that token.  With
 * normalised inputs and int4 codes with scales up to 0.02 (|W| <= 0.16),
 * |gate|, |up| <= 0.16 * 1280 and h stays below 42,000 whatever the input;
 * int8 codes allow a 16x larger |W|, so there only inputs aligned with the
 * weights far beyond random ones could leave the range.  The per-token path
 * has no such limit.
 * Inputs are meant to be finite.  A token whose row holds a NaN or an
 * infinity gets non-finite outputs and weights, but its ids are still six
 * distinct experts in 0..63 (a NaN logit ranks below every number), so no
 * access goes out of bounds and the other tokens are unaffected.
 * ------------------------------------------------------------------------ */
moe_status_t moe_layer_forward(const void* x, int32_t x_dtype, int32_t n_tokens,
                               const float* router_w, const float* router_b,
                               const void* expert_q, const float* expert_scales,
                               int32_t expert_bits, int32_t expert_group,
                               const void* shared_q, const float* shared_scales,
                               int32_t shared_bits, int32_t shared_group,
                               float* y, int32_t* topk_ids, float* topk_w,
                               void* workspace, size_t workspace_bytes,
                               uint32_t flags, void* stream);

/* ------------------------------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * layer as moe_layer_forward, same arguments, results and flags, without a
 * workspace argument.  Its scratch is a file-scope device array of the
 * library, MOE_STATIC_SCRATCH_BYTES per GPU, held by every GPU the library
 * runs on until the process ends; its device address is looked up once per
 * GPU (with that GPU current) at the first call there.  The call allocates
 * nothing and frees nothing.
 * n_tokens      0 .. MOE_STATIC_MAX_TOKENS; more returns MOE_E_SHAPE without
 *               enqueueing anything.  MOE_FORCE_DECODE is accepted only up to
 *               18 tokens (MOE_E_SHAPE beyond), the largest count any format
 *               sends to the per-token path by default.
 * All calls on one GPU share that GPU's scratch: two calls whose executions
 * overlap on one GPU (on different streams, or from different threads without
 * ordering) race and give undefined results.  Calls ordered on one stream are
 * safe.  The scratch needs no initialisation; it holds the last call's
 * intermediates afterwards.
 * ------------------------------------------------------------------------ */
#define MOE_STATIC_MAX_TOKENS 256
#define MOE_STATIC_SCRATCH_BYTES (20u << 20)
moe_status_t moe_layer_forward_static(const void* x, int32_t x_dtype, int32_t n_tokens,
                                      const float* router_w, const float* router_b,
                                      const void* expert_q, const float* expert_scales,
                                      int32_t expert_bits, int32_t expert_group,
                                      const void* shared_q, const float* shared_scales,
                                      int32_t shared_bits, int32_t shared_group,
                                      float* y, int32_t* topk_ids, float* topk_w,
                                      uint32_t flags, void* stream);

/* z[t] = h[t] / sqrt(mean(h[t]^2) + eps) over the 1280 features (no gain);
 * h [n_tokens][1280] f32, z [n_tokens][1280] of z_dtype (bf16: nearest, ties
 * to even).  The decoder's RMSNorm (demo page step 7; README "Architecture"). */
moe_status_t moe_rmsnorm(const float* h, void* z, int32_t z_dtype, int32_t n_tokens,
                         float eps, void* stream);

/* ------------------------------------------------------------------------
 * Decode step: one token through n_layers chained MoE layers in a single
 * persistent kernel launch -- the decoder's per-token path
 * (demo page step 6: layers 1..11 are MoE; step 7: greedy decoding runs one
 * token at a time).  With MOE_NORM_INPUT | MOE_ACCUMULATE each layer computes
 *   h_l = h_{l-1} + MoE_l(RMSNorm(h_{l-1})),   h_0 = x,   y = h_L,
 * which is exactly n_layers calls of moe_layer_forward with those flags.
 * Without MOE_ACCUMULATE, h_l = MoE_l(...); without MOE_NORM_INPUT the layer
 * input is h_{l-1} itself.  MOE_NORM_BF16 and the FORCE flags are not accepted.
 * A non-finite x gives non-finite outputs with valid ids, as for
 * moe_layer_forward.
 *
 * x          [1280] f32 or bf16 (x_dtype); may equal y when f32.
 * y          [1280] f32 output (the residual stream after the last layer).
 * layers     host array of n_layers (1..MOE_DECODE_MAX_LAYERS) device-pointer
 *            sets, each laid out as for moe_layer_forward; all layers share the
 *            routed format (expert_bits, expert_group) and the shared format.
 * topk_ids   [n_layers][6] int32 out, topk_w [n_layers][6] f32 out: each
 *            layer's routing, as moe_layer_forward reports it.
 * workspace  >= moe_decode_workspace_bytes() bytes, 16-byte aligned, cleared
 *            once with moe_decode_workspace_init() after allocation and then
 *            reused across calls without further initialisation (it carries a
 *            call counter).  Calls sharing a workspace must be stream ordered.
 *            Word 2 of the workspace becomes nonzero if a wait inside the
 *            kernel gave up (a bug guard; results are then invalid).
 * The kernel's 256 workgroups (one per compute unit on MI355X) must all be
 * resident at once: the call returns MOE_E_HIP without launching when the
 * device cannot hold them, and the caller must not run other kernels on the
 * device concurrently with it (a workgroup kept waiting for a CU would make
 * the others' bounded waits give up and set the error word).
 * ------------------------------------------------------------------------ */
#define MOE_DECODE_MAX_LAYERS 16

typedef struct {
  const float* router_w;       /* [64][1280] f32 */
  const float* router_b;       /* [64] f32 or NULL */
  const void* expert_q;        /* 64 packed routed experts */
  const float* expert_scales;  /* their packed scales */
  const void* shared_q;        /* the packed fused shared expert */
  const float* shared_scales;  /* its packed scales */
} moe_layer_weights_t;

size_t moe_decode_workspace_bytes(void);
moe_status_t moe_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream);
moe_status_t moe_decode_forward(const void* x, int32_t x_dtype, float* y, int32_t n_layers,
                                const moe_layer_weights_t* layers, int32_t expert_bits,
                                int32_t expert_group, int32_t shared_bits, int32_t shared_group,
                                int32_t* topk_ids, float* topk_w, void* workspace,
                                size_t workspace_bytes, uint32_t flags, void* stream);

/* ------------------------------------------------------------------------
 * Measurement helper (not a step of the layer): *sink ^= the XOR of every
 * 32-bit word of the `bytes` bytes at src, read once with 16-byte loads spread
 * over every compute unit.  Timed on `stream` over a buffer much larger than
 * the last-level cache, it gives the device's practical streaming-read rate,
 * against which the decode step's bandwidth is reported beside the HBM peak.
 * src: device memory, 16-byte aligned, bytes a multiple of 16 (MOE_E_ALIGN
 * otherwise); sink: one device word, 4-byte aligned, that the caller clears
 * first.  bytes == 0 launches nothing.  Asynchronous on `stream`.
 * ------------------------------------------------------------------------ */
moe_status_t moe_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
