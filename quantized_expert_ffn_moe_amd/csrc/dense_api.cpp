// Host side of the C ABI declared in include/moe_dense.h: argument validation
// and kernel dispatch for the lm_head GEMV + greedy token and the dense
// layer-0 SwiGLU MLP.
#include "../../include/moe_dense.h"
#include "moe_internal.h"

using namespace moe;

static_assert(MOE_DENSE_MAX_TOKENS == DENSE_MAX_T && MOE_DENSE_MAX_INTER == DENSE_MAX_INTER,
              "public and internal dense constants disagree");

namespace {
bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool al4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }
bool group_ok(int g) { return g == 32 || g == 64 || g == 128; }
}  // namespace

extern "C" {

size_t moe_lm_head_workspace_bytes(int32_t n_tokens, int32_t vocab) {
  if (n_tokens < 0 || n_tokens > DENSE_MAX_T || vocab < 1 || vocab > MOE_HEAD_MAX_VOCAB) return 0;
  return round256((size_t)head_workgroups(vocab) * (n_tokens ? n_tokens : 1) * 8);
}

moe_status_t moe_lm_head_argmax(const float* h, int32_t n_tokens, uint32_t flags, const void* w, int32_t w_bits,
                                const float* w_scales, int32_t group, int32_t vocab, float* logits, int32_t* token,
                                float* token_logit, void* workspace, size_t workspace_bytes, void* stream) {
  if (!h || !w || !token || !token_logit || !workspace) return MOE_E_NULLPTR;
  if (w_bits != MOE_HEAD_BF16 && w_bits != MOE_HEAD_INT8) return MOE_E_FORMAT;
  if (w_bits == MOE_HEAD_INT8 && (!group_ok(group))) return MOE_E_FORMAT;
  if (w_bits == MOE_HEAD_INT8 && !w_scales) return MOE_E_NULLPTR;
  if (n_tokens < 0 || n_tokens > DENSE_MAX_T || vocab < 1 || vocab > MOE_HEAD_MAX_VOCAB) return MOE_E_SHAPE;
  if (flags & ~(uint32_t)MOE_NORM_INPUT) return MOE_E_ARG;
  if (!al16(h) || !al16(w) || !al16(workspace)) return MOE_E_ALIGN;
  if ((w_scales && !al4(w_scales)) || (logits && !al4(logits)) || !al4(token) || !al4(token_logit))
    return MOE_E_ALIGN;
  if (workspace_bytes < moe_lm_head_workspace_bytes(n_tokens, vocab)) return MOE_E_WORKSPACE;
  if (n_tokens == 0) return MOE_OK;
  HeadArgs a;
  a.h = h; a.T = n_tokens; a.norm = (flags & MOE_NORM_INPUT) != 0; a.eps = 1e-6f;
  a.w = w; a.s = w_bits == MOE_HEAD_INT8 ? w_scales : nullptr; a.group = w_bits == MOE_HEAD_INT8 ? group : 128;
  a.vocab = vocab; a.logits = logits; a.cand = (float*)workspace; a.token = token; a.token_logit = token_logit;
  (void)hipGetLastError();
  if (launch_head(a, w_bits == MOE_HEAD_BF16, (hipStream_t)stream) != hipSuccess) return MOE_E_HIP;
  return MOE_OK;
}

size_t moe_dense_ffn_code_bytes(int32_t bits, int32_t inter) {
  if ((bits != 4 && bits != 8) || inter < 64 || inter > DENSE_MAX_INTER || inter % 64) return 0;
  return (size_t)3 * inter * H * bits / 8;
}

moe_status_t moe_pack_dense_ffn(const int8_t* gate, const int8_t* up, const int8_t* down, int32_t bits,
                                int32_t inter, void* codes_out) {
  if (!gate || !up || !down || !codes_out) return MOE_E_NULLPTR;
  if (bits != 4 && bits != 8) return MOE_E_FORMAT;
  if (inter < 64 || inter > DENSE_MAX_INTER || inter % 64) return MOE_E_SHAPE;
  const size_t n = (size_t)inter * H;   // codes per matrix
  const int8_t* mats[3] = {gate, up, down};
  if (bits == 4)
    for (const int8_t* m : mats)
      for (size_t i = 0; i < n; ++i)
        if (m[i] < -8 || m[i] > 7) return MOE_E_FORMAT;
  uint8_t* out = (uint8_t*)codes_out;
  for (const int8_t* m : mats) {
    if (bits == 8) {
      for (size_t i = 0; i < n; ++i) out[i] = (uint8_t)m[i];
      out += n;
    } else {
      // every row length (1280 or inter) is even, so pairs never straddle rows
      for (size_t i = 0; i < n / 2; ++i)
        out[i] = (uint8_t)(((uint8_t)m[2 * i] & 0x0Fu) | (((uint8_t)m[2 * i + 1] & 0x0Fu) << 4));
      out += n / 2;
    }
  }
  return MOE_OK;
}

size_t moe_dense_ffn_workspace_bytes(int32_t n_tokens, int32_t inter) {
  if (n_tokens < 0 || n_tokens > DENSE_MAX_T || inter < 64 || inter > DENSE_MAX_INTER || inter % 64) return 0;
  return round256((size_t)(n_tokens ? n_tokens : 1) * inter * 4);
}

moe_status_t moe_dense_ffn_forward(const float* x, int32_t n_tokens, const void* codes, const float* scales,
                                   int32_t bits, int32_t group, int32_t inter, float* y, uint32_t flags,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !codes || !scales || !y || !workspace) return MOE_E_NULLPTR;
  if ((bits != 4 && bits != 8) || !group_ok(group)) return MOE_E_FORMAT;
  if (n_tokens < 0 || n_tokens > DENSE_MAX_T || inter < 64 || inter > DENSE_MAX_INTER || inter % 64 ||
      inter % group)
    return MOE_E_SHAPE;
  if (flags & ~(uint32_t)(MOE_NORM_INPUT | MOE_ACCUMULATE)) return MOE_E_ARG;
  if (!al16(x) || !al16(codes) || !al16(y) || !al16(workspace) || !al4(scales)) return MOE_E_ALIGN;
  if (workspace_bytes < moe_dense_ffn_workspace_bytes(n_tokens, inter)) return MOE_E_WORKSPACE;
  if (n_tokens == 0) return MOE_OK;
  const size_t mat = (size_t)inter * H * bits / 8, sg = (size_t)inter * (H / group);
  DenseGateUpArgs g;
  g.x = x; g.T = n_tokens; g.norm = (flags & MOE_NORM_INPUT) != 0; g.eps = 1e-6f;
  g.q = (const uint8_t*)codes; g.s = scales; g.bits = bits; g.group = group; g.inter = inter;
  g.hmid = (float*)workspace;
  DenseDownArgs d;
  d.hmid = (const float*)workspace; d.T = n_tokens;
  d.q = (const uint8_t*)codes + 2 * mat; d.s = scales + 2 * sg; d.bits = bits; d.group = group; d.inter = inter;
  d.y = y; d.accumulate = (flags & MOE_ACCUMULATE) != 0;
  (void)hipGetLastError();
  if (launch_dense(g, d, (hipStream_t)stream) != hipSuccess) return MOE_E_HIP;
  return MOE_OK;
}

}  // extern "C"
