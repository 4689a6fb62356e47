// Host side of the C ABI declared in include/moe_attn.h: argument validation
// and dispatch of the R-SWA decode step.
#include "../../include/moe_attn.h"
#include "moe_internal.h"

#include <math.h>

using namespace moe;

static_assert(MOE_HEADS == ATT_HEADS && MOE_HEAD_DIM == ATT_D && MOE_RSWA_WINDOW == RSWA_W,
              "public and internal attention constants disagree");

namespace {
bool a16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
}  // namespace

extern "C" {

size_t moe_rswa_workspace_bytes(int32_t n_streams, int32_t n_ref) {
  if (n_streams < 0 || n_streams > MOE_RSWA_MAX_STREAMS || n_ref < 0 || n_ref > MOE_RSWA_MAX_REF) return 0;
  const size_t b = (size_t)(n_streams ? n_streams : 1) * ATT_HEADS * rswa_chunks(n_ref) * RSWA_PART * 4;
  return (b + 255) & ~(size_t)255;
}

moe_status_t moe_rswa_decode(int32_t n_streams, int32_t n_ref, const float* q, const float* k_new,
                             const float* v_new, const void* ref_k, const void* ref_v, void* ring_k, void* ring_v,
                             const int32_t* n_gen, float* out, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (!q || !k_new || !v_new || !ring_k || !ring_v || !n_gen || !out || !workspace) return MOE_E_NULLPTR;
  if (n_ref > 0 && (!ref_k || !ref_v)) return MOE_E_NULLPTR;
  if (n_streams < 0 || n_streams > MOE_RSWA_MAX_STREAMS || n_ref < 0 || n_ref > MOE_RSWA_MAX_REF) return MOE_E_SHAPE;
  if (!a16(q) || !a16(k_new) || !a16(v_new) || !a16(ring_k) || !a16(ring_v) || !a16(out) || !a16(workspace) ||
      (n_ref > 0 && (!a16(ref_k) || !a16(ref_v))) || ((uintptr_t)n_gen & 3u))
    return MOE_E_ALIGN;
  if (workspace_bytes < moe_rswa_workspace_bytes(n_streams, n_ref)) return MOE_E_WORKSPACE;
  if (n_streams == 0) return MOE_OK;
  RswaArgs a;
  a.S = n_streams; a.n_ref = n_ref; a.n_chunks = rswa_chunks(n_ref); a.scale = 1.0f / sqrtf((float)ATT_D);
  a.q = q; a.k_new = k_new; a.v_new = v_new;
  a.ref_k = (const uint16_t*)ref_k; a.ref_v = (const uint16_t*)ref_v;
  a.ring_k = (uint16_t*)ring_k; a.ring_v = (uint16_t*)ring_v;
  a.n_gen = n_gen; a.part = (float*)workspace; a.out = out;
  (void)hipGetLastError();
  if (launch_rswa(a, (hipStream_t)stream) != hipSuccess) return MOE_E_HIP;
  return MOE_OK;
}

size_t moe_attn_block_workspace_bytes(int32_t n_streams, int32_t n_ref) {
  const size_t rs = moe_rswa_workspace_bytes(n_streams, n_ref);
  if (rs == 0) return 0;
  const size_t rows = (size_t)(n_streams ? n_streams : 1) * H * 4;   // one [S][1280] f32 array
  const size_t r256 = (rows + 255) & ~(size_t)255;
  return 5 * r256 + rs;   // z, q | k | v, attention output, then the R-SWA partials
}

moe_status_t moe_attn_block_forward(int32_t n_streams, int32_t n_ref, float* h, const void* w_qkv, const void* w_o,
                                    const void* ref_k, const void* ref_v, void* ring_k, void* ring_v,
                                    const int32_t* n_gen, void* workspace, size_t workspace_bytes, void* stream) {
  // an empty call may pass NULL for the per-stream buffers (empty tensors)
  if (!w_qkv || !w_o || !workspace) return MOE_E_NULLPTR;
  if (n_streams > 0 && (!h || !ring_k || !ring_v || !n_gen || (n_ref > 0 && (!ref_k || !ref_v))))
    return MOE_E_NULLPTR;
  if (n_streams < 0 || n_streams > MOE_RSWA_MAX_STREAMS || n_ref < 0 || n_ref > MOE_RSWA_MAX_REF) return MOE_E_SHAPE;
  const void* v16[] = {h, w_qkv, w_o, ring_k, ring_v, workspace, ref_k, ref_v};
  for (const void* p : v16)
    if (p && !a16(p)) return MOE_E_ALIGN;
  if ((uintptr_t)n_gen & 3u) return MOE_E_ALIGN;
  if (workspace_bytes < moe_attn_block_workspace_bytes(n_streams, n_ref)) return MOE_E_WORKSPACE;
  if (n_streams == 0) return MOE_OK;
  const int S = n_streams;
  const size_t r256 = ((size_t)S * H * 4 + 255) & ~(size_t)255;
  char* ws = (char*)workspace;
  float* z = (float*)ws;
  float* qkv = (float*)(ws + r256);   // three [S][1280] arrays, r256 apart
  float* att = (float*)(ws + 4 * r256);
  void* part = ws + 5 * r256;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  // the norm and the attention step write their outputs as split bf16 halves
  // (same bytes as f32), which the projections read as they are; for a few
  // streams the q/k/v projection forms the normalised rows itself (one launch
  // fewer)
  ProjArgs pq;
  pq.w = (const uint16_t*)w_qkv; pq.y = qkv; pq.T = S; pq.N = 3 * H; pq.accumulate = 0;
  if (S <= PJ_NORM_MAX_T) {
    pq.a_hl = nullptr; pq.h_norm = h; pq.eps = 1e-6f;
  } else {
    if (launch_rmsnorm(h, z, 2, S, 1e-6f, s) != hipSuccess) return MOE_E_HIP;
    pq.a_hl = (const uint16_t*)z;
  }
  static_assert(H * 4 % 256 == 0, "q, k and v arrays [S][1280] apart, as the projection writes them");
  if (launch_proj(pq, s) != hipSuccess) return MOE_E_HIP;
  RswaArgs a;
  a.S = S; a.n_ref = n_ref; a.n_chunks = rswa_chunks(n_ref); a.scale = 1.0f / sqrtf((float)ATT_D);
  a.q = qkv; a.k_new = qkv + (size_t)S * H; a.v_new = qkv + 2 * (size_t)S * H;
  a.ref_k = (const uint16_t*)ref_k; a.ref_v = (const uint16_t*)ref_v;
  a.ring_k = (uint16_t*)ring_k; a.ring_v = (uint16_t*)ring_v;
  a.n_gen = n_gen; a.part = (float*)part; a.out = nullptr; a.out_hl = (uint16_t*)att;
  if (launch_rswa(a, s) != hipSuccess) return MOE_E_HIP;
  ProjArgs po;
  po.a_hl = (const uint16_t*)att; po.w = (const uint16_t*)w_o; po.y = h; po.T = S; po.N = H; po.accumulate = 1;
  if (launch_proj(po, s) != hipSuccess) return MOE_E_HIP;
  return MOE_OK;
}

}  // extern "C"
