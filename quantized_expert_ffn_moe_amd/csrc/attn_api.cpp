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

}  // extern "C"
