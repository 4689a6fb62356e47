// Host side of the C ABI declared in include/moe.h: argument validation,
// workspace carving, weight packing and kernel dispatch.
#include "../../include/moe.h"
#include "moe_internal.h"

#include <string.h>

using namespace moe;

static_assert(MOE_HIDDEN == H && MOE_EXPERTS == E && MOE_TOPK == TOPK && MOE_INTER == I &&
                  MOE_SHARED_INTER == IS && MOE_MAX_TOKENS == MAX_T,
              "public and internal shape constants disagree");

namespace {

bool fmt_ok(int bits, int group) {
  return (bits == 4 || bits == 8) && (group == 32 || group == 64 || group == 128);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Workspace {
  float* z;          // [T][H]
  float* h_routed;   // [T*6][I]
  float* h_shared;   // [T][IS]
  float* ysorted;    // [T*6][H]
  float* ys;         // [T][H]
  int32_t* counts;   // [E]
  int32_t* offsets;  // [E+1]
  int32_t* ntiles;   // [1]
  int32_t* tiles;    // [max_tiles][2]
  int32_t* perm;     // [T*6]
  int32_t* pos_of;   // [T*6]
  size_t bytes;
  int max_tiles;
};

Workspace carve(void* base, int T) {
  Workspace w;
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return base ? (void*)((char*)base + o) : nullptr;
  };
  const size_t slots = (size_t)T * TOPK;
  w.max_tiles = (int)(slots / MT) + E + 1;
  w.z = (float*)take((size_t)T * H * 4);
  w.h_routed = (float*)take(slots * I * 4);
  w.h_shared = (float*)take((size_t)T * IS * 4);
  w.ysorted = (float*)take(slots * H * 4);
  w.ys = (float*)take((size_t)T * H * 4);
  w.counts = (int32_t*)take(E * 4);
  w.offsets = (int32_t*)take((E + 1) * 4);
  w.ntiles = (int32_t*)take(4);
  w.tiles = (int32_t*)take((size_t)w.max_tiles * 2 * 4);
  w.perm = (int32_t*)take(slots * 4);
  w.pos_of = (int32_t*)take(slots * 4);
  w.bytes = off;
  return w;
}

QW make_qw(const void* q, const float* s, int bits, int group, int inter, bool routed) {
  QW w;
  w.q = (const uint8_t*)q;
  w.s = s;
  w.bits = bits;
  w.group = group;
  w.inter = inter;
  w.e_bytes = routed ? moe_expert_code_bytes(bits, inter) : 0;
  w.e_scales = routed ? moe_expert_scale_count(group, inter) : 0;
  return w;
}

void pack_matrix(const int8_t* Q, int N, int K, int bits, uint8_t* out) {
  const int KB = kb_cols(bits), nkb = K / KB;
  for (int nt = 0; nt < N / 16; ++nt)
    for (int kb = 0; kb < nkb; ++kb) {
      uint8_t* tile = out + ((size_t)nt * nkb + kb) * TILE;
      for (int lane = 0; lane < 64; ++lane) {
        const int row = nt * 16 + (lane & 15), q = lane >> 4;
        const int8_t* src = Q + (size_t)row * K + (size_t)kb * KB;
        uint8_t* dst = tile + lane * 16;
        for (int j = 0; j < 4; ++j) {
          uint32_t word = 0;
          if (bits == 4) {
            for (int i = 0; i < 8; ++i) {
              const int k = 32 * j + 8 * q + i;
              word |= (uint32_t)(src[k] + 8) << (4 * i);
            }
          } else {
            for (int i = 0; i < 4; ++i) {
              const int k = 32 * (j >> 1) + 8 * q + 4 * (j & 1) + i;
              word |= (uint32_t)(uint8_t)(src[k] + 128) << (8 * i);
            }
          }
          memcpy(dst + 4 * j, &word, 4);
        }
      }
    }
}

void pack_scales(const float* S, int N, int K, int group, float* out) {
  const int ng = K / group;
  for (int nt = 0; nt < N / 16; ++nt)
    for (int g = 0; g < ng; ++g)
      for (int r = 0; r < 16; ++r) out[((size_t)nt * ng + g) * 16 + r] = S[(size_t)(nt * 16 + r) * ng + g];
}

bool codes_in_range(const int8_t* Q, size_t n, int bits) {
  if (bits == 8) return true;
  for (size_t i = 0; i < n; ++i)
    if (Q[i] < -8 || Q[i] > 7) return false;
  return true;
}

}  // namespace

extern "C" {

const char* moe_status_str(int32_t status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_E_NULLPTR: return "MOE_E_NULLPTR: a required pointer is NULL";
    case MOE_E_SHAPE: return "MOE_E_SHAPE: token count or intermediate size out of range";
    case MOE_E_FORMAT: return "MOE_E_FORMAT: unsupported bits/group or code out of range";
    case MOE_E_ALIGN: return "MOE_E_ALIGN: device pointer not 16-byte aligned";
    case MOE_E_WORKSPACE: return "MOE_E_WORKSPACE: workspace too small";
    case MOE_E_HIP: return "MOE_E_HIP: HIP runtime error while enqueueing";
    case MOE_E_ARG: return "MOE_E_ARG: invalid argument";
    default: return "unknown moe status";
  }
}

size_t moe_expert_code_bytes(int32_t bits, int32_t inter) {
  if (bits != 4 && bits != 8) return 0;
  return 3 * matrix_bytes(bits, inter, H);
}

size_t moe_expert_scale_count(int32_t group_size, int32_t inter) {
  if (group_size != 32 && group_size != 64 && group_size != 128) return 0;
  return 3 * (size_t)inter * H / group_size;
}

moe_status_t moe_pack_expert(const int8_t* gate, const int8_t* up, const int8_t* down,
                             const float* gate_scales, const float* up_scales,
                             const float* down_scales, int32_t inter, int32_t bits,
                             int32_t group_size, void* codes_out, float* scales_out) {
  if (!gate || !up || !down || !gate_scales || !up_scales || !down_scales || !codes_out || !scales_out)
    return MOE_E_NULLPTR;
  if (inter != I && inter != IS) return MOE_E_SHAPE;
  if (!fmt_ok(bits, group_size)) return MOE_E_FORMAT;
  const size_t n = (size_t)inter * H;
  if (!codes_in_range(gate, n, bits) || !codes_in_range(up, n, bits) || !codes_in_range(down, n, bits))
    return MOE_E_FORMAT;
  uint8_t* out = (uint8_t*)codes_out;
  const size_t mb = matrix_bytes(bits, inter, H);
  pack_matrix(gate, inter, H, bits, out);
  pack_matrix(up, inter, H, bits, out + mb);
  pack_matrix(down, H, inter, bits, out + 2 * mb);
  const size_t ms = (size_t)inter * H / group_size;
  pack_scales(gate_scales, inter, H, group_size, scales_out);
  pack_scales(up_scales, inter, H, group_size, scales_out + ms);
  pack_scales(down_scales, H, inter, group_size, scales_out + 2 * ms);
  return MOE_OK;
}

size_t moe_workspace_bytes(int32_t n_tokens) {
  if (n_tokens < 0 || n_tokens > MAX_T) return 0;
  return carve(nullptr, n_tokens).bytes;
}

moe_status_t moe_layer_forward(const void* x, int32_t x_dtype, int32_t n_tokens,
                               const float* router_w, const float* router_b,
                               const void* expert_q, const float* expert_scales,
                               int32_t expert_bits, int32_t expert_group,
                               const void* shared_q, const float* shared_scales,
                               int32_t shared_bits, int32_t shared_group,
                               float* y, int32_t* topk_ids, float* topk_w,
                               void* workspace, size_t workspace_bytes,
                               uint32_t flags, void* stream) {
  const int T = n_tokens;
  if (T < 0 || T > MAX_T) return MOE_E_SHAPE;
  // an empty call may pass NULL for the per-token buffers (empty tensors)
  if ((T > 0 && (!x || !y || !topk_ids || !topk_w)) || !router_w || !expert_q || !expert_scales ||
      !shared_q || !shared_scales || !workspace)
    return MOE_E_NULLPTR;
  if (!fmt_ok(expert_bits, expert_group) || !fmt_ok(shared_bits, shared_group)) return MOE_E_FORMAT;
  const uint32_t known = MOE_ACCUMULATE | MOE_NORM_INPUT | MOE_NORM_BF16 | MOE_FORCE_DECODE | MOE_FORCE_GROUPED;
  if ((flags & ~known) || (x_dtype != MOE_F32 && x_dtype != MOE_BF16)) return MOE_E_ARG;
  if ((flags & MOE_FORCE_DECODE) && (flags & MOE_FORCE_GROUPED)) return MOE_E_ARG;
  if ((flags & MOE_NORM_BF16) && !(flags & MOE_NORM_INPUT)) return MOE_E_ARG;
  if ((flags & MOE_NORM_INPUT) && x_dtype != MOE_F32) return MOE_E_ARG;
  if (x && x == (const void*)y && !((flags & MOE_ACCUMULATE) && x_dtype == MOE_F32)) return MOE_E_ARG;
  const void* ptrs[] = {x, router_w, router_b, expert_q, expert_scales, shared_q, shared_scales,
                        y, topk_ids, topk_w, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOE_E_ALIGN;
  const Workspace ws = carve(workspace, T);
  if (workspace_bytes < ws.bytes) return MOE_E_WORKSPACE;
  if (T == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();  // clear a stale error so that only our launches are reported

  const bool norm = (flags & MOE_NORM_INPUT) != 0;
  RouterArgs ra;
  ra.x = x; ra.x_bf16 = x_dtype == MOE_BF16; ra.T = T;
  ra.wr = router_w; ra.bias = router_b;
  ra.norm = norm; ra.norm_bf16 = (flags & MOE_NORM_BF16) != 0; ra.eps = 1e-6f;
  ra.z = ws.z; ra.ids = topk_ids; ra.w = topk_w;
  if (launch_router(ra, s) != hipSuccess) return MOE_E_HIP;

  // input rows of the experts: the normalised z (f32) or x itself
  const float* xf = norm ? ws.z : (x_dtype == MOE_F32 ? (const float*)x : nullptr);
  const uint16_t* xb = (!norm && x_dtype == MOE_BF16) ? (const uint16_t*)x : nullptr;
  const QW rw = make_qw(expert_q, expert_scales, expert_bits, expert_group, I, true);
  const QW sw = make_qw(shared_q, shared_scales, shared_bits, shared_group, IS, false);
  const int accumulate = (flags & MOE_ACCUMULATE) != 0;

  const bool decode = (flags & MOE_FORCE_DECODE) || (!(flags & MOE_FORCE_GROUPED) && T <= DECODE_MAX_T);
  if (decode) {
    DecGateUpArgs g;
    g.xf = xf; g.xb = xb;
    g.units_per_token = TOPK; g.ids = topk_ids; g.w = rw; g.h = ws.h_routed;
    if (launch_dec_gateup(g, T * TOPK, s) != hipSuccess) return MOE_E_HIP;
    g.units_per_token = 1; g.ids = nullptr; g.w = sw; g.h = ws.h_shared;
    if (launch_dec_gateup(g, T, s) != hipSuccess) return MOE_E_HIP;
    DecDownArgs d;
    d.ids = topk_ids; d.tw = topk_w; d.h_routed = ws.h_routed; d.h_shared = ws.h_shared;
    d.rw = rw; d.sw = sw; d.y = y; d.accumulate = accumulate;
    if (launch_dec_down(d, T, s) != hipSuccess) return MOE_E_HIP;
    return MOE_OK;
  }

  HistArgs ha;
  ha.ids = topk_ids; ha.T = T; ha.counts = ws.counts; ha.offsets = ws.offsets;
  ha.perm = ws.perm; ha.pos_of = ws.pos_of; ha.tiles = ws.tiles; ha.ntiles = ws.ntiles;
  if (launch_hist(ha, s) != hipSuccess) return MOE_E_HIP;

  GroupedArgs ga;
  ga.T = T; ga.tiles = ws.tiles; ga.ntiles = ws.ntiles; ga.offsets = ws.offsets; ga.perm = ws.perm;
  // routed gate/up: A rows are tokens gathered through the permutation
  ga.af = xf; ga.ab = xb; ga.shared = 0; ga.a_by_token = 1; ga.w = rw; ga.out = ws.h_routed;
  if (launch_grouped_gateup(ga, ws.max_tiles, s) != hipSuccess) return MOE_E_HIP;
  // shared gate/up over all tokens
  ga.shared = 1; ga.w = sw; ga.out = ws.h_shared;
  if (launch_grouped_gateup(ga, (T + MT - 1) / MT, s) != hipSuccess) return MOE_E_HIP;
  // routed down: A rows are h in sorted order
  ga.af = ws.h_routed; ga.ab = nullptr; ga.shared = 0; ga.a_by_token = 0; ga.w = rw; ga.out = ws.ysorted;
  if (launch_grouped_down(ga, ws.max_tiles, s) != hipSuccess) return MOE_E_HIP;
  ga.af = ws.h_shared; ga.shared = 1; ga.w = sw; ga.out = ws.ys;
  if (launch_grouped_down(ga, (T + MT - 1) / MT, s) != hipSuccess) return MOE_E_HIP;
  CombineArgs ca;
  ca.ys = ws.ys; ca.ysorted = ws.ysorted; ca.pos_of = ws.pos_of; ca.tw = topk_w;
  ca.y = y; ca.T = T; ca.accumulate = accumulate;
  if (launch_combine(ca, s) != hipSuccess) return MOE_E_HIP;
  return MOE_OK;
}

moe_status_t moe_rmsnorm(const float* h, void* z, int32_t z_dtype, int32_t n_tokens, float eps, void* stream) {
  if (!h || !z) return MOE_E_NULLPTR;
  if (n_tokens < 0 || n_tokens > MAX_T) return MOE_E_SHAPE;
  if (z_dtype != MOE_F32 && z_dtype != MOE_BF16) return MOE_E_ARG;
  if (!(eps >= 0.f)) return MOE_E_ARG;
  if (!aligned16(h) || !aligned16(z)) return MOE_E_ALIGN;
  if (n_tokens == 0) return MOE_OK;
  (void)hipGetLastError();
  if (launch_rmsnorm(h, z, z_dtype == MOE_BF16, n_tokens, eps, (hipStream_t)stream) != hipSuccess) return MOE_E_HIP;
  return MOE_OK;
}

}  // extern "C"
