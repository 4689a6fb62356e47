// Host side of the C ABI declared in include/moe.h: argument validation,
// workspace carving, weight packing and kernel dispatch.
#include "../../include/moe.h"
#include "moe_internal.h"

#include <string.h>

using namespace moe;

static_assert(MOE_HIDDEN == H && MOE_EXPERTS == E && MOE_TOPK == TOPK && MOE_INTER == I &&
                  MOE_SHARED_INTER == IS && MOE_MAX_TOKENS == MAX_T && MOE_Q4K == Q4K,
              "public and internal shape constants disagree");
static_assert(MOE_STATIC_MAX_TOKENS == STATIC_MAX_T && MOE_STATIC_SCRATCH_BYTES == STATIC_SCRATCH_BYTES,
              "public and internal scratch constants disagree");

namespace {

#ifdef MOE_DEVICE_TRACE
unsigned long long* g_trace_buffer = nullptr;
#endif

bool fmt_ok(int bits, int group) {
  return ((bits == 4 || bits == 8) && (group == 32 || group == 64 || group == 128)) || (bits == 4 && group == Q4K);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Workspace {
  float* z;          // [T][H] normalised input
  float* logits;     // [T][E] router logits (two-pass router)
  // grouped path
  float* h_routed;   // [T*6][I]
  float* h_shared;   // [T][IS]
  float* ysorted;    // [T*6][H]
  float* ys;         // [2][T][H]: the shared expert's down projection in two K halves
  int32_t* counts;   // [E]
  int32_t* offsets;  // [E+1]
  int32_t* ntiles;   // [1]
  int32_t* tiles;    // [max_tiles][4]
  int32_t* perm;     // [T*6]
  int32_t* pos_of;   // [T*6]
  int32_t* blkcnt;   // [T*6/1024 + 1][E] per-block histogram counts
  // decode path (aliases the grouped buffers)
  float* part;       // [T][N_ITEMS][H]
  size_t bytes;
  int max_tiles;
};

constexpr int DECODE_FORCE_MAX_T = 64;   // largest token count the per-token path accepts

struct Carver {
  char* base; size_t off;
  void* take(size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return base ? (void*)(base + o) : nullptr;
  }
};

// part_max_t: largest token count that may take the per-token path (its
// partials share the bytes of the grouped path's buffers)
Workspace carve(void* base, int T, int part_max_t = DECODE_FORCE_MAX_T) {
  Workspace w;
  Carver c{(char*)base, 0};
  const size_t slots = (size_t)T * TOPK;
  w.max_tiles = (int)(slots / MT_TINY) + E + 1;    // enough for every tile height
  w.z = (float*)c.take((size_t)T * H * 4);
  w.logits = (float*)c.take((size_t)T * E * 4);
  const size_t union_start = c.off;
  w.h_routed = (float*)c.take(slots * I * 4);
  w.h_shared = (float*)c.take((size_t)T * IS * 4);
  w.ysorted = (float*)c.take(slots * H * 4);
  w.ys = (float*)c.take(2 * (size_t)T * H * 4);
  w.counts = (int32_t*)c.take(E * 4);
  w.offsets = (int32_t*)c.take((E + 1) * 4);
  w.ntiles = (int32_t*)c.take(4);
  w.tiles = (int32_t*)c.take((size_t)w.max_tiles * 4 * 4);
  w.perm = (int32_t*)c.take(slots * 4);
  w.pos_of = (int32_t*)c.take(slots * 4);
  w.blkcnt = (int32_t*)c.take((slots / HIST_BLOCK + 1) * E * 4);
  const size_t grouped_end = c.off;
  c.off = union_start;
  w.part = T <= part_max_t ? (float*)c.take((size_t)T * N_ITEMS * H * 4) : nullptr;
  w.bytes = c.off > grouped_end ? c.off : grouped_end;
  return w;
}

struct DecodeWorkspace {
  uint32_t* hdr; uint32_t* ipart; uint32_t* rec;
  size_t clear_words;  // words cleared by moe_decode_workspace_init (all of it: tags must start stale)
  size_t bytes;
};

DecodeWorkspace carve_decode(void* base) {
  DecodeWorkspace w;
  Carver c{(char*)base, 0};
  w.hdr = (uint32_t*)c.take(64 * 4);
  w.ipart = (uint32_t*)c.take((size_t)N_ITEMS * ITEM_U4 * 16);
  w.rec = (uint32_t*)c.take((size_t)N_RED * REC_U4 * 16);
  w.bytes = c.off;
  w.clear_words = c.off / 4;
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
  w.e_scales = routed ? scale_words(group, inter) : 0;
  return w;
}

// gate/up matrices: 1 KiB tiles of 16 rows x KB columns, tile (nt, kb); the
// stored code of an element is its value plus `off` (-8: two-level codes)
template <typename C>
void pack_rows(const C* Q, int N, int K, int bits, uint8_t* out, int off = 0) {
  const int KB = kb_cols(bits), nkb = K / KB;
  for (int nt = 0; nt < N / 16; ++nt)
    for (int kb = 0; kb < nkb; ++kb) {
      uint8_t* tile = out + ((size_t)nt * nkb + kb) * TILE;
      for (int lane = 0; lane < 64; ++lane) {
        const int row = nt * 16 + (lane & 15), q = lane >> 4;
        const C* src = Q + (size_t)row * K + (size_t)kb * KB;
        for (int j = 0; j < 4; ++j) {
          uint32_t word = 0;
          if (bits == 4) {
            for (int i = 0; i < 8; ++i) word |= (uint32_t)(((int)src[32 * j + 8 * q + i] + off) & 15) << (4 * i);
          } else {
            for (int i = 0; i < 4; ++i)
              word |= (uint32_t)(uint8_t)src[32 * (j >> 1) + 8 * q + 4 * (j & 1) + i] << (8 * i);
          }
          memcpy(tile + lane * 16 + 4 * j, &word, 4);
        }
      }
    }
}

// down matrices: 1 KiB tiles of DR rows x 32 columns, tile (kc, rt)
template <typename C>
void pack_slabs(const C* Q, int N, int K, int bits, uint8_t* out, int off = 0) {
  const int DR = down_rows(bits), nrt = N / DR, nkc = K / 32;
  for (int kc = 0; kc < nkc; ++kc)
    for (int rt = 0; rt < nrt; ++rt) {
      uint8_t* tile = out + ((size_t)kc * nrt + rt) * TILE;
      for (int lane = 0; lane < 64; ++lane) {
        const int r = lane & 15, q = lane >> 4;
        for (int j = 0; j < 4; ++j) {
          uint32_t word = 0;
          if (bits == 4) {
            const C* src = Q + (size_t)(DR * rt + 16 * j + r) * K + 32 * kc + 8 * q;
            for (int i = 0; i < 8; ++i) word |= (uint32_t)(((int)src[i] + off) & 15) << (4 * i);
          } else {
            const C* src = Q + (size_t)(DR * rt + 16 * (j >> 1) + r) * K + 32 * kc + 8 * q + 4 * (j & 1);
            for (int i = 0; i < 4; ++i) word |= (uint32_t)(uint8_t)src[i] << (8 * i);
          }
          memcpy(tile + lane * 16 + 4 * j, &word, 4);
        }
      }
    }
}

// gate/up scales stay row-major [row][group]
void pack_row_scales(const float* S, int N, int K, int group, float* out) {
  memcpy(out, S, (size_t)N * (K / group) * sizeof(float));
}

void pack_slab_scales(const float* S, int N, int K, int group, int bits, float* out) {
  const int DR = down_rows(bits), nrt = N / DR, ns = DR / 16, ng = K / group;
  for (int g = 0; g < ng; ++g)
    for (int rt = 0; rt < nrt; ++rt)
      for (int r = 0; r < 16; ++r)
        for (int j = 0; j < ns; ++j)
          out[(((size_t)g * nrt + rt) * 16 + r) * ns + j] = S[(size_t)(DR * rt + 16 * j + r) * ng + g];
}

// One gate/up record (row r, super-block b) of a matrix with K columns:
// word 0 = d | dmin << 16; word 1 byte j = sc_j | (m_j >> 4) << 6; word 2
// byte j = sc_{4+j} | (m_{4+j} >> 4) << 6; word 3 byte j = (m_j & 15) |
// (m_{4+j} & 15) << 4.  Sub-blocks past the end of the row stay zero.
void q4k_record(const moe_q4k_matrix_t& M, int K, int r, int b, uint8_t* out) {
  const int nsb = q4k_superblocks(K), nsub = K / Q4K_SUB;
  uint8_t sc[8] = {0}, m[8] = {0};
  for (int j = 0; j < Q4K_SB / Q4K_SUB; ++j) {
    const int g = b * (Q4K_SB / Q4K_SUB) + j;
    if (g >= nsub) break;
    sc[j] = M.sc[(size_t)r * nsub + g];
    m[j] = M.m[(size_t)r * nsub + g];
  }
  uint32_t w[4] = {(uint32_t)M.d[(size_t)r * nsb + b] | ((uint32_t)M.dmin[(size_t)r * nsb + b] << 16), 0u, 0u, 0u};
  for (int j = 0; j < 4; ++j) {
    w[1] |= (uint32_t)(sc[j] | ((m[j] >> 4) << 6)) << (8 * j);
    w[2] |= (uint32_t)(sc[4 + j] | ((m[4 + j] >> 4) << 6)) << (8 * j);
    w[3] |= (uint32_t)((m[j] & 15) | ((m[4 + j] & 15) << 4)) << (8 * j);
  }
  memcpy(out, w, sizeof(w));
}

// Down metadata of a [H][K] matrix in the down tiles' row order (row
// 64 rt + 16 j + r at [rt][r][j]): d | dmin words per super-block, then
// sc | m << 8 halfwords per sub-block.
void q4k_down_meta(const moe_q4k_matrix_t& M, int K, uint8_t* out) {
  const int nsb = q4k_superblocks(K), nsub = K / Q4K_SUB;
  uint32_t* dd = (uint32_t*)out;
  uint16_t* sm = (uint16_t*)(out + (size_t)4 * nsb * H);
  for (int rt = 0; rt < H / 64; ++rt)
    for (int r = 0; r < 16; ++r)
      for (int j = 0; j < 4; ++j) {
        const size_t row = (size_t)64 * rt + 16 * j + r, slot = ((size_t)rt * 16 + r) * 4 + j;
        for (int b = 0; b < nsb; ++b)
          dd[(size_t)b * H + slot] = (uint32_t)M.d[row * nsb + b] | ((uint32_t)M.dmin[row * nsb + b] << 16);
        for (int g = 0; g < nsub; ++g)
          sm[(size_t)g * H + slot] = (uint16_t)(M.sc[row * nsub + g] | (M.m[row * nsub + g] << 8));
      }
}

// every field in range: codes <= 15, sc and m <= 63, d and dmin finite f16
bool q4k_fields_ok(const moe_q4k_matrix_t& M, int N, int K) {
  if (!M.q || !M.d || !M.dmin || !M.sc || !M.m) return false;
  for (size_t i = 0; i < (size_t)N * K; ++i)
    if (M.q[i] > 15) return false;
  for (size_t i = 0; i < (size_t)N * (K / Q4K_SUB); ++i)
    if (M.sc[i] > 63 || M.m[i] > 63) return false;
  for (size_t i = 0; i < (size_t)N * q4k_superblocks(K); ++i)
    if ((M.d[i] & 0x7C00u) == 0x7C00u || (M.dmin[i] & 0x7C00u) == 0x7C00u) return false;
  return true;
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
  if (group_size != 32 && group_size != 64 && group_size != 128 && group_size != Q4K) return 0;
  return scale_words(group_size, inter);
}

moe_status_t moe_pack_expert_q4k(const moe_q4k_matrix_t* gate, const moe_q4k_matrix_t* up,
                                 const moe_q4k_matrix_t* down, int32_t inter, void* codes_out, void* meta_out) {
  if (!gate || !up || !down || !codes_out || !meta_out) return MOE_E_NULLPTR;
  if (inter != I && inter != IS) return MOE_E_SHAPE;
  if ((uintptr_t)meta_out & 3u) return MOE_E_ALIGN;
  if (!gate->q || !gate->d || !gate->dmin || !gate->sc || !gate->m || !up->q || !up->d || !up->dmin || !up->sc ||
      !up->m || !down->q || !down->d || !down->dmin || !down->sc || !down->m)
    return MOE_E_NULLPTR;
  if (!q4k_fields_ok(*gate, inter, H) || !q4k_fields_ok(*up, inter, H) || !q4k_fields_ok(*down, H, inter))
    return MOE_E_FORMAT;
  uint8_t* out = (uint8_t*)codes_out;
  const size_t mb = matrix_bytes(4, inter, H);
  pack_rows(gate->q, inter, H, 4, out, -8);
  pack_rows(up->q, inter, H, 4, out + mb, -8);
  pack_slabs(down->q, H, inter, 4, out + 2 * mb, -8);
  uint8_t* meta = (uint8_t*)meta_out;
  const int nsb = q4k_superblocks(H);
  for (int r = 0; r < inter; ++r)
    for (int b = 0; b < nsb; ++b) {
      q4k_record(*gate, H, r, b, meta + ((size_t)r * nsb + b) * Q4K_REC);
      q4k_record(*up, H, r, b, meta + ((size_t)(inter + r) * nsb + b) * Q4K_REC);
    }
  q4k_down_meta(*down, inter, meta + q4k_rec_bytes(inter));
  return MOE_OK;
}

moe_status_t moe_pack_expert(const int8_t* gate, const int8_t* up, const int8_t* down,
                             const float* gate_scales, const float* up_scales,
                             const float* down_scales, int32_t inter, int32_t bits,
                             int32_t group_size, void* codes_out, float* scales_out) {
  if (!gate || !up || !down || !gate_scales || !up_scales || !down_scales || !codes_out || !scales_out)
    return MOE_E_NULLPTR;
  if (inter != I && inter != IS) return MOE_E_SHAPE;
  if (!fmt_ok(bits, group_size) || group_size == Q4K) return MOE_E_FORMAT;
  const size_t n = (size_t)inter * H;
  if (!codes_in_range(gate, n, bits) || !codes_in_range(up, n, bits) || !codes_in_range(down, n, bits))
    return MOE_E_FORMAT;
  uint8_t* out = (uint8_t*)codes_out;
  const size_t mb = matrix_bytes(bits, inter, H);
  pack_rows(gate, inter, H, bits, out);
  pack_rows(up, inter, H, bits, out + mb);
  pack_slabs(down, H, inter, bits, out + 2 * mb);
  const size_t ms = (size_t)inter * H / group_size;
  pack_row_scales(gate_scales, inter, H, group_size, scales_out);
  pack_row_scales(up_scales, inter, H, group_size, scales_out + ms);
  pack_slab_scales(down_scales, H, inter, group_size, bits, scales_out + 2 * ms);
  return MOE_OK;
}

size_t moe_workspace_bytes(int32_t n_tokens) {
  if (n_tokens < 0 || n_tokens > MAX_T) return 0;
  return carve(nullptr, n_tokens).bytes;
}

}  // extern "C"

namespace {

// moe_layer_forward with the largest per-token-path call as a parameter
// (the workspace-free entry point keeps that path to its default range)
moe_status_t layer_forward(const void* x, int32_t x_dtype, int32_t n_tokens,
                           const float* router_w, const float* router_b,
                           const void* expert_q, const float* expert_scales,
                           int32_t expert_bits, int32_t expert_group,
                           const void* shared_q, const float* shared_scales,
                           int32_t shared_bits, int32_t shared_group,
                           float* y, int32_t* topk_ids, float* topk_w,
                           void* workspace, size_t workspace_bytes,
                           uint32_t flags, void* stream, int part_max_t) {
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
  if ((flags & MOE_FORCE_DECODE) && T > part_max_t) return MOE_E_SHAPE;
  // a call with a two-level expert set runs the grouped path's small (16- or
  // 32-row) tiles at every token count, both expert sets alike
  const bool two_level = expert_group == Q4K || shared_group == Q4K;
  if ((flags & MOE_NORM_BF16) && !(flags & MOE_NORM_INPUT)) return MOE_E_ARG;
  if ((flags & MOE_NORM_INPUT) && x_dtype != MOE_F32) return MOE_E_ARG;
  if (x && x == (const void*)y && !((flags & MOE_ACCUMULATE) && x_dtype == MOE_F32)) return MOE_E_ARG;
  const void* vec_ptrs[] = {x, router_w, expert_q, shared_q, y, workspace};  // read/written 16 B at a time
  for (const void* p : vec_ptrs)
    if (p && !aligned16(p)) return MOE_E_ALIGN;
  const void* word_ptrs[] = {router_b, expert_scales, shared_scales, topk_ids, topk_w};
  for (const void* p : word_ptrs)
    if (p && ((uintptr_t)p & 3u)) return MOE_E_ALIGN;
  const Workspace ws = carve(workspace, T, part_max_t);
  if (workspace_bytes < ws.bytes) return MOE_E_WORKSPACE;
  if (T == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();  // clear a stale error so that only our launches are reported

  const bool norm = (flags & MOE_NORM_INPUT) != 0;
  RouterArgs ra;
  ra.x = x; ra.x_bf16 = x_dtype == MOE_BF16; ra.T = T;
  ra.wr = router_w; ra.bias = router_b;
  ra.norm = norm; ra.norm_bf16 = (flags & MOE_NORM_BF16) != 0; ra.eps = 1e-6f;
  ra.z = ws.z; ra.ids = topk_ids; ra.w = topk_w; ra.logits = ws.logits;

  // input rows of the experts: the normalised z (f32, or bf16 when rounded to
  // bf16, which the grouped path then feeds to the MFMAs without a lo half)
  const bool zb = norm && (flags & MOE_NORM_BF16);
  const float* xf = norm ? (zb ? nullptr : ws.z) : (x_dtype == MOE_F32 ? (const float*)x : nullptr);
  const uint16_t* xb = zb ? (const uint16_t*)ws.z : ((!norm && x_dtype == MOE_BF16) ? (const uint16_t*)x : nullptr);
  const QW rw = make_qw(expert_q, expert_scales, expert_bits, expert_group, I, true);
  const QW sw = make_qw(shared_q, shared_scales, shared_bits, shared_group, IS, false);
  const int accumulate = (flags & MOE_ACCUMULATE) != 0;

  const bool decode = (flags & MOE_FORCE_DECODE) ||
                      (!(flags & MOE_FORCE_GROUPED) && T <= part_max_t &&
                       T <= decode_switch_t(expert_bits, expert_group, xf != nullptr));
  if (decode) {
    // few tokens: the items select their own picks from the logits (no
    // selection launch)
    const bool self_select = T <= DEC_SELF_SELECT_MAX_T;
    if (launch_router(ra, s, !self_select) != hipSuccess) return MOE_E_HIP;
    DecItemsArgs d;
    d.xf = xf; d.xb = xb; d.logits = self_select ? ws.logits : nullptr; d.ids = topk_ids; d.tw = topk_w; d.rw = rw; d.sw = sw; d.part = ws.part;
    if (launch_dec_items(d, T, s) != hipSuccess) return MOE_E_HIP;
    DecReduceArgs rd;
    rd.part = ws.part; rd.y = y; rd.accumulate = accumulate;
    if (launch_dec_reduce(rd, T, s) != hipSuccess) return MOE_E_HIP;
    return MOE_OK;
  }
  if (launch_router(ra, s) != hipSuccess) return MOE_E_HIP;

  // tile shape: 32-row tiles while the experts see few rows each (about 64 or
  // fewer on average), 64-row tiles beyond
  // (32-column scale groups, the two-level format included, stay on the small
  // tiles at every token count: measured faster than the 64-row tiles there)
  const bool small = two_level || rw.group == 32 || sw.group == 32 || (size_t)T * TOPK <= (size_t)SMALL_TILE_MAX_SLOTS;
  const bool pair = small && small_pair_available(rw.bits, rw.group, sw.bits, sw.group);
  const int mtl = !small ? MT : (pair && (size_t)T * TOPK <= TINY_TILE_MAX_SLOTS) ? MT_TINY : MT_SMALL;
  const int max_tiles = (int)((size_t)T * TOPK / mtl) + E + 1;
  HistArgs ha;
  ha.ids = topk_ids; ha.T = T; ha.counts = ws.counts; ha.offsets = ws.offsets;
  ha.perm = ws.perm; ha.pos_of = ws.pos_of; ha.tiles = ws.tiles; ha.ntiles = ws.ntiles; ha.mt = mtl;
  ha.blkcnt = ws.blkcnt;
  if (launch_hist(ha, s) != hipSuccess) return MOE_E_HIP;

  GroupedArgs ga;
  ga.T = T; ga.tiles = ws.tiles; ga.ntiles = ws.ntiles; ga.offsets = ws.offsets; ga.perm = ws.perm;
  ga.ksplit = 1;
  const int s_tiles = (T + mtl - 1) / mtl;
  // routed gate/up: A rows are tokens gathered through the permutation;
  // shared gate/up over all tokens
  GroupedArgs gr = ga, gs = ga;
  gr.af = xf; gr.ab = xb; gr.shared = 0; gr.a_by_token = 1; gr.a_rows = T; gr.w = rw; gr.out = ws.h_routed;
  gs.af = xf; gs.ab = xb; gs.shared = 1; gs.a_by_token = 1; gs.a_rows = T; gs.w = sw; gs.out = ws.h_shared;
  // routed down: A rows are h in sorted order; with small tiles the shared
  // down has few row tiles, so two K halves double its workgroups
  GroupedArgs dr = ga, ds = ga;
  dr.af = ws.h_routed; dr.ab = nullptr; dr.shared = 0; dr.a_by_token = 0; dr.a_rows = T * TOPK; dr.w = rw;
  dr.out = ws.ysorted;
  ds.af = ws.h_shared; ds.ab = nullptr; ds.shared = 1; ds.a_by_token = 0; ds.a_rows = T; ds.w = sw; ds.out = ws.ys;
  ds.ksplit = small ? 2 : 1;
  if (pair && launch_small_pair(gr, max_tiles, gs, s_tiles, false, mtl, s)) {
    if (hipGetLastError() != hipSuccess) return MOE_E_HIP;
    if (!launch_small_pair(dr, max_tiles, ds, s_tiles, true, mtl, s) || hipGetLastError() != hipSuccess) return MOE_E_HIP;
  } else if (two_level) {
    auto gateup = [&](const GroupedArgs& g, int tiles) {
      return g.w.group == Q4K ? launch_grouped_q4k(g, tiles, false, s) : launch_grouped_gateup(g, tiles, true, s);
    };
    auto down = [&](const GroupedArgs& g, int tiles) {
      return g.w.group == Q4K ? launch_grouped_q4k(g, tiles, true, s) : launch_grouped_down(g, tiles, true, s);
    };
    if (gateup(gr, max_tiles) != hipSuccess || gateup(gs, s_tiles) != hipSuccess ||
        down(dr, max_tiles) != hipSuccess || down(ds, s_tiles) != hipSuccess)
      return MOE_E_HIP;
  } else {
    if (launch_grouped_gateup(gr, max_tiles, small, s) != hipSuccess) return MOE_E_HIP;
    if (launch_grouped_gateup(gs, s_tiles, small, s) != hipSuccess) return MOE_E_HIP;
    if (launch_grouped_down(dr, max_tiles, small, s) != hipSuccess) return MOE_E_HIP;
    if (launch_grouped_down(ds, s_tiles, small, s) != hipSuccess) return MOE_E_HIP;
  }
  CombineArgs ca;
  ca.ys = ws.ys; ca.ys2 = small ? ws.ys + (size_t)T * H : nullptr; ca.ysorted = ws.ysorted; ca.pos_of = ws.pos_of; ca.tw = topk_w;
  ca.y = y; ca.T = T; ca.accumulate = accumulate;
  if (launch_combine(ca, s) != hipSuccess) return MOE_E_HIP;
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status_t moe_layer_forward(const void* x, int32_t x_dtype, int32_t n_tokens,
                               const float* router_w, const float* router_b,
                               const void* expert_q, const float* expert_scales,
                               int32_t expert_bits, int32_t expert_group,
                               const void* shared_q, const float* shared_scales,
                               int32_t shared_bits, int32_t shared_group,
                               float* y, int32_t* topk_ids, float* topk_w,
                               void* workspace, size_t workspace_bytes,
                               uint32_t flags, void* stream) {
  return layer_forward(x, x_dtype, n_tokens, router_w, router_b, expert_q, expert_scales, expert_bits,
                       expert_group, shared_q, shared_scales, shared_bits, shared_group, y, topk_ids, topk_w,
                       workspace, workspace_bytes, flags, stream, DECODE_FORCE_MAX_T);
}

moe_status_t moe_layer_forward_static(const void* x, int32_t x_dtype, int32_t n_tokens,
                                      const float* router_w, const float* router_b,
                                      const void* expert_q, const float* expert_scales,
                                      int32_t expert_bits, int32_t expert_group,
                                      const void* shared_q, const float* shared_scales,
                                      int32_t shared_bits, int32_t shared_group,
                                      float* y, int32_t* topk_ids, float* topk_w,
                                      uint32_t flags, void* stream) {
  if (n_tokens < 0 || n_tokens > STATIC_MAX_T) return MOE_E_SHAPE;
  if (carve(nullptr, n_tokens, DECODE_MAX_T).bytes > STATIC_SCRATCH_BYTES) return MOE_E_WORKSPACE;
  void* ws = nullptr;
  if (static_scratch(&ws) != hipSuccess) return MOE_E_HIP;
  return layer_forward(x, x_dtype, n_tokens, router_w, router_b, expert_q, expert_scales, expert_bits,
                       expert_group, shared_q, shared_scales, shared_bits, shared_group, y, topk_ids, topk_w,
                       ws, STATIC_SCRATCH_BYTES, flags, stream, DECODE_MAX_T);
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

size_t moe_decode_workspace_bytes(void) { return carve_decode(nullptr).bytes; }

moe_status_t moe_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return MOE_E_NULLPTR;
  if (!aligned16(workspace)) return MOE_E_ALIGN;
  const DecodeWorkspace dw = carve_decode(workspace);
  if (workspace_bytes < dw.bytes) return MOE_E_WORKSPACE;
  (void)hipGetLastError();
  if (launch_zero_words((uint32_t*)workspace, dw.clear_words, (hipStream_t)stream) != hipSuccess) return MOE_E_HIP;
  return MOE_OK;
}

moe_status_t moe_decode_forward(const void* x, int32_t x_dtype, float* y, int32_t n_layers,
                                const moe_layer_weights_t* layers, int32_t expert_bits, int32_t expert_group,
                                int32_t shared_bits, int32_t shared_group, int32_t* topk_ids, float* topk_w,
                                void* workspace, size_t workspace_bytes, uint32_t flags, void* stream) {
  if (!x || !y || !layers || !topk_ids || !topk_w || !workspace) return MOE_E_NULLPTR;
  if (n_layers < 1 || n_layers > MOE_DECODE_MAX_LAYERS) return MOE_E_SHAPE;
  if (!fmt_ok(expert_bits, expert_group) || !fmt_ok(shared_bits, shared_group)) return MOE_E_FORMAT;
  if (flags & ~(uint32_t)(MOE_ACCUMULATE | MOE_NORM_INPUT)) return MOE_E_ARG;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_E_ARG;
  if (x == (const void*)y && x_dtype != MOE_F32) return MOE_E_ARG;
  if (!aligned16(workspace) || ((uintptr_t)x & 3u) || ((uintptr_t)y & 3u) || ((uintptr_t)topk_ids & 3u) ||
      ((uintptr_t)topk_w & 3u))
    return MOE_E_ALIGN;
  ChainArgs a;
  memset(&a, 0, sizeof(a));
  for (int l = 0; l < n_layers; ++l) {
    const moe_layer_weights_t& L = layers[l];
    if (!L.router_w || !L.expert_q || !L.expert_scales || !L.shared_q || !L.shared_scales) return MOE_E_NULLPTR;
    if (!aligned16(L.expert_q) || !aligned16(L.shared_q) || ((uintptr_t)L.router_w & 3u) ||
        ((uintptr_t)L.router_b & 3u) || ((uintptr_t)L.expert_scales & 3u) || ((uintptr_t)L.shared_scales & 3u))
      return MOE_E_ALIGN;
    a.layer[l].wr = L.router_w; a.layer[l].bias = L.router_b;
    a.layer[l].eq = (const uint8_t*)L.expert_q; a.layer[l].es = L.expert_scales;
    a.layer[l].sq = (const uint8_t*)L.shared_q; a.layer[l].ss = L.shared_scales;
  }
  const DecodeWorkspace dw = carve_decode(workspace);
  if (workspace_bytes < dw.bytes) return MOE_E_WORKSPACE;
  a.n_layers = n_layers;
  a.x = x; a.x_bf16 = x_dtype == MOE_BF16; a.y = y;
  a.norm = (flags & MOE_NORM_INPUT) != 0; a.accumulate = (flags & MOE_ACCUMULATE) != 0; a.eps = 1e-6f;
  a.rbits = expert_bits; a.rgroup = expert_group; a.sbits = shared_bits; a.sgroup = shared_group;
  a.ids = topk_ids; a.tw = topk_w;
  a.hdr = dw.hdr; a.ipart = dw.ipart; a.rec = dw.rec;
#ifdef MOE_DEVICE_TRACE
  a.trace = g_trace_buffer;
#endif
  (void)hipGetLastError();
  if (launch_chain(a, (hipStream_t)stream) != hipSuccess) return MOE_E_HIP;
  return MOE_OK;
}

}  // extern "C"

#ifdef MOE_DEVICE_TRACE
extern "C" int moe_debug_set_trace(void* p) {
  g_trace_buffer = (unsigned long long*)p;
  return 0;
}
#endif
