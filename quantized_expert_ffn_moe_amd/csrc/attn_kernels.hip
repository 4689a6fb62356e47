// gfx950 kernels of one R-SWA (Reference Sliding Window Attention) decode
// step: every generated token attends, per head, to a frozen reference block
// (the visual prefill and prompt prefix) and to the newest generated tokens
// held in a ring of 128 slots (franken_ocr README, "Design Philosophy":
// bounded generated-token KV; browser demo page "A 3-billion-parameter OCR
// model. In this tab.", "One forward pass, left to right", step 6: ten heads
// of dimension 128).
//
// The key list of a (stream, head) is [reference block | live ring slots],
// taken in chunks of 64 keys whose keys and values are staged in LDS as bf16
// with coalesced 16-byte loads.  The new token's key and value, rounded to
// bf16, stand in for ring slot n_gen mod 128 and are written there by the one
// workgroup whose chunk holds that slot (no other workgroup reads it).
//  * Many streams: one workgroup per (stream, head) walks its chunks with an
//    online softmax (running max, sum and output rescaled per chunk), the next
//    chunk's loads in flight while the current one is multiplied.
//  * Few streams: split-KV, one workgroup per (stream, head, chunk) leaving
//    the chunk's max score, sum of exp(s - max) and unnormalised output, then
//    a merge in chunk order.
// Both orders are fixed, so results are bitwise reproducible.  The KV streams
// through once per step: HBM-bound for many streams.
#include "moe_internal.h"
#include "moe_wave.h"

namespace moe {

namespace {
__device__ __forceinline__ uint16_t to_bf16(float v) {
  const uint32_t u = __float_as_uint(v);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);   // nearest, ties to even
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ int live_slots(int n_gen) { return min(max(n_gen, 0) + 1, RSWA_W); }

// one output element: f32, or as the bf16 halves of the split_row layout
// (hi = bf16(v), lo = bf16(v - hi)) that the attention block's output
// projection reads
__device__ __forceinline__ void store_out(const RswaArgs& a, size_t idx, float v) {
  if (a.out_hl) {
    const uint16_t hi = to_bf16(v);
    uint16_t* g = a.out_hl + (idx & ~(size_t)7) * 2 + (idx & 7);
    g[0] = hi;
    g[8] = to_bf16(v - __uint_as_float((uint32_t)hi << 16));
  } else {
    a.out[idx] = v;
  }
}
}  // namespace

// The key list of one (stream, head).
struct KeyList {
  const uint16_t *rk, *rv;      // reference block rows [n_ref][128]
  uint16_t *gk, *gv;            // ring rows [128][128]
  const float *kn, *vn;         // the new token's key and value [128]
  int n_ref, n_keys, slot;      // the new token sits in ring slot `slot`
};
__device__ __forceinline__ KeyList key_list(const RswaArgs& a, int s, int h) {
  KeyList L;
  const size_t sh = (size_t)s * ATT_HEADS + h;
  L.rk = a.ref_k + sh * a.n_ref * ATT_D;
  L.rv = a.ref_v + sh * a.n_ref * ATT_D;
  L.gk = a.ring_k + sh * RSWA_W * ATT_D;
  L.gv = a.ring_v + sh * RSWA_W * ATT_D;
  L.kn = a.k_new + sh * ATT_D;
  L.vn = a.v_new + sh * ATT_D;
  const int g = max(a.n_gen[s], 0);
  L.n_ref = a.n_ref;
  L.n_keys = a.n_ref + min(g + 1, RSWA_W);
  L.slot = g % RSWA_W;
  return L;
}
// The 16-byte pieces f = tid + 256 i (i < 4) of a chunk's key and value rows
// (row f / 16, piece f % 16): loaded from the reference block or the ring, or
// for the new token's slot formed from its f32 key and value (and written to
// the ring).  Keys past the end read as zeros.
__device__ __forceinline__ uint4 pack8(const float* p) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  return make_uint4((uint32_t)to_bf16(a.x) | ((uint32_t)to_bf16(a.y) << 16),
                    (uint32_t)to_bf16(a.z) | ((uint32_t)to_bf16(a.w) << 16),
                    (uint32_t)to_bf16(b.x) | ((uint32_t)to_bf16(b.y) << 16),
                    (uint32_t)to_bf16(b.z) | ((uint32_t)to_bf16(b.w) << 16));
}
// (A workgroup of NT threads takes chunks of NT / 4 keys: 4 NT pieces of each
// matrix, 4 per thread.)
template <int NT>
__device__ __forceinline__ void fetch_chunk(const KeyList& L, int j0, uint4 (&kb)[4], uint4 (&vb)[4]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int f = tid + NT * i, j = j0 + f / 16, u = f % 16;
    kb[i] = make_uint4(0, 0, 0, 0);
    vb[i] = make_uint4(0, 0, 0, 0);
    if (j < L.n_ref) {
      kb[i] = *((const uint4*)(L.rk + (size_t)j * ATT_D) + u);
      vb[i] = *((const uint4*)(L.rv + (size_t)j * ATT_D) + u);
    } else if (j < L.n_keys) {
      const int r = j - L.n_ref;
      if (r == L.slot) {
        kb[i] = pack8(L.kn + 8 * u);
        vb[i] = pack8(L.vn + 8 * u);
        *((uint4*)(L.gk + (size_t)r * ATT_D) + u) = kb[i];
        *((uint4*)(L.gv + (size_t)r * ATT_D) + u) = vb[i];
      } else {
        kb[i] = *((const uint4*)(L.gk + (size_t)r * ATT_D) + u);
        vb[i] = *((const uint4*)(L.gv + (size_t)r * ATT_D) + u);
      }
    }
  }
}
template <int NT>
__device__ __forceinline__ void stage_chunk(uint16_t* kl, uint16_t* vl, const uint4 (&kb)[4], const uint4 (&vb)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int f = threadIdx.x + NT * i;
    *((uint4*)kl + f) = kb[i];
    *((uint4*)vl + f) = vb[i];
  }
}
// score of key j = tid / 4 over the quarter tid % 4 of the dims, summed over
// the 4 lanes of the key (all four hold it)
__device__ __forceinline__ float chunk_score(const uint16_t* kl, const float* ql) {
  const int j = threadIdx.x >> 2, qq = threadIdx.x & 3;
  float sc = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint4 w = *((const uint4*)(kl + j * ATT_D + 32 * qq) + u);
    const float4 q0 = *(const float4*)&ql[32 * qq + 8 * u];
    const float4 q1 = *(const float4*)&ql[32 * qq + 8 * u + 4];
    sc = __fmaf_rn(bf16_lo(w.x), q0.x, sc); sc = __fmaf_rn(bf16_hi(w.x), q0.y, sc);
    sc = __fmaf_rn(bf16_lo(w.y), q0.z, sc); sc = __fmaf_rn(bf16_hi(w.y), q0.w, sc);
    sc = __fmaf_rn(bf16_lo(w.z), q1.x, sc); sc = __fmaf_rn(bf16_hi(w.z), q1.y, sc);
    sc = __fmaf_rn(bf16_lo(w.w), q1.z, sc); sc = __fmaf_rn(bf16_hi(w.w), q1.w, sc);
  }
  return group_sum<4>(sc);
}
// sum over the 32 keys of this thread's part (tid / 128) of the chunk of
// p_j v_j[d], d = tid % 128
__device__ __forceinline__ float chunk_pv(const uint16_t* vl, const float* pl) {
  const int d = threadIdx.x & (ATT_D - 1), part = threadIdx.x >> 7;
  float acc = 0.f;
#pragma unroll 8
  for (int jj = 0; jj < 32; ++jj) {
    const int k = part * 32 + jj;
    acc = __fmaf_rn(pl[k], __uint_as_float((uint32_t)vl[k * ATT_D + d] << 16), acc);
  }
  return acc;
}

// Many streams: one workgroup of NT threads per (head, stream) = blockIdx
// (x, y), chunks of NT / 4 keys.
template <int NT>
__global__ __launch_bounds__(NT) void rswa_row_kernel(RswaArgs a) {
  constexpr int CH = NT / 4, NW = NT / 64;
  __shared__ __attribute__((aligned(16))) uint16_t kl[CH * ATT_D];
  __shared__ __attribute__((aligned(16))) uint16_t vl[CH * ATT_D];
  __shared__ __attribute__((aligned(16))) float ql[ATT_D];
  __shared__ float pl[CH];
  __shared__ float red[2 * NW];
  __shared__ float acc2[NT > ATT_D ? NT - ATT_D : 1];
  const int h = blockIdx.x, s = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, j = tid >> 2, qq = tid & 3;
  const KeyList L = key_list(a, s, h);
  const int nch = (L.n_keys + CH - 1) / CH;
  uint4 kb[4], vb[4];
  fetch_chunk<NT>(L, 0, kb, vb);
  if (tid < ATT_D) ql[tid] = a.q[((size_t)s * ATT_HEADS + h) * ATT_D + tid] * a.scale;
  float m_run = -__builtin_inff(), l_run = 0.f, acc = 0.f;
  for (int c = 0; c < nch; ++c) {
    __syncthreads();                              // previous chunk's LDS reads are done
    stage_chunk<NT>(kl, vl, kb, vb);
    if (c + 1 < nch) fetch_chunk<NT>(L, (c + 1) * CH, kb, vb);
    __syncthreads();
    const bool valid = c * CH + j < L.n_keys;
    float sc = chunk_score(kl, ql);
    if (!valid) sc = -__builtin_inff();
    const float wm = wave_max(sc);
    if (lane == 0) red[wv] = wm;
    __syncthreads();
    float cm = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) cm = fmaxf(cm, red[w]);
    const float m_new = fmaxf(m_run, cm);
    const float p = valid ? expf(sc - m_new) : 0.f;
    if (qq == 0) pl[j] = p;
    const float ws = wave_sum(qq == 0 ? p : 0.f);
    if (lane == 0) red[NW + wv] = ws;
    __syncthreads();
    float cs = red[NW];
#pragma unroll
    for (int w = 1; w < NW; ++w) cs += red[NW + w];
    const float resc = expf(m_run - m_new);       // 0 on the first chunk
    l_run = __fmaf_rn(l_run, resc, cs);
    acc = __fmaf_rn(acc, resc, chunk_pv(vl, pl));
    m_run = m_new;
  }
  if (NT > ATT_D) {                               // the key parts' sums, in part order
    if (tid >= ATT_D) acc2[tid - ATT_D] = acc;
    __syncthreads();
    if (tid < ATT_D)
#pragma unroll
      for (int p = 0; p < NT / ATT_D - 1; ++p) acc += acc2[ATT_D * p + tid];
  }
  if (tid < ATT_D) store_out(a, ((size_t)s * ATT_HEADS + h) * ATT_D + tid, acc / l_run);
}

// 2. partials of one chunk: blockIdx = (chunk, head, stream)
__global__ __launch_bounds__(256) void rswa_chunk_kernel(RswaArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t kl[RSWA_CHUNK * ATT_D];
  __shared__ __attribute__((aligned(16))) uint16_t vl[RSWA_CHUNK * ATT_D];
  __shared__ __attribute__((aligned(16))) float ql[ATT_D];
  __shared__ float pl[RSWA_CHUNK];
  __shared__ float red[8];
  __shared__ float acc2[ATT_D];
  const int c = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, j = tid >> 2, qq = tid & 3;
  const KeyList L = key_list(a, s, h);
  const int j0 = c * RSWA_CHUNK;
  float* part = a.part + (((size_t)s * ATT_HEADS + h) * a.n_chunks + c) * RSWA_PART;
  if (j0 >= L.n_keys) {                     // past this stream's keys: an empty partial
    if (tid < RSWA_PART) part[tid] = tid == 0 ? -__builtin_inff() : 0.f;
    return;
  }
  static_assert(RSWA_CHUNK == 256 / 4, "split-KV chunks of a 256-thread workgroup");
  uint4 kb[4], vb[4];
  fetch_chunk<256>(L, j0, kb, vb);
  if (tid < ATT_D) ql[tid] = a.q[((size_t)s * ATT_HEADS + h) * ATT_D + tid] * a.scale;
  stage_chunk<256>(kl, vl, kb, vb);
  __syncthreads();
  const bool valid = j0 + j < L.n_keys;
  float sc = chunk_score(kl, ql);
  if (!valid) sc = -__builtin_inff();
  const float wm = wave_max(sc);
  if (lane == 0) red[wv] = wm;
  __syncthreads();
  const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));   // finite: key j0 is valid
  const float p = valid ? expf(sc - m) : 0.f;
  if (qq == 0) pl[j] = p;
  const float ws = wave_sum(qq == 0 ? p : 0.f);
  if (lane == 0) red[4 + wv] = ws;
  __syncthreads();
  const float acc = chunk_pv(vl, pl);
  if (tid >= ATT_D) acc2[tid & (ATT_D - 1)] = acc;
  __syncthreads();
  if (tid < ATT_D) {
    part[2 + tid] = acc + acc2[tid];
    if (tid == 0) {
      part[0] = m;
      part[1] = (red[4] + red[5]) + (red[6] + red[7]);
    }
  }
}

// 3. merge: blockIdx = (head, stream), thread = dim
__global__ __launch_bounds__(ATT_D) void rswa_merge_kernel(RswaArgs a) {
  const int h = blockIdx.x, s = blockIdx.y, d = threadIdx.x;
  const float* part = a.part + ((size_t)s * ATT_HEADS + h) * a.n_chunks * RSWA_PART;
  // all loads of a batch of 8 chunks are issued before any is used (an empty
  // chunk reads as m = -inf, l = 0, o = 0 and gets weight 0)
  float M = -__builtin_inff();
  for (int c0 = 0; c0 < a.n_chunks; c0 += 8) {
    float mc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) mc[i] = c0 + i < a.n_chunks ? part[(c0 + i) * RSWA_PART] : -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 8; ++i) M = fmaxf(M, mc[i]);
  }
  float L = 0.f, o = 0.f;
  for (int c0 = 0; c0 < a.n_chunks; c0 += 8) {
    float mc[8], lc[8], oc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool in = c0 + i < a.n_chunks;
      const float* pc = part + (c0 + i) * RSWA_PART;
      mc[i] = in ? pc[0] : -__builtin_inff();
      lc[i] = in ? pc[1] : 0.f;
      oc[i] = in ? pc[2 + d] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float w = mc[i] == -__builtin_inff() ? 0.f : expf(mc[i] - M);
      L = __fmaf_rn(lc[i], w, L);
      o = __fmaf_rn(oc[i], w, o);
    }
  }
  store_out(a, ((size_t)s * ATT_HEADS + h) * ATT_D + d, o / L);
}

int rswa_chunks(int n_ref) { return (n_ref + RSWA_W + RSWA_CHUNK - 1) / RSWA_CHUNK; }

hipError_t launch_rswa(const RswaArgs& a, hipStream_t st) {
  if (a.S * ATT_HEADS >= RSWA_ROW_MIN_WG) {
    hipLaunchKernelGGL(rswa_row_kernel<RSWA_ROW_THREADS>, dim3(ATT_HEADS, a.S), dim3(RSWA_ROW_THREADS), 0, st, a);
  } else {
    hipLaunchKernelGGL(rswa_chunk_kernel, dim3(a.n_chunks, ATT_HEADS, a.S), dim3(256), 0, st, a);
    hipLaunchKernelGGL(rswa_merge_kernel, dim3(ATT_HEADS, a.S), dim3(ATT_D), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace moe
