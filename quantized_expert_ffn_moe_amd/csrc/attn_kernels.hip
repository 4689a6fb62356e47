// gfx950 kernels of one R-SWA (Reference Sliding Window Attention) decode
// step: every generated token attends, per head, to a frozen reference block
// (the visual prefill and prompt prefix) and to the newest generated tokens
// held in a ring of 128 slots (franken_ocr README, "Design Philosophy":
// bounded generated-token KV; browser demo page "A 3-billion-parameter OCR
// model. In this tab.", "One forward pass, left to right", step 6: ten heads
// of dimension 128).
//
// Three launches per step:
//  1. the new key and value, rounded to bf16, go into ring slot n_gen mod 128;
//  2. split-KV partials: a workgroup takes one (stream, head, chunk of 64 keys)
//     of the key list [reference block | live ring slots], stages the chunk's
//     keys and values in LDS with coalesced 16-byte loads, and leaves the
//     chunk's max score m, sum of exp(s - m) and unnormalised output;
//  3. per (stream, head) the chunks merge in chunk order (fixed, so the result
//     is bitwise reproducible) into softmax(q k / sqrt(128)) v.
// The KV streams through once per step: HBM-bound for many streams.
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
}  // namespace

// 1. ring write: one workgroup per stream, thread = (head, 5 dims)
__global__ __launch_bounds__(256) void rswa_ring_write_kernel(RswaArgs a) {
  const int s = blockIdx.x;
  const int slot = max(a.n_gen[s], 0) % RSWA_W;
  for (int f = threadIdx.x; f < ATT_HEADS * ATT_D; f += 256) {
    const int h = f / ATT_D, d = f % ATT_D;
    const size_t src = ((size_t)s * ATT_HEADS + h) * ATT_D + d;
    const size_t dst = (((size_t)s * ATT_HEADS + h) * RSWA_W + slot) * ATT_D + d;
    a.ring_k[dst] = to_bf16(a.k_new[src]);
    a.ring_v[dst] = to_bf16(a.v_new[src]);
  }
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
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n_live = live_slots(a.n_gen[s]);
  const int n_keys = a.n_ref + n_live;
  const int j0 = c * RSWA_CHUNK;
  float* part = a.part + (((size_t)s * ATT_HEADS + h) * a.n_chunks + c) * RSWA_PART;
  if (j0 >= n_keys) {                       // past this stream's keys: an empty partial
    if (tid < RSWA_PART) part[tid] = tid == 0 ? -__builtin_inff() : 0.f;
    return;
  }
  const size_t sh = (size_t)s * ATT_HEADS + h;
  const uint16_t* rk = a.ref_k + sh * a.n_ref * ATT_D;
  const uint16_t* rv = a.ref_v + sh * a.n_ref * ATT_D;
  const uint16_t* gk = a.ring_k + sh * RSWA_W * ATT_D;
  const uint16_t* gv = a.ring_v + sh * RSWA_W * ATT_D;
  // stage the chunk: 64 rows x 16 uint4 per matrix, 4 of each per thread
  uint4 kb[4], vb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int f = tid + 256 * i, j = j0 + f / 16, u = f % 16;
    const uint16_t* pk = nullptr;
    const uint16_t* pv = nullptr;
    if (j < a.n_ref) { pk = rk + (size_t)j * ATT_D; pv = rv + (size_t)j * ATT_D; }
    else if (j < n_keys) { pk = gk + (size_t)(j - a.n_ref) * ATT_D; pv = gv + (size_t)(j - a.n_ref) * ATT_D; }
    kb[i] = pk ? *((const uint4*)pk + u) : make_uint4(0, 0, 0, 0);
    vb[i] = pv ? *((const uint4*)pv + u) : make_uint4(0, 0, 0, 0);
  }
  if (tid < ATT_D) ql[tid] = a.q[sh * ATT_D + tid] * a.scale;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int f = tid + 256 * i;
    *((uint4*)kl + f) = kb[i];
    *((uint4*)vl + f) = vb[i];
  }
  __syncthreads();
  // scores: thread (key j = tid / 4, quarter qq = tid % 4 of the 128 dims)
  const int j = tid >> 2, qq = tid & 3;
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
  sc = group_sum<4>(sc);
  const bool valid = j0 + j < n_keys;
  if (!valid) sc = -__builtin_inff();
  const float wm = wave_max(sc);
  if (lane == 0) red[wv] = wm;
  __syncthreads();
  const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));   // finite: key j0 is valid
  const float p = valid ? expf(sc - m) : 0.f;
  if (qq == 0) pl[j] = p;
  const float ws = wave_sum(qq == 0 ? p : 0.f);
  __syncthreads();
  if (lane == 0) red[4 + wv] = ws;
  // p v: thread (dim d = tid % 128, key half = tid / 128)
  const int d = tid & (ATT_D - 1), half = tid >> 7;
  float acc = 0.f;
#pragma unroll 8
  for (int jj = 0; jj < RSWA_CHUNK / 2; ++jj) {
    const int k = half * (RSWA_CHUNK / 2) + jj;
    acc = __fmaf_rn(pl[k], __uint_as_float((uint32_t)vl[k * ATT_D + d] << 16), acc);
  }
  if (half == 1) acc2[d] = acc;
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
  float M = -__builtin_inff();
  for (int c = 0; c < a.n_chunks; ++c) M = fmaxf(M, part[c * RSWA_PART]);
  float L = 0.f, o = 0.f;
  for (int c = 0; c < a.n_chunks; ++c) {
    const float mc = part[c * RSWA_PART];
    if (mc == -__builtin_inff()) continue;
    const float w = expf(mc - M);
    L = __fmaf_rn(part[c * RSWA_PART + 1], w, L);
    o = __fmaf_rn(part[c * RSWA_PART + 2 + d], w, o);
  }
  a.out[((size_t)s * ATT_HEADS + h) * ATT_D + d] = o / L;
}

int rswa_chunks(int n_ref) { return (n_ref + RSWA_W + RSWA_CHUNK - 1) / RSWA_CHUNK; }

hipError_t launch_rswa(const RswaArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(rswa_ring_write_kernel, dim3(a.S), dim3(256), 0, st, a);
  hipLaunchKernelGGL(rswa_chunk_kernel, dim3(a.n_chunks, ATT_HEADS, a.S), dim3(256), 0, st, a);
  hipLaunchKernelGGL(rswa_merge_kernel, dim3(ATT_HEADS, a.S), dim3(ATT_D), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
