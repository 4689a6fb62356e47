// gfx950 kernels of the quantized expert-FFN MoE layer.
//
// The layer (browser demo page "A 3-billion-parameter OCR model. In this tab.",
// "One forward pass, left to right", step 6; franken_ocr README "Architecture"):
// softmax router over 64 experts, greedy top-6 without renormalisation,
// SwiGLU experts on int4/int8 codes with one f32 scale per group of K
// ("Four bits, one shared scale"), two fused shared experts, weighted combine.
//
// Two expert paths:
//  * GEMV path (few tokens; the persistent decode step and the per-token
//    layer path): every (token, pick) streams its expert's packed 1 KiB tiles
//    with 16-byte loads per lane.  The input is written in block floating
//    point as three int8 digit planes, and the int8 matrix cores
//    (v_mfma_i32_16x16x64_i8) multiply them with the codes exactly; the group
//    scale multiplies the exact integer partial sum of its group.  The
//    two-level 4-bit format (Q4_K-style, GEMV path only) runs on the int4
//    tiles of q - 8: W = d sc q - dmin m = s (q - 8) + beta with s = d sc and
//    beta = 8 s - dmin m, so each sub-block adds beta times the sum of its
//    inputs to the scaled integer product.
//  * Grouped path (many tokens): tokens are bucketed per expert (histogram +
//    stable permutation) and each expert's bucket runs as a dense GEMM on the
//    MFMA units (v_mfma_f32_16x16x32_f16).  The codes become exact f16 integers
//    in registers (one AND and one XOR per pair of codes, then one packed f16
//    add); activations are staged in LDS as f16, split into hi + lo halves
//    when they are f32, so the products are exact and only the fp32
//    accumulation rounds.  Group scales are applied to the fp32 partial sums
//    of each group.
#include "moe_internal.h"
#include "moe_wave.h"

#include <mutex>

namespace moe {

// Optional device timestamps for timeline studies: compiled only when
// MOE_DEVICE_TRACE is defined (never in the shipped library).
#ifdef MOE_DEVICE_TRACE
#define MOE_TRACE(a, b, l, e) \
  do { if (threadIdx.x == 0 && (a).trace) (a).trace[((b) * 16 + (l)) * 16 + (e)] = __builtin_amdgcn_s_memrealtime(); } while (0)
#else
#define MOE_TRACE(a, b, l, e) do { } while (0)
#endif

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));

// 16-byte device-scope (L2-coherent, sc1) loads through a bounds-checked buffer
// descriptor: used for everything one workgroup of the persistent kernel reads
// that another one wrote during the same launch.
typedef unsigned int u32x4 __attribute__((vector_size(16)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}
constexpr int CPOL_SC1 = 16;
__device__ __forceinline__ u32x4 load16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, CPOL_SC1);
}
__device__ __forceinline__ float4 as_float4(u32x4 v) {
  return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ float bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// SiLU(g) * u with the hardware exp2 and reciprocal (about 1 ulp each; the
// decode step has it on the path between its gate/up and down products)
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504088896341f * g)) * u;
}

// RMSNorm pieces shared by the router and the standalone norm so that both
// produce bit-identical z: thread tid owns features tid + 256 i (i < 5).
__device__ __forceinline__ float thread_sumsq(const float* v) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 5; ++i) ss = __fmaf_rn(v[i], v[i], ss);
  return ss;
}
__device__ __forceinline__ float inv_rms(const float* red4, float eps) {
  const float ms = ((red4[0] + red4[1]) + (red4[2] + red4[3])) / (float)H;
  return 1.0f / sqrtf(ms + eps);
}

// ---------------------------------------------------------------------------
// Router: (optional RMSNorm) -> 64 logits -> softmax -> greedy top-6.
// One workgroup of 256 threads per 4 tokens, so that even a few hundred tokens
// spread over many compute units.  Pass 1 normalises the rows (the same
// per-thread sums and reduction order as the standalone RMSNorm, so both give
// bit-identical z) into LDS and to z; pass 2: 16 lanes per expert row read
// W_r in coalesced float4 runs (the 327 KB matrix stays in L2) against z from
// LDS and add up across the 16 lanes in a fixed order.  The selection takes
// the largest remaining logit six times (ties to the lower index): the
// softmax is increasing in the logit, so these are the 6 largest
// probabilities.
// ---------------------------------------------------------------------------
// Pass 1 of both routers (256 threads): the TB rows of x starting at token t0
// into LDS as f32 (all loads issued at once; rows past the end read zeros),
// and with the norm, z = RMSNorm(x) (bf16-rounded when asked) both in LDS and
// written out.  The per-token sums of squares use the standalone RMSNorm's
// per-thread order and reduction, so the two give bit-identical z.
template <int TB, int ROW>
__device__ __forceinline__ void router_rows(const RouterArgs& a, int t0, float* zs, float* red,
                                            bool store_z = true) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nt = min(TB, a.T - t0);
  const uint32_t elt = a.x_bf16 ? 2 : 4;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(a.x), (short)0, (uint32_t)a.T * H * elt, 0x00020000);
  if (a.x_bf16) {
    constexpr int NU = TB * H / 8, NV = (NU + 255) / 256;   // uint4 (8 bf16) in all, per thread
    u32x4 v[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int u = tid + 256 * j;
      v[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, u < NU ? ((uint32_t)t0 * H + 8 * u) * 2 : 0x80000000u, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if (tid + 256 * j >= NU) continue;
      const int f0 = 8 * (tid + 256 * j), f = (f0 / H) * ROW + f0 % H;
      float4 lo, hi;
      lo.x = bf16_to_f32((uint16_t)v[j][0]); lo.y = bf16_to_f32((uint16_t)(v[j][0] >> 16));
      lo.z = bf16_to_f32((uint16_t)v[j][1]); lo.w = bf16_to_f32((uint16_t)(v[j][1] >> 16));
      hi.x = bf16_to_f32((uint16_t)v[j][2]); hi.y = bf16_to_f32((uint16_t)(v[j][2] >> 16));
      hi.z = bf16_to_f32((uint16_t)v[j][3]); hi.w = bf16_to_f32((uint16_t)(v[j][3] >> 16));
      *(float4*)&zs[f] = lo;
      *(float4*)&zs[f + 4] = hi;
    }
  } else {
    constexpr int NU = TB * H / 4, NV = (NU + 255) / 256;   // uint4 (4 f32) in all, per thread
    u32x4 v[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int u = tid + 256 * j;
      v[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, u < NU ? ((uint32_t)t0 * H + 4 * u) * 4 : 0x80000000u, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if (tid + 256 * j < NU) {
        const int f0 = 4 * (tid + 256 * j);
        *(float4*)&zs[(f0 / H) * ROW + f0 % H] = as_float4(v[j]);
      }
  }
  __syncthreads();
  if (!a.norm) return;
  // all rows' per-thread sums first, then the wave reductions (independent
  // chains the scheduler interleaves); the same sums in the same order as the
  // standalone RMSNorm
  float ssr[TB];
#pragma unroll
  for (int tt = 0; tt < TB; ++tt) {
    float v[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) v[i] = zs[tt * ROW + tid + 256 * i];
    ssr[tt] = thread_sumsq(v);
  }
#pragma unroll
  for (int tt = 0; tt < TB; ++tt) {
    const float ss = wave_sum(ssr[tt]);
    if (lane == 0) red[tt * 4 + wv] = ss;
  }
  __syncthreads();
  // 1/rms of row tt once, by thread tt, into red[tt][0]
  float invt = 0.f;
  if (tid < nt) invt = inv_rms(&red[tid * 4], a.eps);
  __syncthreads();
  if (tid < nt) red[tid * 4] = invt;
  __syncthreads();
  // z = x / rms, element by element: thread u takes 8 consecutive columns of
  // a row, so z leaves in 16-byte stores (the values do not depend on which
  // thread forms them)
  constexpr int NG = TB * H / 8;
#pragma unroll
  for (int j = 0; j < (NG + 255) / 256; ++j) {
    const int u = tid + 256 * j;
    if (u >= NG) break;
    const int tt = u / (H / 8), c0 = 8 * (u % (H / 8));
    if (tt >= nt) continue;
    const float inv = red[tt * 4];
    float* zr = &zs[tt * ROW + c0];
    const float4 x0 = *(const float4*)zr, x1 = *(const float4*)(zr + 4);
    float z[8] = {x0.x * inv, x0.y * inv, x0.z * inv, x0.w * inv, x1.x * inv, x1.y * inv, x1.z * inv, x1.w * inv};
    if (a.norm_bf16) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 8; ++i) z[i] = bf16_rne(z[i]);
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = (__float_as_uint(z[2 * i]) >> 16) | (__float_as_uint(z[2 * i + 1]) & 0xFFFF0000u);
      if (store_z) *(uint4*)((uint16_t*)a.z + (size_t)(t0 + tt) * H + c0) = make_uint4(w[0], w[1], w[2], w[3]);
    } else if (store_z) {
      float* zg = (float*)a.z + (size_t)(t0 + tt) * H + c0;
      *(float4*)zg = make_float4(z[0], z[1], z[2], z[3]);
      *(float4*)(zg + 4) = make_float4(z[4], z[5], z[6], z[7]);
    }
    *(float4*)zr = make_float4(z[0], z[1], z[2], z[3]);
    *(float4*)(zr + 4) = make_float4(z[4], z[5], z[6], z[7]);
  }
  __syncthreads();
}

// Greedy top-6 of one token's 64 logits, lane = expert (all lanes active):
// six rounds of "largest remaining logit, lowest index among equals", which
// is the order of the 6 largest softmax probabilities (the softmax is
// increasing).  Lane e_j writes pick j: its expert id and exp(l - max) / sum.
// A NaN logit (a non-finite input row) ranks below every number, and a round
// only looks at lanes not yet picked, so six distinct ids in 0..63 are written
// whatever the values are.
__device__ __forceinline__ void select_top6(float le, int32_t* ids, float* w) {
  const int lane = threadIdx.x & 63;
  const float mx = wave_max(le);
  const float ex = expf(le - mx);
  const float sm = wave_sum(ex);
  const float key = le == le ? le : -__builtin_inff();
  bool picked = false;
#pragma unroll
  for (int j = 0; j < TOPK; ++j) {
    const float m = wave_max(picked ? -__builtin_inff() : key);
    const uint64_t hit = __ballot(!picked && key == m);
    const int ej = (int)__builtin_ctzll(hit);
    if (lane == ej) {
      ids[j] = lane;
      w[j] = ex / sm;
      picked = true;
    }
  }
}

// ---------------------------------------------------------------------------
// Two-pass router up to a thousand tokens: the logits pass splits the experts
// over sixteen workgroups per 4 tokens (each reads one sixteenth of W_r, 20 KB,
// so every compute unit has work and none streams the whole matrix), and a
// selection pass turns each token's 64 logits into its top 6.
// Logits pass: wave w of workgroup (bx, by) owns experts 4 EPW by + EPW w ..;
// lane l owns the columns 4 (64 j + l) .. + 3 (j < 5) and keeps its z values
// in registers, its W_r values in flight all at once; every (expert, token)
// sum is then added across the wave in a fixed order.  The workgroups with
// by = 0 write z.
// ---------------------------------------------------------------------------
// Pick pj (0..5) of select_top6 for one token, lane = expert: the same rounds
// and arithmetic, so the id and the weight are those select_top6 writes.
// Returns the wave-uniform expert id; *w gets its softmax probability.
__device__ __forceinline__ int select_pick(float le, int pj, float* w) {
  const int lane = threadIdx.x & 63;
  const float mx = wave_max(le);
  const float ex = expf(le - mx);
  const float sm = wave_sum(ex);
  const float key = le == le ? le : -__builtin_inff();
  bool picked = false;
  int ej = 0;
  for (int j = 0; j <= pj; ++j) {
    const float m = wave_max(picked ? -__builtin_inff() : key);
    const uint64_t hit = __ballot(!picked && key == m);
    ej = (int)__builtin_ctzll(hit);
    if (lane == ej) picked = true;
  }
  *w = lane_value(ex / sm, ej);
  return ej;
}

constexpr int RS_TB = 4;       // tokens per workgroup

// EPW experts per wave (4 EPW per workgroup, E / (4 EPW) workgroups per
// 4-token block): each workgroup reads 20 EPW KB of W_r.  The sums are the
// same for every EPW (per lane in a fixed order, then across the wave).
template <int EPW>
__global__ __launch_bounds__(256) void router_logits_kernel(RouterArgs a) {
  __shared__ __attribute__((aligned(16))) float zs[RS_TB][H];
  __shared__ float red[RS_TB][4];
  const int t0 = blockIdx.x * RS_TB;
  const int nt = min(RS_TB, a.T - t0);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int e0 = 4 * EPW * blockIdx.y + EPW * wv;
  float4 w[EPW][H / 256];
#pragma unroll
  for (int e = 0; e < EPW; ++e)
#pragma unroll
    for (int j = 0; j < H / 256; ++j) w[e][j] = *(const float4*)(a.wr + (size_t)(e0 + e) * H + 4 * (64 * j + lane));
  router_rows<RS_TB, H>(a, t0, &zs[0][0], &red[0][0], blockIdx.y == 0);
  float acc[EPW][RS_TB];
#pragma unroll
  for (int e = 0; e < EPW; ++e)
#pragma unroll
    for (int t = 0; t < RS_TB; ++t) acc[e][t] = 0.f;
#pragma unroll
  for (int j = 0; j < H / 256; ++j)
#pragma unroll
    for (int t = 0; t < RS_TB; ++t) {
      const float4 z4 = *(const float4*)&zs[t][4 * (64 * j + lane)];
#pragma unroll
      for (int e = 0; e < EPW; ++e)
        acc[e][t] += w[e][j].x * z4.x + w[e][j].y * z4.y + w[e][j].z * z4.z + w[e][j].w * z4.w;
    }
  float mine = 0.f;
#pragma unroll
  for (int e = 0; e < EPW; ++e)
#pragma unroll
    for (int t = 0; t < RS_TB; ++t) {
      const float v = wave_sum(acc[e][t]);
      if (lane == e * RS_TB + t) mine = v;
    }
  const int e = lane / RS_TB, t = lane % RS_TB;
  if (lane < EPW * RS_TB && t < nt)
    a.logits[(size_t)(t0 + t) * E + e0 + e] = mine + (a.bias ? a.bias[e0 + e] : 0.f);
}

// Selection pass: wave = token, lane = expert.
__global__ __launch_bounds__(256) void router_select_kernel(RouterArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t < a.T) select_top6(a.logits[(size_t)t * E + (threadIdx.x & 63)], a.ids + (size_t)t * TOPK, a.w + (size_t)t * TOPK);
}

// ---------------------------------------------------------------------------
// GEMV arithmetic: exact integer products on the matrix cores.  A vector is
// written in block floating point: a block of consecutive elements shares 2^e
// with max|x| < 2^e, and each element becomes a signed integer mantissa
// m = rint(x * 2^(XF - e)), |m| <= 2^XF, XF = 22, held as three balanced
// base-256 digits d_p in [-128, 128): m = d_0 + 256 d_1 + 65536 d_2.  The
// digits are int8, so v_mfma_i32_16x16x{64,32}_i8 multiplies them by int8
// weight codes with exact int32 sums: the three digit planes are rows 0..2 of
// the A operand and the 16 rows of a packed weight tile are the 16 columns of
// B.  A 4-bit code enters B as 16 * code (its nibble moved to the top of an
// int8), which the block unit absorbs (2^-4).  The planes are recombined in
// f32 per scale group, f = C_0 + 256 C_1 + 65536 C_2, and the group's f32
// scale applied once.  The only roundings are that of m (at most 2^-(XF+1) of
// 2^e) and the f32 recombination and accumulation across groups.
//
// Operand layout.  A lane l of a 16x16 product supplies A row l % 16 and
// B column l % 16 for lane group q = l / 16, and the same K positions in both;
// C[4 q + v][l % 16] comes back in register v of lane l, so lanes 0..15 hold
// the three recombinable sums of weight row l % 16.  In a packed tile, lane
// (r, q) holds row r at columns 32 c + 8 q + (0..7) of its word(s) of chunk c,
// so one 64-column unit (x64 product) of a lane is chunks 0 and 1 of the unit:
// the digits of A are stored in that same order.  int8 words are used as
// they are; a 4-bit word splits into its even codes (one int8 operand word)
// and its odd codes (another), so the A digits of each 8-element block are
// stored even elements first.
// ---------------------------------------------------------------------------
constexpr int XF = 22;
constexpr uint32_t XOFF = 0x808080u;   // m + XOFF has digits d_p + 128 (ordinary base-256 digits)
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 mfma_x64(const i32x4& a, const i32x4& b, const i32x4& c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ i32x4 mfma_x32(uint64_t a, uint64_t b) {
  const i32x4 z = {0, 0, 0, 0};
  return __builtin_amdgcn_mfma_i32_16x16x32_i8((long)a, (long)b, z, 0, 0, 0);
}
__device__ __forceinline__ uint64_t pack64(uint32_t lo, uint32_t hi) { return ((uint64_t)hi << 32) | lo; }

// int8 operand words of a 4-bit code word: 16 * even codes, 16 * odd codes
__device__ __forceinline__ uint32_t even_codes(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t odd_codes(uint32_t w) { return w & 0xF0F0F0F0u; }

// B operand of x64 unit u (0 or 1 for int4, 0 for int8) of a lane's tile words
template <int BITS>
__device__ __forceinline__ i32x4 unit_b(const uint4& v, int u) {
  if (BITS == 8) return (i32x4){(int)v.x, (int)v.y, (int)v.z, (int)v.w};
  const uint32_t w0 = word_of(v, 2 * u), w1 = word_of(v, 2 * u + 1);
  return (i32x4){(int)even_codes(w0), (int)odd_codes(w0), (int)even_codes(w1), (int)odd_codes(w1)};
}

// f32 value of the three digit-plane sums in registers 0..2 of C
__device__ __forceinline__ float digits_value(const i32x4& c) {
  return fmaf(65536.0f, (float)c[2], (float)(c[0] + 256 * c[1]));
}

// Byte position of element i (0..7) of an 8-element block in an A operand
template <int BITS>
__device__ __forceinline__ int digit_pos(int i) {
  return BITS == 4 ? ((i & 1) ? 4 + (i >> 1) : (i >> 1)) : i;
}

// Digits of the input vector x * mul for weights of BITS: thread kg < n/8 owns
// elements 8kg..8kg+7; blocks of `blk` elements (blk / 8 consecutive lanes of
// one wave) share an exponent.  xa: [unit k / 64][plane 0..3][q][4 words] (the
// unused plane 3 is never written: it only feeds C rows that are not read);
// xs[block] = 2^(e - XF) (2^(e - XF - 4) for int4: the 16x codes).
// With SUMS (blocks of 32 only), xsum[block] = 8 x the f32 sum of the
// block's elements of x * mul (the two-level format's minimum term).
template <int BITS, bool SUMS = false>
__device__ __forceinline__ void x_digits(const float* x, float mul, int kg, int blk, uint32_t* xa, float* xs,
                                         bool active, float* xsum = nullptr) {
  float v[8];
  float amax = 0.f, vsum = 0.f;
  if (active) {
    *(float4*)&v[0] = *(const float4*)&x[8 * kg];
    *(float4*)&v[4] = *(const float4*)&x[8 * kg + 4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] *= mul;
      amax = fmaxf(amax, fabsf(v[i]));
    }
    if (SUMS) vsum = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
  }
  amax = blk >= 128 ? group_max<16>(amax) : blk >= 64 ? group_max<8>(amax) : group_max<4>(amax);
  if (SUMS) vsum = group_sum<4>(vsum);
  if (!active) return;
  int e;
  frexpf(amax, &e);                       // amax < 2^e (e = 0 when the block is zero)
  if ((kg & (blk / 8 - 1)) == 0) xs[(8 * kg) / blk] = ldexpf(1.0f, e - XF - (BITS == 4 ? 4 : 0));
  if (SUMS && (kg & 3) == 0) xsum[kg / 4] = 8.0f * vsum;
  uint32_t M[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) M[i] = (uint32_t)((int)rintf(ldexpf(v[i], XF - e)) + (int)XOFF);
  const int unit = kg >> 3, half = (kg >> 2) & 1, q = kg & 3;
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int pos = digit_pos<BITS>(i);
      w[pos >> 2] |= ((M[i] >> (8 * p)) & 255u) << (8 * (pos & 3));
    }
    *(uint2*)&xa[((unit * 4 + p) * 4 + q) * 4 + 2 * half] = make_uint2(w[0] ^ 0x80808080u, w[1] ^ 0x80808080u);
  }
}

// ---------------------------------------------------------------------------
// Decode items.  An item is 32 intermediate columns (slice J) of one expert for
// one token: gate/up rows 32J..32J+31 over all 1280 inputs, h = SiLU(g) * u,
// then the split-K share of the down projection,
//   part[r] = coef * sum_{j in slice} W_d[r, j] h_j   for all 1280 rows r,
// coef being the router weight of the pick (1 for the shared expert).  The
// partials of all items of a token add up to the layer output.  A workgroup of
// 512 threads (8 waves) runs one item; all of the item's weight bytes are
// requested up front (ItemRegs) so that they are in flight together.
// ---------------------------------------------------------------------------
// Plain (cached) loads through a buffer descriptor of `bytes` bytes: offsets
// at or beyond the end return zeros without touching memory, which lets a
// wave issue a fixed number of loads with no branches around them.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t weight_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ uint4 wload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int BITS, int G>
struct ItemRegs {
  static constexpr bool K4 = G == Q4K;     // two-level format (4-bit codes, 32-column sub-blocks)
  static_assert(!K4 || BITS == 4, "the two-level format has 4-bit codes");
  static constexpr int SG = K4 ? Q4K_SUB : G;   // columns per scale
  static constexpr int KB = kb_cols(BITS), NKB = H / KB, CPT = KB / 32;
  static constexpr int GU_TPW = NKB / 2;   // wave w: n-tile w/2 (gate 2J, gate 2J+1, up 2J, up 2J+1), K half w%2
  static constexpr int NGW = (H / 2) / SG; // scale groups in a K half
  static constexpr int NSB = H / Q4K_SB;   // two-level: super-blocks of a gate/up row (5)
  static constexpr int NREC = 3;           // ... that a K half touches (640 columns from 0 or 640)
  static constexpr int DR = down_rows(BITS), NRT = H / DR, D_TPW = (NRT + 7) / 8, RS = DR / 16;
  uint4 gu[GU_TPW];
  float gsc[K4 ? 1 : NGW];
  u32x4 gm[K4 ? NREC : 1];                 // two-level: this lane's row, the K half's super-blocks
  uint4 dn[D_TPW];
  float dns[D_TPW][K4 ? 1 : RS];
  u32x4 dd[K4 ? D_TPW : 1];               // two-level: d | dmin << 16 of this lane's 4 down rows per tile
  uint2 dsm[K4 ? D_TPW : 1];              // ... and their sc | m << 8 halfwords for the slice
};

__device__ __forceinline__ float f16_bits_value(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}
__device__ __forceinline__ float byte_value(uint32_t w, int k) { return (float)((w >> (8 * k)) & 255u); }
// The scales and minimums of a gate/up record as bytes: w1 byte j = sc_j |
// (m_j >> 4) << 6, w2 byte j = sc_{4+j} | (m_{4+j} >> 4) << 6, w3 byte j =
// (m_j & 15) | (m_{4+j} & 15) << 4 (word 0 = d | dmin << 16, f16).
struct Q4kBytes {
  uint32_t sc[2], m[2];   // sc_0..3, sc_4..7, m_0..3, m_4..7, one per byte
};
__device__ __forceinline__ Q4kBytes q4k_bytes(const u32x4& r) {
  Q4kBytes b;
  b.sc[0] = r[1] & 0x3F3F3F3Fu;
  b.sc[1] = r[2] & 0x3F3F3F3Fu;
  b.m[0] = (r[3] & 0x0F0F0F0Fu) | ((r[1] >> 2) & 0x30303030u);
  b.m[1] = ((r[3] >> 4) & 0x0F0F0F0Fu) | ((r[2] >> 2) & 0x30303030u);
  return b;
}

// A pointer or index the whole wave agrees on, as a scalar value (lets buffer
// descriptors live in scalar registers).
template <typename T>
__device__ __forceinline__ T* wave_uniform(T* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T*)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <int BITS, int G>
__device__ __forceinline__ void item_load(ItemRegs<BITS, G>& R, const uint8_t* eq, const float* es, int inter,
                                          int J, int wv, int lane) {
  using IR = ItemRegs<BITS, G>;
  eq = wave_uniform(eq);
  es = wave_uniform(es);
  J = wave_uniform(J);
  wv = wave_uniform(wv);
  constexpr int NG = H / G;
  const size_t mbytes = matrix_bytes(BITS, inter, H);
  const size_t mscales = (size_t)inter * NG;
  const int r = lane & 15;
  const int i = wv >> 1, ntile = 2 * J + (i & 1), mat = i >> 1, kb0 = (wv & 1) * IR::GU_TPW;
  // Issue order = use order (loads return in order): the gate/up scales, the
  // gate/up tiles, then the down scales and tiles, so that the first tiles can
  // be multiplied while later ones are still in flight.  No branches: the
  // down tiles past the end of the slab read as zeros (buffer range check).
  // gate/up scales are row-major [row][group]: this lane's row, this wave's K half
  // (buffer loads throughout: a pending flat load would make the compiler wait
  // for every outstanding load before the first use of any of them)
  if constexpr (IR::K4) {
    // two-level records [mat][row][5]: this lane's row, super-blocks 2h .. 2h + 2 of K half h
    const uint8_t* gmb = (const uint8_t*)es + (size_t)mat * inter * IR::NSB * Q4K_REC;
    const __amdgpu_buffer_rsrc_t rgm = weight_rsrc(
        gmb + ((size_t)(16 * ntile) * IR::NSB + 2 * (wv & 1)) * Q4K_REC, 16 * IR::NSB * Q4K_REC);
    const uint32_t mo = (uint32_t)(r * IR::NSB) * Q4K_REC;
#pragma unroll
    for (int k = 0; k < IR::NREC; ++k) R.gm[k] = __builtin_amdgcn_raw_buffer_load_b128(rgm, mo + k * Q4K_REC, 0, 0);
  } else {
  const __amdgpu_buffer_rsrc_t rgs =
      weight_rsrc(es + mat * mscales + (size_t)(16 * ntile) * NG + (wv & 1) * IR::NGW, 16 * NG * 4);
  const uint32_t go = (uint32_t)(r * NG) * 4;
  if (IR::NGW % 4 == 0) {
#pragma unroll
    for (int g = 0; g < IR::NGW; g += 4) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rgs, go + 4 * g, 0, 0);
#pragma unroll
      for (int t = 0; t < 4; ++t) R.gsc[(g + t) % IR::NGW] = __uint_as_float(v[t]);
    }
  } else if (IR::NGW % 2 == 0) {
#pragma unroll
    for (int g = 0; g < IR::NGW; g += 2) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(rgs, go + 4 * g, 0, 0);
      R.gsc[g] = __uint_as_float(v[0]);
      R.gsc[(g + 1) % IR::NGW] = __uint_as_float(v[1]);
    }
  } else {
#pragma unroll
    for (int g = 0; g < IR::NGW; ++g) R.gsc[g] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rgs, go + 4 * g, 0, 0));
  }
  }
  const __amdgpu_buffer_rsrc_t rg =
      weight_rsrc(eq + mat * mbytes + ((size_t)ntile * IR::NKB + kb0) * TILE, IR::GU_TPW * TILE);
#pragma unroll
  for (int m = 0; m < IR::GU_TPW; ++m) R.gu[m] = wload16(rg, m * TILE + lane * 16);
  const __amdgpu_buffer_rsrc_t rd = weight_rsrc(eq + 2 * mbytes + (size_t)J * IR::NRT * TILE, IR::NRT * TILE);
  if constexpr (IR::K4) {
    // two-level down metadata in tile row order: the d | dmin words of the
    // slice's super-block and the sc | m << 8 halfwords of its sub-block (= the
    // slice), for rows DR rt + 16 j + r, j = 0..3 (tiles past the end read
    // as zeros)
    static_assert(IR::RS == 4, "4 down rows per lane and tile");
    const uint8_t* dmeta = (const uint8_t*)es + q4k_rec_bytes(inter);
    const __amdgpu_buffer_rsrc_t rdd =
        weight_rsrc(dmeta + (size_t)(J / (Q4K_SB / SLICE)) * H * 4, H * 4);
    const __amdgpu_buffer_rsrc_t rsm = weight_rsrc(dmeta + q4k_dd_bytes(inter) + (size_t)J * H * 2, H * 2);
#pragma unroll
    for (int m = 0; m < IR::D_TPW; ++m) {
      const uint32_t rt = wv + 8 * m;
      R.dd[m] = __builtin_amdgcn_raw_buffer_load_b128(rdd, (rt * 16 + r) * 16, 0, 0);
      const auto sm = __builtin_amdgcn_raw_buffer_load_b64(rsm, (rt * 16 + r) * 8, 0, 0);
      R.dsm[m] = make_uint2(sm[0], sm[1]);
      R.dn[m] = wload16(rd, rt * TILE + lane * 16);
    }
    return;
  }
  const int gd = (SLICE * J) / G;
  const __amdgpu_buffer_rsrc_t rds =
      weight_rsrc(es + 2 * mscales + (size_t)gd * IR::NRT * 16 * IR::RS, IR::NRT * 16 * IR::RS * 4);
#pragma unroll
  for (int m = 0; m < IR::D_TPW; ++m) {
    const uint32_t rt = wv + 8 * m;
    const uint32_t so = ((rt * 16 + r) * IR::RS) * 4;
    if (IR::RS == 4) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rds, so, 0, 0);
      R.dns[m][0] = __uint_as_float(v[0]);
      R.dns[m][1 % IR::RS] = __uint_as_float(v[1]);
      R.dns[m][2 % IR::RS] = __uint_as_float(v[2]);
      R.dns[m][3 % IR::RS] = __uint_as_float(v[3]);
    } else {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(rds, so, 0, 0);
      R.dns[m][0] = __uint_as_float(v[0]);
      R.dns[m][1] = __uint_as_float(v[1]);
    }
    R.dn[m] = wload16(rd, rt * TILE + lane * 16);
  }
}

__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_coherent_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct ItemLds {
  uint32_t xa[(H / 64) * 4 * 4 * 4];   // A-operand digits of the layer input: [unit][plane][q][4]
  float xs[H / 32];                    // per-block unit of the input digits
  float gpart[8][16];                  // per-wave gate/up sums of the wave's 16 rows (one K half)
  uint32_t ha[8][4 * 4 * 2];           // per wave: A-operand digits of h: [plane][q][2]
  float hs;                            // unit of the h digits (times 2^-4 for int4 codes)
  float dout[H];                       // down rows of the item in units of hs
  float xsum[H / 32];                  // two-level format: 8 x the per-32-block sums of the input
};

// Digits of the layer input z (in LDS) for weights of format (BITS, G).
template <int BITS, int G>
__device__ __forceinline__ void item_planes(const float* z, float mul, ItemLds& L) {
  const int tid = threadIdx.x;
  x_digits<BITS, G == Q4K>(z, mul, tid, G == Q4K ? Q4K_SUB : G, L.xa, L.xs, tid < H / 8, L.xsum);
  __syncthreads();
}

// x with its lowest bit set to the parity of tag
__device__ __forceinline__ uint32_t with_parity(float x, uint32_t tag) {
  return (__float_as_uint(x) & ~1u) | (tag & 1u);
}
// a value as readers use it: the parity bit cleared, so that what they see
// does not depend on the stage tag (repeated calls give the same bits)
__device__ __forceinline__ float word_value(uint32_t u) { return __uint_as_float(u & ~1u); }
// all four values of a word carry the parity of tag
__device__ __forceinline__ bool word_of_tag(const u32x4& v, uint32_t tag) {
  const uint32_t all1 = v[0] & v[1] & v[2] & v[3], any1 = v[0] | v[1] | v[2] | v[3];
  return ((tag & 1u) ? all1 : ~any1) & 1u;
}

__device__ __forceinline__ void store16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, CPOL_SC1);
}

// Input digits in L.xa/L.xs (item_planes) -> L.dout (the item's down rows) and
// L.hs.  Wave w multiplies the 16 gate/up rows of its n-tile over its K half
// (x64 products, one scale group per G/64 of them; G = 32 splits each into two
// x32 products), every wave forms h = SiLU(g) * u and its digits, then each wave
// takes its down tiles (x32 products over the 32-column slice).  Ends with a
// workgroup barrier.
// Gate/up sums of a two-level item over K half HH (lanes 0..15 hold rows).
// Per super-block record: d * sum_j sc_j (scaled integer product_j + 8 X_j)
// - dmin * sum_j m_j X_j over its sub-blocks j, X_j the sum of the
// sub-block's inputs (W = d sc (q - 8) + 8 d sc - dmin m).
template <int HH>
__device__ __forceinline__ float q4k_gateup(const ItemRegs<4, Q4K>& R, const ItemLds& L, int pl, int q) {
  using IR = ItemRegs<4, Q4K>;
  constexpr int NU = IR::GU_TPW * 2;            // x64 units in a K half
  constexpr int u0 = HH * NU;
  Q4kBytes fb[IR::NREC];
  float Dk[IR::NREC], Mk[IR::NREC];
#pragma unroll
  for (int k = 0; k < IR::NREC; ++k) {
    fb[k] = q4k_bytes(R.gm[k]);
    Dk[k] = 0.f;
    Mk[k] = 0.f;
  }
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const uint4 a4 = *(const uint4*)&L.xa[(((u0 + u) * 4 + pl) * 4 + q) * 4];
    const i32x4 B = unit_b<4>(R.gu[u / 2], u % 2);
    const i32x4 c[2] = {mfma_x32(pack64(a4.x, a4.y), pack64((uint32_t)B[0], (uint32_t)B[1])),
                        mfma_x32(pack64(a4.z, a4.w), pack64((uint32_t)B[2], (uint32_t)B[3]))};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int gg = IR::NGW * HH + 2 * u + t;    // sub-block of the row (0..39)
      const int k = gg / 8 - 2 * HH, j = gg % 8;
      const float x8 = L.xsum[gg];
      const float tt = fmaf(L.xs[gg], digits_value(c[t]), x8);
      Dk[k] = fmaf(byte_value(fb[k].sc[j / 4], j % 4), tt, Dk[k]);
      Mk[k] = fmaf(byte_value(fb[k].m[j / 4], j % 4), x8, Mk[k]);
    }
  }
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < IR::NREC; ++k) {
    acc = fmaf(f16_bits_value(R.gm[k][0] & 0xFFFFu), Dk[k], acc);
    acc = fmaf(-0.125f * f16_bits_value(R.gm[k][0] >> 16), Mk[k], acc);
  }
  return acc;
}

template <int BITS, int G>
__device__ __forceinline__ void item_compute(const ItemRegs<BITS, G>& R, ItemLds& L, int J) {
  using IR = ItemRegs<BITS, G>;
  constexpr int UPT = BITS == 4 ? 2 : 1;          // x64 units per tile
  constexpr int NU = IR::GU_TPW * UPT;            // units in a K half
  constexpr int UPG = G >= 64 ? G / 64 : 1;       // units per scale group (G >= 64)
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, q = lane >> 4, pl = lane & 3;
  const int u0 = (wv & 1) * NU;                   // first unit of the wave's K half
  const i32x4 zero = {0, 0, 0, 0};
  float acc = 0.f;
  i32x4 C = zero;
  if constexpr (IR::K4) {
    acc = (wv & 1) ? q4k_gateup<1>(R, L, pl, q) : q4k_gateup<0>(R, L, pl, q);
  } else {
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const uint32_t* ap = &L.xa[(((u0 + u) * 4 + pl) * 4 + q) * 4];
    const i32x4 B = unit_b<BITS>(R.gu[u / UPT], u % UPT);
    if (G >= 64) {
      C = mfma_x64(*(const i32x4*)ap, B, u % UPG == 0 ? zero : C);
      if (u % UPG == UPG - 1) {
        const int gl = u / UPG;
        acc = fmaf(R.gsc[gl] * L.xs[(u0 * 64) / G + gl], digits_value(C), acc);
      }
    } else {
      const uint4 a4 = *(const uint4*)ap;
      const i32x4 c0 = mfma_x32(pack64(a4.x, a4.y), pack64((uint32_t)B[0], (uint32_t)B[1]));
      const i32x4 c1 = mfma_x32(pack64(a4.z, a4.w), pack64((uint32_t)B[2], (uint32_t)B[3]));
      acc = fmaf(R.gsc[2 * u] * L.xs[2 * u0 + 2 * u], digits_value(c0), acc);
      acc = fmaf(R.gsc[2 * u + 1] * L.xs[2 * u0 + 2 * u + 1], digits_value(c1), acc);
    }
  }
  }
  if (lane < 16) L.gpart[wv][lane] = acc;
  __syncthreads();
  // every wave: h for the 32 slice columns and its digits, into its own copy
  // of the A operand (identical arithmetic in every wave; a wave reads back its
  // own LDS writes in order, so no workgroup barrier is needed)
  uint64_t Ah;
  float xh = 0.f, xh8 = 0.f;
  {
    float hv = 0.f;
    if (lane < SLICE) {
      const int ti = lane >> 4, rr = lane & 15;   // column 16 ti + rr of the slice
      const float g = L.gpart[2 * ti][rr] + L.gpart[2 * ti + 1][rr];
      const float u = L.gpart[4 + 2 * ti][rr] + L.gpart[4 + 2 * ti + 1][rr];
      hv = silu_mul(g, u);
    }
    const float amax = wave_max(fabsf(hv));
    int e;
    frexpf(amax, &e);
    if (tid == 0) L.hs = ldexpf(1.0f, e - XF - (BITS == 4 ? 4 : 0));
    // two-level format: the slice's inputs summed in units of L.hs (16 x the
    // integer mantissas: the unit carries the 2^-4 of the 4-bit codes)
    if (IR::K4) {
      xh = 16.0f * wave_sum(rintf(ldexpf(hv, XF - e)));
      xh8 = 8.0f * xh;
    }
    uint8_t* hb = (uint8_t*)L.ha[wv];
    if (lane < SLICE) {
      const uint32_t M = (uint32_t)((int)rintf(ldexpf(hv, XF - e)) + (int)XOFF);
      const int at = (lane >> 3) * 8 + digit_pos<BITS>(lane & 7);
#pragma unroll
      for (int p = 0; p < 3; ++p) hb[p * 32 + at] = (uint8_t)(((M >> (8 * p)) & 255u) ^ 0x80u);
    }
    Ah = *(const uint64_t*)&L.ha[wv][(pl * 4 + q) * 2];
  }
  // all products first, then the recombination (lanes 0..15 hold the rows);
  // the last tile of waves with one tile fewer is all zeros (range-checked loads)
  float dv[IR::D_TPW][IR::RS];
#pragma unroll
  for (int m = 0; m < IR::D_TPW; ++m) {
#pragma unroll
    for (int j = 0; j < IR::RS; ++j) {
      const uint64_t Bd = BITS == 4 ? pack64(even_codes(word_of(R.dn[m], j)), odd_codes(word_of(R.dn[m], j)))
                                    : pack64(word_of(R.dn[m], 2 * j), word_of(R.dn[m], 2 * j + 1));
      if constexpr (IR::K4) {
        // halfword j = sc | m << 8: W = d sc (q - 8) + 8 d sc - dmin m
        const uint32_t hw = j < 2 ? R.dsm[m].x : R.dsm[m].y;
        const float sc = byte_value(hw, 2 * (j & 1)), mm = byte_value(hw, 2 * (j & 1) + 1);
        const float ds = f16_bits_value(R.dd[m][j] & 0xFFFFu) * sc;
        const float dm = f16_bits_value(R.dd[m][j] >> 16) * mm;
        dv[m][j] = fmaf(ds, digits_value(mfma_x32(Ah, Bd)) + xh8, -dm * xh);
      } else {
        dv[m][j] = R.dns[m][j] * digits_value(mfma_x32(Ah, Bd));
      }
    }
  }
  if (lane < 16) {
#pragma unroll
    for (int m = 0; m < IR::D_TPW; ++m) {
      const int rt = wv + 8 * m;
      if (m < IR::D_TPW - 1 || rt < IR::NRT) {
#pragma unroll
        for (int j = 0; j < IR::RS; ++j) L.dout[IR::DR * rt + 16 * j + lane] = dv[m][j];
      }
    }
  }
  __syncthreads();
}

// Final value of down row `row` of an item: coef * unit(h) * its down sum.
__device__ __forceinline__ float item_row(const ItemLds& L, float cs, int row) { return cs * L.dout[row]; }

// One decode item end to end (loads, planes, compute), 1280 rows to out.
template <int BITS, int G>
__device__ __forceinline__ void run_item(const uint8_t* eq, const float* es, int inter, int J, const float* z,
                                         float coef, float* out, ItemLds& L) {
  const int tid = threadIdx.x;
  ItemRegs<BITS, G> R;
  item_load<BITS, G>(R, eq, es, inter, J, tid >> 6, tid & 63);
  item_planes<BITS, G>(z, 1.0f, L);
  item_compute<BITS, G>(R, L, J);
  const float cs = coef * L.hs;
  for (int row = tid; row < H; row += 512) out[row] = item_row(L, cs, row);
}

template <int BITS, bool K4>
__device__ __forceinline__ void run_item_g(int group, const uint8_t* eq, const float* es, int inter, int J,
                                           const float* z, float coef, float* out, ItemLds& L) {
  if constexpr (K4) {
    run_item<4, Q4K>(eq, es, inter, J, z, coef, out, L);
    return;
  }
  switch (group) {
    case 32: run_item<BITS, 32>(eq, es, inter, J, z, coef, out, L); break;
    case 64: run_item<BITS, 64>(eq, es, inter, J, z, coef, out, L); break;
    default: run_item<BITS, 128>(eq, es, inter, J, z, coef, out, L); break;
  }
}

// Decode path of moe_layer_forward: one workgroup per (token, item).
// QK: bit 0 = routed experts in the two-level format, bit 1 = shared expert
// (separate instantiations keep the symmetric kernels' registers as they were).
// WPE: waves per SIMD the registers are allotted for.  With 4 (two workgroups
// per CU, 128 VGPRs, 28-84 bytes of scratch per lane) one item's weight fetch
// and arithmetic overlap another's: measured 15-21% faster per call from 2
// tokens on (int4 G64 / int8 G128 at 11 tokens 51.5 -> 41.1 us, int4 G128 at
// 10 tokens 45.6 -> 35.9 us) and equal at 1 token.  Expert sets with 32-column
// groups keep 2 (one workgroup per CU, no scratch): with 4 they ran 1-2 us
// slower up to 8 tokens.
template <int BR, int BS, int QK, int WPE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(WPE))) void dec_items_kernel(DecItemsArgs a) {
  __shared__ __attribute__((aligned(16))) float z[H];
  __shared__ __attribute__((aligned(16))) ItemLds L;
  const int t = blockIdx.x / N_ITEMS, item = blockIdx.x % N_ITEMS;
  const int tid = threadIdx.x;
  float* out = a.part + ((size_t)t * N_ITEMS + item) * H;
  // with a.logits (calls of at most DEC_SELF_SELECT_MAX_T tokens): the token's
  // router logits (lane = expert), requested with the input row
  const bool self_select = a.logits != nullptr;
  const float le = self_select && item < R_ITEMS ? a.logits[(size_t)t * E + (tid & 63)] : 0.f;
  for (int k = tid; k < H; k += 512) z[k] = a.xf ? a.xf[(size_t)t * H + k] : bf16_to_f32(a.xb[(size_t)t * H + k]);
  __syncthreads();
  if (item < R_ITEMS) {
    const int p = item / (I / SLICE), J = item % (I / SLICE);
    float coef;
    int e;
    if (self_select) {
      // every wave selects the item's pick itself (no selection launch); the
      // first item of each token reports the token's six picks
      if (item == 0 && tid < 64) select_top6(le, a.ids + (size_t)t * TOPK, a.tw + (size_t)t * TOPK);
      e = select_pick(le, p, &coef);
    } else {
      e = a.ids[(size_t)t * TOPK + p];
      coef = a.tw[(size_t)t * TOPK + p];
    }
    run_item_g<BR, (QK & 1) != 0>(a.rw.group, a.rw.q + (size_t)e * a.rw.e_bytes, a.rw.s + (size_t)e * a.rw.e_scales, I, J, z,
                          coef, out, L);
  } else {
    run_item_g<BS, (QK & 2) != 0>(a.sw.group, a.sw.q, a.sw.s, IS, item - R_ITEMS, z, 1.0f, out, L);
  }
}

// y[t][r] (+)= sum over the token's items of part[t][item][r], items in order.
__global__ __launch_bounds__(256) void dec_reduce_kernel(DecReduceArgs a) {
  __shared__ float red[8][32];
  const int t = blockIdx.x / (H / 32), r0 = (blockIdx.x % (H / 32)) * 32;
  const int tid = threadIdx.x, r = tid & 31, ig = tid >> 5;
  const float* base = a.part + (size_t)t * N_ITEMS * H + r0 + r;
  // every load is issued before the first add (the old output too), so the
  // kernel waits for one round of loads, not one per few items
  static_assert(N_ITEMS % 8 == 0, "items per thread");
  const size_t yi = (size_t)t * H + r0 + tid;
  const float yold = (tid < 32 && a.accumulate) ? a.y[yi] : 0.f;
  float pv[N_ITEMS / 8];
#pragma unroll
  for (int k = 0; k < N_ITEMS / 8; ++k) pv[k] = base[(size_t)(ig + 8 * k) * H];
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < N_ITEMS / 8; ++k) s += pv[k];
  red[ig][r] = s;
  __syncthreads();
  if (tid < 32) {
    float v = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) v += red[g][tid];
    a.y[yi] = yold + v;
  }
}

// ---------------------------------------------------------------------------
// Persistent decode step: one token through n_layers chained layers in one
// launch of 256 co-resident workgroups (one per compute unit).  Workgroups
// 0..223 are items (routed picks 0..5 x 28 slices, then 56 shared slices),
// workgroups 224..255 are reducers owning 40 rows of the residual stream
// each.  Per layer:
//   reducers (stage s): h_s = (h_{s-1}) + sum of the items' partials of layer
//     s-1 for their rows; then a record of those rows of h_s, the partial
//     router logits W_r[:, rows] h_s[rows] and the partial sum of squares;
//   items (layer s): read all 32 records, rebuild RMSNorm(h_s), the 64
//     logits, softmax and top-6 (every routed item computes the same routing),
//     stream their expert slice and write their partial for each reducer.
// Exchange without flags: every 16-byte word carries four f32 values whose
// lowest mantissa bits all hold the parity of the writer's stage tag (a
// counter that runs on across calls: the tags of a call are base + 1 ..
// base + n_layers, and the next call starts at base + n_layers).  A 16-byte
// aligned vector store lands as one piece, so a reader that sees the expected
// parity in all four values sees the word of the current stage.  One bit is
// enough because the chain runs in lock step: an item writes its layer-s
// partial only after every reducer has published its stage-s record, which a
// reducer does only after reading all layer-(s-1) partials (and the same the
// other way round), so a word holds the current stage or the one before it.
// Readers poll the words themselves with device-scope (L2-coherent) loads.
// Writers never wait for their stores, and nothing is cleared between calls.
// (Readers clear the bit: a value moves by at most one ulp, the same in every
// call.)
// ---------------------------------------------------------------------------
constexpr long SPIN_LIMIT = 1L << 20;  // polls before a wait gives up (about a second)

// Lane 0 of each wave polls one word (off[0], valid in lane 0) until it
// carries the parity of `tag`: a few bytes per wave while the writers are still busy.  The
// full loads follow (load_tagged), which check every word.
__device__ __forceinline__ void wait_first(__amdgpu_buffer_rsrc_t r, uint32_t off0, uint32_t tag, long& spins) {
  const int lane = threadIdx.x & 63;
  while (true) {
    bool ok = true;
    if (lane == 0) ok = word_of_tag(load16_coherent(r, off0), tag);
    if (__all(ok)) break;
    __builtin_amdgcn_s_sleep(1);
    if (++spins > SPIN_LIMIT) break;
  }
}

// Load the words at off[m] (where valid[m]) and poll until every one
// carries the parity of `tag` (after wait_first this usually takes one round trip).
// Branch-free: every round issues all N loads back to back, a word that is
// not wanted (invalid, or already carrying the tag) at an offset past the end
// of the buffer, which returns zeros without a memory access; a conditional
// load would be followed by a wait of its own, serialising the round.
// Wave-uniform exit; a wait that runs out sets the error word.
template <int N>
__device__ __forceinline__ void load_tagged(__amdgpu_buffer_rsrc_t r, const uint32_t* off, const bool* valid,
                                            u32x4* v, uint32_t tag, long& spins, uint32_t* err) {
  constexpr uint32_t SKIP = 0x80000000u;
  bool need[N];
#pragma unroll
  for (int m = 0; m < N; ++m) need[m] = valid[m];
  while (true) {
    u32x4 nv[N];
#pragma unroll
    for (int m = 0; m < N; ++m) nv[m] = load16_coherent(r, need[m] ? off[m] : SKIP);
    bool done = true;
#pragma unroll
    for (int m = 0; m < N; ++m) {
#pragma unroll
      for (int k = 0; k < 4; ++k) v[m][k] = need[m] ? nv[m][k] : v[m][k];
      need[m] = need[m] && !word_of_tag(v[m], tag);
      done = done && !need[m];
    }
    if (__all(done)) break;
    __builtin_amdgcn_s_sleep(1);
    if (++spins > SPIN_LIMIT) {
      if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
  }
}

// LDS of the persistent kernel: items and reducers use disjoint parts.
struct ItemSide {
  float z[H];
  ItemLds item;
  float qs[N_RED * Q_STRIDE];
  float lg[E];            // logits
  int pick_e[TOPK];
};
struct ReducerSide {
  float red[N_ITEMS / 7][RED_ROWS];      // per item group, per row
  float hrow[RED_ROWS];
  float rec[REC_U4 * 4];
};
union ChainLds {
  ItemSide it;
  ReducerSide rd;
};

// Wait for the reducer records of stage l, then rebuild this layer's input in
// LDS (z = h, to be multiplied by the returned 1/rms) and, for routed items,
// the picks (softmax_weight gives their weights).  Every workgroup runs identical
// arithmetic, so every item sees the same z, picks and weights.  The 512 threads work as 64 groups of 8
// (group e = expert e): logits and the sum of squares come from the 32 reducer
// partials in a fixed order; the softmax is increasing in the logit, so the 6
// largest logits (ties to the lower index) are the 6 largest probabilities.
__device__ __forceinline__ float chain_layer_input(const ChainArgs& a, const LayerPtrs* LP, ItemSide& S, int l,
                                                   uint32_t epoch, bool routed, bool report, uint32_t* err) {
  const int tid = threadIdx.x;
  // the router bias of this thread's expert, requested before the wait (a
  // layer without bias reads zeros through an empty buffer range)
  const float* bias = LP[l].bias;
  const float bias_e = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
      coherent_rsrc(bias, bias ? E * 4 : 0), (uint32_t)(tid >> 3) * 4, 0, 0));
  {
    constexpr int NR = N_RED * REC_U4;          // 864 words
    constexpr int PT = (NR + 511) / 512;        // 2 per thread
    const __amdgpu_buffer_rsrc_t rr = coherent_rsrc(a.rec, NR * 16);
    uint32_t off[PT];
    bool valid[PT];
    u32x4 v[PT];
#pragma unroll
    for (int m = 0; m < PT; ++m) {
      const int f = tid + 512 * m;
      valid[m] = f < NR;
      off[m] = (uint32_t)f * 16;
    }
    long spins = 0;
    wait_first(rr, off[0], epoch, spins);
    load_tagged<PT>(rr, off, valid, v, epoch, spins, err);
    MOE_TRACE(a, blockIdx.x, l, 1);
#pragma unroll
    for (int m = 0; m < PT; ++m) {
      if (!valid[m]) continue;
      const int f = tid + 512 * m, rid = f / REC_U4, k = f % REC_U4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int vi = 4 * k + i;
        const float val = word_value(v[m][i]);
        if (vi < RED_ROWS) S.z[RED_ROWS * rid + vi] = val;
        else if (vi < RED_ROWS + E) S.qs[rid * Q_STRIDE + vi - RED_ROWS] = val;
        else if (vi == REC_VALS - 1) S.qs[rid * Q_STRIDE + E] = val;
      }
    }
  }
  __syncthreads();
  MOE_TRACE(a, blockIdx.x, l, 6);
  const int e = tid >> 3, sub = tid & 7;
  float part = 0.f, sq = 0.f;
#pragma unroll
  for (int m = 0; m < N_RED / 8; ++m) {
    part += S.qs[(sub + 8 * m) * Q_STRIDE + e];
    sq += S.qs[(sub + 8 * m) * Q_STRIDE + E];
  }
  part = group_sum<8>(part);
  sq = group_sum<8>(sq);
  // 1/rms with the hardware reciprocal square root (about 1 ulp): this sits on
  // the path from the records to the routed weight loads of every layer
  const float inv = a.norm ? __builtin_amdgcn_rsqf(sq * (1.0f / H) + a.eps) : 1.0f;
  if (routed) {
    // a NaN logit (non-finite input) ranks below every number, so the ranks
    // below are a permutation of 0..63 whatever the values are
    const float lraw = part * inv + bias_e;
    const float lge = lraw == lraw ? lraw : -__builtin_inff();
    if (sub == 0) S.lg[e] = lge;
    __syncthreads();
    MOE_TRACE(a, blockIdx.x, l, 7);
    // rank of expert e among the 64 (ties to the lower index): 8 per lane
    int rank = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = sub + 8 * j;
      const float lk = S.lg[k];
      rank += (lk > lge || (lk == lge && k < e)) ? 1 : 0;
    }
    rank = (int)group_sum<8>((float)rank);
    if (sub == 0 && rank < TOPK) {
      S.pick_e[rank] = e;
      if (report) a.ids[l * TOPK + rank] = e;
    }
    __syncthreads();
  }
  MOE_TRACE(a, blockIdx.x, l, 12);
  return inv;
}

// An item's partial (item_compute done, cs = coef * unit of h) as parity
// words [reducer][10]: word w of the item holds rows 4w .. 4w + 3.
__device__ __forceinline__ void chain_item_store(const ChainArgs& a, const ItemLds& L, float cs, int b, uint32_t tag) {
  const int tid = threadIdx.x;
  if (tid < ITEM_U4) {
    const __amdgpu_buffer_rsrc_t rp = coherent_rsrc(a.ipart, N_ITEMS * ITEM_U4 * 16);
    const float4 d = *(const float4*)&L.dout[4 * tid];
    u32x4 w;
    w[0] = with_parity(cs * d.x, tag); w[1] = with_parity(cs * d.y, tag);
    w[2] = with_parity(cs * d.z, tag); w[3] = with_parity(cs * d.w, tag);
    store16_coherent(rp, ((uint32_t)b * ITEM_U4 + tid) * 16, w);
  }
}

// Softmax weight of the logit of expert e among the 64 logits in S.lg (lane i
// of every wave takes logit i: the same arithmetic in every wave and
// workgroup).  Called by all lanes of a wave, after the pick's weight loads are
// issued: only the final scaling of the item's partial needs it.
__device__ __forceinline__ float softmax_weight(const ItemSide& S, int e) {
  const float li = S.lg[threadIdx.x & 63];
  const float mx = wave_max(li);
  const float sm = wave_sum(expf(li - mx));
  return expf(S.lg[e] - mx) / sm;
}

template <int BR, int GR>
__device__ void chain_routed(const ChainArgs& a, const LayerPtrs* LP, ItemSide& S, int b, uint32_t base, uint32_t* err) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int p = b / (I / SLICE), J = b % (I / SLICE);
  const size_t ebytes = 3 * matrix_bytes(BR, I, H), escales = scale_words(GR, I);
  for (int l = 0; l < a.n_layers; ++l) {
    MOE_TRACE(a, b, l, 0);
    const float inv = chain_layer_input(a, LP, S, l, base + l + 1, true, b == 0, err);
    MOE_TRACE(a, b, l, 2);
    const int e = S.pick_e[p];
    ItemRegs<BR, GR> R;
    item_load<BR, GR>(R, LP[l].eq + (size_t)e * ebytes, LP[l].es + (size_t)e * escales, I, J, wv, lane);
    MOE_TRACE(a, b, l, 3);
    const float coef = softmax_weight(S, e);
    if (b == 0) {
      const float wt = softmax_weight(S, S.pick_e[tid < TOPK ? tid : 0]);
      if (tid < TOPK) a.tw[l * TOPK + tid] = wt;
    }
    item_planes<BR, GR>(S.z, inv, S.item);
    MOE_TRACE(a, b, l, 13);
    item_compute<BR, GR>(R, S.item, J);
    MOE_TRACE(a, b, l, 4);
    chain_item_store(a, S.item, coef * S.item.hs, b, base + l + 1);
    MOE_TRACE(a, b, l, 5);
  }
}

template <int BS, int GS>
__device__ void chain_shared(const ChainArgs& a, const LayerPtrs* LP, ItemSide& S, int b, uint32_t base, uint32_t* err) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int J = b - R_ITEMS;
  // The shared slice's weights do not depend on the routing, so they are
  // fetched before the layer's records arrive, but not while the routed items
  // stream theirs (that would share the HBM bandwidth on the critical path):
  // the fetch for layer l + 1 starts 3/8 of a layer period (measured on the
  // 100 MHz real-time clock between record arrivals) after layer l's records.
  uint64_t t_prev = 0, t_go = 0;
  for (int l = 0; l < a.n_layers; ++l) {
    MOE_TRACE(a, b, l, 0);
    while (__builtin_amdgcn_s_memrealtime() < t_go) __builtin_amdgcn_s_sleep(8);
    ItemRegs<BS, GS> R;
    item_load<BS, GS>(R, LP[l].sq, LP[l].ss, IS, J, wv, lane);  // routing-independent: before the wait
    const float inv = chain_layer_input(a, LP, S, l, base + l + 1, false, false, err);
    const uint64_t t_rec = __builtin_amdgcn_s_memrealtime();
    t_go = t_rec + (t_prev ? (t_rec - t_prev) * 3 / 8 : 400u);
    t_prev = t_rec;
    MOE_TRACE(a, b, l, 2);
    item_planes<BS, GS>(S.z, inv, S.item);
    MOE_TRACE(a, b, l, 13);
    item_compute<BS, GS>(R, S.item, J);
    MOE_TRACE(a, b, l, 4);
    chain_item_store(a, S.item, S.item.hs, b, base + l + 1);
    MOE_TRACE(a, b, l, 5);
  }
}

__device__ void chain_reducer(const ChainArgs& a, const LayerPtrs* LP, ReducerSide& S, int rid, uint32_t base, uint32_t* err) {
  const int tid = threadIdx.x;
  const int r0 = rid * RED_ROWS;
  const int e = tid >> 3, sub = tid & 7;      // partial logits: expert e, rows sub + 8m
  // summation: thread t < 320 owns word c = t % 10 (rows 4c..4c+3 of this
  // reducer) of items ig + 32j, ig = t / 10, j = 0..6
  constexpr int NG = N_ITEMS / 7;             // 32 item groups
  const bool summer = tid < NG * PART_U4;
  const int c = tid % PART_U4, ig = tid / PART_U4;
  const __amdgpu_buffer_rsrc_t rp = coherent_rsrc(a.ipart, N_ITEMS * ITEM_U4 * 16);
  const __amdgpu_buffer_rsrc_t rr = coherent_rsrc(a.rec, N_RED * REC_U4 * 16);
  uint32_t off[7];
  bool valid[7];
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    const int it = summer ? ig + NG * j : NG * j;
    valid[j] = summer;
    off[j] = (((uint32_t)it * N_RED + rid) * PART_U4 + (summer ? c : 0)) * 16;
  }
  for (int s = 0; s <= a.n_layers; ++s) {
    float wr[5];
    if (s < a.n_layers) {
#pragma unroll
      for (int m = 0; m < 5; ++m) wr[m] = LP[s].wr[(size_t)e * H + r0 + sub + 8 * m];
    }
    MOE_TRACE(a, N_ITEMS + rid, s, 0);
    if (s == 0) {
      if (tid < RED_ROWS) {
        const int k = r0 + tid;
        const float hv = a.x_bf16 ? bf16_to_f32(((const uint16_t*)a.x)[k]) : ((const float*)a.x)[k];
        S.hrow[tid] = hv;
        S.rec[tid] = hv;
      }
    } else {
      u32x4 v[7];
      long spins = 0;   // each reducer polls its own data directly (nobody else reads it)
      load_tagged<7>(rp, off, valid, v, base + s, spins, err);
      MOE_TRACE(a, N_ITEMS + rid, s, 1);
      if (summer) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 7; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] += word_value(v[j][i]);
#pragma unroll
        for (int i = 0; i < 4; ++i) S.red[ig][4 * c + i] = acc[i];
      }
      __syncthreads();
      // row r = t / 8: groups k, k + 8, k + 16, k + 24 (k = t % 8), then over the 8 lanes
      if (tid < RED_ROWS * 8) {
        const int row = tid >> 3, k = tid & 7;
        float vv = (S.red[k][row] + S.red[k + 8][row]) + (S.red[k + 16][row] + S.red[k + 24][row]);
        vv = group_sum<8>(vv);
        if (k == 0) {
          const float hv = (a.accumulate ? S.hrow[row] : 0.f) + vv;
          S.hrow[row] = hv;
          S.rec[row] = hv;
        }
      }
    }
    __syncthreads();
    if (s == a.n_layers) {
      if (tid < RED_ROWS) a.y[r0 + tid] = S.hrow[tid];
    } else {
      float part = 0.f, sq = 0.f;
#pragma unroll
      for (int m = 0; m < 5; ++m) {
        const float hv = S.hrow[sub + 8 * m];
        part += wr[m] * hv;
        sq += hv * hv;
      }
      part = group_sum<8>(part);
      sq = group_sum<8>(sq);
      if (sub == 0) S.rec[RED_ROWS + e] = part;
      if (tid == 0) S.rec[REC_VALS - 1] = sq;
      __syncthreads();
      if (tid < REC_U4) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int vi = 4 * tid + i;
          w[i] = with_parity(vi < REC_VALS ? S.rec[vi] : 0.f, base + s + 1);
        }
        store16_coherent(rr, ((uint32_t)rid * REC_U4 + tid) * 16, w);
      }
    }
    MOE_TRACE(a, N_ITEMS + rid, s, 5);
  }
}

template <int BR, int BS, int QK>   // QK as for dec_items_kernel
__global__ __launch_bounds__(512) void chain_kernel(ChainArgs a) {
  __shared__ __attribute__((aligned(16))) ChainLds S;
  // the per-layer pointer table, read once from the kernel arguments
  __shared__ __attribute__((aligned(16))) LayerPtrs LP[MAX_LAYERS];
  static_assert(sizeof(LayerPtrs) % 8 == 0, "pointer table copy");
  constexpr int LPW = sizeof(LayerPtrs) / 8;
  if ((int)threadIdx.x < a.n_layers * LPW)
    ((uint64_t*)LP)[threadIdx.x] = ((const uint64_t*)a.layer)[threadIdx.x];
  __syncthreads();
  const int b = blockIdx.x;
  const uint32_t base = load_coherent_u32(a.hdr);   // this call's stage tags are base + 1 .. base + n_layers
  uint32_t* err = a.hdr + 2;
  if (b < R_ITEMS) {
    if constexpr ((QK & 1) != 0) {
      // two-level: workgroup b (on XCD b % 8) takes item 21 (b % 8) + b / 8,
      // so each XCD runs a contiguous run of slices and the 8 slices of a
      // super-block, which share its d | dmin words, mostly share one L2
      chain_routed<4, Q4K>(a, LP, S.it, (b % 8) * (R_ITEMS / 8) + b / 8, base, err);
    } else {
      switch (a.rgroup) {
        case 32: chain_routed<BR, 32>(a, LP, S.it, b, base, err); break;
        case 64: chain_routed<BR, 64>(a, LP, S.it, b, base, err); break;
        default: chain_routed<BR, 128>(a, LP, S.it, b, base, err); break;
      }
    }
  } else if (b < N_ITEMS) {
    if constexpr ((QK & 2) != 0) {
      chain_shared<4, Q4K>(a, LP, S.it, R_ITEMS + (b % 8) * (S_ITEMS / 8) + (b - R_ITEMS) / 8, base, err);
    } else {
      switch (a.sgroup) {
        case 32: chain_shared<BS, 32>(a, LP, S.it, b, base, err); break;
        case 64: chain_shared<BS, 64>(a, LP, S.it, b, base, err); break;
        default: chain_shared<BS, 128>(a, LP, S.it, b, base, err); break;
      }
    }
  } else {
    chain_reducer(a, LP, S.rd, b - N_ITEMS, base, err);
  }
  // the last workgroup to finish advances the stage counter
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(a.hdr + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == gridDim.x - 1) {
      store_coherent_u32(a.hdr + 1, 0u);
      store_coherent_u32(a.hdr, base + (uint32_t)a.n_layers);
    }
  }
}

__global__ void zero_words_kernel(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Router for many tokens: 16 tokens per workgroup, logits on the fp32 matrix
// cores (v_mfma_f32_16x16x4_f32: exact fp32 products, fp32 accumulation).
// Wave w computes the 16 x 16 tile of experts 16w .. 16w + 15: lane (r, q)
// feeds token r / expert 16w + r with inputs kb + 4q + j of each 16-wide K
// step (component j of a float4), so one float4 of z (LDS) and one of W_r
// (global, L2-resident) per lane feed four MFMAs.  Pass 1 (router_rows) is
// that of the two-pass router; the selection is select_top6 per token.
// ---------------------------------------------------------------------------
constexpr int RM_TB = 16;
constexpr int RM_ROW = H + 4;   // padded z rows: the 16 rows an MFMA operand read touches hit distinct banks

__global__ __launch_bounds__(256) void router_mfma_kernel(RouterArgs a) {
  __shared__ __attribute__((aligned(16))) float zs[RM_TB][RM_ROW];     // 80 KB
  __shared__ float red[RM_TB][4];
  __shared__ __attribute__((aligned(16))) float lg[RM_TB][E];
  const int t0 = blockIdx.x * RM_TB;
  const int nt = min(RM_TB, a.T - t0);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  router_rows<RM_TB, RM_ROW>(a, t0, &zs[0][0], &red[0][0]);
  {
    const int r = lane & 15, q = lane >> 4, e = 16 * wv + r;
    // W_r rows of this wave's experts through a buffer descriptor (reads past
    // the row end return zeros), eight 16-wide K steps in flight
    const __amdgpu_buffer_rsrc_t rw = weight_rsrc(a.wr + (size_t)16 * wave_uniform(wv) * H, 16 * H * 4);
    const uint32_t wo = (uint32_t)(r * H + 4 * q) * 4;
    const float* zr = &zs[r][4 * q];
    constexpr int PF = 8;
    // workgroups start their K walk at different blocks of 128 columns, so
    // that they do not all ask the same L2 lines of W_r at the same time
    const int rot = 16 * PF * (int)(blockIdx.x % (H / (16 * PF)));
    auto kwrap = [&](int k) { return k >= H ? k - H : k; };
    u32x4 wq[PF];
#pragma unroll
    for (int j = 0; j < PF; ++j) wq[j] = __builtin_amdgcn_raw_buffer_load_b128(rw, wo + 4 * kwrap(rot + 16 * j), 0, 0);
    // four independent accumulation chains (component j of each float4)
    float4v acc[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll 1
    for (int kb0 = 0; kb0 < H; kb0 += 16 * PF) {
      const int kb = kwrap(kb0 + rot);
#pragma unroll
      for (int j = 0; j < PF; ++j) {
        const u32x4 w4 = wq[j];
        const uint32_t nk = (uint32_t)(kb0 + 16 * PF + 16 * j);
        wq[j] = __builtin_amdgcn_raw_buffer_load_b128(rw, nk < (uint32_t)H ? wo + 4 * (uint32_t)kwrap((int)nk + rot) : 0x80000000u, 0, 0);
        const float4 z4 = *(const float4*)(zr + kb + 16 * j);
        acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(z4.x, __uint_as_float(w4[0]), acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(z4.y, __uint_as_float(w4[1]), acc[1], 0, 0, 0);
        acc[2] = __builtin_amdgcn_mfma_f32_16x16x4f32(z4.z, __uint_as_float(w4[2]), acc[2], 0, 0, 0);
        acc[3] = __builtin_amdgcn_mfma_f32_16x16x4f32(z4.w, __uint_as_float(w4[3]), acc[3], 0, 0, 0);
      }
    }
    const float b = a.bias ? a.bias[e] : 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) lg[4 * q + j][e] = ((acc[0][j] + acc[1][j]) + (acc[2][j] + acc[3][j])) + b;
  }
  __syncthreads();
  // selection: wave w handles tokens w, w + 4, w + 8, w + 12; lane = expert
  for (int tt = wv; tt < nt; tt += 4)
    select_top6(lg[tt][lane], a.ids + (size_t)(t0 + tt) * TOPK, a.w + (size_t)(t0 + tt) * TOPK);
}

// Row tiles of expert e (tiles t0, t0 + 1, ... in row order): one 16-byte
// record each, (expert, first row within the expert, first sorted slot, rows),
// so that a grouped workgroup finds its rows with a single dependent load.
__device__ __forceinline__ void write_tiles(const HistArgs& a, int e, int t0, int off0, int cnt) {
  for (int r0 = 0, t = t0; r0 < cnt; r0 += a.mt, ++t)
    *(int4*)&a.tiles[4 * t] = make_int4(e, r0, off0 + r0, min(a.mt, cnt - r0));
}

// ---------------------------------------------------------------------------
// Histogram + stable permutation of the (token, pick) slots by expert, one
// workgroup of 16 waves.  Wave w owns a contiguous chunk of slots: per-wave
// counts (LDS atomics), an exclusive scan over (expert, wave) gives every
// wave its starting position per expert, then each wave walks its chunk in
// order, 64 slots at a time, and places the slots of one expert at a time
// (ballot + prefix popcount), which keeps the order of slots within an expert.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void hist_kernel(HistArgs a) {
  __shared__ uint8_t sid[MOE_MAX_SLOTS];
  __shared__ int cntw[16][E];
  __shared__ int basew[16][E];
  __shared__ int cnt[E], off[E + 1], toff[E + 1];
  const int N = a.T * TOPK;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int chunk = ((N + 15) / 16 + 63) / 64 * 64;
  const int c0 = wv * chunk, c1 = min(N, c0 + chunk);
  for (int i = tid; i < N; i += 1024) sid[i] = (uint8_t)a.ids[i];
  (&cntw[0][0])[tid] = 0;   // 16 x 64 = 1024 entries
  __syncthreads();
  for (int i = c0 + lane; i < c1; i += 64) atomicAdd(&cntw[wv][sid[i]], 1);
  __syncthreads();
  {   // thread (w, e): slots of expert e in the chunks of waves before w
    const int w = wv, e = lane;
    int run = 0;
    for (int u = 0; u < w; ++u) run += cntw[u][e];
    basew[w][e] = run;
    if (w == 15) cnt[e] = run + cntw[15][e];
  }
  __syncthreads();
  if (wv == 0) {   // exclusive scans over the experts (wave 0, lane = expert)
    const int c = cnt[lane], tl = (c + a.mt - 1) / a.mt;
    int inc = c, tinc = tl;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {   // Hillis-Steele in registers via lane shuffles
      const int o = __shfl_up(inc, d), to = __shfl_up(tinc, d);
      if (lane >= d) { inc += o; tinc += to; }
    }
    off[lane + 1] = inc;
    toff[lane + 1] = tinc;
    if (lane == 0) { off[0] = 0; toff[0] = 0; }
    if (lane == 63) { *a.ntiles = tinc; a.offsets[E] = inc; }
  }
  __syncthreads();
  if (tid < E) {
    a.counts[tid] = cnt[tid];
    a.offsets[tid] = off[tid];
    write_tiles(a, tid, toff[tid], off[tid], cnt[tid]);
  }
  basew[wv][lane] += off[lane];
  __syncthreads();
  // stable placement, 64 slots at a time per wave: the lanes holding the same
  // expert are found with one ballot per bit of the 6-bit expert id; a lane's
  // position is its expert's running base plus the number of such lanes below
  // it, and the lowest of them advances the base.
  const uint64_t below = (1ull << lane) - 1ull;
  for (int g = c0; g < c1; g += 64) {
    const int i = g + lane;
    const bool valid = i < c1;
    const int my_e = valid ? sid[i] : 0;
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int bt = 0; bt < 6; ++bt) {
      const uint64_t ones = __ballot(valid && ((my_e >> bt) & 1));
      same &= ((my_e >> bt) & 1) ? ones : ~ones;
    }
    const int base = basew[wv][my_e];
    const int rank = __popcll(same & below);
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      const int p = base + rank;
      a.perm[p] = i;
      a.pos_of[i] = p;
      if (rank == 0) basew[wv][my_e] = base + __popcll(same);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Many slots: the same result from one workgroup per block of HIST_BLOCK
// slots (wave w of block b owns slots 1024 b + 64 w .. + 63), in two launches:
// every block's counts, then every block places its slots after those of the
// blocks before it (per expert, blocks in order, then waves, then lanes), so
// the permutation is the same stable sort.
__global__ __launch_bounds__(1024) void hist_count_kernel(HistArgs a) {
  __shared__ int cnt[E];
  const int N = a.T * TOPK, tid = threadIdx.x, i = blockIdx.x * HIST_BLOCK + tid;
  if (tid < E) cnt[tid] = 0;
  __syncthreads();
  if (i < N) atomicAdd(&cnt[a.ids[i]], 1);
  __syncthreads();
  if (tid < E) a.blkcnt[blockIdx.x * E + tid] = cnt[tid];
}

__global__ __launch_bounds__(1024) void hist_place_kernel(HistArgs a) {
  __shared__ int cntw[16][E];
  __shared__ int basew[16][E];
  __shared__ int off[E + 1], toff[E + 1], before[E];
  const int N = a.T * TOPK, nb = gridDim.x, b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int i = b * HIST_BLOCK + tid;
  const bool valid = i < N;
  const int my_e = valid ? a.ids[i] : 0;
  (&cntw[0][0])[tid] = 0;   // 16 x 64 = 1024 entries
  if (wv == 0) {   // totals and this block's start per expert (lane = expert), blocks in order
    int tot = 0, bef = 0;
    for (int u = 0; u < nb; ++u) {
      const int c = a.blkcnt[u * E + lane];
      bef += u < b ? c : 0;
      tot += c;
    }
    before[lane] = bef;
    const int tl = (tot + a.mt - 1) / a.mt;
    int inc = tot, tinc = tl;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(inc, d), to = __shfl_up(tinc, d);
      if (lane >= d) { inc += o; tinc += to; }
    }
    off[lane + 1] = inc;
    toff[lane + 1] = tinc;
    if (lane == 0) { off[0] = 0; toff[0] = 0; }
    if (b == 0) {
      a.counts[lane] = tot;
      if (lane == 63) { *a.ntiles = tinc; a.offsets[E] = inc; }
    }
  }
  __syncthreads();
  if (valid) atomicAdd(&cntw[wv][my_e], 1);
  if (b == 0 && tid < E) {
    a.offsets[tid] = off[tid];
    write_tiles(a, tid, toff[tid], off[tid], off[tid + 1] - off[tid]);
  }
  __syncthreads();
  {   // thread (w, e): the expert's start for wave w of this block
    int run = off[lane] + before[lane];
    for (int u = 0; u < wv; ++u) run += cntw[u][lane];
    basew[wv][lane] = run;
  }
  __syncthreads();
  // one round of 64 slots per wave: lanes of the same expert matched by one
  // ballot per bit of the expert id, positions by prefix popcount
  const uint64_t below = (1ull << lane) - 1ull;
  uint64_t same = __ballot(valid);
#pragma unroll
  for (int bt = 0; bt < 6; ++bt) {
    const uint64_t ones = __ballot(valid && ((my_e >> bt) & 1));
    same &= ((my_e >> bt) & 1) ? ones : ~ones;
  }
  if (valid) {
    const int p = basew[wv][my_e] + __popcll(same & below);
    a.perm[p] = i;
    a.pos_of[i] = p;
  }
}

// ---------------------------------------------------------------------------
// Grouped path: exact-integer f16 operands on v_mfma_f32_16x16x32_f16.
// ---------------------------------------------------------------------------
__device__ __forceinline__ half2v as_h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }

// int4 word (codes k0..k7 in nibbles 0..7, two's complement) -> exact f16
// codes in MFMA operand order [k0, k4, k1, k5, k2, k6, k3, k7].  The XOR turns
// every nibble into n = code + 8; 0x6400 | n is the f16 value 1024 + n, and
// 0x6400 | (n << 4) is 1024 + 16n.
__device__ __forceinline__ half8 unpack_int4(uint32_t w) {
  // (nibble ^ 8) = code + 8 under the f16 exponent of 1024: one AND-XOR per
  // pair (the XOR also sets the exponent bits, which the AND cleared)
  const half2v m1032 = {(_Float16)-1032.f, (_Float16)-1032.f};
  const half2v m72 = {(_Float16)-72.f, (_Float16)-72.f};
  const half2v inv16 = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t w8 = w >> 8;
  const half2v a = as_h2((w & 0x000F000Fu) ^ 0x64086408u) + m1032;
  const half2v b = as_h2((w & 0x00F000F0u) ^ 0x64806480u) * inv16 + m72;
  const half2v c = as_h2((w8 & 0x000F000Fu) ^ 0x64086408u) + m1032;
  const half2v d = as_h2((w8 & 0x00F000F0u) ^ 0x64806480u) * inv16 + m72;
  return half8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// two int8 words (codes k0..k3, k4..k7 in bytes, two's complement) -> exact
// f16 codes in order [k0, k2, k1, k3, k4, k6, k5, k7] (byte ^ 0x80 = code + 128).
// Values fetched stages ahead of their use: an empty asm that takes the
// registers as in/out operands keeps every operation on them after this point
// (its place after the stage's workgroup barrier is fixed).  Without it the
// compiler moved the f32/bf16 -> f16 conversion of the A rows up to their
// load, and the wait for that just-issued load drained every fetch in flight
// (the in-order load counter), which left the software pipeline one stage deep.
__device__ __forceinline__ void hold(uint4& v) {
  u32x4 t = {v.x, v.y, v.z, v.w};
  asm volatile("" : "+v"(t));
  v = make_uint4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ void hold(uint2& v) {
  uint32_t x = v.x, y = v.y;
  asm volatile("" : "+v"(x), "+v"(y));
  v = make_uint2(x, y);
}

__device__ __forceinline__ half8 unpack_int8(uint32_t w0, uint32_t w1) {
  const half2v m1152 = {(_Float16)-1152.f, (_Float16)-1152.f};
  const half2v a = as_h2((w0 & 0x00FF00FFu) ^ 0x64806480u) + m1152;
  const half2v b = as_h2(((w0 >> 8) & 0x00FF00FFu) ^ 0x64806480u) + m1152;
  const half2v c = as_h2((w1 & 0x00FF00FFu) ^ 0x64806480u) + m1152;
  const half2v d = as_h2(((w1 >> 8) & 0x00FF00FFu) ^ 0x64806480u) + m1152;
  return half8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// position p of an 8-wide operand slice holds element perm_k<BITS>(p)
template <int BITS> __device__ __forceinline__ int perm_k(int p) {
  return BITS == 4 ? ((p & 1) * 4 + (p >> 1)) : ((p & 4) + ((p & 1) << 1) + ((p >> 1) & 1));
}

constexpr int KS = 128;             // K staged in LDS per step
constexpr int LDS_ROW = KS + 8;     // f16 per LDS row (16-byte pad against bank conflicts)

// Grouped GEMMs come in two tile shapes, both with 8 waves per workgroup:
// 32-row tiles when experts see few rows each, 64 x 256 tiles when they see
// many.  Both stage A (f16, hi and lo planes for
// f32 inputs, permuted within each 8-group into the B operand order) and use
// the same exact-integer B unpacking; the large tiles share B through LDS.
// Small-tile A staging, split into a global fetch (into registers, issued two
// stages ahead) and an LDS store (f16 hi plane, and lo plane when SPLIT,
// permuted within each 8-group into the B operand order).  Thread tid owns the
// 8-element segments tid + 256 j: row = seg / 16, k = 8 (seg % 16).  The loads
// go through a buffer descriptor: padding rows (arow < 0) and stages past the
// end read zeros without a branch, so the compiler can count the loads in
// flight precisely.
template <int MTL, bool F32>
struct AStageS {
  static constexpr int NSEG = MTL / 16;       // segments per thread with 256 threads
  uint4 raw[NSEG][F32 ? 2 : 1];
};

template <int MTL, bool F32>
__device__ __forceinline__ void fetch_a_s(AStageS<MTL, F32>& A, __amdgpu_buffer_rsrc_t ra, const int* arow, int K,
                                        int k0, bool live) {
  const int tid = threadIdx.x;
  constexpr uint32_t ELT = F32 ? 4 : 2;
#pragma unroll
  for (int j = 0; j < AStageS<MTL, F32>::NSEG; ++j) {
    const int seg = tid + 256 * j, row = seg >> 4, kk = 8 * (seg & 15);
    const int src = arow[row];
    const uint32_t off = (live && src >= 0) ? ((uint32_t)src * K + k0 + kk) * ELT : 0x80000000u;
    A.raw[j][0] = wload16(ra, off);
    if (F32) A.raw[j][F32 ? 1 : 0] = wload16(ra, off + 16);
  }
}

template <int BITS, int MTL, bool F32, bool SPLIT>
__device__ __forceinline__ void store_a_s(_Float16* lds, const AStageS<MTL, F32>& A) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < AStageS<MTL, F32>::NSEG; ++j) {
    const int seg = tid + 256 * j, row = seg >> 4, kk = 8 * (seg & 15);
    float v[8];
    if (F32) {
      const uint4 a0 = A.raw[j][0], a1 = A.raw[j][F32 ? 1 : 0];
      v[0] = __uint_as_float(a0.x); v[1] = __uint_as_float(a0.y); v[2] = __uint_as_float(a0.z); v[3] = __uint_as_float(a0.w);
      v[4] = __uint_as_float(a1.x); v[5] = __uint_as_float(a1.y); v[6] = __uint_as_float(a1.z); v[7] = __uint_as_float(a1.w);
    } else {
      const uint4 u = A.raw[j][0];
      const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(uw[i] << 16);
        v[2 * i + 1] = __uint_as_float(uw[i] & 0xFFFF0000u);
      }
    }
    half8 hi, lo;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const float x = v[perm_k<BITS>(p)];
      const _Float16 xh = (_Float16)x;
      hi[p] = xh;
      lo[p] = (_Float16)(x - (float)xh);
    }
    *(half8*)(lds + row * LDS_ROW + kk) = hi;
    if (SPLIT) *(half8*)(lds + MTL * LDS_ROW + row * LDS_ROW + kk) = lo;
  }
}

// Grouped GEMM tiles: a workgroup of 8 waves computes MT = 64 rows x 256
// output columns over K stages of KS = 128.  Per stage the workgroup stages
// the A rows (f16, hi and lo planes for f32 inputs, permuted within each
// 8-group into the B operand order) and the packed B tiles (raw, 1 KiB each)
// in LDS, double-buffered; global loads run two stages ahead in registers so
// that the memory latency hides behind the MFMA work.  Wave (wm, wn) = (w % 2,
// w / 2) owns rows 32 wm .. 32 wm + 31 and four 16-column n-subtiles.  All
// global loads go through buffer descriptors: padding rows and stages past the
// end read zeros without branches, so the compiler counts loads in flight
// exactly.
constexpr int GT = 512;                    // threads per grouped workgroup
constexpr int A_SEG = MT * KS / 8 / GT;    // 8-element A segments per thread per stage (2)

template <bool F32>
struct AStage {
  uint4 raw[A_SEG][F32 ? 2 : 1];
};

__device__ __forceinline__ float wload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

template <bool F32>
__device__ __forceinline__ void fetch_a(AStage<F32>& A, __amdgpu_buffer_rsrc_t ra, const int* arow, int K, int k0,
                                        bool live) {
  const int tid = threadIdx.x;
  constexpr uint32_t ELT = F32 ? 4 : 2;
#pragma unroll
  for (int j = 0; j < A_SEG; ++j) {
    const int seg = tid + GT * j, row = seg >> 4, kk = 8 * (seg & 15);
    const int src = arow[row];
    const uint32_t off = (live && src >= 0) ? ((uint32_t)src * K + k0 + kk) * ELT : 0x80000000u;
    A.raw[j][0] = wload16(ra, off);
    if (F32) A.raw[j][F32 ? 1 : 0] = wload16(ra, off + 16);
  }
}

// The same for an A whose 8-element groups are stored as f16 hi8 then lo8,
// already in operand order (the grouped gate/up output): a copy.
__device__ __forceinline__ void store_a_h16(_Float16* lds, const AStage<true>& A) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < A_SEG; ++j) {
    const int seg = tid + GT * j, row = seg >> 4, kk = 8 * (seg & 15);
    *(uint4*)(lds + row * LDS_ROW + kk) = A.raw[j][0];
    *(uint4*)(lds + MT * LDS_ROW + row * LDS_ROW + kk) = A.raw[j][1];
  }
}

// Position of element k (0..7) of an 8-element group in the operand order
// (the inverse of perm_k).
template <int BITS> __device__ __forceinline__ int perm_pos(int k) {
  return BITS == 4 ? (((k & 3) << 1) | (k >> 2)) : ((k & 4) | ((k & 1) << 1) | ((k >> 1) & 1));
}

// A plane layout in LDS: [row][LDS_ROW] f16 (hi), then the lo plane.
template <int BITS, bool F32, bool SPLIT>
__device__ __forceinline__ void store_a(_Float16* lds, const AStage<F32>& A) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < A_SEG; ++j) {
    const int seg = tid + GT * j, row = seg >> 4, kk = 8 * (seg & 15);
    float v[8];
    if (F32) {
      uint4 a0 = A.raw[j][0], a1 = A.raw[j][F32 ? 1 : 0];
      hold(a0);
      hold(a1);
      v[0] = __uint_as_float(a0.x); v[1] = __uint_as_float(a0.y); v[2] = __uint_as_float(a0.z); v[3] = __uint_as_float(a0.w);
      v[4] = __uint_as_float(a1.x); v[5] = __uint_as_float(a1.y); v[6] = __uint_as_float(a1.z); v[7] = __uint_as_float(a1.w);
    } else {
      uint4 u = A.raw[j][0];
      hold(u);
      const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(uw[i] << 16);
        v[2 * i + 1] = __uint_as_float(uw[i] & 0xFFFF0000u);
      }
    }
    half8 hi, lo;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const float x = v[perm_k<BITS>(p)];
      const _Float16 xh = (_Float16)x;
      hi[p] = xh;
      lo[p] = (_Float16)(x - (float)xh);
    }
    *(half8*)(lds + row * LDS_ROW + kk) = hi;
    if (SPLIT) *(half8*)(lds + MT * LDS_ROW + row * LDS_ROW + kk) = lo;
  }
}

struct TileInfo { int valid, nrows, pbase, row0, e; };

// Workgroup b of a launch is dispatched to XCD b mod 8.  xcd_run(b, n) maps the
// n live workgroups to logical indices so that every XCD takes one contiguous
// run of them: the column blocks of a row tile, and the row tiles of one
// expert, then run on the same XCD and share its L2 (each A tile and each
// expert's B tiles come from HBM about once per XCD that uses them, not once
// per workgroup).  Indices from n on keep their number, find no tile and exit.
__device__ __forceinline__ int xcd_run(int b, int n) {
  if (b >= n) return b;
  const int x = b & 7, j = b >> 3, q = n >> 3, rem = n & 7;
  return x * q + min(x, rem) + j;
}

// Row tiles of a grouped launch: the histogram's count (routed) or the token
// tiles (shared expert).
__device__ __forceinline__ int live_tiles(const GroupedArgs& a, int mtl) {
  return a.shared ? (a.T + mtl - 1) / mtl : *a.ntiles;
}

__device__ __forceinline__ TileInfo tile_info(const GroupedArgs& a, int tile, int mtl) {
  TileInfo ti;
  if (a.shared) {
    ti.row0 = tile * mtl;
    ti.valid = ti.row0 < a.T;
    ti.nrows = min(mtl, a.T - ti.row0);
    ti.pbase = 0; ti.e = 0;
  } else {
    ti.valid = tile < *a.ntiles;
    if (!ti.valid) { ti.nrows = 0; ti.pbase = 0; ti.row0 = 0; ti.e = 0; return ti; }
    const int4 rec = *(const int4*)&a.tiles[4 * tile];   // the histogram's record
    ti.e = rec.x;
    ti.pbase = rec.z;
    ti.nrows = rec.w;
    ti.row0 = 0;
  }
  return ti;
}

// Gate/up: output block cb covers intermediate columns 128 cb .. 128 cb + 127
// of both the gate and the up matrix, so that h = SiLU(gate) * up is formed
// in registers.  Wave w owns all 64 rows of the tile and one 16-column
// n-subtile of each matrix (n-tile 8 cb + w): every packed B word is unpacked
// by exactly one wave.  B per stage: 16 n-tiles x NB packed tiles.
template <int BITS, bool SPLIT, int G>
__global__ __launch_bounds__(GT) void grouped_gateup_kernel(GroupedArgs a) {
  constexpr int KB = kb_cols(BITS), NKB = H / KB, NB = KS / KB, NSTAGE = H / KS, MS = MT / 16;
  constexpr int CPG = G / 32, GPS = KS / G, NG = H / G;
  constexpr bool F32 = SPLIT;
  constexpr int APL = SPLIT ? 2 : 1;
  constexpr int BT = 16 * NB;                       // B tiles per stage
  constexpr int BU = BT * 64 / GT;                  // B uint4 per thread per stage (2 or 4)
  const int inter = a.w.inter, ncb = inter / 128;
  const int lb = xcd_run(blockIdx.x, live_tiles(a, MT) * ncb);
  const int tile = lb / ncb, cb = lb % ncb;
  const TileInfo ti = tile_info(a, tile, MT);
  if (!ti.valid) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = wave_uniform((int)(threadIdx.x >> 6)), r = lane & 15,
            q4 = lane >> 4;
  __shared__ __attribute__((aligned(16))) _Float16 lds_a[2][APL * MT * LDS_ROW];
  __shared__ __attribute__((aligned(16))) uint4 lds_b[2][BT * 64];
  __shared__ int arow[MT];
  if (tid < MT) {
    int src = -1;
    if (tid < ti.nrows) src = a.shared ? ti.row0 + tid : a.perm[ti.pbase + tid] / TOPK;
    arow[tid] = src;
  }
  const int e = wave_uniform(ti.e);
  const uint8_t* eq = a.w.q + (size_t)e * a.w.e_bytes;
  const float* es = a.w.s + (size_t)e * a.w.e_scales;
  const size_t mbytes = matrix_bytes(BITS, inter, H), mscales = (size_t)inter * NG;
  // B: the 16 n-tiles of this block (gate 8cb.., then up 8cb..), each a row of NKB tiles
  const __amdgpu_buffer_rsrc_t rbg = weight_rsrc(eq + (size_t)(8 * cb) * NKB * TILE, 8 * NKB * TILE);
  const __amdgpu_buffer_rsrc_t rbu = weight_rsrc(eq + mbytes + (size_t)(8 * cb) * NKB * TILE, 8 * NKB * TILE);
  // scales of this wave's gate and up n-subtile (row 16 nt + r)
  const int nt = 8 * cb + wv;
  const __amdgpu_buffer_rsrc_t rsg = weight_rsrc(es + (size_t)16 * nt * NG, 16 * NG * 4);
  const __amdgpu_buffer_rsrc_t rsu = weight_rsrc(es + mscales + (size_t)16 * nt * NG, 16 * NG * 4);
  const __amdgpu_buffer_rsrc_t ra =
      weight_rsrc(F32 ? (const void*)a.af : (const void*)a.ab, (uint32_t)a.a_rows * H * (F32 ? 4 : 2));

  struct Stage {
    AStage<F32> A;
    uint4 B[BU];
    float S[2][GPS];
  };
  // uint4 u = tid + GT k of the stage's B: tile bt = u / 64 = (m * 8 + ntl) * NB + h, lane slot u % 64
  auto fetch = [&](Stage& R, int st) {
    fetch_a<F32>(R.A, ra, arow, H, st * KS, st < NSTAGE);
#pragma unroll
    for (int g = 0; g < GPS; ++g) {
      R.S[0][g] = wload4(rsg, (uint32_t)(r * NG + st * GPS + g) * 4);
      R.S[1][g] = wload4(rsu, (uint32_t)(r * NG + st * GPS + g) * 4);
    }
#pragma unroll
    for (int k = 0; k < BU; ++k) {
      const int u = tid + GT * k, bt = u >> 6, sl = u & 63;
      const int h = bt % NB, ntl = (bt / NB) & 7, m = bt / (8 * NB);
      const uint32_t off = (st < NSTAGE) ? ((uint32_t)(ntl * NKB + st * NB + h) * TILE + sl * 16) : 0x80000000u;
      R.B[k] = wload16(m ? rbu : rbg, off);
    }
  };
  auto put = [&](const Stage& R, int buf) {
    store_a<BITS, F32, SPLIT>(lds_a[buf], R.A);
#pragma unroll
    for (int k = 0; k < BU; ++k) lds_b[buf][tid + GT * k] = R.B[k];
  };

  float4v acc[2][MS], ctmp[2][MS];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) { acc[i][ms] = float4v{0, 0, 0, 0}; ctmp[i][ms] = float4v{0, 0, 0, 0}; }
  __syncthreads();   // arow

  // one stage: the registers of stage st (already in LDS) take stage st + 2,
  // the waves multiply stage st, then stage st + 1 (in registers since the
  // previous stage) goes to the other LDS buffer, so every global load has
  // two stages of MFMA work to arrive.  Stages past the end read zeros.
  auto step = [&](int st, Stage& cur, Stage& nxt, int buf) {
    __syncthreads();   // buffer buf holds stage st; buffer buf ^ 1 is free
    float sq[2][GPS];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int g = 0; g < GPS; ++g) sq[i][g] = cur.S[i][g];
    fetch(cur, st + 2);
    const _Float16* la = lds_a[buf];
    const uint4* lb = lds_b[buf];
    uint4 bw[2][NB];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int h = 0; h < NB; ++h) bw[i][h] = lb[((i * 8 + wv) * NB + h) * 64 + lane];
#pragma unroll
    for (int c = 0; c < KS / 32; ++c) {
      const bool first = (c % CPG) == 0, last = (c % CPG) == CPG - 1;
      half8 bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (BITS == 4) bfr[i] = unpack_int4(word_of(bw[i][0], c));
        else bfr[i] = unpack_int8(word_of(bw[i][c >> 1], 2 * (c & 1)), word_of(bw[i][c >> 1], 2 * (c & 1) + 1));
      }
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
        const int lrow = 16 * ms + r, lcol = 32 * c + 8 * q4;
        const half8 ahi = *(const half8*)(la + lrow * LDS_ROW + lcol);
        half8 alo;
        if (SPLIT) alo = *(const half8*)(la + MT * LDS_ROW + lrow * LDS_ROW + lcol);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          float4v cc = first ? float4v{0, 0, 0, 0} : ctmp[i][ms];
          cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bfr[i], cc, 0, 0, 0);
          if (SPLIT) cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bfr[i], cc, 0, 0, 0);
          ctmp[i][ms] = cc;
        }
      }
      if (last) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float sv = sq[i][c / CPG];
#pragma unroll
          for (int ms = 0; ms < MS; ++ms) acc[i][ms] += sv * ctmp[i][ms];
        }
      }
    }
    put(nxt, buf ^ 1);
  };
  Stage R0, R1;
  fetch(R0, 0);
  fetch(R1, 1);
  put(R0, 0);
  static_assert(NSTAGE % 2 == 0, "stage pairs");
#pragma unroll 1
  for (int st = 0; st < NSTAGE; st += 2) {
    step(st, R0, R1, 0);
    step(st + 1, R1, R0, 1);
  }
  // h = SiLU(gate) * up as f16 hi/lo pairs per 8-column group in the down
  // tiles' operand order (h16 layout), staged in LDS (the A buffers are free)
  // and written as whole 16-byte runs: [64 rows][16 groups][hi8, lo8].
  __syncthreads();
  _Float16* hs = &lds_a[0][0];
  static_assert(sizeof(lds_a) >= MT * 128 * 4, "h staging fits the A buffers");
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int m = 16 * ms + 4 * q4 + k, cl = 16 * wv + r;
      const float x = silu_mul(acc[0][ms][k], acc[1][ms][k]);
      const _Float16 xh = (_Float16)x;
      _Float16* g = hs + (m * 16 + (cl >> 3)) * 16;
      const int p = perm_pos<BITS>(cl & 7);
      g[p] = xh;
      g[8 + p] = (_Float16)(x - (float)xh);
    }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < MT * 32 / GT; ++j) {
    const int u = tid + GT * j, m = u >> 5, c16 = u & 31;
    if (m < ti.nrows) {
      const size_t orow = a.shared ? (size_t)(ti.row0 + m) : (size_t)(ti.pbase + m);
      *(uint4*)((char*)a.out + (orow * inter + 128 * cb) * 4 + c16 * 16) = *(const uint4*)(hs + (m * 16) * 16 + c16 * 8);
    }
  }
}

// Down: output block cb covers rows 256 cb .. 256 cb + 255 of W_d (output
// columns of the layer), i.e. NRTB packed row tiles of DR rows; wave (wm, wn)
// owns 64 of them (four 16-row n-subtiles).  A = h as the f16 hi/lo pairs the
// grouped gate/up kernel writes, copied to LDS as they are.
// B per stage: 4 K-chunks of 32 x NRTB row tiles.
template <int BITS, int G, int INTER, int KSPLIT = 1>
__global__ __launch_bounds__(GT) void grouped_down_kernel(GroupedArgs a) {
  constexpr int DR = down_rows(BITS), NRT = H / DR, NRTB = 256 / DR, MS = 2, NSUB = DR / 16;
  constexpr int CPG = G / 32, GPS = KS / G, NSTAGE = INTER / KS / KSPLIT, NCB = H / 256;
  static_assert((INTER / KS) % KSPLIT == 0, "K halves of whole stages");
  constexpr int BT = 4 * NRTB;                      // B tiles per stage (16 or 32)
  constexpr int BU = BT * 64 / GT;
  constexpr int WRT = 4 / NSUB;                     // row tiles per wave (1 or 2)
  // KSPLIT > 1: workgroup kh takes stages kh NSTAGE .. and writes its partial
  // sum to out + kh T H (the combine adds the parts)
  const int lb = xcd_run(blockIdx.x, live_tiles(a, MT) * NCB * KSPLIT);
  const int kh = lb % KSPLIT, tb = lb / KSPLIT, s0 = kh * NSTAGE;
  const int tile = tb / NCB, cb = tb % NCB;
  const TileInfo ti = tile_info(a, tile, MT);
  if (!ti.valid) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = wave_uniform((int)(threadIdx.x >> 6)), r = lane & 15,
            q4 = lane >> 4, wm = wv & 1, wn = wv >> 1;
  __shared__ __attribute__((aligned(16))) _Float16 lds_a[2][2 * MT * LDS_ROW];
  __shared__ __attribute__((aligned(16))) uint4 lds_b[2][BT * 64];
  __shared__ int arow[MT];
  if (tid < MT) arow[tid] = tid < ti.nrows ? (a.shared ? ti.row0 + tid : ti.pbase + tid) : -1;
  const int e = wave_uniform(ti.e);
  const size_t mbytes = matrix_bytes(BITS, INTER, H);
  const int ngk = INTER / G;
  const __amdgpu_buffer_rsrc_t rb = weight_rsrc(a.w.q + (size_t)e * a.w.e_bytes + 2 * mbytes, (uint32_t)mbytes);
  const __amdgpu_buffer_rsrc_t rs =
      weight_rsrc(a.w.s + (size_t)e * a.w.e_scales + 2 * (size_t)INTER * (H / G), (uint32_t)ngk * H * 4);
  const __amdgpu_buffer_rsrc_t ra = weight_rsrc(a.af, (uint32_t)a.a_rows * INTER * 4);

  struct Stage {
    AStage<true> A;
    uint4 B[BU];
    float S[GPS][4];
  };
  // B uint4 u: tile bt = u / 64 = c * NRTB + rtl, lane slot u % 64
  auto fetch = [&](Stage& R, int st) {
    fetch_a<true>(R.A, ra, arow, INTER, (s0 + st) * KS, st < NSTAGE);
#pragma unroll
    for (int g = 0; g < GPS; ++g)
#pragma unroll
      for (int w2 = 0; w2 < WRT; ++w2) {
        const int rt = cb * NRTB + WRT * wn + w2;
        const uint32_t so = ((((uint32_t)((s0 + st) * GPS + g) * NRT + rt) * 16 + r) * NSUB) * 4;
        if (NSUB == 4) {
          const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, so, 0, 0);
#pragma unroll
          for (int j = 0; j < 4; ++j) R.S[g][j] = __uint_as_float(v[j]);
        } else {
          const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, so, 0, 0);
          R.S[g][2 * w2] = __uint_as_float(v[0]);
          R.S[g][2 * w2 + 1] = __uint_as_float(v[1]);
        }
      }
#pragma unroll
    for (int k = 0; k < BU; ++k) {
      const int u = tid + GT * k, bt = u >> 6, sl = u & 63;
      const int c = bt / NRTB, rtl = bt % NRTB;
      const uint32_t off =
          (st < NSTAGE) ? ((uint32_t)((4 * (s0 + st) + c) * NRT + cb * NRTB + rtl) * TILE + sl * 16) : 0x80000000u;
      R.B[k] = wload16(rb, off);
    }
  };
  auto put = [&](const Stage& R, int buf) {
    store_a_h16(lds_a[buf], R.A);
#pragma unroll
    for (int k = 0; k < BU; ++k) lds_b[buf][tid + GT * k] = R.B[k];
  };

  float4v acc[4][MS], ctmp[4][MS];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) { acc[j][ms] = float4v{0, 0, 0, 0}; ctmp[j][ms] = float4v{0, 0, 0, 0}; }
  __syncthreads();   // arow

  auto step = [&](int st, Stage& cur, Stage& nxt, int buf) {
    __syncthreads();
    float sq[GPS][4];
#pragma unroll
    for (int g = 0; g < GPS; ++g)
#pragma unroll
      for (int j = 0; j < 4; ++j) sq[g][j] = cur.S[g][j];
    fetch(cur, st + 2);
    const _Float16* la = lds_a[buf];
    const uint4* lb = lds_b[buf];
#pragma unroll
    for (int c = 0; c < KS / 32; ++c) {
      const bool first = (c % CPG) == 0, last = (c % CPG) == CPG - 1;
      const int lcol = 32 * c + 8 * q4;
      half8 ahi[MS], alo[MS];
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
        ahi[ms] = *(const half8*)(la + (32 * wm + 16 * ms + r) * LDS_ROW + lcol);
        alo[ms] = *(const half8*)(la + MT * LDS_ROW + (32 * wm + 16 * ms + r) * LDS_ROW + lcol);
      }
      uint4 bw[WRT];
#pragma unroll
      for (int w2 = 0; w2 < WRT; ++w2) bw[w2] = lb[(c * NRTB + WRT * wn + w2) * 64 + lane];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int w2 = j / NSUB, jj = j % NSUB;
        const half8 bfr = BITS == 4 ? unpack_int4(word_of(bw[w2], jj))
                                    : unpack_int8(word_of(bw[w2], 2 * jj), word_of(bw[w2], 2 * jj + 1));
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
          float4v cc = first ? float4v{0, 0, 0, 0} : ctmp[j][ms];
          cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[ms], bfr, cc, 0, 0, 0);
          cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[ms], bfr, cc, 0, 0, 0);
          ctmp[j][ms] = cc;
        }
      }
      if (last) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float sj = sq[c / CPG][j];
#pragma unroll
          for (int ms = 0; ms < MS; ++ms) acc[j][ms] += sj * ctmp[j][ms];
        }
      }
    }
    put(nxt, buf ^ 1);
  };
  Stage R0, R1;
  fetch(R0, 0);
  fetch(R1, 1);
  put(R0, 0);
#pragma unroll 1
  for (int st = 0; st + 1 < NSTAGE; st += 2) {
    step(st, R0, R1, 0);
    step(st + 1, R1, R0, 1);
  }
  if (NSTAGE % 2) step(NSTAGE - 1, R0, R1, 0);
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int m = 32 * wm + 16 * ms + 4 * q4 + k;
      if (m < ti.nrows) {
        const size_t orow = a.shared ? (size_t)(ti.row0 + m) : (size_t)(ti.pbase + m);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rt = cb * NRTB + WRT * wn + j / NSUB;
          a.out[(size_t)kh * a.T * H + orow * H + DR * rt + 16 * (j % NSUB) + r] = acc[j][ms][k];
        }
      }
    }
}

// Small tiles (few rows per expert): gate/up, a workgroup of 8 waves owns one
// 32-row tile of one expert and 128 intermediate columns; wave w computes
// gate and up for columns 16w..16w+15 of them (n-subtile 8cb + w of both
// matrices) and writes h = SiLU(gate) * up.  Software pipeline over K stages of 128: the packed B
// tiles and their group scales are fetched D stages ahead into a register
// ring, A two stages ahead (one in registers beyond the one in a double buffer
// in LDS), so that memory latency hides behind the MFMA work and behind the
// second workgroup on the compute unit.
// G = Q4K: the two-level format.  The codes are the int4 tiles of q - 8 and
// each 32-column sub-block adds beta * X to its scaled product (X = the sum of
// the row's inputs over the sub-block, formed while A is staged; s and beta
// from the row's super-block record, fetched with the B tiles).
template <int BITS, bool SPLIT, int G, int MTL, int NW>
__device__ __forceinline__ void gateup_small_body(const GroupedArgs& a, int bid) {
  constexpr bool K4 = G == Q4K;
  static_assert(!K4 || BITS == 4, "two-level codes are 4-bit");
  constexpr int GG = K4 ? Q4K_SUB : G;     // columns per scale
  constexpr int KB = kb_cols(BITS), NKB = H / KB, NB = KS / KB, NSTAGE = H / KS, MS = MTL / 16;
  constexpr int CPG = GG / 32, GPS = KS / GG, NG = H / GG;
  constexpr int NSB = H / Q4K_SB;          // two-level records per gate/up row
  // B stages in flight (D), and A stages fetched ahead into registers (AR - 1
  // of them beyond the one in LDS); the stages run in blocks of SB with a
  // loop between the blocks.  Blocks of 2 stages with 2-deep B and A rings
  // keep every G >= 64 kernel within 128 VGPRs, so that two workgroups share
  // a compute unit and each hides the other's memory waits: the fully
  // unrolled stage loop with 3- and 4-deep rings took 150-250 VGPRs (one
  // workgroup per CU), and measured slower (128-stream step 0.816 against
  // 0.760 ms, 256 streams 1.002 against 0.932 ms, 273-token prefill 76.9
  // against 76.2 us).  With 32-column scale groups (G = 32 and the two-level
  // format) every K step is its own scale group; there a fully unrolled loop
  // also let the compiler hoist matrix-core products far ahead of their scale
  // multiply and spill them (blocks of 6 with 3-deep rings spilled up to 0.8
  // KiB per lane and ran 2.3-2.6x slower).
  constexpr int D = 2;
  constexpr int AR = 2;
  constexpr int SB = 2;
  static_assert((SB % D == 0 && SB % AR == 0 && SB % 2 == 0) || SB == NSTAGE, "ring slots fixed within a block");
  static_assert(!K4 || (SB % 2 == 0 && Q4K_SB == 2 * KS), "a stage is a fixed half of a super-block");
  constexpr bool F32 = SPLIT;
  constexpr int APL = SPLIT ? 2 : 1;
  constexpr int NT = 64 * NW;               // threads of the workgroup
  constexpr int NSEG = MTL * KS / 8;        // A segments (8 elements) per stage
  constexpr int AS = NSEG > NT ? NSEG / NT : 1;   // ... per thread
  static_assert(NSEG <= NT * AS, "every A segment has a thread");
  const int inter = a.w.inter, ncb = inter / (16 * NW);
  const int tile = bid / ncb, cb = bid % ncb;
  const TileInfo ti = tile_info(a, tile, MTL);
  if (!ti.valid) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = wave_uniform((int)(threadIdx.x >> 6)), r = lane & 15,
            q4 = lane >> 4;
  __shared__ __attribute__((aligned(16))) _Float16 lds[2][APL * MTL * LDS_ROW];
  __shared__ __attribute__((aligned(16))) float xsl[2][K4 ? KS / 32 : 1][MTL];   // two-level: 8 X per row, sub-block
  __shared__ int arow[MTL];
  if (tid < MTL) {
    int src = -1;
    if (tid < ti.nrows) src = a.shared ? ti.row0 + tid : a.perm[ti.pbase + tid] / TOPK;
    arow[tid] = src;
  }
  const int e = wave_uniform(ti.e);
  const uint8_t* eq = a.w.q + (size_t)e * a.w.e_bytes;
  const float* es = a.w.s + (size_t)e * a.w.e_scales;
  const size_t mbytes = matrix_bytes(BITS, inter, H), mscales = (size_t)inter * NG;
  // B tiles of this wave: n-subtile NW cb + w of the gate (i = 0) and the up
  // (i = 1) matrix; each descriptor spans one n-tile's row of K tiles
  const int nt = NW * cb + wv;
  __amdgpu_buffer_rsrc_t rb[2], rs[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    rb[i] = weight_rsrc(eq + i * mbytes + (size_t)nt * NKB * TILE, NKB * TILE);
    rs[i] = K4 ? weight_rsrc((const uint8_t*)es + ((size_t)i * inter + 16 * nt) * NSB * Q4K_REC, 16 * NSB * Q4K_REC)
               : weight_rsrc(es + i * mscales + (size_t)16 * nt * NG, 16 * NG * 4);
  }
  const __amdgpu_buffer_rsrc_t ra =
      weight_rsrc(F32 ? (const void*)a.af : (const void*)a.ab, (uint32_t)a.a_rows * H * (F32 ? 4 : 2));

  uint4 bq[D][2][NB];
  float sq[D][2][K4 ? 1 : GPS];
  u32x4 rq[K4 ? D : 1][2];                 // two-level: the row's record of the stage's super-block
  auto load_b = [&](uint4 (&bd)[2][NB], float (&sd)[2][K4 ? 1 : GPS], u32x4 (&rd)[2], int st) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (K4) {
        rd[i] = __builtin_amdgcn_raw_buffer_load_b128(rs[i], (uint32_t)(r * NSB + st / 2) * Q4K_REC, 0, 0);
      } else {
#pragma unroll
        for (int g = 0; g < GPS; ++g) sd[i][g] = wload4(rs[i], (uint32_t)(r * NG + st * GPS + g) * 4);
      }
#pragma unroll
      for (int h = 0; h < NB; ++h) bd[i][h] = wload16(rb[i], (uint32_t)(st * NB + h) * TILE + lane * 16);
    }
  };
  // A: AS 8-element segments per thread per stage (segment u = tid + NT j:
  // row u / 16, columns 8 (u % 16)); when the workgroup has more threads than
  // segments only the first NSEG threads hold one
  const bool a_act = NSEG >= NT || tid < NSEG;
  auto fetch_a1 = [&](uint4 (&ar)[AS][APL], int k0, bool live) {
#pragma unroll
    for (int j = 0; j < AS; ++j) {
      const int u = tid + NT * j;
      const int row = a_act ? u >> 4 : 0, kk = 8 * (u & 15);
      const int src = a_act ? arow[row] : -1;
      constexpr uint32_t ELT = F32 ? 4 : 2;
      const uint32_t off = (live && src >= 0) ? ((uint32_t)src * H + k0 + kk) * ELT : 0x80000000u;
      ar[j][0] = wload16(ra, off);
      if (F32) ar[j][APL - 1] = wload16(ra, off + 16);
    }
  };
  auto store_a1 = [&](_Float16* l, float* xl, const uint4 (&ar)[AS][APL]) {
#pragma unroll
  for (int j = 0; j < AS; ++j) {
    const int u = tid + NT * j;
    const int row = u >> 4, kk = 8 * (u & 15);
    float v[8];
    uint4 r0 = ar[j][0], r1 = ar[j][APL - 1];
    hold(r0);
    if (F32) hold(r1);
    if (F32) {
      const uint4 a0 = r0, a1 = r1;
      v[0] = __uint_as_float(a0.x); v[1] = __uint_as_float(a0.y); v[2] = __uint_as_float(a0.z); v[3] = __uint_as_float(a0.w);
      v[4] = __uint_as_float(a1.x); v[5] = __uint_as_float(a1.y); v[6] = __uint_as_float(a1.z); v[7] = __uint_as_float(a1.w);
    } else {
      const uint32_t uw[4] = {r0.x, r0.y, r0.z, r0.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(uw[i] << 16);
        v[2 * i + 1] = __uint_as_float(uw[i] & 0xFFFF0000u);
      }
    }
    half8 hi, lo;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const float x = v[perm_k<BITS>(p)];
      const _Float16 xh = (_Float16)x;
      hi[p] = xh;
      lo[p] = (_Float16)(x - (float)xh);
    }
    if constexpr (K4) {
      // 8 x the sub-block sum: the 4 threads of a 32-column sub-block are 4
      // consecutive lanes (whole waves are active or idle together)
      float xs = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
      xs = group_sum<4>(xs);
      if (a_act && (u & 3) == 0) xl[((u & 15) >> 2) * MTL + row] = 8.0f * xs;
    }
    if (!a_act) continue;
    *(half8*)(l + row * LDS_ROW + kk) = hi;
    if (SPLIT) *(half8*)(l + MTL * LDS_ROW + row * LDS_ROW + kk) = lo;
  }
  };
  float4v acc[2][MS], ctmp[2][MS];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) { acc[i][ms] = float4v{0, 0, 0, 0}; ctmp[i][ms] = float4v{0, 0, 0, 0}; }
  __syncthreads();   // arow

  // Fully unrolled stage loop: every ring slot is a fixed register set, so no
  // value is copied while its load is still in flight.
  uint4 A[AR][AS][APL];   // A(s) lives in slot s % AR until it is stored to LDS
#pragma unroll
  for (int s0 = 0; s0 < AR; ++s0) fetch_a1(A[s0], s0 * KS, s0 < NSTAGE);
#pragma unroll
  for (int d = 0; d < D; ++d) load_b(bq[d], sq[d], rq[K4 ? d : 0], d);
  store_a1(lds[0], &xsl[0][0][0], A[0]);

#pragma unroll 1
  for (int s0 = 0; s0 < NSTAGE; s0 += SB) {
#pragma unroll
  for (int d = 0; d < SB; ++d) {
    const int st = s0 + d;
    if (SB != NSTAGE && st >= NSTAGE) break;
    __syncthreads();   // lds[st & 1] holds A(st); lds[(st + 1) & 1] is free
    if (st + 1 < NSTAGE) store_a1(lds[(d + 1) & 1], &xsl[(d + 1) & 1][0][0], A[(d + 1) % AR]);
    if (st + AR < NSTAGE) fetch_a1(A[d % AR], (st + AR) * KS, true);
    const _Float16* la = lds[d & 1];
    const int sl = d % D;
    // two-level: this stage is half d % 2 of its super-block (s0 is even)
    Q4kBytes fb[2];
    if constexpr (K4) {
#pragma unroll
      for (int i = 0; i < 2; ++i) fb[i] = q4k_bytes(rq[sl][i]);
    }
#pragma unroll
    for (int c = 0; c < KS / 32; ++c) {
      const bool first = (c % CPG) == 0, last = (c % CPG) == CPG - 1;
      half8 bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (BITS == 4) bfr[i] = unpack_int4(word_of(bq[sl][i][0], c));
        else bfr[i] = unpack_int8(word_of(bq[sl][i][c >> 1], 2 * (c & 1)), word_of(bq[sl][i][c >> 1], 2 * (c & 1) + 1));
      }
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
        const int lrow = ms * 16 + r, lcol = 32 * c + 8 * q4;
        const half8 ahi = *(const half8*)(la + lrow * LDS_ROW + lcol);
        half8 alo;
        if (SPLIT) alo = *(const half8*)(la + MTL * LDS_ROW + lrow * LDS_ROW + lcol);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          float4v cc = first ? float4v{0, 0, 0, 0} : ctmp[i][ms];
          cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bfr[i], cc, 0, 0, 0);
          if (SPLIT) cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bfr[i], cc, 0, 0, 0);
          ctmp[i][ms] = cc;
        }
      }
      if (last) {
        if constexpr (K4) {
          // sub-block 4 (d % 2) + c of the super-block: s = d sc
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const float sv = f16_bits_value(rq[sl][i][0] & 0xFFFFu) * byte_value(fb[i].sc[d & 1], c);
#pragma unroll
            for (int ms = 0; ms < MS; ++ms) acc[i][ms] += sv * ctmp[i][ms];
          }
        } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float sv = sq[sl][i][c / CPG];
#pragma unroll
          for (int ms = 0; ms < MS; ++ms) acc[i][ms] += sv * ctmp[i][ms];
        }
        }
      }
    }
    if constexpr (K4) {
      // the minimum term of the stage's 4 sub-blocks in one f32 product per
      // 16 x 16 output block: A = 8X [rows][sub-blocks], B = beta / 8 =
      // s - dmin m / 8 [sub-blocks][columns] (lane (r, q4): row / column r,
      // sub-block q4)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float bsc = (float)((fb[i].sc[d & 1] >> (8 * q4)) & 255u);
        const float bm = (float)((fb[i].m[d & 1] >> (8 * q4)) & 255u);
        const float bv = fmaf(-0.125f * f16_bits_value(rq[sl][i][0] >> 16), bm,
                              f16_bits_value(rq[sl][i][0] & 0xFFFFu) * bsc);
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
          acc[i][ms] = __builtin_amdgcn_mfma_f32_16x16x4f32(xsl[d & 1][q4][ms * 16 + r], bv, acc[i][ms], 0, 0, 0);
      }
    }
    if (st + D < NSTAGE) load_b(bq[sl], sq[sl], rq[K4 ? sl : 0], st + D);   // the slot just used takes stage st + D
  }
  }
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int m = ms * 16 + 4 * q4 + k;
      if (m < ti.nrows) {
        const size_t orow = a.shared ? (size_t)(ti.row0 + m) : (size_t)(ti.pbase + m);
        a.out[orow * inter + 16 * nt + r] = silu_mul(acc[0][ms][k], acc[1][ms][k]);
      }
    }
}

// Small tiles: down, a workgroup of 8 waves owns one 32-row tile of A (h,
// fp32 split hi/lo) and four packed down tiles' worth of output rows: waves
// 2i and 2i + 1 share row tile 4cb + i (64 int4 or 32 int8 output columns),
// each taking half of its 16-row n-subtiles (the matching half of every
// 16-byte lane word).  Same software pipeline as gate/up.
template <int BITS, int G, int INTER, int KSPLIT, int MTL, int NW>
__device__ __forceinline__ void down_small_body(const GroupedArgs& a, int bid) {
  constexpr bool K4 = G == Q4K;            // two-level format (see gateup_small_body)
  static_assert(!K4 || BITS == 4, "two-level codes are 4-bit");
  constexpr int GG = K4 ? Q4K_SUB : G;
  constexpr int DR = down_rows(BITS), NRT = H / DR, NSUB = DR / 16, NCB = NRT / (NW / 2), MS = MTL / 16;
  constexpr int NT = 64 * NW, NSEG = MTL * KS / 8, AS = NSEG > NT ? NSEG / NT : 1;
  static_assert(NSEG <= NT * AS, "every A segment has a thread");
  constexpr int NSW = NSUB / 2;             // n-subtiles per wave (half a row tile)
  constexpr int CPG = GG / 32, GPS = KS / GG, NSTAGE = INTER / KS / KSPLIT;
  static_assert((INTER / KS) % KSPLIT == 0, "K halves of whole stages");
  // B stages in flight, A stages ahead and blocks of 2 stages with a loop
  // between them, as in gateup_small_body (two workgroups per CU for G >= 64,
  // no scratch)
  constexpr int D = 2;
  constexpr int AR = 2;
  constexpr int SB = 2;
  static_assert((SB % D == 0 && SB % AR == 0 && SB % 2 == 0) || SB == NSTAGE, "ring slots fixed within a block");
  const int inter = INTER;
  const int kh = bid % KSPLIT, tb = bid / KSPLIT, s0 = kh * NSTAGE;   // K part kh
  const int tile = tb / NCB, cb = tb % NCB;
  const TileInfo ti = tile_info(a, tile, MTL);
  if (!ti.valid) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = wave_uniform((int)(threadIdx.x >> 6)), r = lane & 15,
            q4 = lane >> 4;
  __shared__ __attribute__((aligned(16))) _Float16 lds[2][2 * MTL * LDS_ROW];
  __shared__ __attribute__((aligned(16))) float xsl[2][K4 ? KS / 32 : 1][MTL];   // two-level: 8 X per row, sub-block
  __shared__ int arow[MTL];
  if (tid < MTL) arow[tid] = tid < ti.nrows ? (a.shared ? ti.row0 + tid : ti.pbase + tid) : -1;
  const int e = wave_uniform(ti.e);
  const size_t mbytes = matrix_bytes(BITS, inter, H);
  const int ngk = inter / GG;
  const int rt = (NW / 2) * cb + (wv >> 1), hh = wv & 1;
  const __amdgpu_buffer_rsrc_t rb = weight_rsrc(a.w.q + (size_t)e * a.w.e_bytes + 2 * mbytes, (uint32_t)mbytes);
  // two-level: d | dmin words [super-block][slot] and sc | m << 8 halfwords
  // [sub-block][slot], slot (rt, r, j) = row DR rt + 16 j + r
  const uint8_t* dmeta = (const uint8_t*)(a.w.s + (size_t)e * a.w.e_scales) + q4k_rec_bytes(inter);
  const __amdgpu_buffer_rsrc_t rs =
      K4 ? weight_rsrc(dmeta, (uint32_t)q4k_dd_bytes(inter))
         : weight_rsrc(a.w.s + (size_t)e * a.w.e_scales + 2 * (size_t)inter * (H / GG), (uint32_t)ngk * H * 4);
  const __amdgpu_buffer_rsrc_t rsm = weight_rsrc(dmeta + q4k_dd_bytes(inter), (uint32_t)ngk * H * 2);
  const __amdgpu_buffer_rsrc_t ra = weight_rsrc(a.af, (uint32_t)a.a_rows * inter * 4);
  const uint32_t slot0 = ((uint32_t)rt * 16 + r) * 4 + NSW * hh;   // this lane's first row slot

  // this wave's half of each 16-byte lane word of a down tile: words 2hh, 2hh+1
  uint2 bq[D][KS / 32];
  float sq[D][GPS][NSW];
  uint2 dq[K4 ? D : 1];                    // two-level: d | dmin of the lane's NSW rows
  uint32_t mq[K4 ? D : 1][GPS];            // ... and their sc | m << 8 halfwords per sub-block
  auto load_b = [&](uint2 (&bd)[KS / 32], float (&sd)[GPS][NSW], uint2& dd, uint32_t (&mm)[GPS], int st) {
    if constexpr (K4) {
      static_assert(NSW == 2 && Q4K_SB == 2 * KS, "two rows per lane, two stages per super-block");
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, (((uint32_t)(s0 + st) / 2) * H + slot0) * 4, 0, 0);
      dd = make_uint2(v[0], v[1]);
#pragma unroll
      for (int g = 0; g < GPS; ++g)
        mm[g] = __builtin_amdgcn_raw_buffer_load_b32(rsm, ((uint32_t)((s0 + st) * GPS + g) * H + slot0) * 2, 0, 0);
    } else {
#pragma unroll
      for (int g = 0; g < GPS; ++g) {
        const uint32_t so = ((((uint32_t)((s0 + st) * GPS + g) * NRT + rt) * 16 + r) * NSUB + NSW * hh) * 4;
        if (NSW == 2) {
          const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, so, 0, 0);
          sd[g][0] = __uint_as_float(v[0]);
          sd[g][NSW - 1] = __uint_as_float(v[1]);
        } else {
          sd[g][0] = wload4(rs, so);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < KS / 32; ++c) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(
          rb, ((uint32_t)((s0 + st) * (KS / 32) + c) * NRT + rt) * TILE + lane * 16 + 8 * hh, 0, 0);
      bd[c] = make_uint2(v[0], v[1]);
    }
  };
  // A (h, f32 as hi/lo f16 planes): one 8-element segment per thread per
  // stage; with 16-row tiles only the first 256 threads hold one
  const bool a_act = NSEG >= NT || tid < NSEG;
  auto fetch_a1 = [&](uint4 (&ar)[AS][2], int k0, bool live) {
#pragma unroll
    for (int j = 0; j < AS; ++j) {
      const int u = tid + NT * j;
      const int row = a_act ? u >> 4 : 0, kk = 8 * (u & 15);
      const int src = a_act ? arow[row] : -1;
      const uint32_t off = (live && src >= 0) ? ((uint32_t)src * INTER + k0 + kk) * 4 : 0x80000000u;
      ar[j][0] = wload16(ra, off);
      ar[j][1] = wload16(ra, off + 16);
    }
  };
  auto store_a1 = [&](_Float16* l, float* xl, const uint4 (&ar)[AS][2]) {
#pragma unroll
  for (int j = 0; j < AS; ++j) {
    const int u = tid + NT * j;
    const int row = u >> 4, kk = 8 * (u & 15);
    uint4 r0 = ar[j][0], r1 = ar[j][1];
    hold(r0);
    hold(r1);
    const float v[8] = {__uint_as_float(r0.x), __uint_as_float(r0.y), __uint_as_float(r0.z),
                        __uint_as_float(r0.w), __uint_as_float(r1.x), __uint_as_float(r1.y),
                        __uint_as_float(r1.z), __uint_as_float(r1.w)};
    half8 hi, lo;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const float x = v[perm_k<BITS>(p)];
      const _Float16 xh = (_Float16)x;
      hi[p] = xh;
      lo[p] = (_Float16)(x - (float)xh);
    }
    if constexpr (K4) {
      float xs = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
      xs = group_sum<4>(xs);
      if (a_act && (u & 3) == 0) xl[((u & 15) >> 2) * MTL + row] = 8.0f * xs;
    }
    if (!a_act) continue;
    *(half8*)(l + row * LDS_ROW + kk) = hi;
    *(half8*)(l + MTL * LDS_ROW + row * LDS_ROW + kk) = lo;
  }
  };
  float4v acc[NSW][MS], ctmp[NSW][MS];
#pragma unroll
  for (int j = 0; j < NSW; ++j)
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) { acc[j][ms] = float4v{0, 0, 0, 0}; ctmp[j][ms] = float4v{0, 0, 0, 0}; }
  __syncthreads();   // arow

  uint4 A[AR][AS][2];
#pragma unroll
  for (int sp = 0; sp < AR; ++sp) fetch_a1(A[sp], (s0 + sp) * KS, sp < NSTAGE);
#pragma unroll
  for (int d = 0; d < D; ++d) load_b(bq[d], sq[d], dq[K4 ? d : 0], mq[K4 ? d : 0], d);
  store_a1(lds[0], &xsl[0][0][0], A[0]);

#pragma unroll 1
  for (int b0 = 0; b0 < NSTAGE; b0 += SB) {
#pragma unroll
  for (int d = 0; d < SB; ++d) {
    const int st = b0 + d;
    if (SB != NSTAGE && st >= NSTAGE) break;
    __syncthreads();
    if (st + 1 < NSTAGE) store_a1(lds[(d + 1) & 1], &xsl[(d + 1) & 1][0][0], A[(d + 1) % AR]);
    if (st + AR < NSTAGE) fetch_a1(A[d % AR], (s0 + st + AR) * KS, true);
    const _Float16* la = lds[d & 1];
    const int sl = d % D;
#pragma unroll
    for (int c = 0; c < KS / 32; ++c) {
      const bool first = (c % CPG) == 0, last = (c % CPG) == CPG - 1;
      const int lcol = 32 * c + 8 * q4;
      half8 ahi[MS], alo[MS];
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
        ahi[ms] = *(const half8*)(la + (ms * 16 + r) * LDS_ROW + lcol);
        alo[ms] = *(const half8*)(la + MTL * LDS_ROW + (ms * 16 + r) * LDS_ROW + lcol);
      }
#pragma unroll
      for (int j = 0; j < NSW; ++j) {
        const uint2 w2 = bq[sl][c];
        const half8 bfr = BITS == 4 ? unpack_int4(j == 0 ? w2.x : w2.y) : unpack_int8(w2.x, w2.y);
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
          float4v cc = first ? float4v{0, 0, 0, 0} : ctmp[j][ms];
          cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[ms], bfr, cc, 0, 0, 0);
          cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[ms], bfr, cc, 0, 0, 0);
          ctmp[j][ms] = cc;
        }
      }
      if (last) {
        if constexpr (K4) {
#pragma unroll
          for (int j = 0; j < NSW; ++j) {
            const uint32_t ddw = j == 0 ? dq[sl].x : dq[sl].y;
            const float sv = f16_bits_value(ddw & 0xFFFFu) * byte_value(mq[sl][c], 2 * j);
#pragma unroll
            for (int ms = 0; ms < MS; ++ms) acc[j][ms] += sv * ctmp[j][ms];
          }
        } else {
#pragma unroll
        for (int j = 0; j < NSW; ++j) {
          const float sj = sq[sl][c / CPG][j];
#pragma unroll
          for (int ms = 0; ms < MS; ++ms) acc[j][ms] += sj * ctmp[j][ms];
        }
        }
      }
    }
    if constexpr (K4) {
      // the minimum term of the stage's sub-blocks as in gateup_small_body:
      // lane (r, q4) supplies 8X of row r and beta / 8 of column r, sub-block q4
      const uint32_t mw = q4 == 0 ? mq[sl][0] : q4 == 1 ? mq[sl][1] : q4 == 2 ? mq[sl][2] : mq[sl][3];
#pragma unroll
      for (int j = 0; j < NSW; ++j) {
        const uint32_t ddw = j == 0 ? dq[sl].x : dq[sl].y;
        const float bv = fmaf(-0.125f * f16_bits_value(ddw >> 16), byte_value(mw, 2 * j + 1),
                              f16_bits_value(ddw & 0xFFFFu) * byte_value(mw, 2 * j));
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
          acc[j][ms] = __builtin_amdgcn_mfma_f32_16x16x4f32(xsl[d & 1][q4][ms * 16 + r], bv, acc[j][ms], 0, 0, 0);
      }
    }
    if (st + D < NSTAGE) load_b(bq[sl], sq[sl], dq[K4 ? sl : 0], mq[K4 ? sl : 0], st + D);
  }
  }
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int m = ms * 16 + 4 * q4 + k;
      if (m < ti.nrows) {
        const size_t orow = a.shared ? (size_t)(ti.row0 + m) : (size_t)(ti.pbase + m);
#pragma unroll
        for (int j = 0; j < NSW; ++j)
          a.out[(size_t)kh * a.T * H + orow * H + DR * rt + 16 * (NSW * hh + j) + r] = acc[j][ms][k];
      }
    }
}

// Workgroups per row tile: gate/up 128 intermediate columns each; down four
// packed row tiles each, times the K parts.
__host__ __device__ constexpr int gateup_blocks(int inter) { return inter / (16 * SMALL_WAVES); }
__host__ __device__ constexpr int down_blocks(int bits, int ksplit) {
  return H / (SMALL_WAVES / 2 * down_rows(bits)) * ksplit;
}

template <int BITS, bool SPLIT, int G, int MTL>
__global__ __launch_bounds__(64 * SMALL_WAVES) void gateup_small_kernel(GroupedArgs a) {
  const int nb = gateup_blocks(a.w.inter);
  gateup_small_body<BITS, SPLIT, G, MTL, SMALL_WAVES>(a, xcd_run(blockIdx.x, live_tiles(a, MTL) * nb));
}
template <int BITS, int G, int INTER, int KSPLIT, int MTL>
__global__ __launch_bounds__(64 * SMALL_WAVES) void down_small_kernel(GroupedArgs a) {
  down_small_body<BITS, G, INTER, KSPLIT, MTL, SMALL_WAVES>(
      a, xcd_run(blockIdx.x, live_tiles(a, MTL) * down_blocks(BITS, KSPLIT)));
}
// The shared expert does not depend on routing: with small tiles its
// workgroups run in the same launch as the routed experts' (shared tiles
// first, so they start at once; routed tiles past the histogram's count exit
// at once), which fills the compute units the few shared tiles would leave idle.
template <int BR, int GR, int BS, int GS, bool SPLIT, int MTL>
__global__ __launch_bounds__(64 * SMALL_WAVES) void gateup_small_pair_kernel(GroupedArgs r, GroupedArgs sh, int n_shared) {
  const int lb = xcd_run(blockIdx.x, n_shared + *r.ntiles * gateup_blocks(I));
  if (lb < n_shared) gateup_small_body<BS, SPLIT, GS, MTL, SMALL_WAVES>(sh, lb);
  else gateup_small_body<BR, SPLIT, GR, MTL, SMALL_WAVES>(r, lb - n_shared);
}
template <int BR, int GR, int BS, int GS, int MTL>
__global__ __launch_bounds__(64 * SMALL_WAVES) void down_small_pair_kernel(GroupedArgs r, GroupedArgs sh, int n_shared) {
  const int lb = xcd_run(blockIdx.x, n_shared + *r.ntiles * down_blocks(BR, 1));
  if (lb < n_shared) down_small_body<BS, GS, IS, 2, MTL, SMALL_WAVES>(sh, lb);
  else down_small_body<BR, GR, I, 1, MTL, SMALL_WAVES>(r, lb - n_shared);
}

// y[t] (+)= ys[t] (+ ys2[t]) + sum_j w[t,j] * ysorted[pos_of[t*6+j]], picks added in order.
__global__ __launch_bounds__(320) void combine_kernel(CombineArgs a) {
  const int t = blockIdx.x, c = threadIdx.x * 4;
  float4* yp = (float4*)(a.y + (size_t)t * H + c);
  // the old output is requested first: it does not wait behind the rows
  const float4 o = a.accumulate ? *yp : make_float4(0.f, 0.f, 0.f, 0.f);
  float4 v = *(const float4*)(a.ys + (size_t)t * H + c);
  if (a.ys2) {   // the second K part of the shared expert's down projection
    const float4 v2 = *(const float4*)(a.ys2 + (size_t)t * H + c);
    v.x += v2.x; v.y += v2.y; v.z += v2.z; v.w += v2.w;
  }
#pragma unroll
  for (int j = 0; j < TOPK; ++j) {
    const float wj = a.tw[(size_t)t * TOPK + j];
    const float4 p = *(const float4*)(a.ysorted + (size_t)a.pos_of[(size_t)t * TOPK + j] * H + c);
    v.x += wj * p.x; v.y += wj * p.y; v.z += wj * p.z; v.w += wj * p.w;
  }
  if (a.accumulate) {
    v.x = o.x + v.x; v.y = o.y + v.y; v.z = o.z + v.z; v.w = o.w + v.w;
  }
  *yp = v;
}

__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* h, void* z, int z_mode, float eps) {
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  float v[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) v[i] = h[(size_t)t * H + tid + 256 * i];
  const float ss = wave_sum(thread_sumsq(v));
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float inv = inv_rms(red, eps);
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const float zz = v[i] * inv;
    const size_t idx = (size_t)t * H + tid + 256 * i;
    if (z_mode == 1) {
      ((uint16_t*)z)[idx] = (uint16_t)(__float_as_uint(bf16_rne(zz)) >> 16);
    } else if (z_mode == 2) {
      // split_row: bf16 hi and lo halves of the group's 8 elements, 16 bytes each
      const float hi = bf16_rne(zz);
      uint16_t* g = (uint16_t*)z + (idx & ~(size_t)7) * 2 + (idx & 7);
      g[0] = (uint16_t)(__float_as_uint(hi) >> 16);
      g[8] = (uint16_t)(__float_as_uint(bf16_rne(zz - hi)) >> 16);
    } else {
      ((float*)z)[idx] = zz;
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
constexpr int RS_MAX_T = 1024;
// experts per wave of the logits pass.  Measured: one expert per wave (16
// workgroups of 20 KB of W_r per 4 tokens) against four (4 workgroups of 80
// KB): one per-token layer call of 1 token 17.7 -> 16.2 us, 16 tokens 52.3 ->
// 50.7 us, 128-stream step 0.762 -> 0.750 ms, 32 pages 41.3 -> 40.0 us, 273-token
// prefill equal.  The one-pass router it replaced below 8 tokens (one
// workgroup per 4 tokens streaming all 327 KB of W_r) took 12.6 us at 1 token.
constexpr int RS_EPW = 1;
hipError_t launch_router(const RouterArgs& a, hipStream_t s, bool select) {
  // measured: the two-pass router wins up to about a thousand tokens, where
  // re-reading W_r per 4-token block starts to dominate and the 16-token MFMA
  // workgroups take over (2184 tokens: 25 us per 11-layer step faster)
  if (a.T < RS_MAX_T) {
    hipLaunchKernelGGL(router_logits_kernel<RS_EPW>, dim3((a.T + RS_TB - 1) / RS_TB, E / (4 * RS_EPW)), dim3(256), 0,
                       s, a);
    if (select) hipLaunchKernelGGL(router_select_kernel, dim3((a.T + 3) / 4), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(router_mfma_kernel, dim3((a.T + RM_TB - 1) / RM_TB), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <int WPE>
static hipError_t dec_items_dispatch(const DecItemsArgs& a, int T, hipStream_t s) {
  const dim3 grid(T * N_ITEMS);
  const int qk = (a.rw.group == Q4K) + 2 * (a.sw.group == Q4K);
  const int key = (a.rw.bits == 8) * 2 + (a.sw.bits == 8) + 4 * qk;
  switch (key) {
    case 0: hipLaunchKernelGGL((dec_items_kernel<4, 4, 0, WPE>), grid, dim3(512), 0, s, a); break;
    case 1: hipLaunchKernelGGL((dec_items_kernel<4, 8, 0, WPE>), grid, dim3(512), 0, s, a); break;
    case 2: hipLaunchKernelGGL((dec_items_kernel<8, 4, 0, WPE>), grid, dim3(512), 0, s, a); break;
    case 3: hipLaunchKernelGGL((dec_items_kernel<8, 8, 0, WPE>), grid, dim3(512), 0, s, a); break;
    case 4: hipLaunchKernelGGL((dec_items_kernel<4, 4, 1, WPE>), grid, dim3(512), 0, s, a); break;
    case 5: hipLaunchKernelGGL((dec_items_kernel<4, 8, 1, WPE>), grid, dim3(512), 0, s, a); break;
    case 8: hipLaunchKernelGGL((dec_items_kernel<4, 4, 2, WPE>), grid, dim3(512), 0, s, a); break;
    case 10: hipLaunchKernelGGL((dec_items_kernel<8, 4, 2, WPE>), grid, dim3(512), 0, s, a); break;
    case 12: hipLaunchKernelGGL((dec_items_kernel<4, 4, 3, WPE>), grid, dim3(512), 0, s, a); break;
    default: return hipErrorInvalidValue;   // the two-level format has 4-bit codes
  }
  return hipGetLastError();
}

hipError_t launch_dec_items(const DecItemsArgs& a, int T, hipStream_t s) {
  // the two-level format and the G = 32 symmetric kernels share nothing but
  // the name: only symmetric 32-column groups keep one workgroup per CU
  const bool g32 = a.rw.group == 32 || a.sw.group == 32;
  return g32 ? dec_items_dispatch<2>(a, T, s) : dec_items_dispatch<4>(a, T, s);
}

hipError_t launch_dec_reduce(const DecReduceArgs& a, int T, hipStream_t s) {
  hipLaunchKernelGGL(dec_reduce_kernel, dim3(T * (H / 32)), dim3(256), 0, s, a);
  return hipGetLastError();
}

// The persistent kernel needs all N_ITEMS + N_RED workgroups resident at once.
// hipLaunchCooperativeKernel guarantees that but costs ~15 us per launch on
// this stack, so the launch is a plain one, preceded by a check that one
// compute unit holds at least one workgroup and the device has enough compute
// units (the workgroup size and LDS use make it one workgroup per CU).  Every
// wait inside the kernel is bounded, so a violated assumption (e.g. other
// kernels occupying CUs) ends in the workspace error word, not in a hang.
hipError_t launch_chain(const ChainArgs& a, hipStream_t s) {
  const void* fn;
  const int qk = (a.rgroup == Q4K) + 2 * (a.sgroup == Q4K);
  const int key = (a.rbits == 8) * 2 + (a.sbits == 8) + 4 * qk;
  switch (key) {
    case 0: fn = (const void*)chain_kernel<4, 4, 0>; break;
    case 1: fn = (const void*)chain_kernel<4, 8, 0>; break;
    case 2: fn = (const void*)chain_kernel<8, 4, 0>; break;
    case 3: fn = (const void*)chain_kernel<8, 8, 0>; break;
    case 4: fn = (const void*)chain_kernel<4, 4, 1>; break;
    case 5: fn = (const void*)chain_kernel<4, 8, 1>; break;
    case 8: fn = (const void*)chain_kernel<4, 4, 2>; break;
    case 10: fn = (const void*)chain_kernel<8, 4, 2>; break;
    case 12: fn = (const void*)chain_kernel<4, 4, 3>; break;
    default: return hipErrorInvalidValue;   // the two-level format has 4-bit codes
  }
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 512, 0);
  if (e != hipSuccess) return e;
  if ((long)cus * per_cu < N_ITEMS + N_RED) return hipErrorCooperativeLaunchTooLarge;
  void* args[] = {(void*)&a};
  return hipLaunchKernel(fn, dim3(N_ITEMS + N_RED), dim3(512), args, 0, s);
}

hipError_t launch_zero_words(uint32_t* p, size_t n, hipStream_t s) {
  hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_hist(const HistArgs& a, hipStream_t s) {
  const int n = a.T * TOPK;
  if (n <= HIST_ONE_WG_MAX) {
    hipLaunchKernelGGL(hist_kernel, dim3(1), dim3(1024), 0, s, a);
  } else {
    const int nb = (n + HIST_BLOCK - 1) / HIST_BLOCK;
    hipLaunchKernelGGL(hist_count_kernel, dim3(nb), dim3(1024), 0, s, a);
    hipLaunchKernelGGL(hist_place_kernel, dim3(nb), dim3(1024), 0, s, a);
  }
  return hipGetLastError();
}

template <int BITS, int G>
static void gateup_dispatch(const GroupedArgs& a, int max_tiles, bool small, hipStream_t s) {
  if (small) {
    const dim3 grid(max_tiles * gateup_blocks(a.w.inter));
    if (a.af) hipLaunchKernelGGL((gateup_small_kernel<BITS, true, G, MT_SMALL>), grid, dim3(64 * SMALL_WAVES), 0, s, a);
    else hipLaunchKernelGGL((gateup_small_kernel<BITS, false, G, MT_SMALL>), grid, dim3(64 * SMALL_WAVES), 0, s, a);
  } else {
    const dim3 grid(max_tiles * (a.w.inter / 128));   // 128 gate + 128 up columns per workgroup
    if (a.af) hipLaunchKernelGGL((grouped_gateup_kernel<BITS, true, G>), grid, dim3(GT), 0, s, a);
    else hipLaunchKernelGGL((grouped_gateup_kernel<BITS, false, G>), grid, dim3(GT), 0, s, a);
  }
}

hipError_t launch_grouped_gateup(const GroupedArgs& a, int max_tiles, bool small, hipStream_t s) {
  const int key = (a.w.bits == 8) * 3 + (a.w.group == 64) + 2 * (a.w.group == 128);
  switch (key) {
    case 0: gateup_dispatch<4, 32>(a, max_tiles, small, s); break;
    case 1: gateup_dispatch<4, 64>(a, max_tiles, small, s); break;
    case 2: gateup_dispatch<4, 128>(a, max_tiles, small, s); break;
    case 3: gateup_dispatch<8, 32>(a, max_tiles, small, s); break;
    case 4: gateup_dispatch<8, 64>(a, max_tiles, small, s); break;
    default: gateup_dispatch<8, 128>(a, max_tiles, small, s); break;
  }
  return hipGetLastError();
}

template <int BITS, int G>
static void down_dispatch(const GroupedArgs& a, int max_tiles, bool small, hipStream_t s) {
  if (small) {
    const dim3 grid(max_tiles * down_blocks(BITS, 1));
    if (a.w.inter == IS && a.ksplit == 2)
      hipLaunchKernelGGL((down_small_kernel<BITS, G, IS, 2, MT_SMALL>), dim3(2 * grid.x), dim3(64 * SMALL_WAVES), 0, s, a);
    else if (a.w.inter == IS) hipLaunchKernelGGL((down_small_kernel<BITS, G, IS, 1, MT_SMALL>), grid, dim3(64 * SMALL_WAVES), 0, s, a);
    else hipLaunchKernelGGL((down_small_kernel<BITS, G, I, 1, MT_SMALL>), grid, dim3(64 * SMALL_WAVES), 0, s, a);
  } else {
    const dim3 grid(max_tiles * (H / 256));             // 256 output columns per workgroup
    if (a.w.inter == IS && a.ksplit == 2)
      hipLaunchKernelGGL((grouped_down_kernel<BITS, G, IS, 2>), dim3(2 * grid.x), dim3(GT), 0, s, a);
    else if (a.w.inter == IS) hipLaunchKernelGGL((grouped_down_kernel<BITS, G, IS>), grid, dim3(GT), 0, s, a);
    else hipLaunchKernelGGL((grouped_down_kernel<BITS, G, I>), grid, dim3(GT), 0, s, a);
  }
}

// Two-level format: the 32-row small tiles at every token count.
hipError_t launch_grouped_q4k(const GroupedArgs& a, int max_tiles, bool down, hipStream_t s) {
  if (!down) {
    const dim3 grid(max_tiles * gateup_blocks(a.w.inter));
    if (a.af) hipLaunchKernelGGL((gateup_small_kernel<4, true, Q4K, MT_SMALL>), grid, dim3(64 * SMALL_WAVES), 0, s, a);
    else hipLaunchKernelGGL((gateup_small_kernel<4, false, Q4K, MT_SMALL>), grid, dim3(64 * SMALL_WAVES), 0, s, a);
  } else {
    const dim3 grid(max_tiles * down_blocks(4, 1));
    if (a.w.inter == IS && a.ksplit == 2)
      hipLaunchKernelGGL((down_small_kernel<4, Q4K, IS, 2, MT_SMALL>), dim3(2 * grid.x), dim3(64 * SMALL_WAVES), 0, s, a);
    else if (a.w.inter == IS) hipLaunchKernelGGL((down_small_kernel<4, Q4K, IS, 1, MT_SMALL>), grid, dim3(64 * SMALL_WAVES), 0, s, a);
    else hipLaunchKernelGGL((down_small_kernel<4, Q4K, I, 1, MT_SMALL>), grid, dim3(64 * SMALL_WAVES), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_grouped_down(const GroupedArgs& a, int max_tiles, bool small, hipStream_t s) {
  const int key = (a.w.bits == 8) * 3 + (a.w.group == 64) + 2 * (a.w.group == 128);
  switch (key) {
    case 0: down_dispatch<4, 32>(a, max_tiles, small, s); break;
    case 1: down_dispatch<4, 64>(a, max_tiles, small, s); break;
    case 2: down_dispatch<4, 128>(a, max_tiles, small, s); break;
    case 3: down_dispatch<8, 32>(a, max_tiles, small, s); break;
    case 4: down_dispatch<8, 64>(a, max_tiles, small, s); break;
    default: down_dispatch<8, 128>(a, max_tiles, small, s); break;
  }
  return hipGetLastError();
}

template <int BR, int GR, int BS, int GS, int MTL>
static void pair_dispatch(const GroupedArgs& r, int r_tiles, const GroupedArgs& sh, int s_tiles, bool down,
                          hipStream_t s) {
  if (!down) {
    const int ns = s_tiles * gateup_blocks(IS), nr = r_tiles * gateup_blocks(I);
    if (r.af)
      hipLaunchKernelGGL((gateup_small_pair_kernel<BR, GR, BS, GS, true, MTL>), dim3(ns + nr), dim3(64 * SMALL_WAVES), 0, s, r, sh, ns);
    else
      hipLaunchKernelGGL((gateup_small_pair_kernel<BR, GR, BS, GS, false, MTL>), dim3(ns + nr), dim3(64 * SMALL_WAVES), 0, s, r, sh, ns);
  } else {
    const int ns = s_tiles * down_blocks(BS, 2), nr = r_tiles * down_blocks(BR, 1);
    hipLaunchKernelGGL((down_small_pair_kernel<BR, GR, BS, GS, MTL>), dim3(ns + nr), dim3(64 * SMALL_WAVES), 0, s, r, sh, ns);
  }
}
template <int BR, int GR, int BS, int GS>
static void pair_dispatch_h(const GroupedArgs& r, int r_tiles, const GroupedArgs& sh, int s_tiles, bool down, int mtl,
                            hipStream_t s) {
  if (mtl == MT_TINY) pair_dispatch<BR, GR, BS, GS, MT_TINY>(r, r_tiles, sh, s_tiles, down, s);
  else pair_dispatch<BR, GR, BS, GS, MT_SMALL>(r, r_tiles, sh, s_tiles, down, s);
}

bool small_pair_available(int rbits, int rgroup, int sbits, int sgroup) {
  return (rbits == sbits && rgroup == sgroup) ||
         (rbits == 4 && (rgroup == 64 || rgroup == Q4K) && sbits == 8 && sgroup == 128);
}

bool launch_small_pair(const GroupedArgs& r, int r_tiles, const GroupedArgs& sh, int s_tiles, bool down, int mtl,
                       hipStream_t s) {
  const int rb = r.w.bits, rg = r.w.group, sb = sh.w.bits, sg = sh.w.group;
  if (!small_pair_available(rb, rg, sb, sg)) return false;
  if (rg == Q4K) {
    if (sg == Q4K) pair_dispatch_h<4, Q4K, 4, Q4K>(r, r_tiles, sh, s_tiles, down, mtl, s);
    else pair_dispatch_h<4, Q4K, 8, 128>(r, r_tiles, sh, s_tiles, down, mtl, s);
  } else if (rb == sb && rg == sg) {
    const int key = (rb == 8) * 3 + (rg == 64) + 2 * (rg == 128);
    switch (key) {
      case 0: pair_dispatch_h<4, 32, 4, 32>(r, r_tiles, sh, s_tiles, down, mtl, s); break;
      case 1: pair_dispatch_h<4, 64, 4, 64>(r, r_tiles, sh, s_tiles, down, mtl, s); break;
      case 2: pair_dispatch_h<4, 128, 4, 128>(r, r_tiles, sh, s_tiles, down, mtl, s); break;
      case 3: pair_dispatch_h<8, 32, 8, 32>(r, r_tiles, sh, s_tiles, down, mtl, s); break;
      case 4: pair_dispatch_h<8, 64, 8, 64>(r, r_tiles, sh, s_tiles, down, mtl, s); break;
      default: pair_dispatch_h<8, 128, 8, 128>(r, r_tiles, sh, s_tiles, down, mtl, s); break;
    }
  } else {
    pair_dispatch_h<4, 64, 8, 128>(r, r_tiles, sh, s_tiles, down, mtl, s);
  }
  return true;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel, dim3(a.T), dim3(320), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* h, void* z, int z_mode, int T, float eps, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(256), 0, s, h, z, z_mode, eps);
  return hipGetLastError();
}

// Scratch of the workspace-free layer entry point: every GPU the library runs
// on holds its own copy until the process ends.  Host code never passes the
// array's name to a kernel or a copy (on the host it is only a stand-in for
// the symbol): the device address of each GPU's copy is taken once, with that
// GPU current, and kept per device.
static __device__ __align__(256) unsigned char scratch[STATIC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;

hipError_t static_scratch(void** out) {
  static std::mutex mu;
  static void* addr[MAX_DEVICES] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || ((uintptr_t)p & 255u)) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace moe

