// gfx950 kernels of the decoder's two dense ends, for a few tokens (decode):
// the layer-0 SwiGLU MLP and the lm_head projection with the greedy token
// (browser demo page "A 3-billion-parameter OCR model. In this tab.", "One
// forward pass, left to right", steps 6 and 7; franken_ocr README
// "Architecture").
//
// Both are GEMVs that read every weight once, so HBM bandwidth bounds them.
// A weight row is read in 16-byte pieces (8 bf16 values, 16 int8 codes or 32
// int4 codes).  A group of LPR consecutive lanes shares one row, lane l of the
// group taking pieces l, l + LPR, l + 2 LPR, ...: one wave load instruction
// reads whole 1 KiB runs of consecutive rows.  The codes are decoded in
// registers to f32 and multiplied with the activations (f32 rows in LDS) by
// f32 FMAs; a piece never straddles a scale group, so each piece's partial sum
// takes its group scale once.  The lanes of a row add up with DPP in a fixed
// order, so results are bitwise reproducible.  Every weight load goes through
// a buffer descriptor bounded by the matrix: rows or pieces past the end read
// zeros without a branch, and all of a wave's loads for the next rows are in
// flight while it multiplies the current ones.
#include "moe_internal.h"
#include "moe_wave.h"

namespace moe {

namespace {

typedef unsigned int u32x4d __attribute__((vector_size(16)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dense_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}
// weights are read once per call: non-temporal loads (they would only evict
// the activations from the caches)
constexpr int CPOL_NT = 2;
__device__ __forceinline__ uint4 dload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4d v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CPOL_NT);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ float dload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
constexpr uint32_t OUT_OF_RANGE = 0x80000000u;   // offset past every descriptor: reads zeros

__device__ __forceinline__ uint32_t wword(const uint4& w, int k) {
  return k == 0 ? w.x : k == 1 ? w.y : k == 2 ? w.z : w.w;
}

// Value i of a 16-byte piece: WT = 16 (bf16, 8 values), 8 (int8, 16 codes),
// 4 (int4, 32 codes; element 2j in the low nibble of its byte).
template <int WT>
__device__ __forceinline__ float piece_value(const uint4& w, int i) {
  if (WT == 16) {
    const uint32_t u = wword(w, i >> 1);
    return __uint_as_float((i & 1) ? (u & 0xFFFF0000u) : (u << 16));
  } else if (WT == 8) {
    const uint32_t u = wword(w, i >> 2);
    return (float)((int)(u << (24 - 8 * (i & 3))) >> 24);
  } else {
    const uint32_t u = wword(w, i >> 3);
    return (float)((int)(u << (28 - 4 * (i & 7))) >> 28);
  }
}

// int8 code i of a piece as offset binary, code + 128 in [1, 255], one
// unsigned-byte conversion each (the word is XORed with 0x80808080 once)
__device__ __forceinline__ float ubyte_value(uint32_t u, int b) { return (float)((u >> (8 * b)) & 0xFFu); }

// acc[t] += scale * sum_i value_i * x[t][e0 + i] over the EPP values of one
// piece (x rows of stride XS floats in LDS).  With xsum (int8 only: per token
// and piece, the sum of the piece's x values) the codes are read in offset
// binary and the sum corrected by -128 * xsum.
template <int WT, int NT, int XS>
__device__ __forceinline__ void piece_fma(const uint4& w, const float* x, int e0, float scale, float (&acc)[NT],
                                          const float* xsum = nullptr, int xs_stride = 0) {
  constexpr int EPP = 128 / WT;
  float d[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) d[t] = 0.f;
  if (WT == 8 && xsum) {
    const uint32_t ob[4] = {w.x ^ 0x80808080u, w.y ^ 0x80808080u, w.z ^ 0x80808080u, w.w ^ 0x80808080u};
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float4 x4 = *(const float4*)&x[t * XS + e0 + 4 * k];
        d[t] = __fmaf_rn(ubyte_value(ob[k], 0), x4.x, d[t]);
        d[t] = __fmaf_rn(ubyte_value(ob[k], 1), x4.y, d[t]);
        d[t] = __fmaf_rn(ubyte_value(ob[k], 2), x4.z, d[t]);
        d[t] = __fmaf_rn(ubyte_value(ob[k], 3), x4.w, d[t]);
      }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      d[t] = __fmaf_rn(-128.0f, xsum[t * xs_stride + e0 / EPP], d[t]);
      acc[t] = __fmaf_rn(scale, d[t], acc[t]);
    }
    return;
  }
  // (with several tokens, unrolled in pairs: a full unroll keeps every x value
  // of the piece live at once)
  constexpr int UNR = NT == 1 ? EPP / 4 : 2;
#pragma unroll UNR
  for (int i4 = 0; i4 < EPP / 4; ++i4) {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = piece_value<WT>(w, 4 * i4 + j);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float4 x4 = *(const float4*)&x[t * XS + e0 + 4 * i4];
      d[t] = __fmaf_rn(v[0], x4.x, d[t]);
      d[t] = __fmaf_rn(v[1], x4.y, d[t]);
      d[t] = __fmaf_rn(v[2], x4.z, d[t]);
      d[t] = __fmaf_rn(v[3], x4.w, d[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = WT == 16 ? acc[t] + d[t] : __fmaf_rn(scale, d[t], acc[t]);
}

// NT rows of H floats into LDS (stride H); with norm, each becomes
// x / sqrt(mean(x^2) + eps).  256 threads; ends with a barrier.  issue() runs
// right after the rows' loads are issued: loads it issues (the first weight
// steps) complete after the rows' (the load counter is in order), so waiting
// for the rows does not wait for them.
template <int NT, typename F>
__device__ __forceinline__ void rows_to_lds(const float* x, int T, int norm, float eps, float* xs, float* red,
                                            F&& issue) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const __amdgpu_buffer_rsrc_t rx = dense_rsrc(x, (uint32_t)T * H * 4);
  constexpr int NU = NT * H / 4;          // float4 in all
  constexpr int NV = (NU + 255) / 256;
  uint4 v[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int u = tid + 256 * j;
    const u32x4d q = __builtin_amdgcn_raw_buffer_load_b128(rx, u < NU ? (uint32_t)u * 16 : OUT_OF_RANGE, 0, 0);
    v[j] = make_uint4(q[0], q[1], q[2], q[3]);
  }
  issue();
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int u = tid + 256 * j;
    if (u < NU) *(uint4*)&xs[4 * u] = v[j];
  }
  __syncthreads();
  if (!norm) return;
  float ss[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < H / 256; ++i) {
      const float q = xs[t * H + tid + 256 * i];
      s = __fmaf_rn(q, q, s);
    }
    ss[t] = wave_sum(s);
  }
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) red[4 * t + wv] = ss[t];
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float ms = ((red[4 * t] + red[4 * t + 1]) + (red[4 * t + 2] + red[4 * t + 3])) / (float)H;
    const float inv = 1.0f / sqrtf(ms + eps);
#pragma unroll
    for (int i = 0; i < H / 256; ++i) xs[t * H + tid + 256 * i] *= inv;
  }
  __syncthreads();
}

// (v, i) is a better greedy candidate than (bv, bi): larger value, or the
// same value at a lower index (index -1 = none, which loses every tie).
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && (uint32_t)i < (uint32_t)bi);
}

}  // namespace

// ---------------------------------------------------------------------------
// lm_head: logits = W z (z = RMSNorm(h) or h), W [vocab][1280] bf16 or int8
// with f32 group scales; every workgroup also leaves its best (logit, id) per
// token, which the selection kernel reduces to the greedy token.
// A workgroup of 4 waves covers HEAD_ROWS consecutive rows: 16 lanes per
// row, 4 rows per wave step, HEAD_ROWS / 16 steps per wave.
// ---------------------------------------------------------------------------
template <int WT, int NT>
__global__ __launch_bounds__(256) void head_kernel(HeadArgs a) {
  constexpr int EPP = 128 / WT, P = H / EPP;          // pieces per row: 160 (bf16), 80 (int8)
  constexpr int LPR = 16, KPL = P / LPR, RG = 64 / LPR;
  constexpr int NSTEP = HEAD_ROWS / (4 * RG);         // wave steps
  static_assert(P % LPR == 0, "whole pieces per lane");
  __shared__ __attribute__((aligned(16))) float xs[NT * H];
  __shared__ float xsum[WT == 8 ? NT * P : 1];        // int8: per token and piece, the sum of its z
  __shared__ float red[4 * NT];
  __shared__ float cv[4][NT];
  __shared__ int ci[4][NT];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, rg = lane / LPR, l = lane % LPR;
  const int row0 = (blockIdx.x * 4 + wv) * RG * NSTEP;
  const uint32_t rb = H * WT / 8;                     // bytes per row
  const __amdgpu_buffer_rsrc_t rw = dense_rsrc(a.w, (uint32_t)a.vocab * rb);
  const int ng = H / a.group;
  const __amdgpu_buffer_rsrc_t rs = dense_rsrc(a.s, WT == 16 ? 0u : (uint32_t)a.vocab * ng * 4);

  uint4 wb[2][KPL];
  float sc[2][KPL];
  auto load = [&](int s, int slot) {
    const int row = row0 + s * RG + rg;
    const bool live = row < a.vocab;
#pragma unroll
    for (int m = 0; m < KPL; ++m) {
      const int p = l + LPR * m;
      wb[slot][m] = dload16(rw, live ? (uint32_t)row * rb + 16 * p : OUT_OF_RANGE);
      if (WT != 16) sc[slot][m] = dload4(rs, live ? ((uint32_t)row * ng + (EPP * p) / a.group) * 4 : OUT_OF_RANGE);
    }
  };
  rows_to_lds<NT>(a.h, a.T, a.norm, a.eps, xs, red, [&] { load(0, 0); });
  if (WT == 8) {
    for (int u = tid; u < NT * P; u += 256) {
      const float* xp = xs + (u / P) * H + EPP * (u % P);
      float sm = 0.f;
#pragma unroll
      for (int i = 0; i < EPP; ++i) sm += xp[i];
      xsum[u] = sm;
    }
    __syncthreads();
  }

  float bv[NT];
  int bi[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) { bv[t] = -__builtin_inff(); bi[t] = -1; }
#pragma unroll
  for (int s = 0; s < NSTEP; ++s) {
    if (s + 1 < NSTEP) load(s + 1, (s + 1) & 1);
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.f;
#pragma unroll
    for (int m = 0; m < KPL; ++m)
      piece_fma<WT, NT, H>(wb[s & 1][m], xs, EPP * (l + LPR * m), sc[s & 1][m], acc, WT == 8 ? xsum : nullptr, P);
    const int row = row0 + s * RG + rg;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float v = group_sum<LPR>(acc[t]);
      if (l == 0 && row < a.vocab) {
        if (a.logits) a.logits[(size_t)t * a.vocab + row] = v;
        if (better(v, row, bv[t], bi[t])) { bv[t] = v; bi[t] = row; }
      }
    }
  }
  // best of the wave: the four row groups' leaders (lanes 0, 16, 32, 48)
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float v = lane_value(bv[t], 0);
    int i = __builtin_amdgcn_readlane(bi[t], 0);
#pragma unroll
    for (int g = 1; g < RG; ++g) {
      const float vg = lane_value(bv[t], LPR * g);
      const int ig = __builtin_amdgcn_readlane(bi[t], LPR * g);
      if (better(vg, ig, v, i)) { v = vg; i = ig; }
    }
    if (lane == 0) { cv[wv][t] = v; ci[wv][t] = i; }
  }
  __syncthreads();
  if (tid < NT) {
    float v = cv[0][tid];
    int i = ci[0][tid];
#pragma unroll
    for (int w = 1; w < 4; ++w)
      if (better(cv[w][tid], ci[w][tid], v, i)) { v = cv[w][tid]; i = ci[w][tid]; }
    a.cand[((size_t)tid * gridDim.x + blockIdx.x) * 2] = v;
    a.cand[((size_t)tid * gridDim.x + blockIdx.x) * 2 + 1] = __int_as_float(i);
  }
}

// Greedy token of token t (= blockIdx.x) from the n_wg workgroup candidates
// ([T][n_wg] (logit, id) pairs): 256 threads, each with four candidates in
// flight per round, then a butterfly over each wave's lanes and the four
// wave winners in order.  "better" is a total order, so the winner does not
// depend on the order of the comparisons.
__global__ __launch_bounds__(256) void head_select_kernel(HeadArgs a, int n_wg) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float2* c = (const float2*)a.cand + (size_t)t * n_wg;
  float v = -__builtin_inff();
  int i = -1;
  for (int w0 = tid; w0 < n_wg; w0 += 4 * 256) {
    float2 q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int w = w0 + 256 * u;
      q[u] = w < n_wg ? c[w] : make_float2(-__builtin_inff(), __int_as_float(-1));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (better(q[u].x, __float_as_int(q[u].y), v, i)) { v = q[u].x; i = __float_as_int(q[u].y); }
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) {
    const float ov = __shfl_xor(v, d);
    const int oi = __shfl_xor(i, d);
    if (better(ov, oi, v, i)) { v = ov; i = oi; }
  }
  if (lane == 0) { sv[wv] = v; si[wv] = i; }
  __syncthreads();
  if (tid == 0) {
#pragma unroll
    for (int w = 1; w < 4; ++w)
      if (better(sv[w], si[w], v, i)) { v = sv[w]; i = si[w]; }
    a.token[t] = i;
    a.token_logit[t] = v;
  }
}

// ---------------------------------------------------------------------------
// Dense MLP, gate/up: h[t][j] = SiLU(g_j) * u_j with g = W_g z, u = W_u z
// (z = RMSNorm(x) or x), codes int8 or int4 with f32 group scales.  The row
// groups of a wave step alternate gate and up rows of the same intermediate
// columns, so a column's two sums meet with one lane exchange.
// ---------------------------------------------------------------------------
template <int BITS, int NT>
__global__ __launch_bounds__(256) void dense_gateup_kernel(DenseGateUpArgs a) {
  constexpr int EPP = 128 / BITS, P = H / EPP;        // 80 (int8) or 40 (int4) pieces per row
  constexpr int LPR = BITS == 8 ? 16 : 8, KPL = P / LPR, RG = 64 / LPR, CPS = RG / 2;
  static_assert(P % LPR == 0, "whole pieces per lane");
  __shared__ __attribute__((aligned(16))) float xs[NT * H];
  __shared__ float red[4 * NT];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, rg = lane / LPR, l = lane % LPR;
  const int mat = rg & 1;                             // 0: gate row, 1: up row
  const int col0 = (blockIdx.x * 4 + wv) * CPS * DENSE_GU_STEPS;
  const uint32_t rb = H * BITS / 8;
  const int ng = H / a.group;
  const __amdgpu_buffer_rsrc_t rw = dense_rsrc(a.q, 2u * a.inter * rb);
  const __amdgpu_buffer_rsrc_t rs = dense_rsrc(a.s, 2u * a.inter * ng * 4);

  uint4 wb[2][KPL];
  float sc[2][KPL];
  auto load = [&](int s, int slot) {
    const int col = col0 + s * CPS + (rg >> 1);
    const bool live = col < a.inter;
    const uint32_t row = (uint32_t)(mat * a.inter + col);
#pragma unroll
    for (int m = 0; m < KPL; ++m) {
      const int p = l + LPR * m;
      wb[slot][m] = dload16(rw, live ? row * rb + 16 * p : OUT_OF_RANGE);
      sc[slot][m] = dload4(rs, live ? (row * ng + (EPP * p) / a.group) * 4 : OUT_OF_RANGE);
    }
  };
  static_assert(DENSE_GU_STEPS == 2, "both steps' weights are in flight from the start");
  rows_to_lds<NT>(a.x, a.T, a.norm, a.eps, xs, red, [&] {
    load(0, 0);
    load(1, 1);
  });
#pragma unroll
  for (int s = 0; s < DENSE_GU_STEPS; ++s) {
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.f;
#pragma unroll
    for (int m = 0; m < KPL; ++m) piece_fma<BITS, NT, H>(wb[s & 1][m], xs, EPP * (l + LPR * m), sc[s & 1][m], acc);
    const int col = col0 + s * CPS + (rg >> 1);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float v = group_sum<LPR>(acc[t]);
      const float u = __shfl_xor(v, LPR);              // the partner group's sum
      if (mat == 0 && l == 0 && col < a.inter) a.hmid[(size_t)t * a.inter + col] = v / (1.0f + expf(-v)) * u;
    }
  }
}

// ---------------------------------------------------------------------------
// Dense MLP, down: y[t][r] (+)= sum_j W_d[r][j] h[t][j] over the intermediate
// (up to DENSE_MAX_INTER), one row per wave, h in LDS padded with zeros to
// whole pieces of every lane.
// ---------------------------------------------------------------------------
template <int BITS, int NT>
__global__ __launch_bounds__(256) void dense_down_kernel(DenseDownArgs a) {
  constexpr int EPP = 128 / BITS, KPL = DENSE_MAX_INTER / EPP / 64, XS = DENSE_MAX_INTER;
  __shared__ __attribute__((aligned(16))) float xs[NT * XS];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int row = blockIdx.x * 4 + wv;
  const uint32_t rb = (uint32_t)a.inter * BITS / 8;
  const int P = a.inter / EPP, ng = a.inter / a.group;
  const __amdgpu_buffer_rsrc_t rw = dense_rsrc(a.q, (uint32_t)H * rb);
  const __amdgpu_buffer_rsrc_t rs = dense_rsrc(a.s, (uint32_t)H * ng * 4);
  uint4 wb[KPL];
  float sc[KPL];
#pragma unroll
  for (int m = 0; m < KPL; ++m) {
    const int p = lane + 64 * m;
    const bool live = p < P;
    wb[m] = dload16(rw, live ? (uint32_t)row * rb + 16 * p : OUT_OF_RANGE);
    sc[m] = dload4(rs, live ? ((uint32_t)row * ng + (EPP * p) / a.group) * 4 : OUT_OF_RANGE);
  }
  // h rows into LDS, zeros past the intermediate
  const __amdgpu_buffer_rsrc_t rh = dense_rsrc(a.hmid, (uint32_t)a.T * a.inter * 4);
  const int nq = a.inter / 4;
  for (int u = tid; u < NT * XS / 4; u += 256) {
    const int t = u / (XS / 4), k = u % (XS / 4);
    const bool live = t < a.T && k < nq;
    const u32x4d q = __builtin_amdgcn_raw_buffer_load_b128(rh, live ? ((uint32_t)t * a.inter + 4 * k) * 4 : OUT_OF_RANGE, 0, 0);
    *(uint4*)&xs[4 * u] = make_uint4(q[0], q[1], q[2], q[3]);
  }
  __syncthreads();
  float acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = 0.f;
#pragma unroll
  for (int m = 0; m < KPL; ++m) piece_fma<BITS, NT, XS>(wb[m], xs, EPP * (lane + 64 * m), sc[m], acc);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float v = wave_sum(acc[t]);
    if (lane == 0 && row < H && t < a.T) {
      float* yp = a.y + (size_t)t * H + row;
      *yp = a.accumulate ? *yp + v : v;
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
int head_workgroups(int vocab) { return (vocab + HEAD_ROWS - 1) / HEAD_ROWS; }

template <int NT>
static void launch_head_nt(const HeadArgs& a, bool bf16, hipStream_t s) {
  const dim3 grid(head_workgroups(a.vocab));
  if (bf16) hipLaunchKernelGGL((head_kernel<16, NT>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((head_kernel<8, NT>), grid, dim3(256), 0, s, a);
}

hipError_t launch_head(const HeadArgs& a, bool bf16, hipStream_t s) {
  switch (a.T) {
    case 1: launch_head_nt<1>(a, bf16, s); break;
    case 2: launch_head_nt<2>(a, bf16, s); break;
    case 3: launch_head_nt<3>(a, bf16, s); break;
    default: launch_head_nt<4>(a, bf16, s); break;
  }
  hipLaunchKernelGGL(head_select_kernel, dim3(a.T), dim3(256), 0, s, a, head_workgroups(a.vocab));
  return hipGetLastError();
}

template <int BITS, int NT>
static void launch_dense_nt(const DenseGateUpArgs& g, const DenseDownArgs& d, hipStream_t s) {
  constexpr int CPW = (BITS == 8 ? 2 : 4) * DENSE_GU_STEPS;   // intermediate columns per wave
  hipLaunchKernelGGL((dense_gateup_kernel<BITS, NT>), dim3((g.inter + 4 * CPW - 1) / (4 * CPW)), dim3(256), 0, s, g);
  hipLaunchKernelGGL((dense_down_kernel<BITS, NT>), dim3(H / 4), dim3(256), 0, s, d);
}

hipError_t launch_dense(const DenseGateUpArgs& g, const DenseDownArgs& d, hipStream_t s) {
  const bool b8 = g.bits == 8;
  switch (g.T) {
    case 1: b8 ? launch_dense_nt<8, 1>(g, d, s) : launch_dense_nt<4, 1>(g, d, s); break;
    case 2: b8 ? launch_dense_nt<8, 2>(g, d, s) : launch_dense_nt<4, 2>(g, d, s); break;
    case 3: b8 ? launch_dense_nt<8, 3>(g, d, s) : launch_dense_nt<4, 3>(g, d, s); break;
    default: b8 ? launch_dense_nt<8, 4>(g, d, s) : launch_dense_nt<4, 4>(g, d, s); break;
  }
  return hipGetLastError();
}

}  // namespace moe
