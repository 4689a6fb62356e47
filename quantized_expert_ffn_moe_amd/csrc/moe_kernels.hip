// gfx950 kernels of the quantized expert-FFN MoE layer.
//
// The layer (browser demo page "A 3-billion-parameter OCR model. In this tab.",
// "One forward pass, left to right", step 6; franken_ocr README "Architecture"):
// softmax router over 64 experts, greedy top-6 without renormalisation,
// SwiGLU experts on int4/int8 codes with one f32 scale per group of K
// ("Four bits, one shared scale"), two fused shared experts, weighted combine.
//
// Two expert paths:
//  * GEMV path (few tokens): every (token, pick) streams its expert's packed
//    1 KiB tiles with 16-byte loads per lane, converts the offset-binary codes
//    in registers (v_cvt_f32_ubyte*) and accumulates in fp32 on the VALU.  The
//    group scale multiplies the fp32 partial sum of its group.
//  * Grouped path (many tokens): tokens are bucketed per expert (histogram +
//    stable permutation) and each expert's bucket runs as a dense GEMM on the
//    MFMA units (v_mfma_f32_16x16x32_f16).  The codes become exact f16 integers
//    in registers (magic-exponent trick); activations are staged in LDS as f16,
//    split into hi + lo halves when they are f32, so the products are exact and
//    only the fp32 accumulation rounds.  Group scales are applied to the fp32
//    partial sums of each group.
#include "moe_internal.h"

namespace moe {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ float bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
  return __uint_as_float(u);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

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
// One workgroup per 8 tokens; wave w owns experts 16w..16w+15 for the logits
// and tokens w, w+4 for the selection (one lane per expert).
// ---------------------------------------------------------------------------
constexpr int RT_TB = 8;

__global__ __launch_bounds__(256) void router_kernel(RouterArgs a) {
  __shared__ float zs[RT_TB][H];
  __shared__ float lg[RT_TB][E];
  __shared__ float red[RT_TB][4];
  const int t0 = blockIdx.x * RT_TB;
  const int nt = min(RT_TB, a.T - t0);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  for (int tt = 0; tt < nt; ++tt) {
    float v[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const size_t idx = (size_t)(t0 + tt) * H + tid + 256 * i;
      v[i] = a.x_bf16 ? bf16_to_f32(((const uint16_t*)a.x)[idx]) : ((const float*)a.x)[idx];
      zs[tt][tid + 256 * i] = v[i];
    }
    if (a.norm) {
      const float ss = wave_sum(thread_sumsq(v));
      if (lane == 0) red[tt][wv] = ss;
    }
  }
  __syncthreads();
  if (a.norm) {
    for (int tt = 0; tt < nt; ++tt) {
      const float inv = inv_rms(red[tt], a.eps);
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int k = tid + 256 * i;
        float z = zs[tt][k] * inv;
        if (a.norm_bf16) z = bf16_rne(z);
        zs[tt][k] = z;
        a.z[(size_t)(t0 + tt) * H + k] = z;
      }
    }
    __syncthreads();
  }
  for (int ei = 0; ei < 16; ++ei) {
    const int e = wv * 16 + ei;
    const float4* wrow = (const float4*)(a.wr + (size_t)e * H);
    float4 wr4[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) wr4[i] = wrow[lane + 64 * i];
    const float b = a.bias ? a.bias[e] : 0.f;
    for (int tt = 0; tt < nt; ++tt) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const float4 z4 = *(const float4*)&zs[tt][4 * (lane + 64 * i)];
        acc += wr4[i].x * z4.x + wr4[i].y * z4.y + wr4[i].z * z4.z + wr4[i].w * z4.w;
      }
      acc = wave_sum(acc);
      if (lane == 0) lg[tt][e] = acc + b;
    }
  }
  __syncthreads();
  for (int tt = wv; tt < nt; tt += 4) {
    const float v = lg[tt][lane];
    const float m = wave_max(v);
    const float ex = expf(v - m);
    const float p = ex / wave_sum(ex);
    bool taken = false;
    for (int j = 0; j < TOPK; ++j) {
      float bv = taken ? -1.f : p;
      int bi = lane;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      if (lane == bi) taken = true;
      if (lane == 0) {
        a.ids[(size_t)(t0 + tt) * TOPK + j] = bi;
        a.w[(size_t)(t0 + tt) * TOPK + j] = bv;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// GEMV path helpers.  A lane of a packed tile holds, per 32-wide K chunk, the
// 8 codes k = 32c + 8q + i (q = lane / 16) of row lane % 16.
// dot8 returns sum_i code_i * x_i over those 8 codes, codes read offset-binary.
// ---------------------------------------------------------------------------
template <int BITS>
__device__ __forceinline__ float dot8(const uint4& v, int c, const float* xv);

template <>
__device__ __forceinline__ float dot8<4>(const uint4& v, int c, const float* xv) {
  const uint32_t w = word_of(v, c);
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  float d = (float)(lo & 0xFFu) * xv[0];
  d += (float)(hi & 0xFFu) * xv[1];
  d += (float)((lo >> 8) & 0xFFu) * xv[2];
  d += (float)((hi >> 8) & 0xFFu) * xv[3];
  d += (float)((lo >> 16) & 0xFFu) * xv[4];
  d += (float)((hi >> 16) & 0xFFu) * xv[5];
  d += (float)(lo >> 24) * xv[6];
  d += (float)(hi >> 24) * xv[7];
  return d;
}

template <>
__device__ __forceinline__ float dot8<8>(const uint4& v, int c, const float* xv) {
  const uint32_t w0 = word_of(v, 2 * c), w1 = word_of(v, 2 * c + 1);
  float d = (float)(w0 & 0xFFu) * xv[0];
  d += (float)((w0 >> 8) & 0xFFu) * xv[1];
  d += (float)((w0 >> 16) & 0xFFu) * xv[2];
  d += (float)(w0 >> 24) * xv[3];
  d += (float)(w1 & 0xFFu) * xv[4];
  d += (float)((w1 >> 8) & 0xFFu) * xv[5];
  d += (float)((w1 >> 16) & 0xFFu) * xv[6];
  d += (float)(w1 >> 24) * xv[7];
  return d;
}

template <int BITS> __device__ constexpr float code_offset() { return BITS == 4 ? 8.f : 128.f; }

// One workgroup = one (token, expert) unit x 32 intermediate columns
// (gate and up tiles 2cb, 2cb+1).  The four waves split the K tiles.
template <int BITS>
__global__ __launch_bounds__(256) void dec_gateup_kernel(DecGateUpArgs a) {
  constexpr int KB = kb_cols(BITS), NKB = H / KB, CPT = KB / 32, KPW = (NKB + 3) / 4;
  constexpr float OFF = code_offset<BITS>();
  const int inter = a.w.inter;
  const int ncb = inter / 32;
  const int unit = blockIdx.x / ncb, cb = blockIdx.x % ncb;
  const int t = unit / a.units_per_token;
  const int e = a.ids ? a.ids[unit] : 0;
  const uint8_t* gq = a.w.q + (size_t)e * a.w.e_bytes;
  const float* gs = a.w.s + (size_t)e * a.w.e_scales;
  const size_t mbytes = matrix_bytes(BITS, inter, H);
  const int ng = H / a.w.group;
  const int gshift = __builtin_ctz(a.w.group);
  const size_t mscales = (size_t)inter * ng;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r = lane & 15, q4 = lane >> 4;
  __shared__ float xs[H];
  __shared__ float red[4][4][16];

  uint4 code[4][KPW];
  float sc[4][KPW][CPT];
#pragma unroll
  for (int kk = 0; kk < KPW; ++kk) {
    const int kb = wv + 4 * kk;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ntile = 2 * cb + (i & 1);
      const uint8_t* mq = gq + (i >= 2 ? mbytes : 0);
      const float* ms = gs + (i >= 2 ? mscales : 0);
      if (kb < NKB) {
        code[i][kk] = *(const uint4*)(mq + ((size_t)ntile * NKB + kb) * TILE + lane * 16);
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          const int grp = (kb * KB + 32 * c) >> gshift;
          sc[i][kk][c] = ms[((size_t)ntile * ng + grp) * 16 + r];
        }
      }
    }
  }
  for (int k = tid; k < H; k += 256)
    xs[k] = a.xf ? a.xf[(size_t)t * H + k] : bf16_to_f32(a.xb[(size_t)t * H + k]);
  __syncthreads();

  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < KPW; ++kk) {
    const int kb = wv + 4 * kk;
    if (kb < NKB) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const float* xp = xs + kb * KB + 32 * c + 8 * q4;
        float xv[8];
        *(float4*)&xv[0] = *(const float4*)xp;
        *(float4*)&xv[4] = *(const float4*)(xp + 4);
        const float X = ((xv[0] + xv[1]) + (xv[2] + xv[3])) + ((xv[4] + xv[5]) + (xv[6] + xv[7]));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float d = dot8<BITS>(code[i][kk], c, xv);
          acc[i] += sc[i][kk][c] * (d - OFF * X);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v = acc[i];
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    if (q4 == 0) red[wv][i][r] = v;
  }
  __syncthreads();
  if (tid < 32) {
    const int ti = tid >> 4, rr = tid & 15;
    const float g = (red[0][ti][rr] + red[1][ti][rr]) + (red[2][ti][rr] + red[3][ti][rr]);
    const float u = (red[0][2 + ti][rr] + red[1][2 + ti][rr]) + (red[2][2 + ti][rr] + red[3][2 + ti][rr]);
    a.h[(size_t)unit * inter + cb * 32 + tid] = silu_mul(g, u);
  }
}

// One workgroup = one token x 16 output rows; its 8 waves share the
// (source, K tile) items of the six routed down projections and the shared one,
// and the partial sums are added in a fixed order (deterministic).
template <int BR, int BS>
__global__ __launch_bounds__(512) void dec_down_kernel(DecDownArgs a) {
  constexpr int KBR = kb_cols(BR), NKR = I / KBR, CPR = KBR / 32;
  constexpr int KBS = kb_cols(BS), NKS = IS / KBS, CPS = KBS / 32;
  constexpr int CPM = CPR > CPS ? CPR : CPS;
  constexpr int ITEMS = TOPK * NKR + NKS, IPW = (ITEMS + 7) / 8;
  constexpr float OFFR = code_offset<BR>(), OFFS = code_offset<BS>();
  const int t = blockIdx.x / (H / 16), ntile = blockIdx.x % (H / 16);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r = lane & 15, q4 = lane >> 4;
  __shared__ float hs[TOPK * I + IS];
  __shared__ float red[8][16];

  const size_t rdown = 2 * matrix_bytes(BR, I, H), sdown = 2 * matrix_bytes(BS, IS, H);
  const int ngr = I / a.rw.group, ngs = IS / a.sw.group;
  const int shr = __builtin_ctz(a.rw.group), shs = __builtin_ctz(a.sw.group);
  const size_t rdown_s = 2 * (size_t)I * (H / a.rw.group), sdown_s = 2 * (size_t)IS * (H / a.sw.group);

  uint4 code[IPW];
  float sc[IPW][CPM];
#pragma unroll
  for (int m = 0; m < IPW; ++m) {
    const int it = wv + 8 * m;
    if (it < TOPK * NKR) {
      const int j = it / NKR, kb = it % NKR;
      const int e = a.ids[(size_t)t * TOPK + j];
      const uint8_t* base = a.rw.q + (size_t)e * a.rw.e_bytes + rdown;
      const float* sbase = a.rw.s + (size_t)e * a.rw.e_scales + rdown_s;
      code[m] = *(const uint4*)(base + ((size_t)ntile * NKR + kb) * TILE + lane * 16);
#pragma unroll
      for (int c = 0; c < CPR; ++c)
        sc[m][c] = sbase[((size_t)ntile * ngr + ((kb * KBR + 32 * c) >> shr)) * 16 + r];
    } else if (it < ITEMS) {
      const int kb = it - TOPK * NKR;
      const uint8_t* base = a.sw.q + sdown;
      const float* sbase = a.sw.s + sdown_s;
      code[m] = *(const uint4*)(base + ((size_t)ntile * NKS + kb) * TILE + lane * 16);
#pragma unroll
      for (int c = 0; c < CPS; ++c)
        sc[m][c] = sbase[((size_t)ntile * ngs + ((kb * KBS + 32 * c) >> shs)) * 16 + r];
    }
  }
  for (int k = tid; k < TOPK * I; k += 512) hs[k] = a.h_routed[(size_t)t * TOPK * I + k];
  for (int k = tid; k < IS; k += 512) hs[TOPK * I + k] = a.h_shared[(size_t)t * IS + k];
  __syncthreads();

  float acc = 0.f;
#pragma unroll
  for (int m = 0; m < IPW; ++m) {
    const int it = wv + 8 * m;
    if (it < TOPK * NKR) {
      const int j = it / NKR, kb = it % NKR;
      const float coef = a.tw[(size_t)t * TOPK + j];
#pragma unroll
      for (int c = 0; c < CPR; ++c) {
        const float* xp = hs + j * I + kb * KBR + 32 * c + 8 * q4;
        float xv[8];
        *(float4*)&xv[0] = *(const float4*)xp;
        *(float4*)&xv[4] = *(const float4*)(xp + 4);
        const float X = ((xv[0] + xv[1]) + (xv[2] + xv[3])) + ((xv[4] + xv[5]) + (xv[6] + xv[7]));
        acc += coef * sc[m][c] * (dot8<BR>(code[m], c, xv) - OFFR * X);
      }
    } else if (it < ITEMS) {
      const int kb = it - TOPK * NKR;
#pragma unroll
      for (int c = 0; c < CPS; ++c) {
        const float* xp = hs + TOPK * I + kb * KBS + 32 * c + 8 * q4;
        float xv[8];
        *(float4*)&xv[0] = *(const float4*)xp;
        *(float4*)&xv[4] = *(const float4*)(xp + 4);
        const float X = ((xv[0] + xv[1]) + (xv[2] + xv[3])) + ((xv[4] + xv[5]) + (xv[6] + xv[7]));
        acc += sc[m][c] * (dot8<BS>(code[m], c, xv) - OFFS * X);
      }
    }
  }
  acc += __shfl_xor(acc, 16);
  acc += __shfl_xor(acc, 32);
  if (q4 == 0) red[wv][r] = acc;
  __syncthreads();
  if (tid < 16) {
    float total = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) total += red[w][tid];
    const size_t yi = (size_t)t * H + ntile * 16 + tid;
    a.y[yi] = (a.accumulate ? a.y[yi] : 0.f) + total;
  }
}

// ---------------------------------------------------------------------------
// Histogram + stable permutation of the (token, pick) slots by expert.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void hist_kernel(HistArgs a) {
  __shared__ uint8_t sid[MOE_MAX_SLOTS];
  __shared__ int cnt[E], off[E + 1];
  const int N = a.T * TOPK;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int i = tid; i < N; i += 1024) sid[i] = (uint8_t)a.ids[i];
  __syncthreads();
  for (int ee = 0; ee < 4; ++ee) {
    const int e = wv * 4 + ee;
    int c = 0;
    for (int base = 0; base < N; base += 64) {
      const int i = base + lane;
      c += __popcll(__ballot(i < N && sid[i] == e));
    }
    if (lane == 0) cnt[e] = c;
  }
  __syncthreads();
  if (tid == 0) {
    off[0] = 0;
    int n = 0;
    for (int e = 0; e < E; ++e) {
      off[e + 1] = off[e] + cnt[e];
      a.counts[e] = cnt[e];
      a.offsets[e] = off[e];
      for (int r0 = 0; r0 < cnt[e]; r0 += MT) {
        a.tiles[2 * n] = e;
        a.tiles[2 * n + 1] = r0;
        ++n;
      }
    }
    a.offsets[E] = off[E];
    *a.ntiles = n;
  }
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1ull;
  for (int ee = 0; ee < 4; ++ee) {
    const int e = wv * 4 + ee;
    int run = off[e];
    for (int base = 0; base < N; base += 64) {
      const int i = base + lane;
      const bool m = i < N && sid[i] == e;
      const uint64_t mask = __ballot(m);
      if (m) {
        const int p = run + __popcll(mask & below);
        a.perm[p] = i;
        a.pos_of[i] = p;
      }
      run += __popcll(mask);
    }
  }
}

// ---------------------------------------------------------------------------
// Grouped path: exact-integer f16 operands on v_mfma_f32_16x16x32_f16.
// ---------------------------------------------------------------------------
__device__ __forceinline__ half2v as_h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }

// int4 word (codes k0..k7 in nibbles 0..7, offset-binary) -> exact f16 codes
// in MFMA operand order [k0, k4, k1, k5, k2, k6, k3, k7]:
// 0x6400 | n is the f16 value 1024 + n, and 0x6400 | (n << 4) is 1024 + 16n.
__device__ __forceinline__ half8 unpack_int4(uint32_t w) {
  const half2v m1032 = {(_Float16)-1032.f, (_Float16)-1032.f};
  const half2v m72 = {(_Float16)-72.f, (_Float16)-72.f};
  const half2v inv16 = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t w8 = w >> 8;
  const half2v a = as_h2((w & 0x000F000Fu) | 0x64006400u) + m1032;
  const half2v b = as_h2((w & 0x00F000F0u) | 0x64006400u) * inv16 + m72;
  const half2v c = as_h2((w8 & 0x000F000Fu) | 0x64006400u) + m1032;
  const half2v d = as_h2((w8 & 0x00F000F0u) | 0x64006400u) * inv16 + m72;
  return half8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// two int8 words (codes k0..k3, k4..k7 in bytes, offset-binary) -> exact f16
// codes in order [k0, k2, k1, k3, k4, k6, k5, k7].
__device__ __forceinline__ half8 unpack_int8(uint32_t w0, uint32_t w1) {
  const half2v m1152 = {(_Float16)-1152.f, (_Float16)-1152.f};
  const half2v a = as_h2((w0 & 0x00FF00FFu) | 0x64006400u) + m1152;
  const half2v b = as_h2(((w0 >> 8) & 0x00FF00FFu) | 0x64006400u) + m1152;
  const half2v c = as_h2((w1 & 0x00FF00FFu) | 0x64006400u) + m1152;
  const half2v d = as_h2(((w1 >> 8) & 0x00FF00FFu) | 0x64006400u) + m1152;
  return half8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// position p of an 8-wide operand slice holds element perm_k<BITS>(p)
template <int BITS> __device__ __forceinline__ int perm_k(int p) {
  return BITS == 4 ? ((p & 1) * 4 + (p >> 1)) : ((p & 4) + ((p & 1) << 1) + ((p >> 1) & 1));
}

constexpr int KS = 128;             // K staged in LDS per step
constexpr int LDS_ROW = KS + 8;     // f16 per LDS row (16-byte pad against bank conflicts)

// Stage A rows [row tile][k0 .. k0+KS) into LDS as f16 (hi plane, and lo plane
// when SPLIT), permuted within each 8-group to the B operand order.
template <int BITS, bool SPLIT>
__device__ __forceinline__ void stage_a(_Float16* lds, const float* af, const uint16_t* ab, const int* arow,
                                        int K, int k0) {
  const int tid = threadIdx.x;
  const int row = tid >> 3, seg = tid & 7;           // 32 rows x 8 segments of 16
  const int src = arow[row];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int kk = 16 * seg + 8 * h;
    float v[8];
    if (src < 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    } else if (af) {
      const float4* p = (const float4*)(af + (size_t)src * K + k0 + kk);
      const float4 a0 = p[0], a1 = p[1];
      v[0] = a0.x; v[1] = a0.y; v[2] = a0.z; v[3] = a0.w;
      v[4] = a1.x; v[5] = a1.y; v[6] = a1.z; v[7] = a1.w;
    } else {
      const uint4 u = *(const uint4*)(ab + (size_t)src * K + k0 + kk);
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
    if (SPLIT) *(half8*)(lds + 32 * LDS_ROW + row * LDS_ROW + kk) = lo;
  }
}

struct TileInfo { int valid, nrows, pbase, row0, e; };

__device__ __forceinline__ TileInfo tile_info(const GroupedArgs& a, int tile) {
  TileInfo ti;
  if (a.shared) {
    ti.row0 = tile * MT;
    ti.valid = ti.row0 < a.T;
    ti.nrows = min(MT, a.T - ti.row0);
    ti.pbase = 0; ti.e = 0;
  } else {
    ti.valid = tile < *a.ntiles;
    if (!ti.valid) { ti.nrows = 0; ti.pbase = 0; ti.row0 = 0; ti.e = 0; return ti; }
    ti.e = a.tiles[2 * tile];
    const int r0 = a.tiles[2 * tile + 1];
    const int cnt = a.offsets[ti.e + 1] - a.offsets[ti.e];
    ti.nrows = min(MT, cnt - r0);
    ti.pbase = a.offsets[ti.e] + r0;
    ti.row0 = 0;
  }
  return ti;
}

// Gate/up: a workgroup owns one 32-row tile of one expert and 64 intermediate
// columns; wave w computes gate and up for the 16 columns of n-subtile
// 4cb + w, then writes h = SiLU(gate) * up.
template <int BITS, bool SPLIT>
__global__ __launch_bounds__(256) void grouped_gateup_kernel(GroupedArgs a) {
  constexpr int KB = kb_cols(BITS), NKB = H / KB;
  constexpr int NSTAGE = H / KS;
  const int inter = a.w.inter, ncb = inter / 64;
  const int tile = blockIdx.x / ncb, cb = blockIdx.x % ncb;
  const TileInfo ti = tile_info(a, tile);
  if (!ti.valid) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r = lane & 15, q4 = lane >> 4;
  __shared__ __attribute__((aligned(16))) _Float16 lds[(SPLIT ? 2 : 1) * 32 * LDS_ROW];
  __shared__ int arow[MT];
  if (tid < MT) {
    int src = -1;
    if (tid < ti.nrows) src = a.shared ? ti.row0 + tid : a.perm[ti.pbase + tid] / TOPK;
    arow[tid] = src;
  }
  const uint8_t* eq = a.w.q + (size_t)ti.e * a.w.e_bytes;
  const float* es = a.w.s + (size_t)ti.e * a.w.e_scales;
  const size_t mbytes = matrix_bytes(BITS, inter, H);
  const int ng = H / a.w.group, cpg = a.w.group / 32;
  const size_t mscales = (size_t)inter * ng;
  const int ntile = 4 * cb + wv;

  float4v acc[2][2], ctmp[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) { acc[i][ms] = float4v{0, 0, 0, 0}; ctmp[i][ms] = float4v{0, 0, 0, 0}; }
  __syncthreads();

  for (int st = 0; st < NSTAGE; ++st) {
    // B tiles of this stage: int4 -> 1 tile (128 K), int8 -> 2 tiles (64 K each)
    uint4 bq[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int h = 0; h < (BITS == 4 ? 1 : 2); ++h) {
        const int kb = st * (KS / KB) + h;
        bq[i][h] = *(const uint4*)(eq + (i ? mbytes : 0) + ((size_t)ntile * NKB + kb) * TILE + lane * 16);
      }
    __syncthreads();
    stage_a<BITS, SPLIT>(lds, a.af, a.ab, arow, H, st * KS);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < KS / 32; ++c) {
      const int gc = st * (KS / 32) + c;
      const bool first = (gc % cpg) == 0, last = (gc % cpg) == cpg - 1;
      half8 bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (BITS == 4) bfr[i] = unpack_int4(word_of(bq[i][0], c));
        else bfr[i] = unpack_int8(word_of(bq[i][c >> 1], 2 * (c & 1)), word_of(bq[i][c >> 1], 2 * (c & 1) + 1));
      }
#pragma unroll
      for (int ms = 0; ms < 2; ++ms) {
        const int lrow = ms * 16 + r, lcol = 32 * c + 8 * q4;
        const half8 ahi = *(const half8*)(lds + lrow * LDS_ROW + lcol);
        half8 alo;
        if (SPLIT) alo = *(const half8*)(lds + 32 * LDS_ROW + lrow * LDS_ROW + lcol);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          float4v cc = first ? float4v{0, 0, 0, 0} : ctmp[i][ms];
          cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bfr[i], cc, 0, 0, 0);
          if (SPLIT) cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bfr[i], cc, 0, 0, 0);
          ctmp[i][ms] = cc;
        }
      }
      if (last) {
        const int grp = gc / cpg;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float s = es[(i ? mscales : 0) + ((size_t)ntile * ng + grp) * 16 + r];
#pragma unroll
          for (int ms = 0; ms < 2; ++ms) acc[i][ms] += s * ctmp[i][ms];
        }
      }
    }
  }
#pragma unroll
  for (int ms = 0; ms < 2; ++ms)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int m = ms * 16 + 4 * q4 + k;
      if (m < ti.nrows) {
        const size_t orow = a.shared ? (size_t)(ti.row0 + m) : (size_t)(ti.pbase + m);
        a.out[orow * inter + 16 * ntile + r] = silu_mul(acc[0][ms][k], acc[1][ms][k]);
      }
    }
}

// Down: a workgroup owns one 32-row tile and 128 output columns; wave w
// computes n-subtiles 8cb + 2w and 8cb + 2w + 1.  A = h (fp32) split hi/lo.
template <int BITS>
__global__ __launch_bounds__(256) void grouped_down_kernel(GroupedArgs a) {
  constexpr int KB = kb_cols(BITS);
  const int inter = a.w.inter, nkb = inter / KB, nstage = inter / KS;
  constexpr int NCB = H / 128;
  const int tile = blockIdx.x / NCB, cb = blockIdx.x % NCB;
  const TileInfo ti = tile_info(a, tile);
  if (!ti.valid) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r = lane & 15, q4 = lane >> 4;
  __shared__ __attribute__((aligned(16))) _Float16 lds[2 * 32 * LDS_ROW];
  __shared__ int arow[MT];
  if (tid < MT) arow[tid] = tid < ti.nrows ? (a.shared ? ti.row0 + tid : ti.pbase + tid) : -1;
  const uint8_t* dq = a.w.q + (size_t)ti.e * a.w.e_bytes + 2 * matrix_bytes(BITS, inter, H);
  const int ng = inter / a.w.group, cpg = a.w.group / 32;
  const float* ds = a.w.s + (size_t)ti.e * a.w.e_scales + 2 * (size_t)inter * (H / a.w.group);
  const int nt0 = 8 * cb + 2 * wv;

  float4v acc[2][2], ctmp[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) { acc[i][ms] = float4v{0, 0, 0, 0}; ctmp[i][ms] = float4v{0, 0, 0, 0}; }
  __syncthreads();

  for (int st = 0; st < nstage; ++st) {
    uint4 bq[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int h = 0; h < (BITS == 4 ? 1 : 2); ++h) {
        const int kb = st * (KS / KB) + h;
        bq[i][h] = *(const uint4*)(dq + ((size_t)(nt0 + i) * nkb + kb) * TILE + lane * 16);
      }
    __syncthreads();
    stage_a<BITS, true>(lds, a.af, nullptr, arow, inter, st * KS);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < KS / 32; ++c) {
      const int gc = st * (KS / 32) + c;
      const bool first = (gc % cpg) == 0, last = (gc % cpg) == cpg - 1;
      half8 bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (BITS == 4) bfr[i] = unpack_int4(word_of(bq[i][0], c));
        else bfr[i] = unpack_int8(word_of(bq[i][c >> 1], 2 * (c & 1)), word_of(bq[i][c >> 1], 2 * (c & 1) + 1));
      }
#pragma unroll
      for (int ms = 0; ms < 2; ++ms) {
        const int lrow = ms * 16 + r, lcol = 32 * c + 8 * q4;
        const half8 ahi = *(const half8*)(lds + lrow * LDS_ROW + lcol);
        const half8 alo = *(const half8*)(lds + 32 * LDS_ROW + lrow * LDS_ROW + lcol);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          float4v cc = first ? float4v{0, 0, 0, 0} : ctmp[i][ms];
          cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bfr[i], cc, 0, 0, 0);
          cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bfr[i], cc, 0, 0, 0);
          ctmp[i][ms] = cc;
        }
      }
      if (last) {
        const int grp = gc / cpg;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float s = ds[((size_t)(nt0 + i) * ng + grp) * 16 + r];
#pragma unroll
          for (int ms = 0; ms < 2; ++ms) acc[i][ms] += s * ctmp[i][ms];
        }
      }
    }
  }
#pragma unroll
  for (int ms = 0; ms < 2; ++ms)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int m = ms * 16 + 4 * q4 + k;
      if (m < ti.nrows) {
        const size_t orow = a.shared ? (size_t)(ti.row0 + m) : (size_t)(ti.pbase + m);
#pragma unroll
        for (int i = 0; i < 2; ++i) a.out[orow * H + 16 * (nt0 + i) + r] = acc[i][ms][k];
      }
    }
}

// y[t] (+)= ys[t] + sum_j w[t,j] * ysorted[pos_of[t*6+j]], picks added in order.
__global__ __launch_bounds__(320) void combine_kernel(CombineArgs a) {
  const int t = blockIdx.x, c = threadIdx.x * 4;
  float4 v = *(const float4*)(a.ys + (size_t)t * H + c);
#pragma unroll
  for (int j = 0; j < TOPK; ++j) {
    const float wj = a.tw[(size_t)t * TOPK + j];
    const float4 p = *(const float4*)(a.ysorted + (size_t)a.pos_of[(size_t)t * TOPK + j] * H + c);
    v.x += wj * p.x; v.y += wj * p.y; v.z += wj * p.z; v.w += wj * p.w;
  }
  float4* yp = (float4*)(a.y + (size_t)t * H + c);
  if (a.accumulate) {
    const float4 o = *yp;
    v.x = o.x + v.x; v.y = o.y + v.y; v.z = o.z + v.z; v.w = o.w + v.w;
  }
  *yp = v;
}

__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* h, void* z, int z_bf16, float eps) {
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
    if (z_bf16) ((uint16_t*)z)[idx] = (uint16_t)(__float_as_uint(bf16_rne(zz)) >> 16);
    else ((float*)z)[idx] = zz;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_router(const RouterArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(router_kernel, dim3((a.T + RT_TB - 1) / RT_TB), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dec_gateup(const DecGateUpArgs& a, int units, hipStream_t s) {
  const dim3 grid(units * (a.w.inter / 32));
  if (a.w.bits == 4) hipLaunchKernelGGL(dec_gateup_kernel<4>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(dec_gateup_kernel<8>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dec_down(const DecDownArgs& a, int T, hipStream_t s) {
  const dim3 grid(T * (H / 16));
  const int key = (a.rw.bits == 8) * 2 + (a.sw.bits == 8);
  switch (key) {
    case 0: hipLaunchKernelGGL((dec_down_kernel<4, 4>), grid, dim3(512), 0, s, a); break;
    case 1: hipLaunchKernelGGL((dec_down_kernel<4, 8>), grid, dim3(512), 0, s, a); break;
    case 2: hipLaunchKernelGGL((dec_down_kernel<8, 4>), grid, dim3(512), 0, s, a); break;
    default: hipLaunchKernelGGL((dec_down_kernel<8, 8>), grid, dim3(512), 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_hist(const HistArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(hist_kernel, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_grouped_gateup(const GroupedArgs& a, int max_tiles, hipStream_t s) {
  const dim3 grid(max_tiles * (a.w.inter / 64));
  const bool split = a.af != nullptr;
  if (a.w.bits == 4) {
    if (split) hipLaunchKernelGGL((grouped_gateup_kernel<4, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((grouped_gateup_kernel<4, false>), grid, dim3(256), 0, s, a);
  } else {
    if (split) hipLaunchKernelGGL((grouped_gateup_kernel<8, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((grouped_gateup_kernel<8, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_grouped_down(const GroupedArgs& a, int max_tiles, hipStream_t s) {
  const dim3 grid(max_tiles * (H / 128));
  if (a.w.bits == 4) hipLaunchKernelGGL(grouped_down_kernel<4>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(grouped_down_kernel<8>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel, dim3(a.T), dim3(320), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* h, void* z, int z_bf16, int T, float eps, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(256), 0, s, h, z, z_bf16, eps);
  return hipGetLastError();
}

}  // namespace moe
