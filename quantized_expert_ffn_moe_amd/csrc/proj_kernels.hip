// gfx950 kernel of the decoder's attention projections: q, k, v = W z and the
// output projection W_o a, for a decode step of T streams.  The attention is
// plain multi-head attention of ten heads of 128 (browser demo page "A
// 3-billion-parameter OCR model. In this tab.", "One forward pass, left to
// right", step 6; model card "The rest of the pipeline"), with bf16 weights
// (the conservative recipe keeps attention at source precision: franken_ocr
// README, "focr convert").
//
// y[t][n] (+)= sum_k a[t][k] W[n][k] over K = 1280, W bf16 row-major [N][1280].
// The f32 activations a arrive split into two bf16 halves by their producer
// (hi = bf16(a), lo = bf16(a - hi), 16 significant bits together; the
// split_row layout: the RMSNorm writes z so, the attention step its output),
// and both halves are multiplied on the bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16): the products are exact in fp32 and only the
// fp32 accumulation rounds.
#include "moe_internal.h"
#include "moe_wave.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float4p __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4p __attribute__((ext_vector_type(4)));

namespace {
constexpr int PJ_KW = H / 4;        // K columns of one wave (320)
constexpr int PJ_KS = PJ_KW / 32;   // its 32-wide k-steps (10)
constexpr int PJ_TT = 4;            // stream tiles of 16 per workgroup

// RMSNorm of a row with the standalone norm's arithmetic (thread tid owns
// features tid + 256 i, i < 5; squares added in that order, the four wave
// sums in a fixed order), so that both give bit-identical z
__device__ __forceinline__ float row_sumsq(const float (&v)[5]) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 5; ++i) ss = __fmaf_rn(v[i], v[i], ss);
  return ss;
}
__device__ __forceinline__ uint32_t bf16_bits(float v) {   // nearest, ties to even
  const uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
}  // namespace

// A workgroup of 4 waves owns NS 16-column subtiles and up to 64 streams (four
// tiles of 16).  With NORM (at most PJ_NORM_MAX_T streams) the workgroup
// first forms the split rows of RMSNorm(h) itself, in LDS, instead of reading
// them from a norm launch before it.  The waves split K in quarters: each keeps its quarter of the
// subtiles' weight rows in registers (read once) and multiplies every stream
// tile with it, each lane's two 16-byte loads being its A operands as they
// are (hi, then lo); the next tile is fetched while the current one is
// multiplied, and rows past T read as zeros (buffer range), so every load is
// issued without a branch.  The four K-quarter partials meet in LDS and are
// added by all 256 threads in a fixed order, one output each per subtile.
template <int NS, bool NORM>
__global__ __launch_bounds__(256) void proj_hl_kernel(ProjArgs p) {
  constexpr int NC = 16 * NS;                    // columns of the workgroup
  constexpr int NT = NORM ? PJ_NORM_MAX_T : 1;
  __shared__ float red[2][4][16][NC + 1];
  __shared__ __attribute__((aligned(16))) uint16_t als[NORM ? PJ_NORM_MAX_T * H * 2 : 8];
  __shared__ float nred[NT][4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r = lane & 15, q = lane >> 4;
  const int n0 = NC * blockIdx.x, tb = 64 * blockIdx.y;
  const int k0 = PJ_KW * wv + 8 * q;
  // NORM: the rows of h are requested before the weights, so that waiting for
  // them does not wait for the weights too (the load counter is in order);
  // rows past T read zeros (buffer range)
  float hv[NT][5];
  if constexpr (NORM) {
    const __amdgpu_buffer_rsrc_t rh =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.h_norm), (short)0, (uint32_t)p.T * H * 4, 0x00020000);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 5; ++i)
        hv[t][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rh, (uint32_t)(t * H + tid + 256 * i) * 4, 0, 0));
  }
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.w), (short)0, (uint32_t)p.N * H * 2, 0x00020000);
  uint4 b[NS][PJ_KS];
#pragma unroll
  for (int ns = 0; ns < NS; ++ns)
#pragma unroll
    for (int s = 0; s < PJ_KS; ++s) {
      const u32x4p v =
          __builtin_amdgcn_raw_buffer_load_b128(rw, ((uint32_t)(n0 + 16 * ns + r) * H + k0 + 32 * s) * 2, 0, 0);
      b[ns][s] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  // rows past T read zeros (buffer range); 4 bytes per element
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.a_hl), (short)0, NORM ? 0u : (uint32_t)p.T * H * 4,
                                        0x00020000);
  u32x4p x[2][PJ_KS][2];
  auto load = [&](u32x4p (&xb)[PJ_KS][2], int t0) {
#pragma unroll
    for (int s = 0; s < PJ_KS; ++s) {
      const uint32_t off = ((uint32_t)(t0 + r) * H + k0 + 32 * s) * 4;
      xb[s][0] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);        // hi of the 8 elements
      xb[s][1] = __builtin_amdgcn_raw_buffer_load_b128(ra, off + 16, 0, 0);   // lo
    }
  };
  if constexpr (NORM) {
    // z = h / sqrt(mean(h^2) + eps) per row, as split rows in LDS
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float ss = wave_sum(row_sumsq(hv[t]));
      if (lane == 0) nred[t][wv] = ss;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float inv = 1.0f / sqrtf(((nred[t][0] + nred[t][1]) + (nred[t][2] + nred[t][3])) / (float)H + p.eps);
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int idx = tid + 256 * i;
        const float zz = hv[t][i] * inv;
        const uint32_t hi = bf16_bits(zz);
        uint16_t* g = als + (t * H + (idx & ~7)) * 2 + (idx & 7);
        g[0] = (uint16_t)hi;
        g[8] = (uint16_t)bf16_bits(zz - __uint_as_float(hi << 16));
      }
    }
    __syncthreads();
    // the single stream tile (rows from T on are zeros)
#pragma unroll
    for (int s = 0; s < PJ_KS; ++s) {
      const u32x4p* ap = (const u32x4p*)(als + ((r < NT ? r : 0) * H + k0 + 32 * s) * 2);
      x[0][s][0] = r < p.T ? ap[0] : u32x4p{0u, 0u, 0u, 0u};
      x[0][s][1] = r < p.T ? ap[1] : u32x4p{0u, 0u, 0u, 0u};
    }
  } else {
    load(x[0], tb);
  }
  // this thread's outputs of each tile: token row tid / 16, columns
  // n0 + tid % 16 + 16 ns, through a descriptor over y (rows past T: loads
  // read zeros, stores are dropped)
  const int rr = tid >> 4, cc = tid & 15;
  const __amdgpu_buffer_rsrc_t ry =
      __builtin_amdgcn_make_buffer_rsrc(p.y, (short)0, (uint32_t)(p.N / H) * p.T * H * 4, 0x00020000);
#pragma unroll
  for (int tt = 0; tt < PJ_TT; ++tt) {
    const int t0 = tb + 16 * tt;
    if (t0 >= p.T) break;
    const int t = t0 + rr;
    uint32_t yo[NS];
    float yold[NS];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      const int n = n0 + 16 * ns + cc;
      yo[ns] = t < p.T ? (((uint32_t)(n / H) * p.T + t) * H + n % H) * 4 : 0x80000000u;
      // the old output (accumulating) is requested before the next tile's
      // activations, so waiting for it never waits for them (in-order counter)
      yold[ns] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ry, p.accumulate ? yo[ns] : 0x80000000u, 0, 0));
    }
    asm volatile("" ::: "memory");
    if (!NORM && tt + 1 < PJ_TT) load(x[(tt + 1) & 1], t0 + 16);   // unconditional: rows past T read zeros
    float4p c[NS];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) c[ns] = float4p{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < PJ_KS; ++s) {
      const bf16x8 hi = __builtin_bit_cast(bf16x8, x[tt & 1][s][0]);
      const bf16x8 lo = __builtin_bit_cast(bf16x8, x[tt & 1][s][1]);
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        const bf16x8 bw = __builtin_bit_cast(bf16x8, u32x4p{b[ns][s].x, b[ns][s].y, b[ns][s].z, b[ns][s].w});
        c[ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, bw, c[ns], 0, 0, 0);
        c[ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, bw, c[ns], 0, 0, 0);
      }
    }
    // lane (r, q) holds tokens t0 + 4 q + j of column n0 + 16 ns + r; red is
    // double buffered, so one barrier per tile separates its writes from its reads
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int j = 0; j < 4; ++j) red[tt & 1][wv][4 * q + j][16 * ns + r] = c[ns][j];
    __syncthreads();
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      const int cl = 16 * ns + cc;
      const float v = ((red[tt & 1][0][rr][cl] + red[tt & 1][1][rr][cl]) + red[tt & 1][2][rr][cl]) + red[tt & 1][3][rr][cl];
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(p.accumulate ? yold[ns] + v : v), ry, yo[ns], 0, 0);
    }
  }
}

hipError_t launch_proj(const ProjArgs& p, hipStream_t s) {
  if (p.T <= 0) return hipSuccess;
  if (p.h_norm) {
    if (p.T > PJ_NORM_MAX_T) return hipErrorInvalidValue;
    hipLaunchKernelGGL((proj_hl_kernel<1, true>), dim3(p.N / 16, 1), dim3(256), 0, s, p);
    return hipGetLastError();
  }
  const int tblocks = (p.T + 16 * PJ_TT - 1) / (16 * PJ_TT);
  if ((p.N / 32) * tblocks >= 200) {
    // 32 columns per workgroup halve the activation reads while keeping enough workgroups
    hipLaunchKernelGGL((proj_hl_kernel<2, false>), dim3(p.N / 32, tblocks), dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((proj_hl_kernel<1, false>), dim3(p.N / 16, tblocks), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace moe
