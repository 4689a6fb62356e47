// gfx950 kernel of the decoder's attention projections: q, k, v = W z and the
// output projection W_o a, for a decode step of T streams.  The attention is
// plain multi-head attention of ten heads of 128 (browser demo page "A
// 3-billion-parameter OCR model. In this tab.", "One forward pass, left to
// right", step 6; model card "The rest of the pipeline"), with bf16 weights
// (the conservative recipe keeps attention at source precision: franken_ocr
// README, "focr convert").
//
// y[t][n] (+)= sum_k a[t][k] W[n][k] over K = 1280, W bf16 row-major [N][1280],
// a f32 [T][1280].  Each f32 activation is split into two bf16 halves
// (hi = bf16(a), lo = bf16(a - hi), 16 significant bits together) and both
// halves are multiplied on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16):
// the products are exact in fp32 and only the fp32 accumulation rounds.
//
// A workgroup of 4 waves owns 16 output columns and up to 64 tokens (four
// tiles of 16).  The waves split K in quarters: each keeps its quarter of the
// 16 weight rows in registers (10 KB per wave, read once), multiplies every
// token tile with it and leaves a 16 x 16 partial in LDS; wave 0 adds the four
// quarters in a fixed order and writes the tile.  Activation rows past T read
// as zeros (buffer range), so every load is issued without a branch.
#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float4p __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4p __attribute__((ext_vector_type(4)));

namespace {
constexpr int PJ_KW = H / 4;        // K columns of one wave (320)
constexpr int PJ_KS = PJ_KW / 32;   // its 32-wide k-steps (10)
constexpr int PJ_TT = 4;            // token tiles of 16 per workgroup

__device__ __forceinline__ uint32_t bf16_rne_bits(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// 8 f32 -> (hi, lo) bf16x8 in element order
__device__ __forceinline__ void split8(const float4& x0, const float4& x1, bf16x8& hi, bf16x8& lo) {
  const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h0 = bf16_rne_bits(v[2 * i]), h1 = bf16_rne_bits(v[2 * i + 1]);
    const uint32_t l0 = bf16_rne_bits(v[2 * i] - __uint_as_float(h0 << 16));
    const uint32_t l1 = bf16_rne_bits(v[2 * i + 1] - __uint_as_float(h1 << 16));
    h[i] = h0 | (h1 << 16);
    l[i] = l0 | (l1 << 16);
  }
  hi = __builtin_bit_cast(bf16x8, u32x4p{h[0], h[1], h[2], h[3]});
  lo = __builtin_bit_cast(bf16x8, u32x4p{l[0], l[1], l[2], l[3]});
}
}  // namespace

__global__ __launch_bounds__(256) void proj_kernel(ProjArgs p) {
  __shared__ float red[4][16][17];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r = lane & 15, q = lane >> 4;
  const int n0 = 16 * blockIdx.x, tb = 64 * blockIdx.y;
  const int k0 = PJ_KW * wv + 8 * q;
  // this lane's weight pieces: row n0 + r, columns k0 + 32 s .. + 7
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.w), (short)0, (uint32_t)p.N * H * 2, 0x00020000);
  uint4 b[PJ_KS];
#pragma unroll
  for (int s = 0; s < PJ_KS; ++s) {
    const u32x4p v = __builtin_amdgcn_raw_buffer_load_b128(rw, ((uint32_t)(n0 + r) * H + k0 + 32 * s) * 2, 0, 0);
    b[s] = make_uint4(v[0], v[1], v[2], v[3]);
  }
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.a), (short)0, (uint32_t)p.T * H * 4, 0x00020000);
  const int n = n0 + r, blk = n / H, col = n % H;
#pragma unroll 1
  for (int tt = 0; tt < PJ_TT; ++tt) {
    const int t0 = tb + 16 * tt;
    if (t0 >= p.T) break;
    float4 x[PJ_KS][2];
#pragma unroll
    for (int s = 0; s < PJ_KS; ++s) {
      const uint32_t off = ((uint32_t)(t0 + r) * H + k0 + 32 * s) * 4;
      const u32x4p v0 = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
      const u32x4p v1 = __builtin_amdgcn_raw_buffer_load_b128(ra, off + 16, 0, 0);
      x[s][0] = make_float4(__uint_as_float(v0[0]), __uint_as_float(v0[1]), __uint_as_float(v0[2]), __uint_as_float(v0[3]));
      x[s][1] = make_float4(__uint_as_float(v1[0]), __uint_as_float(v1[1]), __uint_as_float(v1[2]), __uint_as_float(v1[3]));
    }
    float4p c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < PJ_KS; ++s) {
      bf16x8 hi, lo;
      split8(x[s][0], x[s][1], hi, lo);
      const bf16x8 bw = __builtin_bit_cast(bf16x8, u32x4p{b[s].x, b[s].y, b[s].z, b[s].w});
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, bw, c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, bw, c, 0, 0, 0);
    }
    // lane (r, q) holds tokens t0 + 4 q + j of column n0 + r
#pragma unroll
    for (int j = 0; j < 4; ++j) red[wv][4 * q + j][r] = c[j];
    __syncthreads();
    if (wv == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tr = 4 * q + j, t = t0 + tr;
        if (t < p.T) {
          const float v = ((red[0][tr][r] + red[1][tr][r]) + red[2][tr][r]) + red[3][tr][r];
          float* yp = p.y + ((size_t)blk * p.T + t) * H + col;
          *yp = p.accumulate ? *yp + v : v;
        }
      }
    }
    __syncthreads();
  }
}

// The same product for many streams, with the activations already split into
// bf16 halves by their producer (the RMSNorm, or the attention step, in the
// split_row layout): the per-tile split, which every column workgroup
// repeated for every stream, is gone, each lane's two 16-byte loads are its
// A operands as they are, and the next 16-stream tile is fetched while the
// current one is multiplied.  A workgroup owns NS 16-column subtiles (each
// wave keeps its K quarter of all of them in registers), so the activations
// are read once per 16 NS columns.  The four K-quarter partials are added by
// all 256 threads in the order of proj_kernel, and every column sees
// proj_kernel's MFMA sequence, so both give the same bits.
template <int NS>
__global__ __launch_bounds__(256) void proj_hl_kernel(ProjArgs p) {
  constexpr int NC = 16 * NS;                    // columns of the workgroup
  __shared__ float red[2][4][16][NC + 1];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r = lane & 15, q = lane >> 4;
  const int n0 = NC * blockIdx.x, tb = 64 * blockIdx.y;
  const int k0 = PJ_KW * wv + 8 * q;
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
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.a_hl), (short)0, (uint32_t)p.T * H * 4, 0x00020000);
  u32x4p x[2][PJ_KS][2];
  auto load = [&](u32x4p (&xb)[PJ_KS][2], int t0) {
#pragma unroll
    for (int s = 0; s < PJ_KS; ++s) {
      const uint32_t off = ((uint32_t)(t0 + r) * H + k0 + 32 * s) * 4;
      xb[s][0] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);        // hi of the 8 elements
      xb[s][1] = __builtin_amdgcn_raw_buffer_load_b128(ra, off + 16, 0, 0);   // lo
    }
  };
  load(x[0], tb);
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
    if (tt + 1 < PJ_TT) load(x[(tt + 1) & 1], t0 + 16);   // unconditional: rows past T read zeros
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
  const int tblocks = (p.T + 16 * PJ_TT - 1) / (16 * PJ_TT);
  if (!p.a_hl) {
    hipLaunchKernelGGL(proj_kernel, dim3(p.N / 16, tblocks), dim3(256), 0, s, p);
  } else if ((p.N / 32) * tblocks >= 200) {
    // 32 columns per workgroup halve the activation reads while keeping enough workgroups
    hipLaunchKernelGGL(proj_hl_kernel<2>, dim3(p.N / 32, tblocks), dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL(proj_hl_kernel<1>, dim3(p.N / 16, tblocks), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace moe
