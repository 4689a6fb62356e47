// Internal declarations shared by the host API and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int H = 1280;      // hidden size
constexpr int E = 64;        // routed experts
constexpr int TOPK = 6;      // experts picked per token
constexpr int I = 896;       // routed expert intermediate
constexpr int IS = 1792;     // fused shared expert intermediate
constexpr int TILE = 1024;   // bytes of one packed 16-row tile
constexpr int MT = 32;       // token rows per grouped-GEMM tile
constexpr int DECODE_MAX_T = 4;  // largest token count routed to the GEMV path by default
constexpr int MAX_T = 8192;      // largest token count of one call
constexpr int MOE_MAX_SLOTS = MAX_T * TOPK;

__host__ __device__ constexpr int kb_cols(int bits) { return bits == 4 ? 128 : 64; }
__host__ __device__ constexpr size_t matrix_bytes(int bits, int n, int k) { return (size_t)n * k * bits / 8; }

struct QW {            // one packed expert set (routed experts or the shared expert)
  const uint8_t* q;    // packed codes of expert 0
  const float* s;      // packed scales of expert 0
  size_t e_bytes;      // byte stride between experts
  size_t e_scales;     // float stride between experts
  int bits, group, inter;
};

struct RouterArgs {
  const void* x; int x_bf16; int T;
  const float* wr; const float* bias;
  int norm, norm_bf16; float eps;
  float* z;            // [T][H] normalised input (written when norm)
  int32_t* ids; float* w;
};

struct DecGateUpArgs {
  const float* xf; const uint16_t* xb;  // layer input, exactly one non-null
  int units_per_token;                  // 6 (routed) or 1 (shared)
  const int32_t* ids;                   // [T*6] expert of each routed unit, null for shared
  QW w;
  float* h;                             // [units][inter]
};

struct DecDownArgs {
  const int32_t* ids; const float* tw;  // routing of each token
  const float* h_routed;                // [T*6][I]
  const float* h_shared;                // [T][IS]
  QW rw, sw;
  float* y; int accumulate;
};

struct HistArgs {
  const int32_t* ids; int T;
  int32_t* counts; int32_t* offsets;    // [E], [E+1]
  int32_t* perm; int32_t* pos_of;       // [T*6]: sorted slot -> (t*6+j); (t*6+j) -> sorted position
  int32_t* tiles; int32_t* ntiles;      // [max][2] (expert, first row), count
};

struct GroupedArgs {
  // A rows
  const float* af; const uint16_t* ab;  // f32 or bf16 rows, row stride = K
  int T;
  int shared;                           // 1: rows are tokens 0..T-1 of the shared expert
  const int32_t* tiles; const int32_t* ntiles; const int32_t* offsets; const int32_t* perm;
  int a_by_token;                       // routed A rows: 1 = token rows (gate/up), 0 = sorted rows (down)
  QW w;
  float* out;                           // routed: [T*6][N] by sorted position; shared: [T][N]
};

struct CombineArgs {
  const float* ys; const float* ysorted; const int32_t* pos_of; const float* tw;
  float* y; int T; int accumulate;
};

hipError_t launch_router(const RouterArgs& a, hipStream_t s);
hipError_t launch_dec_gateup(const DecGateUpArgs& a, int units, hipStream_t s);
hipError_t launch_dec_down(const DecDownArgs& a, int T, hipStream_t s);
hipError_t launch_hist(const HistArgs& a, hipStream_t s);
hipError_t launch_grouped_gateup(const GroupedArgs& a, int max_tiles, hipStream_t s);
hipError_t launch_grouped_down(const GroupedArgs& a, int max_tiles, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_rmsnorm(const float* h, void* z, int z_bf16, int T, float eps, hipStream_t s);

}  // namespace moe
