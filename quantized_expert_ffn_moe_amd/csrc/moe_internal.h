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
constexpr int MT = 64;       // token rows per tile of the grouped GEMMs (large tiles)
constexpr int MT_SMALL = 32; // rows per tile when experts see few rows each
constexpr int MT_TINY = 16;  // rows per tile when experts see very few rows each (fused shared/routed launches)
constexpr int SMALL_WAVES = 8; // waves per workgroup of the small tiles (16 gate/up columns or half a down row tile each)
constexpr int SMALL_TILE_MAX_SLOTS = 64 * 64;   // (token, pick) slots up to which the small tiles run
constexpr int TINY_TILE_MAX_SLOTS = 64 * 8;     // ... and the 16-row tiles (about 8 rows per expert or fewer)
constexpr int DECODE_MAX_T = 18; // largest token count any format routes to the GEMV path by default
constexpr int MAX_T = 8192;      // largest token count of one call
constexpr int STATIC_MAX_T = 256;                      // largest call of the workspace-free entry point
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)20 << 20;  // its per-GPU scratch (the carve for 256 tokens fits)
constexpr int MOE_MAX_SLOTS = MAX_T * TOPK;

__host__ __device__ constexpr int kb_cols(int bits) { return bits == 4 ? 128 : 64; }
// rows of one packed down-projection tile (tiles cover 32 K columns)
__host__ __device__ constexpr int down_rows(int bits) { return bits == 4 ? 64 : 32; }
__host__ __device__ constexpr size_t matrix_bytes(int bits, int n, int k) { return (size_t)n * k * bits / 8; }

// Two-level 4-bit (Q4_K-style) format, selected by group == Q4K with 4-bit
// codes: super-blocks of Q4K_SB columns along K with f16 d and dmin, split
// into sub-blocks of Q4K_SUB columns with a 6-bit scale and a 6-bit minimum;
// the codes are the int4 tiles of q - 8.  Metadata of one expert:
//   gate and up: one 16-byte record per (row, super-block), [N][H / 256];
//   down, in the down tiles' row order (row 64 rt + 16 j + r at [rt][r][j]):
//     [ceil(inter / 256)][H / 64][16][4] words d | dmin << 16, then
//     [inter / 32][H / 64][16][4] halfwords sc | m << 8,
//   so that a down slice (one sub-block) reads 6 bytes per row.
constexpr int Q4K = 256;
constexpr int Q4K_SB = 256;
constexpr int Q4K_SUB = 32;
// Largest token count that moe_layer_forward routes to the per-token (GEMV)
// path by default, per routed format: the measured crossover of one layer call
// against the grouped path.  f32_in: the grouped path's expert input is f32
// (two f16 planes on the matrix cores), which moves the crossover up.
constexpr int decode_switch_t(int rbits, int rgroup, bool f32_in) {
  return rgroup == 32 ? 6 : rgroup == Q4K ? 16 : rbits == 8 ? 12 : f32_in ? 18 : 13;
}
constexpr int Q4K_REC = 16;
__host__ __device__ constexpr int q4k_superblocks(int k) { return (k + Q4K_SB - 1) / Q4K_SB; }
__host__ __device__ constexpr size_t q4k_rec_bytes(int inter) {   // gate + up records
  return (size_t)Q4K_REC * 2 * (size_t)inter * q4k_superblocks(H);
}
__host__ __device__ constexpr size_t q4k_dd_bytes(int inter) {    // down d/dmin words
  return (size_t)4 * q4k_superblocks(inter) * H;
}
__host__ __device__ constexpr size_t q4k_meta_bytes(int inter) {
  return q4k_rec_bytes(inter) + q4k_dd_bytes(inter) + (size_t)2 * (inter / Q4K_SUB) * H;
}
// 4-byte words of one expert's scale data (f32 group scales, or two-level metadata)
__host__ __device__ constexpr size_t scale_words(int group, int inter) {
  return group == Q4K ? q4k_meta_bytes(inter) / 4 : 3 * (size_t)inter * H / group;
}

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
  void* z;             // [T][H] normalised input (written when norm): f32, or bf16 with norm_bf16
  int32_t* ids; float* w;
  float* logits;       // [T][E] scratch of the two-pass router (below 1024 tokens)
};

// Decode items: one item = 32 intermediate columns of one (token, expert):
// gate/up for those columns, then their split-K share of the down projection,
// written as a 1280-float partial.  Routed picks give I/32 = 28 items each,
// the shared expert IS/32 = 56.
constexpr int SLICE = 32;
constexpr int R_ITEMS = TOPK * (I / SLICE);       // 168
constexpr int S_ITEMS = IS / SLICE;               // 56
constexpr int N_ITEMS = R_ITEMS + S_ITEMS;        // 224 per token

// Largest per-token call whose items select their own picks.  Measured: the
// selection launch saved (one token 16.2 -> 14.1 us, four 23.7 -> 22.5 us for
// int4 G64 / int8 G128) outweighs the selection each item then runs before its
// weight loads up to 4 tokens; from 8 tokens on, with several items per CU,
// it does not (16 tokens 50.8 -> 53.5 us).
constexpr int DEC_SELF_SELECT_MAX_T = 4;
struct DecItemsArgs {
  const float* xf; const uint16_t* xb;  // layer input rows (f32 or bf16), exactly one non-null
  // [T][E] router logits: every routed item selects its own pick and each
  // token's first item writes ids / tw; null: ids / tw come from the
  // selection launch
  const float* logits;
  int32_t* ids; float* tw;              // routing [T][6]
  QW rw, sw;
  float* part;                          // [T][N_ITEMS][H]
};

struct DecReduceArgs {
  const float* part; float* y; int accumulate;
};

// Persistent decode step (one token, n_layers chained layers).
constexpr int MAX_LAYERS = 16;
constexpr int N_RED = 32;                 // reducer workgroups
constexpr int RED_ROWS = H / N_RED;       // 40 rows each
constexpr int Q_STRIDE = 68;              // 64 partial logits + sum of squares, padded
// Exchanged 16-byte words: four f32 values, the lowest mantissa bit of each
// set to the parity of the writer's stage.
constexpr int PART_U4 = RED_ROWS / 4;            // 10 words: one item's partial for one reducer
static_assert(RED_ROWS % 4 == 0, "reducer bands of whole words");
constexpr int ITEM_U4 = N_RED * PART_U4;         // 320 words per item
constexpr int REC_VALS = RED_ROWS + E + 1;       // reducer record: h rows, partial logits, sum of squares
constexpr int REC_U4 = (REC_VALS + 3) / 4;       // 27 words
struct LayerPtrs {
  const float* wr; const float* bias;
  const uint8_t* eq; const float* es;
  const uint8_t* sq; const float* ss;
};
struct ChainArgs {
  LayerPtrs layer[MAX_LAYERS];
  int n_layers;
  const void* x; int x_bf16;
  float* y;                               // residual stream / output [H]
  int norm, accumulate;
  float eps;
  int rbits, rgroup, sbits, sgroup;
  int32_t* ids; float* tw;                // [n_layers][6]
  uint32_t* hdr;                          // [0] stage counter (tags of a call are hdr[0] + 1 ..), [1] done count, [2] error
  uint32_t* ipart;                        // [N_ITEMS][N_RED][PART_U4] parity words (16 B each)
  uint32_t* rec;                          // [N_RED][REC_U4] parity words
#ifdef MOE_DEVICE_TRACE
  unsigned long long* trace;              // [256][16][16] timestamps (timeline studies only)
#endif
};

struct HistArgs {
  const int32_t* ids; int T;
  int32_t* counts; int32_t* offsets;    // [E], [E+1]
  int32_t* perm; int32_t* pos_of;       // [T*6]: sorted slot -> (t*6+j); (t*6+j) -> sorted position
  int32_t* tiles; int32_t* ntiles;      // [max][4] (expert, first row, first sorted slot, rows), count
  int mt;                               // rows per tile
  int32_t* blkcnt;                      // [blocks][E] per-block counts (the multi-workgroup histogram)
};
constexpr int HIST_BLOCK = 1024;        // slots per workgroup of the multi-workgroup histogram
constexpr int HIST_ONE_WG_MAX = 4096;   // slots up to which one workgroup does it all

struct GroupedArgs {
  // A rows
  const float* af; const uint16_t* ab;  // f32 or bf16 rows, row stride = K
  int T;
  int shared;                           // 1: rows are tokens 0..T-1 of the shared expert
  const int32_t* tiles; const int32_t* ntiles; const int32_t* offsets; const int32_t* perm;
  int a_by_token;                       // routed A rows: 1 = token rows (gate/up), 0 = sorted rows (down)
  int a_rows;                           // rows of the A matrix (bounds its buffer descriptor)
  QW w;
  float* out;                           // routed: [T*6][N] by sorted position; shared: [T][N]
  int ksplit;                           // down of the shared expert: 2 = two K halves, half k to out + k T H
};

struct CombineArgs {
  const float* ys; const float* ys2;    // shared expert output (ys2: second K half, or null)
  const float* ysorted; const int32_t* pos_of; const float* tw;
  float* y; int T; int accumulate;
};

// Dense ends of the decoder for a few tokens (lm_head + greedy token, the
// layer-0 SwiGLU MLP): GEMVs over row-major weights.
constexpr int DENSE_MAX_T = 4;
constexpr int DENSE_MAX_INTER = 8192;
constexpr int HEAD_STEPS = 16;                // wave steps of 4 rows
constexpr int HEAD_ROWS = 4 * 4 * HEAD_STEPS; // rows per workgroup (256)
constexpr int DENSE_GU_STEPS = 2;
struct HeadArgs {
  const float* h; int T; int norm; float eps;   // [T][H]
  const void* w; const float* s; int group;     // [vocab][H] bf16 or int8 (+ [vocab][H/group] scales)
  int vocab;
  float* logits;                                // [T][vocab] or null
  float* cand;                                  // [T][workgroups][2]: best logit, its id (int bits)
  int32_t* token; float* token_logit;           // [T]
};
struct DenseGateUpArgs {
  const float* x; int T; int norm; float eps;   // [T][H]
  const uint8_t* q; const float* s;             // gate [inter][H] then up [inter][H]; scales likewise
  int bits, group, inter;
  float* hmid;                                  // [T][inter]
};
struct DenseDownArgs {
  const float* hmid; int T;
  const uint8_t* q; const float* s;             // down [H][inter]; scales [H][inter/group]
  int bits, group, inter;
  float* y; int accumulate;                     // [T][H]
};
int head_workgroups(int vocab);
hipError_t launch_head(const HeadArgs& a, bool bf16, hipStream_t s);
hipError_t launch_dense(const DenseGateUpArgs& g, const DenseDownArgs& d, hipStream_t s);

// One R-SWA attention decode step for S independent streams.
constexpr int ATT_HEADS = 10, ATT_D = 128;
constexpr int RSWA_W = 128;                   // ring slots of generated tokens
constexpr int RSWA_CHUNK = 64;                // keys per split-KV workgroup
constexpr int RSWA_PART = 132;                // floats per partial: m, l, 128 outputs, pad
constexpr int RSWA_ROW_MIN_WG = 160;          // (stream, head) pairs from which one workgroup takes a whole row
constexpr int RSWA_ROW_THREADS = 128;         // ... of this many threads (chunks of a quarter as many keys)
struct RswaArgs {
  int S, n_ref, n_chunks; float scale;
  const float* q; const float* k_new; const float* v_new;   // [S][10][128]
  const uint16_t* ref_k; const uint16_t* ref_v;             // [S][10][n_ref][128] bf16
  uint16_t* ring_k; uint16_t* ring_v;                       // [S][10][128][128] bf16
  const int32_t* n_gen;                                     // [S]
  float* part;                                              // [S][10][n_chunks][RSWA_PART]
  float* out;                                               // [S][10][128]
  uint16_t* out_hl = nullptr;   // if set, the output goes here instead, as bf16 halves (split_row layout)
};
int rswa_chunks(int n_ref);
hipError_t launch_rswa(const RswaArgs& a, hipStream_t s);

// Attention projections: y[t][n] (+)= sum_k a[t][k] W[n][k], K = H, bf16 W
// [N][H]; output column n of token t at y[((n / H) * T + t) * H + n % H]
// (so q, k and v of a [3H][H] weight land in three [T][H] arrays).
// The activations come already split into bf16 halves (a_hl, the split_row
// layout below).
struct ProjArgs {
  const uint16_t* a_hl; const uint16_t* w; float* y;
  int T, N, accumulate;
  // instead of a_hl: the f32 rows h, whose RMSNorm (eps) the projection forms
  // itself in split_row layout in LDS (T <= PJ_NORM_MAX_T)
  const float* h_norm = nullptr; float eps = 0.f;
};
constexpr int PJ_NORM_MAX_T = 4;
// split_row layout of an f32 row [H] as bf16 halves: per 8-element group g,
// 16 bytes of hi = bf16_rne(x) for its 8 elements, then 16 bytes of
// lo = bf16_rne(x - hi); 4 bytes per element, like the f32 row.
hipError_t launch_proj(const ProjArgs& p, hipStream_t s);

// Router launches.  select = false (below 1024 tokens only): the logits pass
// alone, for the per-token path, whose items select their picks themselves.
hipError_t launch_router(const RouterArgs& a, hipStream_t s, bool select = true);
hipError_t launch_dec_items(const DecItemsArgs& a, int T, hipStream_t s);
hipError_t launch_dec_reduce(const DecReduceArgs& a, int T, hipStream_t s);
hipError_t launch_chain(const ChainArgs& a, hipStream_t s);
hipError_t launch_zero_words(uint32_t* p, size_t n, hipStream_t s);
// device address of the current GPU's copy of the workspace-free entry
// point's scratch array (STATIC_SCRATCH_BYTES, 256-byte aligned)
hipError_t static_scratch(void** out);
hipError_t launch_hist(const HistArgs& a, hipStream_t s);
hipError_t launch_grouped_gateup(const GroupedArgs& a, int max_tiles, bool small, hipStream_t s);
hipError_t launch_grouped_down(const GroupedArgs& a, int max_tiles, bool small, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
// Grouped gate/up (down = false) or down GEMMs of a two-level expert set (32-row tiles).
hipError_t launch_grouped_q4k(const GroupedArgs& a, int max_tiles, bool down, hipStream_t s);
// Routed and shared small-tile GEMMs in one launch (gate/up, or down with the
// shared expert in two K halves); false if the format pair has no fused kernel.
bool small_pair_available(int rbits, int rgroup, int sbits, int sgroup);
bool launch_small_pair(const GroupedArgs& r, int r_tiles, const GroupedArgs& sh, int s_tiles, bool down, int mtl,
                       hipStream_t s);
// z_mode: 0 f32, 1 bf16, 2 split_row bf16 halves
hipError_t launch_rmsnorm(const float* h, void* z, int z_mode, int T, float eps, hipStream_t s);

}  // namespace moe
