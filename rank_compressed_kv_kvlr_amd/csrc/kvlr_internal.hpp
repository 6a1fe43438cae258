// Internal declarations of libkvlr: kernel parameter blocks, launchers and
// small device helpers shared by the gfx950 kernels. Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvlr.h"

namespace kvlr {

constexpr int kMaxKvHeads = 64;   // per-head tables travel in the kernel argument block
constexpr int kMaxRank = 128;     // rank bound of the decode kernels' register tiles
constexpr int kHeadsPerWg = 4;    // query heads sharing one KV head handled by one workgroup
constexpr int kTile = 64;         // tokens per wave iteration of the fp32 decode kernel; splits are multiples of it
constexpr int kWaves = 4;         // waves per decode workgroup
constexpr int kApportionPairs = 512;   // balanced plan, one segment per workgroup: at most this many (row, KV head) pairs

// Per-KV-head tables: ranks and prefix sums of ranks (latent and basis offsets).
struct HeadTable {
  int rk[kMaxKvHeads];
  int rv[kMaxKvHeads];
  int rk_pre[kMaxKvHeads];
  int rv_pre[kMaxKvHeads];
  int split_len[kMaxKvHeads];   // decode: tokens per split of KV head h (splits past the sequence are empty)
  int cost[kMaxKvHeads];        // decode, balanced plan: work per token of KV head h (a fixed part + r_k + r_v)
  int cost_pre[kMaxKvHeads];    // decode, balanced plan: sum of cost[h'] over KV heads h' < h
  int sk_pre[kMaxKvHeads];      // prefix sums of per-row storage (elements; bytes for 4/3-bit rows)
  int sv_pre[kMaxKvHeads];
};

struct DecodeParams {
  const float* q;        // [B][Hq][d]
  const float* qt_in;    // optional q~ [B][Hq][qt_stride] (bases folded into the query projection)
  int qt_stride;
  float* qt_out;         // query projection kernel: destination of q~ [B][Hq][qt_stride]
  const float* pk;       // packed [h][d][rk(h)]
  const void* lat_k;     // latent caches
  const void* lat_v;
  const int* seq_lens;   // [B]
  float* ws;             // partial records [B][Hq][n_splits][ws_stride]
  int* counters;         // arrival counters [B][Hkv][n_head_groups] (single-launch merge)
  const float* pv;       // single-launch merge: packed [h][d][rv(h)]
  float* out;            // single-launch merge: [B][Hq][d]
  int fuse;              // 1: the last split workgroup of a group merges and back-projects
  int balanced;          // bf16 latents: balanced plan, n_wg workgroups with equal shares of the work
  int apportion;         // balanced plan: one segment per workgroup (see decode_balanced)
  int n_wg;
  int row_cost;          // balanced plan: n_head_groups * sum_h cost[h], work per token of a batch row
  int out_latent;        // 1: write the normalised latent output o_lat [B][Hq][out_stride] (no P_V^T)
  int out_stride;
  int B, Hq, Hkv, G, d, cap;
  int split_len, n_splits, ws_stride, n_head_groups;
  int Rk, Rv;            // sum of ranks over heads
  int Sk, Sv;            // per-row storage summed over heads (elements; bytes for 4/3-bit rows)
  float scale_log2;      // scale * log2(e): scores live in the base-2 domain
  // fused append (bf16 per-head caches): the new rows k_new, v_new [B][Hkv][d] (in_bf16
  // says their dtype) are written at row pos[b] of app_k / app_v (the caches, writable)
  // by the workgroups whose split holds that row, before they read it
  void* app_k;
  void* app_v;
  const void* k_new;
  const void* v_new;
  const int* pos;
  int in_bf16;
  HeadTable ht;
};

struct MergeParams {
  const float* ws;
  const float* pv;       // packed [h][d][rv(h)]
  float* out;            // [B][Hq][d], or [B][Hq][out_stride] latent rows when out_latent
  int out_latent, out_stride;
  int B, Hq, Hkv, G, d;
  int n_splits, ws_stride, n_head_groups;
  HeadTable ht;
};

struct CompressParams {
  const void* x_k;       // [B][n_tok][Hkv][d] in_dtype (keys)
  const void* x_v;       // values
  const float* pk;
  const float* pv;
  void* lat_k;
  void* lat_v;
  int B, Hkv, d, cap, start, n_tok;
  int Rk, Rv;
  int Sk, Sv;
  int in_bf16, out_bf16, out_q43;
  int only_kind;         // -1: keys and values (grid.y = 2 Hkv); 0 or 1: that kind only (grid.y = Hkv)
  int joint_v;           // values: one latent per token from all heads (grid.y = 1 for the value launch)
  int n_cu;              // compute units of the device (the MFMA kernel's schedule fills them)
  // MFMA kernel schedule (set by the launcher): per batch row, segment s (values of head
  // s for s < Hkv, keys of head s - Hkv) has sched_pre[s + 1] - sched_pre[s] workgroups
  // of sched_chunk[s] tokens; sched_row workgroups per batch row.
  int sched_row;
  int sched_pre[2 * kMaxKvHeads + 1];
  int sched_chunk[2 * kMaxKvHeads];
  HeadTable ht;
};

struct AppendParams {
  const void* k_new;     // [B][Hkv][d]
  const void* v_new;
  const int* pos;        // [B]
  const float* pk;
  const float* pv;
  void* lat_k;
  void* lat_v;
  int B, Hkv, d, cap;
  int Rk, Rv;
  int Sk, Sv;
  int in_bf16, out_bf16, out_q43;
  int joint_v;           // values: one latent per token from all heads, written by the h == 0 workgroup
  HeadTable ht;
};

// Rows allocated per (batch row, KV head) block: the capacity rounded up to
// whole 16-row MFMA blocks (whole 32-row tiles for 4/3-bit latents).
__host__ __device__ inline int cap_rows_of(int cap) { return (cap + 15) & ~15; }
__host__ __device__ inline int cap_rows_q43(int cap) { return (cap + 31) & ~31; }

// Offset (elements) of bf16 joint value latent (t, j) inside its batch row's
// block (joint rank r, a multiple of 16). Each 16-row block holds the rows in
// the order the value MFMA (v_mfma_f32_16x16x16_bf16, tokens as K) reads its
// B operand: for every 32-channel pair, lane n + 16 q holds tokens 4 q .. 4 q + 3
// of channel n, then the same tokens of channel n + 16 (16 contiguous bytes);
// a 16-channel tail holds the tokens of channel n alone (8 bytes per lane).
__host__ __device__ inline size_t v_joint_offset(int t, int j, int r) {
  const size_t base = (size_t)(t >> 4) * 16 * r;
  const int q = (t & 15) >> 2, e = t & 3, np = r >> 5;
  if (j < 32 * np) return base + (size_t)(j >> 5) * 512 + q * 128 + (j & 15) * 8 + ((j >> 4) & 1) * 4 + e;
  return base + (size_t)np * 512 + q * 64 + (j - 32 * np) * 4 + e;
}

// Offset (elements) of bf16 key latent (t, j) inside its (batch row, KV head)
// block, rank rk (a multiple of 16). Each 16-row block holds the rows in the
// order the score MFMA reads its key operand (lane n + 16 q: token n, channels
// 8 q .. 8 q + 7 of a pair; the A operand of the transposed score product):
// for every 32-channel pair
// [lane group q][token n][8 channels], then a 16-channel tail as
// [q][n][4 channels]; a 64-lane load then reads 1 KiB (512 B for the tail)
// contiguously.
__host__ __device__ inline size_t k_tiled_offset(int t, int j, int rk) {
  const size_t base = (size_t)(t >> 4) * 16 * rk;
  const int n = t & 15, np = rk >> 5;
  if (j < 32 * np) return base + (size_t)(j >> 5) * 512 + ((j >> 3) & 3) * 128 + n * 8 + (j & 7);
  const int jj = j - 32 * np;
  return base + (size_t)np * 512 + (jj >> 2) * 64 + n * 4 + (jj & 3);
}

// Mixed 4/3-bit latents (STAR-KV technical summary, "Metodologia" section 3):
// channels in the 4-bit outlier block (20% of r in whole 16-channel blocks) and
// bytes per stored token: 4 half-float block parameters, n_o 4-bit and
// r - n_o 3-bit codes. Tokens are stored in tiles of 32 (layout in kvlr.h).
__host__ __device__ constexpr int q43_outlier(int r) {
  const int n = (r + 40) / 80;
  return 16 * (n > 1 ? n : 1);
}
__host__ __device__ constexpr int q43_row_bytes(int r) {
  return 8 + q43_outlier(r) / 2 + 3 * (r - q43_outlier(r)) / 8;
}
constexpr int kQ43Tile = 32;            // tokens per 4/3-bit tile
constexpr int kQ43MetaBytes = 256;      // block parameters of a tile: [4 slot groups][4 params][8 slots] fp16
constexpr int kQ43OutGroupBytes = 256;  // one 16-channel 4-bit group of a tile
constexpr int kQ43InGroupBytes = 192;   // one 16-channel 3-bit group of a tile
__host__ __device__ inline int q43_slot(int u) { return 8 * ((u & 15) >> 2) + 4 * (u >> 4) + (u & 3); }

// Launchers (return hipGetLastError() of their launches).
hipError_t launch_decode(const DecodeParams& p, int latent_dtype, int rank_bound, int tile, hipStream_t s);
hipError_t launch_hadamard(const float* in, float* out, size_t n_groups, hipStream_t s);
hipError_t launch_merge(const MergeParams& p, int rank_bound, hipStream_t s);
// Joint bf16 values: q~ into p.qt_out, the split kernel (q~ from p.qt_in, key rank
// bound rk_bound, `blocks` 16-token blocks per wave step: 1 or 2), and the merge
// with one workgroup per (query head, batch row).
hipError_t launch_project_queries(const DecodeParams& p, int rk_bound, hipStream_t s);
hipError_t launch_decode_joint(const DecodeParams& p, int rk_bound, int blocks, hipStream_t s);
hipError_t launch_merge_heads(const MergeParams& p, hipStream_t s);
hipError_t launch_compress(const CompressParams& p, hipStream_t s);
hipError_t launch_append(const AppendParams& p, hipStream_t s);

// ------------------------------------------------------------------------
// device helpers
// ------------------------------------------------------------------------
typedef short bf16x8_t __attribute__((ext_vector_type(8)));
typedef short bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Streaming (non-temporal) loads for data read exactly once per call.
__device__ __forceinline__ u32x4_t load_stream16(const void* ptr) {
  return __builtin_nontemporal_load(static_cast<const u32x4_t*>(ptr));
}
__device__ __forceinline__ u32x2_t load_stream8(const void* ptr) {
  return __builtin_nontemporal_load(static_cast<const u32x2_t*>(ptr));
}

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 h = static_cast<__bf16>(x);
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float half_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// All-reduce over the 16 lanes of a DPP row (max or sum) with row rotations
// and quad permutations; every lane of the row ends with the result.
template <bool kMax>
__device__ __forceinline__ float row16_allreduce(float x) {
  float y;
  y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));  // row_ror:8
  x = kMax ? fmaxf(x, y) : x + y;
  y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xf, 0xf, false));  // row_ror:4
  x = kMax ? fmaxf(x, y) : x + y;
  y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4e, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
  x = kMax ? fmaxf(x, y) : x + y;
  y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xb1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
  x = kMax ? fmaxf(x, y) : x + y;
  return x;
}

// Reductions over the lanes n, n + 16, n + 32, n + 48 (the four 16-lane rows of a wave)
// with gfx950's row swaps: after swapping rows 1 <-> 0 and 3 <-> 2 of two copies of x,
// the two results hold, lane by lane, x and its partner 16 lanes away; likewise for the
// 32-lane halves.
__device__ __forceinline__ float max_over_rows(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_over_rows(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// All-reduce over the 64 lanes of a wave (butterfly through ds_swizzle/bpermute).
template <bool kMax>
__device__ __forceinline__ float wave_allreduce(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float y = __shfl_xor(x, off, 64);
    x = kMax ? fmaxf(x, y) : x + y;
  }
  return x;
}

__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace kvlr
