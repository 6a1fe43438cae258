// Latent storage of keys and values (gfx950): prefill compression and
// single-token append.
//
// Method (StiefAttention technical summary, "Mecanismo Central" item 5):
// during inference keys are stored compressed as K P_K (values as V P_V);
// the cache grows by one row per decoded token ("Definição do Problema").
//
// Prefill with bf16 inputs is a dense contraction [n_tok x d] . [d x r] per
// (batch row, KV head) and runs on MFMA (v_mfma_f32_16x16x32_bf16) with the
// roles swapped so that each lane ends with 4 consecutive latent channels of
// one token (one 8-byte store): A = P^T (latent channels as rows), B = the
// token rows (16 tokens as columns, 16 contiguous input bytes per lane).
// The fp32 basis enters as a high and a low bf16 part (two MFMAs into one
// fp32 accumulator), so products carry ~16 bits of the basis and the only
// rounding of note is the final one to the latent dtype. The basis operands
// are staged once per workgroup in LDS, pre-arranged in operand order.
// bf16 value latents take the product the other way round (A = the token
// rows), so that each lane ends with 4 consecutive tokens of one latent
// channel: the decode kernels' value-product operand order, stored as one
// 8-byte piece.
// A workgroup owns one token range of one (batch row, KV head, kind); the
// host sizes the ranges by bytes per token so that workgroups carry about the
// same work, about eight rounds of resident workgroups in all. Each wave keeps
// the next 64-row tile in flight (buffer loads) while it multiplies the
// current one, and stores through a buffer resource with wave-uniform offsets.
//
// fp32 inputs, ranks that are not whole 16-channel tiles and joint value latents
// use a plain VALU kernel, 4/3-bit latents a VALU kernel of their own
// (compress_q43); append uses one workgroup per (batch row, KV head, K or V).
//
// Mixed 4/3-bit latents (STAR-KV technical summary, "Metodologia" section 3)
// are quantised from the fp32 latents of a row by one thread per row; the
// block-wise Hadamard rotation is already folded into the bases it receives
// (hadamard_fold below, run once per set of bases).
#include <algorithm>
#include <cmath>

#include "kvlr_internal.hpp"

namespace kvlr {
namespace {

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));   // one v_cvt_pk_bf16_f32 per pair

// ---- 4/3-bit rows --------------------------------------------------------
__device__ __forceinline__ uint32_t half_bits(_Float16 h) { return (uint32_t)__builtin_bit_cast(uint16_t, h); }

// Step, base and 1/step of one block of x[c0, c1) (fp32, in the order of the
// layout comment in kvlr.h); meta = step | base << 16 as half floats. A zero
// step gives inv = 0 and therefore code 0 everywhere.
__device__ __forceinline__ void q43_block_params(const float* x, int c0, int c1, float levels, float& base,
                                                 float& inv, uint32_t& meta) {
  float lo = x[c0], hi = x[c0];
  for (int c = c0 + 1; c < c1; ++c) {
    lo = fminf(lo, x[c]);
    hi = fmaxf(hi, x[c]);
  }
  const _Float16 s16 = (_Float16)((hi - lo) / levels);
  const _Float16 b16 = (_Float16)lo;
  const float step = (float)s16;
  base = (float)b16;
  inv = step != 0.f ? 1.f / step : 0.f;
  meta = half_bits(s16) | (half_bits(b16) << 16);
}

__device__ __forceinline__ uint32_t q43_code(float x, float base, float inv, float levels) {
  const float t = rintf((x - base) * inv);
  return (uint32_t)fminf(fmaxf(t, 0.f), levels);
}

// Quantise one row of r fp32 latents x[] into codes[] (one byte per channel) and its
// 4 block parameters (half-float bits: outlier step, minimum, inlier step, minimum).
__device__ void q43_quantise_row(const float* x, int r, uint8_t* codes, uint16_t* prm) {
  const int no = q43_outlier(r);
  float base, inv;
  uint32_t meta;
  q43_block_params(x, 0, no, 15.f, base, inv, meta);
  prm[0] = (uint16_t)(meta & 0xFFFFu);
  prm[1] = (uint16_t)(meta >> 16);
  for (int c = 0; c < no; ++c) codes[c] = (uint8_t)q43_code(x[c], base, inv, 15.f);
  if (r > no) {
    q43_block_params(x, no, r, 7.f, base, inv, meta);
    for (int c = no; c < r; ++c) codes[c] = (uint8_t)q43_code(x[c], base, inv, 7.f);
  } else {
    meta = 0;
  }
  prm[2] = (uint16_t)(meta & 0xFFFFu);
  prm[3] = (uint16_t)(meta >> 16);
}

// Tile layout (kvlr.h): what (block, n, kq, i) of a lane position means, as
// (token in the tile, channel in the 16-channel group).
__device__ __forceinline__ int q43_token(int kind, int n, int kq, int blk, int i) {
  return kind == 0 ? 16 * blk + n : 16 * blk + 4 * kq + i;
}
__device__ __forceinline__ int q43_channel(int kind, int n, int kq, int i) { return kind == 0 ? 4 * kq + i : n; }
// (block, i) of position e of a 24-bit 3-bit field, and the inverse
__device__ __forceinline__ int q43_field_blk(int e) { return (e >> 1) & 1; }
__device__ __forceinline__ int q43_field_i(int e) { return 2 * (e & 1) + (e >> 2); }
__device__ __forceinline__ int q43_field_pos(int blk, int i) { return 2 * blk + (i >> 1) + 4 * (i & 1); }

// Byte offset in a tile and bit shift of code (token u, channel c), rank r.
__device__ __forceinline__ void q43_code_pos(int kind, int u, int c, int r, int& byte, int& shift) {
  const int no = q43_outlier(r);
  const int blk = u >> 4;
  const bool four = c < no;
  const int g = four ? c >> 4 : (c - no) >> 4, cc = four ? c & 15 : (c - no) & 15;
  int n, kq, i;
  if (kind == 0) {
    n = u & 15;
    kq = cc >> 2;
    i = cc & 3;
  } else {
    n = cc;
    kq = (u & 15) >> 2;
    i = u & 3;
  }
  const int w = n + 16 * kq;
  if (four) {
    byte = kQ43MetaBytes + kQ43OutGroupBytes * g + 4 * w + i;
    shift = 4 * blk;
  } else {
    byte = kQ43MetaBytes + kQ43OutGroupBytes * (no >> 4) + kQ43InGroupBytes * g + 3 * w;
    shift = 3 * q43_field_pos(blk, i);
  }
}

// Block-wise Hadamard fold: every run of 16 floats becomes x H16 / 4 (a fast
// Walsh-Hadamard transform in registers; in place is safe).
__global__ __launch_bounds__(256) void hadamard_fold(const float* __restrict__ in, float* __restrict__ out,
                                                     size_t n_groups) {
  const size_t g = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= n_groups) return;
  float v[16];
  const float4* src = reinterpret_cast<const float4*>(in + 16 * g);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float4 f = src[k];
    v[4 * k] = f.x;
    v[4 * k + 1] = f.y;
    v[4 * k + 2] = f.z;
    v[4 * k + 3] = f.w;
  }
#pragma unroll
  for (int len = 1; len < 16; len <<= 1)
#pragma unroll
    for (int i = 0; i < 16; i += 2 * len)
#pragma unroll
      for (int j = 0; j < len; ++j) {
        const float a = v[i + j], c = v[i + j + len];
        v[i + j] = a + c;
        v[i + j + len] = a - c;
      }
  float4* dst = reinterpret_cast<float4*>(out + 16 * g);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    dst[k] = make_float4(0.25f * v[4 * k], 0.25f * v[4 * k + 1], 0.25f * v[4 * k + 2], 0.25f * v[4 * k + 3]);
}

constexpr int kCompressWaves = 4;
constexpr int kTokensPerWave = 64;        // 4 MFMA column tiles of 16 tokens
constexpr int kCompressGroup = kCompressWaves * kTokensPerWave;   // 256: token ranges are multiples of this
constexpr int kCompressRounds = 8;        // workgroups per resident slot in the schedule

// One wave's 64 input rows: lane (n16, q4) holds channels 32 kb + 8 q4 + [0, 8) of
// token tw0 + 16 nt + n16. Four lanes read 64 contiguous bytes of a row, so two loads
// complete a 128-byte line. The buffer resource covers the workgroup's rows only:
// rows past its end read as zeros without a memory access (their results are not
// stored). The rows are read once: non-temporal loads.
template <int NKB>
__device__ __forceinline__ void compress_load(u32x4_t (&x)[4][NKB], __amdgpu_buffer_rsrc_t rs, int row_bytes, int u0,
                                              int n16, int q4) {
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    // unsigned: offsets of rows past the range may pass 2^31 (they read nothing)
    const uint32_t off = (uint32_t)(u0 + 16 * nt + n16) * (uint32_t)row_bytes + 16u * q4;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      x[nt][kb] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(off + 64u * kb), 0, 2));
  }
}

// Where a workgroup's whole tiles store their latents: a buffer resource from the
// 16-row block (bf16 layouts) or the row (fp32) of its first token, and each lane's
// byte offset in it, for the paired 32-channel part and for a trailing 16-channel
// tile (bf16 layouts of ranks that are odd multiples of 16). The rest of an offset is
// wave-uniform: the tile, the 16-row block and the channel tile (see compress_tile).
struct LatentStoreMap {
  __amdgpu_buffer_rsrc_t rs;
  int lane_pair;
  int lane_tail;
};

template <int KIND, bool kOutBf16>
__device__ __forceinline__ LatentStoreMap latent_store_map(const CompressParams& p, void* lat, size_t lat_base,
                                                           int r, int t0, int t1, int lane) {
  const int n16 = lane & 15, q4 = lane >> 4;
  LatentStoreMap m;
  if (!kOutBf16) {   // [row][r] fp32: lane holds channels 4 q4 .. of token n16
    m.rs = __builtin_amdgcn_make_buffer_rsrc(static_cast<float*>(lat) + lat_base + (size_t)(p.start + t0) * r, (short)0,
                                             (t1 - t0) * r * 4, 0x00020000);
    m.lane_pair = m.lane_tail = 4 * (n16 * r + 4 * q4);
    return m;
  }
  const int r16 = 16 * r;   // elements of a 16-row block
  m.rs = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<uint16_t*>(lat) + lat_base + (size_t)((p.start >> 4) + (t0 >> 4)) * r16, (short)0,
      ((t1 - t0) / 16 + 2) * r16 * 2, 0x00020000);
  const int s15 = p.start & 15;
  if (KIND == 0) {   // keys: lane holds 4 channels of token n16 (row (start + n16) mod 16 of its block)
    const int bl = (s15 + n16) >> 4, n = (s15 + n16) & 15;
    m.lane_pair = 2 * (bl * r16 + (q4 >> 1) * 128 + n * 8 + 4 * (q4 & 1));
    m.lane_tail = 2 * (bl * r16 + q4 * 64 + n * 4);
  } else {           // values: lane holds tokens 4 q4 .. 4 q4 + 3 of channel n16 (start is a multiple of 4)
    const int bl = (s15 + 4 * q4) >> 4, q = ((s15 + 4 * q4) & 15) >> 2;
    m.lane_pair = 2 * (bl * r16 + q * 128 + n16 * 8);
    m.lane_tail = 2 * (bl * r16 + q * 64 + n16 * 4);
  }
  return m;
}

// Latents of one wave's 64 rows, 16 channels (one A tile) at a time, stored as they
// are formed. WHOLE: every row is below t_end and (value latents) the first row is a
// multiple of 4, so every store is a whole piece; those go through the store map with
// wave-uniform offsets, the others element by element.
template <int KIND, bool kOutBf16, int NKB, bool WHOLE>
__device__ __forceinline__ void compress_tile(const CompressParams& p, const u32x4_t (&xin)[4][NKB],
                                              const uint4* st_hi, const uint4* st_lo, int n_mt, int r, int tw0,
                                              int t0, int t_end, void* lat, size_t lat_base,
                                              const LatentStoreMap& sm, int lane) {
  const int n16 = lane & 15, q4 = lane >> 4;
  // The rows pass through an empty asm statement, so that the wait for them comes here,
  // counted exactly (the next tile's loads and earlier stores stay in flight), and not
  // as a wait for every outstanding access before the channel-tile loop.
  u32x4_t x[4][NKB];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      x[nt][kb] = xin[nt][kb];
      asm volatile("" : "+v"(x[nt][kb]));
    }
  constexpr bool v_tiled = kOutBf16 && KIND == 1;   // bf16 values: value-product operand order
  constexpr bool k_tiled = kOutBf16 && KIND == 0;   // bf16 keys: MFMA operand order
  const int np = r >> 5;                            // paired 32-channel groups of the bf16 layouts
  const int blk0 = (tw0 - t0) >> 4;                 // 16-row block of the tile in the store map
  for (int mt = 0; mt < n_mt; ++mt) {
    f32x4_t acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int e = (mt * NKB + kb) * 64 + lane;
      const bf16x8_t ahi = __builtin_bit_cast(bf16x8_t, st_hi[e]);
      const bf16x8_t alo = __builtin_bit_cast(bf16x8_t, st_lo[e]);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const bf16x8_t xb = __builtin_bit_cast(bf16x8_t, x[nt][kb]);
        if (v_tiled) {   // transposed product: lane ends with 4 consecutive tokens of one channel
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb, ahi, acc[nt], 0, 0, 0);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb, alo, acc[nt], 0, 0, 0);
        } else {
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, xb, acc[nt], 0, 0, 0);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, xb, acc[nt], 0, 0, 0);
        }
      }
    }
    if (WHOLE) {
      // byte offset = lane part + tile/block part + channel-tile part (wave-uniform)
      const bool tail = kOutBf16 && mt >= 2 * np;
      const int lane_off = tail ? sm.lane_tail : sm.lane_pair;
      int uni;   // bytes, for nt = 0
      if (!kOutBf16)
        uni = 4 * ((tw0 - t0) * r + 16 * mt);
      else if (k_tiled)
        uni = 2 * (blk0 * 16 * r + 256 * mt);
      else
        uni = 2 * (blk0 * 16 * r + (tail ? 512 * np : (mt >> 1) * 512 + (mt & 1) * 4));
      const int nt_step = kOutBf16 ? 2 * 16 * r : 4 * 16 * r;   // 16 rows further
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int soff = __builtin_amdgcn_readfirstlane(uni + nt * nt_step);
        if (kOutBf16) {
          const bf16x2_t lo2 = __builtin_convertvector((f32x2_t){acc[nt][0], acc[nt][1]}, bf16x2_t);
          const bf16x2_t hi2 = __builtin_convertvector((f32x2_t){acc[nt][2], acc[nt][3]}, bf16x2_t);
          const u32x2_t v = {__builtin_bit_cast(uint32_t, lo2), __builtin_bit_cast(uint32_t, hi2)};
          __builtin_amdgcn_raw_buffer_store_b64(v, sm.rs, lane_off, soff, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc[nt]), sm.rs, lane_off, soff, 0);
        }
      }
      continue;
    }
    if (v_tiled) {
      // lane holds tokens tw0 + 16nt + 4q4 + i (i < 4) of latent channel 16mt + n16
      uint16_t* V = static_cast<uint16_t*>(lat) + lat_base;
      const int j = 16 * mt + n16;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int t = tw0 + 16 * nt + 4 * q4;
        const int row = p.start + t;
        if (t + 3 < t_end && (row & 3) == 0) {
          const uint32_t w0 = (uint32_t)f32_to_bf16_bits(acc[nt][0]) | ((uint32_t)f32_to_bf16_bits(acc[nt][1]) << 16);
          const uint32_t w1 = (uint32_t)f32_to_bf16_bits(acc[nt][2]) | ((uint32_t)f32_to_bf16_bits(acc[nt][3]) << 16);
          *reinterpret_cast<uint2*>(V + v_joint_offset(row, j, r)) = make_uint2(w0, w1);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (t + i < t_end) V[v_joint_offset(row + i, j, r)] = f32_to_bf16_bits(acc[nt][i]);
        }
      }
      continue;
    }
    // lane holds latent channels 16mt + 4q4 + i (i < 4) of token tw0 + 16nt + n16
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int t = tw0 + 16 * nt + n16;
      if (t < t_end) {
        const int j0 = 16 * mt + 4 * q4;   // 4 consecutive channels stay contiguous in both layouts
        const size_t off = lat_base + (k_tiled ? k_tiled_offset(p.start + t, j0, r) : (size_t)(p.start + t) * r + j0);
        if (kOutBf16) {
          const uint32_t w0 = (uint32_t)f32_to_bf16_bits(acc[nt][0]) | ((uint32_t)f32_to_bf16_bits(acc[nt][1]) << 16);
          const uint32_t w1 = (uint32_t)f32_to_bf16_bits(acc[nt][2]) | ((uint32_t)f32_to_bf16_bits(acc[nt][3]) << 16);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(lat) + off) = make_uint2(w0, w1);
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(lat) + off) =
              make_float4(acc[nt][0], acc[nt][1], acc[nt][2], acc[nt][3]);
        }
      }
    }
  }
}

// Tokens [t0, t1) of one (batch row, KV head, kind): the basis is staged once, then
// wave w takes the 64-row tiles t0 + 64 (4k + w).
template <int KIND, bool kOutBf16, int NKB>
__device__ __forceinline__ void compress_range(const CompressParams& p, int h, int b, int t0, int t1, uint4* stage) {
  const int d = 32 * NKB;
  const int r = KIND ? p.ht.rv[h] : p.ht.rk[h];
  const int r_pre = KIND ? p.ht.rv_pre[h] : p.ht.rk_pre[h];
  const float* P = (KIND ? p.pv : p.pk) + (size_t)d * r_pre;
  const uint16_t* X = static_cast<const uint16_t*>(KIND ? p.x_v : p.x_k);
  void* lat = KIND ? p.lat_v : p.lat_k;
  const int n_mt = r >> 4;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: tile counts and loops stay scalar
  const int n16 = lane & 15, q4 = lane >> 4;
  const size_t row_stride = (size_t)p.Hkv * d;   // elements between consecutive tokens
  const int row_bytes = (int)(row_stride * 2);
  // rows [t0, t1) of this head (the host keeps (t1 - t0) * row_bytes below 2^31)
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(X + ((size_t)b * p.n_tok + t0) * row_stride + (size_t)h * d), (short)0,
      (t1 - t0) * row_bytes, 0x00020000);
  const size_t lat_base = (size_t)cap_rows_of(p.cap) * ((size_t)b * (KIND ? p.Sv : p.Sk) +
                                                      (KIND ? p.ht.sv_pre[h] : p.ht.sk_pre[h]));
  auto tile_u = [&](int k) { return (k * kCompressWaves + wave) * kTokensPerWave; };   // offset from t0
  const int span = t1 - t0;
  const int n_all = span > tile_u(0) ? (span - tile_u(0) + kCompressGroup - 1) / kCompressGroup : 0;
  const int n_full = span >= tile_u(0) + kTokensPerWave ? (span - tile_u(0) - kTokensPerWave) / kCompressGroup + 1 : 0;

  // the first tile's rows are in flight while the basis is staged
  u32x4_t xa[4][NKB];
  compress_load<NKB>(xa, rs, row_bytes, tile_u(0), n16, q4);

  // ---- stage P^T operands: entry (mt, kb, lane) holds P[32kb + 8(lane/16) + e][16mt + lane%16], e < 8,
  // as a high and a low bf16 part. A thread reads an 8-row x 4-column block of P (8 rows of
  // 16 bytes, consecutive threads on consecutive columns) and writes the 4 entries it holds.
  const int n_entries = n_mt * NKB * 64;
  uint4* st_hi = stage;
  uint4* st_lo = stage + n_entries;
  const int n_cq = r >> 2;              // column quads
  const int n_units = n_cq * (d >> 3);  // (8-row group, column quad) blocks
  for (int u = tid; u < n_units; u += 256) {
    const int cq = u % n_cq, kg = u / n_cq;
    float4 v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = *reinterpret_cast<const float4*>(P + (size_t)(8 * kg + e) * r + 4 * cq);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 4 * cq + i;
      const int idx = ((c >> 4) * NKB + (kg >> 2)) * 64 + (kg & 3) * 16 + (c & 15);
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float x0 = i == 0 ? v[e].x : i == 1 ? v[e].y : i == 2 ? v[e].z : v[e].w;
        const float x1 = i == 0 ? v[e + 1].x : i == 1 ? v[e + 1].y : i == 2 ? v[e + 1].z : v[e + 1].w;
        const uint16_t h0 = f32_to_bf16_bits(x0), h1 = f32_to_bf16_bits(x1);
        const uint16_t l0 = f32_to_bf16_bits(x0 - bf16_bits_to_f32(h0));
        const uint16_t l1 = f32_to_bf16_bits(x1 - bf16_bits_to_f32(h1));
        hi[e >> 1] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        lo[e >> 1] = (uint32_t)l0 | ((uint32_t)l1 << 16);
      }
      st_hi[idx] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      st_lo[idx] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
  }
  __syncthreads();

  const bool aligned = KIND == 0 || !kOutBf16 || (p.start & 3) == 0;   // whole 8-byte value pieces
  const LatentStoreMap sm = latent_store_map<KIND, kOutBf16>(p, lat, lat_base, r, t0, t1, lane);
  int k = 0;
  if (aligned && NKB <= 4) {
    // whole tiles in pairs: the next tile's rows load while the current one is multiplied
    // (head_dim <= 128: two tiles of rows fit in registers at two waves per SIMD)
    u32x4_t xb[4][NKB];
    for (; k + 1 < n_full; k += 2) {
      compress_load<NKB>(xb, rs, row_bytes, tile_u(k + 1), n16, q4);
      compress_tile<KIND, kOutBf16, NKB, true>(p, xa, st_hi, st_lo, n_mt, r, t0 + tile_u(k), t0, t1, lat, lat_base,
                                               sm, lane);
      compress_load<NKB>(xa, rs, row_bytes, tile_u(k + 2), n16, q4);
      compress_tile<KIND, kOutBf16, NKB, true>(p, xb, st_hi, st_lo, n_mt, r, t0 + tile_u(k + 1), t0, t1, lat,
                                               lat_base, sm, lane);
    }
  }
  // xa holds tile k; the rest one tile at a time
  for (; k < n_all; ++k) {
    if (aligned && k < n_full)
      compress_tile<KIND, kOutBf16, NKB, true>(p, xa, st_hi, st_lo, n_mt, r, t0 + tile_u(k), t0, t1, lat, lat_base,
                                               sm, lane);
    else
      compress_tile<KIND, kOutBf16, NKB, false>(p, xa, st_hi, st_lo, n_mt, r, t0 + tile_u(k), t0, t1, lat,
                                                lat_base, sm, lane);
    if (k + 1 < n_all) compress_load<NKB>(xa, rs, row_bytes, tile_u(k + 1), n16, q4);
  }
}

// One workgroup per token range of a (batch row, KV head, kind) segment. Per batch row
// the segments are ordered values (heads 0..Hkv-1), then keys; segment s has
// sched_pre[s + 1] - sched_pre[s] workgroups of sched_chunk[s] tokens (the host sizes
// them so that workgroups carry about the same work, about eight rounds of resident
// workgroups in all).
template <bool kOutBf16, int NKB>
__global__ __launch_bounds__(256) void compress_bf16_mfma(CompressParams p) {
  extern __shared__ __attribute__((aligned(16))) uint4 stage[];   // [mt][kb][lane] hi, then lo
  const int b = (int)blockIdx.x / p.sched_row;
  const int rem = (int)blockIdx.x - b * p.sched_row;
  int lo = 0, hi = 2 * p.Hkv;   // segment s with sched_pre[s] <= rem < sched_pre[s + 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.sched_pre[mid] <= rem) lo = mid; else hi = mid;
  }
  const int s = lo;
  const int t0 = (rem - p.sched_pre[s]) * p.sched_chunk[s];
  const int t1 = min(p.n_tok, t0 + p.sched_chunk[s]);
  if (s < p.Hkv)
    compress_range<1, kOutBf16, NKB>(p, s, b, t0, t1, stage);
  else
    compress_range<0, kOutBf16, NKB>(p, s - p.Hkv, b, t0, t1, stage);
}

// Plain VALU compression (fp32 inputs, ranks that are not whole 16-channel
// tiles, joint values): one workgroup per (64-token tile,
// KV head x {K, V}, batch row); the tile is staged in LDS as fp32 and each
// thread forms latent channels as fp32 dot products, kept in registers (at
// most 64 * 128 / 256 = 32 per thread). Joint values
// (STAR-KV technical summary, "Metodologia" section 2) sum the contributions of
// every KV head's rows, V_all P_J = sum_h V_h P_J[h d .. (h+1) d), staging one
// head's tile at a time.
constexpr int kValuTile = 64;
constexpr int kValuOuts = kValuTile * kMaxRank / 256;

__global__ __launch_bounds__(256) void compress_valu(CompressParams p) {
  extern __shared__ __attribute__((aligned(16))) float xs[];   // [64][d], then (4/3-bit rows) latents [64][r]
  const int kind = p.only_kind >= 0 ? p.only_kind : (int)(blockIdx.y & 1);
  const int h = p.only_kind >= 0 ? (int)blockIdx.y : (int)(blockIdx.y >> 1);
  const bool joint = kind == 1 && p.joint_v;
  const int b = blockIdx.z;
  const int d = p.d;
  const int r = kind ? p.ht.rv[h] : p.ht.rk[h];
  const void* X = kind ? p.x_v : p.x_k;
  const int t0 = blockIdx.x * kValuTile;
  const int nt = min(kValuTile, p.n_tok - t0);
  const size_t row_stride = (size_t)p.Hkv * d;
  float acc[kValuOuts];
#pragma unroll
  for (int k = 0; k < kValuOuts; ++k) acc[k] = 0.f;
  const int heads = joint ? p.Hkv : 1;
  for (int hs = 0; hs < heads; ++hs) {
    const int hh = joint ? hs : h;          // KV head whose input rows are staged
    if (hs > 0) __syncthreads();             // the previous head's tile is no longer read
    for (int idx = threadIdx.x; idx < nt * d; idx += blockDim.x) {
      const int t = idx / d, i = idx - t * d;
      const size_t src = ((size_t)b * p.n_tok + t0 + t) * row_stride + (size_t)hh * d + i;
      xs[idx] = p.in_bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(X)[src]) : static_cast<const float*>(X)[src];
    }
    __syncthreads();
    const float* P = (kind ? p.pv : p.pk) + (size_t)d * (kind ? p.ht.rv_pre[hh] : p.ht.rk_pre[hh]);
#pragma unroll
    for (int k = 0; k < kValuOuts; ++k) {
      const int idx = threadIdx.x + k * blockDim.x;
      if (idx < nt * r) {
        const int t = idx / r, j = idx - t * r;
        const float* x = xs + t * d;
        float a = acc[k];
        for (int i = 0; i < d; ++i) a = fmaf(x[i], P[(size_t)i * r + j], a);
        acc[k] = a;
      }
    }
  }
  const int S = kind ? p.Sv : p.Sk;
  const int s_pre = kind ? p.ht.sv_pre[h] : p.ht.sk_pre[h];
  const size_t lat_base = (size_t)cap_rows_of(p.cap) * ((size_t)b * S + s_pre);
  const bool k_tiled = p.out_bf16 && kind == 0;
  const bool v_tiled = p.out_bf16 && kind == 1;   // bf16 values: value-product operand order
#pragma unroll
  for (int k = 0; k < kValuOuts; ++k) {
    const int idx = threadIdx.x + k * blockDim.x;
    if (idx < nt * r) {
      const int t = idx / r, j = idx - t * r;
      const int row = p.start + t0 + t;
      const size_t off = lat_base + (k_tiled   ? k_tiled_offset(row, j, r)
                                     : v_tiled ? v_joint_offset(row, j, r)
                                               : (size_t)row * r + j);
      if (p.out_bf16)
        static_cast<uint16_t*>(kind ? p.lat_v : p.lat_k)[off] = f32_to_bf16_bits(acc[k]);
      else
        static_cast<float*>(kind ? p.lat_v : p.lat_k)[off] = acc[k];
    }
  }
}

// LDS of the 4/3-bit compression: the inputs [64][d] (later the codes [64][128] and
// parameters [64][4]), then the fp32 latents [64][r]; offset of the latents in floats.
__host__ __device__ constexpr int q43_lat_offset(int d) {
  return kValuTile * d > (kValuTile * kMaxRank + kValuTile * 8) / 4 ? kValuTile * d
                                                                     : (kValuTile * kMaxRank + kValuTile * 8) / 4;
}

// 4/3-bit latents (tile layout in kvlr.h): one workgroup per (64 rows starting on a
// 32-row tile, KV head x {K, V}, batch row), so that no tile is shared between
// workgroups. The chunk's rows inside [start, start + n_tok) get fp32 latents as in
// compress_valu, one thread per row quantises them (codes and block parameters into
// LDS), and one thread per 4-bit word or 24-bit field assembles it; words that also
// hold rows outside the range keep those rows' bits.
__global__ __launch_bounds__(256) void compress_q43(CompressParams p) {
  extern __shared__ __attribute__((aligned(16))) float xs[];   // [64][d], then latents [64][r]
  const int kind = p.only_kind >= 0 ? p.only_kind : (int)(blockIdx.y & 1);
  const int h = p.only_kind >= 0 ? (int)blockIdx.y : (int)(blockIdx.y >> 1);
  const bool joint = kind == 1 && p.joint_v;
  const int b = blockIdx.z;
  const int d = p.d;
  const int r = kind ? p.ht.rv[h] : p.ht.rk[h];
  const void* X = kind ? p.x_v : p.x_k;
  const int T0 = (p.start & ~(kQ43Tile - 1)) + kValuTile * (int)blockIdx.x;   // first row of the chunk
  const int lo = max(T0, p.start), hi = min(T0 + kValuTile, p.start + p.n_tok);  // rows written
  const size_t row_stride = (size_t)p.Hkv * d;
  float acc[kValuOuts];
#pragma unroll
  for (int k = 0; k < kValuOuts; ++k) acc[k] = 0.f;
  const int heads = joint ? p.Hkv : 1;
  for (int hs = 0; hs < heads; ++hs) {
    const int hh = joint ? hs : h;
    if (hs > 0) __syncthreads();
    for (int idx = threadIdx.x; idx < kValuTile * d; idx += blockDim.x) {
      const int t = idx / d, i = idx - t * d;
      const int row = T0 + t;
      float v = 0.f;
      if (row >= lo && row < hi) {
        const size_t src = ((size_t)b * p.n_tok + (row - p.start)) * row_stride + (size_t)hh * d + i;
        v = p.in_bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(X)[src]) : static_cast<const float*>(X)[src];
      }
      xs[idx] = v;
    }
    __syncthreads();
    const float* P = (kind ? p.pv : p.pk) + (size_t)d * (kind ? p.ht.rv_pre[hh] : p.ht.rk_pre[hh]);
#pragma unroll
    for (int k = 0; k < kValuOuts; ++k) {
      const int idx = threadIdx.x + k * blockDim.x;
      if (idx < kValuTile * r) {
        const int t = idx / r, j = idx - t * r;
        const float* x = xs + t * d;
        float a = acc[k];
        for (int i = 0; i < d; ++i) a = fmaf(x[i], P[(size_t)i * r + j], a);
        acc[k] = a;
      }
    }
  }
  float* lat = xs + q43_lat_offset(d);
#pragma unroll
  for (int k = 0; k < kValuOuts; ++k) {
    const int idx = threadIdx.x + k * blockDim.x;
    if (idx < kValuTile * r) lat[idx] = acc[k];
  }
  __syncthreads();
  uint8_t* codes = reinterpret_cast<uint8_t*>(xs);                                // [64][r]; inputs no longer read
  uint16_t* prm = reinterpret_cast<uint16_t*>(codes + kValuTile * kMaxRank);      // [64][4]
  for (int t = threadIdx.x; t < kValuTile; t += blockDim.x)
    if (T0 + t >= lo && T0 + t < hi) q43_quantise_row(lat + t * r, r, codes + t * r, prm + 4 * t);
  __syncthreads();

  const int S = kind ? p.Sv : p.Sk;
  const int s_pre = kind ? p.ht.sv_pre[h] : p.ht.sk_pre[h];
  uint8_t* blk = static_cast<uint8_t*>(kind ? p.lat_v : p.lat_k) + (size_t)cap_rows_q43(p.cap) * ((size_t)b * S + s_pre);
  const size_t tb = (size_t)kQ43Tile * q43_row_bytes(r);
  const int no = q43_outlier(r), go = no >> 4, gi = (r - no) >> 4;
  const int per_tile = 128 + 64 * (go + gi);   // parameter halves (4 x 32), then one unit per lane and group
  for (int idx = threadIdx.x; idx < 2 * per_tile; idx += blockDim.x) {
    const int k = idx / per_tile, x = idx - k * per_tile;
    const int t_lo = T0 + kQ43Tile * k;          // rows of this tile: [t_lo, t_lo + 32)
    if (t_lo >= hi || t_lo + kQ43Tile <= lo) continue;
    uint8_t* tile = blk + (size_t)(t_lo / kQ43Tile) * tb;
    auto live = [&](int u) { return t_lo + u >= lo && t_lo + u < hi; };
    auto code = [&](int u, int c) { return (uint32_t)codes[(kQ43Tile * k + u) * r + c]; };
    if (x < 128) {                              // parameter P of tile token u
      const int u = x >> 2, P = x & 3;
      if (live(u)) {
        const int sl = q43_slot(u);
        reinterpret_cast<uint16_t*>(tile + 64 * (sl >> 3) + 16 * P)[sl & 7] = prm[4 * (kQ43Tile * k + u) + P];
      }
      continue;
    }
    const int unit = x - 128, g = unit >> 6, w = unit & 63, n = w & 15, kq = w >> 4;
    if (g < go) {                               // 4-bit word: byte i, nibble = block
      uint32_t bits = 0, keep = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          const int u = q43_token(kind, n, kq, bb, i);
          const int sh = 8 * i + 4 * bb;
          if (live(u)) bits |= code(u, 16 * g + q43_channel(kind, n, kq, i)) << sh;
          else keep |= 0xFu << sh;
        }
      uint32_t* dst = reinterpret_cast<uint32_t*>(tile + kQ43MetaBytes + kQ43OutGroupBytes * g) + w;
      *dst = keep ? ((*dst & keep) | bits) : bits;
    } else {                                    // 24-bit field of 8 3-bit codes
      const int gg = g - go;
      uint32_t bits = 0, keep = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int bb = q43_field_blk(e), i = q43_field_i(e);
        const int u = q43_token(kind, n, kq, bb, i);
        if (live(u)) bits |= code(u, no + 16 * gg + q43_channel(kind, n, kq, i)) << (3 * e);
        else keep |= 0x7u << (3 * e);
      }
      uint8_t* dst = tile + kQ43MetaBytes + kQ43OutGroupBytes * go + kQ43InGroupBytes * gg + 3 * w;
      if (keep) bits = ((dst[0] | (uint32_t)dst[1] << 8 | (uint32_t)dst[2] << 16) & keep) | bits;
      dst[0] = (uint8_t)bits;
      dst[1] = (uint8_t)(bits >> 8);
      dst[2] = (uint8_t)(bits >> 16);
    }
  }
}

// Append: one workgroup per (batch row, KV head, K or V); thread j forms latent
// channel j (r <= 128 = blockDim). Joint values: the h == 0 workgroup sums the
// contributions of every head's new row; the others have nothing to write.
__global__ __launch_bounds__(128) void append_kernel(AppendParams p) {
  __shared__ float xs[256];
  __shared__ float lat[kMaxRank];   // 4/3-bit rows: the fp32 latents before quantisation
  const int b = blockIdx.x, h = blockIdx.y, kind = blockIdx.z;
  const bool joint = kind == 1 && p.joint_v;
  if (joint && h != 0) return;
  const int d = p.d;
  const int pos = p.pos[b];
  if (pos < 0 || pos >= p.cap) return;   // rows outside the cache are not written
  const int r = kind ? p.ht.rv[h] : p.ht.rk[h];
  const void* X = kind ? p.v_new : p.k_new;
  const int j = threadIdx.x;
  float acc = 0.f;
  const int heads = joint ? p.Hkv : 1;
  for (int hs = 0; hs < heads; ++hs) {
    const int hh = joint ? hs : h;
    if (hs > 0) __syncthreads();
    const size_t src0 = ((size_t)b * p.Hkv + hh) * d;
    for (int i = threadIdx.x; i < d; i += blockDim.x)
      xs[i] = p.in_bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(X)[src0 + i])
                        : static_cast<const float*>(X)[src0 + i];
    __syncthreads();
    const float* P = (kind ? p.pv : p.pk) + (size_t)d * (kind ? p.ht.rv_pre[hh] : p.ht.rk_pre[hh]);
    if (j < r)
      for (int i = 0; i < d; ++i) acc = fmaf(xs[i], P[(size_t)i * r + j], acc);
  }
  const int S = kind ? p.Sv : p.Sk;
  const int s_pre = kind ? p.ht.sv_pre[h] : p.ht.sk_pre[h];
  if (p.out_q43) {   // thread 0 finds the block parameters; thread j quantises channel j
    __shared__ float qb[4];   // outlier base, 1/step, inlier base, 1/step
    __shared__ uint16_t qp[4];
    if (j < r) lat[j] = acc;
    __syncthreads();
    const int no = q43_outlier(r);
    if (threadIdx.x == 0) {
      uint32_t meta = 0;
      q43_block_params(lat, 0, no, 15.f, qb[0], qb[1], meta);
      qp[0] = (uint16_t)(meta & 0xFFFFu);
      qp[1] = (uint16_t)(meta >> 16);
      meta = 0;
      qb[2] = qb[3] = 0.f;
      if (r > no) q43_block_params(lat, no, r, 7.f, qb[2], qb[3], meta);
      qp[2] = (uint16_t)(meta & 0xFFFFu);
      qp[3] = (uint16_t)(meta >> 16);
    }
    __syncthreads();
    uint8_t* tile = static_cast<uint8_t*>(kind ? p.lat_v : p.lat_k) +
                    (size_t)cap_rows_q43(p.cap) * ((size_t)b * S + s_pre) +
                    (size_t)(pos / kQ43Tile) * kQ43Tile * q43_row_bytes(r);
    const int u = pos & (kQ43Tile - 1);
    if (j < 4) {
      const int sl = q43_slot(u);
      reinterpret_cast<uint16_t*>(tile + 64 * (sl >> 3) + 16 * j)[sl & 7] = qp[j];
    }
    if (j < r) {
      const bool four = j < no;
      const uint32_t c = q43_code(lat[j], qb[four ? 0 : 2], qb[four ? 1 : 3], four ? 15.f : 7.f);
      int byte, shift;
      q43_code_pos(kind, u, j, r, byte, shift);
      // the code's bits inside the tile's dwords (tiles start on 32-byte boundaries); other
      // threads change other bits of the same dwords, hence the atomic AND / OR
      const int bit = 8 * byte + shift, width = four ? 4 : 3;
      uint32_t* wd = reinterpret_cast<uint32_t*>(tile) + (bit >> 5);
      const int b0 = bit & 31;
      const uint32_t m0 = ((1u << width) - 1u) << b0;
      __hip_atomic_fetch_and(wd, ~m0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_or(wd, c << b0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (b0 + width > 32) {
        const int hi_bits = b0 + width - 32;
        __hip_atomic_fetch_and(wd + 1, ~((1u << hi_bits) - 1u), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_or(wd + 1, c >> (width - hi_bits), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    return;
  }
  if (j >= r) return;
  const size_t base = (size_t)cap_rows_of(p.cap) * ((size_t)b * S + s_pre);
  const bool k_tiled = p.out_bf16 && kind == 0;
  const bool v_tiled = p.out_bf16 && kind == 1;
  const size_t off = base + (k_tiled   ? k_tiled_offset(pos, j, r)
                             : v_tiled ? v_joint_offset(pos, j, r)
                                       : (size_t)pos * r + j);
  if (p.out_bf16)
    static_cast<uint16_t*>(kind ? p.lat_v : p.lat_k)[off] = f32_to_bf16_bits(acc);
  else
    static_cast<float*>(kind ? p.lat_v : p.lat_k)[off] = acc;
}

}  // namespace

// 4/3-bit compression: chunks of 64 rows from the tile holding row `start`, and their LDS
// (inputs [64][d] then latents [64][r]; codes and parameters reuse the input area).
int q43_chunks(const CompressParams& p) {
  const int t0 = p.start & ~(kQ43Tile - 1);
  return (p.start + p.n_tok - t0 + kValuTile - 1) / kValuTile;
}
size_t q43_lds(const CompressParams& p, int max_r) {
  return ((size_t)q43_lat_offset(p.d) + (size_t)kValuTile * max_r) * sizeof(float);
}

// Work of the MFMA compression: per batch row, segments (values of heads 0..Hkv-1, then
// keys; a kind that this launch does not write has none) get workgroups in proportion to
// their bytes per token (2 d read, 2 r written, writes counted twice), about `slots` in
// all, so that workgroups have about the same work; every workgroup takes a whole
// number of 256-token groups, and at least one.
void compress_schedule(CompressParams& p, int slots) {
  const int H = p.Hkv;
  double w[2 * kMaxKvHeads], total = 0.0;
  for (int s = 0; s < 2 * H; ++s) {
    const int kind = s < H ? 1 : 0, h = s < H ? s : s - H;
    const bool on = p.only_kind < 0 || p.only_kind == kind;
    w[s] = on ? 2.0 * p.d + 4.0 * (kind ? p.ht.rv[h] : p.ht.rk[h]) : 0.0;
    total += w[s];
  }
  const double per_row = (double)slots / p.B;
  const int groups = (p.n_tok + kCompressGroup - 1) / kCompressGroup;
  // the rows of one workgroup stay below 2^31 bytes (32-bit buffer offsets)
  const long long row_bytes = 2LL * p.Hkv * p.d;
  const int max_groups = (int)std::max(1LL, ((1LL << 31) - 1) / (row_bytes * kCompressGroup));
  p.sched_pre[0] = 0;
  for (int s = 0; s < 2 * H; ++s) {
    int n = 0, chunk = kCompressGroup;
    if (w[s] > 0.0) {
      n = std::min(groups, std::max(1, (int)std::lround(per_row * w[s] / total)));
      int g = (groups + n - 1) / n;   // groups per workgroup
      g = std::min(g, max_groups);
      chunk = g * kCompressGroup;
      n = (p.n_tok + chunk - 1) / chunk;
    }
    p.sched_chunk[s] = chunk;
    p.sched_pre[s + 1] = p.sched_pre[s] + n;
  }
  p.sched_row = p.sched_pre[2 * H];
}

hipError_t launch_compress(const CompressParams& p_in, hipStream_t stream) {
  if (p_in.n_tok <= 0) return hipSuccess;
  int max_r = 0;
  bool tiles16 = true;   // the MFMA kernel writes whole 16-channel tiles (fp32 latents allow ranks of 4 k)
  for (int h = 0; h < p_in.Hkv; ++h) {
    max_r = max(max_r, max(p_in.ht.rk[h], p_in.ht.rv[h]));
    tiles16 = tiles16 && p_in.ht.rk[h] % 16 == 0 && (p_in.joint_v || p_in.ht.rv[h] % 16 == 0);
  }
  CompressParams p = p_in;
  p.only_kind = p.joint_v ? 0 : -1;   // joint values get a launch of their own below
  const int ykinds = p.joint_v ? 1 : 2;
  if (p.in_bf16 && !p.out_q43 && tiles16) {
    const size_t lds = (size_t)4 * max_r * p.d;   // hi + lo operand tiles
    const void* fn = nullptr;
#define KVLR_COMPRESS_CASE(NKB)                                                                             \
  case NKB:                                                                                                 \
    fn = p.out_bf16 ? (const void*)compress_bf16_mfma<true, NKB> : (const void*)compress_bf16_mfma<false, NKB>; \
    break;
    switch (p.d / 32) {
      KVLR_COMPRESS_CASE(1)
      KVLR_COMPRESS_CASE(2)
      KVLR_COMPRESS_CASE(3)
      KVLR_COMPRESS_CASE(4)
      KVLR_COMPRESS_CASE(5)
      KVLR_COMPRESS_CASE(6)
      KVLR_COMPRESS_CASE(7)
      default: KVLR_COMPRESS_CASE(8)
    }
#undef KVLR_COMPRESS_CASE
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, lds) != hipSuccess || per_cu < 1) per_cu = 1;
    // about 8 rounds of resident workgroups: measured faster than one round of long
    // workgroups (whose waves fall into step) and than finer splits (basis staging)
    compress_schedule(p, kCompressRounds * per_cu * max(p.n_cu, 1));
    const dim3 grid((unsigned)(p.B * p.sched_row));
    void* args[] = {&p};
    const hipError_t e = hipLaunchKernel(fn, grid, dim3(256), args, lds, stream);
    if (e != hipSuccess) return e;
  } else if (p.out_q43) {
    const dim3 grid(q43_chunks(p), ykinds * p.Hkv, p.B);
    hipLaunchKernelGGL(compress_q43, grid, dim3(256), q43_lds(p, max_r), stream, p);
  } else {
    const size_t lds = (size_t)kValuTile * p.d * sizeof(float);
    const dim3 grid((p.n_tok + kValuTile - 1) / kValuTile, ykinds * p.Hkv, p.B);
    hipLaunchKernelGGL(compress_valu, grid, dim3(256), lds, stream, p);
  }
  if (p.joint_v) {   // joint values: one workgroup per (tile, batch row) sums over every head
    CompressParams pv = p_in;
    pv.only_kind = 1;
    if (p.out_q43) {
      hipLaunchKernelGGL(compress_q43, dim3(q43_chunks(pv), 1, p.B), dim3(256), q43_lds(pv, max_r), stream, pv);
    } else {
      const size_t lds = (size_t)kValuTile * p.d * sizeof(float);
      const dim3 grid((p.n_tok + kValuTile - 1) / kValuTile, 1, p.B);
      hipLaunchKernelGGL(compress_valu, grid, dim3(256), lds, stream, pv);
    }
  }
  return hipGetLastError();
}

hipError_t launch_hadamard(const float* in, float* out, size_t n_groups, hipStream_t stream) {
  if (n_groups == 0) return hipSuccess;
  hipLaunchKernelGGL(hadamard_fold, dim3((unsigned)((n_groups + 255) / 256)), dim3(256), 0, stream, in, out, n_groups);
  return hipGetLastError();
}

hipError_t launch_append(const AppendParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(append_kernel, dim3(p.B, p.Hkv, 2), dim3(128), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kvlr
