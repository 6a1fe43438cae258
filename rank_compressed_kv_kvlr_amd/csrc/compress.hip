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
//
// fp32 inputs, ranks that are not whole 16-channel tiles, 4/3-bit latents and
// joint value latents use a plain VALU kernel; append uses one workgroup per
// (batch row, KV head, K or V).
//
// Mixed 4/3-bit latents (STAR-KV technical summary, "Metodologia" section 3)
// are quantised from the fp32 latents of a row by one thread per row; the
// block-wise Hadamard rotation is already folded into the bases it receives
// (hadamard_fold below, run once per set of bases).
#include "kvlr_internal.hpp"

namespace kvlr {
namespace {

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
constexpr int kWaveIters = 4;             // tiles per wave per workgroup
constexpr int kTokensPerWg = kCompressWaves * kTokensPerWave * kWaveIters;   // 1024

// LDS budget for the staged basis: (r/16) * (d/32) * 64 lanes * 16 B * 2 = 4 r d bytes.
constexpr int kStageBytes = 4 * kMaxRank * 256;   // r <= 128, d <= 256

// NKB = d / 32: 32-channel input blocks (one MFMA each per 16 tokens).
template <bool kOutBf16, int NKB>
__global__ __launch_bounds__(256) void compress_bf16_mfma(CompressParams p) {
  extern __shared__ __attribute__((aligned(16))) uint4 stage[];   // [mt][kb][lane] hi, then lo
  const int kind = p.only_kind >= 0 ? p.only_kind : (int)(blockIdx.y & 1);   // 0 keys, 1 values
  const int h = p.only_kind >= 0 ? (int)blockIdx.y : (int)(blockIdx.y >> 1);
  const int b = blockIdx.z;
  const int d = p.d;
  const int r = kind ? p.ht.rv[h] : p.ht.rk[h];
  const int r_pre = kind ? p.ht.rv_pre[h] : p.ht.rk_pre[h];
  const float* P = (kind ? p.pv : p.pk) + (size_t)d * r_pre;
  const uint16_t* X = static_cast<const uint16_t*>(kind ? p.x_v : p.x_k);
  const int n_mt = r >> 4, dq = d >> 2;
  constexpr int n_kb = NKB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, q4 = lane >> 4;

  // ---- stage P^T operands: entry (mt, kb, lane) holds P[q*dq + 8kb + e][16mt + lane%16], e < 8
  const int n_entries = n_mt * n_kb * 64;
  uint4* st_hi = stage;
  uint4* st_lo = stage + n_entries;
  for (int idx = tid; idx < n_entries; idx += blockDim.x) {
    const int ln = idx & 63;
    const int kb = (idx >> 6) % n_kb;
    const int mt = (idx >> 6) / n_kb;
    const int col = 16 * mt + (ln & 15);
    const int row0 = (ln >> 4) * dq + 8 * kb;
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float x0 = P[(size_t)(row0 + e) * r + col];
      const float x1 = P[(size_t)(row0 + e + 1) * r + col];
      const uint16_t h0 = f32_to_bf16_bits(x0), h1 = f32_to_bf16_bits(x1);
      const uint16_t l0 = f32_to_bf16_bits(x0 - bf16_bits_to_f32(h0));
      const uint16_t l1 = f32_to_bf16_bits(x1 - bf16_bits_to_f32(h1));
      hi[e >> 1] = (uint32_t)h0 | ((uint32_t)h1 << 16);
      lo[e >> 1] = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
    st_hi[idx] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    st_lo[idx] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
  __syncthreads();

  const size_t row_stride = (size_t)p.Hkv * d;   // elements between consecutive tokens
  const uint16_t* Xb = X + (size_t)b * p.n_tok * row_stride + (size_t)h * d;
  const size_t lat_base = (size_t)cap_rows_of(p.cap) * ((size_t)b * (kind ? p.Sv : p.Sk) +
                                                      (kind ? p.ht.sv_pre[h] : p.ht.sk_pre[h]));
  const bool k_tiled = kOutBf16 && kind == 0;   // bf16 key latents: MFMA operand order
  const bool v_tiled = kOutBf16 && kind == 1;   // bf16 value latents: value-product operand order
  const int tok_wg0 = blockIdx.x * kTokensPerWg;

  for (int it = 0; it < kWaveIters; ++it) {
    const int tw0 = tok_wg0 + (it * kCompressWaves + wave) * kTokensPerWave;
    if (tw0 >= p.n_tok) break;
    // input rows: 4 column tiles of 16 tokens, lane covers d/4 channels
    uint4 xin[4][NKB];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int t = min(tw0 + 16 * nt + n16, p.n_tok - 1);
      const uint16_t* row = Xb + (size_t)t * row_stride + q4 * dq;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) xin[nt][kb] = *reinterpret_cast<const uint4*>(row + 8 * kb);
    }
    for (int mt = 0; mt < n_mt; ++mt) {
      f32x4_t acc[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[nt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        {
          const int e = (mt * n_kb + kb) * 64 + lane;
          const bf16x8_t ahi = __builtin_bit_cast(bf16x8_t, st_hi[e]);
          const bf16x8_t alo = __builtin_bit_cast(bf16x8_t, st_lo[e]);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            const bf16x8_t xb = __builtin_bit_cast(bf16x8_t, xin[nt][kb]);
            if (v_tiled) {   // transposed product: lane ends with 4 consecutive tokens of one channel
              acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb, ahi, acc[nt], 0, 0, 0);
              acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb, alo, acc[nt], 0, 0, 0);
            } else {
              acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, xb, acc[nt], 0, 0, 0);
              acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, xb, acc[nt], 0, 0, 0);
            }
          }
        }
      }
      if (v_tiled) {
        // lane holds tokens tw0 + 16nt + 4q4 + i (i < 4) of latent channel 16mt + n16: one
        // 8-byte piece when the 4 tokens are whole and aligned, single values otherwise
        uint16_t* V = static_cast<uint16_t*>(p.lat_v) + lat_base;
        const int j = 16 * mt + n16;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int t = tw0 + 16 * nt + 4 * q4;
          const int row = p.start + t;
          if (t + 3 < p.n_tok && (row & 3) == 0) {
            const uint32_t w0 = (uint32_t)f32_to_bf16_bits(acc[nt][0]) | ((uint32_t)f32_to_bf16_bits(acc[nt][1]) << 16);
            const uint32_t w1 = (uint32_t)f32_to_bf16_bits(acc[nt][2]) | ((uint32_t)f32_to_bf16_bits(acc[nt][3]) << 16);
            *reinterpret_cast<uint2*>(V + v_joint_offset(row, j, r)) = make_uint2(w0, w1);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (t + i < p.n_tok) V[v_joint_offset(row + i, j, r)] = f32_to_bf16_bits(acc[nt][i]);
          }
        }
        continue;
      }
      // lane holds latent channels 16mt + 4q4 + i (i < 4) of token tw0 + 16nt + n16
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int t = tw0 + 16 * nt + n16;
        if (t < p.n_tok) {
          const int j0 = 16 * mt + 4 * q4;   // 4 consecutive channels stay contiguous in both layouts
          const size_t off = lat_base + (k_tiled ? k_tiled_offset(p.start + t, j0, r) : (size_t)(p.start + t) * r + j0);
          if (kOutBf16) {
            const uint32_t w0 = (uint32_t)f32_to_bf16_bits(acc[nt][0]) | ((uint32_t)f32_to_bf16_bits(acc[nt][1]) << 16);
            const uint32_t w1 = (uint32_t)f32_to_bf16_bits(acc[nt][2]) | ((uint32_t)f32_to_bf16_bits(acc[nt][3]) << 16);
            uint16_t* dst = static_cast<uint16_t*>(kind ? p.lat_v : p.lat_k) + off;
            *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
          } else {
            float* dst = static_cast<float*>(kind ? p.lat_v : p.lat_k) + off;
            *reinterpret_cast<float4*>(dst) = make_float4(acc[nt][0], acc[nt][1], acc[nt][2], acc[nt][3]);
          }
        }
      }
    }
  }
}

// Plain VALU compression (fp32 inputs, ranks that are not whole 16-channel
// tiles, 4/3-bit latents, joint values): one workgroup per (64-token tile,
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
    const dim3 grid((p.n_tok + kTokensPerWg - 1) / kTokensPerWg, ykinds * p.Hkv, p.B);
#define KVLR_COMPRESS_CASE(NKB)                                                              \
  case NKB:                                                                                  \
    if (p.out_bf16)                                                                          \
      hipLaunchKernelGGL((compress_bf16_mfma<true, NKB>), grid, dim3(256), lds, stream, p);  \
    else                                                                                     \
      hipLaunchKernelGGL((compress_bf16_mfma<false, NKB>), grid, dim3(256), lds, stream, p); \
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
