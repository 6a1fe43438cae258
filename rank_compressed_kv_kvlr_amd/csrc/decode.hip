// Split-sequence decode attention over a rank-compressed KV cache (gfx950).
//
// Method (StiefAttention technical summary, "Mecanismo Central" item 5):
// keys and values are stored as latents K P_K, V P_V and reconstructed with
// P^T before softmax attention. By associativity the kernels never rebuild
// K~ or V~: the query is projected once (q~ = q P_K), scored against the
// stored latents, and the softmax-weighted sum of value latents is
// back-projected once by P_V^T after the splits are merged.
//
// Work decomposition: one workgroup (4 waves) per (split of the sequence,
// KV head, group of <= 4 query heads sharing it, batch row). Each wave walks
// 64-token tiles of the split; waves keep a running max / sum / weighted
// latent sum (online softmax, base-2 domain) and the workgroup merges its 4
// waves into one partial record (m, l, o_lat[r_v]) per query head. A second
// kernel merges the records of all splits with log-sum-exp weights and
// applies P_V^T.
//
// bf16 latents: the score tile S[head][token] = q~ . K_lat is one MFMA chain
// per 16 tokens (v_mfma_f32_16x16x32_bf16, query heads as rows, tokens as
// columns, the key latent rows loaded straight from HBM into the B operand,
// 16 contiguous bytes per lane). q~ is fp32; it enters the MFMA as a high
// and a low bf16 part (two MFMAs into one fp32 accumulator), so scores keep
// ~16 bits of the query. The value side (p-weighted sum of V_lat rows) runs
// on VALU: each lane owns 8 latent channels of a subset of rows, reading 16
// coalesced bytes per row chunk, and p comes through LDS.
#include "kvlr_internal.hpp"

namespace kvlr {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

// Largest number of 64-lane value loads per 64-token tile over ranks r <= rb
// (multiples of 16): a row has r/8 chunks of 8 channels, a load instruction
// covers floor(64 / (r/8)) rows.
constexpr int value_iters_bound(int rb) {
  int worst = 0;
  for (int r = 16; r <= rb; r += 16) {
    const int rpi = 64 / (r / 8);
    const int it = (64 + rpi - 1) / rpi;
    worst = it > worst ? it : worst;
  }
  return worst;
}

// ---------------------------------------------------------------------------
// shared prologue: q~ = (q P_K) * scale * log2(e) for the workgroup's heads
// ---------------------------------------------------------------------------
__device__ __forceinline__ void project_query(const DecodeParams& p, int b, int h, int hq0, int gpw,
                                              int rk, float* q_lds, float* qt_lds, int qt_stride) {
  const int tid = threadIdx.x;
  const int d = p.d;
  for (int idx = tid; idx < gpw * d; idx += blockDim.x) {
    const int g = idx / d, i = idx - g * d;
    q_lds[g * d + i] = p.q[((size_t)b * p.Hq + hq0 + g) * d + i];
  }
  __syncthreads();
  const float* P = p.pk + (size_t)d * p.ht.rk_pre[h];
  for (int idx = tid; idx < kHeadsPerWg * qt_stride; idx += blockDim.x) {
    const int g = idx / qt_stride, j = idx - g * qt_stride;
    float acc = 0.f;
    if (g < gpw && j < rk) {
      const float* qg = q_lds + g * d;
      for (int i = 0; i < d; ++i) acc = fmaf(qg[i], P[(size_t)i * rk + j], acc);
      acc *= p.scale_log2;
    }
    qt_lds[idx] = acc;   // zero rows for heads beyond gpw and channels beyond rk
  }
  __syncthreads();
}

__device__ __forceinline__ void write_empty_records(const DecodeParams& p, int b, int hq0, int gpw, int s, int rv) {
  for (int idx = threadIdx.x; idx < gpw * (rv + 2); idx += blockDim.x) {
    const int g = idx / (rv + 2), j = idx - g * (rv + 2);
    float* rec = p.ws + (((size_t)b * p.Hq + hq0 + g) * p.n_splits + s) * p.ws_stride;
    rec[j] = (j == 0) ? kNegInf : 0.f;
  }
}

// Merge of the 4 waves' states into one record per head.
//   wm, wl: [4 waves][4 heads]; red: per-wave per-lane partial sums laid out by
//   the caller; value(w, g, j) returns wave w's unnormalised latent sum for
//   head g, channel j.
template <typename ValueFn>
__device__ __forceinline__ void merge_waves_and_store(const DecodeParams& p, int b, int hq0, int gpw, int s,
                                                      int rv, const float* wm, const float* wl, ValueFn value) {
  for (int idx = threadIdx.x; idx < gpw * rv; idx += blockDim.x) {
    const int g = idx / rv, j = idx - g * rv;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wm[w * 4 + g]);
    float o = 0.f, L = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = fast_exp2(wm[w * 4 + g] - M);   // -inf -> 0
        L = fmaf(f, wl[w * 4 + g], L);
        o = fmaf(f, value(w, g, j), o);
      }
    }
    float* rec = p.ws + (((size_t)b * p.Hq + hq0 + g) * p.n_splits + s) * p.ws_stride;
    rec[2 + j] = o;
    if (j == 0) {
      rec[0] = M;
      rec[1] = L;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 latents: MFMA scores, VALU value mix
// ---------------------------------------------------------------------------
// RB: rank bound (32, 64, 96 or 128) sizing the register tiles; the actual
// per-head ranks are runtime values <= RB (multiples of 16).
template <int RB>
__global__ __launch_bounds__(256) void decode_split_bf16(DecodeParams p) {
  constexpr int NP = RB / 32;                 // full 32-channel key pairs
  constexpr int NIT = value_iters_bound(RB);  // bound on value iterations (see n_it below)
  constexpr int QTS = RB;                     // q~ LDS row stride
  __shared__ __attribute__((aligned(16))) float smem[kWaves * 64 * 4 * 8 + 64];

  const int s = blockIdx.x;
  const int h = blockIdx.y / p.n_head_groups;
  const int hg = blockIdx.y - h * p.n_head_groups;
  const int b = blockIdx.z;
  const int hq0 = h * p.G + hg * kHeadsPerWg;
  const int gpw = min(kHeadsPerWg, p.G - hg * kHeadsPerWg);
  const int rk = p.ht.rk[h], rv = p.ht.rv[h];
  const int T = min(max(p.seq_lens[b], 0), p.cap);
  const int t_begin = s * p.split_len;
  const int t_end = min(T, t_begin + p.split_len);
  if (t_begin >= t_end) {
    write_empty_records(p, b, hq0, gpw, s, rv);
    return;
  }

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, q4 = lane >> 4;

  // ---- prologue: q~ into LDS, then MFMA A operands (hi/lo) into registers
  float* q_lds = smem;                          // [4][d]  (d <= 256)
  float* qt_lds = smem + kHeadsPerWg * 256;     // [4][QTS]
  project_query(p, b, h, hq0, gpw, rk, q_lds, qt_lds, QTS);

  const int np = rk >> 5;           // full 32-channel pairs
  const int tail = (rk >> 4) & 1;   // one trailing 16-channel block
  bf16x8_t a_hi[NP], a_lo[NP];
  bf16x4_t t_hi, t_lo;
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = (n16 < kHeadsPerWg) ? qt_lds[n16 * QTS + 32 * pp + 8 * q4 + e] : 0.f;
      if (32 * pp + 8 * q4 + e >= rk) x = 0.f;
      const uint16_t hi = f32_to_bf16_bits(x);
      const uint16_t lo = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
      a_hi[pp][e] = (short)hi;
      a_lo[pp][e] = (short)lo;
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = 32 * np + 4 * q4 + e;
    float x = (n16 < kHeadsPerWg && tail && j < rk) ? qt_lds[n16 * QTS + j] : 0.f;
    const uint16_t hi = f32_to_bf16_bits(x);
    const uint16_t lo = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
    t_hi[e] = (short)hi;
    t_lo[e] = (short)lo;
  }
  __syncthreads();   // LDS is reused below

  // ---- value-side lane mapping: C chunks of 8 channels per row
  const int C = rv >> 3;
  const int rpi = 64 / C;                 // rows per load instruction
  const int ro = lane / C, cch = lane - ro * C;
  const bool v_active = ro < rpi;
  const int n_it = (64 + rpi - 1) / rpi;  // <= NIT

  const uint16_t* Kb = static_cast<const uint16_t*>(p.lat_k) + (size_t)p.cap * ((size_t)b * p.Rk + p.ht.rk_pre[h]);
  const uint16_t* Vb = static_cast<const uint16_t*>(p.lat_v) + (size_t)p.cap * ((size_t)b * p.Rv + p.ht.rv_pre[h]);

  float* p_lds = smem + wave * (64 * 4);  // [64 tokens][4 heads] per wave

  float m[4], l[4], acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = kNegInf;
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
  }

  uint4 kreg[4][NP];
  uint2 ktail[4];
  uint4 vreg[NIT];

  auto load_k = [&](int t0) {
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const int t = min(t0 + 16 * blk + n16, t_end - 1);
      const uint16_t* row = Kb + (size_t)t * rk;
#pragma unroll
      for (int pp = 0; pp < NP; ++pp)
        if (pp < np) kreg[blk][pp] = *reinterpret_cast<const uint4*>(row + 32 * pp + 8 * q4);
      if (tail) ktail[blk] = *reinterpret_cast<const uint2*>(row + 32 * np + 4 * q4);
    }
  };
  auto load_v = [&](int t0) {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      if (it < n_it) {
        const int r = it * rpi + ro;
        const int t = min(t0 + min(r, 63), t_end - 1);
        vreg[it] = *reinterpret_cast<const uint4*>(Vb + (size_t)t * rv + 8 * cch);
      }
    }
  };

  int t0 = t_begin + wave * kTile;
  if (t0 < t_end) {
    load_k(t0);
    load_v(t0);
  }
  for (; t0 < t_end; t0 += kWaves * kTile) {
    const int t_next = t0 + kWaves * kTile;
    // ---- scores on MFMA
    f32x4_t sc[4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        if (pp < np) {
          const bf16x8_t kb = __builtin_bit_cast(bf16x8_t, kreg[blk][pp]);
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi[pp], kb, d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_lo[pp], kb, d, 0, 0, 0);
        }
      }
      if (tail) {
        const bf16x4_t kb = __builtin_bit_cast(bf16x4_t, ktail[blk]);
        d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(t_hi, kb, d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(t_lo, kb, d, 0, 0, 0);
      }
      sc[blk] = d;
    }
    if (t_next < t_end) load_k(t_next);   // key registers are free again

    // ---- online softmax (lanes 0..15 hold heads 0..3 of 16 tokens per block)
    float alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mx = kNegInf;
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const bool valid = (t0 + 16 * blk + n16) < t_end;
        sc[blk][i] = valid ? sc[blk][i] : kNegInf;
        mx = fmaxf(mx, sc[blk][i]);
      }
      mx = row16_allreduce<true>(mx);
      const float m_new = fmaxf(m[i], mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      alpha[i] = fast_exp2(m[i] - m_use);
      float ls = 0.f;
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const float pr = fast_exp2(sc[blk][i] - m_use);
        sc[blk][i] = pr;
        ls += pr;
      }
      l[i] = fmaf(l[i], alpha[i], ls);
      m[i] = m_new;
    }
    if (q4 == 0) {
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
        *reinterpret_cast<float4*>(p_lds + (16 * blk + n16) * 4) =
            make_float4(sc[blk][0], sc[blk][1], sc[blk][2], sc[blk][3]);
    }
    // scale factors live in lane 0 (group of heads 0..3)
    float a_s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a_s[i] = readlane_f(alpha[i], 0);
    if (a_s[0] != 1.f || a_s[1] != 1.f || a_s[2] != 1.f || a_s[3] != 1.f) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] *= a_s[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- value mix on VALU
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      if (it < n_it) {
        const int r = it * rpi + ro;
        if (v_active && r < 64) {
          const float4 pw = *reinterpret_cast<const float4*>(p_lds + r * 4);
          const uint4 w = vreg[it];
          const float v[8] = {bf16lo_to_f32(w.x), bf16hi_to_f32(w.x), bf16lo_to_f32(w.y), bf16hi_to_f32(w.y),
                              bf16lo_to_f32(w.z), bf16hi_to_f32(w.z), bf16lo_to_f32(w.w), bf16hi_to_f32(w.w)};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            acc[0][e] = fmaf(pw.x, v[e], acc[0][e]);
            acc[1][e] = fmaf(pw.y, v[e], acc[1][e]);
            acc[2][e] = fmaf(pw.z, v[e], acc[2][e]);
            acc[3][e] = fmaf(pw.w, v[e], acc[3][e]);
          }
        }
      }
    }
    if (t_next < t_end) load_v(t_next);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- workgroup merge of the 4 waves
#pragma unroll
  for (int i = 0; i < 4; ++i) l[i] = row16_allreduce<false>(l[i]);
  __syncthreads();
  float* red = smem;                          // [wave][lane][head][8]
  float* wm = smem + kWaves * 64 * 32;        // [wave][head]
  float* wl = wm + 16;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; e += 4)
      *reinterpret_cast<float4*>(red + ((wave * 64 + lane) * 4 + i) * 8 + e) =
          make_float4(acc[i][e], acc[i][e + 1], acc[i][e + 2], acc[i][e + 3]);
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wm[wave * 4 + i] = m[i];
      wl[wave * 4 + i] = l[i];
    }
  }
  __syncthreads();
  merge_waves_and_store(p, b, hq0, gpw, s, rv, wm, wl, [&](int w, int g, int j) {
    const int c = j >> 3, e = j & 7;
    float sum = 0.f;
    for (int r = 0; r < rpi; ++r) sum += red[((w * 64 + r * C + c) * 4 + g) * 8 + e];
    return sum;
  });
}

// ---------------------------------------------------------------------------
// fp32 latents: VALU throughout (token per lane for scores, channel per lane
// for the value mix)
// ---------------------------------------------------------------------------
template <int RB>
__global__ __launch_bounds__(256) void decode_split_f32(DecodeParams p) {
  constexpr int QTS = RB;
  constexpr int VJ = (RB + 63) / 64;          // value channels per lane
  constexpr int RED = kWaves * 4 * (RB > 64 ? RB : 64);   // also holds the per-wave [64][4] p tiles
  __shared__ __attribute__((aligned(16))) float smem[RED + kHeadsPerWg * 256 + kHeadsPerWg * RB + 64];

  const int s = blockIdx.x;
  const int h = blockIdx.y / p.n_head_groups;
  const int hg = blockIdx.y - h * p.n_head_groups;
  const int b = blockIdx.z;
  const int hq0 = h * p.G + hg * kHeadsPerWg;
  const int gpw = min(kHeadsPerWg, p.G - hg * kHeadsPerWg);
  const int rk = p.ht.rk[h], rv = p.ht.rv[h];
  const int T = min(max(p.seq_lens[b], 0), p.cap);
  const int t_begin = s * p.split_len;
  const int t_end = min(T, t_begin + p.split_len);
  if (t_begin >= t_end) {
    write_empty_records(p, b, hq0, gpw, s, rv);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  float* red = smem;                                  // [wave][4 heads][RB] at the end
  float* q_lds = smem + RED;                          // [4][d]
  float* qt_lds = q_lds + kHeadsPerWg * 256;          // [4][QTS]
  float* wm = qt_lds + kHeadsPerWg * QTS;             // [wave][head]
  float* wl = wm + 16;
  project_query(p, b, h, hq0, gpw, rk, q_lds, qt_lds, QTS);

  const float* Kb = static_cast<const float*>(p.lat_k) + (size_t)p.cap * ((size_t)b * p.Rk + p.ht.rk_pre[h]);
  const float* Vb = static_cast<const float*>(p.lat_v) + (size_t)p.cap * ((size_t)b * p.Rv + p.ht.rv_pre[h]);
  // per-wave probability tile lives in the (not yet used) reduction area
  float* p_lds = red + wave * 64 * 4;

  float m[4], l[4], acc[4][VJ];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = kNegInf;
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < VJ; ++e) acc[i][e] = 0.f;
  }

  for (int t0 = t_begin + wave * kTile; t0 < t_end; t0 += kWaves * kTile) {
    const int t = t0 + lane;
    const bool valid = t < t_end;
    const float* row = Kb + (size_t)min(t, t_end - 1) * rk;
    float sc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < rk; j += 4) {
      const float4 k4 = *reinterpret_cast<const float4*>(row + j);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 q4 = *reinterpret_cast<const float4*>(qt_lds + i * QTS + j);
        sc[i] = fmaf(q4.x, k4.x, sc[i]);
        sc[i] = fmaf(q4.y, k4.y, sc[i]);
        sc[i] = fmaf(q4.z, k4.z, sc[i]);
        sc[i] = fmaf(q4.w, k4.w, sc[i]);
      }
    }
    float pr[4], alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float sv = valid ? sc[i] : kNegInf;
      const float mx = wave_allreduce<true>(sv);
      const float m_new = fmaxf(m[i], mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      alpha[i] = fast_exp2(m[i] - m_use);
      pr[i] = fast_exp2(sv - m_use);
      l[i] = fmaf(l[i], alpha[i], pr[i]);
      m[i] = m_new;
    }
    *reinterpret_cast<float4*>(p_lds + lane * 4) = make_float4(pr[0], pr[1], pr[2], pr[3]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < VJ; ++e) acc[i][e] *= alpha[i];
    const int nt = min(kTile, t_end - t0);
    for (int u = 0; u < nt; ++u) {
      const float4 pw = *reinterpret_cast<const float4*>(p_lds + u * 4);
      const float* vrow = Vb + (size_t)(t0 + u) * rv;
#pragma unroll
      for (int e = 0; e < VJ; ++e) {
        const int j = lane + 64 * e;
        if (j < rv) {
          const float v = vrow[j];
          acc[0][e] = fmaf(pw.x, v, acc[0][e]);
          acc[1][e] = fmaf(pw.y, v, acc[1][e]);
          acc[2][e] = fmaf(pw.z, v, acc[2][e]);
          acc[3][e] = fmaf(pw.w, v, acc[3][e]);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) l[i] = wave_allreduce<false>(l[i]);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < VJ; ++e) {
      const int j = lane + 64 * e;
      if (j < RB) red[(wave * 4 + i) * RB + j] = acc[i][e];
    }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wm[wave * 4 + i] = m[i];
      wl[wave * 4 + i] = l[i];
    }
  }
  __syncthreads();
  merge_waves_and_store(p, b, hq0, gpw, s, rv, wm, wl,
                        [&](int w, int g, int j) { return red[(w * 4 + g) * RB + j]; });
}

// ---------------------------------------------------------------------------
// merge of split records and back-projection by P_V^T
// ---------------------------------------------------------------------------
constexpr int kMergeThreads = 256;
constexpr int kMergeChunk = 1024;

__global__ __launch_bounds__(kMergeThreads) void decode_merge(MergeParams p) {
  __shared__ float f_lds[kMergeChunk];
  __shared__ float olat[kMaxRank];
  __shared__ float red[kMergeThreads / 64];
  const int i = blockIdx.x, b = blockIdx.y;
  const int h = i / p.G;
  const int rv = p.ht.rv[h];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* recs = p.ws + ((size_t)b * p.Hq + i) * p.n_splits * p.ws_stride;

  // global max of the split maxima
  float M = kNegInf;
  for (int s = tid; s < p.n_splits; s += kMergeThreads) M = fmaxf(M, recs[(size_t)s * p.ws_stride]);
  M = wave_allreduce<true>(M);
  if (lane == 0) red[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();

  float* outp = p.out + ((size_t)b * p.Hq + i) * p.d;
  if (M == kNegInf) {   // empty sequence
    for (int dd = tid; dd < p.d; dd += kMergeThreads) outp[dd] = 0.f;
    return;
  }
  float L = 0.f, o = 0.f;   // thread j < rv accumulates channel j
  for (int s0 = 0; s0 < p.n_splits; s0 += kMergeChunk) {
    const int ns = min(kMergeChunk, p.n_splits - s0);
    for (int s = tid; s < ns; s += kMergeThreads) {
      const float* r = recs + (size_t)(s0 + s) * p.ws_stride;
      f_lds[s] = fast_exp2(r[0] - M);   // empty split: exp2(-inf) = 0
    }
    __syncthreads();
    if (tid < rv) {
      for (int s = 0; s < ns; ++s) {
        const float f = f_lds[s];
        if (f != 0.f) {
          const float* r = recs + (size_t)(s0 + s) * p.ws_stride;
          o = fmaf(f, r[2 + tid], o);
          L = fmaf(f, r[1], L);
        }
      }
    }
    __syncthreads();
  }
  if (tid < rv) olat[tid] = o / L;
  __syncthreads();
  const float* P = p.pv + (size_t)p.d * p.ht.rv_pre[h];
  for (int dd = tid; dd < p.d; dd += kMergeThreads) {
    const float* prow = P + (size_t)dd * rv;
    float acc = 0.f;
    for (int j = 0; j < rv; ++j) acc = fmaf(olat[j], prow[j], acc);
    outp[dd] = acc;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int latent_bf16, int rank_bound, hipStream_t stream) {
  const dim3 grid(p.n_splits, p.Hkv * p.n_head_groups, p.B);
  const dim3 block(kWaves * 64);
  if (latent_bf16) {
    switch (rank_bound) {
      case 32: hipLaunchKernelGGL(decode_split_bf16<32>, grid, block, 0, stream, p); break;
      case 64: hipLaunchKernelGGL(decode_split_bf16<64>, grid, block, 0, stream, p); break;
      case 96: hipLaunchKernelGGL(decode_split_bf16<96>, grid, block, 0, stream, p); break;
      default: hipLaunchKernelGGL(decode_split_bf16<128>, grid, block, 0, stream, p); break;
    }
  } else {
    switch (rank_bound) {
      case 32: hipLaunchKernelGGL(decode_split_f32<32>, grid, block, 0, stream, p); break;
      case 64: hipLaunchKernelGGL(decode_split_f32<64>, grid, block, 0, stream, p); break;
      case 96: hipLaunchKernelGGL(decode_split_f32<96>, grid, block, 0, stream, p); break;
      default: hipLaunchKernelGGL(decode_split_f32<128>, grid, block, 0, stream, p); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(decode_merge, dim3(p.Hq, p.B), dim3(kMergeThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kvlr
