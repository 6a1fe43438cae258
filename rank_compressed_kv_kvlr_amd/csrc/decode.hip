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
// KV head, group of <= 4 query heads sharing it, batch row). The waves take
// the split's token steps round robin and keep a running max / sum /
// weighted latent sum (online softmax, base-2 domain); the workgroup merges
// its 4 waves into one partial record (m, l, o_lat[r_v]) per query head. In
// the single-launch form the workgroup that finishes last for its group
// merges the records of all splits with log-sum-exp weights and applies
// P_V^T (finish_split); the two-stage form leaves the records to decode_merge.
//
// bf16 latents (decode_split_bf16): both products on MFMA. Scores are formed
// transposed, S^T = K_lat q~^T, with the key rows as the A operand straight
// from HBM (operand-order layout, 16 contiguous bytes per lane) and q~ as B
// in a high and a low bf16 part, so a lane ends with 4 consecutive tokens of
// one query head: the A operand of the value product, whose value rows are
// stored in its B-operand order. 4/3-bit latents (decode_split_q43): keys on
// MFMA from the stored codes, values on VALU. fp32 latents
// (decode_split_f32): VALU throughout.
#include "decode_common.hpp"

namespace kvlr {
namespace {

// Largest number of 64-lane value loads per tile of `tile` tokens over ranks r <= rb
// (multiples of 16): a row has r/8 chunks of 8 channels, a load instruction
// covers floor(64 / (r/8)) rows.
constexpr int value_iters_bound(int rb, int tile) {
  int worst = 0;
  for (int r = 16; r <= rb; r += 16) {
    const int rpi = 64 / (r / 8);
    const int it = (tile + rpi - 1) / rpi;
    worst = it > worst ? it : worst;
  }
  return worst;
}

// Merge of the 4 waves' states into one record per head.
//   wm, wl: [4 waves][4 heads]; red: per-wave per-lane partial sums laid out by
//   the caller; value(w, g, j) returns wave w's unnormalised latent sum for
//   head g, channel j.
template <typename ValueFn>
__device__ __forceinline__ void merge_waves_and_store(const RecLayout& rl, int k, int gpw, int rv, const float* wm,
                                                      const float* wl, ValueFn value) {
  for (int idx = thread_id(); idx < gpw * rv; idx += blockDim.x) {
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
    float* rec = rec_at(rl, k, g);
    store_rec(rec + 2 + j, o);
    if (j == 0) {
      store_rec(rec, M);
      store_rec(rec + 1, L);
    }
  }
}

// ---------------------------------------------------------------------------
// merge in the last split workgroup of a group (single-launch decode)
// ---------------------------------------------------------------------------
// Every split workgroup of a (batch row, KV head, head group) counts its
// arrival after its records are complete (s_waitcnt 0 + barrier: the sc1
// stores have reached the coherence point); the workgroup that arrives last
// merges the records and applies P_V^T, then resets the counter, so every
// completed call leaves the counters at zero.
//   wave g merges head g: one pass over the records with a running maximum;
//   then o[dd] = sum_j o_lat[j] P_V[dd][j]. For head_dim <= 128 the basis is
//   already in registers (prefetched when the split work ended): each thread
//   forms partial sums over its 4-column slices for its 8 rows and 4 heads,
//   and the 16 lanes of a DPP row add them up. Larger head dims stage P_V
//   rows through LDS.
constexpr int kTailLds = 12288;   // floats of LDS a split kernel provides for the merge tail

// P_V[h] in registers for head_dim <= 128 (256 threads): thread t holds rows
// t/16 + 16 k (k < 8) and the 4-column slices t%16 and, when r_v > 64,
// t%16 + 16. The workgroup that turns out to merge has the basis on chip.
template <int RB>
struct BasisPrefetch {
  static constexpr int kS = RB > 64 ? 2 : 1;   // column slices per thread
  float4 v[8][kS];
};

template <int RB>
__device__ __forceinline__ void prefetch_basis(const DecodeParams& p, int h, int rv, BasisPrefetch<RB>& pf) {
  if (!p.fuse || p.out_latent || p.d > 128) return;
  const float* P = p.pv + (size_t)p.d * p.ht.rv_pre[h];
  const int m = thread_id() & 15, rg = thread_id() >> 4;
  const int per_row4 = rv >> 2;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int sl = 0; sl < BasisPrefetch<RB>::kS; ++sl) {
      const int r = rg + 16 * k, c4 = m + 16 * sl;
      pf.v[k][sl] = (r < p.d && c4 < per_row4) ? *reinterpret_cast<const float4*>(P + (size_t)r * rv + 4 * c4)
                                                : make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

template <int RB>
__device__ __forceinline__ void finish_split(const DecodeParams& p, int b, int h, int hg, int hq0, int gpw,
                                             int rv, float* scratch, const BasisPrefetch<RB>& pf,
                                             const RecLayout& rl, int n_rec) {
  if (!p.fuse) return;
  int* flag = reinterpret_cast<int*>(scratch + kTailLds - 1);
  int* counter = p.counters + ((size_t)b * p.Hkv + h) * p.n_head_groups + hg;
  // Hand-off between workgroups without a release/acquire fence. This relies on
  // gfx950 behaviour that the HIP memory model does not promise at relaxed order:
  //  - the records are agent-scope relaxed stores (store_rec), which compile to
  //    global stores with the sc1 bit: they write through to the device-coherent
  //    level rather than staying in this XCD's L2;
  //  - s_waitcnt(0) returns only once every such store is acknowledged, and the
  //    barrier makes that true for all waves before thread 0 counts the arrival;
  //  - the merging workgroup reads the records with agent-scope relaxed loads
  //    (load_rec, sc1: they bypass non-coherent cached copies).
  // A release fence per workgroup (buffer_wbl2 sc1, a writeback of the whole L2)
  // gives the same ordering at a measured cost of 16-63 us per call.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (thread_id() == 0)
    *flag = (__hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n_rec - 1);
  __syncthreads();
  if (*flag == 0) return;

  const int tid = thread_id(), lane = tid & 63, g = tid >> 6;
  const int d = p.d;
  const bool reg_basis = d <= 128;              // P_V already in registers (see BasisPrefetch)
  float* olat = scratch;                        // [RB][4] head-minor
  float* p_lds = scratch + 4 * RB;              // P_V rows, padded stride (head_dim > 128)
  const int pst = rv + 4;
  const int p_rows = min(d, (kTailLds - 4 * RB - 16) / pst);
  const float* P = p.pv + (size_t)d * p.ht.rv_pre[h];
  const int per_row4 = rv / 4;
  auto stage_basis = [&](int r0, int nr) {      // rows [r0, r0 + nr) into LDS
    for (int i = tid; i < nr * per_row4; i += blockDim.x) {
      const int r = i / per_row4, c4 = i - r * per_row4;
      *reinterpret_cast<float4*>(p_lds + r * pst + 4 * c4) =
          *reinterpret_cast<const float4*>(P + (size_t)(r0 + r) * rv + 4 * c4);
    }
  };
  if (!p.out_latent && !reg_basis) stage_basis(0, p_rows);   // in flight with the record loads below

  // wave g folds the records of head g in one pass with a running maximum
  float M = kNegInf, L = 0.f, o0 = 0.f, o1 = 0.f;
  if (g < gpw) {
    for (int s0 = 0; s0 < n_rec; s0 += 8) {
      float ms[8], ls[8], v0[8], v1[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool ok = s0 + u < n_rec;
        const float* r = rec_at(rl, ok ? s0 + u : 0, g);
        ms[u] = ok ? load_rec(r) : kNegInf;
        ls[u] = ok ? load_rec(r + 1) : 0.f;
        v0[u] = (ok && lane < rv) ? load_rec(r + 2 + lane) : 0.f;
        v1[u] = (ok && lane + 64 < rv) ? load_rec(r + 66 + lane) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (ms[u] == kNegInf) continue;   // empty split or beyond n_splits
        const float Mn = fmaxf(M, ms[u]);
        const float a = fast_exp2(M - Mn), f = fast_exp2(ms[u] - Mn);
        L = fmaf(L, a, f * ls[u]);
        o0 = fmaf(o0, a, f * v0[u]);
        o1 = fmaf(o1, a, f * v1[u]);
        M = Mn;
      }
    }
  }
  const float inv = (g < gpw && L > 0.f) ? 1.f / L : 0.f;   // empty sequence or idle head: zero
  if (p.out_latent) {
    // folded mode: the caller applies P_V^T (absorbed into its output projection)
    if (g < gpw) {
      float* o = p.out + ((size_t)b * p.Hq + hq0 + g) * p.out_stride;
      if (lane < p.out_stride) o[lane] = o0 * inv;
      if (lane + 64 < p.out_stride) o[lane + 64] = o1 * inv;
    }
    __syncthreads();
    if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if (lane < RB) olat[lane * 4 + g] = o0 * inv;
  if (lane + 64 < RB) olat[(lane + 64) * 4 + g] = o1 * inv;
  __syncthreads();

  if (reg_basis) {
    // back-projection from registers: partial sums over this thread's column slices,
    // then a sum over the 16 lanes of the DPP row (which share the rows)
    const int m = tid & 15, rg = tid >> 4;
    float part[8][4];
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) part[k][gg] = 0.f;
#pragma unroll
    for (int sl = 0; sl < BasisPrefetch<RB>::kS; ++sl) {
      const int c4 = m + 16 * sl;
      if (c4 < per_row4) {
        float4 o[4];   // o_lat of channels 4 c4 .. 4 c4 + 3, four heads each
#pragma unroll
        for (int c = 0; c < 4; ++c) o[c] = *reinterpret_cast<const float4*>(olat + (4 * c4 + c) * 4);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float4 pv = pf.v[k][sl];
          part[k][0] += pv.x * o[0].x + pv.y * o[1].x + pv.z * o[2].x + pv.w * o[3].x;
          part[k][1] += pv.x * o[0].y + pv.y * o[1].y + pv.z * o[2].y + pv.w * o[3].y;
          part[k][2] += pv.x * o[0].z + pv.y * o[1].z + pv.z * o[2].z + pv.w * o[3].z;
          part[k][3] += pv.x * o[0].w + pv.y * o[1].w + pv.z * o[2].w + pv.w * o[3].w;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) part[k][gg] = row16_allreduce<false>(part[k][gg]);
    // lane m of the row stores outputs (k, head) with (4 k + head) % 16 == m
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int r = rg + 16 * k;
        if (((4 * k + gg) & 15) == m && gg < gpw && r < d)
          p.out[((size_t)b * p.Hq + hq0 + gg) * d + r] = part[k][gg];
      }
    if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }

  // back-projection of the 4 heads, P_V rows from LDS (restaged when they do not fit)
  for (int r0 = 0; r0 < d; r0 += p_rows) {
    const int nr = min(p_rows, d - r0);
    if (r0 > 0) {
      __syncthreads();
      stage_basis(r0, nr);
      __syncthreads();
    }
    for (int r = tid; r < nr; r += blockDim.x) {
      float acc[kHeadsPerWg] = {0.f, 0.f, 0.f, 0.f};
      const float* prow = p_lds + r * pst;
#pragma unroll 2
      for (int j = 0; j < rv; j += 4) {
        const float4 pj = *reinterpret_cast<const float4*>(prow + j);
        const float pk[4] = {pj.x, pj.y, pj.z, pj.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float4 ol = *reinterpret_cast<const float4*>(olat + (j + e) * 4);
          acc[0] = fmaf(ol.x, pk[e], acc[0]);
          acc[1] = fmaf(ol.y, pk[e], acc[1]);
          acc[2] = fmaf(ol.z, pk[e], acc[2]);
          acc[3] = fmaf(ol.w, pk[e], acc[3]);
        }
      }
#pragma unroll
      for (int gg = 0; gg < kHeadsPerWg; ++gg)
        if (gg < gpw) p.out[((size_t)b * p.Hq + hq0 + gg) * d + r0 + r] = acc[gg];
    }
  }
  if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// fused append: new latent rows written by the workgroup that reads them
// ---------------------------------------------------------------------------
// One decode step of autoregressive generation appends the new token's row and
// attends over it (StiefAttention technical summary, "Definição do Problema": the
// cache grows by one row per generated token). In the fused form the workgroups
// whose split holds row pos[b] form the new latent rows themselves (thread j < 128:
// key channel j, thread 128 + j: value channel j; fp32 dot products over d in the
// order of the append kernel, rounded to bf16), store them, and wait until the
// stores are acknowledged before any of their waves loads a tile, so the row is
// read back from L2. No other workgroup reads that row. With several head groups
// per KV head every group's workgroup writes the same bytes.
__device__ __forceinline__ bool append_owner(const DecodeParams& p, int b, int h, int s) {
  if (p.app_k == nullptr) return false;
  const int pos = p.pos[b];
  return pos >= 0 && pos < p.cap && pos / p.ht.split_len[h] == s;
}

__device__ void append_rows(const DecodeParams& p, int b, int h, int rk, int rv, float* xs) {
  const int d = p.d, tid = thread_id();
  const int pos = p.pos[b];
  for (int i = tid; i < 2 * d; i += blockDim.x) {   // k_new row to xs[0, d), v_new row to xs[256, 256 + d)
    const int kind = i >= d, ii = i - kind * d;
    const void* X = kind ? p.v_new : p.k_new;
    const size_t src = ((size_t)b * p.Hkv + h) * d + ii;
    xs[kind * 256 + ii] = p.in_bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(X)[src])
                                    : static_cast<const float*>(X)[src];
  }
  __syncthreads();
  const int kind = tid >> 7, j = tid & 127;
  const int r = kind ? rv : rk;
  if (j < r) {
    const float* P = (kind ? p.pv : p.pk) + (size_t)d * (kind ? p.ht.rv_pre[h] : p.ht.rk_pre[h]);
    const float* x = xs + kind * 256;
    float acc = 0.f;
    for (int i = 0; i < d; ++i) acc = fmaf(x[i], P[(size_t)i * r + j], acc);
    const size_t rows = cap_rows_of(p.cap);
    if (kind == 0) {
      uint16_t* K = static_cast<uint16_t*>(p.app_k) + rows * ((size_t)b * p.Sk + p.ht.sk_pre[h]);
      K[k_tiled_offset(pos, j, rk)] = f32_to_bf16_bits(acc);
    } else {
      uint16_t* V = static_cast<uint16_t*>(p.app_v) + rows * ((size_t)b * p.Sv + p.ht.sv_pre[h]);
      V[v_joint_offset(pos, j, rv)] = f32_to_bf16_bits(acc);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // the new rows are in L2 before any wave of this workgroup loads a tile
  __syncthreads();
}

// ---------------------------------------------------------------------------
// bf16 latents: scores and value mix on MFMA
// ---------------------------------------------------------------------------
// RB: rank bound (32, 64, 96 or 128) sizing the register tiles; the actual
// per-head ranks are runtime values <= RB (multiples of 16).
// TT: tokens per wave step (16 or 32), i.e. TT/16 blocks of 16 tokens.
// Waves take TT-token steps of the split round robin. Per 16-token block:
//  - scores transposed, S^T = K_lat q~^T (v_mfma_f32_16x16x32_bf16, key rows as
//    the A operand straight from HBM in their operand-order layout, q~ as B with
//    the workgroup's query heads in columns 0..3, a high and a low bf16 part);
//    a 16-channel tail uses v_mfma_f32_16x16x16_bf16. Lane (n, q) then holds
//    tokens 4q .. 4q + 3 of query head n;
//  - online softmax per query head in the log2 domain (in-lane over 4 tokens,
//    then two cross-lane steps);
//  - value product o_lat[head][ch] += p V_lat on v_mfma_f32_16x16x16_bf16: the
//    softmax weights are already the A operand (tokens as the reduction
//    dimension; high and low bf16 parts), the value rows are stored in that
//    product's B-operand order (v_joint_offset), 16 bytes per lane per channel
//    pair. Value rows past the sequence end may hold any bits and are zeroed.
// The waves' states meet in LDS and leave one record per query head and split.
// One segment [t_begin, t_end) of the sequence of (batch row b, KV head h, head
// group hg): stream it, leave record k of the group's records rl, and, in the
// single-launch form, take part in the group's merge of its n_rec records.
template <int RB, int TT>
__device__ __forceinline__ void bf16_segment(const DecodeParams& p, int b, int h, int hg, int t_begin, int t_end,
                                             const RecLayout& rl, int k, int n_rec, float* smem) {
  constexpr int NB = TT / 16;
  constexpr int NP = RB / 32;                 // key channel pairs bound
  constexpr int kVP = RB / 32;                // value channel pairs bound (a tail fills half a pair)
  constexpr int kCT = RB / 16;                // value column tiles bound
  constexpr int QTS = RB;                     // q~ LDS row stride

  const int hq0 = h * p.G + hg * kHeadsPerWg;
  const int gpw = min(kHeadsPerWg, p.G - hg * kHeadsPerWg);
  const int rk = p.ht.rk[h], rv = p.ht.rv[h];
  if (t_begin >= t_end) {
    write_empty_records(rl, k, gpw, rv);
    BasisPrefetch<RB> pf;
    prefetch_basis<RB>(p, h, rv, pf);
    finish_split<RB>(p, b, h, hg, hq0, gpw, rv, smem, pf, rl, n_rec);
    return;
  }

  const int tid = thread_id(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, q4 = lane >> 4;
  const int np = rk >> 5, ktail = (rk >> 4) & 1;
  const int vnp = rv >> 5, vtail = (rv >> 4) & 1;
  const size_t rows = cap_rows_of(p.cap);
  const uint16_t* Kb = static_cast<const uint16_t*>(p.lat_k) + rows * ((size_t)b * p.Sk + p.ht.sk_pre[h]);
  const uint16_t* Vb = static_cast<const uint16_t*>(p.lat_v) + rows * ((size_t)b * p.Sv + p.ht.sv_pre[h]);

  // blocks wholly past the valid rows re-read the last valid block; their tokens are masked
  const int last_blk = (t_end - 1) >> 4;
  u32x4_t kreg[NB][NP];
  u32x2_t ktl[NB];
  u32x4_t vreg[NB][kVP];
  auto load_k = [&](int t0) {
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const uint16_t* kb = Kb + (size_t)min((t0 >> 4) + blk, last_blk) * 16 * rk;
#pragma unroll
      for (int pp = 0; pp < NP; ++pp)
        if (pp < np) kreg[blk][pp] = load_stream16(kb + pp * 512 + lane * 8);
      if (ktail) ktl[blk] = load_stream8(kb + np * 512 + lane * 4);
    }
  };
  auto load_v = [&](int t0) {
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const uint16_t* vb = Vb + (size_t)min((t0 >> 4) + blk, last_blk) * 16 * rv;
#pragma unroll
      for (int c = 0; c < kVP; ++c) {
        if (c < vnp) {
          vreg[blk][c] = load_stream16(vb + c * 512 + lane * 8);
        } else if (c == vnp && vtail) {
          const u32x2_t t = load_stream8(vb + vnp * 512 + lane * 4);
          vreg[blk][c] = u32x4_t{t.x, t.y, 0u, 0u};
        } else {
          vreg[blk][c] = u32x4_t{0u, 0u, 0u, 0u};   // channels past the rank: the products stay zero
        }
      }
    }
  };

  // the first step's loads do not depend on q~: issue them before the prologue
  int t0 = t_begin + wave * TT;
  if (t0 < t_end) {
    load_k(t0);
    load_v(t0);
  }

  // ---- prologue: q~ into LDS, then this lane's query head as B operands (hi/lo)
  float* q_lds = smem;                          // [4][d]  (d <= 256)
  float* qt_lds = smem + kHeadsPerWg * 256;     // [4][QTS]
  float* qred = qt_lds + kHeadsPerWg * QTS;     // [4 waves][4][QTS]
  project_query<RB>(p, b, h, hq0, gpw, rk, q_lds, qred, qt_lds);
  const bool q_ok = n16 < gpw;
  const int qrow = q_ok ? n16 : 0;
  bf16x8_t a_hi[NP], a_lo[NP];
  bf16x4_t t_hi, t_lo;
#pragma unroll
  for (int pp = 0; pp < NP; ++pp)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = q_ok ? qt_lds[qrow * QTS + 32 * pp + 8 * q4 + e] : 0.f;   // zero past rk
      const uint16_t hi = f32_to_bf16_bits(x);
      a_hi[pp][e] = (short)hi;
      a_lo[pp][e] = (short)f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
    }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = 32 * np + 4 * q4 + e;
    const float x = (q_ok && ktail) ? qt_lds[qrow * QTS + j] : 0.f;
    const uint16_t hi = f32_to_bf16_bits(x);
    t_hi[e] = (short)hi;
    t_lo[e] = (short)f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
  }
  __syncthreads();   // LDS is reused below

  float m = kNegInf, l = 0.f;
  f32x4_t acc[kCT];
#pragma unroll
  for (int c = 0; c < kCT; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (; t0 < t_end; t0 += kWaves * TT) {
    const int t_next = t0 + kWaves * TT;
    // ---- S^T[token][query head] per block
    f32x4_t sc[NB];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        if (pp < np) {
          const bf16x8_t kb = __builtin_bit_cast(bf16x8_t, kreg[blk][pp]);
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, a_hi[pp], d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, a_lo[pp], d, 0, 0, 0);
        }
      }
      if (ktail) {
        const bf16x4_t kb = __builtin_bit_cast(bf16x4_t, ktl[blk]);
        d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kb, t_hi, d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kb, t_lo, d, 0, 0, 0);
      }
      sc[blk] = d;
    }
    if (t_next < t_end) load_k(t_next);   // key registers are free again

    // ---- online softmax: lane (n16, q4) holds tokens t0 + 16 blk + 4 q4 + i of query head n16
    float mx = kNegInf;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool valid = q_ok && (t0 + 16 * blk + 4 * q4 + i) < t_end;
        sc[blk][i] = valid ? sc[blk][i] : kNegInf;
        mx = fmaxf(mx, sc[blk][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = q_ok ? fast_exp2(m - m_use) : 1.f;
    bf16x4_t p_hi[NB], p_lo[NB];
    float ls = 0.f;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pr = fast_exp2(sc[blk][i] - m_use);   // masked: exp2(-inf) = 0
        ls += pr;
        const uint16_t hi = f32_to_bf16_bits(pr);
        p_hi[blk][i] = (short)hi;
        p_lo[blk][i] = (short)f32_to_bf16_bits(pr - bf16_bits_to_f32(hi));
      }
    l = fmaf(l, alpha, ls);
    m = m_new;
    // accumulator rows are query heads 4 q4 + i; their factors sit in lanes 4 q4 + i
    if (__ballot(alpha != 1.f)) {
      float ar[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * q4 + i, 64);
#pragma unroll
      for (int c = 0; c < kCT; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[c][i] *= ar[i];
    }

    // ---- value product; rows past the sequence end hold arbitrary bits: zeroed
    if (t0 + TT > t_end) {
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
        const int nv = t_end - t0 - 16 * blk - 4 * q4;   // valid tokens among this lane's 4
        const uint32_t m01 = (nv > 0 ? 0xFFFFu : 0u) | (nv > 1 ? 0xFFFF0000u : 0u);
        const uint32_t m23 = (nv > 2 ? 0xFFFFu : 0u) | (nv > 3 ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int c = 0; c < kVP; ++c) {
          vreg[blk][c].x &= m01;
          vreg[blk][c].y &= m23;
          vreg[blk][c].z &= m01;
          vreg[blk][c].w &= m23;
        }
      }
    }
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
      for (int c = 0; c < kVP; ++c) {
        const bf16x4_t v0 = __builtin_bit_cast(bf16x4_t, u32x2_t{vreg[blk][c].x, vreg[blk][c].y});
        const bf16x4_t v1 = __builtin_bit_cast(bf16x4_t, u32x2_t{vreg[blk][c].z, vreg[blk][c].w});
        acc[2 * c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p_hi[blk], v0, acc[2 * c], 0, 0, 0);
        acc[2 * c + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p_hi[blk], v1, acc[2 * c + 1], 0, 0, 0);
        acc[2 * c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p_lo[blk], v0, acc[2 * c], 0, 0, 0);
        acc[2 * c + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p_lo[blk], v1, acc[2 * c + 1], 0, 0, 0);
      }
    if (t_next < t_end) load_v(t_next);
  }

  BasisPrefetch<RB> pf;
  prefetch_basis<RB>(p, h, rv, pf);
  // ---- workgroup merge of the 4 waves: rows 0..3 of each wave's accumulators (q4 = 0 lanes)
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  float* red = smem;                          // [wave][head][RB]
  float* wm = smem + kWaves * kHeadsPerWg * RB;
  float* wl = wm + kWaves * kHeadsPerWg;
  if (q4 == 0) {
    const int n_ct = rv >> 4;
#pragma unroll
    for (int c = 0; c < kCT; ++c)
      if (c < n_ct)
#pragma unroll
        for (int i = 0; i < kHeadsPerWg; ++i) red[(wave * kHeadsPerWg + i) * RB + 16 * c + n16] = acc[c][i];
    if (n16 < kHeadsPerWg) {
      wm[wave * kHeadsPerWg + n16] = m;
      wl[wave * kHeadsPerWg + n16] = l;
    }
  }
  __syncthreads();
  merge_waves_and_store(rl, k, gpw, rv, wm, wl,
                        [&](int w, int g, int j) { return red[(w * kHeadsPerWg + g) * RB + j]; });
  finish_split<RB>(p, b, h, hg, hq0, gpw, rv, smem, pf, rl, n_rec);
}

// Values equal in every lane, made wave-uniform for the compiler (scalar registers).
__device__ __forceinline__ int uniform32(int x) { return __builtin_amdgcn_readfirstlane(x); }

// floor(a / b) for 0 <= a < 2^62 and 0 < b: a double-precision quotient (within one
// of the exact one for every operand here) corrected with the remainder; far fewer
// instructions than a 64-bit integer division.
__device__ __forceinline__ long long div64(long long a, long long b) {
  long long q = (long long)((double)a / (double)b);
  long long r = a - q * b;
  while (r < 0) {
    --q;
    r += b;
  }
  while (r >= b) {
    ++q;
    r -= b;
  }
  return q;
}

// Lane `src` (wave-uniform) of a 64-bit value, as a wave-uniform value.
__device__ __forceinline__ long long readlane64(long long x, int src) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(x & 0xFFFFFFFFll), src);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(x >> 32), src);
  return (long long)(((unsigned long long)hi << 32) | lo);
}

// 64-bit shuffle up by d lanes (two 32-bit halves).
__device__ __forceinline__ long long shfl_up64(long long x, int d) {
  const int lo = __shfl_up((int)(unsigned)(x & 0xFFFFFFFFll), d, 64);
  const int hi = __shfl_up((int)(x >> 32), d, 64);
  return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

// Balanced plan: the call's work W = sum_b T_b * row_cost (row_cost = sum over the
// (KV head, head group) units of a batch row of cost[h], the work of one token:
// its latent elements r_k + r_v plus a fixed part for the per-step arithmetic)
// is cut into P = gridDim.x equal shares [w W / P, (w + 1) W / P) along
// the units in (b, h, hg) order. A share may span several units and a unit
// several shares; inside a unit the cuts fall on multiples of kBalancedTokens
// tokens, computed the same way by both neighbours. Workgroup w streams its
// segment of every unit it meets and leaves a record in slot w_first(u) + u + k,
// where w_first(u) is the first workgroup whose share meets unit u; the last
// workgroup to arrive for a unit merges its records. Batch rows without tokens
// get zero output rows from workgroup b % P. The plan reads seq_lens on the
// device and depends on nothing else, so every run gives the same result.
constexpr int kBalancedTokens = 128;

template <int RB, int TT>
__device__ __forceinline__ void decode_balanced(const DecodeParams& p, float* smem) {
  const int tid = thread_id(), lane = tid & 63;
  const int B = p.B, w = blockIdx.x;
  const long long C = p.row_cost;
  // Every wave works out the plan on its own, from the clamped lengths 64 rows at a
  // time (an inclusive scan across the lanes), so the plan needs no LDS and no barrier.
  auto len_of = [&](int bi) { return bi < B ? (long long)min(max(p.seq_lens[bi], 0), p.cap) : 0ll; };
  auto scan = [&](long long v) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long y = shfl_up64(v, off);
      if (lane >= off) v += y;
    }
    return v;
  };
  long long total = 0;
  for (int c0 = 0; c0 < B; c0 += 64) total += readlane64(scan(len_of(c0 + lane)), 63);
  const long long W = total * C;
  for (int b = w; b < B; b += gridDim.x) {   // rows without tokens: zero outputs
    if (len_of(b) == 0) {
      const int n = p.Hq * p.out_stride;
      float* o = p.out + (size_t)b * n;
      for (int i = tid; i < n; i += blockDim.x) o[i] = 0.f;
    }
  }
  const long long P = min((long long)gridDim.x, W);   // every share non-empty
  if (w >= P) return;
  const long long x0 = div64(w * W, P), x1 = div64((w + 1) * W, P);
  // the unit holding x0: its batch row is the last one whose rows before it hold
  // at most x0 / C work (a row with tokens, since x0 < W)
  int b = -1;
  long long row0 = 0;
  int T = 0;
  long long carry = 0;
  for (int c0 = 0; c0 < B; c0 += 64) {
    const long long v = len_of(c0 + lane);
    const long long incl = scan(v);
    const long long excl = carry + incl - v;
    const unsigned long long m = __ballot(c0 + lane < B && excl * C <= x0);
    if (m) {
      const int last = 63 - __builtin_clzll(m);
      b = c0 + last;
      row0 = readlane64(excl, last) * C;
      T = (int)readlane64(v, last);
    }
    carry += readlane64(incl, 63);
  }
  b = uniform32(b);
  T = uniform32(T);
  const int n_hg = p.n_head_groups;
  const long long v0 = div64(x0 - row0, T);   // position along the row's per-token cost axis
  // its KV head: the last h with n_hg cost_pre[h] <= v0 (one load per lane, then a ballot)
  const unsigned long long hm =
      __ballot(lane < p.Hkv && (long long)n_hg * p.ht.cost_pre[lane < p.Hkv ? lane : 0] <= v0);
  int h = uniform32(63 - __builtin_clzll(hm));
  int hg = (int)div64(v0 - (long long)n_hg * p.ht.cost_pre[h], p.ht.cost[h]);
  hg = min(hg, n_hg - 1);
  // The walk over units keeps its state in LDS between segments: held in registers
  // across the whole segment body, it would push the kernel past its scalar registers.
  __shared__ long long st_row0, st_x[4];   // st_x: x0, x1, W, P
  __shared__ int st_b, st_T, st_h, st_hg;
  if (tid == 0) {
    st_x[0] = x0;
    st_x[1] = x1;
    st_x[2] = W;
    st_x[3] = P;
    st_row0 = row0;
    st_b = b;
    st_T = T;
    st_h = h;
    st_hg = hg;
  }
  __syncthreads();
  for (;;) {
    b = st_b;
    T = st_T;
    h = st_h;
    hg = st_hg;
    row0 = st_row0;
    const long long x0 = st_x[0], x1 = st_x[1], W = st_x[2], P = st_x[3];
    const int ch = p.ht.cost[h];
    const long long S = row0 + (long long)T * ((long long)n_hg * p.ht.cost_pre[h] + (long long)hg * ch);
    if (S >= x1) return;
    const long long Wu = (long long)T * ch;
    auto tok = [&](long long x) {   // token boundary of work position x inside this unit
      if (x <= S) return 0;
      long long t = div64(x - S + ch - 1, ch);
      t = (t + kBalancedTokens - 1) / kBalancedTokens * kBalancedTokens;
      return (int)min(t, (long long)T);
    };
    const int ta = tok(max(x0, S)), te = tok(min(x1, S + Wu));
    const long long wf = div64((S + 1) * P - 1, W), wl = div64((S + Wu) * P - 1, W);
    const long long u = ((long long)b * p.Hkv + h) * n_hg + hg;
    const RecLayout rl{p.ws + (size_t)(wf + u) * kHeadsPerWg * p.ws_stride, (size_t)kHeadsPerWg * p.ws_stride,
                       (size_t)p.ws_stride};
    __syncthreads();   // every thread has read the state; the previous segment's LDS reads are done
    if (tid == 0) {    // the next unit: head group, KV head, then the next batch row with tokens
      int nb = b, nT = T, nh = h, nhg = hg + 1;
      long long nrow0 = row0;
      if (nhg == n_hg) {
        nhg = 0;
        if (++nh == p.Hkv) {
          nh = 0;
          do {
            nrow0 += (long long)nT * C;
            if (++nb >= B) break;
            nT = min(max(p.seq_lens[nb], 0), p.cap);
          } while (nT == 0);
          if (nb >= B) nrow0 = x1;   // past the end: the next S >= x1 stops the walk
        }
      }
      st_b = min(nb, B - 1);
      st_T = nT;
      st_h = nh;
      st_hg = nhg;
      st_row0 = nrow0;
    }
    bf16_segment<RB, TT>(p, b, h, hg, ta, te, rl, (int)(w - wf), (int)(wl - wf + 1), smem);
  }
}

// Fixed plan: one workgroup per (split, KV head and head group, batch row).
template <int RB, int TT>
__global__ __launch_bounds__(256) void decode_split_bf16(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) float smem[kTailLds];
  const int s = blockIdx.x;
  const int h = blockIdx.y / p.n_head_groups;
  const int hg = blockIdx.y - h * p.n_head_groups;
  const int b = blockIdx.z;
  const int T = min(max(p.seq_lens[b], 0), p.cap);
  const int t_begin = min(s * p.ht.split_len[h], T);   // clamped: no overflow for far splits
  const int t_end = min(T, t_begin + p.ht.split_len[h]);
  if (append_owner(p, b, h, s)) append_rows(p, b, h, p.ht.rk[h], p.ht.rv[h], smem);
  bf16_segment<RB, TT>(p, b, h, hg, t_begin, t_end, fixed_records(p, b, h * p.G + hg * kHeadsPerWg), s,
                       p.n_splits, smem);
}

// Balanced plan: one workgroup per share.
template <int RB, int TT>
__global__ __launch_bounds__(256) void decode_balanced_bf16(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) float smem[kTailLds];
  decode_balanced<RB, TT>(p, smem);
}

// ---------------------------------------------------------------------------
// 4/3-bit latents (STAR-KV technical summary, "Metodologia" section 3): keys on
// MFMA, values on VALU, both read as stored codes
// ---------------------------------------------------------------------------
// A wave streams ST consecutive rows of keys and of values per iteration with
// 16-byte loads (the rows of a (batch row, KV head) block are contiguous and a
// tile starts 16-byte aligned), parks them in its own LDS region while the
// next ST rows are in flight, and reads the codes it needs from LDS. For ranks
// up to 64 the tile is one 32-token step (ST = 32), which keeps the kernel
// within 168 registers, i.e. 3 waves per SIMD and 3 workgroups per CU. The
// kernel is bound by VALU work and latency, so the third workgroup gains more
// than the deeper tile. Larger ranks would spill at that size and keep
// 64-row tiles at 2 waves per SIMD.
// Scores: a code c enters the MFMA as the bf16 number 128 + c (bits 0x4300 | c,
// exact), so per token and block of channels
//   sum_j q~_j (step c_j + base) = step (acc - 128 Q) + base Q,
// with acc = sum_j q~_j (128 + c_j) from the MFMA and Q = sum_j q~_j over the
// block, q~ as the MFMA sees it (high plus low bf16 part). Outlier slices hold
// 16 channels (16x16x16), inlier slices 32 (16x16x32) plus a 16-channel tail.
// Values: a lane owns 8 channels of a row, all inside one block, and
// accumulates sum_t p_t step_t c_t per channel and sum_t p_t base_t once per
// head; the two are added when the split ends.
template <int RB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(RB <= 64 ? 3 : 1)))
void decode_split_q43(DecodeParams p) {
  constexpr int TT = 32;                     // tokens per score/softmax/value step
  constexpr int NB = TT / 16;
  constexpr int ST = RB <= 64 ? 32 : 64;     // rows per wave iteration
  constexpr int NSUB = ST / TT;
  constexpr int RBM = q43_row_bytes(RB);     // bytes of the longest row
  constexpr int CH = (ST * RBM + 1023) / 1024;   // 16-byte chunks per lane per tile (keys or values)
  constexpr int MSO = RB == 128 ? 2 : 1;     // outlier 16-channel slices (bound)
  constexpr int MSI = RB > 32 ? (RB - 16) / 32 : 1;   // full 32-channel inlier slices (bound; >= 1)
  constexpr int NIT = value_iters_bound(RB, TT);
  constexpr int QTS = RB;
  constexpr int kRS = 36;                    // per-lane stride of the wave reduction
  constexpr int kStageF = kWaves * ST * 2 * RBM / 4;   // floats of LDS for the staged rows
  static_assert(kStageF + kWaves * TT * 4 <= kTailLds, "staged rows and p tiles must fit the LDS block");
  __shared__ __attribute__((aligned(16))) float smem[kWaves * 64 * kRS + 64 > kTailLds ? kWaves * 64 * kRS + 64 : kTailLds];
  __shared__ float qsum[2][kHeadsPerWg];     // Q of the outlier and inlier key blocks per head

  const int s = blockIdx.x;
  const int h = blockIdx.y / p.n_head_groups;
  const int hg = blockIdx.y - h * p.n_head_groups;
  const int b = blockIdx.z;
  const int hq0 = h * p.G + hg * kHeadsPerWg;
  const int gpw = min(kHeadsPerWg, p.G - hg * kHeadsPerWg);
  const int rk = p.ht.rk[h], rv = p.ht.rv[h];
  const int T = min(max(p.seq_lens[b], 0), p.cap);
  const int t_begin = min(s * p.ht.split_len[h], T);
  const int t_end = min(T, t_begin + p.ht.split_len[h]);
  if (t_begin >= t_end) {
    write_empty_records(fixed_records(p, b, hq0), s, gpw, rv);
    BasisPrefetch<RB> pf;
    prefetch_basis<RB>(p, h, rv, pf);
    finish_split<RB>(p, b, h, hg, hq0, gpw, rv, smem, pf, fixed_records(p, b, hq0), p.n_splits);
    return;
  }

  const int tid = thread_id(), lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, q4 = lane >> 4;

  // ---- key row geometry and this lane's byte offsets inside a row
  const int nok = q43_outlier(rk), nik = rk - nok;
  const int nso = nok >> 4, nsi = nik >> 5, ktail = (nik >> 4) & 1;
  const int rbk = q43_row_bytes(rk);
  const int kib = 8 + nok / 2;                          // inlier bit stream
  const int ko_off = 8 + 4 * (q4 >> 1), ko_sh = 16 * (q4 & 1);
  const int ki_off = kib + 4 * ((24 * q4) >> 5), ki_sh = (24 * q4) & 31;
  const bool ki_two = ki_sh > 8;
  const int kt_off = kib + 4 * (3 * nsi + ((12 * q4) >> 5)), kt_sh = (12 * q4) & 31;
  const bool kt_two = kt_sh > 20;
  // ---- value row geometry: C chunks of 8 channels per row
  const int nov = q43_outlier(rv);
  const int rbv = q43_row_bytes(rv);
  const int C = rv >> 3;
  const int rpi = 64 / C;
  const int ro = lane / C, cch = lane - ro * C;
  const bool v_active = ro < rpi;
  const int n_it = (TT + rpi - 1) / rpi;
  const bool v_out = cch < (nov >> 3);                 // chunk in the 4-bit outlier block
  const int v_meta = v_out ? 0 : 4;
  const int v_bits = v_out ? 4 : 3;
  const int v_bit0 = v_out ? 0 : 24 * (cch - (nov >> 3));
  const int v_off = v_out ? 8 + 4 * cch : 8 + nov / 2 + 4 * (v_bit0 >> 5);
  const int v_sh = v_out ? 0 : v_bit0 & 31;
  const bool v_two = v_sh > 8;

  const size_t rows = cap_rows_of(p.cap);
  const uint8_t* Kb = static_cast<const uint8_t*>(p.lat_k) + rows * ((size_t)b * p.Sk + p.ht.sk_pre[h]);
  const uint8_t* Vb = static_cast<const uint8_t*>(p.lat_v) + rows * ((size_t)b * p.Sv + p.ht.sv_pre[h]);

  // this wave's LDS: staged key rows, staged value rows, then (after all staging) its p tile
  uint8_t* kst = reinterpret_cast<uint8_t*>(smem) + (size_t)wave * ST * 2 * RBM;
  uint8_t* vst = kst + ST * RBM;
  float* p_lds = smem + kStageF + wave * (TT * 4);     // [TT tokens][4 heads]

  float m[4], l[4], acc[4][8], accb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = kNegInf;
    l[i] = 0.f;
    accb[i] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
  }

  // ---- tile streaming: rows [t0, t0 + ST) of keys and values as 16-byte chunks.
  // Chunks past the last valid row's bytes are not read (they never cross the end
  // of the block: it is a multiple of 16 bytes, as is every tile start).
  u32x4_t kraw[CH], vraw[CH];
  int nk_ch = 0, nv_ch = 0;
  auto load_raw = [&](int t0) {
    const int n = min(ST, t_end - t0);
    nk_ch = (n * rbk + 15) >> 4;
    nv_ch = (n * rbv + 15) >> 4;
    const uint8_t* ks = Kb + (size_t)t0 * rbk;
    const uint8_t* vs = Vb + (size_t)t0 * rbv;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ch = c * 64 + lane;
      if (ch < nk_ch) kraw[c] = load_stream16(ks + 16 * ch);
      if (ch < nv_ch) vraw[c] = load_stream16(vs + 16 * ch);
    }
  };
  auto stage_raw = [&]() {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ch = c * 64 + lane;
      if (ch < nk_ch) *reinterpret_cast<u32x4_t*>(kst + 16 * ch) = kraw[c];
      if (ch < nv_ch) *reinterpret_cast<u32x4_t*>(vst + 16 * ch) = vraw[c];
    }
  };
  auto lds32 = [](const uint8_t* ptr) { return *reinterpret_cast<const uint32_t*>(ptr); };

  // the first tile's loads do not depend on q~: issue them before the prologue
  int t0 = t_begin + wave * ST;
  if (t0 < t_end) load_raw(t0);

  // ---- prologue: q~ into LDS, block sums Q, MFMA A operands (hi/lo) into registers
  float* q_lds = smem;                          // [4][d]  (d <= 256)
  float* qt_lds = smem + kHeadsPerWg * 256;     // [4][QTS]
  float* qred = qt_lds + kHeadsPerWg * QTS;     // [4 waves][4][QTS]
  project_query<RB>(p, b, h, hq0, gpw, rk, q_lds, qred, qt_lds);
  if (tid < 2 * kHeadsPerWg) {
    const int g = tid & 3, region = tid >> 2;
    const int j1 = region ? rk : nok;
    float Q = 0.f;
    for (int j = region ? nok : 0; j < j1; ++j) {
      const float x = qt_lds[g * QTS + j];
      const uint16_t hi = f32_to_bf16_bits(x);
      const uint16_t lo = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
      Q += bf16_bits_to_f32(hi) + bf16_bits_to_f32(lo);
    }
    qsum[region][g] = Q;
  }
  auto qt_at = [&](int j, bool valid) { return (n16 < kHeadsPerWg && valid) ? qt_lds[n16 * QTS + j] : 0.f; };
  auto bf_hi = [](float x) { return (short)f32_to_bf16_bits(x); };
  auto bf_lo = [](float x) { return (short)f32_to_bf16_bits(x - bf16_bits_to_f32(f32_to_bf16_bits(x))); };
  bf16x4_t ao_hi[MSO], ao_lo[MSO], at_hi, at_lo;
  bf16x8_t ai_hi[MSI], ai_lo[MSI];
#pragma unroll
  for (int sl = 0; sl < MSO; ++sl)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = qt_at(16 * sl + 4 * q4 + e, sl < nso);
      ao_hi[sl][e] = bf_hi(x);
      ao_lo[sl][e] = bf_lo(x);
    }
#pragma unroll
  for (int sl = 0; sl < MSI; ++sl)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = qt_at(nok + 32 * sl + 8 * q4 + e, sl < nsi);
      ai_hi[sl][e] = bf_hi(x);
      ai_lo[sl][e] = bf_lo(x);
    }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float x = qt_at(nok + 32 * nsi + 4 * q4 + e, ktail != 0);
    at_hi[e] = bf_hi(x);
    at_lo[e] = bf_lo(x);
  }
  __syncthreads();   // LDS is reused below
  float Qo[4], Qi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    Qo[i] = qsum[0][i];
    Qi[i] = qsum[1][i];
  }
  if (t0 < t_end) stage_raw();

  for (; t0 < t_end; t0 += kWaves * ST) {
    const int t_next = t0 + kWaves * ST;
    const int n_valid = min(ST, t_end - t0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (t_next < t_end) load_raw(t_next);   // in flight while this tile is processed from LDS

    for (int sub = 0; sub < NSUB; ++sub) {
      const int ts = 32 * sub;                 // first row of the step inside the tile
      if (ts >= n_valid) break;
      // ---- scores on MFMA from the codes (128 + c as bf16)
      f32x4_t sc[NB];
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
        const uint8_t* row = kst + min(ts + 16 * blk + n16, n_valid - 1) * rbk;
        f32x4_t ao = {0.f, 0.f, 0.f, 0.f}, ai = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sl = 0; sl < MSO; ++sl) {
          if (sl < nso) {
            const uint32_t x = lds32(row + ko_off + 8 * sl) >> ko_sh;   // 4 nibbles: channels 4 q4 ..
            const uint32_t lo = x & 0x0F0Fu, hi = (x >> 4) & 0x0F0Fu;
            u32x2_t w;
            w.x = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u) | 0x43004300u;
            w.y = __builtin_amdgcn_perm(hi, lo, 0x0C050C01u) | 0x43004300u;
            const bf16x4_t kb = __builtin_bit_cast(bf16x4_t, w);
            ao = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ao_hi[sl], kb, ao, 0, 0, 0);
            ao = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ao_lo[sl], kb, ao, 0, 0, 0);
          }
        }
#pragma unroll
        for (int sl = 0; sl < MSI; ++sl) {
          if (sl < nsi) {
            const uint32_t w0 = lds32(row + ki_off + 12 * sl);
            const uint32_t w1 = ki_two ? lds32(row + ki_off + 12 * sl + 4) : 0u;
            const uint32_t bits = __builtin_amdgcn_alignbit(w1, w0, ki_sh);
            u32x4_t w;
#pragma unroll
            for (int k = 0; k < 4; ++k)
              w[k] = __builtin_amdgcn_ubfe(bits, 6 * k, 3) | (__builtin_amdgcn_ubfe(bits, 6 * k + 3, 3) << 16) |
                     0x43004300u;
            const bf16x8_t kb = __builtin_bit_cast(bf16x8_t, w);
            ai = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ai_hi[sl], kb, ai, 0, 0, 0);
            ai = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ai_lo[sl], kb, ai, 0, 0, 0);
          }
        }
        if (ktail) {
          const uint32_t w0 = lds32(row + kt_off);
          const uint32_t w1 = kt_two ? lds32(row + kt_off + 4) : 0u;
          const uint32_t bits = __builtin_amdgcn_alignbit(w1, w0, kt_sh);
          u32x2_t w;
          w.x = __builtin_amdgcn_ubfe(bits, 0, 3) | (__builtin_amdgcn_ubfe(bits, 3, 3) << 16) | 0x43004300u;
          w.y = __builtin_amdgcn_ubfe(bits, 6, 3) | (__builtin_amdgcn_ubfe(bits, 9, 3) << 16) | 0x43004300u;
          const bf16x4_t kb = __builtin_bit_cast(bf16x4_t, w);
          ai = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(at_hi, kb, ai, 0, 0, 0);
          ai = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(at_lo, kb, ai, 0, 0, 0);
        }
        // block parameters of this lane's token (lanes 0..15 hold heads 0..3)
        const uint32_t m0 = lds32(row), m1 = lds32(row + 4);
        const float so = half_bits_to_f32(m0 & 0xFFFFu), bo = half_bits_to_f32(m0 >> 16);
        const float si = half_bits_to_f32(m1 & 0xFFFFu), bi = half_bits_to_f32(m1 >> 16);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sc[blk][i] = so * (ao[i] - 128.f * Qo[i]) + bo * Qo[i] + si * (ai[i] - 128.f * Qi[i]) + bi * Qi[i];
      }

      // ---- online softmax (as in the bf16 kernel)
      const int tb = t0 + ts;
      float alpha[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float mx = kNegInf;
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
          const bool valid = (tb + 16 * blk + n16) < t_end;
          sc[blk][i] = valid ? sc[blk][i] : kNegInf;
          mx = fmaxf(mx, sc[blk][i]);
        }
        mx = row16_allreduce<true>(mx);
        const float m_new = fmaxf(m[i], mx);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        alpha[i] = fast_exp2(m[i] - m_use);
        float ls = 0.f;
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
          const float pr = fast_exp2(sc[blk][i] - m_use);
          sc[blk][i] = pr;
          ls += pr;
        }
        l[i] = fmaf(l[i], alpha[i], ls);
        m[i] = m_new;
      }
      if (q4 == 0) {
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
          *reinterpret_cast<float4*>(p_lds + (16 * blk + n16) * 4) =
              make_float4(sc[blk][0], sc[blk][1], sc[blk][2], sc[blk][3]);
      }
      float a_s[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a_s[i] = readlane_f(alpha[i], 0);
      if (a_s[0] != 1.f || a_s[1] != 1.f || a_s[2] != 1.f || a_s[3] != 1.f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          accb[i] *= a_s[i];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[i][e] *= a_s[i];
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      // ---- value mix on VALU from the codes
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        if (it < n_it) {
          const int r = it * rpi + ro;
          if (v_active && r < TT) {
            const uint8_t* row = vst + min(ts + r, n_valid - 1) * rbv;
            const float4 pw = *reinterpret_cast<const float4*>(p_lds + r * 4);
            const uint32_t mt = lds32(row + v_meta);
            const float step = half_bits_to_f32(mt & 0xFFFFu), base = half_bits_to_f32(mt >> 16);
            const uint32_t c0 = lds32(row + v_off);
            const uint32_t c1 = v_two ? lds32(row + v_off + 4) : 0u;
            const uint32_t bits = __builtin_amdgcn_alignbit(c1, c0, v_sh);
            accb[0] = fmaf(pw.x, base, accb[0]);
            accb[1] = fmaf(pw.y, base, accb[1]);
            accb[2] = fmaf(pw.z, base, accb[2]);
            accb[3] = fmaf(pw.w, base, accb[3]);
            const float w0 = pw.x * step, w1 = pw.y * step, w2 = pw.z * step, w3 = pw.w * step;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float c = (float)__builtin_amdgcn_ubfe(bits, e * v_bits, v_bits);
              acc[0][e] = fmaf(w0, c, acc[0][e]);
              acc[1][e] = fmaf(w1, c, acc[1][e]);
              acc[2][e] = fmaf(w2, c, acc[2][e]);
              acc[3][e] = fmaf(w3, c, acc[3][e]);
            }
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if (t_next < t_end) stage_raw();   // this tile's LDS reads are done (in order within the wave)
  }
  // the block minimum enters every channel of this lane's chunk once per unit of weight
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] += accb[i];

  BasisPrefetch<RB> pf;
  prefetch_basis<RB>(p, h, rv, pf);
  // ---- workgroup merge of the 4 waves
#pragma unroll
  for (int i = 0; i < 4; ++i) l[i] = row16_allreduce<false>(l[i]);
  __syncthreads();
  float* red = smem;                          // [wave][lane][kRS]
  float* wm = smem + kWaves * 64 * kRS;       // [wave][head]
  float* wl = wm + 16;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; e += 4)
      *reinterpret_cast<float4*>(red + (wave * 64 + lane) * kRS + i * 8 + e) =
          make_float4(acc[i][e], acc[i][e + 1], acc[i][e + 2], acc[i][e + 3]);
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wm[wave * 4 + i] = m[i];
      wl[wave * 4 + i] = l[i];
    }
  }
  __syncthreads();
  merge_waves_and_store(fixed_records(p, b, hq0), s, gpw, rv, wm, wl, [&](int w, int g, int j) {
    const int c = j >> 3, e = j & 7;
    const float* base = red + (w * 64 + c) * kRS + g * 8 + e;
    const int step = C * kRS;
    float sum = 0.f;
#pragma unroll 8
    for (int r = 0; r < rpi; ++r) sum += base[r * step];
    return sum;
  });
  finish_split<RB>(p, b, h, hg, hq0, gpw, rv, smem, pf, fixed_records(p, b, hq0), p.n_splits);
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
  constexpr int SM = RED + kHeadsPerWg * 256 + kHeadsPerWg * RB + 64;
  __shared__ __attribute__((aligned(16))) float smem[SM > kTailLds ? SM : kTailLds];

  const int s = blockIdx.x;
  const int h = blockIdx.y / p.n_head_groups;
  const int hg = blockIdx.y - h * p.n_head_groups;
  const int b = blockIdx.z;
  const int hq0 = h * p.G + hg * kHeadsPerWg;
  const int gpw = min(kHeadsPerWg, p.G - hg * kHeadsPerWg);
  const int rk = p.ht.rk[h], rv = p.ht.rv[h];
  const int T = min(max(p.seq_lens[b], 0), p.cap);
  const int t_begin = min(s * p.ht.split_len[h], T);   // clamped: no overflow for far splits
  const int t_end = min(T, t_begin + p.ht.split_len[h]);
  if (t_begin >= t_end) {
    write_empty_records(fixed_records(p, b, hq0), s, gpw, rv);
    BasisPrefetch<RB> pf;
    prefetch_basis<RB>(p, h, rv, pf);
    finish_split<RB>(p, b, h, hg, hq0, gpw, rv, smem, pf, fixed_records(p, b, hq0), p.n_splits);
    return;
  }
  const int tid = thread_id(), lane = tid & 63, wave = tid >> 6;

  float* red = smem;                                  // [wave][4 heads][RB] at the end
  float* q_lds = smem + RED;                          // [4][d]
  float* qt_lds = q_lds + kHeadsPerWg * 256;          // [4][QTS]
  float* wm = qt_lds + kHeadsPerWg * QTS;             // [wave][head]
  float* wl = wm + 16;
  project_query<RB>(p, b, h, hq0, gpw, rk, q_lds, red, qt_lds);

  const size_t rows = cap_rows_of(p.cap);
  const float* Kb = static_cast<const float*>(p.lat_k) + rows * ((size_t)b * p.Sk + p.ht.sk_pre[h]);
  const float* Vb = static_cast<const float*>(p.lat_v) + rows * ((size_t)b * p.Sv + p.ht.sv_pre[h]);
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
  BasisPrefetch<RB> pf;
  prefetch_basis<RB>(p, h, rv, pf);
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
  merge_waves_and_store(fixed_records(p, b, hq0), s, gpw, rv, wm, wl,
                        [&](int w, int g, int j) { return red[(w * 4 + g) * RB + j]; });
  finish_split<RB>(p, b, h, hg, hq0, gpw, rv, smem, pf, fixed_records(p, b, hq0), p.n_splits);
}

// ---------------------------------------------------------------------------
// merge of split records and back-projection by P_V^T
// ---------------------------------------------------------------------------
// One workgroup per (KV head, group of <= 4 query heads, batch row): the
// group shares its P_V[h] rows. The group's split records and the rows of
// P_V[h] are staged in LDS with all loads issued at once, so the kernel
// costs about one memory round trip. Records are combined with log-sum-exp
// weights exp2(m_s - M); the normalised latent output is back-projected,
// o[dd] = sum_j o_lat[j] P_V[dd][j], one output channel dd per thread.
constexpr int kMergeThreads = 256;
constexpr int kMergeRecLds = 8192;    // floats of staged records (32 KiB)
constexpr int kMergePLds = 16384;     // floats of staged basis rows (64 KiB)

template <int RB>
__global__ __launch_bounds__(kMergeThreads) void decode_merge(MergeParams p) {
  __shared__ __attribute__((aligned(16))) float rec_lds[kMergeRecLds];
  __shared__ __attribute__((aligned(16))) float p_lds[kMergePLds];
  __shared__ __attribute__((aligned(16))) float olat[RB][kHeadsPerWg];   // head-minor
  __shared__ float m_red[kHeadsPerWg][4];
  const int h = blockIdx.x / p.n_head_groups;
  const int hg = blockIdx.x - h * p.n_head_groups;
  const int b = blockIdx.y;
  const int hq0 = h * p.G + hg * kHeadsPerWg;
  const int gpw = min(kHeadsPerWg, p.G - hg * kHeadsPerWg);
  const int rv = p.ht.rv[h];
  const int tid = thread_id(), lane = tid & 63, wave = tid >> 6;
  const int ns = p.n_splits, stride = p.ws_stride, d = p.d;
  const size_t head_stride = (size_t)ns * stride;
  const float* recs = p.ws + ((size_t)b * p.Hq + hq0) * head_stride;
  const int chunk = kMergeRecLds / (kHeadsPerWg * stride);   // splits staged per pass (>= 15)
  const float* P = p.pv + (size_t)d * p.ht.rv_pre[h];
  const int pst = rv + 4;                                    // padded LDS row stride of P_V
  const int p_rows = min(d, kMergePLds / pst);                // rows staged per pass

  auto stage_records = [&](int s0, int nc) {
    const int per_head4 = nc * stride / 4;   // stride is a multiple of 4
    for (int i = tid; i < gpw * per_head4; i += kMergeThreads) {
      const int g = i / per_head4, k4 = i - g * per_head4;
      *reinterpret_cast<float4*>(rec_lds + (size_t)g * chunk * stride + 4 * k4) =
          *reinterpret_cast<const float4*>(recs + g * head_stride + (size_t)s0 * stride + 4 * k4);
    }
  };
  auto stage_basis = [&](int r0, int nr) {
    const int per_row4 = rv / 4;
    for (int i = tid; i < nr * per_row4; i += kMergeThreads) {
      const int r = i / per_row4, c4 = i - r * per_row4;
      *reinterpret_cast<float4*>(p_lds + r * pst + 4 * c4) =
          *reinterpret_cast<const float4*>(P + (size_t)(r0 + r) * rv + 4 * c4);
    }
  };

  // 1. stage records and the first rows of P_V; maximum of the split maxima per head
  const bool one_pass = ns <= chunk;
  if (one_pass) stage_records(0, ns);
  stage_basis(0, p_rows);
  __syncthreads();
#pragma unroll
  for (int g = 0; g < kHeadsPerWg; ++g) {
    float mx = kNegInf;
    if (g < gpw)
      for (int s = tid; s < ns; s += kMergeThreads)
        mx = fmaxf(mx, one_pass ? rec_lds[((size_t)g * chunk + s) * stride] : recs[g * head_stride + (size_t)s * stride]);
    mx = wave_allreduce<true>(mx);
    if (lane == 0) m_red[g][wave] = mx;
  }
  __syncthreads();

  // 2. weighted sum of the split latents: wave g owns head g, lane j channels j, j + 64
  const int g_own = wave;
  const bool own = g_own < gpw;
  const float M = fmaxf(fmaxf(m_red[g_own][0], m_red[g_own][1]), fmaxf(m_red[g_own][2], m_red[g_own][3]));
  float o0 = 0.f, o1 = 0.f, L = 0.f;
  for (int s0 = 0; s0 < ns; s0 += chunk) {
    const int nc = min(chunk, ns - s0);
    if (!one_pass) {
      __syncthreads();
      stage_records(s0, nc);
      __syncthreads();
    }
    if (own && M != kNegInf) {
      const float* r = rec_lds + (size_t)g_own * chunk * stride;
#pragma unroll 4
      for (int s = 0; s < nc; ++s, r += stride) {
        const float f = fast_exp2(r[0] - M);   // empty split: exp2(-inf) = 0
        L = fmaf(f, r[1], L);
        if (lane < rv) o0 = fmaf(f, r[2 + lane], o0);
        if (lane + 64 < rv) o1 = fmaf(f, r[2 + 64 + lane], o1);
      }
    }
  }
  {
    const float inv = (own && L > 0.f) ? 1.f / L : 0.f;   // empty sequence or idle head: zero
    if (lane < RB) olat[lane][g_own] = (lane < rv) ? o0 * inv : 0.f;
    if (lane + 64 < RB) olat[lane + 64][g_own] = (lane + 64 < rv) ? o1 * inv : 0.f;
  }
  __syncthreads();

  // 3. back-projection, P_V rows from LDS (restaged when d * (rv + 4) exceeds the buffer)
  for (int r0 = 0; r0 < d; r0 += p_rows) {
    const int nr = min(p_rows, d - r0);
    if (r0 > 0) {
      __syncthreads();
      stage_basis(r0, nr);
      __syncthreads();
    }
    for (int r = tid; r < nr; r += kMergeThreads) {
      float acc[kHeadsPerWg] = {0.f, 0.f, 0.f, 0.f};
      const float* prow = p_lds + r * pst;
#pragma unroll 2
      for (int j = 0; j < rv; j += 4) {
        const float4 pj = *reinterpret_cast<const float4*>(prow + j);
        const float pk[4] = {pj.x, pj.y, pj.z, pj.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float4 ol = *reinterpret_cast<const float4*>(&olat[j + k][0]);
          acc[0] = fmaf(ol.x, pk[k], acc[0]);
          acc[1] = fmaf(ol.y, pk[k], acc[1]);
          acc[2] = fmaf(ol.z, pk[k], acc[2]);
          acc[3] = fmaf(ol.w, pk[k], acc[3]);
        }
      }
#pragma unroll
      for (int g = 0; g < kHeadsPerWg; ++g)
        if (g < gpw) p.out[((size_t)b * p.Hq + hq0 + g) * d + r0 + r] = acc[g];
    }
  }
}


}  // namespace

hipError_t launch_decode(const DecodeParams& p, int latent_dtype, int rank_bound, int tile, hipStream_t stream) {
  const bool latent_bf16 = latent_dtype == KVLR_BF16;
  const dim3 grid(p.n_splits, p.Hkv * p.n_head_groups, p.B);
  const dim3 block(kWaves * 64);
  if (latent_dtype == KVLR_Q43) {
    switch (rank_bound) {
      case 32: hipLaunchKernelGGL(decode_split_q43<32>, grid, block, 0, stream, p); break;
      case 64: hipLaunchKernelGGL(decode_split_q43<64>, grid, block, 0, stream, p); break;
      case 96: hipLaunchKernelGGL(decode_split_q43<96>, grid, block, 0, stream, p); break;
      default: hipLaunchKernelGGL(decode_split_q43<128>, grid, block, 0, stream, p); break;
    }
    return hipGetLastError();
  }
  if (latent_bf16) {
    if (p.balanced) {   // one workgroup per share of the balanced plan
      const dim3 grid_b(p.n_wg);
      switch (rank_bound) {   // 32-token steps (64 would leave one wave per SIMD at bound 96)
        case 32: hipLaunchKernelGGL((decode_balanced_bf16<32, 32>), grid_b, block, 0, stream, p); break;
        case 64: hipLaunchKernelGGL((decode_balanced_bf16<64, 32>), grid_b, block, 0, stream, p); break;
        case 96: hipLaunchKernelGGL((decode_balanced_bf16<96, 32>), grid_b, block, 0, stream, p); break;
        default: hipLaunchKernelGGL((decode_balanced_bf16<128, 32>), grid_b, block, 0, stream, p); break;
      }
    } else if (tile == 32) {
      switch (rank_bound) {
        case 32: hipLaunchKernelGGL((decode_split_bf16<32, 32>), grid, block, 0, stream, p); break;
        case 64: hipLaunchKernelGGL((decode_split_bf16<64, 32>), grid, block, 0, stream, p); break;
        case 96: hipLaunchKernelGGL((decode_split_bf16<96, 32>), grid, block, 0, stream, p); break;
        default: hipLaunchKernelGGL((decode_split_bf16<128, 32>), grid, block, 0, stream, p); break;
      }
    } else {
      switch (rank_bound) {
        case 32: hipLaunchKernelGGL((decode_split_bf16<32, 64>), grid, block, 0, stream, p); break;
        case 64: hipLaunchKernelGGL((decode_split_bf16<64, 64>), grid, block, 0, stream, p); break;
        case 96: hipLaunchKernelGGL((decode_split_bf16<96, 64>), grid, block, 0, stream, p); break;
        default: hipLaunchKernelGGL((decode_split_bf16<128, 64>), grid, block, 0, stream, p); break;
      }
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

hipError_t launch_merge(const MergeParams& p, int rank_bound, hipStream_t stream) {
  const dim3 grid(p.Hkv * p.n_head_groups, p.B);
  switch (rank_bound) {
    case 32: hipLaunchKernelGGL(decode_merge<32>, grid, dim3(kMergeThreads), 0, stream, p); break;
    case 64: hipLaunchKernelGGL(decode_merge<64>, grid, dim3(kMergeThreads), 0, stream, p); break;
    case 96: hipLaunchKernelGGL(decode_merge<96>, grid, dim3(kMergeThreads), 0, stream, p); break;
    default: hipLaunchKernelGGL(decode_merge<128>, grid, dim3(kMergeThreads), 0, stream, p); break;
  }
  return hipGetLastError();
}


}  // namespace kvlr
