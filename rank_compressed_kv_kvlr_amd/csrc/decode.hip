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
// stored in its B-operand order. 4/3-bit latents (decode_split_q43): the same
// two products on MFMA, fed from the stored codes (tiles in operand order).
// fp32 latents (decode_split_f32): VALU throughout.
#include "decode_common.hpp"

namespace kvlr {
namespace {

// Merge of the waves' states into one record per head.
//   wm, wl: [NW states][4 heads]; red: per-wave per-lane partial sums laid out by
//   the caller; value(w, g, j) returns wave w's unnormalised latent sum for
//   head g, channel j.
//   NW partial states per head (the 4 waves, or 8 where each wave keeps one per
//   16-token block).
template <int NW = kWaves, typename ValueFn>
__device__ __forceinline__ void merge_waves_and_store(const RecLayout& rl, int k, int gpw, int rv, const float* wm,
                                                      const float* wl, ValueFn value) {
  for (int idx = thread_id(); idx < gpw * rv; idx += blockDim.x) {
    const int g = idx / rv, j = idx - g * rv;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, wm[w * 4 + g]);
    float o = 0.f, L = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
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

// scratch: LDS_FLOATS floats of LDS (at least 4 RB + 17 plus a few basis rows).
// REC: split records folded per memory round trip.
template <int RB, int LDS_FLOATS = kTailLds, int REC = 8>
__device__ __forceinline__ void finish_split(const DecodeParams& p, int b, int h, int hg, int hq0, int gpw,
                                             int rv, float* scratch, const BasisPrefetch<RB>& pf,
                                             const RecLayout& rl, int n_rec) {
  if (!p.fuse) return;
  int* flag = reinterpret_cast<int*>(scratch + LDS_FLOATS - 1);
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
  const int p_rows = min(d, (LDS_FLOATS - 4 * RB - 16) / pst);
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

  // wave g folds the records of head g with a running maximum, REC records per memory
  // round trip
  float M = kNegInf, L = 0.f, o0 = 0.f, o1 = 0.f;
  if (g < gpw) {
    for (int s0 = 0; s0 < n_rec; s0 += REC) {
      float ms[REC], ls[REC], v0[REC], v1[REC];
#pragma unroll
      for (int u = 0; u < REC; ++u) {
        const bool ok = s0 + u < n_rec;
        const float* r = rec_at(rl, ok ? s0 + u : 0, g);
        ms[u] = ok ? load_rec(r) : kNegInf;
        ls[u] = ok ? load_rec(r + 1) : 0.f;
        v0[u] = (ok && lane < rv) ? load_rec(r + 2 + lane) : 0.f;
        v1[u] = (ok && lane + 64 < rv) ? load_rec(r + 66 + lane) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < REC; ++u) {
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
    mx = max_over_rows(mx);
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
  l = sum_over_rows(l);
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

// One segment of the balanced plan: a token range of unit (b, h, hg), its record
// index k among the unit's n_rec records, and the record slot of the unit's first.
struct Segment {
  int b, h, hg, t_begin, t_end, k, n_rec;
  size_t slot;
};

// The balanced plan with one segment per workgroup (used when the units are few next
// to the workgroups): unit (b, h, hg) is cut into k(b, h) segments of equal token
// counts, with k(b, h) = ceil(T_b cost[h] / lam), at most one per kBalancedTokens
// tokens, and lam the least work per segment (found by bisection) for which all the
// segments number at most gridDim.x. Workgroup w takes segment w in (b, h, hg, j)
// order and leaves its record in slot w; the segments of a unit are consecutive, so
// the unit's records are too, and its last arrival merges them. No workgroup pays for
// two segments' prologues and tails. Wave 0 of every workgroup computes the plan with
// the same float operations from the same lengths, so all workgroups agree on it: a
// geometric bisection for lam inside a bracket that the rounding bound gives, then one
// prefix sum over the units' segment counts to find the unit that holds segment w.
template <typename LenOf>
__device__ __forceinline__ bool apportioned_segment(const DecodeParams& p, const LenOf& len_of, Segment& sg) {
  constexpr int R = kApportionPairs / 64;   // (row, KV head) pairs per lane
  const int lane = thread_id() & 63, w = blockIdx.x;
  const int Hkv = p.Hkv, n_hg = p.n_head_groups, n_pairs = p.B * Hkv;
  float work[R];   // T_b cost[h] of pair i = lane + 64 r
  float kmax[R];
  int tlen[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = lane + 64 * r;
    const int bi = i / Hkv, hi = i - bi * Hkv;
    tlen[r] = i < n_pairs ? (int)len_of(bi) : 0;
    work[r] = (float)tlen[r] * (float)p.ht.cost[i < n_pairs ? hi : 0];
    kmax[r] = (float)((tlen[r] + kBalancedTokens - 1) / kBalancedTokens);
  }
  auto segs = [&](int r, float inv_lam) { return fminf(ceilf(work[r] * inv_lam), kmax[r]); };
  const int n_r = (n_pairs + 63) >> 6;   // chunks in use
  // segments of all the units (wave-uniform; exact below 2^24)
  auto count = [&](float inv_lam) {
    float n = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < n_r) n += segs(r, inv_lam);
    return sum_over_rows(row16_allreduce<false>(n)) * (float)n_hg;
  };
  // the bracket: W / P is the least work per segment that could do; every unit rounds
  // its count up by less than one segment, so the count is below W / lam + U (U: the
  // non-empty units) and lam = W / (P - U) does when P > U (checked; else lam = W: one
  // segment per non-empty unit, two where rounding lifts a share past 1, at most
  // 2 U <= P in this form)
  float wsum = 0.f, nz = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (r < n_r) {
      wsum += work[r];
      nz += work[r] > 0.f ? 1.f : 0.f;
    }
  const float W = sum_over_rows(row16_allreduce<false>(wsum)) * (float)n_hg;
  const float U = sum_over_rows(row16_allreduce<false>(nz)) * (float)n_hg;
  const float Pf = (float)gridDim.x;
  float lo = W / Pf, hi = Pf > U ? W / (Pf - U) : W;
  if (count(1.f / hi) > Pf) hi = W;
  for (int it = 0; it < 16 && hi > 1.0005f * lo; ++it) {   // geometric bisection to 0.05%
    const float mid = sqrtf(lo * hi);
    if (count(1.f / mid) <= Pf) hi = mid; else lo = mid;
  }
  const float inv_lam = 1.f / hi;
  // first segment of every pair: an exclusive prefix sum over the pairs in order
  float first[R], sk[R];
  float run = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r < n_r) {
      sk[r] = lane + 64 * r < n_pairs ? segs(r, inv_lam) : 0.f;
      float v = sk[r];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(v, off, 64);
        if (lane >= off) v += y;
      }
      first[r] = (run + v - sk[r]) * (float)n_hg;
      run += readlane_f(v, 63);
    }
  }
  if (w >= (int)(run * (float)n_hg)) return false;
  // the pair holding segment w: the last pair whose first segment is at most w
  int n_le = 0;
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (r < n_r) n_le += __builtin_popcountll(__ballot(lane + 64 * r < n_pairs && first[r] <= (float)w));
  const int ilo = n_le - 1;
  float kl = 0.f, el = 0.f;
  int tl = 0;
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (r == (ilo >> 6)) {
      kl = sk[r];
      el = first[r];
      tl = tlen[r];
    }
  const int E = (int)readlane_f(el, ilo & 63);
  const int k = (int)readlane_f(kl, ilo & 63);
  const long long T = __builtin_amdgcn_readlane(tl, ilo & 63);
  const int b = ilo / Hkv, h = ilo - b * Hkv;
  const int off = w - E, hg = off / k, j = off - hg * k;
  auto tok = [&](int x) {   // start of segment x of the unit, on a kBalancedTokens boundary
    const long long t = ((long long)x * T / k + kBalancedTokens - 1) / kBalancedTokens * kBalancedTokens;
    return (int)min(t, T);
  };
  sg = Segment{b, h, hg, tok(j), tok(j + 1), j, k, (size_t)(E + hg * k)};
  return true;
}


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

// Balanced plan with one segment per workgroup (see apportioned_segment); three
// workgroups per CU up to rank bound 96.
template <int RB, int TT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(RB <= 96 ? 3 : 2)))
void decode_apportioned_bf16(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) float smem[kTailLds];
  const int B = p.B, tid = thread_id();
  auto len_of = [&](int bi) { return bi < B ? (long long)min(max(p.seq_lens[bi], 0), p.cap) : 0ll; };
  // every length this workgroup needs is loaded at once (one memory round trip): its
  // zero-row duty (rows without tokens get zero outputs; B <= gridDim.x / 2 here) and
  // the plan's pairs
  const bool zero_duty = (int)blockIdx.x < B;
  const long long Tz = zero_duty ? len_of(blockIdx.x) : 1;
  // the segment passes through LDS: its values are then re-read where needed instead of
  // being held in scalar registers across the segment body (which would spill them)
  // Wave 0 works out the plan; the other waves wait at the barrier (every workgroup
  // computes the same plan from the same lengths, so one wave of each is enough).
  __shared__ Segment st;
  __shared__ int st_has;
  if (tid < 64) {
    Segment sg;
    const bool has = apportioned_segment(p, len_of, sg);
    if (tid == 0) {
      st = sg;
      st_has = has;
    }
  }
  if (zero_duty && Tz == 0) {
    const int n = p.Hq * p.out_stride;
    float* o = p.out + (size_t)blockIdx.x * n;
    for (int i = tid; i < n; i += blockDim.x) o[i] = 0.f;
  }
  __syncthreads();
  if (!st_has) return;
  const RecLayout rl{p.ws + st.slot * kHeadsPerWg * p.ws_stride, (size_t)kHeadsPerWg * p.ws_stride,
                     (size_t)p.ws_stride};
  bf16_segment<RB, TT>(p, st.b, st.h, st.hg, st.t_begin, st.t_end, rl, st.k, st.n_rec, smem);
}

// ---------------------------------------------------------------------------
// 4/3-bit latents (STAR-KV technical summary, "Metodologia" section 3): both
// products on MFMA, straight from the stored codes
// ---------------------------------------------------------------------------
// The cache holds tiles of 32 tokens whose words are already in the operand
// order of the two products (layout in kvlr.h): one 32-bit word or 24-bit field
// per lane and 16-channel group holds the 8 codes that lane feeds to them. A
// wave takes one tile per step; the waves of a workgroup take the split's tiles
// round robin. A code c enters an MFMA as the bf16 number 128 + c (bits
// 0x4300 | c, exact).
//  - Scores, transposed: S^T = K q~^T per group of 16 key channels, both 16-token
//    blocks of the tile in one v_mfma_f32_16x16x32_bf16: the lane's 8 codes are the
//    A operand as stored, and column 4 sb + hd of the B operand holds q~ of head hd
//    in the slots of block sb (zeros in the other block's), once with its high and
//    once with its low bf16 parts. Outlier and inlier groups go into separate
//    accumulators that start at -128 C (C = sum of the B operands), so they end as
//    sum_j q~_j c_j. Lane (n < 8, q) then holds tokens 4 q .. 4 q + 3 of block n / 4
//    for head n % 4 and applies the tokens' block parameters:
//      s = step_o acc_o + base_o Q_o + step_i acc_i + base_i Q_i.
//  - Online softmax per (block, head) column in the log2 domain; the workgroup
//    merge takes 8 states per query head (2 per wave).
//  - Values: o_lat[row][ch] += sum_t w_t (1024 + c_t,ch) on
//    v_mfma_f32_16x16x32_f16 over the tile's 32 tokens, rows = the (block, head)
//    columns of the scores: a value code enters as the half float 1024 + c (bits
//    0x6400 | c, exact), and the weights w = half(half(p) step_o) or
//    half(half(p) step_i), formed two tokens per packed multiply in the slots of
//    the lane's block, are already the A operand in registers. An MFMA against a
//    B operand of ones gives sum_t w_t (the 1024 offset), and one against the
//    tokens' minima gives sum_t p_t base_t; the three are combined when the
//    split ends. The weights carry half-float precision (11 bits), the scores'
//    q~ about 16 bits (high and low bf16 parts).
// Codes are turned into MFMA operands with a handful of bit operations: a
// 4-bit word splits into its low and high nibbles (blocks 0 and 1) and v_perm
// interleaves them with the exponent byte 0x43; a 24-bit 3-bit field is
// rotated so that codes e and e + 4 sit 16 bits apart, and each pair is one
// AND-OR, after a shift for two of the four pairs (keys keep two pairs at bits 3..5,
// i.e. 128 + 8 c, and value pairs take one shift each).
constexpr uint32_t kBf16Code = 0x43434343u;   // bf16 exponent bytes of 128 + c (keys)
constexpr uint32_t kF16Code = 0x64646464u;    // f16 exponent bytes of 1024 + c (values)

// v_perm selectors: bytes 0 and 1 (2 and 3) of x, each followed by the exponent byte
__device__ __forceinline__ u32x2_t nibbles_to_num(uint32_t x, uint32_t ebytes) {
  return u32x2_t{__builtin_amdgcn_perm(ebytes, x, 0x04010400u), __builtin_amdgcn_perm(ebytes, x, 0x04030402u)};
}

// One 4-bit group word of a lane -> the 8 codes as 16-bit pairs (exponent byte ebytes):
// dwords 0, 1 block 0 (positions i = 0..3), dwords 2, 3 block 1.
__device__ __forceinline__ u32x4_t codes4_to_num(uint32_t w, uint32_t ebytes) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  const u32x2_t a = nibbles_to_num(lo, ebytes), b = nibbles_to_num(hi, ebytes);
  return u32x4_t{a.x, a.y, b.x, b.y};
}

// One 24-bit 3-bit field (bits 0..23 of x) -> the same order: field position e
// holds (block, i) = (0,0) (0,2) (1,0) (1,2) (0,1) (0,3) (1,1) (1,3), so after
// moving bits 12..23 to 16..27 the pairs (e, e + 4) are (block e / 2, i = 2 (e % 2) + {0, 1}).
// m7 = 0x00070007 and e2 = the exponent bytes in the high byte of each half come in
// registers: the AND-OR of two of them is then one instruction.
__device__ __forceinline__ u32x4_t codes3_to_num(uint32_t x, uint32_t m7, uint32_t e2) {
  const uint32_t y = (x & 0xFFFFu) | ((x << 4) & 0xFFFF0000u);   // bits 12..23 to 16..27
  u32x4_t o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = ((y >> (3 * e)) & m7) | e2;
  return o;
}

// Keys: the same fields with dwords 1 and 3 left at bits 3..5 of each half, i.e. the
// bf16 numbers 128 + 8 c (exact); the score product scales those slots of q~ by 1/8.
// m7s = m7 << 3.
__device__ __forceinline__ u32x4_t codes3_to_num_keys(uint32_t x, uint32_t m7, uint32_t m7s, uint32_t e2) {
  const uint32_t y = (x & 0xFFFFu) | ((x << 4) & 0xFFFF0000u);   // bits 12..23 to 16..27
  const uint32_t y6 = y >> 6;
  return u32x4_t{(y & m7) | e2, (y & m7s) | e2, (y6 & m7) | e2, (y6 & m7s) | e2};
}

// The lane's 24-bit field of an inlier group: bytes 3 lane .. 3 lane + 2 of the group,
// from the two dwords that hold them (the same dword when they do not straddle).
__device__ __forceinline__ uint32_t field24(uint32_t w_a, uint32_t w_b, int shift) {
  return __builtin_amdgcn_alignbit(w_b, w_a, shift);
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
// A vector element is copied to a scalar before it is bit-cast: clang's __builtin_bit_cast
// applied straight to an element of an ext_vector_type value reads element 0 whatever
// the index (found in the ISA of this file; the copy is compiled as intended).
__device__ __forceinline__ half2_t half2_of(uint32_t w) { return __builtin_bit_cast(half2_t, w); }
__device__ __forceinline__ float half2_at(const u32x2_t& v, int k) {   // half float k (0..3) of an 8-byte piece
  const uint32_t w = v[k >> 1];
  return (float)__builtin_bit_cast(half2_t, w)[k & 1];
}

// Raw buffer access to one (batch row, KV head) block of a 4/3-bit cache: base and size
// in a resource (word 3 = 0x00020000: the raw 32-bit data format of gfx9 buffers), a
// per-lane offset in a VGPR and the tile offset in an SGPR; loads stream (non-temporal).
typedef __amdgpu_buffer_rsrc_t q43_rsrc_t;
constexpr int kBufNonTemporal = 2;
__device__ __forceinline__ q43_rsrc_t q43_block_rsrc(const uint8_t* base, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, nbytes, 0x00020000);
}
// 16 bytes per lane from the block into LDS: lane i's bytes land at lds + 16 i (the LDS
// address is the wave's base plus the lane's index; the block offset is voff + soff).
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ void q43_dma16(q43_rsrc_t rs, uint8_t* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)lds, 16, voff, soff, 0, kBufNonTemporal);
}
// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector-memory
// operations of this wave are in flight, and for nothing else
constexpr int vmcnt_at_most(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Tiles reach LDS by direct buffer-to-LDS loads. Each wave keeps a ring of kStages
// stages (a key tile, then a value tile) and has the tiles of its next kStages - 1
// steps in flight while it computes on the current one. Every tile of a kind takes
// kLoads load instructions (with two, the first covers up to 64 lanes of 16 bytes and
// the second the rest, at least one lane), so after a step issues its look-ahead tile,
// at most kWait loads may still be in flight once the step's own tile has landed.
template <int RB>
struct Q43Ring {
  static constexpr int kTileBytes = kQ43Tile * q43_row_bytes(RB);   // the largest tile of the class
  static constexpr int kLoads = kTileBytes / 16 > 64 ? 2 : 1;
  static constexpr int kStage = 2 * kTileBytes;
  static constexpr int kStages = RB <= 32 ? 8 : RB <= 96 ? 5 : 4;
  static constexpr int kRingBytes = kWaves * kStages * kStage;
  static constexpr int kProFloats = 1024 + 20 * RB;                  // query projection: q, q~, partial sums
  static constexpr int kWait = (kStages - 1) * 2 * kLoads;
  static_assert(kWait < 64, "vmcnt holds 6 bits");
  static_assert(kLoads == 2 || kTileBytes / 16 <= 64, "one instruction covers 64 lanes");
};

// EXACT: every KV head has r_k = r_v = RB, so the group structure is known at compile time.
template <int RB, bool EXACT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(RB <= 64 ? 3 : 2)))
void decode_split_q43(DecodeParams p) {
  constexpr int GO = RB == 128 ? 2 : 1;                    // 4-bit groups (bound): group 0 always is one
  constexpr int GI = RB == 128 ? 6 : (RB - 16) / 16;       // 3-bit groups (bound)
  constexpr int NG = GO + GI;                              // groups from GO on are always 3-bit
  constexpr int QTS = RB;
  using Ring = Q43Ring<RB>;
  constexpr int NS = Ring::kStages, STAGE = Ring::kStage, TB = Ring::kTileBytes;
  constexpr int EPI = Ring::kRingBytes / 4;   // the epilogue reuses the ring once every tile has landed
  // Two LDS objects: the compiler then knows that the prologue's LDS writes do not
  // touch the ring that the tile loads write, and does not wait for those loads.
  __shared__ __attribute__((aligned(16))) float ring_lds[EPI];
  __shared__ __attribute__((aligned(16))) float pro_lds[Ring::kProFloats];
  float* const smem = ring_lds;
  static_assert(EPI >= 2 * kWaves * kHeadsPerWg * (RB + 2) && EPI >= 4 * RB + 17 + 16 * (RB + 4),
                "the ring holds the epilogue's partial sums and some basis rows");

  const int s = blockIdx.x;
  const int h = blockIdx.y / p.n_head_groups;
  const int hg = blockIdx.y - h * p.n_head_groups;
  const int b = blockIdx.z;
  const int hq0 = h * p.G + hg * kHeadsPerWg;
  const int gpw = min(kHeadsPerWg, p.G - hg * kHeadsPerWg);
  const int rk = EXACT ? RB : p.ht.rk[h], rv = EXACT ? RB : p.ht.rv[h];
  const int T = min(max(p.seq_lens[b], 0), p.cap);
  const int t_begin = min(s * p.ht.split_len[h], T);
  const int t_end = min(T, t_begin + p.ht.split_len[h]);
  const RecLayout rl = fixed_records(p, b, hq0);
  if (t_begin >= t_end) {
    write_empty_records(rl, s, gpw, rv);
    BasisPrefetch<RB> pf;
    prefetch_basis<RB>(p, h, rv, pf);
    finish_split<RB, EPI, 16>(p, b, h, hg, hq0, gpw, rv, smem, pf, rl, p.n_splits);
    return;
  }

  const int tid = thread_id(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, q4 = lane >> 4;
  const int gok = EXACT ? GO : q43_outlier(rk) >> 4, ngk = EXACT ? NG : rk >> 4;   // 4-bit and all groups of the keys
  const int gov = EXACT ? GO : q43_outlier(rv) >> 4, ngv = EXACT ? NG : rv >> 4;
  const int tbk = kQ43Tile * q43_row_bytes(rk), tbv = kQ43Tile * q43_row_bytes(rv);
  const size_t rows = cap_rows_q43(p.cap);
  // Buffer resources over this (batch row, KV head) block of each cache
  const q43_rsrc_t rs_k = q43_block_rsrc(static_cast<const uint8_t*>(p.lat_k) + rows * ((size_t)b * p.Sk + p.ht.sk_pre[h]),
                                         (int)rows / kQ43Tile * tbk);
  const q43_rsrc_t rs_v = q43_block_rsrc(static_cast<const uint8_t*>(p.lat_v) + rows * ((size_t)b * p.Sv + p.ht.sv_pre[h]),
                                         (int)rows / kQ43Tile * tbv);

  // ---- this wave's tiles: every kWaves-th tile of the split (split starts are
  // multiples of 64 tokens, so whole tiles), n_w of them; the ring's stage u holds
  // the wave's tiles u, u + NS, ...
  uint8_t* const ring = reinterpret_cast<uint8_t*>(ring_lds) + wave * NS * STAGE;
  const int tile0 = (t_begin >> 5) + wave;
  const int left = t_end - t_begin - wave * kQ43Tile;
  const int n_w = left > 0 ? (left + kWaves * kQ43Tile - 1) / (kWaves * kQ43Tile) : 0;
  // The wave's tile j (past its last tile: the last one again, unused) into ring stage u.
  // The full 64-lane instructions of both kinds come first, then the partial ones, each
  // in one branch of its own: the count of instructions a tile takes stays 2 kLoads.
  const int nk = tbk >> 4, nv = tbv >> 4;   // 16-byte pieces of a tile
  const int nk0 = Ring::kLoads == 1 ? nk : min(64, nk - 1), nv0 = Ring::kLoads == 1 ? nv : min(64, nv - 1);
  // The lane limits of the partial instructions pass through an empty asm statement at
  // each call, so the compiler cannot merge or thread branches with equal conditions
  // across calls (which would issue an instruction once per lane subset).
  auto issue = [&](int j, int u) {
    const int tile = tile0 + kWaves * min(j, n_w - 1);
    uint8_t* const dk = ring + u * STAGE;
    uint8_t* const dv = dk + TB;
    int lk = Ring::kLoads == 1 ? nk : nk - nk0, lv = Ring::kLoads == 1 ? nv : nv - nv0;
    asm volatile("" : "+s"(lk), "+s"(lv));
    if (Ring::kLoads == 1) {
      if (lane < lk) q43_dma16(rs_k, dk, 16 * lane, tile * tbk);
      if (lane < lv) q43_dma16(rs_v, dv, 16 * lane, tile * tbv);
    } else {
      if (lane < nk0) q43_dma16(rs_k, dk, 16 * lane, tile * tbk);
      if (lane < nv0) q43_dma16(rs_v, dv, 16 * lane, tile * tbv);
      if (lane < lk) q43_dma16(rs_k, dk + 16 * nk0, 16 * lane, tile * tbk + 16 * nk0);
      if (lane < lv) q43_dma16(rs_v, dv + 16 * nv0, 16 * lane, tile * tbv + 16 * nv0);
    }
  };

  // this lane's bytes of a stage: its parameter slots, its 4-bit word, and the two
  // dwords that hold bytes 3 lane .. 3 lane + 2 of a 3-bit group (its 24-bit field).
  // Group g starts at byte 256 + 256 g while g is a 4-bit group, at 256 + 64 go + 192 g
  // once it is a 3-bit one (go 4-bit groups first).
  // Score columns: lane column n16 = 4 sb + hd holds query head hd of 16-token block
  // sb (columns 8..15 stay empty), so each lane scores 4 tokens of one block, and the
  // scores of a lane are the value product's A operand of the same lane (row n16).
  const int sb = (n16 >> 2) & 1, hd = n16 & 3;
  const bool s_ok = n16 < 8 && hd < gpw;
  const int off_a = (3 * lane) & ~3, off_b = (3 * lane + 2) & ~3, f_shift = 8 * ((3 * lane) & 3);
  const uint8_t* const la_meta = ring + 64 * q4;            // the 8 tokens' parameters of lane group q4
  const uint8_t* const la_own = la_meta + 8 * sb;           // those of this lane's 4 tokens
  const uint8_t* const la_4 = ring + 4 * lane;
  const uint8_t* const la_a = ring + off_a;
  const uint8_t* const la_b = ring + off_b;
  u32x2_t kp[4], vs[2];   // per lane: keys' step_o, base_o, step_i, base_i; values' step_o, step_i
  u32x4_t vb[2];          // values' base_o, base_i of all 8 tokens (B operands)
  uint32_t kwa[NG], kwb[NG], vwa[NG], vwb[NG];
  auto read_codes = [&](int at, int go, int ng, uint32_t* wa, uint32_t* wb) {
    const int in = at + kQ43MetaBytes + (kQ43OutGroupBytes - kQ43InGroupBytes) * go;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const bool four = g == 0 || (GO == 2 && g == 1 && go == 2);
      if (four) {
        wa[g] = *reinterpret_cast<const uint32_t*>(la_4 + at + kQ43MetaBytes + kQ43OutGroupBytes * g);
      } else if (g < ng) {
        wa[g] = *reinterpret_cast<const uint32_t*>(la_a + in + kQ43InGroupBytes * g);
        wb[g] = *reinterpret_cast<const uint32_t*>(la_b + in + kQ43InGroupBytes * g);
      }
    }
  };
  auto read_tile = [&](int at) {
#pragma unroll
    for (int P = 0; P < 4; ++P) kp[P] = *reinterpret_cast<const u32x2_t*>(la_own + at + 16 * P);
    read_codes(at, gok, ngk, kwa, kwb);
    const int av = at + TB;
    vs[0] = *reinterpret_cast<const u32x2_t*>(la_own + av);
    vs[1] = *reinterpret_cast<const u32x2_t*>(la_own + av + 32);
    vb[0] = *reinterpret_cast<const u32x4_t*>(la_meta + av + 16);
    vb[1] = *reinterpret_cast<const u32x4_t*>(la_meta + av + 48);
    read_codes(av, gov, ngv, vwa, vwb);
  };
  // operands of group g: 16-bit pairs with exponent bytes eb, block 0 then block 1
  // constants of the 3-bit conversion, held in registers (see codes3_to_num)
  uint32_t m7 = 0x00070007u, m7s = 0x00380038u, e2_k = kBf16Code & 0xFF00FF00u, e2_v = kF16Code & 0xFF00FF00u;
  asm volatile("" : "+v"(m7), "+v"(m7s), "+s"(e2_k), "+s"(e2_v));
  // key groups (3-bit ones with slots 2, 3 of each block at 128 + 8 c) and value groups
  auto key_codes = [&](int g) -> u32x4_t {
    if (g == 0) return codes4_to_num(kwa[0], kBf16Code);
    if (g >= GO) return codes3_to_num_keys(field24(kwa[g], kwb[g], f_shift), m7, m7s, e2_k);
    return gok == 2 ? codes4_to_num(kwa[g], kBf16Code)
                    : codes3_to_num_keys(field24(kwa[g], kwb[g], f_shift), m7, m7s, e2_k);
  };
  auto value_codes = [&](int g) -> u32x4_t {
    if (g == 0) return codes4_to_num(vwa[0], kF16Code);
    if (g >= GO) return codes3_to_num(field24(vwa[g], vwb[g], f_shift), m7, e2_v);
    return gov == 2 ? codes4_to_num(vwa[g], kF16Code) : codes3_to_num(field24(vwa[g], vwb[g], f_shift), m7, e2_v);
  };

  // ---- prologue: q~ (scaled to log2 units) and, per key group, the B operands of the
  // score product. The A operand of lane (n, q) holds its 8 codes as they are: token n
  // of block 0 at channels 4 q .. 4 q + 3 of the group, then token n of block 1. Column
  // 4 sb + hd takes q~ of head hd at those channels in the slots of block sb and zero in
  // the others, so it sums block sb only; one product takes the high bf16 parts of q~,
  // a second the low parts. In 3-bit groups the codes of channels 2 and 3 of each 4
  // enter as 128 + 8 c, so q~ enters there divided by 8 (exact): the products still sum
  // c q~, on top of 128 times the sum of the B operands (C below).
  float* q_lds = pro_lds;                       // [4][d]
  float* qt_lds = q_lds + kHeadsPerWg * 256;    // [4][QTS]
  float* qred = qt_lds + kHeadsPerWg * QTS;     // [4 waves][4][QTS]
  project_query<RB>(p, b, h, hq0, gpw, rk, q_lds, qred, qt_lds);
  bf16x8_t qbh[NG], qbl[NG];
  float Qo = 0.f, Qi = 0.f, Ci = 0.f;   // Q: sums of q~ as the products see it; Ci: of the B operands
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const bool four = g < gok;
    const bool ok = g < ngk;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = 16 * g + 4 * q4 + i;   // 4-bit groups first, then 3-bit: channels in order
      const float x = (s_ok && ok) ? qt_lds[hd * QTS + ch] : 0.f;
      const bool eighth = !four && i >= 2;
      const float xs = eighth ? 0.125f * x : x;
      const uint16_t hi = f32_to_bf16_bits(xs);
      const uint16_t lo = f32_to_bf16_bits(xs - bf16_bits_to_f32(hi));
      qbh[g][i] = sb == 0 ? (short)hi : (short)0;
      qbh[g][4 + i] = sb == 1 ? (short)hi : (short)0;
      qbl[g][i] = sb == 0 ? (short)lo : (short)0;
      qbl[g][4 + i] = sb == 1 ? (short)lo : (short)0;
      const float seen = bf16_bits_to_f32(hi) + bf16_bits_to_f32(lo);
      if (four) {
        Qo += seen;
      } else {
        Qi += eighth ? 8.f * seen : seen;
        Ci += seen;
      }
    }
  }
  Qo = sum_over_rows(Qo);
  Qi = sum_over_rows(Qi);
  Ci = sum_over_rows(Ci);
  const float c_o = -128.f * Qo, c_i = -128.f * Ci;
  // A-operand masks of the value product: this lane's weights sit in the slots of its block
  const uint32_t own_lo = sb == 0 ? ~0u : 0u, own_hi = ~own_lo;
  // The first NS - 1 tiles go out once the prologue is done with memory: the waits of
  // its loads would cover them, and so would those of its LDS reads (the compiler
  // orders LDS accesses after direct-to-LDS loads issued under a lane mask).
  if (n_w > 0) {
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) issue(j, j);
  }

  const half8_t ones = __builtin_bit_cast(half8_t, u32x4_t{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u});
  // running maximum and sum of this lane's score column (head hd, block sb)
  float m = kNegInf, l = 0.f;
  // value accumulators (rows: score columns 4 q4 + i, i.e. (block, head) pairs; rows
  // 8..15 stay unused) and the sums over tokens of w_o, w_i, p base_o and p base_i (the
  // same rows, every column alike)
  f32x4_t acc[NG], sw_o = {0.f, 0.f, 0.f, 0.f}, sw_i = {0.f, 0.f, 0.f, 0.f};
  f32x4_t sb_o = {0.f, 0.f, 0.f, 0.f}, sb_i = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < NG; ++g) acc[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int it0 = 0; it0 < n_w; it0 += NS) {
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const int it = it0 + u;
    if (it >= n_w) break;
    const int t0 = (tile0 + kWaves * it) * kQ43Tile;
    // look ahead NS - 1 tiles, into the stage the previous step used; then wait for this one
    issue(it + NS - 1, (u + NS - 1) % NS);
    __builtin_amdgcn_s_waitcnt(vmcnt_at_most(Ring::kWait));
    asm volatile("" ::: "memory");   // the stage's LDS reads stay after the wait
    read_tile(u * STAGE);
    // ---- scores S^T[token][column] of both blocks; accumulators start at -128 Q
    f32x4_t ao = {c_o, c_o, c_o, c_o}, ai = {c_i, c_i, c_i, c_i};
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g < ngk) {
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, key_codes(g));
        if (g == 0 || (GO == 2 && g == 1 && gok == 2)) {
          ao = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qbh[g], ao, 0, 0, 0);
          ao = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qbl[g], ao, 0, 0, 0);
        } else {
          ai = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qbh[g], ai, 0, 0, 0);
          ai = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qbl[g], ai, 0, 0, 0);
        }
      }
    }
    // the keys' block parameters: s = step_o acc_o + base_o Q_o + step_i acc_i + base_i Q_i
    // (lane: tokens t0 + 16 sb + 4 q4 + i)
    const bool tail = t0 + kQ43Tile > t_end;   // rows past the end may hold any bits
    const int tl = t0 + 16 * sb + 4 * q4;
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sc[i] = fmaf(half2_at(kp[0], i), ao[i],
                   fmaf(half2_at(kp[2], i), ai[i], fmaf(half2_at(kp[1], i), Qo, fmaf(half2_at(kp[3], i), Qi, 0.f))));
    if (__builtin_expect(tail, 0)) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tl + i >= t_end) sc[i] = kNegInf;
    }

    // ---- online softmax per score column
    // in-lane maximum by med3(a, b, +inf) = max(a, b): scores are never NaN here
    float mx = __builtin_amdgcn_fmed3f(__builtin_amdgcn_fmed3f(sc[0], sc[1], kPosInf),
                                       __builtin_amdgcn_fmed3f(sc[2], sc[3], kPosInf), kPosInf);
    mx = max_over_rows(mx);
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = s_ok ? fast_exp2(m - m_use) : 1.f;
    float pr[4], ls = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = fast_exp2(sc[i] - m_use);   // masked: exp2(-inf) = 0
      ls += pr[i];
    }
    l = fmaf(l, alpha, ls);
    m = m_new;
    if (__ballot(alpha != 1.f)) {
      // accumulator rows are score columns 4 q4 + i; their factors sit in lanes 4 q4 + i
      float ar[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * q4 + i, 64);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int g = 0; g < NG; ++g) acc[g][i] *= ar[i];
        sw_o[i] *= ar[i];
        sw_i[i] *= ar[i];
        sb_o[i] *= ar[i];
        sb_i[i] *= ar[i];
      }
    }

    // ---- value weights in half floats, two tokens per operation: w = p step, and p
    // itself, in the A-operand slots of this lane's block (zero in the other block's).
    // In the last tile the parameters of rows past the end are zeroed (they may hold
    // any bits).
    if (tail) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t msk = (tl + 2 * j < t_end ? 0xFFFFu : 0u) | (tl + 2 * j + 1 < t_end ? 0xFFFF0000u : 0u);
        vs[0][j] &= msk;
        vs[1][j] &= msk;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = 2 * j, t_k = t0 + 16 * (k >> 2) + 4 * q4 + (k & 3);
        const uint32_t msk = (t_k < t_end ? 0xFFFFu : 0u) | (t_k + 1 < t_end ? 0xFFFF0000u : 0u);
        vb[0][j] &= msk;
        vb[1][j] &= msk;
      }
    }
    const half2_t p01 = __builtin_convertvector((float __attribute__((ext_vector_type(2)))){pr[0], pr[1]}, half2_t);
    const half2_t p23 = __builtin_convertvector((float __attribute__((ext_vector_type(2)))){pr[2], pr[3]}, half2_t);
    const uint32_t w01 = __builtin_bit_cast(uint32_t, p01), w23 = __builtin_bit_cast(uint32_t, p23);
    const u32x4_t pw = {w01 & own_lo, w23 & own_lo, w01 & own_hi, w23 & own_hi};
    u32x4_t wo, wi;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wo[j] = __builtin_bit_cast(uint32_t, half2_of(pw[j]) * half2_of(vs[0][j & 1]));
      wi[j] = __builtin_bit_cast(uint32_t, half2_of(pw[j]) * half2_of(vs[1][j & 1]));
    }
    const half8_t awo = __builtin_bit_cast(half8_t, wo), awi = __builtin_bit_cast(half8_t, wi);
    const half8_t ap = __builtin_bit_cast(half8_t, pw);

    // ---- value product per group of 16 channels (codes as 1024 + c), and the four sums
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g < ngv) {
        const half8_t bv = __builtin_bit_cast(half8_t, value_codes(g));
        const bool four = g == 0 || (GO == 2 && g == 1 && gov == 2);
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(four ? awo : awi, bv, acc[g], 0, 0, 0);
      }
    }
    sw_o = __builtin_amdgcn_mfma_f32_16x16x32_f16(awo, ones, sw_o, 0, 0, 0);
    sw_i = __builtin_amdgcn_mfma_f32_16x16x32_f16(awi, ones, sw_i, 0, 0, 0);
    // the B operand of lane (n, q) holds slots 8 q .. 8 q + 7 for column n: its own parameters
    sb_o = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap, __builtin_bit_cast(half8_t, vb[0]), sb_o, 0, 0, 0);
    sb_i = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap, __builtin_bit_cast(half8_t, vb[1]), sb_i, 0, 0, 0);
  }
  }

  BasisPrefetch<RB> pf;
  prefetch_basis<RB>(p, h, rv, pf);
  // ---- per (block, head) state: l over the lane groups; rows 4 q4 + i of lane groups
  // q4 = 0, 1 hold block q4's heads i:
  // o_lat = sum_t w_t (1024 + c_t) - 1024 sum_t w_t + sum_t p_t base_t
  l = sum_over_rows(l);
  __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));   // this wave's tile loads have landed: the ring is reused
  __syncthreads();
  constexpr int kStates = 2 * kWaves;          // one per (wave, block)
  float* red = smem;                          // [state][head][RB]
  float* wm = smem + kStates * kHeadsPerWg * RB;
  float* wl = wm + kStates * kHeadsPerWg;
  if (q4 < 2) {
    const int st = 2 * wave + q4;
#pragma unroll
    for (int g = 0; g < NG; ++g)
      if (g < ngv) {
        const bool four = g == 0 || (GO == 2 && g == 1 && gov == 2);
#pragma unroll
        for (int i = 0; i < kHeadsPerWg; ++i)
          red[(st * kHeadsPerWg + i) * RB + 16 * g + n16] =
              acc[g][i] - 1024.f * (four ? sw_o[i] : sw_i[i]) + (four ? sb_o[i] : sb_i[i]);
      }
    if (q4 == 0 && n16 < 8) {
      wm[(2 * wave + sb) * kHeadsPerWg + hd] = m;
      wl[(2 * wave + sb) * kHeadsPerWg + hd] = l;
    }
  }
  __syncthreads();
  merge_waves_and_store<kStates>(rl, s, gpw, rv, wm, wl,
                                 [&](int w, int g, int j) { return red[(w * kHeadsPerWg + g) * RB + j]; });
  finish_split<RB, EPI, 16>(p, b, h, hg, hq0, gpw, rv, smem, pf, rl, p.n_splits);
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
    bool exact = true;   // every head at r_k = r_v = the bound: no per-head group conditions
    for (int h = 0; h < p.Hkv; ++h) exact = exact && p.ht.rk[h] == rank_bound && p.ht.rv[h] == rank_bound;
#define KVLR_Q43_LAUNCH(RB)                                                     \
  if (exact) hipLaunchKernelGGL((decode_split_q43<RB, true>), grid, block, 0, stream, p); \
  else hipLaunchKernelGGL((decode_split_q43<RB, false>), grid, block, 0, stream, p)
    switch (rank_bound) {
      case 32: KVLR_Q43_LAUNCH(32); break;
      case 64: KVLR_Q43_LAUNCH(64); break;
      case 96: KVLR_Q43_LAUNCH(96); break;
      default: KVLR_Q43_LAUNCH(128); break;
    }
#undef KVLR_Q43_LAUNCH
    return hipGetLastError();
  }
  if (latent_bf16) {
    if (p.balanced) {   // one workgroup per share of the balanced plan
      const dim3 grid_b(p.n_wg);
#define KVLR_BAL_LAUNCH(RB)                                                                   \
  if (p.apportion) hipLaunchKernelGGL((decode_apportioned_bf16<RB, 32>), grid_b, block, 0, stream, p); \
  else hipLaunchKernelGGL((decode_balanced_bf16<RB, 32>), grid_b, block, 0, stream, p)
      switch (rank_bound) {   // 32-token steps (64 would leave one wave per SIMD at bound 96)
        case 32: KVLR_BAL_LAUNCH(32); break;
        case 64: KVLR_BAL_LAUNCH(64); break;
        case 96: KVLR_BAL_LAUNCH(96); break;
        default: KVLR_BAL_LAUNCH(128); break;
#undef KVLR_BAL_LAUNCH
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
