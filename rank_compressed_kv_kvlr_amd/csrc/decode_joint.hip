// Decode attention with joint value latents in bf16 (gfx950): the STAR-KV
// hybrid decomposition (STAR-KV technical summary, "Metodologia" section 2)
// keeps keys per KV head and stores one value latent per token for all heads,
// so one workgroup can stream every head's keys and the shared value latent of
// a token range once. Three launches: the query projection, the split kernel,
// and a merge with one workgroup per (query head, batch row).
#include "decode_common.hpp"

namespace kvlr {
namespace {

// ---------------------------------------------------------------------------
// joint value latents in bf16 (STAR-KV technical summary, "Metodologia"
// section 2: keys per head, one value latent per token shared by every head)
// ---------------------------------------------------------------------------
// q~ = q P_K for every query head, written to the workspace: one workgroup per
// (KV head, group of <= 4 query heads, batch row), the prologue of the
// per-head kernels on its own.
template <int RB>
__global__ __launch_bounds__(256) void project_queries(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) float smem[kHeadsPerWg * 256 + kHeadsPerWg * RB + kWaves * kHeadsPerWg * RB];
  const int h = blockIdx.x / p.n_head_groups;
  const int hg = blockIdx.x - h * p.n_head_groups;
  const int b = blockIdx.y;
  const int hq0 = h * p.G + hg * kHeadsPerWg;
  const int gpw = min(kHeadsPerWg, p.G - hg * kHeadsPerWg);
  const int rk = p.ht.rk[h];
  float* q_lds = smem;
  float* qt_lds = smem + kHeadsPerWg * 256;
  float* red = qt_lds + kHeadsPerWg * RB;
  project_query<RB>(p, b, h, hq0, gpw, rk, q_lds, red, qt_lds);
  for (int idx = threadIdx.x; idx < gpw * rk; idx += blockDim.x) {
    const int g = idx / rk, j = idx - g * rk;
    p.qt_out[((size_t)b * p.Hq + hq0 + g) * p.qt_stride + j] = qt_lds[g * RB + j];
  }
}

// Split kernel. One workgroup per (split, batch row) streams the keys of every
// KV head and the shared value latent of its token range once. Query heads are
// taken in row tiles of qpt = min(16, 4 G) (four KV heads, or 16 query heads
// when G > 4); a wave owns one row tile and one token stream (16-token blocks
// dealt round robin to the streams).
// Scores are formed transposed, S^T = K q~^T (v_mfma_f32_16x16x32_bf16 with key
// rows as the A operand, q~ as B): the KV heads of a row tile chain into one
// accumulator, each with a B operand that is zero outside its own query
// columns. A lane then holds 4 consecutive tokens of one query head, which is
// the A operand of the value product o_lat[qh][ch] += sum_t p[qh][t] V_lat[t][ch]
// (v_mfma_f32_16x16x16_bf16; p as a high and a low bf16 part), so the softmax
// weights stay in registers; the value rows are stored in that product's
// B-operand order (v_joint_offset). The waves of a row tile are merged through
// LDS into one record per (query head, split); merge_heads combines the splits.
template <int RK, int NB>
__global__ __launch_bounds__(256) void decode_split_joint(DecodeParams p) {
  constexpr int NP = RK / 32;          // key channel pairs bound
  constexpr int kSlots = 4;            // KV heads per row tile
  constexpr int kVP = kMaxRank / 32;   // value channel pairs bound
  constexpr int kCT = kMaxRank / 16;   // value column tiles bound
  constexpr int kRS = kMaxRank + 4;    // LDS row stride of the wave merge
  constexpr int TT = 16 * NB;          // tokens per wave step (NB 16-token blocks)
  __shared__ __attribute__((aligned(16))) float red[kWaves * 16 * kRS];
  __shared__ float wm[kWaves * 16], wl[kWaves * 16];

  const int s = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: slots, pointers in SGPRs
  const int n16 = lane & 15, q4 = lane >> 4;
  const int G = p.G, Hq = p.Hq;
  const int r = p.ht.rv[0];
  const int qpt = min(16, 4 * G);
  const int n_rt = (Hq + qpt - 1) / qpt;   // 1 or 2 (at most 32 query heads and 8 KV heads)
  const int n_streams = kWaves / n_rt;
  const int rt = wave % n_rt, ts = wave / n_rt;
  const int T = min(max(p.seq_lens[b], 0), p.cap);
  const int t_begin = min(s * p.split_len, T);
  const int t_end = min(T, t_begin + p.split_len);
  if (t_begin >= t_end) {
    write_empty_records(p, b, 0, Hq, s, r);
    return;
  }

  // this lane's query column and the KV heads of the row tile
  const int qh = rt * qpt + n16;
  const bool q_ok = n16 < qpt && qh < Hq;
  const int hq = q_ok ? qh / G : -1;
  const int h0 = __builtin_amdgcn_readfirstlane((rt * qpt) / G);
  const int n_slots = __builtin_amdgcn_readfirstlane((min(Hq, (rt + 1) * qpt) - 1) / G - h0 + 1);   // <= 4
  const size_t rows = cap_rows_of(p.cap);
  const uint16_t* Kb[kSlots];
  int rks[kSlots];
#pragma unroll
  for (int k = 0; k < kSlots; ++k) {
    const int hk = min(h0 + k, p.Hkv - 1);
    rks[k] = __builtin_amdgcn_readfirstlane(k < n_slots ? p.ht.rk[hk] : 0);
    Kb[k] = static_cast<const uint16_t*>(p.lat_k) + rows * ((size_t)b * p.Sk + p.ht.sk_pre[hk]);
  }
  const uint16_t* Vb = static_cast<const uint16_t*>(p.lat_v) + rows * (size_t)b * p.Sv;
  const int vnp = r >> 5, vtail = (r >> 4) & 1;

  // One step = NB 16-token blocks. Blocks wholly past the sequence end re-read the
  // last valid block; every token of theirs is masked below.
  const int last_blk = (t_end - 1) >> 4;
  u32x4_t kreg[NB][kSlots][NP];
  u32x2_t ktail[NB][kSlots];
  u32x4_t vreg[NB][kVP];   // pair c: channels 32 c + n16 and 32 c + 16 + n16; a 16-channel tail fills the first half
  auto load_k = [&](int t0) {
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const size_t row0 = (size_t)min((t0 >> 4) + blk, last_blk) * 16;
#pragma unroll
      for (int k = 0; k < kSlots; ++k) {
        const int rk = rks[k];
        const uint16_t* kb = Kb[k] + row0 * rk;
#pragma unroll
        for (int pp = 0; pp < NP; ++pp)
          if (pp < (rk >> 5)) kreg[blk][k][pp] = load_stream16(kb + pp * 512 + lane * 8);
        if ((rk >> 4) & 1) ktail[blk][k] = load_stream8(kb + (rk >> 5) * 512 + lane * 4);
      }
    }
  };
  auto load_v = [&](int t0) {
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const uint16_t* vb = Vb + (size_t)min((t0 >> 4) + blk, last_blk) * 16 * r;
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

  // q~ of this lane's query head as B operands (high and low bf16 parts), in
  // log2 units: pairs cover channels 32 pp + 8 q4 + e, the 16-channel tail of
  // the head's rank channels 32 np + 4 q4 + e. Its loads go first, so that
  // forming the operands waits for them alone, not for the first tile's.
  const int rk_own = q_ok ? p.ht.rk[hq] : 0;
  const float* qrow = p.qt_in + ((size_t)b * Hq + (q_ok ? qh : 0)) * p.qt_stride;
  float4 qx[NP][2];
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
    const int j0 = 32 * pp + 8 * q4;
    qx[pp][0] = qx[pp][1] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (j0 < rk_own) {
      qx[pp][0] = *reinterpret_cast<const float4*>(qrow + j0);
      qx[pp][1] = *reinterpret_cast<const float4*>(qrow + j0 + 4);
    }
  }
  float4 qtail = make_float4(0.f, 0.f, 0.f, 0.f);
  if ((rk_own >> 4) & 1) qtail = *reinterpret_cast<const float4*>(qrow + 32 * (rk_own >> 5) + 4 * q4);

  int t0 = t_begin + TT * ts;
  if (t0 < t_end) {
    load_k(t0);
    load_v(t0);
  }

  bf16x8_t a_hi[NP], a_lo[NP];
  bf16x4_t t_hi, t_lo;
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
    const float4 x0 = qx[pp][0], x1 = qx[pp][1];
    const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = x[e] * p.scale_log2;
      const uint16_t hi = f32_to_bf16_bits(v);
      a_hi[pp][e] = (short)hi;
      a_lo[pp][e] = (short)f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
    }
  }
  {
    const float4 x = qtail;
    const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = xs[e] * p.scale_log2;
      const uint16_t hi = f32_to_bf16_bits(v);
      t_hi[e] = (short)hi;
      t_lo[e] = (short)f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
    }
  }
  // per-slot lane masks (all ones where the lane's query head belongs to the
  // slot's KV head); an empty asm makes them opaque inside the loop so that the
  // masked operands are formed per use instead of being kept for every slot
  int slot_mask[kSlots];
#pragma unroll
  for (int k = 0; k < kSlots; ++k) slot_mask[k] = (hq == h0 + k) ? -1 : 0;

  float m = kNegInf, l = 0.f;
  f32x4_t acc[kCT];
#pragma unroll
  for (int c = 0; c < kCT; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (; t0 < t_end; t0 += TT * n_streams) {
    const int t_next = t0 + TT * n_streams;
    // ---- S^T[token][query] of each block, every KV head of the row tile chained
    f32x4_t sc[NB];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) sc[blk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kSlots; ++k) {
      if (k < n_slots) {
        asm volatile("" : "+v"(slot_mask[k]));
        const uint32_t mk = (uint32_t)slot_mask[k];
        const int rk = rks[k];
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) {
          if (pp < (rk >> 5)) {
            const bf16x8_t mh = __builtin_bit_cast(bf16x8_t, __builtin_bit_cast(u32x4_t, a_hi[pp]) & mk);
            const bf16x8_t ml = __builtin_bit_cast(bf16x8_t, __builtin_bit_cast(u32x4_t, a_lo[pp]) & mk);
#pragma unroll
            for (int blk = 0; blk < NB; ++blk) {
              const bf16x8_t kb = __builtin_bit_cast(bf16x8_t, kreg[blk][k][pp]);
              sc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, mh, sc[blk], 0, 0, 0);
              sc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, ml, sc[blk], 0, 0, 0);
            }
          }
        }
        if ((rk >> 4) & 1) {
          const bf16x4_t mh = __builtin_bit_cast(bf16x4_t, __builtin_bit_cast(u32x2_t, t_hi) & mk);
          const bf16x4_t ml = __builtin_bit_cast(bf16x4_t, __builtin_bit_cast(u32x2_t, t_lo) & mk);
#pragma unroll
          for (int blk = 0; blk < NB; ++blk) {
            const bf16x4_t kb = __builtin_bit_cast(bf16x4_t, ktail[blk][k]);
            sc[blk] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kb, mh, sc[blk], 0, 0, 0);
            sc[blk] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kb, ml, sc[blk], 0, 0, 0);
          }
        }
      }
    }
    if (t_next < t_end) load_k(t_next);   // key registers are free again

    // ---- online softmax: lane (n16, q4) holds tokens t0 + 16 blk + 4 q4 + i of query column n16
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

  // ---- merge the token streams of each row tile: the waves of streams > 0 leave
  // their state in LDS, the stream-0 wave adds it to its own and writes one record
  // per (query head, split). Accumulator rows are query heads 4 q4 + i.
  l = sum_over_rows(l);
  if (q4 == 0) {
    wm[wave * 16 + n16] = m;
    wl[wave * 16 + n16] = l;
  }
  if (ts > 0) {
    float* dst = red + (size_t)(wave - n_rt) * 16 * kRS;   // wave - n_rt = (ts - 1) * n_rt + rt
#pragma unroll
    for (int c = 0; c < kCT; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(4 * q4 + i) * kRS + 16 * c + n16] = acc[c][i];
  }
  __syncthreads();
  if (ts != 0) return;
  float f[kWaves][4], M[4], L[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ql = 4 * q4 + i;
    M[i] = kNegInf;
    for (int st = 0; st < n_streams; ++st) M[i] = fmaxf(M[i], wm[(st * n_rt + rt) * 16 + ql]);
    L[i] = 0.f;
#pragma unroll
    for (int st = 0; st < kWaves; ++st) {
      const float ms = st < n_streams ? wm[(st * n_rt + rt) * 16 + ql] : kNegInf;
      f[st][i] = M[i] == kNegInf ? 0.f : fast_exp2(ms - M[i]);   // idle stream: exp2(-inf) = 0
      if (st < n_streams) L[i] = fmaf(f[st][i], wl[(st * n_rt + rt) * 16 + ql], L[i]);
    }
  }
  float* rec[4];
  bool row_ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ql = 4 * q4 + i, qh2 = rt * qpt + ql;
    row_ok[i] = ql < qpt && qh2 < Hq;
    rec[i] = p.ws + (((size_t)b * Hq + (row_ok[i] ? qh2 : 0)) * p.n_splits + s) * p.ws_stride;
    if (row_ok[i] && n16 == 0) {
      rec[i][0] = M[i];
      rec[i][1] = L[i];
    }
  }
  const int n_ct = r >> 4;
#pragma unroll
  for (int c = 0; c < kCT; ++c) {
    if (c < n_ct) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float o = f[0][i] * acc[c][i];
#pragma unroll
        for (int st = 1; st < kWaves; ++st)
          if (st < n_streams)
            o = fmaf(f[st][i], red[((size_t)((st - 1) * n_rt + rt) * 16 + 4 * q4 + i) * kRS + 16 * c + n16], o);
        if (row_ok[i]) rec[i][2 + 16 * c + n16] = o;
      }
    }
  }
}

// Merge of the split records of one query head (joint values): one workgroup
// per (query head, batch row). Thread (c4, sg) loads float4 c4 of the records
// of splits sg, sg + nsg, ... (16 per pass, all in flight at once); the record
// maxima go through LDS, the weighted sums are added across split groups
// through LDS. The normalised latent row is back-projected with the head's d
// rows of P_J (prefetched when the kernel starts), or written as it is.
constexpr int kMergeKS = 16;

__global__ __launch_bounds__(256) void merge_heads(MergeParams p) {
  __shared__ __attribute__((aligned(16))) float4 part_lds[256];
  __shared__ float m_lds[1024];
  __shared__ __attribute__((aligned(16))) float ofull[kMaxRank + 8];
  __shared__ __attribute__((aligned(16))) float olat[kMaxRank];
  __shared__ float mred[kWaves];
  const int qh = blockIdx.x, b = blockIdx.y;
  const int h = qh / p.G;
  const int r = p.ht.rv[h], d = p.d;
  const int stride = p.ws_stride, ns = p.n_splits;
  const int nc4 = stride >> 2;
  const int nsg = 256 / nc4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c4 = tid % nc4, sg = tid / nc4;
  const bool act = sg < nsg;
  const float* recs = p.ws + ((size_t)b * p.Hq + qh) * ns * stride;

  // basis rows: thread (dd, part) takes float4 slices part, part + tpr, ... of row dd
  int tpr = 1;
  while (tpr * 2 * d <= 256) tpr *= 2;
  const int dd = tid / tpr, part = tid - dd * tpr;
  const bool row_ok = !p.out_latent && dd < d;
  const int n4 = r >> 2;
  const float* prow = p.pv + (size_t)d * p.ht.rv_pre[h] + (size_t)(row_ok ? dd : 0) * r;
  float4 pf[kMergeKS];
#pragma unroll
  for (int k = 0; k < kMergeKS; ++k) {
    const int j4 = part + tpr * k;
    pf[k] = (row_ok && j4 < n4) ? *reinterpret_cast<const float4*>(prow + 4 * j4) : make_float4(0.f, 0.f, 0.f, 0.f);
  }

  float M = kNegInf;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < ns; s0 += nsg * kMergeKS) {
    float4 v[kMergeKS];
#pragma unroll
    for (int k = 0; k < kMergeKS; ++k) {
      const int sp = s0 + sg + nsg * k;
      v[k] = (act && sp < ns) ? *reinterpret_cast<const float4*>(recs + (size_t)sp * stride + 4 * c4)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float mx = kNegInf;
    if (act && c4 == 0) {
#pragma unroll
      for (int k = 0; k < kMergeKS; ++k) {
        const float ms = (s0 + sg + nsg * k < ns) ? v[k].x : kNegInf;
        m_lds[sg * kMergeKS + k] = ms;
        mx = fmaxf(mx, ms);
      }
    }
    mx = wave_allreduce<true>(mx);
    if (lane == 0) mred[wave] = mx;
    __syncthreads();
    const float Mn = fmaxf(M, fmaxf(fmaxf(mred[0], mred[1]), fmaxf(mred[2], mred[3])));
    if (Mn != kNegInf && act) {
      const float a = fast_exp2(M - Mn);   // first pass: exp2(-inf) = 0
      acc.x *= a;
      acc.y *= a;
      acc.z *= a;
      acc.w *= a;
#pragma unroll
      for (int k = 0; k < kMergeKS; ++k) {
        const float f = fast_exp2(m_lds[sg * kMergeKS + k] - Mn);   // empty or absent split: 0
        acc.x = fmaf(f, v[k].x, acc.x);
        acc.y = fmaf(f, v[k].y, acc.y);
        acc.z = fmaf(f, v[k].z, acc.z);
        acc.w = fmaf(f, v[k].w, acc.w);
      }
    }
    M = Mn;
    __syncthreads();   // m_lds and mred are rewritten by the next pass
  }
  part_lds[tid] = acc;
  __syncthreads();
  if (tid < nc4) {
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int g = 0; g < nsg; ++g) {
      const float4 u = part_lds[g * nc4 + tid];
      t.x += u.x;
      t.y += u.y;
      t.z += u.z;
      t.w += u.w;
    }
    *reinterpret_cast<float4*>(ofull + 4 * tid) = t;   // [m-sum (unused), L, o_lat ...]
  }
  __syncthreads();
  const float L = ofull[1];
  const float inv = L > 0.f ? 1.f / L : 0.f;   // empty sequence: zero output
  if (p.out_latent) {
    float* o = p.out + ((size_t)b * p.Hq + qh) * p.out_stride;
    for (int j = tid; j < p.out_stride; j += blockDim.x) o[j] = j < r ? ofull[2 + j] * inv : 0.f;
    return;
  }
  if (tid < r) olat[tid] = ofull[2 + tid] * inv;
  __syncthreads();
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < kMergeKS; ++k) {
    const int j4 = part + tpr * k;
    if (j4 < n4) {
      const float4 o4 = *reinterpret_cast<const float4*>(olat + 4 * j4);
      sum += pf[k].x * o4.x + pf[k].y * o4.y + pf[k].z * o4.z + pf[k].w * o4.w;
    }
  }
  for (int j4 = part + tpr * kMergeKS; j4 < n4; j4 += tpr) {   // rows wider than the prefetch (head_dim > 128)
    if (!row_ok) break;
    const float4 pv = *reinterpret_cast<const float4*>(prow + 4 * j4);
    const float4 o4 = *reinterpret_cast<const float4*>(olat + 4 * j4);
    sum += pv.x * o4.x + pv.y * o4.y + pv.z * o4.z + pv.w * o4.w;
  }
  for (int off = 1; off < tpr; off <<= 1) sum += __shfl_xor(sum, off, 64);
  if (row_ok && part == 0) p.out[((size_t)b * p.Hq + qh) * d + dd] = sum;
}

}  // namespace

hipError_t launch_project_queries(const DecodeParams& p, int rk_bound, hipStream_t stream) {
  const dim3 grid(p.Hkv * p.n_head_groups, p.B);
  switch (rk_bound) {
    case 32: hipLaunchKernelGGL(project_queries<32>, grid, dim3(256), 0, stream, p); break;
    case 64: hipLaunchKernelGGL(project_queries<64>, grid, dim3(256), 0, stream, p); break;
    case 96: hipLaunchKernelGGL(project_queries<96>, grid, dim3(256), 0, stream, p); break;
    default: hipLaunchKernelGGL(project_queries<128>, grid, dim3(256), 0, stream, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_decode_joint(const DecodeParams& p, int rk_bound, int blocks, hipStream_t stream) {
  const dim3 grid(p.n_splits, p.B);
  const dim3 block(kWaves * 64);
#define KVLR_JOINT_CASE(RK)                                                                   \
  case RK:                                                                                    \
    if (blocks == 2)                                                                          \
      hipLaunchKernelGGL((decode_split_joint<RK, 2>), grid, block, 0, stream, p);             \
    else                                                                                      \
      hipLaunchKernelGGL((decode_split_joint<RK, 1>), grid, block, 0, stream, p);             \
    break;
  switch (rk_bound) {
    KVLR_JOINT_CASE(32)
    KVLR_JOINT_CASE(64)
    KVLR_JOINT_CASE(96)
    default: KVLR_JOINT_CASE(128)
  }
#undef KVLR_JOINT_CASE
  return hipGetLastError();
}

hipError_t launch_merge_heads(const MergeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(merge_heads, dim3(p.Hq, p.B), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kvlr
