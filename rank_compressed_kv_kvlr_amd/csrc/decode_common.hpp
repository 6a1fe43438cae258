// Device helpers shared by the decode kernels (per-head and joint-value):
// the query projection prologue and the split-record accessors. Internal.
#pragma once

#include "kvlr_internal.hpp"

namespace kvlr {
namespace {

// threadIdx.x through an empty asm: a value the compiler cannot hoist out of a
// loop. Without it, the balanced decode kernel (a loop over segments, each the
// whole split body) keeps every lane-derived address of the body live across
// the loop and runs out of registers.
__device__ __forceinline__ int thread_id() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();

// A workgroup barrier for data exchanged through LDS by ds_read/ds_write: the
// wave's LDS accesses complete (lgkmcnt), then all waves meet. Unlike
// __syncthreads() it does not wait for outstanding vector-memory loads, so
// loads issued before it (including direct-to-LDS loads into a region the
// barrier does not guard) stay in flight. The memory clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------
// shared prologue: q~ = (q P_K) * scale * log2(e) for the workgroup's heads
// ---------------------------------------------------------------------------
// The four waves split the d rows of P_K[h]; each lane issues all of its
// 16-byte basis loads at once (one memory round trip), forms partial dot
// products for the 4 heads, and partials are summed across lanes with
// shuffles and across waves through LDS. With a caller-given q~ (bases
// folded into the query projection) the loads are of q~ itself.
//   q_lds [4][d], red [4 waves][4 heads][RB], qt_lds [4][RB]
template <int RB>
__device__ __forceinline__ void project_query(const DecodeParams& p, int b, int h, int hq0, int gpw, int rk,
                                              float* q_lds, float* red, float* qt_lds) {
  const int tid = thread_id(), lane = tid & 63, wave = tid >> 6;
  const int d = p.d;
  if (p.qt_in) {   // folded mode: q~ [B][Hq][qt_stride] given in latent space
    constexpr int kPer = (kHeadsPerWg * RB + 255) / 256;   // values per thread (256 threads)
    float v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int idx = tid + 256 * k, g = idx / RB, j = idx - g * RB;
      v[k] = (idx < kHeadsPerWg * RB && g < gpw && j < rk)
                 ? p.qt_in[((size_t)b * p.Hq + hq0 + g) * p.qt_stride + j] * p.scale_log2 : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      if (tid + 256 * k < kHeadsPerWg * RB) qt_lds[tid + 256 * k] = v[k];
    lds_barrier();
    return;
  }
  constexpr int NH = (RB + 63) / 64;      // 64-column halves of P
  constexpr int RPL = 16;                 // rows per lane bound: d / 16 <= 16
  const float* P = p.pk + (size_t)d * p.ht.rk_pre[h];
  const int isub = lane >> 4, m = lane & 15;
  const int rows_per_wave = d >> 2, rpl = d >> 4;
  float4 pr[RPL];
  // lanes past the rank take zeros without a load (their loads are masked off, so a
  // small rank reads only its own columns)
  auto load_half = [&](int hf) {
    const int col = 64 * hf + 4 * m;
    const bool ok = col < rk;
#pragma unroll
    for (int e = 0; e < RPL; ++e) {
      const int i = wave * rows_per_wave + isub + 4 * e;
      pr[e] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e < rpl && ok) pr[e] = *reinterpret_cast<const float4*>(P + (size_t)i * rk + col);
    }
  };
  load_half(0);   // basis loads in flight together with the query rows
  float qv[4];     // kHeadsPerWg * d <= 1024 values, 256 threads; invalid ones read row 0 and are masked
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = tid + 256 * k, g = idx / d, i = idx - g * d;
    const bool ok = idx < kHeadsPerWg * d && g < gpw;
    const float v = p.q[((size_t)b * p.Hq + hq0) * d + (ok ? g * d + i : 0)];
    qv[k] = ok ? v : 0.f;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (tid + 256 * k < kHeadsPerWg * d) q_lds[tid + 256 * k] = qv[k];
  lds_barrier();
#pragma unroll
  for (int hf = 0; hf < NH; ++hf) {
    const int col = 64 * hf + 4 * m;
    if (hf > 0 && 64 * hf >= rk) break;   // halves past the rank: nothing to load (red is read below rk only)
    if (hf > 0) load_half(hf);
    float part[4][4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) part[g][jj] = 0.f;
#pragma unroll
    for (int e = 0; e < RPL; ++e) {
      if (e < rpl) {
        const int i = wave * rows_per_wave + isub + 4 * e;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float qv = q_lds[g * d + i];
          part[g][0] = fmaf(qv, pr[e].x, part[g][0]);
          part[g][1] = fmaf(qv, pr[e].y, part[g][1]);
          part[g][2] = fmaf(qv, pr[e].z, part[g][2]);
          part[g][3] = fmaf(qv, pr[e].w, part[g][3]);
        }
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) part[g][jj] = sum_over_rows(part[g][jj]);
    if (isub == 0 && col < RB) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(red + (wave * 4 + g) * RB + col) =
            make_float4(part[g][0], part[g][1], part[g][2], part[g][3]);
    }
  }
  lds_barrier();
  for (int idx = tid; idx < kHeadsPerWg * RB; idx += blockDim.x) {
    const int g = idx / RB, j = idx - g * RB;
    float v = 0.f;
    if (g < gpw && j < rk)
      v = (red[(0 * 4 + g) * RB + j] + red[(1 * 4 + g) * RB + j] + red[(2 * 4 + g) * RB + j] +
           red[(3 * 4 + g) * RB + j]) * p.scale_log2;
    qt_lds[idx] = v;   // zero rows for heads beyond gpw and channels beyond rk
  }
  lds_barrier();
}

// Split records are written and read with agent-scope relaxed atomic
// accesses: on gfx950 these are plain stores/loads with the agent-coherence
// bit (sc1), so a record written by one workgroup is read back coherently by
// another workgroup on any XCD without a whole-L2 writeback.
__device__ __forceinline__ void store_rec(float* addr, float v) {
  __hip_atomic_store(addr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_rec(const float* addr) {
  return __hip_atomic_load(addr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Where a workgroup's split records live: record k of the group's head g
// (m, l, o_lat[r_v]) starts at base + k * k_stride + g * g_stride floats.
struct RecLayout {
  float* base;
  size_t k_stride, g_stride;
};
__device__ __forceinline__ float* rec_at(const RecLayout& rl, int k, int g) {
  return rl.base + (size_t)k * rl.k_stride + (size_t)g * rl.g_stride;
}
// Fixed split plan: records [B][Hq][n_splits][ws_stride], heads hq0 .. of batch row b.
__device__ __forceinline__ RecLayout fixed_records(const DecodeParams& p, int b, int hq0) {
  return RecLayout{p.ws + ((size_t)b * p.Hq + hq0) * p.n_splits * p.ws_stride, (size_t)p.ws_stride,
                   (size_t)p.n_splits * p.ws_stride};
}

// Record k of an empty split (m = -inf, l = 0, o_lat = 0) for heads 0 .. gpw-1.
__device__ __forceinline__ void write_empty_records(const RecLayout& rl, int k, int gpw, int rv) {
  for (int idx = thread_id(); idx < gpw * (rv + 2); idx += blockDim.x) {
    const int g = idx / (rv + 2), j = idx - g * (rv + 2);
    store_rec(rec_at(rl, k, g) + j, (j == 0) ? kNegInf : 0.f);
  }
}
__device__ __forceinline__ void write_empty_records(const DecodeParams& p, int b, int hq0, int gpw, int s, int rv) {
  write_empty_records(fixed_records(p, b, hq0), s, gpw, rv);
}

}  // namespace
}  // namespace kvlr
