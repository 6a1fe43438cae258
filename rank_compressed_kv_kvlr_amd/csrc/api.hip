// Host side of the libkvlr C ABI: argument validation, split planning and
// kernel launches on the caller's stream. Allocates nothing and never
// synchronises; the only state is per-device caches (the compute-unit count,
// the address of the static decode scratch). Every check runs before any
// work is enqueued.
#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <initializer_list>
#include <mutex>
#include <stdint.h>
#include <string.h>
#include <utility>
#include <vector>

#include "kvlr_internal.hpp"

namespace {

using kvlr::HeadTable;

constexpr int kVersion = 10000;   // 1.0.0
constexpr int kSplitGranule = kvlr::kTile;

// Compute units of the current device, queried once per device and cached. The
// plans size one round of workgroups over them, so a partitioned device (fewer
// CUs per logical device) gets plans for what it has. Without a device (size
// queries on a host with no GPU) the MI355X count is assumed.
constexpr int kDefaultComputeUnits = 256;
constexpr int kMaxDevices = 64;
std::atomic<int> g_compute_units[kMaxDevices];   // 0: not queried yet

int compute_units() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return kDefaultComputeUnits;
  int n = g_compute_units[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = kDefaultComputeUnits;
  g_compute_units[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Tuning overrides from the environment, read once, the first time a plan is
// made (see kvlr.h); later changes to the environment have no effect.
struct Tuning {
  long long split_tokens;   // KVLR_SPLIT_TOKENS: tokens per split of the fixed plan (0: library choice)
  int balance_fixed;        // KVLR_BALANCE_FIXED: fixed work per token of the balanced plan (-1: default)
  int tile;                 // KVLR_TILE: 64-token wave steps of the bf16 split kernel (default 32)
};
const Tuning& tuning() {
  static const Tuning t = [] {
    Tuning r{0, -1, 32};
    if (const char* e = getenv("KVLR_SPLIT_TOKENS")) r.split_tokens = atoll(e);
    if (const char* e = getenv("KVLR_BALANCE_FIXED")) r.balance_fixed = atoi(e);
    if (const char* e = getenv("KVLR_TILE")) r.tile = atoi(e) == 64 ? 64 : 32;
    return r;
  }();
  return t;
}

// Resident split workgroups per CU for each kernel variant (4 waves each;
// limited by the variant's register count on gfx950). The default split
// length gives one such round of workgroups over the whole device.
int resident_wgs_per_cu(int latent_dtype, int rank_bound) {
  if (latent_dtype == KVLR_BF16) return rank_bound <= 32 ? 3 : 2;   // measured best
  if (latent_dtype == KVLR_Q43) return rank_bound <= 64 ? 3 : 2;   // 3 waves per SIMD up to rank 64
  return 3;   // fp32 variants: limited by the 48 KiB of LDS the merge tail needs
}

// Split workgroups per CU of the joint-value kernel (one per (split, batch row)).
constexpr int kJointResident = 2;

bool valid_dtype(int t) { return t == KVLR_F32 || t == KVLR_BF16; }

// Joint values in bf16 run the joint split kernel (its own value layout, a
// separate query projection and merge); every other combination the per-head kernels.
bool joint_bf16(const kvlr_desc* d) {
  return d->value_mode == KVLR_VALUES_JOINT && d->latent_dtype == KVLR_BF16;
}

int rank_bound_of(int r) { return r <= 32 ? 32 : r <= 64 ? 64 : r <= 96 ? 96 : 128; }

// Balanced plan (bf16 latents, per-head values, single-launch decode): the kernel
// reads seq_lens and gives every workgroup an equal share of the bytes. Taken on
// request (split_tokens = -1) and by default when the KV heads' ranks differ; the
// batch's prefix sums live in LDS (int64) and the kernel's 64-bit work positions
// times the workgroup count must not overflow.
constexpr int kSplitBalanced = -1;
constexpr int kTokenFixedCost = 512;   // measured on ragged per-head ranks 16..96 (256..2048 within 3%)
constexpr int kMaxBalancedBatch = 4096;

int head_groups_of(const kvlr_desc* d) {
  return (d->n_q_heads / d->n_kv_heads + kvlr::kHeadsPerWg - 1) / kvlr::kHeadsPerWg;
}

// Work of one token of KV head h in the balanced plan: its latent elements plus a
// fixed part for the arithmetic every token costs whatever its rank (softmax,
// masks, loop control); KVLR_BALANCE_FIXED overrides the fixed part for tuning.
int token_fixed_cost() {
  const int v = tuning().balance_fixed;
  if (v < 0) return kTokenFixedCost;
  return v > 4096 ? 4096 : v;
}
// With one segment per workgroup the steps of a segment are bound by memory latency
// more than by its bytes: a token costs nearly the same at every rank (on ragged
// per-head ranks 16..96: 14.6 us per 1000 tokens at r_k + r_v = 48, 16.6 at 176).
constexpr int kTokenFixedCostOneSegment = 896;
int token_cost(const kvlr_desc* d, int h, bool one_segment = false) {
  return (one_segment ? kTokenFixedCostOneSegment : token_fixed_cost()) + d->r_k[h] + d->r_v[h];
}

long long row_cost_of(const kvlr_desc* d, bool one_segment = false) {
  long long c = 0;
  for (int h = 0; h < d->n_kv_heads; ++h) c += token_cost(d, h, one_segment);
  return c * head_groups_of(d);
}

bool ranks_differ(const kvlr_desc* d) {
  for (int h = 1; h < d->n_kv_heads; ++h)
    if (d->r_k[h] != d->r_k[0] || d->r_v[h] != d->r_v[0]) return true;
  return false;
}

bool supports_balanced(const kvlr_desc* d) {
  if (d->latent_dtype != KVLR_BF16 || d->value_mode != KVLR_VALUES_PER_HEAD) return false;
  if (d->batch > kMaxBalancedBatch) return false;
  return (long long)d->batch * d->capacity * row_cost_of(d) <= (1LL << 46);   // row_cost <= 2^20 x 4 groups
}

bool balanced_plan(const kvlr_desc* d, int32_t split_tokens) {
  return supports_balanced(d) && (split_tokens == kSplitBalanced || (split_tokens == 0 && ranks_differ(d)));
}

// Workgroups of the balanced plan: one round over the device.
int balanced_wgs(const kvlr_desc* d, int rank_bound) {
  return compute_units() * resident_wgs_per_cu(d->latent_dtype, rank_bound);
}
// The balanced plan's one-segment-per-workgroup form (three workgroups per CU up to
// rank bound 96), used while the (row, KV head, head group) units are few next to
// the workgroups: the apportionment needs about two workgroups per unit or more.
int one_segment_wgs(int rank_bound) { return compute_units() * (rank_bound <= 96 ? 3 : 2); }
bool one_segment_plan(const kvlr_desc* d, int rank_bound) {
  const long long units = (long long)d->batch * d->n_kv_heads * head_groups_of(d);
  return units * 2 <= one_segment_wgs(rank_bound) && d->batch * d->n_kv_heads <= kvlr::kApportionPairs;
}
int balanced_grid(const kvlr_desc* d, int rank_bound) {
  return one_segment_plan(d, rank_bound) ? one_segment_wgs(rank_bound) : balanced_wgs(d, rank_bound);
}

// Largest key rank and its kernel bound.
int rk_max_of(const kvlr_desc* d) {
  int m = 0;
  for (int h = 0; h < d->n_kv_heads; ++h) m = d->r_k[h] > m ? d->r_k[h] : m;
  return m;
}

// Buffers the kernels access with 16-byte vector loads or stores (K/V rows, latent
// caches, bases, workspace) must start on a 16-byte boundary. NULLs pass (they are
// checked separately).
bool aligned16(std::initializer_list<const void*> ptrs) {
  uintptr_t bits = 0;
  for (const void* ptr : ptrs) bits |= (uintptr_t)ptr;
  return (bits & 15) == 0;
}
bool valid_latent_dtype(int t) { return valid_dtype(t) || t == KVLR_Q43; }

// Storage of one latent row of rank r: elements, or bytes for 4/3-bit rows.
int row_storage(int latent_dtype, int r) { return latent_dtype == KVLR_Q43 ? kvlr::q43_row_bytes(r) : r; }

// Validates the descriptor and fills the per-head tables (ranks, rank and
// storage prefix sums); Sk / Sv receive the per-row storage summed over heads.
int check_desc(const kvlr_desc* d, HeadTable* ht, int* Rk, int* Rv, int* rank_bound, int* Sk = nullptr,
               int* Sv = nullptr) {
  if (!d || !d->r_k || !d->r_v) return KVLR_ERR_NULL;
  if (!valid_dtype(d->in_dtype) || !valid_latent_dtype(d->latent_dtype)) return KVLR_ERR_DTYPE;
  if (d->batch < 1 || d->n_kv_heads < 1 || d->n_kv_heads > kvlr::kMaxKvHeads || d->n_q_heads < 1 ||
      d->n_q_heads % d->n_kv_heads != 0 || d->n_q_heads / d->n_kv_heads > 16 || d->capacity < 1 ||
      d->head_dim < 32 || d->head_dim > 256 || d->head_dim % 32 != 0 || d->capacity > (1 << 30))
    return KVLR_ERR_SHAPE;
  if (d->value_mode != KVLR_VALUES_PER_HEAD && d->value_mode != KVLR_VALUES_JOINT) return KVLR_ERR_ARG;
  // 4/3-bit blocks are addressed with 32-bit buffer offsets: a (row, head) block of
  // cap rows (rounded up to 32) at up to 60 bytes each stays below 2^31 bytes
  if (d->latent_dtype == KVLR_Q43 && (long long)kvlr::cap_rows_q43(d->capacity) * 60 >= (1LL << 31))
    return KVLR_ERR_SHAPE;
  const bool joint = d->value_mode == KVLR_VALUES_JOINT;
  // the joint bf16 kernel holds at most two 16-query row tiles of four KV heads
  if (joint && d->latent_dtype == KVLR_BF16 && (d->n_q_heads > 32 || d->n_kv_heads > 8)) return KVLR_ERR_SHAPE;
  const int granule = d->latent_dtype == KVLR_F32 ? 4 : 16;
  const int rmax = d->head_dim < kvlr::kMaxRank ? d->head_dim : kvlr::kMaxRank;
  const long long jmax_ll = (long long)d->n_kv_heads * d->head_dim;
  const int rvmax = joint ? (int)(jmax_ll < kvlr::kMaxRank ? jmax_ll : kvlr::kMaxRank) : rmax;
  int sk = 0, sv = 0, bound = 0, stk = 0, stv = 0;
  for (int h = 0; h < d->n_kv_heads; ++h) {
    const int rk = d->r_k[h], rv = d->r_v[h];
    if (rk < 1 || rv < 1 || rk > rmax || rv > rvmax || rk % granule || rv % granule) return KVLR_ERR_RANK;
    if (joint && rv != d->r_v[0]) return KVLR_ERR_RANK;   // one joint rank
    if (ht) {
      ht->rk[h] = rk;
      ht->rv[h] = rv;
      ht->rk_pre[h] = sk;
      ht->rv_pre[h] = sv;
      ht->sk_pre[h] = stk;
      ht->sv_pre[h] = joint ? 0 : stv;   // joint values: every head reads the batch row's block
    }
    sk += rk;
    sv += rv;
    stk += row_storage(d->latent_dtype, rk);
    if (!joint || h == 0) stv += row_storage(d->latent_dtype, rv);
    bound = rk > bound ? rk : bound;
    bound = rv > bound ? rv : bound;
  }
  // every per-(b, h) block offset T_cap * (b * R + R_pre) must fit comfortably in size_t;
  // kernels index rows with 32-bit token counts
  if ((long long)d->capacity * d->batch * (stk > stv ? stk : stv) > (1LL << 46)) return KVLR_ERR_SHAPE;
  if (Rk) *Rk = sk;
  if (Rv) *Rv = sv;
  if (Sk) *Sk = stk;
  if (Sv) *Sv = stv;
  if (rank_bound) *rank_bound = rank_bound_of(bound);
  return KVLR_OK;
}

// Split plan of the decode kernels: one split length for every KV head.
// With split_tokens > 0 that length; with 0 the library sizes the splits so
// that one round of workgroups fills the device. (Rank-weighted per-head
// lengths were measured slower on ragged batches: the extra, shorter splits of
// the heavy heads spill into a second round.) split_len (optional) receives the
// per-head lengths the kernels read.
int plan_split(const kvlr_desc* d, int32_t split_tokens, int* n_splits, int* len_out, int* split_len = nullptr) {
  int rank_bound = 0;
  check_desc(d, nullptr, nullptr, nullptr, &rank_bound);   // callers validated the descriptor already
  const int G = d->n_q_heads / d->n_kv_heads;
  const int groups = (G + kvlr::kHeadsPerWg - 1) / kvlr::kHeadsPerWg;
  int len;
  if (split_tokens == kSplitBalanced) split_tokens = 0;   // the fixed plan behind a balanced request
  if (split_tokens < 0 || split_tokens % kSplitGranule != 0) return KVLR_ERR_ARG;
  if (split_tokens > 0) {
    len = split_tokens;
  } else {
    long long want = tuning().split_tokens;   // tuning override
    if (want <= 0 || want % kSplitGranule) {
      const bool jd = joint_bf16(d);   // one workgroup per (split, batch row)
      const long long units = jd ? (long long)d->batch : (long long)d->batch * d->n_kv_heads * groups;
      const long long slots =
          (long long)compute_units() * (jd ? kJointResident : resident_wgs_per_cu(d->latent_dtype, rank_bound));
      want = (units * d->capacity + slots - 1) / slots;
      // whole tiles for every wave; the 4/3-bit kernel steps 32 rows at a time, so any
      // multiple of the granule keeps whole steps (measured: 2752 against 2816 tokens,
      // 88.3 against 89.8 us on an 8 x 32768-token batch at rank 64)
      const long long g4 = d->latent_dtype == KVLR_Q43 ? kSplitGranule : (long long)kSplitGranule * kvlr::kWaves;
      want = (want + g4 - 1) / g4 * g4;
      if (want < g4) want = g4;
    }
    len = want > d->capacity ? ((d->capacity + kSplitGranule - 1) / kSplitGranule) * kSplitGranule : (int)want;
  }
  const long long ns = ((long long)d->capacity + len - 1) / len;
  if (ns > 65535) return KVLR_ERR_ARG;   // grid.x limit of the split kernel
  *n_splits = (int)ns;
  *len_out = len;
  if (split_len)
    for (int h = 0; h < d->n_kv_heads; ++h) split_len[h] = len;
  return KVLR_OK;
}

int ws_stride_of(const HeadTable& ht, int Hkv) {
  int m = 0;
  for (int h = 0; h < Hkv; ++h) m = ht.rv[h] > m ? ht.rv[h] : m;
  return (m + 2 + 3) / 4 * 4;
}

// Record region of the workspace: [B][Hq][n_splits][stride] fp32 for the fixed
// plan; with split_tokens 0 or -1 on caches that allow the balanced plan, also
// room for its (n_wg + B Hkv head_groups) slots of 4 records, so that one
// workspace serves both plans.
size_t record_bytes_of(const kvlr_desc* d, const HeadTable& ht, int32_t split_tokens, int n_splits, int rank_bound) {
  const size_t stride = ws_stride_of(ht, d->n_kv_heads);
  size_t bytes = (size_t)d->batch * d->n_q_heads * n_splits * stride * sizeof(float);
  if ((split_tokens == 0 || split_tokens == kSplitBalanced) && supports_balanced(d)) {
    size_t slots = (size_t)balanced_wgs(d, rank_bound) + (size_t)d->batch * d->n_kv_heads * head_groups_of(d);
    if ((size_t)one_segment_wgs(rank_bound) > slots) slots = one_segment_wgs(rank_bound);
    const size_t bal = slots * kvlr::kHeadsPerWg * stride * sizeof(float);
    bytes = bal > bytes ? bal : bytes;
  }
  return bytes;
}

int hip_status(hipError_t e) { return e == hipSuccess ? KVLR_OK : KVLR_ERR_HIP; }

// Tokens per wave iteration of the bf16 split kernel (32 or 64; 32 measured
// faster: fewer registers, 3 waves per SIMD at rank 64); KVLR_TILE overrides
// for tuning.
int decode_tile() { return tuning().tile; }

// Workspace layout: arrival counters [B][Hkv][head groups] int32, padded to
// 256 bytes, then the split records [B][Hq][n_splits][stride] fp32, then (joint
// bf16 values) the projected queries [B][Hq][max_h r_k[h]] fp32.
size_t counter_bytes_of(const kvlr_desc* d) {
  const int G = d->n_q_heads / d->n_kv_heads;
  const size_t groups = (size_t)(G + kvlr::kHeadsPerWg - 1) / kvlr::kHeadsPerWg;
  const size_t n = (size_t)d->batch * d->n_kv_heads * groups * sizeof(int32_t);
  return (n + 255) / 256 * 256;
}

size_t qt_bytes_of(const kvlr_desc* d) {
  return joint_bf16(d) ? (size_t)d->batch * d->n_q_heads * rk_max_of(d) * sizeof(float) : 0;
}

}  // namespace

extern "C" {

KVLR_API int kvlr_version(void) { return kVersion; }

KVLR_API const char* kvlr_status_string(int status) {
  switch (status) {
    case KVLR_OK: return "ok";
    case KVLR_ERR_NULL: return "a required pointer is NULL";
    case KVLR_ERR_SHAPE: return "inconsistent or unsupported shape";
    case KVLR_ERR_RANK: return "rank out of range or not a multiple of the storage granule";
    case KVLR_ERR_DTYPE: return "unsupported dtype";
    case KVLR_ERR_WORKSPACE: return "workspace missing or too small";
    case KVLR_ERR_HIP: return "HIP launch failed";
    case KVLR_ERR_ARG: return "invalid scalar argument";
    case KVLR_ERR_SCRATCH: return "the call needs more decode scratch than the library's static array holds";
    default: return "unknown status";
  }
}

KVLR_API int kvlr_cache_elems(const kvlr_desc* desc, size_t* k_elems, size_t* v_elems) {
  int Sk = 0, Sv = 0;
  const int rc = check_desc(desc, nullptr, nullptr, nullptr, nullptr, &Sk, &Sv);
  if (rc) return rc;
  if (!k_elems || !v_elems) return KVLR_ERR_NULL;
  const size_t rows = (size_t)(desc->latent_dtype == KVLR_Q43 ? kvlr::cap_rows_q43(desc->capacity)
                                                               : kvlr::cap_rows_of(desc->capacity));
  *k_elems = (size_t)desc->batch * rows * Sk;
  *v_elems = (size_t)desc->batch * rows * Sv;
  return KVLR_OK;
}

KVLR_API int kvlr_decode_plan(const kvlr_desc* desc, int32_t split_tokens, int32_t* n_splits,
                              int32_t* tokens_per_split) {
  int rc = check_desc(desc, nullptr, nullptr, nullptr, nullptr);
  if (rc) return rc;
  if (!n_splits || !tokens_per_split) return KVLR_ERR_NULL;
  int ns = 0, len = 0;
  rc = plan_split(desc, split_tokens, &ns, &len);
  if (rc) return rc;
  if (balanced_plan(desc, split_tokens)) {   // workgroups of equal shares; no fixed split length
    int rank_bound = 0;
    check_desc(desc, nullptr, nullptr, nullptr, &rank_bound);
    ns = balanced_grid(desc, rank_bound);
    len = 0;
  }
  *n_splits = ns;
  *tokens_per_split = len;
  return KVLR_OK;
}

KVLR_API int kvlr_decode_workspace_bytes(const kvlr_desc* desc, int32_t split_tokens, size_t* bytes) {
  HeadTable ht;
  int rank_bound = 0;
  int rc = check_desc(desc, &ht, nullptr, nullptr, &rank_bound);
  if (rc) return rc;
  if (!bytes) return KVLR_ERR_NULL;
  int ns = 0, len = 0;
  rc = plan_split(desc, split_tokens, &ns, &len);
  if (rc) return rc;
  *bytes = counter_bytes_of(desc) + record_bytes_of(desc, ht, split_tokens, ns, rank_bound) + qt_bytes_of(desc);
  return KVLR_OK;
}

KVLR_API int kvlr_decode_counter_bytes(const kvlr_desc* desc, size_t* bytes) {
  const int rc = check_desc(desc, nullptr, nullptr, nullptr, nullptr);
  if (rc) return rc;
  if (!bytes) return KVLR_ERR_NULL;
  *bytes = counter_bytes_of(desc);
  return KVLR_OK;
}

KVLR_API int kvlr_prefill_compress(const kvlr_desc* desc, const void* K, const void* V, int32_t start,
                                   int32_t n_tok, const float* P_K, const float* P_V, void* lat_k,
                                   void* lat_v, void* stream) {
  kvlr::CompressParams p;
  int rc = check_desc(desc, &p.ht, &p.Rk, &p.Rv, nullptr, &p.Sk, &p.Sv);
  if (rc) return rc;
  if (start < 0 || n_tok < 0) return KVLR_ERR_ARG;
  if ((long long)start + n_tok > desc->capacity) return KVLR_ERR_SHAPE;
  if (n_tok == 0) return KVLR_OK;
  if (!K || !V || !P_K || !P_V || !lat_k || !lat_v) return KVLR_ERR_NULL;
  if (!aligned16({K, V, P_K, P_V, lat_k, lat_v})) return KVLR_ERR_ARG;
  if ((long long)desc->batch * n_tok * desc->n_kv_heads * desc->head_dim > (1LL << 40)) return KVLR_ERR_SHAPE;
  p.x_k = K;
  p.x_v = V;
  p.pk = P_K;
  p.pv = P_V;
  p.lat_k = lat_k;
  p.lat_v = lat_v;
  p.B = desc->batch;
  p.Hkv = desc->n_kv_heads;
  p.d = desc->head_dim;
  p.cap = desc->capacity;
  p.start = start;
  p.n_tok = n_tok;
  p.in_bf16 = desc->in_dtype == KVLR_BF16;
  p.out_bf16 = desc->latent_dtype == KVLR_BF16;
  p.out_q43 = desc->latent_dtype == KVLR_Q43;
  p.joint_v = desc->value_mode == KVLR_VALUES_JOINT;
  p.only_kind = -1;
  p.n_cu = compute_units();
  return hip_status(kvlr::launch_compress(p, static_cast<hipStream_t>(stream)));
}

KVLR_API int kvlr_append(const kvlr_desc* desc, const void* k_new, const void* v_new, const int32_t* pos,
                         const float* P_K, const float* P_V, void* lat_k, void* lat_v, void* stream) {
  kvlr::AppendParams p;
  const int rc = check_desc(desc, &p.ht, &p.Rk, &p.Rv, nullptr, &p.Sk, &p.Sv);
  if (rc) return rc;
  if (!k_new || !v_new || !pos || !P_K || !P_V || !lat_k || !lat_v) return KVLR_ERR_NULL;
  if (!aligned16({P_K, P_V, lat_k, lat_v})) return KVLR_ERR_ARG;
  p.k_new = k_new;
  p.v_new = v_new;
  p.pos = pos;
  p.pk = P_K;
  p.pv = P_V;
  p.lat_k = lat_k;
  p.lat_v = lat_v;
  p.B = desc->batch;
  p.Hkv = desc->n_kv_heads;
  p.d = desc->head_dim;
  p.cap = desc->capacity;
  p.in_bf16 = desc->in_dtype == KVLR_BF16;
  p.out_bf16 = desc->latent_dtype == KVLR_BF16;
  p.out_q43 = desc->latent_dtype == KVLR_Q43;
  p.joint_v = desc->value_mode == KVLR_VALUES_JOINT;
  return hip_status(kvlr::launch_append(p, static_cast<hipStream_t>(stream)));
}

KVLR_API int kvlr_hadamard_bases(const kvlr_desc* desc, const float* P_K, const float* P_V, float* out_K,
                                 float* out_V, void* stream) {
  int Rk = 0, Rv = 0;
  const int rc = check_desc(desc, nullptr, &Rk, &Rv, nullptr);
  if (rc) return rc;
  if (!P_K || !P_V || !out_K || !out_V) return KVLR_ERR_NULL;
  if (!aligned16({P_K, P_V, out_K, out_V})) return KVLR_ERR_ARG;
  // every head's block is row-major [d][r(h)] with r(h) a multiple of 16, so the
  // transform acts on consecutive runs of 16 floats of the packed arrays
  if (Rk % 16 || Rv % 16) return KVLR_ERR_RANK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = kvlr::launch_hadamard(P_K, out_K, (size_t)desc->head_dim * Rk / 16, s);
  if (e == hipSuccess) e = kvlr::launch_hadamard(P_V, out_V, (size_t)desc->head_dim * Rv / 16, s);
  return hip_status(e);
}

}  // extern "C"

namespace {

// Shared checks of the decode stages; fills the kernel parameter blocks.
// single_launch: decode_attn and its folded and fused forms, which may take the
// balanced plan; the two stages always take the fixed plan.
int prepare_decode(const kvlr_desc* desc, const float* q, const float* P_K, const void* lat_k, const void* lat_v,
                   const int32_t* seq_lens, float scale, const float* P_V, float* out, bool need_partials,
                   bool need_combine, void* workspace, size_t workspace_bytes, int32_t split_tokens,
                   kvlr::DecodeParams* p, kvlr::MergeParams* m, int* rank_bound, bool single_launch = false) {
  int rc = check_desc(desc, &p->ht, &p->Rk, &p->Rv, rank_bound, &p->Sk, &p->Sv);
  p->qt_in = nullptr;
  p->qt_stride = 0;
  if (rc) return rc;
  if (need_partials && (!q || !P_K || !lat_k || !lat_v || !seq_lens)) return KVLR_ERR_NULL;
  if (need_combine && (!P_V || !out)) return KVLR_ERR_NULL;
  if (need_partials && !isfinite(scale)) return KVLR_ERR_ARG;
  if (!aligned16({P_K, lat_k, lat_v, P_V, workspace})) return KVLR_ERR_ARG;
  int ns = 0, len = 0;
  rc = plan_split(desc, split_tokens, &ns, &len, p->ht.split_len);
  if (rc) return rc;
  const int stride = ws_stride_of(p->ht, desc->n_kv_heads);
  const size_t cbytes = counter_bytes_of(desc);
  const size_t rec_bytes = record_bytes_of(desc, p->ht, split_tokens, ns, *rank_bound);
  const size_t need = cbytes + rec_bytes + qt_bytes_of(desc);
  p->balanced = single_launch && balanced_plan(desc, split_tokens);
  p->apportion = p->balanced && one_segment_plan(desc, *rank_bound);
  p->n_wg = p->balanced ? balanced_grid(desc, *rank_bound) : 0;
  p->row_cost = p->balanced ? (int)row_cost_of(desc, p->apportion) : 0;
  for (int h = 0, c = 0; h < desc->n_kv_heads; ++h) {
    p->ht.cost[h] = token_cost(desc, h, p->apportion);
    p->ht.cost_pre[h] = c;
    c += p->ht.cost[h];
  }
  if (!workspace || workspace_bytes < need) return KVLR_ERR_WORKSPACE;

  const int G = desc->n_q_heads / desc->n_kv_heads;
  p->app_k = p->app_v = nullptr;
  p->k_new = p->v_new = nullptr;
  p->pos = nullptr;
  p->in_bf16 = desc->in_dtype == KVLR_BF16;
  p->q = q;
  p->pk = P_K;
  p->lat_k = lat_k;
  p->lat_v = lat_v;
  p->seq_lens = seq_lens;
  p->out_latent = 0;
  p->out_stride = desc->head_dim;
  p->counters = static_cast<int*>(workspace);
  p->ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + cbytes);
  p->qt_out = joint_bf16(desc) ? reinterpret_cast<float*>(static_cast<char*>(workspace) + cbytes + rec_bytes) : nullptr;
  p->pv = P_V;
  p->out = out;
  p->fuse = 0;
  p->B = desc->batch;
  p->Hq = desc->n_q_heads;
  p->Hkv = desc->n_kv_heads;
  p->G = G;
  p->d = desc->head_dim;
  p->cap = desc->capacity;
  p->split_len = len;
  p->n_splits = ns;
  p->ws_stride = stride;
  p->n_head_groups = (G + kvlr::kHeadsPerWg - 1) / kvlr::kHeadsPerWg;
  p->scale_log2 = scale * 1.4426950408889634f;

  m->ws = p->ws;
  m->pv = P_V;
  m->out = out;
  m->out_latent = 0;
  m->out_stride = desc->head_dim;
  m->B = p->B;
  m->Hq = p->Hq;
  m->Hkv = p->Hkv;
  m->G = G;
  m->d = p->d;
  m->n_splits = ns;
  m->ws_stride = stride;
  m->n_head_groups = p->n_head_groups;
  m->ht = p->ht;
  return KVLR_OK;
}

// 16-token blocks per wave step of the joint split kernel: one (measured faster
// than two at rank 64/128, which doubles the loads in flight and the registers).
constexpr int kJointBlocks = 1;

// Joint bf16 values: q~ = q P_K into the workspace, then the split kernel over it.
hipError_t joint_partials(const kvlr_desc* desc, kvlr::DecodeParams p, hipStream_t s) {
  const int rk_max = rk_max_of(desc);
  kvlr::DecodeParams pq = p;
  pq.qt_in = nullptr;
  pq.qt_stride = rk_max;
  pq.scale_log2 = 1.f;   // the split kernel applies the scale as it loads q~
  hipError_t e = kvlr::launch_project_queries(pq, rank_bound_of(rk_max), s);
  if (e != hipSuccess) return e;
  p.qt_in = p.qt_out;
  p.qt_stride = rk_max;
  return kvlr::launch_decode_joint(p, rank_bound_of(rk_max), kJointBlocks, s);
}

// kvlr_decode_attn's launches for a prepared call: projection, split and merge for
// joint bf16 values; otherwise one launch, whose last split workgroup of each group
// merges and back-projects.
hipError_t launch_decode_attn(const kvlr_desc* desc, kvlr::DecodeParams p, const kvlr::MergeParams& m,
                              int rank_bound, hipStream_t s) {
  if (joint_bf16(desc)) {
    hipError_t e = joint_partials(desc, p, s);
    if (e == hipSuccess) e = kvlr::launch_merge_heads(m, s);
    return e;
  }
  p.fuse = 1;
  return kvlr::launch_decode(p, desc->latent_dtype, rank_bound, decode_tile(), s);
}

// kvlr_decode_attn_layers: one prepared layer, and the library's lanes of a device
// (streams of default priority and the events that fork and join them), made on
// first use and kept until the process ends.
struct PreparedLayer {
  const kvlr_desc* desc;
  kvlr::DecodeParams p;
  kvlr::MergeParams m;
  int rank_bound;
};
struct LaneSet {
  bool ready = false;
  hipStream_t s[KVLR_MAX_LANES];
  hipEvent_t fork;
  hipEvent_t join[KVLR_MAX_LANES];
};
LaneSet g_lanes[kMaxDevices];
std::mutex g_lane_mu[kMaxDevices];   // held while a call enqueues on the device's lanes

hipError_t lane_set(int dev, LaneSet** out) {
  LaneSet& ls = g_lanes[dev];
  if (!ls.ready) {   // all or nothing: on a failure what was made is released, and a later call tries again
    LaneSet t;
    int n_streams = 0, n_joins = 0;
    hipError_t e = hipEventCreateWithFlags(&t.fork, hipEventDisableTiming);
    const bool forked = e == hipSuccess;
    while (e == hipSuccess && n_streams < KVLR_MAX_LANES) {
      e = hipStreamCreateWithFlags(&t.s[n_streams], hipStreamNonBlocking);
      if (e == hipSuccess) ++n_streams;
    }
    while (e == hipSuccess && n_joins < KVLR_MAX_LANES) {
      e = hipEventCreateWithFlags(&t.join[n_joins], hipEventDisableTiming);
      if (e == hipSuccess) ++n_joins;
    }
    if (e != hipSuccess) {
      for (int i = 0; i < n_joins; ++i) (void)hipEventDestroy(t.join[i]);
      for (int i = 0; i < n_streams; ++i) (void)hipStreamDestroy(t.s[i]);
      if (forked) (void)hipEventDestroy(t.fork);
      return e;
    }
    t.ready = true;
    ls = t;
  }
  *out = &ls;
  return hipSuccess;
}

// Whether two layers' workspaces [workspace, workspace + workspace_bytes) overlap.
bool workspaces_overlap(const kvlr_layer* layers, int n) {
  std::vector<std::pair<uintptr_t, uintptr_t>> r((size_t)n);
  for (int l = 0; l < n; ++l) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(layers[l].workspace);
    r[(size_t)l] = {a, a + layers[l].workspace_bytes};
  }
  std::sort(r.begin(), r.end());
  for (int l = 1; l < n; ++l)
    if (r[(size_t)l].first < r[(size_t)l - 1].second) return true;
  return false;
}

}  // namespace

extern "C" {

KVLR_API int kvlr_decode_partials(const kvlr_desc* desc, const float* q, const float* P_K, const void* lat_k,
                                  const void* lat_v, const int32_t* seq_lens, float scale, void* workspace,
                                  size_t workspace_bytes, int32_t split_tokens, void* stream) {
  kvlr::DecodeParams p;
  kvlr::MergeParams m;
  int rank_bound = 0;
  const int rc = prepare_decode(desc, q, P_K, lat_k, lat_v, seq_lens, scale, nullptr, nullptr, true, false,
                                workspace, workspace_bytes, split_tokens, &p, &m, &rank_bound);
  if (rc) return rc;
  if (joint_bf16(desc)) return hip_status(joint_partials(desc, p, static_cast<hipStream_t>(stream)));
  return hip_status(kvlr::launch_decode(p, desc->latent_dtype, rank_bound, decode_tile(),
                                        static_cast<hipStream_t>(stream)));
}

KVLR_API int kvlr_decode_combine(const kvlr_desc* desc, const float* P_V, const void* workspace,
                                 size_t workspace_bytes, int32_t split_tokens, float* out, void* stream) {
  kvlr::DecodeParams p;
  kvlr::MergeParams m;
  int rank_bound = 0;
  const int rc = prepare_decode(desc, nullptr, nullptr, nullptr, nullptr, nullptr, 1.f, P_V, out, false, true,
                                const_cast<void*>(workspace), workspace_bytes, split_tokens, &p, &m, &rank_bound);
  if (rc) return rc;
  if (joint_bf16(desc)) return hip_status(kvlr::launch_merge_heads(m, static_cast<hipStream_t>(stream)));
  return hip_status(kvlr::launch_merge(m, rank_bound, static_cast<hipStream_t>(stream)));
}

KVLR_API int kvlr_decode_attn(const kvlr_desc* desc, const float* q, const float* P_K, const float* P_V,
                              const void* lat_k, const void* lat_v, const int32_t* seq_lens, float scale,
                              float* out, void* workspace, size_t workspace_bytes, int32_t split_tokens,
                              void* stream) {
  kvlr::DecodeParams p;
  kvlr::MergeParams m;
  int rank_bound = 0;
  const int rc = prepare_decode(desc, q, P_K, lat_k, lat_v, seq_lens, scale, P_V, out, true, true, workspace,
                                workspace_bytes, split_tokens, &p, &m, &rank_bound, true);
  if (rc) return rc;
  return hip_status(launch_decode_attn(desc, p, m, rank_bound, static_cast<hipStream_t>(stream)));
}

KVLR_API int kvlr_decode_attn_layers(const kvlr_layer* layers, int32_t n_layers, int32_t lanes, void* stream) {
  if (n_layers < 0 || lanes < 1 || lanes > KVLR_MAX_LANES) return KVLR_ERR_ARG;
  if (n_layers == 0) return KVLR_OK;
  if (!layers) return KVLR_ERR_NULL;
  // every layer checked (and its parameter blocks formed) before anything is enqueued
  std::vector<PreparedLayer> prep((size_t)n_layers);
  for (int l = 0; l < n_layers; ++l) {
    const kvlr_layer& L = layers[l];
    PreparedLayer& P = prep[(size_t)l];
    P.desc = L.desc;
    const int rc = prepare_decode(L.desc, L.q, L.P_K, L.lat_k, L.lat_v, L.seq_lens, L.scale, L.P_V, L.out, true,
                                  true, L.workspace, L.workspace_bytes, L.split_tokens, &P.p, &P.m, &P.rank_bound,
                                  true);
    if (rc) return rc;
  }
  if (lanes > 1 && workspaces_overlap(layers, n_layers)) return KVLR_ERR_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (lanes == 1) {
    for (const PreparedLayer& P : prep) {
      const hipError_t e = launch_decode_attn(P.desc, P.p, P.m, P.rank_bound, s);
      if (e != hipSuccess) return hip_status(e);
    }
    return KVLR_OK;
  }
  LaneSet* ls = nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVLR_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_lane_mu[dev]);
  if (lane_set(dev, &ls) != hipSuccess) return KVLR_ERR_HIP;
  // fork, issue round robin, join (the joins are enqueued even after a failed launch,
  // so that `stream` and a capture in progress stay whole)
  hipError_t first = hipEventRecord(ls->fork, s);
  for (int i = 0; i < lanes && first == hipSuccess; ++i) first = hipStreamWaitEvent(ls->s[i], ls->fork, 0);
  if (first != hipSuccess) return hip_status(first);
  for (int l = 0; l < n_layers && first == hipSuccess; ++l) {
    const PreparedLayer& P = prep[(size_t)l];
    first = launch_decode_attn(P.desc, P.p, P.m, P.rank_bound, ls->s[l % lanes]);
  }
  for (int i = 0; i < lanes; ++i) {
    hipError_t e = hipEventRecord(ls->join[i], ls->s[i]);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, ls->join[i], 0);
    if (first == hipSuccess) first = e;
  }
  return hip_status(first);
}

KVLR_API int kvlr_decode_attn_latent(const kvlr_desc* desc, const float* q_lat, const void* lat_k,
                                     const void* lat_v, const int32_t* seq_lens, float scale, float* o_lat,
                                     void* workspace, size_t workspace_bytes, int32_t split_tokens,
                                     void* stream) {
  kvlr::DecodeParams p;
  kvlr::MergeParams m;
  int rank_bound = 0;
  // q_lat stands in for q and P_K (checked non-NULL through the same slots); no P_V is read
  const int rc = prepare_decode(desc, q_lat, q_lat, lat_k, lat_v, seq_lens, scale, q_lat, o_lat, true, true,
                                workspace, workspace_bytes, split_tokens, &p, &m, &rank_bound, true);
  if (rc) return rc;
  int rk_max = 0, rv_max = 0;
  for (int h = 0; h < desc->n_kv_heads; ++h) {
    rk_max = desc->r_k[h] > rk_max ? desc->r_k[h] : rk_max;
    rv_max = desc->r_v[h] > rv_max ? desc->r_v[h] : rv_max;
  }
  p.q = nullptr;
  p.pk = nullptr;
  p.pv = nullptr;
  p.qt_in = q_lat;
  p.qt_stride = rk_max;
  if (joint_bf16(desc)) {   // split and merge launches
    const hipStream_t s = static_cast<hipStream_t>(stream);
    m.pv = nullptr;
    m.out = o_lat;
    m.out_latent = 1;
    m.out_stride = rv_max;
    hipError_t e = kvlr::launch_decode_joint(p, rank_bound_of(rk_max), kJointBlocks, s);
    if (e == hipSuccess) e = kvlr::launch_merge_heads(m, s);
    return hip_status(e);
  }
  p.out_latent = 1;
  p.out_stride = rv_max;
  p.fuse = 1;
  return hip_status(kvlr::launch_decode(p, desc->latent_dtype, rank_bound, decode_tile(),
                                        static_cast<hipStream_t>(stream)));
}

KVLR_API int kvlr_append_decode_attn(const kvlr_desc* desc, const void* k_new, const void* v_new,
                                     const int32_t* pos, const float* q, const float* P_K, const float* P_V,
                                     void* lat_k, void* lat_v, const int32_t* seq_lens, float scale, float* out,
                                     void* workspace, size_t workspace_bytes, int32_t split_tokens, void* stream) {
  kvlr::DecodeParams p;
  kvlr::MergeParams m;
  int rank_bound = 0;
  int rc = prepare_decode(desc, q, P_K, lat_k, lat_v, seq_lens, scale, P_V, out, true, true, workspace,
                          workspace_bytes, split_tokens, &p, &m, &rank_bound);
  if (rc) return rc;
  if (!k_new || !v_new || !pos) return KVLR_ERR_NULL;
  if (desc->latent_dtype != KVLR_BF16 || desc->value_mode != KVLR_VALUES_PER_HEAD ||
      balanced_plan(desc, split_tokens)) {
    // other caches and the balanced plan: the append kernel, then the decode (two launches, the same result)
    rc = kvlr_append(desc, k_new, v_new, pos, P_K, P_V, lat_k, lat_v, stream);
    if (rc) return rc;
    return kvlr_decode_attn(desc, q, P_K, P_V, lat_k, lat_v, seq_lens, scale, out, workspace, workspace_bytes,
                            split_tokens, stream);
  }
  p.app_k = lat_k;
  p.app_v = lat_v;
  p.k_new = k_new;
  p.v_new = v_new;
  p.pos = pos;
  p.fuse = 1;
  return hip_status(kvlr::launch_decode(p, desc->latent_dtype, rank_bound, decode_tile(),
                                        static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// decode without a caller workspace: the library's static scratch
// ---------------------------------------------------------------------------
// For callers that cannot allocate device memory. The decode workspace (arrival
// counters, split records, projected queries) lives in a file-scope device
// array of KVLR_STATIC_SCRATCH_BYTES. Host code never passes the array's name
// to a kernel: its device address is looked up once per device with
// hipGetSymbolAddress (each device holds its own copy) and cached.
namespace {

static __device__ __align__(256) uint32_t scratch[KVLR_STATIC_SCRATCH_BYTES / 4];

__global__ void zero_words(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

// Set-up on the first call on a device (with that device current): the array's
// device address, and the array zeroed on the caller's stream (the arrival
// counters must start at zero; every completed decode leaves them zero again).
int static_scratch(hipStream_t s, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVLR_ERR_HIP;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!ptr) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return KVLR_ERR_HIP;
      hipLaunchKernelGGL(zero_words, dim3(256), dim3(256), 0, s, static_cast<uint32_t*>(ptr),
                         (size_t)KVLR_STATIC_SCRATCH_BYTES / 4);
      if (hipGetLastError() != hipSuccess) return KVLR_ERR_HIP;
      g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return KVLR_OK;
}

}  // namespace

extern "C" {

KVLR_API int kvlr_decode_attn_noalloc(const kvlr_desc* desc, const float* q, const float* P_K, const float* P_V,
                                      const void* lat_k, const void* lat_v, const int32_t* seq_lens, float scale,
                                      float* out, int32_t split_tokens, void* stream) {
  size_t need = 0;
  int rc = kvlr_decode_workspace_bytes(desc, split_tokens, &need);
  if (rc) return rc;
  if (need > (size_t)KVLR_STATIC_SCRATCH_BYTES) return KVLR_ERR_SCRATCH;
  {   // every other argument check, with a stand-in for the scratch (no memory is read)
    kvlr::DecodeParams p;
    kvlr::MergeParams m;
    int rank_bound = 0;
    rc = prepare_decode(desc, q, P_K, lat_k, lat_v, seq_lens, scale, P_V, out, true, true,
                        reinterpret_cast<void*>(uintptr_t{256}), need, split_tokens, &p, &m, &rank_bound, true);
    if (rc) return rc;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  rc = static_scratch(s, &ws);
  if (rc) return rc;
  return kvlr_decode_attn(desc, q, P_K, P_V, lat_k, lat_v, seq_lens, scale, out, ws, need, split_tokens, stream);
}

}  // extern "C"
