// Seeded synthetic key/value rows on the GPU: the device twin of the numpy
// generator in synth/host.py. It holds no attention arithmetic; it only
// draws inputs, bit for bit the same as the host side:
//   word(key, n)  = SplitMix64 mix of (key + n * 0x9E3779B97F4A7C15)
//                   (Steele, Lea, Flood, OOPSLA 2014)
//   z(e)          = (sum of the twelve 16-bit fields of words 3e+1..3e+3 - 6*65536) / 65536
//   x             = mu + sigma * z   (float64, two roundings, no fused multiply-add)
//   x            *= mult             (1 or 8, exact)
//   stored        = float32 (nearest even) or bf16 (nearest even, directly from float64)
// Element counter of row (b, t, h, j): (((b << 20) | t) * Hkv + h) * d + j.
//
// Built with -ffp-contract=off so that mu + sigma * z is never fused.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ double irwin_hall(uint64_t key, uint64_t e) {
  int64_t total = 0;
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    uint64_t w = mix64(key + (e * 3ull + (uint64_t)(k + 1)) * kGamma);
    total += (int64_t)(w & 0xFFFFull) + (int64_t)((w >> 16) & 0xFFFFull) +
             (int64_t)((w >> 32) & 0xFFFFull) + (int64_t)((w >> 48) & 0xFFFFull);
  }
  return (double)(total - 6 * 65536) * (1.0 / 65536.0);
}

__device__ __forceinline__ uint16_t bf16_from_f64(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  uint64_t lsb = (u >> 45) & 1ull;
  uint64_t r = (u + ((1ull << 44) - 1ull) + lsb) & ~((1ull << 45) - 1ull);
  float f = (float)__longlong_as_double((long long)r);  // exact: 8 significant bits
  return (uint16_t)(__float_as_uint(f) >> 16);
}

__global__ void fill_kv_kernel(void* __restrict__ out, int out_bf16, int B, int n_tok, int t0,
                               int Hkv, int d, uint64_t key, const double* __restrict__ mu,
                               const double* __restrict__ sigma, const double* __restrict__ mult) {
  const uint64_t total = (uint64_t)B * n_tok * Hkv * d;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (uint64_t)gridDim.x * blockDim.x) {
    const int j = (int)(i % d);
    uint64_t r = i / d;
    const int h = (int)(r % Hkv);
    r /= Hkv;
    const int tt = (int)(r % n_tok);
    const int b = (int)(r / n_tok);
    const uint64_t t = (uint64_t)(t0 + tt);
    const uint64_t e = ((((uint64_t)b << 20) | t) * (uint64_t)Hkv + (uint64_t)h) * (uint64_t)d + (uint64_t)j;
    const double z = irwin_hall(key, e);
    const int c = h * d + j;
    const double prod = sigma[c] * z;
    const double x = (mu[c] + prod) * mult[c];
    if (out_bf16)
      static_cast<uint16_t*>(out)[i] = bf16_from_f64(x);
    else
      static_cast<float*>(out)[i] = (float)x;
  }
}

__global__ void touch_kernel(uint4* __restrict__ buf, uint64_t n, uint32_t salt) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (uint64_t)gridDim.x * blockDim.x)
    buf[i] = make_uint4((uint32_t)i, salt, (uint32_t)(i >> 32), ~salt);
}

__global__ void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, uint64_t n) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

// Streaming read with non-temporal 16-byte loads. Workgroup w reads the w-th
// of gridDim.x contiguous chunks; in each pass a wave reads 8 consecutive KiB
// (8 loads in flight per lane). The words read are folded with XOR and stored
// only on a value that practically never occurs, so the loads stay and nothing
// else moves.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ src, uint64_t n,
                                                          uint32_t* __restrict__ sink) {
  constexpr int kDepth = 8;
  const uint64_t chunk = (n + gridDim.x - 1) / gridDim.x;
  const uint64_t begin = blockIdx.x * chunk;
  const uint64_t end = begin + chunk < n ? begin + chunk : n;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  uint64_t i = begin + (uint64_t)wave * kDepth * 64 + lane;
  for (; i + (kDepth - 1) * 64 < end; i += 4 * kDepth * 64) {
    u32x4_t x[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) x[d] = __builtin_nontemporal_load(src + i + d * 64);
#pragma unroll
    for (int d = 0; d < kDepth; ++d) acc ^= x[d];
  }
  for (int d = 0; d < kDepth; ++d)
    if (i + d * 64 < end) acc ^= __builtin_nontemporal_load(src + i + d * 64);
  const uint32_t y = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (y == 0x9E3779B9u) sink[blockIdx.x] = y;
}

}  // namespace

extern "C" {

// Plain copy of `bytes` (multiple of 16): reads and writes exactly that many
// bytes, a reference for scaling hardware traffic counters.
int synth_copy(const void* src, void* dst, uint64_t bytes, void* stream) {
  if (!src || !dst || bytes % 16) return -1;
  const uint64_t n = bytes / 16;
  uint64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), n);
  return (int)hipGetLastError();
}

// Reads `bytes` (multiple of 16) once, `workgroups` (1 .. 2048) contiguous
// chunks streamed with non-temporal loads: the achievable read bandwidth, a
// ceiling for read-bound kernels. `sink` holds at least `workgroups` words and
// is written only on an improbable value of the data.
int synth_stream_read(const void* src, uint64_t bytes, uint32_t* sink, int workgroups, void* stream) {
  if (!src || !sink || bytes % 16 || workgroups < 1 || workgroups > 2048) return -1;
  const uint64_t n = bytes / 16;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const u32x4_t*>(src), n, sink);
  return (int)hipGetLastError();
}

// Writes out[B][n_tok][Hkv][d] (float32 if out_bf16 == 0, bf16 bits otherwise)
// for tokens t0 .. t0+n_tok-1. mu, sigma, mult: device float64 [Hkv][d].
// Returns 0 or the hipError_t of the launch.
int synth_fill_kv(void* out, int out_bf16, int B, int n_tok, int t0, int Hkv, int d,
                  uint64_t key, const double* mu, const double* sigma, const double* mult,
                  void* stream) {
  if (!out || !mu || !sigma || !mult || B <= 0 || n_tok <= 0 || Hkv <= 0 || d <= 0 || t0 < 0 ||
      (int64_t)t0 + n_tok > (1 << 20) || B >= (1 << 11))
    return -1;
  const uint64_t total = (uint64_t)B * n_tok * Hkv * d;
  uint64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_kv_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, out,
                     out_bf16, B, n_tok, t0, Hkv, d, key, mu, sigma, mult);
  return (int)hipGetLastError();
}

// Overwrites `bytes` (multiple of 16) of a scratch buffer, evicting earlier
// data from the GPU caches between timed calls.
int synth_touch(void* buf, uint64_t bytes, uint32_t salt, void* stream) {
  if (!buf || bytes % 16) return -1;
  const uint64_t n = bytes / 16;
  uint64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(touch_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     static_cast<uint4*>(buf), n, salt);
  return (int)hipGetLastError();
}

}  // extern "C"
