// KAP step 1: downsample queries and keys.
//
// CoSA technical summary (gist.science, pt), section 2.2 "Kernel-Aware Proxy",
// block ranking: the proxy works on downsampled queries and keys.  The operator
// is not printed; this library defines MEAN pooling bitwise (fp32 sum of the g
// rows in ascending order, times 2^-log2(g), rounded to the storage dtype) so
// that every implementation produces the same pooled vectors, and STRIDE (the
// first row of each group).
//
// When g does not divide the sequence length, the last pooled row of each head sums
// the rows that exist and keeps the 2^-log2(g) scale.
//
// HBM-streaming pass: one thread owns one 16-byte chunk of one pooled row and
// reads the g input chunks above it; consecutive lanes cover consecutive chunks
// of a row, so every wave load is a few fully used 256-byte row segments.
#include "cosa_common.hpp"
#include "cosa_launch.hpp"

namespace cosa {

template <typename T, int G, bool RAGGED>
__global__ __launch_bounds__(256) void kap_pool_kernel(const T* __restrict__ x0, T* __restrict__ y0,
                                                       long chunks0, const T* __restrict__ x1,
                                                       T* __restrict__ y1, long chunks1, int cpr,
                                                       int N, int Np, int stride_mode) {
  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  long t = (long)blockIdx.x * 256 + threadIdx.x;
  const T* x;
  T* y;
  if (t < chunks0) {
    x = x0;
    y = y0;
  } else {
    t -= chunks0;
    if (t >= chunks1) return;
    x = x1;
    y = y1;
  }
  const long prow = t / cpr;
  const int c = (int)(t - prow * cpr);
  const long rowlen = (long)cpr * EPC;
  // source rows: prow * G onwards; a ragged sequence needs the head and the rows left
  long srow = prow * G;
  int avail = G;
  if constexpr (RAGGED) {
    const long head = prow / Np;
    const int pr = (int)(prow - head * Np);
    srow = head * N + (long)pr * G;
    avail = min(G, N - pr * G);
  }
  const T* src = x + srow * rowlen + (long)c * EPC;
  T* dst = y + prow * rowlen + (long)c * EPC;
  if (stride_mode || G == 1) {
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
    return;
  }
  // Issue the loads in batches of up to 8 rows, then add in ascending row order.
  constexpr int UB = G < 8 ? G : 8;
  float acc[EPC];
#pragma unroll
  for (int t0 = 0; t0 < G; t0 += UB) {
    u32x4 buf[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u)
      if (!RAGGED || t0 + u < avail) buf[u] = *reinterpret_cast<const u32x4*>(src + (long)(t0 + u) * rowlen);
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      if (RAGGED && t0 + u >= avail) break;   // rows past the end of the sequence
      float v[EPC];
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          v[2 * w] = __uint_as_float(buf[u][w] << 16);
          v[2 * w + 1] = __uint_as_float(buf[u][w] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) v[w] = __uint_as_float(buf[u][w]);
      }
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[e] = (t0 + u == 0) ? v[e] : acc[e] + v[e];
    }
  }
  constexpr float inv = 1.0f / (float)G;  // exact: G is a power of two
  u32x4 o;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int w = 0; w < 4; ++w) o[w] = pack_bf16x2(acc[2 * w] * inv, acc[2 * w + 1] * inv);
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) o[w] = __float_as_uint(acc[w] * inv);
  }
  *reinterpret_cast<u32x4*>(dst) = o;
}

template <typename T>
static hipError_t launch_pool_t(const PoolLaunch& a, hipStream_t s) {
  const long total = a.chunks0 + a.chunks1;
  const unsigned grid = (unsigned)((total + 255) / 256);
  const T* x0 = (const T*)a.x0;
  const T* x1 = (const T*)a.x1;
  T* y0 = (T*)a.y0;
  T* y1 = (T*)a.y1;
  const bool ragged = a.N % a.g != 0;
#define COSA_POOL_CASE(GG)                                                                       \
  case GG:                                                                                       \
    if (ragged)                                                                                  \
      hipLaunchKernelGGL((kap_pool_kernel<T, GG, true>), dim3(grid), dim3(256), 0, s, x0, y0,      \
                         a.chunks0, x1, y1, a.chunks1, a.cpr, a.N, a.Np, a.stride_mode);          \
    else                                                                                         \
      hipLaunchKernelGGL((kap_pool_kernel<T, GG, false>), dim3(grid), dim3(256), 0, s, x0, y0,     \
                         a.chunks0, x1, y1, a.chunks1, a.cpr, a.N, a.Np, a.stride_mode);          \
    break;
  switch (a.g) {
    COSA_POOL_CASE(1)
    COSA_POOL_CASE(2)
    COSA_POOL_CASE(4)
    COSA_POOL_CASE(8)
    COSA_POOL_CASE(16)
    COSA_POOL_CASE(32)
    COSA_POOL_CASE(64)
    COSA_POOL_CASE(128)
    default:
      return hipErrorInvalidValue;
  }
#undef COSA_POOL_CASE
  return hipGetLastError();
}

hipError_t launch_pool(const PoolLaunch& a, hipStream_t s) {
  return a.bf16 ? launch_pool_t<bf16_t>(a, s) : launch_pool_t<float>(a, s);
}

}  // namespace cosa
