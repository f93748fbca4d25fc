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

// RAGGED: G does not divide the rows of every batch entry (or the entries differ in
// length); each pooled row then finds its head, its entry's length and the rows left.
template <typename T, int G, bool RAGGED>
__global__ __launch_bounds__(256) void kap_pool_kernel(PoolLaunch a) {
  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  long t = (long)blockIdx.x * 256 + threadIdx.x;
  const T* x;
  T* y;
  int H = a.H0;
  if (t < a.chunks0) {
    x = (const T*)a.x0;
    y = (T*)a.y0;
  } else {
    t -= a.chunks0;
    if (t >= a.chunks1) return;
    x = (const T*)a.x1;
    y = (T*)a.y1;
    H = a.H1;
  }
  const int cpr = a.cpr;
  const long prow = t / cpr;
  const int c = (int)(t - prow * cpr);
  const long rowlen = (long)cpr * EPC;
  long srow = prow * G;
  int avail = G;
  if constexpr (RAGGED) {
    const long head = prow / a.Np;
    const int pr = (int)(prow - head * a.Np);
    srow = head * a.N + (long)pr * G;
    avail = min(G, a.sl.of((int)(head / H), a.N) - pr * G);
    if (avail <= 0) return;   // past the end of this entry: never read
  }
  const T* src = x + srow * rowlen + (long)c * EPC;
  T* dst = y + prow * rowlen + (long)c * EPC;
  if (a.stride_mode || G == 1) {
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
  const bool ragged = a.N % a.g != 0 || a.sl.varlen;
#define COSA_POOL_CASE(GG)                                                                 \
  case GG:                                                                                 \
    if (ragged)                                                                            \
      hipLaunchKernelGGL((kap_pool_kernel<T, GG, true>), dim3(grid), dim3(256), 0, s, a);  \
    else                                                                                   \
      hipLaunchKernelGGL((kap_pool_kernel<T, GG, false>), dim3(grid), dim3(256), 0, s, a); \
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
