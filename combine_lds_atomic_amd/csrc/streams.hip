// libmoe_streams (include/moe_streams.h): plain streaming kernels used only
// as measurement aids beside libmoe_ep.  They move bytes with the row
// kernels' 16-byte non-temporal accesses and workgroup-contiguous chunks, free
// of any row lookup or arithmetic, so that the benchmark can give each phase
// the achievable rate of its own access pattern on its own buffers.
#include <mutex>

#include "moe_internal.h"
#include "moe_streams.h"

namespace moe {
namespace {

constexpr int kCpThreads = kCopyShape.threads();

// Plain streaming copy: each workgroup copies one contiguous chunk, every
// lane with kCopyUnroll loads in flight.  On a 1 GiB copy with one
// 1024-thread workgroup per CU, 16 loads per lane measured 6.1 TB/s against
// 6.0 (8), 5.8 (4) and 5.75 (32): the fastest pattern found.
constexpr int kCopyUnroll = 16;
__global__ __launch_bounds__(kCpThreads) void k_copy16(v4u* __restrict__ dst, const v4u* __restrict__ src,
                                                        int64_t n) {
  const int64_t b0 = n * blockIdx.x / gridDim.x, b1 = n * (blockIdx.x + 1) / gridDim.x;
  constexpr int U = kCopyUnroll;
  int64_t i = b0 + threadIdx.x;
  for (; i + (U - 1) * kCpThreads < b1; i += U * kCpThreads) {
    v4u r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) r[u] = ld16(src + i + u * kCpThreads);
#pragma unroll
    for (int u = 0; u < U; ++u) st16(dst + i + u * kCpThreads, r[u]);
  }
  for (; i < b1; i += kCpThreads) st16(dst + i, ld16(src + i));
}

// The access patterns of the pack and of the receive-side sum: each
// workgroup a contiguous chunk of units, every thread with all the loads of
// several units issued together (the fan-out's units past the chunk repeat
// its last one and store nothing; the reduction's skip their loads, which
// measured 3.5% faster for it).
//   fan-out: unit i reads 32 bytes (src units 2i, 2i+1: a lane's 16 bf16
//            elements) and stores their XOR at dst unit j*n + i for each
//            j < K (the k fp8 rows);
//   reduce:  unit i reads src units j*n + i, j < K (the k slot rows), and
//            stores their XOR at dst unit i.
// Units per thread: 4 for the fan-out (8 loads); for the reduction 32/K
// (32 loads), at most 8: the fastest counts found for plain kernels of
// these shapes.  (At K = 8 the compiler keeps two of the 16-byte values in
// scratch; that form measured as fast as a spill-free one.)
template <int K>
__global__ __launch_bounds__(kCpThreads) void k_stream_fanout(v4u* __restrict__ dst, const v4u* __restrict__ src,
                                                              int64_t n) {
  constexpr int U = 4;
  const int64_t b0 = n * blockIdx.x / gridDim.x, b1 = n * (blockIdx.x + 1) / gridDim.x;
  for (int64_t i0 = b0 + threadIdx.x; i0 < b1; i0 += (int64_t)U * kCpThreads) {
    v4u a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = min(i0 + (int64_t)u * kCpThreads, b1 - 1);
      a[u] = ld16(src + 2 * i);
      b[u] = ld16(src + 2 * i + 1);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + (int64_t)u * kCpThreads;
      if (i < b1) {
        const v4u q = a[u] ^ b[u];
#pragma unroll
        for (int j = 0; j < K; ++j) st16(dst + j * n + i, q);
      }
    }
  }
}

constexpr int stream_reduce_units(int K) { return K <= 3 ? 8 : (K == 4 ? 6 : 32 / K); }   // units per thread

template <int K>
__global__ __launch_bounds__(kCpThreads) void k_stream_reduce(v4u* __restrict__ dst, const v4u* __restrict__ src,
                                                              int64_t n) {
  constexpr int U = stream_reduce_units(K);
  const int64_t b0 = n * blockIdx.x / gridDim.x, b1 = n * (blockIdx.x + 1) / gridDim.x;
  for (int64_t i0 = b0 + threadIdx.x; i0 < b1; i0 += (int64_t)U * kCpThreads) {
    v4u v[U][K];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + (int64_t)u * kCpThreads;
#pragma unroll
      for (int j = 0; j < K; ++j) v[u][j] = i < b1 ? ld16(src + j * n + i) : v4u{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v4u q = v[u][0];
#pragma unroll
      for (int j = 1; j < K; ++j) q ^= v[u][j];
      const int64_t i = i0 + (int64_t)u * kCpThreads;
      if (i < b1) st16(dst + i, q);
    }
  }
}

template <int K>
int launch_stream_k(int pattern, v4u* dst, const v4u* src, int64_t n16, int cus, hipStream_t st) {
  const int64_t per_block = (int64_t)kCpThreads * (pattern == MOE_STREAM_FANOUT ? 4 : stream_reduce_units(K));
  const int grid = stream_grid(kCopyShape, cus, n16, per_block);
  if (pattern == MOE_STREAM_FANOUT)
    return launch("k_stream_fanout", k_stream_fanout<K>, dim3(grid), dim3(kCpThreads), 0, st, dst, src, n16);
  return launch("k_stream_reduce", k_stream_reduce<K>, dim3(grid), dim3(kCpThreads), 0, st, dst, src, n16);
}

int cus_of_device() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> g(mu);
  if (!cache[dev]) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

int moe_copy(void* dst, const void* src, int64_t nbytes, void* stream) {
  if (!dst || !src) return MOE_ENULL;
  if (nbytes < 0 || nbytes % 16) return MOE_EINVAL;
  if (!aligned16(dst) || !aligned16(src)) return MOE_EALIGN;
  const int64_t n16 = nbytes / 16;
  if (n16 == 0) return MOE_OK;
  const int grid = stream_grid(kCopyShape, cus_of_device(), n16, (int64_t)kCpThreads * kCopyUnroll);
  return launch("k_copy16", k_copy16, dim3(grid), dim3(kCpThreads), 0, static_cast<hipStream_t>(stream),
                reinterpret_cast<v4u*>(dst), reinterpret_cast<const v4u*>(src), n16);
}

int moe_stream(int pattern, int k, void* dst, const void* src, int64_t n16, void* stream) {
  if (pattern != MOE_STREAM_FANOUT && pattern != MOE_STREAM_REDUCE) return MOE_EINVAL;
  if (k < 1 || k > 8 || n16 < 0) return MOE_EINVAL;
  if (n16 > ((int64_t)1 << 40)) return MOE_ERANGE;   // keeps n16 * blockIdx within int64 in the kernels
  if (!dst || !src) return MOE_ENULL;
  if (!aligned16(dst) || !aligned16(src)) return MOE_EALIGN;
  if (n16 == 0) return MOE_OK;
  v4u* d = reinterpret_cast<v4u*>(dst);
  const v4u* s = reinterpret_cast<const v4u*>(src);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int cus = cus_of_device();
  switch (k) {
    case 1: return launch_stream_k<1>(pattern, d, s, n16, cus, st);
    case 2: return launch_stream_k<2>(pattern, d, s, n16, cus, st);
    case 3: return launch_stream_k<3>(pattern, d, s, n16, cus, st);
    case 4: return launch_stream_k<4>(pattern, d, s, n16, cus, st);
    case 5: return launch_stream_k<5>(pattern, d, s, n16, cus, st);
    case 6: return launch_stream_k<6>(pattern, d, s, n16, cus, st);
    case 7: return launch_stream_k<7>(pattern, d, s, n16, cus, st);
    default: return launch_stream_k<8>(pattern, d, s, n16, cus, st);
  }
}

}  // extern "C"
