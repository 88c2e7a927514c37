// libmoe_streams (include/moe_streams.h): plain streaming kernels used only
// as measurement aids beside libmoe_ep.  They move bytes with the row
// kernels' 16-byte non-temporal accesses, free of any row lookup or
// arithmetic, each in the fastest grid form found for its pattern on
// MI355X, so that the benchmark can give each phase the achievable rate of
// its own access pattern on its own buffers.
#include <mutex>

#include "moe_internal.h"
#include "moe_streams.h"

namespace moe {
namespace {

// Workgroup size of the one-shot streams: one wave, as the row kernels use;
// 3-5% faster than 256 threads for every pattern below.
constexpr int kStreamThreads = 64;

// Copy in the one-shot form (one unit per thread, workgroups in address
// order): 6.7 TB/s on a 7.5 GB copy, against 5.6 for the best grid-stride
// loop and 4.7 for one contiguous chunk per workgroup.
__global__ __launch_bounds__(kStreamThreads) void k_copy16(v4u* __restrict__ dst, const v4u* __restrict__ src,
                                                       int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kStreamThreads)
    st16(dst + i, ld16(src + i));
}

// The access patterns of the pack and of the receive-side sum:
//   fan-out: unit i reads 32 bytes (src units 2i, 2i+1: a lane's 16 bf16
//            elements) and stores their XOR at dst unit j*n + i for each
//            j < K (the k fp8 rows);
//   reduce:  unit i reads src units j*n + i, j < K (the k slot rows), and
//            stores their XOR at dst unit i.
// The reduction runs one-shot (6.2 TB/s at K = 8 against 5.4 for the best
// chunked form).  The fan-out comes in both forms: one contiguous chunk per
// 1024-thread workgroup, one workgroup per CU, 4 units per thread with all
// 8 loads issued together (5.1 TB/s at K = 8), and one-shot (5.4 TB/s at
// K = 8, 6.4 at K = 1).
template <int K>
__global__ __launch_bounds__(kStreamThreads) void k_stream_reduce(v4u* __restrict__ dst, const v4u* __restrict__ src,
                                                              int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kStreamThreads) {
    v4u v[K];
#pragma unroll
    for (int j = 0; j < K; ++j) v[j] = ld16(src + j * n + i);
    v4u q = v[0];
#pragma unroll
    for (int j = 1; j < K; ++j) q ^= v[j];
    st16(dst + i, q);
  }
}

template <int K>
__global__ __launch_bounds__(kStreamThreads) void k_stream_fanout_os(v4u* __restrict__ dst, const v4u* __restrict__ src,
                                                                 int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kStreamThreads) {
    const v4u q = ld16(src + 2 * i) ^ ld16(src + 2 * i + 1);
#pragma unroll
    for (int j = 0; j < K; ++j) st16(dst + j * n + i, q);
  }
}

constexpr int kFanThreads = 1024, kFanUnits = 4;

template <int K>
__global__ __launch_bounds__(kFanThreads) void k_stream_fanout(v4u* __restrict__ dst, const v4u* __restrict__ src,
                                                               int64_t n) {
  constexpr int U = kFanUnits;
  const int64_t b0 = n * blockIdx.x / gridDim.x, b1 = n * (blockIdx.x + 1) / gridDim.x;
  for (int64_t i0 = b0 + threadIdx.x; i0 < b1; i0 += (int64_t)U * kFanThreads) {
    v4u a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {   // units past the chunk repeat its last one and store nothing
      const int64_t i = min(i0 + (int64_t)u * kFanThreads, b1 - 1);
      a[u] = ld16(src + 2 * i);
      b[u] = ld16(src + 2 * i + 1);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + (int64_t)u * kFanThreads;
      if (i < b1) {
        const v4u q = a[u] ^ b[u];
#pragma unroll
        for (int j = 0; j < K; ++j) st16(dst + j * n + i, q);
      }
    }
  }
}

template <int K>
int launch_stream_k(int pattern, v4u* dst, const v4u* src, int64_t n16, int cus, hipStream_t st) {
  if (pattern == MOE_STREAM_REDUCE)
    return launch("k_stream_reduce", k_stream_reduce<K>, dim3(os_grid(n16, kStreamThreads)), dim3(kStreamThreads), 0, st, dst, src, n16);
  if (pattern == MOE_STREAM_FANOUT_ONESHOT)
    return launch("k_stream_fanout_os", k_stream_fanout_os<K>, dim3(os_grid(n16, kStreamThreads)), dim3(kStreamThreads), 0, st, dst,
                  src, n16);
  const int64_t need = (n16 + (int64_t)kFanThreads * kFanUnits - 1) / ((int64_t)kFanThreads * kFanUnits);
  const int grid = (int)(need < cus ? need : cus);
  return launch("k_stream_fanout", k_stream_fanout<K>, dim3(grid), dim3(kFanThreads), 0, st, dst, src, n16);
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
  return launch("k_copy16", k_copy16, dim3(os_grid(n16, kStreamThreads)), dim3(kStreamThreads), 0, static_cast<hipStream_t>(stream),
                reinterpret_cast<v4u*>(dst), reinterpret_cast<const v4u*>(src), n16);
}

int moe_stream(int pattern, int k, void* dst, const void* src, int64_t n16, void* stream) {
  if (pattern != MOE_STREAM_FANOUT && pattern != MOE_STREAM_REDUCE && pattern != MOE_STREAM_FANOUT_ONESHOT)
    return MOE_EINVAL;
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
