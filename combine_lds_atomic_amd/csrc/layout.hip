// Routing layout: per-expert counts, the count exchange and the exclusive
// prefix sums that give every (source, expert) slot a conflict-free,
// contiguous position ("Enabling trillion-parameter models on AWS EFA",
// sections "Send and receive buffers" and "Dispatch and combine").
//
// The pages count in one block with shared-memory atomics, copy the counts to
// the host and compute the receive-side offsets on the CPU.  Here every rank's
// counts are already in HBM, so the whole exchange is two or three short
// kernels:
//   k_route_count  grid (chunks, N): LDS-atomic occupancy masks per 64-slot
//                  batch give per-expert counts and stable in-chunk ranks;
//                  when a rank's slots fit one chunk it also does that rank's
//                  scan, and the positions it writes are final;
//   k_route_scan   grid (N), only with several chunks per rank: per-rank
//                  scans over chunks and experts;
//   k_route_cross  one block: the cross-rank scans (receive offsets, expert
//                  offsets, region bases) and the capacity / bound checks.
// Kernel boundaries order the three; no grid-wide fence is needed (on a
// multi-XCD GPU an agent-scope fence costs a write-back of the L2).
#include "route_dev.h"

namespace moe {

__global__ __launch_bounds__(kThreads) void k_route_count(Dims D, Ws W, const int* __restrict__ idx,
                                                          int* __restrict__ send_pos) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int wsum[kWavesPerBlock + 1];
  count_chunk(D, W, idx, send_pos, blockIdx.y, blockIdx.x, smem, wsum, 0u);
}

constexpr int kScanThreads = 1024;
constexpr int kScanWaves = kScanThreads / kWave;

// Sum of get(s) for s in [s0, s1), the loads issued eight at a time.
template <typename Get>
__device__ __forceinline__ int sum_range(int s0, int s1, Get get) {
  int acc = 0;
  int s = s0;
  for (; s + 8 <= s1; s += 8) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = get(s + u);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  for (; s < s1; ++s) acc += get(s);
  return acc;
}

// put(s, exclusive prefix) for s in [s0, s1), starting from acc; loads issued
// eight at a time.
template <typename Get, typename Put>
__device__ __forceinline__ void scan_range(int s0, int s1, int acc, Get get, Put put) {
  int s = s0;
  for (; s + 8 <= s1; s += 8) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = get(s + u);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      put(s + u, acc);
      acc += v[u];
    }
  }
  for (; s < s1; ++s) {
    const int v = get(s);
    put(s, acc);
    acc += v;
  }
}

// Per-rank scans over chunks and experts (block s), when a rank has several
// chunks: chunk counts become chunk base positions.
__global__ __launch_bounds__(kScanThreads) void k_route_scan(Dims D, Ws W) {
  __shared__ int wsum[kScanWaves + 1];
  const int s = blockIdx.x, tid = threadIdx.x;
  const int E = D.E;
  // One expert per thread (E <= 1024), its chunk counts loaded four at a time.
  int tot = 0;
  if (tid < E) {
    int* p = W.blk + (int64_t)s * D.B * E + tid;
    int b = 0;
    for (; b + 4 <= D.B; b += 4) {
      const int c0 = p[(int64_t)b * E], c1 = p[(int64_t)(b + 1) * E], c2 = p[(int64_t)(b + 2) * E],
                c3 = p[(int64_t)(b + 3) * E];
      p[(int64_t)b * E] = tot;
      p[(int64_t)(b + 1) * E] = tot + c0;
      p[(int64_t)(b + 2) * E] = tot + c0 + c1;
      p[(int64_t)(b + 3) * E] = tot + c0 + c1 + c2;
      tot += c0 + c1 + c2 + c3;
    }
    for (; b < D.B; ++b) {
      const int c = p[(int64_t)b * E];
      p[(int64_t)b * E] = tot;
      tot += c;
    }
    W.cnt[s * E + tid] = tot;
  }
  int total;
  const int off = block_scan<kScanThreads>(tid < E ? tot : 0, wsum, &total);
  int* so = W.send_off + s * (E + 1);
  if (tid < E) {
    so[tid] = off;
    int* p = W.blk + (int64_t)s * D.B * E + tid;
    for (int b = 0; b < D.B; ++b) p[(int64_t)b * E] += off;
  }
  if (tid == 0) so[E] = total;
}

// Largest N*E whose count table the cross-rank kernel stages in LDS (96 KB),
// and the largest N for which the N x N rank-to-rank counts stay in
// registers while that table is reused for them.
constexpr int kCrossTable = 24576;
constexpr int kCrossMaxN = 128;

// The scans across ranks that the receive side needs; one block.
__global__ __launch_bounds__(kScanThreads) void k_route_cross(Dims D, Ws W) {
  __shared__ int tab[kCrossTable];
  __shared__ int ex[kMaxE + 1];
  __shared__ int rt[kMaxN];   // rows each destination receives
  __shared__ int ro[kMaxN];   // of those, rows beyond the senders' early rows
  __shared__ int wsum[kScanWaves + 1];
  const int tid = threadIdx.x;
  const int N = D.N, E = D.E, L = D.L;

  if (N * E <= kCrossTable && N <= kCrossMaxN) {
    // Stage cnt[N][E] (coalesced, eight loads in flight per thread).
    const int n = N * E;
    for (int i0 = tid; i0 < n; i0 += kScanThreads * 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * kScanThreads;
        v[u] = i < n ? W.cnt[i] : 0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * kScanThreads;
        if (i < n) tab[i] = v[u];
      }
    }
    __syncthreads();
    // (1) src_in_exp[s][e] = rows of expert e from sources before s.
    for (int e = tid; e < E; e += kScanThreads) {
      int acc = 0;
      for (int s = 0; s < N; ++s) {
        W.src_in_exp[s * E + e] = acc;
        acc += tab[s * E + e];
      }
      W.src_in_exp[N * E + e] = acc;
      ex[e] = acc;
    }
    // (3a) c[s][d] = rows from source s to destination d, kept in registers
    // while the table is rewritten as c.
    constexpr int kCPer = kCrossMaxN * kCrossMaxN / kScanThreads;
    int cv[kCPer];
#pragma unroll
    for (int u = 0; u < kCPer; ++u) {
      const int i = tid + u * kScanThreads;   // i = s * N + d
      int c = 0;
      if (i < N * N) {
        const int s = i / N, d = i - s * N;
        for (int l = 0; l < L; ++l) c += tab[s * E + d * L + l];
      }
      cv[u] = c;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kCPer; ++u) {
      const int i = tid + u * kScanThreads;
      if (i < N * N) tab[i] = cv[u];
    }
    __syncthreads();
    // (3b) recv_off[d][s] = rows from sources before s, stacked by source
    // (with early rows: only each source's rows beyond its first Ce).
    for (int d = tid; d < N; d += kScanThreads) {
      int acc = 0, tot = 0;
      for (int s = 0; s < N; ++s) {
        const int c = tab[s * N + d];
        W.recv_off[d * (N + 1) + s] = acc;
        acc += max(c - D.Ce, 0);
        tot += c;
      }
      W.recv_off[d * (N + 1) + N] = acc;
      W.recv_total[d] = tot;
      rt[d] = tot;
      ro[d] = acc;
    }
    __syncthreads();
  } else {
    // General shapes: the same scans from global memory, the sources split
    // over G thread groups per column.
    int* part = tab;
    {
      const int G = min(N, max(1, kScanThreads / E));
      const int e = tid % E, g = tid / E;
      const bool mine = tid < G * E;
      const int per = (N + G - 1) / G;
      const int s0 = min(N, g * per), s1 = min(N, s0 + per);
      const int* cnt = W.cnt;
      auto get = [&](int s2) { return cnt[s2 * E + e]; };
      if (mine) part[g * E + e] = sum_range(s0, s1, get);
      __syncthreads();
      for (int e2 = tid; e2 < E; e2 += kScanThreads) {
        int a = 0;
        for (int g2 = 0; g2 < G; ++g2) {
          const int c = part[g2 * E + e2];
          part[g2 * E + e2] = a;
          a += c;
        }
        ex[e2] = a;
        W.src_in_exp[N * E + e2] = a;
      }
      __syncthreads();
      int* sie = W.src_in_exp;
      if (mine) scan_range(s0, s1, part[g * E + e], get, [&](int s2, int v) { sie[s2 * E + e] = v; });
      __syncthreads();
    }
    {
      const int G = min(N, max(1, kScanThreads / N));
      const int d = tid % N, g = tid / N;
      const bool mine = tid < G * N;
      const int per = (N + G - 1) / G;
      const int s0 = min(N, g * per), s1 = min(N, s0 + per);
      const int* so_all = W.send_off;
      auto getc = [&](int s2) {
        const int* o = so_all + s2 * (E + 1);
        return o[(d + 1) * L] - o[d * L];
      };
      auto get = [&](int s2) { return max(getc(s2) - D.Ce, 0); };   // rows beyond the early ones
      int* partc = part + kScanThreads;
      if (mine) {
        part[g * N + d] = sum_range(s0, s1, get);
        partc[g * N + d] = sum_range(s0, s1, getc);
      }
      __syncthreads();
      for (int d2 = tid; d2 < N; d2 += kScanThreads) {
        int a = 0, b = 0;
        for (int g2 = 0; g2 < G; ++g2) {
          const int c = part[g2 * N + d2];
          part[g2 * N + d2] = a;
          a += c;
          b += partc[g2 * N + d2];
        }
        W.recv_off[d2 * (N + 1) + N] = a;
        W.recv_total[d2] = b;
        rt[d2] = b;
        ro[d2] = a;
      }
      __syncthreads();
      int* rof = W.recv_off + d * (N + 1);
      if (mine) scan_range(s0, s1, part[g * N + d], get, [&](int s2, int v) { rof[s2] = v; });
      __syncthreads();
    }
  }
  // (2) exp_off[d][l] from one exclusive scan over all experts.
  {
    int etot;
    const int x = block_scan<kScanThreads>(tid < E ? ex[tid] : 0, wsum, &etot);
    __syncthreads();
    if (tid < E) ex[tid] = x;
    if (tid == 0) ex[E] = etot;
    __syncthreads();
    for (int i = tid; i < N * (L + 1); i += kScanThreads) {
      const int d = i / (L + 1), l = i - d * (L + 1);
      W.exp_off[i] = ex[d * L + l] - ex[d * L];
    }
  }
  // (4) Region bases and rows written per region; capacity and bound checks.
  {
    const int r = tid < N ? rt[tid] : 0;
    const int used = D.R ? min(r, D.R) : r;
    int all, vall;
    const int b = block_scan<kScanThreads>(r, wsum, &all);
    const int vb = block_scan<kScanThreads>(used, wsum, &vall);
    if (tid < N) {
      W.base[tid] = D.R ? tid * D.R : b;
      W.vprefix[tid] = vb;
      uint32_t fl = 0;
      if (D.R && (r > D.R || D.N * D.Ce + ro[tid] > D.R)) fl |= MOE_FLAG_OVERFLOW;
      if ((int64_t)r > D.bound) fl |= MOE_FLAG_BOUND;
      if (fl) atomicOr(W.err, fl);
    }
    if (tid == 0) {
      W.base[N] = D.R ? N * D.R : all;
      W.vprefix[N] = vall;
    }
  }
}

// ------------------------------------------------------------------ launch

int launch_route(const Dims& D, const Ws& W, const int* idx, int* send_pos, hipStream_t st) {
  if (D.B > 0) {
    const size_t lds = count_lds_bytes(D.E);
    const int rc = launch("k_route_count", k_route_count, dim3(D.B, D.N), dim3(kThreads), lds, st, D, W, idx, send_pos);
    if (rc != MOE_OK) return rc;
  }
  if (D.B != 1) {   // several chunks per rank (or none): per-rank scans
    const int rc = launch("k_route_scan", k_route_scan, dim3(D.N), dim3(kScanThreads), 0, st, D, W);
    if (rc != MOE_OK) return rc;
  }
  return launch("k_route_cross", k_route_cross, dim3(1), dim3(kScanThreads), 0, st, D, W);
}

}  // namespace moe
