// Routing layout: per-expert counts, the count exchange and the exclusive
// prefix sums that give every (source, expert) slot a conflict-free,
// contiguous position ("Enabling trillion-parameter models on AWS EFA",
// sections "Send and receive buffers" and "Dispatch and combine").
//
// The pages count in one block with shared-memory atomics, copy the counts to
// the host and compute the receive-side offsets on the CPU.  Here every rank's
// counts are already in HBM, so the whole exchange is two kernels:
//   k_route_count  grid (chunks, N): LDS-atomic occupancy masks per 64-slot
//                  batch give per-expert counts and stable in-chunk ranks;
//   k_route_scan   grid (N): per-rank scans over chunks and experts; the last
//                  block to arrive (ticket) runs the cross-rank scans.
#include "moe_internal.h"

namespace moe {

// Counts and in-chunk ranks of one chunk of kChunk slots of rank s.
//
// Each wave walks its quarter of the chunk 64 slots at a time.  Lane i ORs
// bit i into an LDS mask of its expert (ds_or_b64: one LDS atomic per slot);
// afterwards every lane reads its expert's mask and knows the lanes of this
// batch that share its expert.  rank = running count of the expert in this
// wave + lanes below it in the mask; the highest lane of each group advances
// the running count and clears the mask.  Ranks therefore follow slot order,
// which makes the final positions unique and reproducible.
__global__ __launch_bounds__(kThreads) void k_route_count(Dims D, Ws W, const int* __restrict__ idx,
                                                          int* __restrict__ send_pos) {
  extern __shared__ unsigned char smem[];
  unsigned long long* mask = reinterpret_cast<unsigned long long*>(smem);   // [4][E]
  int* run = reinterpret_cast<int*>(mask + kWavesPerBlock * D.E);            // [4][E]
  const int s = blockIdx.y, b = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  if (s == 0 && b == 0 && threadIdx.x == 0) *W.ticket = 0;   // the scan kernel runs after this one
  for (int i = threadIdx.x; i < kWavesPerBlock * D.E; i += kThreads) {
    mask[i] = 0ull;
    run[i] = 0;
  }
  __syncthreads();

  const int64_t rbase = (int64_t)s * D.TK;
  const int c0 = b * kChunk + w * kPerWave;
  const int cend = min(c0 + kPerWave, D.TK);
  unsigned long long* wm = mask + w * D.E;
  int* wr = run + w * D.E;
  int ev[kBatches], rv[kBatches];
  bool bad = false;
#pragma unroll
  for (int bt = 0; bt < kBatches; ++bt) {
    const int i = c0 + bt * kWave + lane;
    int e = -1;
    if (i < cend) {
      e = idx[rbase + i];
      if (e < 0 || e >= D.E) {
        bad = true;
        e = -1;
      }
    }
    if (e >= 0) atomicOr(&wm[e], 1ull << lane);
    __builtin_amdgcn_wave_barrier();
    unsigned long long m = 0ull;
    int r = -1;
    if (e >= 0) {
      m = wm[e];
      r = wr[e] + __popcll(m & ((1ull << lane) - 1ull));
    }
    __builtin_amdgcn_wave_barrier();
    if (e >= 0 && (m >> lane) == 1ull) {   // highest lane of its expert group
      wr[e] += __popcll(m);
      wm[e] = 0ull;
    }
    __builtin_amdgcn_wave_barrier();
    ev[bt] = e;
    rv[bt] = r;
  }
  if (__any(bad) && lane == 0) atomicOr(W.err, MOE_FLAG_BADID);
  __syncthreads();

  // Exclusive prefix over the four waves, per expert, and the chunk totals.
  int* blk = W.blk + ((int64_t)s * D.B + b) * D.E;
  for (int e = threadIdx.x; e < D.E; e += kThreads) {
    int p = 0;
#pragma unroll
    for (int ww = 0; ww < kWavesPerBlock; ++ww) {
      const int c = run[ww * D.E + e];
      run[ww * D.E + e] = p;
      p += c;
    }
    blk[e] = p;
  }
  __syncthreads();
#pragma unroll
  for (int bt = 0; bt < kBatches; ++bt) {
    const int i = c0 + bt * kWave + lane;
    if (i < cend) send_pos[rbase + i] = ev[bt] >= 0 ? wr[ev[bt]] + rv[bt] : -1;
  }
}

// Exclusive scan of v[0..n) in LDS by one 256-thread block; returns the total.
__device__ int block_excl_scan(int* v, int n, int* part) {
  const int tid = threadIdx.x;
  const int per = (n + kThreads - 1) / kThreads;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += v[i];
  part[tid] = sum;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int i = 0; i < kThreads; ++i) {
      const int c = part[i];
      part[i] = acc;
      acc += c;
    }
    part[kThreads] = acc;
  }
  __syncthreads();
  int acc = part[tid];
  for (int i = lo; i < hi; ++i) {
    const int c = v[i];
    v[i] = acc;
    acc += c;
  }
  const int total = part[kThreads];
  __syncthreads();
  return total;
}

// Per-rank scans (block s), then -- in the last block to finish -- the scans
// across ranks that the receive side needs.
__global__ __launch_bounds__(kThreads) void k_route_scan(Dims D, Ws W) {
  __shared__ int sv[kMaxE + 1];
  __shared__ int part[kThreads + 1];
  __shared__ int srt[kMaxN];
  __shared__ int last;
  const int s = blockIdx.x, tid = threadIdx.x;

  // Totals per expert; chunk counts become exclusive prefixes over chunks.
  for (int e = tid; e < D.E; e += kThreads) {
    int acc = 0;
    for (int b = 0; b < D.B; ++b) {
      int* p = W.blk + ((int64_t)s * D.B + b) * D.E + e;
      const int c = *p;
      *p = acc;
      acc += c;
    }
    sv[e] = acc;
    W.cnt[s * D.E + e] = acc;
  }
  __syncthreads();
  const int total = block_excl_scan(sv, D.E, part);
  int* so = W.send_off + s * (D.E + 1);
  for (int e = tid; e < D.E; e += kThreads) {
    so[e] = sv[e];
    for (int b = 0; b < D.B; ++b) W.blk[((int64_t)s * D.B + b) * D.E + e] += sv[e];
  }
  if (tid == 0) so[D.E] = total;

  // Release this block's tables device-wide, then take a ticket.
  __threadfence();
  __syncthreads();
  if (tid == 0) last = atomicAdd(W.ticket, 1u) == (unsigned)(D.N - 1);
  __syncthreads();
  if (!last) return;
  __threadfence();

  const int N = D.N, E = D.E, L = D.L;
  // Rows from each source into each destination, stacked by source.
  for (int d = tid; d < N; d += kThreads) {
    int acc = 0;
    for (int s2 = 0; s2 < N; ++s2) {
      W.recv_off[d * (N + 1) + s2] = acc;
      const int* o = W.send_off + s2 * (E + 1);
      acc += o[(d + 1) * L] - o[d * L];
    }
    W.recv_off[d * (N + 1) + N] = acc;
    W.recv_total[d] = acc;
    srt[d] = acc;
  }
  // Rows of expert e contributed by earlier sources, and expert totals.
  for (int e = tid; e < E; e += kThreads) {
    int acc = 0;
    for (int s2 = 0; s2 < N; ++s2) {
      W.src_in_exp[s2 * E + e] = acc;
      acc += W.cnt[s2 * E + e];
    }
    W.src_in_exp[N * E + e] = acc;
    sv[e] = acc;
  }
  __syncthreads();
  for (int d = tid; d < N; d += kThreads) {
    int acc = 0;
    for (int l = 0; l < L; ++l) {
      W.exp_off[d * (L + 1) + l] = acc;
      acc += sv[d * L + l];
    }
    W.exp_off[d * (L + 1) + L] = acc;
  }
  if (tid == 0) {
    int64_t acc = 0, vacc = 0;
    uint32_t fl = 0;
    for (int d = 0; d < N; ++d) {
      const int tot = srt[d];
      W.base[d] = D.R ? d * D.R : (int)acc;
      W.vprefix[d] = (int)vacc;
      vacc += D.R ? min(tot, D.R) : tot;
      acc += tot;
      if (D.R && tot > D.R) fl |= MOE_FLAG_OVERFLOW;
      if ((int64_t)tot > D.bound) fl |= MOE_FLAG_BOUND;
    }
    W.base[N] = D.R ? N * D.R : (int)acc;
    W.vprefix[N] = (int)vacc;
    if (fl) atomicOr(W.err, fl);
  }
}

// ------------------------------------------------------------------ launch

int launch_route(const Dims& D, const Ws& W, const int* idx, int* send_pos, hipStream_t st) {
  if (D.B > 0) {
    const size_t lds = (size_t)kWavesPerBlock * D.E * (sizeof(unsigned long long) + sizeof(int));
    const int rc = launch("k_route_count", k_route_count, dim3(D.B, D.N), dim3(kThreads), lds, st, D, W, idx, send_pos);
    if (rc != MOE_OK) return rc;
  } else {
    // No slots: the scan still publishes zero counts; reset the ticket.
    const int rc = launch_fill_u32(W.ticket, 0u, 1, st);
    if (rc != MOE_OK) return rc;
  }
  return launch("k_route_scan", k_route_scan, dim3(D.N), dim3(kThreads), 0, st, D, W);
}

}  // namespace moe
