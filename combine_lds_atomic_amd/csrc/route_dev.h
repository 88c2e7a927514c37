// Device code of the routing count, shared by the routing kernels and the
// single-launch dispatch ("Enabling trillion-parameter models on AWS EFA",
// sections "Send and receive buffers" and "Dispatch and combine": per-expert
// counts in shared memory with atomics, then exclusive prefix sums that give
// every (source, expert) slot a conflict-free, contiguous position).
#pragma once

#include "moe_internal.h"

namespace moe {

// Exclusive scan of one value per thread over a block of THREADS threads.
// Returns the thread's exclusive prefix; *total gets the block total.
// wsum: LDS scratch of THREADS/64 + 1 ints.
template <int THREADS>
__device__ int block_scan(int v, int* wsum, int* total) {
  constexpr int kW = THREADS / kWave;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == kWave - 1) wsum[w] = x;
  __syncthreads();
  if (w == 0) {
    const int t = lane < kW ? wsum[lane] : 0;
    int u = t;
#pragma unroll
    for (int d = 1; d < kW; d <<= 1) {
      const int y = __shfl_up(u, d);
      if (lane >= d) u += y;
    }
    if (lane < kW) wsum[lane] = u - t;         // exclusive wave offsets
    if (lane == kW - 1) wsum[kW] = u;          // block total
  }
  __syncthreads();
  const int r = wsum[w] + x - v;
  *total = wsum[kW];
  __syncthreads();
  return r;
}

// Exclusive scan of one value per lane over a wave (no barrier); *total
// gets the wave total.
__device__ __forceinline__ int wave_scan(int v, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  int x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  *total = __shfl(x, kWave - 1);
  return x - v;
}

// LDS bytes count_chunk needs for E experts.
inline size_t count_lds_bytes(int E) {
  return (size_t)kWavesPerBlock * E * (sizeof(unsigned long long) + sizeof(int));
}

// Counts and in-chunk ranks of chunk b (D.C slots) of rank s; 256 threads.
//
// Each wave walks its quarter of the chunk 64 slots at a time.  Lane i ORs
// bit i into an LDS mask of its expert (ds_or_b64: one LDS atomic per slot);
// afterwards every lane reads its expert's mask and knows the lanes of this
// batch that share its expert.  rank = running count of the expert in this
// wave + lanes below it in the mask; the highest lane of each group advances
// the running count and clears the mask.  Ranks therefore follow slot order,
// which makes the final positions unique and reproducible.
//
// With one chunk per rank (D.B == 1) the rank's scan over experts is done
// here too: cnt, send_off and send_pos are final.  Otherwise the chunk counts
// go to W.blk and the in-chunk ranks to W.local.  A non-zero `tag` (one chunk
// per rank only) also publishes the positions, counts and per-destination
// send offsets as tagged values for workgroups of the same launch.
__device__ __forceinline__ void count_chunk(const Dims& D, const Ws& W, const int* __restrict__ idx,
                                            int* __restrict__ send_pos, int s, int b, unsigned char* smem,
                                            int* wsum, uint32_t tag) {
  unsigned long long* mask = reinterpret_cast<unsigned long long*>(smem);   // [4][E]
  int* run = reinterpret_cast<int*>(mask + kWavesPerBlock * D.E);            // [4][E]
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  for (int i = threadIdx.x; i < kWavesPerBlock * D.E; i += kThreads) {
    mask[i] = 0ull;
    run[i] = 0;
  }

  const int64_t rbase = (int64_t)s * D.TK;
  const int per_wave = D.C / kWavesPerBlock;
  const int c0 = b * D.C + w * per_wave;
  const int cend = min(c0 + per_wave, D.TK);
  // All of this wave's ids are loaded before any LDS work.  ev[bt] holds the
  // slot's expert and, once ranked, its rank in this wave's run of that
  // expert: (rank << 11) | (e + 1), 0 for no expert (e < 1024, rank < 1024).
  int ev[kMaxBatches];
  bool bad = false;
#pragma unroll
  for (int bt = 0; bt < kMaxBatches; ++bt) {
    const int i = c0 + bt * kWave + lane;
    int e = -1;
    if (bt * kWave < per_wave && i < cend) {
      e = idx[rbase + i];
      if (e < 0 || e >= D.E) {
        bad = true;
        e = -1;
      }
    }
    ev[bt] = e;
  }
  __syncthreads();

  unsigned long long* wm = mask + w * D.E;
  int* wr = run + w * D.E;
#pragma unroll
  for (int bt = 0; bt < kMaxBatches; ++bt) {
    if (bt * kWave < per_wave) {   // wave-uniform
      const int e = ev[bt];   // still the plain expert id here
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
      ev[bt] = e >= 0 ? (r << 11) | (e + 1) : 0;
    }
  }
  if (__any(bad) && lane == 0) atomicOr(W.err, MOE_FLAG_BADID);
  __syncthreads();

  // Exclusive prefix over the four waves, per expert; the chunk totals go to
  // the workspace.  Thread t owns experts [t*per, t*per + per).
  const int per = (D.E + kThreads - 1) / kThreads;
  const int e0 = min(D.E, (int)threadIdx.x * per), e1 = min(D.E, e0 + per);
  int mine = 0;
  for (int e = e0; e < e1; ++e) {
    int p = 0;
#pragma unroll
    for (int ww = 0; ww < kWavesPerBlock; ++ww) {
      const int c = run[ww * D.E + e];
      run[ww * D.E + e] = p;
      p += c;
    }
    if (D.B > 1) {
      W.blk[((int64_t)s * D.B + b) * D.E + e] = p;
    } else {
      W.cnt[s * D.E + e] = p;
      if (tag) tag_put(W.tcnt + (int64_t)s * D.E + e, tag, p);
    }
    mask[e] = (unsigned long long)p;       // masks are all clear again: reuse as scratch
    mine += p;
  }
  if (D.B == 1) {
    // The whole rank is this chunk: its scan over experts makes the
    // positions final here.
    int total;
    int off = block_scan<kThreads>(mine, wsum, &total);
    int* so = W.send_off + s * (D.E + 1);
    for (int e = e0; e < e1; ++e) {
      so[e] = off;
      if (tag && e % D.L == 0) tag_put(W.toff + (int64_t)s * (D.N + 1) + e / D.L, tag, off);
#pragma unroll
      for (int ww = 0; ww < kWavesPerBlock; ++ww) run[ww * D.E + e] += off;
      off += (int)mask[e];
    }
    if (threadIdx.x == 0) {
      so[D.E] = total;
      if (tag) tag_put(W.toff + (int64_t)s * (D.N + 1) + D.N, tag, total);
    }
  }
  __syncthreads();
#pragma unroll
  for (int bt = 0; bt < kMaxBatches; ++bt) {
    const int i = c0 + bt * kWave + lane;
    if (bt * kWave >= per_wave || i >= cend) continue;
    const int e = (ev[bt] & 0x7FF) - 1;
    const int v = e >= 0 ? wr[e] + (ev[bt] >> 11) : -1;
    if (D.B == 1) {
      send_pos[rbase + i] = v;   // final position
      if (tag) tag_put(W.tpos + rbase + i, tag, v);
    } else {
      W.local[rbase + i] = v;    // rank inside the chunk; the pack adds the chunk base
    }
  }
}

}  // namespace moe
