// Combine ("Enabling trillion-parameter models on AWS EFA": section
// "Introduction" -- combine returns the processed rows to their source and
// forms each token's weighted average; section "Dispatch and combine" --
// routing is already known from dispatch, rows go back with one contiguous
// write per peer and the receive side accumulates them into the output).
//
//   k_comb_send_os        comb[row_src[p]] = y[p], one 16-byte unit per
//                         thread over the valid expert-major rows
//                         (k_comb_zero_dropped after a fixed-region
//                         overflow: zero rows for the slots left without a
//                         row)
//   k_comb_recv_os        out = bf16(sum_j w_j * y_j), float32 in slot order,
//                         one 16-byte output unit per thread
//   k_comb_pull_os        the same sum, rows read in place (expert-major),
//                         two output units per thread
//   k_comb_send_partial   send-side partial sums: one bf16 row per (token,
//                         destination rank) group ("Evaluation:
//                         dispatch/combine latency": accumulating on the send
//                         side cuts the data sent); one 1024-thread
//                         workgroup per CU on chunks of tokens,
//                         thread-interleaved 16-byte units
//                         (k_comb_send_partial_os, one-shot, below 16384
//                         tokens)
//   k_comb_recv_partial_os  the receive side of it: float32 sum of a token's
//                         group rows, bf16 out
#include "moe_internal.h"

namespace moe {


// acc = fl(acc + fl(w * y)) in slot order, never fused into an FMA.
__device__ __forceinline__ void acc_row8(float* acc, float w, const v4u& v) {
#pragma clang fp contract(off)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float p0 = w * bf16_lo(v[i]);
    const float p1 = w * bf16_hi(v[i]);
    acc[2 * i] = acc[2 * i] + p0;
    acc[2 * i + 1] = acc[2 * i + 1] + p1;
  }
}

// bf16 bits of 8 float32 sums, packed for one 16-byte store.
__device__ __forceinline__ v4u pack_bf16x8(const float* acc) {
  v4u o;
  o[0] = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
  o[1] = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
  o[2] = f32_to_bf16_rne(acc[4]) | (f32_to_bf16_rne(acc[5]) << 16);
  o[3] = f32_to_bf16_rne(acc[6]) | (f32_to_bf16_rne(acc[7]) << 16);
  return o;
}

constexpr int kSlotGroup = 8;     // slot rows loaded together per sum step

// Expert-major row of a slot of source s with expert e and sender position
// sp, found from the routing tables: the row combine_send would copy back.
// -1 for a bad id, or a row that a full fixed region dropped.
__device__ __forceinline__ int em_row_of(const Dims& D, const Ws& W, int s, int e, int sp) {
  if (e < 0 || e >= D.E || sp < 0 || sp >= D.TK) return -1;
  const int d = e / D.L, l = e - d * D.L;
  const int* so = W.send_off + s * (D.E + 1);
  const int u = sp - so[e];                                                         // index inside (s, e)
  const int i = W.exp_off[d * (D.L + 1) + l] + W.src_in_exp[s * D.E + e] + u;      // expert-major
  const int j = region_row(D, s, (so[e] - so[d * D.L]) + u, W.recv_off[d * (D.N + 1) + s]);   // source-major
  const int p = W.base[d] + i;
  return (u >= 0 && i >= 0 && j >= 0 && (D.R == 0 || (i < D.R && j < D.R)) && p < D.rows) ? p : -1;
}

// With fixed regions that overflowed, a valid slot can be left without an
// expert-major row (its own index or its source-major row did not fit).  No
// row_src entry names its comb row, so the copy loop never writes it; this
// pass writes it as zeros instead, so that the receive half's sum skips the
// slot exactly (adding w * +0 leaves a float32 sum unchanged, and the sum,
// starting at +0, never holds -0), as the pulling combine does.  Comb rows
// at positions no valid slot has are left untouched.  Without an overflow
// every workgroup returns after reading the region totals.
template <int WAVES>
__device__ void zero_dropped_rows(const Dims& D, const Ws& W, uint16_t* __restrict__ comb) {
  __shared__ int over;
  if (threadIdx.x == 0) over = 0;
  __syncthreads();
  for (int d = threadIdx.x; d < D.N; d += WAVES * kWave)
    if (W.recv_total[d] > D.R || D.N * D.Ce + W.recv_off[d * (D.N + 1) + D.N] > D.R) atomicOr(&over, 1);
  __syncthreads();
  if (!over) return;
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int n16 = D.H / 8;
  int lo, hi;
  block_range(D.N * D.TK, lo, hi);   // comb rows s*T*k + sender position
  for (int p0 = lo + wv * kWave; p0 < hi; p0 += WAVES * kWave) {
    const int pos = p0 + lane;
    bool drop = false;
    if (pos < hi) {
      const int s = pos / D.TK, p = pos - s * D.TK;
      const int* so = W.send_off + s * (D.E + 1);
      if (p < so[D.E]) drop = em_row_of(D, W, s, floor_index(so, D.E + 1, p), p) < 0;
    }
    for (uint64_t m = __ballot(drop); m; m &= m - 1) {
      v4u* row = reinterpret_cast<v4u*>(comb + (int64_t)(p0 + __builtin_ctzll(m)) * D.H);
      for (int c = lane; c < n16; c += kWave) st16(row + c, v4u{0, 0, 0, 0});
    }
  }
}

// ------------------------------------------------------------------ one-shot forms

// Combine send, one-shot: comb[row_src[p]] = y[p] over the valid rows
// (region order), one 16-byte unit per thread, 64-thread workgroups.  Each
// thread looks its row up itself (the row's 896 units at H = 7168 share the
// row_src entry in the cache).  Against 256-thread tiles that first resolved
// their rows into LDS: 4% faster at combine-heavy size, 0.3-2.5% at the
// others.
constexpr int kSendThreads = 64;
__global__ __launch_bounds__(kSendThreads) void k_comb_send_os(Dims D, Ws W, const uint16_t* __restrict__ y,
                                                              const int* __restrict__ row_src,
                                                              uint16_t* __restrict__ comb) {
  const int n16 = D.H / 8;
  const int valid = W.vprefix[D.N];
  const int64_t units = (int64_t)valid * n16;
  const int ncomb = D.N * D.TK;
  const v4u* __restrict__ ys = reinterpret_cast<const v4u*>(y);
  v4u* __restrict__ cs = reinterpret_cast<v4u*>(comb);
  for (int64_t tile = blockIdx.x; tile * kSendThreads < units; tile += gridDim.x) {
    const int64_t u0 = tile * kSendThreads;
    if (u0 + threadIdx.x >= units) continue;
    int g0, g, c;
    os_tile_pos(u0, n16, g0, g, c);
    int p = g;                                     // packed regions: valid row g is physical row g
    if (D.R) {
      const int d = floor_index(W.vprefix, D.N + 1, g);
      p = W.base[d] + (g - W.vprefix[d]);
    }
    if (p >= D.rows) continue;
    const int rs = row_src[p];
    if (rs >= 0 && rs < ncomb) st16(cs + (int64_t)rs * n16 + c, ld16(ys + (int64_t)p * n16 + c));
  }
}

// After a fixed-region overflow: the zero rows of valid slots left without a
// row (see zero_dropped_rows), as a kernel of its own beside the one-shot send.
__global__ __launch_bounds__(1024) void k_comb_zero_dropped(Dims D, Ws W, uint16_t* __restrict__ comb) {
  zero_dropped_rows<16>(D, W, comb);
}

enum class CombMode { kPull, kRecvPartial };

// The pulling sum and the sum of group rows, one-shot: one 16-byte output
// unit (8 elements of a token row) per thread.  The tile's tokens have their
// slots resolved into LDS first (slot row, weight; for kRecvPartial only group leaders keep a
// row, with weight 1), then every thread loads the same 16 bytes of each of
// its token's slot rows and sums them in slot order (acc = fl(acc +
// fl(w * y)), no fused multiply-add).
// U output units per thread and TH threads per workgroup (tiles of U * TH
// units).  U = 2: the slot resolution (the routing-table lookups, the leader
// pass) is amortised over twice the units (1-12% faster than 1; 4 was
// slower).  TH = 64 (one wave per workgroup): 1.5-3% faster than 256 from
// the decode shape up, 2-3% slower at the tiny shape; 128 was slower than
// both.
constexpr int kCombThreads = 64;
template <int U, int TH>
constexpr int os_tile_tokens() { return TH * U / 16 + 2; }   // tokens a tile spans (>= 16 units per row)
template <CombMode MODE, int U, int TH>
__device__ __forceinline__ void combine_os(const Dims& D, const Ws& W, const uint16_t* __restrict__ rows,
                                           const int* __restrict__ idx, const int* __restrict__ send_pos,
                                           const float* __restrict__ topk_w, uint16_t* __restrict__ out) {
  constexpr int kTile = TH * U;
  constexpr int kOsSlotTable = os_tile_tokens<U, TH>() * kMaxK;
  __shared__ int t_row[kOsSlotTable];
  // (group rows carry weight 1: the partial receive keeps no weights)
  __shared__ float t_w[MODE == CombMode::kRecvPartial ? 1 : kOsSlotTable];
  __shared__ int t_dest[MODE == CombMode::kRecvPartial ? kOsSlotTable : 1];
  const int n16 = D.H / 8, k = D.k;
  const int64_t units = (int64_t)D.N * D.T * n16;
  const v4u* __restrict__ rs = reinterpret_cast<const v4u*>(rows);
  v4u* __restrict__ os = reinterpret_cast<v4u*>(out);
  for (int64_t tile = blockIdx.x; tile * kTile < units; tile += gridDim.x) {
    const int64_t u0 = tile * kTile;
    int t0, tok, c;
    os_tile_pos(u0, n16, t0, tok, c);
    const int64_t ul = u0 + kTile - 1 < units ? u0 + kTile - 1 : units - 1;
    const int nt = (int)(ul - (int64_t)t0 * n16) / n16 + 1;
    __syncthreads();   // the previous tile's reads of the tables are done
    for (int i = threadIdx.x; i < nt * k; i += TH) {
      const int64_t slot = (int64_t)t0 * k + i;               // token t0 + i / k, slot i % k
      const int s = (t0 + i / k) / D.T;
      const int sp = send_pos[slot];
      const int e = idx[slot];
      int row;
      if constexpr (MODE == CombMode::kRecvPartial) {
        // Only whether the slot has a row matters here: with packed
        // regions every valid slot has one, so the lookup is skipped.
        const bool has = D.R == 0 ? (e >= 0 && e < D.E && sp >= 0 && sp < D.TK) : em_row_of(D, W, s, e, sp) >= 0;
        t_dest[i] = has ? e / D.L : -1;
        row = has ? s * D.TK + sp : -1;
      } else {
        row = em_row_of(D, W, s, e, sp);
      }
      t_row[i] = row;
      if constexpr (MODE != CombMode::kRecvPartial) t_w[i] = topk_w[slot];
    }
    if constexpr (MODE == CombMode::kRecvPartial) {
      // A slot with a row leads its group unless an earlier slot of the
      // token has a row on the same rank; only leaders' group rows are summed.
      // The test reads t_dest only, so each entry drops its own row in one
      // pass.
      __syncthreads();
      for (int i = threadIdx.x; i < nt * k; i += TH) {
        const int j = i % k, b = i - j, d = t_dest[i];
        bool l = d >= 0;
        for (int jj = 0; jj < j; ++jj) l = l && t_dest[b + jj] != d;
        if (!l) t_row[i] = -1;
      }
    }
    __syncthreads();
    for (int q = 0; q < U; ++q) {
      const int64_t uu = u0 + threadIdx.x + q * TH;
      if (q > 0) {   // this thread's next unit, TH further on
        c += TH;
        while (c >= n16) {
          c -= n16;
          ++tok;
        }
      }
      if (uu >= units) break;
      const int* tr = t_row + (tok - t0) * k;
      const float* tw = MODE == CombMode::kRecvPartial ? t_w : t_w + (tok - t0) * k;
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
      for (int j0 = 0; j0 < k; j0 += kSlotGroup) {
        v4u v[kSlotGroup];
        int rr[kSlotGroup];
#pragma unroll
        for (int jj = 0; jj < kSlotGroup; ++jj) {
          rr[jj] = j0 + jj < k ? tr[j0 + jj] : -1;
          v[jj] = rr[jj] >= 0 ? ld16(rs + (int64_t)rr[jj] * n16 + c) : v4u{0, 0, 0, 0};
        }
#pragma unroll
        for (int jj = 0; jj < kSlotGroup; ++jj)
          if (rr[jj] >= 0) acc_row8(acc, MODE == CombMode::kRecvPartial ? 1.0f : tw[j0 + jj], v[jj]);
      }
      st16(os + uu, pack_bf16x8(acc));
    }
  }
}

// The plain sum, one 16-byte output unit (8 elements of token tok, column
// unit c) per thread, each thread looking its token's slots up itself: the
// 64 threads of a workgroup mostly share one token, so the lookups are cache
// hits.  Against tiles that first resolved their tokens' slots into LDS: 3-8%
// faster from the decode shape up (0.7 us slower at the tiny shape).  The
// pulling sum keeps the LDS tiles: its per-slot routing-table lookup done by
// every thread was twice as slow.
__device__ __forceinline__ v4u recv_unit(const Dims& D, const v4u* __restrict__ rs, const int* __restrict__ send_pos,
                                         const float* __restrict__ topk_w, int tok, int c) {
  const int n16 = D.H / 8, k = D.k, s = tok / D.T;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  for (int j0 = 0; j0 < k; j0 += kSlotGroup) {
    v4u v[kSlotGroup];
    int rr[kSlotGroup];
    float ww[kSlotGroup];
#pragma unroll
    for (int jj = 0; jj < kSlotGroup; ++jj) {
      const int j = j0 + jj;
      rr[jj] = -1;
      ww[jj] = 0.0f;
      if (j < k) {
        const int64_t slot = (int64_t)tok * k + j;
        const int sp = send_pos[slot];
        rr[jj] = sp >= 0 && sp < D.TK ? s * D.TK + sp : -1;
        ww[jj] = topk_w[slot];
      }
    }
#pragma unroll
    for (int jj = 0; jj < kSlotGroup; ++jj) v[jj] = rr[jj] >= 0 ? ld16(rs + (int64_t)rr[jj] * n16 + c) : v4u{0, 0, 0, 0};
#pragma unroll
    for (int jj = 0; jj < kSlotGroup; ++jj)
      if (rr[jj] >= 0) acc_row8(acc, ww[jj], v[jj]);
  }
  return pack_bf16x8(acc);
}

constexpr int kPullUnits = 2;   // output units per thread of the pulling sum

__global__ __launch_bounds__(kCombThreads) void k_comb_recv_os(Dims D, Ws W, const uint16_t* __restrict__ comb,
                                                            const int* __restrict__ send_pos,
                                                            const float* __restrict__ topk_w,
                                                            uint16_t* __restrict__ out) {
  const int n16 = D.H / 8;
  const int64_t units = (int64_t)D.N * D.T * n16;
  const v4u* __restrict__ rs = reinterpret_cast<const v4u*>(comb);
  v4u* __restrict__ os = reinterpret_cast<v4u*>(out);
  for (int64_t tile = blockIdx.x; tile * kCombThreads < units; tile += gridDim.x) {
    const int64_t u0 = tile * kCombThreads;
    if (u0 + threadIdx.x >= units) continue;
    int t0, tok, c;
    os_tile_pos(u0, n16, t0, tok, c);
    st16(os + u0 + threadIdx.x, recv_unit(D, rs, send_pos, topk_w, tok, c));
  }
}

__global__ __launch_bounds__(kCombThreads) void k_comb_pull_os(Dims D, Ws W, const uint16_t* __restrict__ y,
                                                            const int* __restrict__ idx,
                                                            const int* __restrict__ send_pos,
                                                            const float* __restrict__ topk_w,
                                                            uint16_t* __restrict__ out) {
  combine_os<CombMode::kPull, kPullUnits, kCombThreads>(D, W, y, idx, send_pos, topk_w, out);
}

__global__ __launch_bounds__(kCombThreads) void k_comb_recv_partial_os(Dims D, Ws W, const uint16_t* __restrict__ comb,
                                                                    const int* __restrict__ idx,
                                                                    const int* __restrict__ send_pos,
                                                                    uint16_t* __restrict__ out) {
  combine_os<CombMode::kRecvPartial, 2, kCombThreads>(D, W, comb, idx, send_pos, nullptr, out);
}

// Send-side partial sums, one-shot: one 16-byte unit (8 columns of a token
// row) per thread.  The tile's tokens have every slot resolved into LDS (its
// expert-major row, weight, destination rank and, for a group leader, the
// comb row its group returns to); each thread loads the same 16 bytes of
// all of its token's slot rows and forms every group's sum from registers
// (k <= kSlotGroup), or takes the groups one after another (larger k), in
// slot order as the chunked form does.  The form for fewer than 16384
// tokens: against the chunked form it took 163 against 188 us at the
// decode shape and 29 against 45 at the tiny one, but 10.9 against 9.4 ms
// at the Kimi combine (one process, same buffers); two units per thread
// were no faster.
__global__ __launch_bounds__(kOsThreads) void k_comb_send_partial_os(Dims D, Ws W, const uint16_t* __restrict__ y,
                                                                    const int* __restrict__ idx,
                                                                    const int* __restrict__ send_pos,
                                                                    const float* __restrict__ topk_w,
                                                                    uint16_t* __restrict__ comb) {
  constexpr int U = 1;
  constexpr int kTile = kOsThreads * U;
  constexpr int kTab = os_tile_tokens<U, kOsThreads>() * kMaxK;
  __shared__ int t_row[kTab], t_dest[kTab], t_out[kTab];
  __shared__ float t_w[kTab];
  const int n16 = D.H / 8, k = D.k;
  const int64_t units = (int64_t)D.N * D.T * n16;
  const v4u* __restrict__ ys = reinterpret_cast<const v4u*>(y);
  v4u* __restrict__ cs = reinterpret_cast<v4u*>(comb);
  for (int64_t tile = blockIdx.x; tile * kTile < units; tile += gridDim.x) {
    const int64_t u0 = tile * kTile;
    int t0, tok, c;
    os_tile_pos(u0, n16, t0, tok, c);
    const int64_t ul = u0 + kTile - 1 < units ? u0 + kTile - 1 : units - 1;
    const int nt = (int)(ul - (int64_t)t0 * n16) / n16 + 1;
    __syncthreads();   // the previous tile's reads of the tables are done
    for (int i = threadIdx.x; i < nt * k; i += kOsThreads) {
      const int64_t slot = (int64_t)t0 * k + i;               // token t0 + i / k, slot i % k
      const int s = (t0 + i / k) / D.T;
      const int sp = send_pos[slot];
      const int e = idx[slot];
      const int row = em_row_of(D, W, s, e, sp);
      t_row[i] = row;
      t_w[i] = topk_w[slot];
      t_dest[i] = row >= 0 ? e / D.L : -1;
      t_out[i] = row >= 0 ? s * D.TK + sp : -1;
    }
    __syncthreads();
    // A slot with a row leads its group unless an earlier slot of the token
    // has a row on the same rank (reads t_dest only; each entry writes its
    // own t_out).
    for (int i = threadIdx.x; i < nt * k; i += kOsThreads) {
      const int j = i % k, b = i - j, d = t_dest[i];
      bool lead = d >= 0;
      for (int jj = 0; jj < j; ++jj) lead = lead && t_dest[b + jj] != d;
      if (!lead) t_out[i] = -1;
    }
    __syncthreads();
    for (int q = 0; q < U; ++q) {
      const int64_t uu = u0 + threadIdx.x + q * kOsThreads;
      if (q > 0) {
        c += kOsThreads;
        while (c >= n16) {
          c -= n16;
          ++tok;
        }
      }
      if (uu >= units) break;
      const int b = (tok - t0) * k;
      if (k <= kSlotGroup) {
        v4u v[kSlotGroup];
#pragma unroll
        for (int j = 0; j < kSlotGroup; ++j) {
          const int r = j < k ? t_row[b + j] : -1;
          v[j] = r >= 0 ? ld16(ys + (int64_t)r * n16 + c) : v4u{0, 0, 0, 0};
        }
#pragma unroll
        for (int g = 0; g < kSlotGroup; ++g) {
          const int og = g < k ? t_out[b + g] : -1;
          if (og < 0) continue;   // not a leader
          const int dg = t_dest[b + g];
          float acc[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
          for (int j = g; j < kSlotGroup; ++j)
            if (j < k && t_dest[b + j] == dg) acc_row8(acc, t_w[b + j], v[j]);
          st16(cs + (int64_t)og * n16 + c, pack_bf16x8(acc));
        }
      } else {
        for (int g = 0; g < k; ++g) {
          const int og = t_out[b + g];
          if (og < 0) continue;
          const int dg = t_dest[b + g];
          float acc[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
          for (int j0 = g; j0 < k; j0 += kSlotGroup) {
            v4u v[kSlotGroup];
            int rr[kSlotGroup];
#pragma unroll
            for (int jj = 0; jj < kSlotGroup; ++jj) {
              const int j = j0 + jj;
              rr[jj] = j < k && t_dest[b + j] == dg ? t_row[b + j] : -1;
              v[jj] = rr[jj] >= 0 ? ld16(ys + (int64_t)rr[jj] * n16 + c) : v4u{0, 0, 0, 0};
            }
#pragma unroll
            for (int jj = 0; jj < kSlotGroup; ++jj)
              if (rr[jj] >= 0) acc_row8(acc, t_w[b + j0 + jj], v[jj]);
          }
          st16(cs + (int64_t)og * n16 + c, pack_bf16x8(acc));
        }
      }
    }
  }
}

// The send-side partial sums with the whole workgroup on a chunk of
// consecutive tokens (the plain copy's pattern, as k_comb_send): each slot's
// expert-major row, weight, destination rank and, for a group leader, its
// comb position are resolved into LDS; then thread t forms the 16-byte
// units t, t + kPsThreads, ... of every group row of the chunk's tokens,
// each from the same 16 bytes of the group's member rows, summed in slot
// order exactly as k_comb_send_partial does.
constexpr int kPsThreads = 1024, kPsUnits = 8, kPsTable = 2048, kPsPair = 1;
__global__ __launch_bounds__(kPsThreads) void k_comb_send_partial(Dims D, Ws W, const uint16_t* __restrict__ y,
                                                                       const int* __restrict__ idx,
                                                                       const int* __restrict__ send_pos,
                                                                       const float* __restrict__ topk_w,
                                                                       uint16_t* __restrict__ comb) {
  __shared__ int t_row[kPsTable], t_dest[kPsTable], t_out[kPsTable];
  __shared__ float t_w[kPsTable];
  const int n16 = D.H / 8, k = D.k;
  int ntok = kPsThreads * kPsUnits / n16;                 // tokens per chunk
  ntok = max(1, min(ntok, kPsTable / k));
  const v4u* __restrict__ ys = reinterpret_cast<const v4u*>(y);
  v4u* __restrict__ cs = reinterpret_cast<v4u*>(comb);
  int lo, hi;
  block_range(D.N * D.T, lo, hi);
  for (int t0 = lo; t0 < hi; t0 += ntok) {
    const int nt = min(ntok, hi - t0);
    for (int i = threadIdx.x; i < nt * k; i += kPsThreads) {
      const int64_t slot = (int64_t)t0 * k + i;               // token t0 + i / k, slot i % k
      const int s = (t0 + i / k) / D.T;
      const int sp = send_pos[slot];
      const int e = idx[slot];
      const int row = em_row_of(D, W, s, e, sp);
      t_row[i] = row;
      t_w[i] = topk_w[slot];
      t_dest[i] = row >= 0 ? e / D.L : -1;
      t_out[i] = row >= 0 ? s * D.TK + sp : -1;
    }
    __syncthreads();
    // A slot with a row leads its group unless an earlier slot of the token
    // has a row on the same rank.
    for (int i = threadIdx.x; i < nt * k; i += kPsThreads) {
      const int j = i % k, b = i - j, d = t_dest[i];
      bool lead = d >= 0;
      for (int jj = 0; jj < j; ++jj) lead = lead && t_dest[b + jj] != d;
      if (!lead) t_out[i] = -1;
    }
    __syncthreads();
    const int nf = nt * n16;
    if (k <= kSlotGroup) {
      // kPsPair units per thread and step, all their slot loads issued first.
      for (int f0 = threadIdx.x; f0 < nf; f0 += kPsThreads * kPsPair) {
        v4u v[kPsPair][kSlotGroup];
#pragma unroll
        for (int q = 0; q < kPsPair; ++q) {
          const int f = f0 + q * kPsThreads, tt = f / n16, c = f - tt * n16, b = tt * k;
#pragma unroll
          for (int j = 0; j < kSlotGroup; ++j) {
            const int r = f < nf && j < k ? t_row[b + j] : -1;
            v[q][j] = r >= 0 ? ld16(ys + (int64_t)r * n16 + c) : v4u{0, 0, 0, 0};
          }
        }
#pragma unroll
        for (int q = 0; q < kPsPair; ++q) {
          const int f = f0 + q * kPsThreads, tt = f / n16, c = f - tt * n16, b = tt * k;
          if (f >= nf) continue;
#pragma unroll
          for (int g = 0; g < kSlotGroup; ++g) {
            const int og = g < k ? t_out[b + g] : -1;
            if (og < 0) continue;   // not a leader
            const int dg = t_dest[b + g];
            float acc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
            for (int j = g; j < kSlotGroup; ++j)
              if (j < k && t_dest[b + j] == dg) acc_row8(acc, t_w[b + j], v[q][j]);
            st16(cs + (int64_t)og * n16 + c, pack_bf16x8(acc));
          }
        }
      }
    } else {
      for (int f = threadIdx.x; f < nf; f += kPsThreads) {
        const int tt = f / n16, c = f - tt * n16, b = tt * k;
        for (int g = 0; g < k; ++g) {
          const int og = t_out[b + g];
          if (og < 0) continue;
          const int dg = t_dest[b + g];
          float acc[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
          for (int j0 = g; j0 < k; j0 += kSlotGroup) {
            v4u v[kSlotGroup];
            int rr[kSlotGroup];
#pragma unroll
            for (int jj = 0; jj < kSlotGroup; ++jj) {
              const int j = j0 + jj;
              rr[jj] = j < k && t_dest[b + j] == dg ? t_row[b + j] : -1;
              v[jj] = rr[jj] >= 0 ? ld16(ys + (int64_t)rr[jj] * n16 + c) : v4u{0, 0, 0, 0};
            }
#pragma unroll
            for (int jj = 0; jj < kSlotGroup; ++jj)
              if (rr[jj] >= 0) acc_row8(acc, t_w[b + j0 + jj], v[jj]);
          }
          st16(cs + (int64_t)og * n16 + c, pack_bf16x8(acc));
        }
      }
    }
    __syncthreads();
  }
}

int launch_comb_send(const Dims& D, const Ws& W, const uint16_t* y, const int* row_src, uint16_t* comb, int cus,
                     hipStream_t st) {
  if (D.N * D.TK == 0) return MOE_OK;
  const int rc = launch("k_comb_send_os", k_comb_send_os, dim3(os_grid((int64_t)D.rows * (D.H / 8), kSendThreads)),
                        dim3(kSendThreads), 0, st, D, W, y, row_src, comb);
  if (rc != MOE_OK || D.R == 0) return rc;   // packed regions never overflow
  return launch("k_comb_zero_dropped", k_comb_zero_dropped, dim3(cus), dim3(1024), 0, st, D, W, comb);
}

int launch_comb_recv(const Dims& D, const uint16_t* comb, const int* send_pos, const float* w, uint16_t* out, int cus,
                     hipStream_t st) {
  if (D.N * D.T == 0) return MOE_OK;
  return launch("k_comb_recv_os", k_comb_recv_os, dim3(os_grid((int64_t)D.N * D.T * (D.H / 8), kCombThreads)),
                dim3(kCombThreads), 0, st, D, Ws{}, comb, send_pos, w, out);
}

int launch_comb_pull(const Dims& D, const Ws& W, const uint16_t* y, const int* idx, const int* send_pos,
                     const float* w, uint16_t* out, int cus, hipStream_t st) {
  if (D.N * D.T == 0) return MOE_OK;
  return launch("k_comb_pull_os", k_comb_pull_os, dim3(os_grid((int64_t)D.N * D.T * (D.H / 8), kPullUnits * kCombThreads)),
                dim3(kCombThreads), 0, st, D, W, y, idx, send_pos, w, out);
}

constexpr int64_t kPsMinTokens = 16384;   // tokens (N*T) from which the cooperative form is used

int launch_comb_send_partial(const Dims& D, const Ws& W, const uint16_t* y, const int* idx, const int* send_pos,
                             const float* w, uint16_t* comb, int cus, hipStream_t st) {
  if (D.N * D.T == 0) return MOE_OK;
  if ((int64_t)D.N * D.T >= kPsMinTokens) {
    const int64_t need = ((int64_t)D.N * D.T * (D.H / 8) + kPsThreads * kPsUnits - 1) / (kPsThreads * kPsUnits);
    const int grid = (int)(need < cus ? (need < 1 ? 1 : need) : cus);
    return launch("k_comb_send_partial", k_comb_send_partial, dim3(grid), dim3(kPsThreads), 0, st, D, W, y,
                  idx, send_pos, w, comb);
  }
  return launch("k_comb_send_partial_os", k_comb_send_partial_os, dim3(os_grid((int64_t)D.N * D.T * (D.H / 8))),
                dim3(kOsThreads), 0, st, D, W, y, idx, send_pos, w, comb);
}

int launch_comb_recv_partial(const Dims& D, const Ws& W, const uint16_t* comb, const int* idx, const int* send_pos,
                             uint16_t* out, int cus, hipStream_t st) {
  if (D.N * D.T == 0) return MOE_OK;
  return launch("k_comb_recv_partial_os", k_comb_recv_partial_os,
                dim3(os_grid((int64_t)D.N * D.T * (D.H / 8), 2 * kCombThreads)), dim3(kCombThreads), 0, st, D, W, comb,
                idx, send_pos, out);
}

}  // namespace moe
