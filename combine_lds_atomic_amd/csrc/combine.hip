// Combine ("Enabling trillion-parameter models on AWS EFA": section
// "Introduction" -- combine returns the processed rows to their source and
// forms each token's weighted average; section "Dispatch and combine" --
// routing is already known from dispatch, rows go back with one contiguous
// write per peer and the receive side accumulates them into the output).
//
//   k_comb_send          comb[row_src[i]] = y[i] (after a fixed-region
//                        overflow, also zero rows for the slots left without
//                        a row): one 1024-thread workgroup per CU copies its
//                        range of expert-major rows as one flat range of
//                        16-byte units, thread-interleaved
//   k_comb_send_rows     the same with one wave per row (problems below
//                        131072 rows)
//   k_comb_recv          each workgroup streams a contiguous range of
//                        tokens: fp32 sum over slots of w * y, bf16 out; one
//                        1024-thread workgroup per CU, thread-interleaved
//                        16-byte output units (k_comb_recv_tokens: one wave
//                        per token, below 16384 tokens)
//   k_comb_pull          the same sum, rows read in place (expert-major);
//                        k_comb_pull_tokens below 16384 tokens
//   k_comb_send_partial  send-side partial sums: one bf16 row per (token,
//                        destination rank) group ("Evaluation:
//                        dispatch/combine latency": accumulating on the send
//                        side cuts the data sent); one 1024-thread
//                        workgroup per CU on chunks of tokens,
//                        thread-interleaved 16-byte units
//                        (k_comb_send_partial_tokens: one wave per token,
//                        below 16384 tokens)
//   k_comb_recv_partial  the receive side of it: fp32 sum of a token's group
//                        rows, bf16 out
#include "moe_internal.h"

namespace moe {

constexpr int kRowsPerPass = 8;   // rows whose metadata one wave resolves at once
constexpr int kCsWaves = kCombSendShape.waves, kCsThreads = kCombSendShape.threads();
// 16-B loads per lane issued together while copying a row.  A 7168-wide bf16
// row needs 14; 32 (with 8-wave workgroups, two per CU) measured 2-5% faster
// than 16 with 16-wave workgroups, in one process at three workloads.
constexpr int kCsUnroll = 32;
constexpr int kCrWaves = kCombRecvShape.waves, kCrThreads = kCombRecvShape.threads();

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

constexpr int kSlotGroup = 8;
constexpr int kCombPieces = 2;   // 1 KB pieces read per slot row per step

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

__global__ __launch_bounds__(kCsThreads) void k_comb_send_rows(Dims D, Ws W, const uint16_t* __restrict__ y,
                                                           const int* __restrict__ row_src,
                                                           uint16_t* __restrict__ comb) {
  __shared__ int svp[kMaxN + 1];
  __shared__ int sbase[kMaxN + 1];
  for (int i = threadIdx.x; i <= D.N; i += kCsThreads) {
    svp[i] = W.vprefix[i];
    sbase[i] = W.base[i];
  }
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int ncomb = D.N * D.TK;
  const int n16 = D.H / 8;
  int lo, hi;
  block_range(svp[D.N], lo, hi);      // valid rows, in region order
  // Wave wv takes rows lo + wv, lo + wv + kCsWaves, ...: the workgroup's
  // waves work on neighbouring rows at any moment.
  for (int g0 = lo + wv; g0 < hi; g0 += kCsWaves * kRowsPerPass) {
    int src = -1, dst = -1;
    const int g = g0 + lane * kCsWaves;
    if (lane < kRowsPerPass && g < hi) {
      const int d = floor_index(svp, D.N + 1, g);
      const int p = sbase[d] + (g - svp[d]);
      if (p < D.rows) {
        const int rs = row_src[p];
        if (rs >= 0 && rs < ncomb) {
          src = p;
          dst = rs;
        }
      }
    }
    for (int r = 0; r < kRowsPerPass; ++r) {
      const int sr = __builtin_amdgcn_readlane(src, r);
      const int dr = __builtin_amdgcn_readlane(dst, r);
      if (sr < 0) continue;
      wave_copy16<kCsUnroll>(reinterpret_cast<v4u*>(comb + (int64_t)dr * D.H),
                      reinterpret_cast<const v4u*>(y + (int64_t)sr * D.H), n16, lane);
    }
  }
  if (D.R) zero_dropped_rows<kCsWaves>(D, W, comb);   // packed regions never overflow
}

// The same copy with the whole workgroup on consecutive rows: the
// workgroup's range of valid rows is one flat range of 16-byte units, and
// thread t copies units t, t + kCcThreads, ... (kCcUnroll per step, loads
// before stores), each to its row's comb position.  This is the access
// pattern of the plain copy; a copy probe with one wave per row ran 4%
// slower than it on the same data.  Measured in one process, alternating
// calls: 5% faster than k_comb_send_rows from combine-heavy size up (prefill 6%,
// Kimi 4%), 7% slower at the decode shape; hence the switch by row count.
// Each unit's load waits for its row_src: issuing the loads first, with
// the row_src reads beside them, made this form 5% slower than the per-row
// one at combine-heavy size.
constexpr int kCcThreads = 1024, kCcUnroll = 16;
__global__ __launch_bounds__(kCcThreads) void k_comb_send(Dims D, Ws W, const uint16_t* __restrict__ y,
                                                               const int* __restrict__ row_src,
                                                               uint16_t* __restrict__ comb) {
  __shared__ int svp[kMaxN + 1];
  __shared__ int sbase[kMaxN + 1];
  for (int i = threadIdx.x; i <= D.N; i += kCcThreads) {
    svp[i] = W.vprefix[i];
    sbase[i] = W.base[i];
  }
  __syncthreads();
  const int ncomb = D.N * D.TK;
  const int n16 = D.H / 8;
  int lo, hi;
  block_range(svp[D.N], lo, hi);      // valid rows, in region order
  const v4u* __restrict__ ys = reinterpret_cast<const v4u*>(y);
  v4u* __restrict__ cs = reinterpret_cast<v4u*>(comb);
  // This thread's unit (valid row g, column c), advanced by kCcThreads units
  // per slot and kCcUnroll * kCcThreads per step without dividing again.
  const int dg1 = kCcThreads / n16, dc1 = kCcThreads % n16;
  const int64_t first = (int64_t)lo * n16 + threadIdx.x;
  int g = (int)(first / n16), c = (int)(first - (int64_t)g * n16);
  while (g < hi) {
    v4u v[kCcUnroll];
    int dst[kCcUnroll];
    int gu = g, cu = c;
#pragma unroll
    for (int u = 0; u < kCcUnroll; ++u) {
      dst[u] = -1;
      if (gu < hi) {
        const int d = floor_index(svp, D.N + 1, gu);
        const int p = sbase[d] + (gu - svp[d]);
        if (p < D.rows) {
          const int rs = row_src[p];
          if (rs >= 0 && rs < ncomb) {
            dst[u] = rs;
            v[u] = ld16(ys + (int64_t)p * n16 + cu);
          }
        }
      }
      gu += dg1;
      cu += dc1;
      if (cu >= n16) {
        cu -= n16;
        ++gu;
      }
    }
    gu = g;
    cu = c;
#pragma unroll
    for (int u = 0; u < kCcUnroll; ++u) {
      if (dst[u] >= 0) st16(cs + (int64_t)dst[u] * n16 + cu, v[u]);
      gu += dg1;
      cu += dc1;
      if (cu >= n16) {
        cu -= n16;
        ++gu;
      }
    }
    g = gu;
    c = cu;
  }
  if (D.R) zero_dropped_rows<kCcThreads / kWave>(D, W, comb);   // packed regions never overflow
}


// Per lane j < k: whether slot j leads its group, i.e. has a row (dest >= 0)
// and no earlier slot of the token has a row on the same rank.
__device__ __forceinline__ bool group_leader(int dest, int k, int lane) {
  bool lead = dest >= 0;
  for (int jj = 0; jj < k; ++jj) {
    const int dj = __builtin_amdgcn_readlane(dest, jj);
    if (jj < lane && dj == dest) lead = false;
  }
  return lead;
}

enum class CombMode { kRecv, kPull, kRecvPartial };

// The weighted sum of one combine, token by token.
//   kRecv: slot rows are rank s's returned rows comb[s*T*k + send_pos];
//   kPull: they are read where the expert wrote them, y_em[base[d] +
//          expert-major index], found from the routing tables;
//   kRecvPartial: only group leaders contribute, with weight 1, their rows
//          comb[s*T*k + send_pos] holding the group's partial sum.
template <CombMode MODE>
__device__ __forceinline__ void combine_tokens(const Dims& D, const Ws& W, const uint16_t* __restrict__ rows,
                                               const int* __restrict__ idx, const int* __restrict__ send_pos,
                                               const float* __restrict__ topk_w, uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  int lo, hi;
  block_range(D.N * D.T, lo, hi);
  for (int tok = lo + wv; tok < hi; tok += kCrWaves) {
    const int s = tok / D.T;
    int row = -1;
    float wt = 0.0f;
    if (MODE == CombMode::kRecvPartial) {
      int dest = -1, sp = -1;
      if (lane < D.k) {
        sp = send_pos[(int64_t)tok * D.k + lane];
        const int e = idx[(int64_t)tok * D.k + lane];
        if (em_row_of(D, W, s, e, sp) >= 0) dest = e / D.L;
      }
      if (group_leader(dest, D.k, lane) && lane < D.k) row = s * D.TK + sp;
      wt = 1.0f;
    } else if (lane < D.k) {
      const int sp = send_pos[(int64_t)tok * D.k + lane];
      wt = topk_w[(int64_t)tok * D.k + lane];
      if (MODE == CombMode::kRecv) {
        if (sp >= 0 && sp < D.TK) row = s * D.TK + sp;
      } else {
        row = em_row_of(D, W, s, idx[(int64_t)tok * D.k + lane], sp);
      }
    }
    uint16_t* orow = out + (int64_t)tok * D.H;
    // Each step reads kCombPieces adjacent 1 KB pieces of every slot row
    // (kCombPieces KB contiguous per row), lane l holding elements
    // [base + c*512 + 8l, +8) of piece c.
    for (int base = 0; base < D.H; base += kWave * 8 * kCombPieces) {
      float acc[kCombPieces][8];
#pragma unroll
      for (int c = 0; c < kCombPieces; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[c][i] = 0.0f;
      for (int j0 = 0; j0 < D.k; j0 += kSlotGroup) {
        v4u v[kSlotGroup][kCombPieces];
        int rr[kSlotGroup];
#pragma unroll
        for (int jj = 0; jj < kSlotGroup; ++jj) {
          const int j = j0 + jj;
          rr[jj] = j < D.k ? __builtin_amdgcn_readlane(row, j) : -1;
#pragma unroll
          for (int c = 0; c < kCombPieces; ++c) {
            const int col = base + c * kWave * 8 + lane * 8;
            v[jj][c] = rr[jj] >= 0 && col < D.H
                           ? ld16(reinterpret_cast<const v4u*>(rows + (int64_t)rr[jj] * D.H + col))
                           : v4u{0, 0, 0, 0};
          }
        }
#pragma unroll
        for (int jj = 0; jj < kSlotGroup; ++jj) {
          const int j = j0 + jj;
          const float wj =
              __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wt), j < D.k ? j : 0));
          if (rr[jj] >= 0) {
#pragma unroll
            for (int c = 0; c < kCombPieces; ++c) acc_row8(acc[c], wj, v[jj][c]);
          }
        }
      }
#pragma unroll
      for (int c = 0; c < kCombPieces; ++c) {
        const int col = base + c * kWave * 8 + lane * 8;
        if (col >= D.H) continue;
        v4u o;
        o[0] = f32_to_bf16_rne(acc[c][0]) | (f32_to_bf16_rne(acc[c][1]) << 16);
        o[1] = f32_to_bf16_rne(acc[c][2]) | (f32_to_bf16_rne(acc[c][3]) << 16);
        o[2] = f32_to_bf16_rne(acc[c][4]) | (f32_to_bf16_rne(acc[c][5]) << 16);
        o[3] = f32_to_bf16_rne(acc[c][6]) | (f32_to_bf16_rne(acc[c][7]) << 16);
        st16(reinterpret_cast<v4u*>(orow + col), o);
      }
    }
  }
}

__global__ __launch_bounds__(kCrThreads) void k_comb_recv_tokens(Dims D, Ws W, const uint16_t* __restrict__ comb,
                                                           const int* __restrict__ send_pos,
                                                           const float* __restrict__ topk_w,
                                                           uint16_t* __restrict__ out) {
  combine_tokens<CombMode::kRecv>(D, W, comb, nullptr, send_pos, topk_w, out);
}

__global__ __launch_bounds__(kCrThreads) void k_comb_pull_tokens(Dims D, Ws W, const uint16_t* __restrict__ y,
                                                           const int* __restrict__ idx,
                                                           const int* __restrict__ send_pos,
                                                           const float* __restrict__ topk_w,
                                                           uint16_t* __restrict__ out) {
  combine_tokens<CombMode::kPull>(D, W, y, idx, send_pos, topk_w, out);
}

__global__ __launch_bounds__(kCrThreads) void k_comb_recv_partial(Dims D, Ws W, const uint16_t* __restrict__ comb,
                                                                   const int* __restrict__ idx,
                                                                   const int* __restrict__ send_pos,
                                                                   uint16_t* __restrict__ out) {
  combine_tokens<CombMode::kRecvPartial>(D, W, comb, idx, send_pos, nullptr, out);
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

// The receive-side sums with the whole workgroup on a chunk of consecutive
// tokens (the plain copy's pattern, as k_comb_send): the chunk's slot rows
// and weights are resolved into LDS, then thread t forms the output's
// 16-byte units t, t + kCoThreads, ..., each from the same 16 bytes of the
// token's k slot rows, summed in slot order exactly as combine_tokens does.
// Measured in one process, alternating calls: 1.5-2% faster than the
// one-wave-per-token form from combine-heavy size up (1655-1661 against
// 1683-1691 us; prefill 3300-3318 against 3360-3391), equal at the decode
// shape, 50% slower at the tiny one; hence the switch by token count.
// One or two workgroups per CU and 4, 8 or 16 units per thread were within
// 1% of each other.
constexpr int kCoThreads = 1024, kCoUnits = 8, kCoTable = 4096;
template <CombMode MODE>
__device__ __forceinline__ void combine_tokens_coop(const Dims& D, const Ws& W, const uint16_t* __restrict__ rows,
                                                    const int* __restrict__ idx, const int* __restrict__ send_pos,
                                                    const float* __restrict__ topk_w, uint16_t* __restrict__ out) {
  __shared__ int t_row[kCoTable];
  __shared__ float t_w[kCoTable];
  const int n16 = D.H / 8, k = D.k;
  int ntok = kCoThreads * kCoUnits / n16;                 // tokens per chunk
  ntok = max(1, min(ntok, kCoTable / k));
  const v4u* __restrict__ rs = reinterpret_cast<const v4u*>(rows);
  v4u* __restrict__ os = reinterpret_cast<v4u*>(out);
  int lo, hi;
  block_range(D.N * D.T, lo, hi);
  for (int t0 = lo; t0 < hi; t0 += ntok) {
    const int nt = min(ntok, hi - t0);
    for (int i = threadIdx.x; i < nt * k; i += kCoThreads) {
      const int64_t slot = (int64_t)t0 * k + i;               // token t0 + i / k, slot i % k
      const int s = (t0 + i / k) / D.T;
      const int sp = send_pos[slot];
      int row;
      if (MODE == CombMode::kRecv) row = sp >= 0 && sp < D.TK ? s * D.TK + sp : -1;
      else row = em_row_of(D, W, s, idx[slot], sp);
      t_row[i] = row;
      t_w[i] = topk_w[slot];
    }
    __syncthreads();
    for (int f = threadIdx.x; f < nt * n16; f += kCoThreads) {
      const int tt = f / n16, c = f - tt * n16;
      const int* tr = t_row + tt * k;
      const float* tw = t_w + tt * k;
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
          if (rr[jj] >= 0) acc_row8(acc, tw[j0 + jj], v[jj]);
      }
      st16(os + (int64_t)(t0 + tt) * n16 + c, pack_bf16x8(acc));
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kCoThreads) void k_comb_recv(Dims D, Ws W, const uint16_t* __restrict__ comb,
                                                               const int* __restrict__ send_pos,
                                                               const float* __restrict__ topk_w,
                                                               uint16_t* __restrict__ out) {
  combine_tokens_coop<CombMode::kRecv>(D, W, comb, nullptr, send_pos, topk_w, out);
}

__global__ __launch_bounds__(kCoThreads) void k_comb_pull(Dims D, Ws W, const uint16_t* __restrict__ y,
                                                               const int* __restrict__ idx,
                                                               const int* __restrict__ send_pos,
                                                               const float* __restrict__ topk_w,
                                                               uint16_t* __restrict__ out) {
  combine_tokens_coop<CombMode::kPull>(D, W, y, idx, send_pos, topk_w, out);
}

// Send-side partial sums, token by token (one wave per token; the form for
// problems below 16384 tokens): for each
// group (a token's slots whose rows sit on one rank) in leader order, its
// members in slot order, acc = fl(acc + fl(w * y)) with no fused
// multiply-add, rounded to bf16 and stored where the leader's row returns
// (comb[s*T*k + send_pos of the leader]).  Each step covers 512 columns
// (lane l holds 8 elements).  With k <= kSlotGroup (every benchmark shape)
// a step loads all k rows at once and forms every group from registers;
// larger k takes the groups one after another, loading each group's
// members kSlotGroup at a time.  Either way every slot row is read once.
constexpr int kSpWaves = kSendPartialShape.waves, kSpThreads = kSendPartialShape.threads();
constexpr int kSendPieces = 2;
__global__ __launch_bounds__(kSpThreads) void k_comb_send_partial_tokens(Dims D, Ws W, const uint16_t* __restrict__ y,
                                                                   const int* __restrict__ idx,
                                                                   const int* __restrict__ send_pos,
                                                                   const float* __restrict__ topk_w,
                                                                   uint16_t* __restrict__ comb) {
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  int lo, hi;
  block_range(D.N * D.T, lo, hi);
  for (int tok = lo + wv; tok < hi; tok += kSpWaves) {
    const int s = tok / D.T;
    int row = -1, dest = -1, sp = -1;
    float wt = 0.0f;
    if (lane < D.k) {
      sp = send_pos[(int64_t)tok * D.k + lane];
      wt = topk_w[(int64_t)tok * D.k + lane];
      const int e = idx[(int64_t)tok * D.k + lane];
      row = em_row_of(D, W, s, e, sp);
      if (row >= 0) dest = e / D.L;
    }
    const bool lead = group_leader(dest, D.k, lane);
    const int orow = lead ? s * D.TK + sp : -1;   // where a leader's group row goes
    auto weight = [&](int j) {
      return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wt), j));
    };
    if (D.k <= kSlotGroup) {
      // kSendPieces adjacent 512-column pieces per step: lane l holds
      // elements [base + c*512 + 8l, +8) of piece c.
      for (int base = 0; base < D.H; base += kWave * 8 * kSendPieces) {
        v4u v[kSlotGroup][kSendPieces];
#pragma unroll
        for (int j = 0; j < kSlotGroup; ++j) {
          const int r = j < D.k ? __builtin_amdgcn_readlane(row, j) : -1;
#pragma unroll
          for (int c = 0; c < kSendPieces; ++c) {
            const int col = base + c * kWave * 8 + lane * 8;
            v[j][c] = r >= 0 && col < D.H ? ld16(reinterpret_cast<const v4u*>(y + (int64_t)r * D.H + col))
                                          : v4u{0, 0, 0, 0};
          }
        }
#pragma unroll
        for (int g = 0; g < kSlotGroup; ++g) {
          const int og = g < D.k ? __builtin_amdgcn_readlane(orow, g) : -1;
          if (og < 0) continue;   // not a leader
          const int dg = __builtin_amdgcn_readlane(dest, g);
          float acc[kSendPieces][8];
#pragma unroll
          for (int c = 0; c < kSendPieces; ++c)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[c][i] = 0.0f;
#pragma unroll
          for (int j = g; j < kSlotGroup; ++j) {
            if (j >= D.k || __builtin_amdgcn_readlane(dest, j) != dg) continue;
            const float wj = weight(j);
#pragma unroll
            for (int c = 0; c < kSendPieces; ++c) acc_row8(acc[c], wj, v[j][c]);
          }
#pragma unroll
          for (int c = 0; c < kSendPieces; ++c) {
            const int col = base + c * kWave * 8 + lane * 8;
            if (col < D.H) st16(reinterpret_cast<v4u*>(comb + (int64_t)og * D.H + col), pack_bf16x8(acc[c]));
          }
        }
      }
    } else {
      for (int g = 0; g < D.k; ++g) {
        const int og = __builtin_amdgcn_readlane(orow, g);
        if (og < 0) continue;
        const int dg = __builtin_amdgcn_readlane(dest, g);
        for (int base = 0; base < D.H; base += kWave * 8) {
          const int col = base + lane * 8;
          float acc[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
          for (int j0 = g; j0 < D.k; j0 += kSlotGroup) {
            v4u v[kSlotGroup];
            int rr[kSlotGroup];
#pragma unroll
            for (int jj = 0; jj < kSlotGroup; ++jj) {
              const int j = j0 + jj;
              rr[jj] = j < D.k && __builtin_amdgcn_readlane(dest, j < D.k ? j : 0) == dg
                           ? __builtin_amdgcn_readlane(row, j < D.k ? j : 0)
                           : -1;
              v[jj] = rr[jj] >= 0 && col < D.H
                          ? ld16(reinterpret_cast<const v4u*>(y + (int64_t)rr[jj] * D.H + col))
                          : v4u{0, 0, 0, 0};
            }
#pragma unroll
            for (int jj = 0; jj < kSlotGroup; ++jj)
              if (rr[jj] >= 0) acc_row8(acc, weight(j0 + jj), v[jj]);
          }
          if (col < D.H) st16(reinterpret_cast<v4u*>(comb + (int64_t)og * D.H + col), pack_bf16x8(acc));
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

constexpr int64_t kCcMinRows = 131072;   // rows from which the cooperative form is used

int launch_comb_send(const Dims& D, const Ws& W, const uint16_t* y, const int* row_src, uint16_t* comb, int cus,
                     hipStream_t st) {
  if (D.N * D.TK == 0) return MOE_OK;
  if ((int64_t)D.rows >= kCcMinRows) {
    const int64_t need = ((int64_t)D.rows * (D.H / 8) + kCcThreads * kCcUnroll - 1) / (kCcThreads * kCcUnroll);
    const int grid = (int)(need < cus ? (need < 1 ? 1 : need) : cus);
    return launch("k_comb_send", k_comb_send, dim3(grid), dim3(kCcThreads), 0, st, D, W, y, row_src, comb);
  }
  const int grid = stream_grid(kCombSendShape, cus, (int64_t)D.rows, kCsWaves);
  return launch("k_comb_send_rows", k_comb_send_rows, dim3(grid), dim3(kCsThreads), 0, st, D, W, y, row_src, comb);
}

constexpr int64_t kCoMinTokens = 16384;   // tokens (N*T) from which the cooperative form is used
static int coop_grid(const Dims& D, int cus) {
  const int64_t need = ((int64_t)D.N * D.T * (D.H / 8) + kCoThreads * kCoUnits - 1) / (kCoThreads * kCoUnits);
  const int64_t cap = cus;   // one workgroup per CU
  return (int)(need < cap ? (need < 1 ? 1 : need) : cap);
}

int launch_comb_recv(const Dims& D, const uint16_t* comb, const int* send_pos, const float* w, uint16_t* out, int cus,
                     hipStream_t st) {
  if (D.N * D.T == 0) return MOE_OK;
  if ((int64_t)D.N * D.T >= kCoMinTokens)
    return launch("k_comb_recv", k_comb_recv, dim3(coop_grid(D, cus)), dim3(kCoThreads), 0, st, D, Ws{}, comb,
                  send_pos, w, out);
  const int grid = stream_grid(kCombRecvShape, cus, (int64_t)D.N * D.T, kCrWaves);
  return launch("k_comb_recv_tokens", k_comb_recv_tokens, dim3(grid), dim3(kCrThreads), 0, st, D, Ws{}, comb, send_pos, w, out);
}

int launch_comb_pull(const Dims& D, const Ws& W, const uint16_t* y, const int* idx, const int* send_pos,
                     const float* w, uint16_t* out, int cus, hipStream_t st) {
  if (D.N * D.T == 0) return MOE_OK;
  if ((int64_t)D.N * D.T >= kCoMinTokens)
    return launch("k_comb_pull", k_comb_pull, dim3(coop_grid(D, cus)), dim3(kCoThreads), 0, st, D, W, y, idx,
                  send_pos, w, out);
  const int grid = stream_grid(kCombRecvShape, cus, (int64_t)D.N * D.T, kCrWaves);
  return launch("k_comb_pull_tokens", k_comb_pull_tokens, dim3(grid), dim3(kCrThreads), 0, st, D, W, y, idx, send_pos, w, out);
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
  const int grid = stream_grid(kSendPartialShape, cus, (int64_t)D.N * D.T, kSpWaves);
  return launch("k_comb_send_partial_tokens", k_comb_send_partial_tokens, dim3(grid), dim3(kSpThreads), 0, st, D, W,
                y, idx, send_pos, w, comb);
}

int launch_comb_recv_partial(const Dims& D, const Ws& W, const uint16_t* comb, const int* idx, const int* send_pos,
                             uint16_t* out, int cus, hipStream_t st) {
  if (D.N * D.T == 0) return MOE_OK;
  const int grid = stream_grid(kCombRecvShape, cus, (int64_t)D.N * D.T, kCrWaves);
  return launch("k_comb_recv_partial", k_comb_recv_partial, dim3(grid), dim3(kCrThreads), 0, st, D, W, comb, idx,
                send_pos, out);
}

}  // namespace moe
