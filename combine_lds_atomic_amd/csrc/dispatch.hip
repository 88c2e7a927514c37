// Dispatch data movement ("Enabling trillion-parameter models on AWS EFA",
// sections "Send and receive buffers", "Dispatch and combine", and
// "Evaluation: dispatch/combine latency" for the block-scaled fp8 payload).
//
//   k_pack_os       one 1024-element pass of one token per wave, workgroups
//                   in (token, pass) order: final slot positions, block-128
//                   amax with DPP, fp8 quantisation, and k 16-byte row
//                   stores straight into the destination ranks' receive
//                   regions (the "remote write"), with the block scales
//   k_unpack_index  one thread per expert-major row: the (expert, source)
//                   segment it belongs to, found from the exchanged counts
//                   alone; writes row_src and the row map
//   k_unpack_os     one 16-byte unit per thread: each expert-major row's fp8
//                   payload, then its scales, copied out of the
//                   source-major receive region
//   k_pack_direct_os  k_pack_os storing each row at its expert-major row
//                   instead (peers mapped into each other's memory push
//                   straight into the grouped-GEMM layout; on one GPU every
//                   rank is such a peer), so neither the receive regions
//                   nor the unpack are needed
//   k_dispatch_ll, k_dispatch_ll_direct  the send half (or the direct
//                   dispatch) in one launch, for decode-sized batches
#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>

#include "route_dev.h"


namespace moe {

constexpr int kPackCols = kWave * 16;         // elements one wave covers per pass (16 per lane)
constexpr int kOsWaves = kOsThreads / kWave;  // one-shot pack work items per workgroup (direct form)
// k_pack_os: one work item (wave) per workgroup, 1-3.5% faster than four
// from the decode shape up (2% slower at the tiny shape); the direct form's
// pack, which also writes row_src, was 1-4% slower with one and keeps four.
constexpr int kPackWaves = 1;
constexpr int kLlWaves = kThreads / kWave;    // single-launch packer waves per workgroup
constexpr int kPackPasses = 4;                // passes whose loads a single-launch packer issues together

// Four quotients x[i] / scale (IEEE division) packed as e4m3fn bytes,
// little end first.  v_cvt_pk_fp8_f32 converts two floats to OCP e4m3fn
// (round to nearest even, saturating) per instruction on gfx950; the
// exhaustive sweep test checks its bytes against the oracle's encoder on
// every bfloat16 pair x <= amax.
__device__ __forceinline__ uint32_t quant4(const float* v, float scale) {
  float q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = v[i] / scale;
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w, true);
  return (uint32_t)w;
}

// This lane's 16 elements of each pass of the chunk starting at column c0
// (zero beyond h1).
__device__ __forceinline__ void load_chunk(const uint16_t* __restrict__ xr, int c0, int h1, int lane,
                                           v4u (&a)[kPackPasses], v4u (&b)[kPackPasses]) {
#pragma unroll
  for (int p = 0; p < kPackPasses; ++p) {
    const int col = c0 + p * kPackCols + lane * 16;
    const bool act = col < h1;
    a[p] = act ? ld16(reinterpret_cast<const v4u*>(xr + col)) : v4u{0, 0, 0, 0};
    b[p] = act ? ld16(reinterpret_cast<const v4u*>(xr + col + 8)) : v4u{0, 0, 0, 0};
  }
}

// This lane's 16 elements as e4m3fn bytes with the scale of their
// 128-element block: amax over the block (with the 7 neighbouring lanes),
// scale = amax / 448, q = x / scale.  An all-zero block has scale 0 and zero
// bytes.  All 64 lanes must call it (cross-lane amax).
__device__ __forceinline__ v4u quant16(const v4u& a, const v4u& b, float& sc) {
  float v[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(a[i]);
    v[2 * i + 1] = bf16_hi(a[i]);
    v[8 + 2 * i] = bf16_lo(b[i]);
    v[8 + 2 * i + 1] = bf16_hi(b[i]);
  }
  int am = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) am = max(am, (int)(__float_as_uint(v[i]) & 0x7FFFFFFFu));
  am = max8_lanes(am);                     // amax of the 128-element block
  const float amax = __uint_as_float((uint32_t)am);
  const float scale = amax / 448.0f;       // IEEE division, round to nearest even
  v4u q = {0, 0, 0, 0};
  if (amax != 0.0f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = quant4(v + 4 * i, scale);
  }
  sc = amax != 0.0f ? scale : 0.0f;
  return q;
}

// One pass of a single-launch pack work item: this lane's 16 elements at
// column col, quantised and stored to the k rows; the block's scale goes to
// the wave's LDS row (stored to the rows once per item, 4 bytes per lane).
__device__ __forceinline__ void pack_pass(const Dims& D, const v4u& a, const v4u& b, int col, bool act, int row,
                                          int lane, uint8_t* __restrict__ recv_q, float* ssw) {
  float sc;
  const v4u q = quant16(a, b, sc);
  if (act && (lane & 7) == 0) ssw[col / kScaleBlock] = sc;
  for (int j = 0; j < D.k; ++j) {
    const int rj = __builtin_amdgcn_readlane(row, j);
    if (rj >= 0 && act) st16(reinterpret_cast<v4u*>(recv_q + (int64_t)rj * D.H + col), q);
  }
}

// The scales of columns [h0, h1) from the wave's LDS row to the k rows.
__device__ __forceinline__ void pack_scales(const Dims& D, int h0, int h1, int row, int lane,
                                            float* __restrict__ recv_s, const float* ssw) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  for (int bi = h0 / kScaleBlock + lane; bi < h1 / kScaleBlock; bi += kWave) {
    const float sc = ssw[bi];
    for (int j = 0; j < D.k; ++j) {
      const int rj = __builtin_amdgcn_readlane(row, j);
      if (rj >= 0) recv_s[(int64_t)rj * D.NB + bi] = sc;
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// Work item = (token, slice): slice sl of a token covers columns [h0, h1),
// passes [sl*pps, (sl+1)*pps) of 1024 elements, pps = ceil(passes / slices).
// Item i of a token is slice (i + rot) % slices: rotating the slices by the
// round a packer wave is in (rot) hands each wave the short last slice in
// turn rather than always or never.
__device__ __forceinline__ void item_cols(const Dims& D, int item, int rot, int& tok, int& sl, int& h0, int& h1) {
  const int passes = (D.H + kPackCols - 1) / kPackCols;
  const int pps = (passes + D.slices - 1) / D.slices;
  tok = item / D.slices;
  sl = (item - tok * D.slices + rot) % D.slices;
  h0 = sl * pps * kPackCols;
  h1 = min(D.H, (sl + 1) * pps * kPackCols);
}

// Pack work item `item` with the calling wave, whose rows are already
// resolved (lane j < k: receive row of slot j, -1 for none).  LOADED: pa and
// pb hold the item's first chunk.
template <bool LOADED>
__device__ __forceinline__ void pack_item(const Dims& D, int item, int rot, int row, const uint16_t* __restrict__ x,
                                          uint8_t* __restrict__ recv_q, float* __restrict__ recv_s, float* ssw,
                                          const v4u* pa = nullptr, const v4u* pb = nullptr) {
  const int lane = threadIdx.x & (kWave - 1);
  int tok, sl, h0, h1;
  item_cols(D, item, rot, tok, sl, h0, h1);
  const uint16_t* xr = x + (int64_t)tok * D.H;
  int c0 = h0;
  if (LOADED) {   // the first chunk, peeled so its registers die here
#pragma unroll
    for (int p = 0; p < kPackPasses; ++p) {
      if (c0 + p * kPackCols >= h1) break;
      const int col = c0 + p * kPackCols + lane * 16;
      pack_pass(D, pa[p], pb[p], col, col < h1, row, lane, recv_q, ssw);
    }
    c0 += kPackCols * kPackPasses;
  }
  for (; c0 < h1; c0 += kPackCols * kPackPasses) {
    v4u a[kPackPasses], b[kPackPasses];
    load_chunk(xr, c0, h1, lane, a, b);   // the loads of several passes before any math
#pragma unroll
    for (int p = 0; p < kPackPasses; ++p) {
      if (c0 + p * kPackCols >= h1) break;
      const int col = c0 + p * kPackCols + lane * 16;   // this lane's 16 elements
      pack_pass(D, a[p], b[p], col, col < h1, row, lane, recv_q, ssw);   // whole 8-lane groups drop out together
    }
  }
  pack_scales(D, h0, h1, row, lane, recv_s, ssw);
}


// Pack work item = (token, 1024-element pass), one per wave: lane l holds
// elements [16l, 16l + 16) of the pass, a 128-element scale block spanning 8
// lanes.  pack_load reads the lane's 16 bf16 values (zero beyond H) and
// returns whether it has any.
__device__ __forceinline__ bool pack_load(const Dims& D, const uint16_t* __restrict__ x, int64_t tok, int col,
                                          v4u& a, v4u& b) {
  a = v4u{0, 0, 0, 0};
  b = v4u{0, 0, 0, 0};
  if (col >= D.H) return false;
  const uint16_t* xr = x + tok * D.H + col;
  a = ld16(reinterpret_cast<const v4u*>(xr));
  b = ld16(reinterpret_cast<const v4u*>(xr + 8));
  return true;
}

// Quantise the lane's 16 elements (quant16) and store them, and from the
// block's first lane its scale, to the row of every slot j < k (lane j of
// `row` holds slot j's row, -1 for none).  All 64 lanes must call it.
__device__ __forceinline__ void pack_store(const Dims& D, const v4u& a, const v4u& b, int col, bool act, int row,
                                           int lane, uint8_t* __restrict__ q_out, float* __restrict__ s_out) {
  float sc;
  const v4u q = quant16(a, b, sc);
  for (int j = 0; j < D.k; ++j) {
    const int rj = __builtin_amdgcn_readlane(row, j);
    if (rj < 0 || !act) continue;
    st16(reinterpret_cast<v4u*>(q_out + (int64_t)rj * D.H + col), q);
    if ((lane & 7) == 0) s_out[(int64_t)rj * D.NB + col / kScaleBlock] = sc;
  }
}


// The row slot i (of rank s's T*k) is packed to, -1 for none.  DIRECT =
// false: its source-major receive row; DIRECT = true: its expert-major row,
// by the same index and rule the unpack uses (it exists if both it and its
// source-major row fit; row_src -1 when only the source-major one does not).
// With several routing chunks per rank the count kernel left the rank
// inside the chunk, and the chunk's base for the expert completes it; then
// the position (or -1 for a dropped slot) is written here, as row_src is in
// the direct form, when `write` is set.
template <bool DIRECT>
__device__ __forceinline__ int pack_slot_row(const Dims& D, const Ws& W, const int* __restrict__ idx,
                                             int* __restrict__ send_pos, int* __restrict__ row_src, int s, int i,
                                             bool write) {
  const int64_t slot = (int64_t)s * D.TK + i;
  const int e = idx[slot];
  if (e < 0 || e >= D.E) {
    if (D.B > 1 && write) send_pos[slot] = -1;   // (the count kernel marks it when it writes positions itself)
    return -1;
  }
  int sp;
  if (D.B > 1) {
    sp = W.local[slot] + W.blk[((int64_t)s * D.B + i / D.C) * D.E + e];
    if (write) send_pos[slot] = sp;
  } else {
    sp = send_pos[slot];
  }
  const int d = e / D.L;
  const int* so = W.send_off + s * (D.E + 1);
  const int bd = W.base[d];
  const int r = region_row(D, s, sp - so[d * D.L], W.recv_off[d * (D.N + 1) + s]);   // source-major
  const bool fits = (D.R == 0 || r < D.R) && r >= 0 && bd + r < D.rows;
  if (!DIRECT) return fits ? bd + r : -1;
  const int ie = W.exp_off[d * (D.L + 1) + (e - d * D.L)] + W.src_in_exp[s * D.E + e] + (sp - so[e]);
  const int pe = bd + ie;
  if ((D.R == 0 || ie < D.R) && ie >= 0 && pe < D.rows) {
    if (write) row_src[pe] = fits ? s * D.TK + sp : -1;
    return fits ? pe : -1;
  }
  return -1;
}

// ------------------------------------------------------------------ single launch
//
// The whole send half of dispatch in one launch, without a host round trip
// or a kernel boundary between the count exchange and the payload stores
// (AWS China blog "750B MoE model migration from a self-built RoCE cluster to
// AWS EFA", section 4.4, "DeepEP low-latency mode": one kernel per dispatch,
// no CPU in the loop, capturable in a graph).  The workgroup index gives
// the role:
//   b <  N         count rank b's slots (count_chunk) and publish them;
//   N <= b < 2N    the column of destination rank d = b - N: from the
//                  counts and send offsets of every source bound for d (one
//                  round of loads), what a packer needs for d's rows, then
//                  d's share of the tables dispatch_recv and the combine read;
//   b == 2N        finish: once every column is out, the scans across
//                  destinations;
//   b >  2N        pack: load tokens while the layout is being computed,
//                  then quantise and store the rows once the positions are
//                  known.  Packers are as many as fit beside the layout
//                  workgroups and take the work items interleaved.
// Splitting the cross-rank work over destinations keeps it to one round of
// tagged loads per column workgroup; one workgroup doing it all needed a
// round per few sources (16 rounds at N = 64), which made the routing alone
// take twice as long as the two routing kernels of moe_dispatch_send.
// A workgroup only ever waits for values that workgroups with smaller
// indices produce.  The dispatcher hands each XCD its workgroups in index
// order, so the 2N + 1 layout workgroups are the first on their XCDs and are
// resident before any packer that could wait for them.  Every wait is also
// bounded (kSpinLimit): were that order ever not kept, a wait would end with
// MOE_FLAG_TIMEOUT instead of hanging.  (Taking a ticket from one global
// counter would not need the order, but its one atomic per workgroup on a
// single address serialises: about 8 ns each, 15 us for a decode-sized
// grid.)
//
// Signalling departs from the fence-then-signal pattern of the Perseus
// write-up (section 3.2, decoupled signaling: one fence per group of puts,
// then the group's signals): on a multi-XCD MI355X a release fence writes
// back the whole L2 of the XCD, so instead every exchanged value carries the
// call's tag in the same 8-byte atomic store and is its own completion
// signal; no fence is issued at all.  A packer workgroup first waits for
// one tagged word (a column's completion, or with early rows its rank's
// count), then reads its values (normally already there, otherwise it keeps
// polling those).

// v[u] = value at addr(u) for u < n (n <= M), once all carry `tag`; false
// after kSpinLimit polls.
template <int M, class Addr>
__device__ __forceinline__ bool tag_gather(Addr addr, int n, uint32_t tag, int (&v)[M]) {
  uint64_t u[M];
#pragma unroll
  for (int i = 0; i < M; ++i) u[i] = i < n ? tag_load(addr(i)) : ((uint64_t)tag << 32);
  for (int it = 0;; ++it) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < M; ++i) ok = ok && tag_ok(u[i], tag);
    if (ok) break;
    if (it == kSpinLimit) return false;
    __builtin_amdgcn_s_sleep(2);
#pragma unroll
    for (int i = 0; i < M; ++i)
      if (!tag_ok(u[i], tag)) u[i] = tag_load(addr(i));
  }
#pragma unroll
  for (int i = 0; i < M; ++i) v[i] = (int)(uint32_t)u[i];
  return true;
}

// Three tagged values at once (p2 may be NULL: v2 is left as it is).
__device__ __forceinline__ bool tag_wait3(const uint64_t* p0, const uint64_t* p1, const uint64_t* p2, uint32_t tag,
                                          int& v0, int& v1, int& v2) {
  const uint64_t ok2 = (uint64_t)tag << 32;
  uint64_t u0 = tag_load(p0), u1 = tag_load(p1), u2 = p2 ? tag_load(p2) : ok2;
  for (int it = 0; !(tag_ok(u0, tag) && tag_ok(u1, tag) && tag_ok(u2, tag)); ++it) {
    if (it == kSpinLimit) return false;
    __builtin_amdgcn_s_sleep(2);
    if (!tag_ok(u0, tag)) u0 = tag_load(p0);
    if (!tag_ok(u1, tag)) u1 = tag_load(p1);
    if (!tag_ok(u2, tag)) u2 = tag_load(p2);
  }
  v0 = (int)(uint32_t)u0;
  v1 = (int)(uint32_t)u1;
  if (p2) v2 = (int)(uint32_t)u2;
  return true;
}

// Tagged values a column thread polls at once (register budget: every role
// of the launch shares one register allocation).
constexpr int kColBatch = 4;

// LDS ints of the column role: counts, then the senders' offsets per
// expert, [N][L]; their column scans [N][L]; the senders' offsets to ranks
// d and d+1, [N] each; the expert totals and their scan [L+1]; 3 totals.
inline size_t column_ll_lds_bytes(int N, int E) { return sizeof(int) * ((size_t)2 * E + 2 * N + E / N + 4); }

// The column role for destination rank d.  From the tagged counts of d's
// experts and the senders' offsets to d and d+1 alone it publishes, for
// every source s, what a packer adds to a sender position to get the row:
//   send form:   trel[s][d] = N*C + recv_off[d][s] - C - send_off[s][d*L]
//                (recv_off: rows beyond the C early ones from sources
//                before s) and tbase[d] = base[d];
//   direct form: temr[s][e] = base[d] + exp_off[d][l] + src_in_exp[s][e] -
//                send_off[s][e] for e = d*L + l, and with fixed regions
//                tlim[s][d], the sender positions below which the
//                source-major row fits region d: send_off[s][d*L] + C +
//                max(0, R - N*C - recv_off[d][s]);
// packed regions: base[d] = sum over s of send_off[s][d*L] (the slots all
// sources send to ranks before d).  Then d's part of the workspace tables
// (recv_off[d], recv_total[d], base[d], src_in_exp and exp_off of d's
// experts; exp_out too in the direct form) and tcold[d] = rows d receives,
// published once the packers' values are (in the send form before the
// tables, which they do not need).
template <bool DIRECT>
__device__ void column_ll(const Dims& D, const Ws& W, uint32_t tag, int d, int* sm, int* wsum,
                          int* __restrict__ exp_out) {
  const int N = D.N, L = D.L, E = D.E, NL = N * L, tid = threadIdx.x;
  int* c = sm;               // [N][L] counts of rank d's experts, then send_off[s][e]
  int* sie = sm + NL;        // [N][L] src_in_exp[s][e]
  int* so0 = sm + 2 * NL;    // [N] send_off[s][d*L]
  int* so1 = so0 + N;        // [N] send_off[s][(d+1)*L]
  int* eo = so1 + N;         // [L+1] totals, then exp_off[d][l]
  int* tot = eo + L + 1;     // [3] rows beyond the early ones, rows, region base
  // (1) The counts and the senders' offsets, kColBatch values per thread at
  // a time: indices below NL are counts, then send_off[s][d*L], then
  // send_off[s][(d+1)*L].
  bool ok = true;
  const int nv = NL + 2 * N;
  for (int i0 = tid * kColBatch; i0 < nv && ok; i0 += kThreads * kColBatch) {
    const int n = min(kColBatch, nv - i0);
    int v[kColBatch] = {};
    ok = tag_gather<kColBatch>(
        [&](int u) {
          const int i = i0 + u;
          if (i < NL) return W.tcnt + (int64_t)(i / L) * E + d * L + i % L;
          const int j = i - NL, hi = j >= N;
          return W.toff + (int64_t)(j - hi * N) * (N + 1) + d + hi;
        },
        n, tag, v);
    for (int u = 0; u < n; ++u) {
      const int i = i0 + u;
      if (i < NL) c[i] = v[u];
      else so0[i - NL] = v[u];   // so0 and so1 are adjacent
    }
  }
  const bool fail = __syncthreads_or(!ok);
  // (2) Per expert: the column scan over sources.
  for (int l = tid; l < L && !fail; l += kThreads) {
    int acc = 0;
    for (int s = 0; s < N; ++s) {
      sie[s * L + l] = acc;
      acc += c[s * L + l];
    }
    eo[l] = acc;
    W.src_in_exp[N * E + d * L + l] = acc;
  }
  // (3) Per source (one per thread, N <= 256): rows to d, those beyond the
  // early ones and their scan over sources (recv_off[d][s]); the region base.
  const int s = tid;
  const int rows = s < N && !fail ? so1[s] - so0[s] : 0;
  const int beyond = max(rows - D.Ce, 0);
  int rover, rt, bd, ro = 0;
  if (N <= kWave) {   // every source in wave 0: scans without barriers, totals to LDS
    if (tid < kWave) {
      ro = wave_scan(beyond, &rover);
      wave_scan(rows, &rt);
      wave_scan(s < N && !fail ? so0[s] : 0, &bd);
      if (tid == 0) {
        tot[0] = rover;
        tot[1] = rt;
        tot[2] = bd;
      }
    }
    __syncthreads();
    rover = tot[0];
    rt = tot[1];
    bd = tot[2];
  } else {
    ro = block_scan<kThreads>(beyond, wsum, &rover);
    block_scan<kThreads>(rows, wsum, &rt);
    block_scan<kThreads>(s < N && !fail ? so0[s] : 0, wsum, &bd);
  }
  if (D.R) bd = d * D.R;
  if (s < N && !fail) {
    W.recv_off[d * (N + 1) + s] = ro;
    if (DIRECT) {
      if (D.R) tag_put(W.tlim + (int64_t)s * N + d, tag, so0[s] + D.Ce + max(0, D.R - N * D.Ce - ro));
      int acc = so0[s];   // send_off[s][e] over rank d's experts
      for (int l = 0; l < L; ++l) {
        const int t = c[s * L + l];
        c[s * L + l] = acc;
        acc += t;
      }
    } else {
      tag_put(W.trel + (int64_t)s * N + d, tag, N * D.Ce + ro - D.Ce - so0[s]);
    }
  }
  if (!DIRECT) {
    // The packers of the send form need nothing more: publish now, the
    // rest of the tables follow.
    __syncthreads();
    if (tid == 0 && !fail) {
      tag_put(W.tbase + d, tag, bd);
      tag_put(W.tcold + d * kReadyStride, tag, rt);
    }
  }
  // (4) exp_off[d][l]: exclusive scan of the totals, four per thread (L <= 1024).
  {
    const int l0 = min(L, tid * 4), l1 = min(L, l0 + 4);
    int v = 0;
    for (int l = l0; l < l1; ++l) v += eo[l];
    int all;
    int x = block_scan<kThreads>(v, wsum, &all);
    for (int l = l0; l < l1; ++l) {
      const int t = eo[l];
      eo[l] = x;
      x += t;
    }
    if (tid == 0) eo[L] = all;
  }
  __syncthreads();
  if (!fail) {
    if (DIRECT)
      for (int i = tid; i < NL; i += kThreads)
        tag_put(W.temr + (int64_t)(i / L) * E + d * L + i % L, tag, bd + eo[i % L] + sie[i] - c[i]);
    for (int i = tid; i < NL; i += kThreads) W.src_in_exp[(int64_t)(i / L) * E + d * L + i % L] = sie[i];
    for (int l = tid; l <= L; l += kThreads) {
      W.exp_off[d * (L + 1) + l] = eo[l];
      if (DIRECT) exp_out[d * (L + 1) + l] = eo[l];
    }
    if (tid == 0) {
      W.base[d] = bd;
      W.recv_total[d] = rt;
      W.recv_off[d * (N + 1) + N] = rover;
      uint32_t fl = 0;
      if (D.R && (rt > D.R || D.N * D.Ce + rover > D.R)) fl |= MOE_FLAG_OVERFLOW;
      if ((int64_t)rt > D.bound) fl |= MOE_FLAG_BOUND;
      if (fl) atomicOr(W.err, fl);
    }
  }
  __syncthreads();
  if (fail) {
    if (tid == 0) atomicOr(W.err, MOE_FLAG_TIMEOUT);
  } else if (DIRECT && tid == 0) {
    tag_put(W.tcold + d * kReadyStride, tag, rt);
  }
}

// The finish role: waits for every column (one tagged word each, carrying
// the rows the destination receives), then the scans across destinations:
// rows written per region (vprefix) and base[N].
__device__ void finish_ll(const Dims& D, const Ws& W, uint32_t tag, int* wsum) {
  const int N = D.N, tid = threadIdx.x;
  int rt = 0;
  const bool ok = tid >= N || tag_wait(W.tcold + tid * kReadyStride, tag, &rt);
  if (__syncthreads_or(!ok)) {
    if (tid == 0) atomicOr(W.err, MOE_FLAG_TIMEOUT);
    return;
  }
  int all, vall;
  block_scan<kThreads>(rt, wsum, &all);
  const int vb = block_scan<kThreads>(D.R ? min(rt, D.R) : rt, wsum, &vall);
  if (tid < N) W.vprefix[tid] = vb;
  if (tid == 0) {
    W.base[N] = D.R ? N * D.R : all;
    W.vprefix[N] = vall;
  }
}

// The single launch.  DIRECT = false: rows go to the receive regions
// (recv_q, recv_s).  DIRECT = true: the packers store every row at its
// expert-major row (recv_q, recv_s = x_q, x_s) and write row_src, and the
// columns copy exp_off out.  Without tokens (x == nullptr) the direct form
// still runs its packers, for row_src; the send form runs none.
template <bool DIRECT>
__device__ __forceinline__ void dispatch_ll(const Dims& D, const Ws& W, const uint16_t* __restrict__ x,
                                            const int* __restrict__ idx, int* __restrict__ send_pos,
                                            uint8_t* __restrict__ recv_q, float* __restrict__ recv_s,
                                            int* __restrict__ row_src, int* __restrict__ exp_out, int npack) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int wsum[kWavesPerBlock + 1];
  __shared__ int sh_fail;
  __shared__ uint32_t sh_epoch;
  const int wg = blockIdx.x;
  const int grp = wg % kCtlGroups;
  uint32_t* gline = W.ctl + grp * kCtlStride;   // [0] finished workgroups, [1] call number
  if (threadIdx.x == 0) {
    sh_epoch = __hip_atomic_load(gline + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh_fail = 0;
  }
  __syncthreads();
  const uint32_t tag = epoch_tag(sh_epoch);

  if (wg < D.N) {
    count_chunk(D, W, idx, send_pos, wg, 0, smem, wsum, tag);
    __syncthreads();
    if (threadIdx.x == 0) tag_put(W.tcdone + wg * kReadyStride, tag, 1);
  } else if (wg < 2 * D.N) {
    column_ll<DIRECT>(D, W, tag, wg - D.N, reinterpret_cast<int*>(smem), wsum, exp_out);
  } else if (wg == 2 * D.N) {
    finish_ll(D, W, tag, wsum);
  } else {
    // Packers: work items (token, slice) interleaved over the workgroups
    // (wave w of packer p takes items 4p + w, then every 4*npack-th), so
    // the packers resident at any moment cover a compact band of tokens, as
    // k_pack_os's grid does.  Round r of the waves (items [r*stride,
    // (r+1)*stride)) rotates the slices of its tokens by r when whole
    // tokens make up a round, so that a wave's items are not all long or
    // all short slices when the slices are unequal (7 passes in slices of
    // 4 and 3 at H = 7168).
    const int p = wg - 2 * D.N - 1;
    const int items = D.N * D.T * D.slices;
    const int stride = npack * kLlWaves;
    const int rstride = stride % D.slices == 0 ? stride : items;   // items per rotation step
    bool fail = false;
    // The workgroup's wait for the layout: one column's word (p % N: the
    // columns finish together, and the values a packer reads are each
    // tagged, so this wait only keeps 4 waves per workgroup from polling
    // them while the layout is computed).  With early rows most rows need
    // only their own source rank's count: the count workgroup of the rank
    // of the first item.
    auto gate = [&] {
      if (threadIdx.x == 0 && p * kLlWaves < items) {
        int one;
        const bool ok = DIRECT || D.Ce == 0
                            ? tag_wait(W.tcold + (p % D.N) * kReadyStride, tag, &one)
                            : tag_wait(W.tcdone + (p * kLlWaves / D.slices / D.T) * kReadyStride, tag, &one);
        if (!ok) {
          sh_fail = 1;
          atomicOr(W.err, MOE_FLAG_TIMEOUT);
        }
      }
      __syncthreads();
      fail = sh_fail != 0;
    };
    const int lane = threadIdx.x & (kWave - 1);
    // Expert of slot j (lane j < k) of work item `item`.
    auto expert = [&](int item) { return lane < D.k ? idx[(int64_t)(item / D.slices) * D.k + lane] : -1; };
    // Rows of slot j (lane j < k) of work item `item`, expert e, from the
    // tagged positions and offsets.
    auto resolve = [&](int item, int e) {
      const int tok = item / D.slices;
      const int s = tok / D.T;
      int row = -1;
      bool ok = true;
      if (!fail && lane < D.k) {
        const int64_t slot = (int64_t)tok * D.k + lane;
        if (DIRECT && e >= 0 && e < D.E) {
          // The column workgroup's values: the expert-major row offset and,
          // with fixed regions, the limit below which the source-major row
          // fits (the unpack's rule: the row exists if it fits region d,
          // its payload only if the source-major row fits too).
          const int d = e / D.L;
          int sp = 0, off = 0, lim = 0;
          ok = tag_wait3(W.tpos + slot, W.temr + (int64_t)s * D.E + e, D.R ? W.tlim + (int64_t)s * D.N + d : nullptr,
                         tag, sp, off, lim);
          const int pe = off + sp, ie = pe - (D.R ? d * D.R : 0);
          if (ok && (D.R == 0 || ie < D.R) && ie >= 0 && pe < D.rows) {
            const bool fits = D.R == 0 || sp < lim;
            if (item % D.slices == 0) row_src[pe] = fits ? s * D.TK + sp : -1;
            if (fits) row = pe;
          }
        } else if (e >= 0 && e < D.E) {
          const int d = e / D.L;
          int sp = 0, rel = 0, bd = D.R ? d * D.R : 0, r = -1;
          if (D.Ce == 0) {
            ok = tag_wait3(W.tpos + slot, W.trel + (int64_t)s * D.N + d, D.R ? nullptr : W.tbase + d, tag, sp, rel,
                           bd);
            r = rel + sp;
          } else {   // fixed regions: an early row needs only the sender's own count
            int so = 0;
            ok = tag_wait3(W.tpos + slot, W.toff + (int64_t)s * (D.N + 1) + d, nullptr, tag, sp, so, bd);
            const int u = sp - so;
            if (ok && u < D.Ce) {
              r = s * D.Ce + u;
            } else if (ok) {
              ok = tag_wait(W.trel + (int64_t)s * D.N + d, tag, &rel);
              r = rel + sp;
            }
          }
          const int pr = bd + r;
          if (ok && (D.R == 0 || r < D.R) && r >= 0 && pr < D.rows) row = pr;
        }
      }
      if (__any(!ok)) {   // stop waiting for anything else in this wave
        fail = true;
        if (lane == 0) atomicOr(W.err, MOE_FLAG_TIMEOUT);
      }
      return row;
    };
    // Each wave loads its first item's first chunk, then the workgroup waits
    // for the layout, then packs.
    const int wv = threadIdx.x / kWave;
    float* ssw = reinterpret_cast<float*>(smem) + wv * D.NB;
    int item = p * kLlWaves + wv;
    if (DIRECT && x == nullptr) {   // layout only: positions and row_src
      gate();
      for (; item < items; item += stride) resolve(item, expert(item));
      item = items;
    }
    const bool has = item < items;
    v4u a[kPackPasses], b[kPackPasses];
    int e1 = -1;
    if (has) {
      int tok, sl, h0, h1;
      item_cols(D, item, item / rstride, tok, sl, h0, h1);
      load_chunk(x + (int64_t)tok * D.H, h0, h1, lane, a, b);
      e1 = expert(item);
    }
    if (!DIRECT || x != nullptr) gate();
    if (has) {
      pack_item<true>(D, item, item / rstride, resolve(item, e1), x, recv_q, recv_s, ssw, a, b);
      item += stride;
    }
    for (; item < items; item += stride)
      pack_item<false>(D, item, item / rstride, resolve(item, expert(item)), x, recv_q, recv_s, ssw);
  }
  // The last workgroup of each group to finish clears the group's counter and
  // counts the group as done; the last group to finish advances every
  // group's call number for the next launch on this workspace (all
  // workgroups of this launch have read theirs by then).
  __syncthreads();
  if (threadIdx.x == 0) {
    const int G = gridDim.x;
    const uint32_t members = (uint32_t)((G - grp + kCtlGroups - 1) / kCtlGroups);
    const uint32_t groups = (uint32_t)min(G, kCtlGroups);
    if (__hip_atomic_fetch_add(gline, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == members - 1) {
      __hip_atomic_store(gline, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      uint32_t* all = W.ctl + kCtlGroups * kCtlStride;
      if (__hip_atomic_fetch_add(all, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == groups - 1) {
        __hip_atomic_store(all, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int g = 0; g < kCtlGroups; ++g)
          __hip_atomic_store(W.ctl + g * kCtlStride + 1, sh_epoch + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_dispatch_ll(Dims D, Ws W, const uint16_t* __restrict__ x,
                                                          const int* __restrict__ idx, int* __restrict__ send_pos,
                                                          uint8_t* __restrict__ recv_q, float* __restrict__ recv_s, int npack) {
  dispatch_ll<false>(D, W, x, idx, send_pos, recv_q, recv_s, nullptr, nullptr, npack);
}

__global__ __launch_bounds__(kThreads) void k_dispatch_ll_direct(Dims D, Ws W, const uint16_t* __restrict__ x,
                                                                 const int* __restrict__ idx,
                                                                 int* __restrict__ send_pos, uint8_t* __restrict__ x_q,
                                                                 float* __restrict__ x_s, int* __restrict__ row_src,
                                                                 int* __restrict__ exp_off, int npack) {
  dispatch_ll<true>(D, W, x, idx, send_pos, x_q, x_s, row_src, exp_off, npack);
}

// Staging of one region's routing tables in LDS (the unpack kernel): the searches
// that map an expert-major row to its segment then read no global memory.
constexpr int kStageInts = 2 * kMaxE + (kMaxE + kMaxN) + (kMaxE + 1) + (kMaxN + 1);

// One region's routing tables staged in LDS, for the row searches.  The
// pointers carry the LDS address space: as plain pointers, merged with the
// global ones of the other branch of unpack_row, they made every staged
// read a flat access (and put a pointer through scratch).
using lds_int = __attribute__((address_space(3))) int;
struct UnpackStage {
  int d0;                                // the region (-1: none staged)
  lds_int *sie, *so, *eo, *ro;           // src_in_exp / send_off columns, exp_off, recv_off of region d0
};

// Region d0 of the workgroup's first row lo (normally its only one):
//   sie[s][l] = src_in_exp[s][d0*L + l], s in [0, N];
//   so[s][l'] = send_off[s][d0*L + l'], l' in [0, L];
//   eo[l']    = exp_off[d0][l'];  ro[s] = recv_off[d0][s].
// Ends with a workgroup barrier.
template <int THREADS>
__device__ __forceinline__ UnpackStage unpack_stage(const Dims& D, const Ws& W, const int* svp, int* stage, int lo,
                                                    int hi) {
  const int N = D.N, E = D.E, L = D.L;
  UnpackStage S;
  S.sie = (lds_int*)stage;
  S.so = S.sie + (N + 1) * L;
  S.eo = S.so + N * (L + 1);
  S.ro = S.eo + (L + 1);
  S.d0 = lo < hi ? floor_index(svp, N + 1, lo) : -1;
  if (S.d0 >= 0) {
    const int d0 = S.d0;
    for (int i = threadIdx.x; i < (N + 1) * L; i += THREADS) S.sie[i] = W.src_in_exp[(i / L) * E + d0 * L + i % L];
    for (int i = threadIdx.x; i < N * (L + 1); i += THREADS)
      S.so[i] = W.send_off[(i / (L + 1)) * (E + 1) + d0 * L + i % (L + 1)];
    for (int i = threadIdx.x; i <= L; i += THREADS) S.eo[i] = W.exp_off[d0 * (L + 1) + i];
    for (int i = threadIdx.x; i <= N; i += THREADS) S.ro[i] = W.recv_off[d0 * (N + 1) + i];
  }
  __syncthreads();
  return S;
}

// Valid row g (region order): its physical expert-major row dst and the
// source-major row src it copies (-1: none; an expert-major row whose
// source-major row was dropped gets dst with src -1).  Writes row_src[dst].
__device__ __forceinline__ void unpack_row(const Dims& D, const Ws& W, const UnpackStage& S, const int* svp, int g,
                                           int* __restrict__ row_src, int& src, int& dst) {
  const int N = D.N, E = D.E, L = D.L;
  src = dst = -1;
  const int d = floor_index(svp, N + 1, g);
  const int i = g - svp[d];                                  // expert-major row inside region d
  int s, u, sp, sd, ro;   // source, index in (s, e), send_off[s][e], send_off[s][d*L], recv_off[d][s]
  if (d == S.d0) {
    const int l = min(floor_index(S.eo, L + 1, i), L - 1);
    const int u1 = i - S.eo[l];
    s = min(floor_index(S.sie + l, N + 1, u1, L), N - 1);
    u = u1 - S.sie[s * L + l];
    sp = S.so[s * (L + 1) + l];
    sd = S.so[s * (L + 1)];
    ro = S.ro[s];
  } else {
    const int* eo = W.exp_off + d * (L + 1);
    const int l = min(floor_index(eo, L + 1, i), L - 1);
    const int e = d * L + l;
    const int u1 = i - eo[l];
    s = min(floor_index(W.src_in_exp + e, N + 1, u1, E), N - 1);
    u = u1 - W.src_in_exp[s * E + e];
    const int* so = W.send_off + s * (E + 1);
    sp = so[e];
    sd = so[d * L];
    ro = W.recv_off[d * (N + 1) + s];
  }
  const int j = region_row(D, s, (sp - sd) + u, ro);   // source-major row
  const int pd = W.base[d] + i;
  if (pd < D.rows) {
    dst = pd;
    const int ps = W.base[d] + j;
    const bool ok = (D.R == 0 || j < D.R) && j >= 0 && ps < D.rows;
    row_src[pd] = ok ? s * D.TK + sp + u : -1;
    if (ok) src = ps;
  }
}

// ------------------------------------------------------------------ one-shot unpack
//
// The receive half in the one-shot form (one 16-byte unit per thread,
// workgroups in row order; 64 or 256 threads each, see launch_unpack): first
// k_unpack_index maps every valid expert-major row g (region order) to the
// source-major row it copies -- the segment search of unpack_row, with the
// workgroup's region tables staged in LDS -- writing row_src and the pair
// {source row, physical row} into the workspace's umap; then k_unpack_os
// copies the fp8 payload units of all rows, then (a tile range of its own)
// their scale units: with each row's 14 scale units interleaved after its
// 448 payload units (H = 7168) the copy took 1456 us at combine-heavy size,
// with the two ranges apart 1271 us (the old one-chunk-per-workgroup form:
// 1411 us).
constexpr int kIdxThreads = 256;   // k_unpack_index: rows per workgroup (one staging of the region tables)

__global__ __launch_bounds__(kIdxThreads) void k_unpack_index(Dims D, Ws W, int* __restrict__ exp_off,
                                                             int* __restrict__ row_src) {
  __shared__ int svp[kMaxN + 1];
  __shared__ int stage[kStageInts];
  for (int i = threadIdx.x; i <= D.N; i += kIdxThreads) svp[i] = W.vprefix[i];
  if (blockIdx.x == 0)   // per-expert offsets for the grouped GEMM, as computed by the scan
    for (int i = threadIdx.x; i < D.N * (D.L + 1); i += kIdxThreads) exp_off[i] = W.exp_off[i];
  __syncthreads();
  const int valid = svp[D.N];
  for (int64_t lo64 = (int64_t)blockIdx.x * kIdxThreads; lo64 < valid; lo64 += (int64_t)gridDim.x * kIdxThreads) {
    const int lo = (int)lo64, hi = min(valid, lo + kIdxThreads);
    const UnpackStage S = unpack_stage<kIdxThreads>(D, W, svp, stage, lo, hi);
    const int g = lo + (int)threadIdx.x;
    if (g < hi) {
      int src, dst;
      unpack_row(D, W, S, svp, g, row_src, src, dst);
      W.umap[g] = make_int2(dst >= 0 ? src : -1, dst);
    }
    __syncthreads();   // the stage is rebuilt for the next range
  }
}

__global__ __launch_bounds__(kOsThreads) void k_unpack_os(Dims D, Ws W, const uint8_t* __restrict__ recv_q,
                                                          const float* __restrict__ recv_s, uint8_t* __restrict__ x_q,
                                                          float* __restrict__ x_s) {
  // Tile width: the workgroup size, 64 or 256 units (the launch chooses), a
  // power of two, so tiles are counted with shifts (a 64-bit division per
  // thread made the kernel 2-4% slower).
  const int lg = __builtin_ctz(blockDim.x);
  const int n16 = D.H / 16;                        // payload units per row
  const bool s16 = (D.NB & 3) == 0;
  const int ns = s16 ? D.NB / 4 : D.NB;
  const int valid = W.vprefix[D.N];
  const int64_t pay = (int64_t)valid * n16;
  const int64_t ptiles = (pay + (1 << lg) - 1) >> lg;
  const int64_t sc = (int64_t)valid * ns;
  const int64_t tiles = ptiles + ((sc + (1 << lg) - 1) >> lg);
  const v4u* __restrict__ qs = reinterpret_cast<const v4u*>(recv_q);
  v4u* __restrict__ qd = reinterpret_cast<v4u*>(x_q);
  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    if (tile < ptiles) {
      const int64_t u0 = tile << lg;
      if (u0 + threadIdx.x >= pay) continue;
      int g0, g, c;
      os_tile_pos(u0, n16, g0, g, c);
      const int2 m = W.umap[g];
      if (m.x >= 0) st16(qd + (int64_t)m.y * n16 + c, ld16(qs + (int64_t)m.x * n16 + c));
    } else {
      const int64_t u0 = (tile - ptiles) << lg;
      if (u0 + threadIdx.x >= sc) continue;
      int g0, g, c;
      os_tile_pos(u0, ns, g0, g, c);
      const int2 m = W.umap[g];
      if (m.x < 0) continue;
      if (s16) st16(reinterpret_cast<v4u*>(x_s + (int64_t)m.y * D.NB) + c, ld16(reinterpret_cast<const v4u*>(recv_s + (int64_t)m.x * D.NB) + c));
      else x_s[(int64_t)m.y * D.NB + c] = recv_s[(int64_t)m.x * D.NB + c];
    }
  }
}

// ------------------------------------------------------------------ one-shot pack
//
// The pack in the one-shot form: a work item is one pass (1024 elements) of
// one token, one item per wave, kOsThreads / 64 items per workgroup, items
// in (token, pass) order, so the workgroups resident at any moment read a
// window of consecutive tokens and store into the matching runs of every
// destination's rows.  Each wave resolves its token's k rows itself (lane j,
// slot j), quantises its 8 blocks of 128 and stores the fp8 bytes and the 8
// block scales to each of the k rows.  The first pass of a token also writes
// the slot's position when the count kernel left it (several routing chunks
// per rank), and in the direct form row_src.
template <bool DIRECT, int WAVES>
__device__ __forceinline__ void pack_tokens_os(const Dims& D, const Ws& W, const uint16_t* __restrict__ x,
                                               const int* __restrict__ idx, int* __restrict__ send_pos,
                                               uint8_t* __restrict__ q_out, float* __restrict__ s_out,
                                               int* __restrict__ row_src, int* __restrict__ exp_off) {
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  if (DIRECT && blockIdx.x == 0)   // per-expert offsets for the grouped GEMM, as computed by the scan
    for (int i = threadIdx.x; i < D.N * (D.L + 1); i += WAVES * kWave) exp_off[i] = W.exp_off[i];
  const int passes = x ? (D.H + kPackCols - 1) / kPackCols : 1;   // layout only: one item per token
  const int64_t items = (int64_t)D.N * D.T * passes;
  for (int64_t it = (int64_t)blockIdx.x * WAVES + wv; it < items; it += (int64_t)gridDim.x * WAVES) {
    const int tok = (int)(it / passes), pass = (int)(it - (int64_t)tok * passes);
    const int s = tok / D.T, t = tok - s * D.T;
    const int col = pass * kPackCols + lane * 16;    // this lane's 16 elements
    v4u a, b;
    const bool act = x != nullptr && pack_load(D, x, tok, col, a, b);
    // Lane j < k resolves slot j.
    const int row = lane < D.k ? pack_slot_row<DIRECT>(D, W, idx, send_pos, row_src, s, t * D.k + lane, pass == 0) : -1;
    if (x != nullptr) pack_store(D, a, b, col, act, row, lane, q_out, s_out);
  }
}

__global__ __launch_bounds__(kPackWaves * kWave) void k_pack_os(Dims D, Ws W, const uint16_t* __restrict__ x,
                                                        const int* __restrict__ idx, int* __restrict__ send_pos,
                                                        uint8_t* __restrict__ recv_q, float* __restrict__ recv_s) {
  pack_tokens_os<false, kPackWaves>(D, W, x, idx, send_pos, recv_q, recv_s, nullptr, nullptr);
}

__global__ __launch_bounds__(kOsThreads) void k_pack_direct_os(Dims D, Ws W, const uint16_t* __restrict__ x,
                                                               const int* __restrict__ idx, int* __restrict__ send_pos,
                                                               uint8_t* __restrict__ x_q, float* __restrict__ x_s,
                                                               int* __restrict__ row_src, int* __restrict__ exp_off) {
  pack_tokens_os<true, kOsWaves>(D, W, x, idx, send_pos, x_q, x_s, row_src, exp_off);
}

int launch_pack(const Dims& D, const Ws& W, const uint16_t* x, const int* idx, int* send_pos, uint8_t* q_out,
                float* s_out, int* row_src, int* exp_off, int cus, hipStream_t st) {
  if (D.N * D.T == 0) return MOE_OK;
  // Without tokens the pack only writes positions: send_pos with several
  // routing chunks per rank, row_src in the direct form.
  if (!x && !row_src && D.B == 1) return MOE_OK;
  const int64_t items = (int64_t)D.N * D.T * (x ? (D.H + kPackCols - 1) / kPackCols : 1);
  if (row_src)
    return launch("k_pack_direct_os", k_pack_direct_os, dim3(os_grid(items, kOsWaves)), dim3(kOsThreads), 0, st, D, W,
                  x, idx, send_pos, q_out, s_out, row_src, exp_off);
  return launch("k_pack_os", k_pack_os, dim3(os_grid(items, kPackWaves)), dim3(kPackWaves * kWave), 0, st, D, W, x,
                idx, send_pos, q_out, s_out);
}

int launch_unpack(const Dims& D, const Ws& W, const uint8_t* recv_q, const float* recv_s, uint8_t* x_q, float* x_s,
                  int* exp_off, int* row_src, int cus, hipStream_t st) {
  const int rc = launch("k_unpack_index", k_unpack_index, dim3(os_grid(D.rows, kIdxThreads)), dim3(kIdxThreads), 0, st, D, W,
                        exp_off, row_src);
  if (rc != MOE_OK || x_q == nullptr || D.rows == 0) return rc;   // layout only
  // Tiles of 64 units (one wave per workgroup) from 2^26 payload units up
  // (a 1-1.6% gain at the combine-heavy and prefill sizes), of 256 below
  // (64 was 1-1.4% slower at the decode, Kimi-dispatch and tiny sizes).
  const int64_t pay = (int64_t)D.rows * (D.H / 16);
  const int th = pay >= ((int64_t)1 << 26) ? 64 : kOsThreads;
  const int64_t tiles = (pay + th - 1) / th + ((int64_t)D.rows * ((D.NB & 3) == 0 ? D.NB / 4 : D.NB) + th - 1) / th;
  return launch("k_unpack_os", k_unpack_os, dim3(os_grid(tiles * th, th)), dim3(th), 0, st, D, W, recv_q, recv_s, x_q,
                x_s);
}

// Slices of its hidden dimension each token is split into in the single
// launch's packers: at least 2 (finer items even out the packers' shares:
// at N = 64, T = 128 whole tokens left the waves 1.46 items each, so half of
// them did twice the work of the rest), then doubled while there are fewer
// work items than the GPU holds waves (about 32 per CU), so small batches
// still keep enough loads and stores in flight.
static int pack_slices(const Dims& D, int cus, bool payload) {
  const int64_t tokens = (int64_t)D.N * D.T;
  const int passes = (D.H + kPackCols - 1) / kPackCols;
  const int64_t wave_slots = (int64_t)cus * 32;
  if (!payload) return 1;
  int sl = passes >= 2 ? 2 : 1;
  while (sl * 2 <= passes && tokens * sl * 2 <= wave_slots) sl *= 2;
  return sl;
}

// Workgroups of k_dispatch_ll to place per CU with `lds` bytes of dynamic
// LDS: what the occupancy query allows, at most kLlBlocksPerCu.  On MI355X
// the first wave of this launch holds 6 per CU although the query reports 7;
// with 7 per CU every 7th packer starts only after another has finished,
// which costs more than it gains (measured at the decode shapes).
constexpr int kLlBlocksPerCu = 6;
static int ll_blocks_per_cu(const void* kernel, size_t lds) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, size_t>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  std::lock_guard<std::mutex> g(mu);
  auto it = cache.find({dev, kernel, lds});
  if (it != cache.end()) return it->second;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, kThreads, lds) != hipSuccess || nb < 1) nb = 1;
  if (nb > kLlBlocksPerCu) nb = kLlBlocksPerCu;
  cache[{dev, kernel, lds}] = nb;
  return nb;
}

int launch_dispatch_ll(const Dims& D0, const Ws& W, const uint16_t* x, const int* idx, int* send_pos,
                       uint8_t* q_out, float* s_out, int* row_src, int* exp_off, int cus, hipStream_t st) {
  if (D0.B != 1 || D0.N * D0.T == 0) return MOE_EINVAL;
  const bool direct = row_src != nullptr;
  Dims D = D0;
  D.slices = pack_slices(D, cus, x != nullptr);
  // Dynamic LDS: the largest role's (the packers' is a scale row per wave).
  const size_t lds = std::max({count_lds_bytes(D.E), column_ll_lds_bytes(D.N, D.E),
                               sizeof(float) * (size_t)kLlWaves * D.NB});
  const void* kernel = direct ? reinterpret_cast<const void*>(k_dispatch_ll_direct)
                              : reinterpret_cast<const void*>(k_dispatch_ll);
  const int layout_wgs = 2 * D.N + 1;
  // Packers: one wave per work item (4 per workgroup), no more than fit on
  // the GPU beside the layout workgroups, so no packer starts late.  The
  // direct form needs packers without tokens too (they write row_src).
  int npack = 0;
  if (x || direct) {
    const int64_t need = ((int64_t)D.N * D.T * D.slices + kLlWaves - 1) / kLlWaves;
    const int64_t resident = (int64_t)cus * ll_blocks_per_cu(kernel, lds) - layout_wgs;
    npack = (int)std::max<int64_t>(1, std::min(need, resident));
  }
  if (direct)
    return launch("k_dispatch_ll_direct", k_dispatch_ll_direct, dim3(layout_wgs + npack), dim3(kThreads), lds, st, D,
                  W, x, idx, send_pos, q_out, s_out, row_src, exp_off, npack);
  return launch("k_dispatch_ll", k_dispatch_ll, dim3(layout_wgs + npack), dim3(kThreads), lds, st, D, W, x, idx,
                send_pos, q_out, s_out, npack);
}

}  // namespace moe
