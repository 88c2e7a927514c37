// Dispatch data movement ("Enabling trillion-parameter models on AWS EFA",
// sections "Send and receive buffers", "Dispatch and combine", and
// "Evaluation: dispatch/combine latency" for the block-scaled fp8 payload).
//
//   k_pack    each workgroup streams a contiguous range of tokens, one wave
//             per token (or per slice of a token when tokens are too few to
//             fill the GPU): final slot positions, block-128 amax with DPP,
//             fp8 quantisation, and k 16-byte row stores straight into the
//             destination ranks' receive regions (the "remote write").
//   k_unpack  each workgroup streams a contiguous range of expert-major rows:
//             the receive side finds each row's (expert, source) segment from
//             the exchanged counts alone and copies it out of the
//             source-major receive region; one 1024-thread workgroup per CU,
//             its rows copied as one thread-interleaved range of 16-byte
//             units.
//   k_pack_direct  k_pack storing each row at its expert-major row instead
//             (peers mapped into each other's memory push straight into the
//             grouped-GEMM layout; on one GPU every rank is such a peer), so
//             neither the receive regions nor k_unpack are needed.
#include <map>
#include <tuple>
#include <mutex>

#include "route_dev.h"


namespace moe {

constexpr int kPkWaves = kPackShape.waves, kPkThreads = kPackShape.threads();
constexpr int kPackCols = kWave * 16;         // elements one wave covers per pass (16 per lane)
constexpr int kPackPasses = 4;                // passes whose loads are issued together

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

// One pass of a pack work item: this lane's 16 elements at column col (all
// in one 128-element block shared with 7 neighbouring lanes): block amax,
// scale, fp8 bytes, the k row stores; the scale goes to the wave's LDS row.
__device__ __forceinline__ void pack_pass(const Dims& D, const v4u& a, const v4u& b, int col, bool act, int row,
                                          int lane, uint8_t* __restrict__ recv_q, float* ssw) {
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
  if (act && (lane & 7) == 0) ssw[col / kScaleBlock] = amax != 0.0f ? scale : 0.0f;
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
__device__ __forceinline__ void item_cols(const Dims& D, int item, int& tok, int& sl, int& h0, int& h1) {
  const int passes = (D.H + kPackCols - 1) / kPackCols;
  const int pps = (passes + D.slices - 1) / D.slices;
  tok = item / D.slices;
  sl = item - tok * D.slices;
  h0 = sl * pps * kPackCols;
  h1 = min(D.H, (sl + 1) * pps * kPackCols);
}

// Pack work item `item` with the calling wave, whose rows are already
// resolved (lane j < k: receive row of slot j, -1 for none).  LOADED: pa and
// pb hold the item's first chunk.
template <bool LOADED>
__device__ __forceinline__ void pack_item(const Dims& D, int item, int row, const uint16_t* __restrict__ x,
                                          uint8_t* __restrict__ recv_q, float* __restrict__ recv_s, float* ssw,
                                          const v4u* pa = nullptr, const v4u* pb = nullptr) {
  const int lane = threadIdx.x & (kWave - 1);
  int tok, sl, h0, h1;
  item_cols(D, item, tok, sl, h0, h1);
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


// The row slot i (of rank s's T*k) is packed to, -1 for none.  DIRECT =
// false: its source-major receive row; DIRECT = true: its expert-major row,
// by the same index and rule k_unpack uses (it exists if both it and its
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

// The pack loop.  DIRECT = false: rows go to the source-major receive
// regions (recv_q, recv_s).  DIRECT = true: they go straight to their
// expert-major rows (x_q, x_s), and the loop also writes row_src and
// exp_off, the outputs of the receive half, which then has nothing left to
// do.
template <bool DIRECT>
__device__ __forceinline__ void pack_tokens(const Dims& D, const Ws& W, const uint16_t* __restrict__ x,
                                            const int* __restrict__ idx, int* __restrict__ send_pos,
                                            uint8_t* __restrict__ recv_q, float* __restrict__ recv_s,
                                            int* __restrict__ row_src, int* __restrict__ exp_off) {
  __shared__ float sscale[kPkWaves][kMaxNB];
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  if (DIRECT && blockIdx.x == 0)   // per-expert offsets for the grouped GEMM, as computed by the scan
    for (int i = threadIdx.x; i < D.N * (D.L + 1); i += kPkThreads) exp_off[i] = W.exp_off[i];
  int lo, hi;
  block_range(D.N * D.T * D.slices, lo, hi);
  for (int item = lo + wv; item < hi; item += kPkWaves) {
    int tok, sl, h0, h1;
    item_cols(D, item, tok, sl, h0, h1);
    const int s = tok / D.T, t = tok - s * D.T;
    // The item's first token loads go out before its rows are resolved, so
    // the two latencies overlap: 2-3 us less at the decode shape, no change
    // from combine-heavy size up (98 VGPRs, 4 workgroups per CU there,
    // against 65 and 7 without).  Staging the routing tables in LDS as the
    // unpack does changed nothing here.
    v4u a[kPackPasses], b[kPackPasses];
    if (x != nullptr) load_chunk(x + (int64_t)tok * D.H, h0, h1, lane, a, b);
    // Lane j < k resolves slot j.
    const int row = lane < D.k ? pack_slot_row<DIRECT>(D, W, idx, send_pos, row_src, s, t * D.k + lane, sl == 0) : -1;
    if (x == nullptr) continue;
    pack_item<true>(D, item, row, x, recv_q, recv_s, sscale[wv], a, b);
  }
}

__global__ __launch_bounds__(kPkThreads) void k_pack(Dims D, Ws W, const uint16_t* __restrict__ x,
                                                     const int* __restrict__ idx, int* __restrict__ send_pos,
                                                     uint8_t* __restrict__ recv_q, float* __restrict__ recv_s) {
  pack_tokens<false>(D, W, x, idx, send_pos, recv_q, recv_s, nullptr, nullptr);
}

__global__ __launch_bounds__(kPkThreads) void k_pack_direct(Dims D, Ws W, const uint16_t* __restrict__ x,
                                                            const int* __restrict__ idx, int* __restrict__ send_pos,
                                                            uint8_t* __restrict__ x_q, float* __restrict__ x_s,
                                                            int* __restrict__ row_src, int* __restrict__ exp_off) {
  pack_tokens<true>(D, W, x, idx, send_pos, x_q, x_s, row_src, exp_off);
}

// ------------------------------------------------------------------ single launch
//
// The whole send half of dispatch in one launch, without a host round trip
// or a kernel boundary between the count exchange and the payload stores
// (AWS China blog "750B MoE model migration from a self-built RoCE cluster to
// AWS EFA", section 4.4, "DeepEP low-latency mode": one kernel per dispatch,
// no CPU in the loop, capturable in a graph).  The workgroup index gives
// the role:
//   b <  N   count rank b's slots (count_chunk) and publish them;
//   b == N   the cross-rank scans: receive offsets and region bases for the
//            packers first, then the tables dispatch_recv reads;
//   b >  N   pack: load tokens while the layout is being computed, then
//            quantise and store the rows once the positions are known.
// A workgroup only ever waits for values that workgroups with smaller
// indices produce.  The dispatcher hands each XCD its workgroups in index
// order, so the N + 1 layout workgroups are the first on their XCDs and are
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
// signal; no fence is issued at all.  The packers poll one of kReadyCopies
// replicated "ready" words, published after the values they need, then read
// their values (normally already there, otherwise they keep polling those).

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

// v[u] = value of p[u * stride] for u < n (n <= M).
template <int M>
__device__ __forceinline__ bool tag_wait_n(const uint64_t* p, int64_t stride, int n, uint32_t tag, int (&v)[M]) {
  return tag_gather<M>([&](int i) { return p + i * stride; }, n, tag, v);
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

// Tagged values the cross-rank role polls at once per thread (register
// budget: every role of the launch shares the pack role's 64 VGPRs).
constexpr int kCrossBatch = 4;

// LDS bytes of the cross-rank role.
inline size_t cross_ll_lds_bytes(int E) { return sizeof(int) * ((size_t)2 * kThreads + E + 1); }

// The cross-rank role: the same tables k_route_cross computes, from the
// tagged send offsets and counts of the count workgroups.  In the direct
// form (exp_out != nullptr) the packers need only the column workgroups'
// values: this role first waits for those and signals the packers, then
// computes the tables (for moe_layout_export, moe_dispatch_recv's
// successors and the combine) and copies exp_off to exp_out.
__device__ void cross_ll(const Dims& D, const Ws& W, uint32_t tag, int* sm, int* wsum, int* exp_out) {
  const int N = D.N, E = D.E, L = D.L, tid = threadIdx.x;
  int* part = sm;                  // [G][N], G*N <= kThreads: rows beyond the early ones
  int* partc = sm + kThreads;      // [G][N]: all rows
  int* ex = sm + 2 * kThreads;     // [E+1]
  bool ok = true;
  if (exp_out) {
    for (int dd = tid; dd < N && ok; dd += kThreads) {
      int one;
      ok = tag_wait(W.tcold + dd * kReadyStride, tag, &one);
    }
    __syncthreads();
    if (tid < kReadyCopies) tag_put(W.tready + tid * kReadyStride, tag, 1);
  }

  // (1) rows from source s to destination d are
  // send_off[s][(d+1)L] - send_off[s][dL]; thread (g, d) sums them over its
  // share of the sources.
  const int G = max(1, kThreads / N);
  const int d = tid % N, g = tid / N;
  const bool mine = g < G;
  const int per = (N + G - 1) / G;
  const int s0 = min(N, g * per), s1 = min(N, s0 + per);
  const int64_t ld = N + 1;
  // A thread whose sources fit one batch keeps the values for step (3).
  int lo1[kCrossBatch] = {}, hi1[kCrossBatch] = {};
  const bool one = s1 - s0 <= kCrossBatch;
  if (mine) {
    int sum = 0, over = 0;
    for (int sb = s0; sb < s1 && ok; sb += kCrossBatch) {
      const int n = min(kCrossBatch, s1 - sb);
      int lo[kCrossBatch] = {}, hi[kCrossBatch] = {};
      ok = tag_wait_n(W.toff + sb * ld + d, ld, n, tag, lo) && tag_wait_n(W.toff + sb * ld + d + 1, ld, n, tag, hi);
#pragma unroll
      for (int u = 0; u < kCrossBatch; ++u) {
        sum += hi[u] - lo[u];
        over += max(hi[u] - lo[u] - D.Ce, 0);
        lo1[u] = lo[u];
        hi1[u] = hi[u];
      }
    }
    part[g * N + d] = over;
    partc[g * N + d] = sum;
  }
  __syncthreads();
  int rt = 0, rover = 0;   // rows received by rank tid; of those, beyond the senders' early rows
  if (tid < N) {
    int a = 0;
    for (int g2 = 0; g2 < G; ++g2) {
      const int c = part[g2 * N + tid];
      part[g2 * N + tid] = a;
      a += c;
      rt += partc[g2 * N + tid];
    }
    rover = a;
  }
  // (2) Region bases, rows written per region, capacity and bound checks.
  int all, vall;
  const int b = block_scan<kThreads>(rt, wsum, &all);
  const int vb = block_scan<kThreads>(D.R ? min(rt, D.R) : rt, wsum, &vall);
  if (tid < N) {
    const int bd = D.R ? tid * D.R : b;
    tag_put(W.tbase + tid, tag, bd);
    W.base[tid] = bd;
    W.vprefix[tid] = vb;
    W.recv_total[tid] = rt;
    W.recv_off[tid * (N + 1) + N] = rover;
    uint32_t fl = 0;
    if (D.R && (rt > D.R || D.N * D.Ce + rover > D.R)) fl |= MOE_FLAG_OVERFLOW;
    if ((int64_t)rt > D.bound) fl |= MOE_FLAG_BOUND;
    if (fl) atomicOr(W.err, fl);
  }
  if (tid == 0) {
    W.base[N] = D.R ? N * D.R : all;
    W.vprefix[N] = vall;
  }
  // (3) recv_off[d][s], and what a packer of source s adds to a sender
  // position to get its row inside region d when the row is not one of the
  // sender's early rows: N*Ce + recv_off[d][s] - Ce - send_off[s][dL].
  if (mine && ok) {
    int acc = part[g * N + d];
    for (int sb = s0; sb < s1 && ok; sb += kCrossBatch) {
      const int n = min(kCrossBatch, s1 - sb);
      int lo[kCrossBatch], hi[kCrossBatch];
#pragma unroll
      for (int u = 0; u < kCrossBatch; ++u) {
        lo[u] = lo1[u];
        hi[u] = hi1[u];
      }
      if (!one)
        ok = tag_wait_n(W.toff + sb * ld + d, ld, n, tag, lo) && tag_wait_n(W.toff + sb * ld + d + 1, ld, n, tag, hi);
      for (int u = 0; u < n && ok; ++u) {
        const int s = sb + u;
        W.recv_off[d * (N + 1) + s] = acc;
        tag_put(W.trel + (int64_t)s * N + d, tag, N * D.Ce + acc - D.Ce - lo[u]);
        acc += max(hi[u] - lo[u] - D.Ce, 0);
      }
    }
  }
  __syncthreads();
  if (!exp_out && tid < kReadyCopies) tag_put(W.tready + tid * kReadyStride, tag, 1);

  // (4) Off the packers' path: src_in_exp and exp_off for dispatch_recv.
  for (int e = tid; e < E; e += kThreads) {
    int acc = 0;
    for (int sb = 0; sb < N && ok; sb += kCrossBatch) {
      const int n = min(kCrossBatch, N - sb);
      int c[kCrossBatch] = {};
      ok = tag_wait_n(W.tcnt + (int64_t)sb * E + e, E, n, tag, c);
      for (int u = 0; u < n && ok; ++u) {
        W.src_in_exp[(sb + u) * E + e] = acc;
        acc += c[u];
      }
    }
    W.src_in_exp[N * E + e] = acc;
    ex[e] = acc;
  }
  __syncthreads();
  {
    // Exclusive scan over all experts, four per thread (E <= 1024).
    const int e0 = min(E, tid * 4), e1 = min(E, e0 + 4);
    int v = 0;
    for (int e = e0; e < e1; ++e) v += ex[e];
    int etot;
    int x = block_scan<kThreads>(v, wsum, &etot);
    for (int e = e0; e < e1; ++e) {
      const int c = ex[e];
      ex[e] = x;
      x += c;
    }
    if (tid == 0) ex[E] = etot;
  }
  __syncthreads();
  for (int i = tid; i < N * (L + 1); i += kThreads) {
    const int dd = i / (L + 1), l = i - dd * (L + 1);
    W.exp_off[i] = ex[dd * L + l] - ex[dd * L];
    if (exp_out) exp_out[i] = ex[dd * L + l] - ex[dd * L];
  }
  if (!ok) atomicOr(W.err, MOE_FLAG_TIMEOUT);
}

// LDS ints of the column role: counts, then their column scans, [N][L]
// each; the senders' offsets to ranks d and d+1, [N] each; the expert
// totals and their scan [L+1]; the rows beyond the early ones per source,
// then their scan [N].
inline size_t column_ll_lds_bytes(int N, int E) { return sizeof(int) * ((size_t)2 * E + 3 * N + E / N + 1); }

// The column role of the direct form, for destination rank d.  From the
// tagged counts and send offsets alone it publishes what a packer needs for
// every row bound for d, so the packers do not wait for the cross-rank role:
//   temr[s][e]  what a packer of source s adds to a sender position of
//               expert e = d*L + l to get the row's expert-major row,
//               base[d] + exp_off[d][l] + src_in_exp[s][e] - send_off[s][e]
//               (packed regions: base[d] = sum over s of send_off[s][d*L],
//               the slots all sources send to ranks before d);
//   tlim[s][d]  (fixed regions) the sender positions below which the row's
//               source-major row fits region d: send_off[s][d*L] + C +
//               max(0, R - N*C - recv_off[d][s]) with C early rows (0: none);
// then tcold[d].
__device__ void column_ll(const Dims& D, const Ws& W, uint32_t tag, int d, int* sm, int* wsum) {
  const int N = D.N, L = D.L, E = D.E, NL = N * L, tid = threadIdx.x;
  int* c = sm;               // [N][L] counts of rank d's experts, then send_off[s][e]
  int* sie = sm + NL;        // [N][L] src_in_exp[s][e]
  int* so0 = sm + 2 * NL;    // [N] send_off[s][d*L]
  int* so1 = so0 + N;        // [N] send_off[s][(d+1)*L]
  int* ov = so1 + N;         // [N] rows beyond the early ones from s, then recv_off[d][s]
  int* eo = ov + N;          // [L+1] totals, then exp_off[d][l]
  // (1) The counts and the senders' offsets, kCrossBatch values per thread
  // at a time: indices below NL are counts, then send_off[s][d*L], then
  // send_off[s][(d+1)*L].
  bool ok = true;
  const int nv = NL + 2 * N;
  for (int i0 = tid * kCrossBatch; i0 < nv && ok; i0 += kThreads * kCrossBatch) {
    const int n = min(kCrossBatch, nv - i0);
    int v[kCrossBatch] = {};
    ok = tag_gather<kCrossBatch>(
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
  // (2) Per source: rows beyond the early ones; per expert: column scans
  // over sources.
  for (int s = tid; s < N && !fail; s += kThreads) ov[s] = max(so1[s] - so0[s] - D.Ce, 0);
  for (int l = tid; l < L && !fail; l += kThreads) {
    int acc = 0;
    for (int s = 0; s < N; ++s) {
      sie[s * L + l] = acc;
      acc += c[s * L + l];
    }
    eo[l] = acc;
  }
  __syncthreads();
  // (3) Per source: send_off[s][e] over rank d's experts, and recv_off[d][s]
  // (exclusive scan of the rows beyond the early ones; one thread, N <= 256).
  for (int s = tid; s < N && !fail; s += kThreads) {
    int acc = so0[s];
    for (int l = 0; l < L; ++l) {
      const int t = c[s * L + l];
      c[s * L + l] = acc;
      acc += t;
    }
  }
  if (tid == 0 && !fail) {
    int acc = 0;
    for (int s = 0; s < N; ++s) {
      const int t = ov[s];
      ov[s] = acc;
      acc += t;
    }
  }
  // (4) exp_off[d][l]: exclusive scan of the totals, four per thread (L <= 1024),
  // and the packed region base: the sum of send_off[s][d*L] over sources.
  int bd;
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
    int b = 0;
    for (int s = tid; s < N; s += kThreads) b += so0[s];
    block_scan<kThreads>(b, wsum, &bd);
    if (D.R) bd = d * D.R;
  }
  __syncthreads();
  if (!fail) {
    for (int i = tid; i < NL; i += kThreads) {
      const int s = i / L, l = i - s * L;
      tag_put(W.temr + (int64_t)s * E + d * L + l, tag, bd + eo[l] + sie[i] - c[i]);
    }
    if (D.R)
      for (int s = tid; s < N; s += kThreads)
        tag_put(W.tlim + (int64_t)s * N + d, tag, so0[s] + D.Ce + max(0, D.R - N * D.Ce - ov[s]));
  }
  __syncthreads();
  if (fail) {
    if (tid == 0) atomicOr(W.err, MOE_FLAG_TIMEOUT);
  } else if (tid == 0) {
    tag_put(W.tcold + d * kReadyStride, tag, 1);
  }
}

static_assert(kPkThreads == kThreads, "the single-launch dispatch runs every role with 256 threads");

// LDS bytes of the pack role (per-wave scales of one token row).
inline size_t pack_lds_bytes(int NB) { return sizeof(float) * (size_t)kPkWaves * NB; }

// The single launch.  DIRECT = false: rows go to the receive regions
// (recv_q, recv_s).  DIRECT = true: N column workgroups (after the count
// workgroups, before the cross-rank one) publish, per destination rank,
// each (source, expert)'s offset into the expert-major layout and the
// source-major fit limits; the cross-rank workgroup signals the packers once
// all columns are out, then computes the workspace tables and copies
// exp_off out; the packers store every row at its expert-major row (recv_q,
// recv_s = x_q, x_s) and write row_src.  Without tokens (x == nullptr) the
// direct form still runs its packers, for row_src.
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

  const int ncol = DIRECT ? D.N : 0;   // column workgroups
  if (wg < D.N) {
    count_chunk(D, W, idx, send_pos, wg, 0, smem, wsum, tag);
    __syncthreads();
    if (threadIdx.x == 0) tag_put(W.tcdone + wg * kReadyStride, tag, 1);
  } else if (DIRECT && wg < D.N + ncol) {
    column_ll(D, W, tag, wg - D.N, reinterpret_cast<int*>(smem), wsum);
  } else if (wg == D.N + ncol) {
    cross_ll(D, W, tag, reinterpret_cast<int*>(smem), wsum, DIRECT ? exp_out : nullptr);
  } else {
    const int p = wg - D.N - ncol - 1;
    const int items = D.N * D.T * D.slices;
    const int lo = (int)((int64_t)items * p / npack), hi = (int)((int64_t)items * (p + 1) / npack);
    bool fail = false;
    // Without early rows every packer needs the cross-rank results: wait
    // for a "ready" copy.  With early rows it needs only its own source
    // ranks' counts for most rows: wait for those ranks' count workgroups.
    auto gate = [&] {
      if (threadIdx.x == 0 && lo < hi) {
        int one;
        bool ok;
        if (DIRECT || D.Ce == 0) {
          ok = tag_wait(W.tready + (p % kReadyCopies) * kReadyStride, tag, &one);
        } else {
          const int s_first = lo / D.slices / D.T, s_last = (hi - 1) / D.slices / D.T;
          ok = tag_wait(W.tcdone + s_first * kReadyStride, tag, &one) &&
               tag_wait(W.tcdone + s_last * kReadyStride, tag, &one);
        }
        if (!ok) {
          sh_fail = 1;
          atomicOr(W.err, MOE_FLAG_TIMEOUT);
        }
      }
      __syncthreads();
      fail = sh_fail != 0;
    };
    // Expert of slot j (lane j < k) of work item `item`.
    auto expert = [&](int item) {
      const int lane = threadIdx.x & (kWave - 1);
      const int tok = item / D.slices;
      return lane < D.k ? idx[(int64_t)tok * D.k + lane] : -1;
    };
    // Rows of slot j (lane j < k) of work item `item`, expert e, from the
    // tagged positions and offsets.
    auto resolve = [&](int item, int e) {
      const int lane = threadIdx.x & (kWave - 1);
      const int tok = item / D.slices;
      const int s = tok / D.T;
      int row = -1;
      bool ok = true;
      if (!fail && lane < D.k) {
        const int64_t slot = (int64_t)tok * D.k + lane;
        if (DIRECT && e >= 0 && e < D.E) {
          // The column workgroup's values: the expert-major row offset and,
          // with fixed regions, the limit below which the source-major row
          // fits (the rule of k_unpack: the row exists if it fits region d,
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
    int item = lo + wv;
    if (DIRECT && x == nullptr) {   // layout only: positions and row_src
      gate();
      for (; item < hi; item += kPkWaves) resolve(item, expert(item));
      item = hi;
    }
    const bool has = item < hi;
    v4u a[kPackPasses], b[kPackPasses];
    int e1 = -1;
    if (has) {
      int tok, sl, h0, h1;
      item_cols(D, item, tok, sl, h0, h1);
      load_chunk(x + (int64_t)tok * D.H, h0, h1, threadIdx.x & (kWave - 1), a, b);
      e1 = expert(item);
    }
    if (!DIRECT || x != nullptr) gate();
    if (has) {
      pack_item<true>(D, item, resolve(item, e1), x, recv_q, recv_s, ssw, a, b);
      item += kPkWaves;
    }
    for (; item < hi; item += kPkWaves) pack_item<false>(D, item, resolve(item, expert(item)), x, recv_q, recv_s, ssw);
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
                                                          uint8_t* __restrict__ recv_q, float* __restrict__ recv_s,
                                                          int npack) {
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

// One region's routing tables staged in LDS, for the row searches.
struct UnpackStage {
  int d0;                      // the region (-1: none staged)
  int *sie, *so, *eo, *ro;     // src_in_exp / send_off columns, exp_off, recv_off of region d0
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
  S.sie = stage;
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

// The unpack, with the whole workgroup on consecutive rows (the access
// pattern of the plain copy, as k_comb_send): per chunk of rows, their
// sources are resolved into LDS, then thread t copies the chunk's 16-byte
// payload units t, t + kUcThreads, ... (kUcUnroll per step, loads before
// stores) and its scale units likewise.  Measured in one process,
// alternating calls, against a form with one wave per row: combine-heavy
// 1307-1402 against 1403-1461 us, prefill 2633-2697 against 2776-2840, equal
// at the decode shape, tiny 21 against 25 us, Kimi dispatch 199-201 against
// 205-213.  (Sixteen units per thread would spill at this workgroup size.)
constexpr int kUcThreads = 1024, kUcUnroll = 8;
constexpr int kUcMaxRows = kUcThreads * kUcUnroll / (kScaleBlock / 16);   // rows per chunk at H = 128
__global__ __launch_bounds__(kUcThreads) void k_unpack(Dims D, Ws W, const uint8_t* __restrict__ recv_q,
                                                            const float* __restrict__ recv_s,
                                                            uint8_t* __restrict__ x_q, float* __restrict__ x_s,
                                                            int* __restrict__ exp_off, int* __restrict__ row_src) {
  __shared__ int svp[kMaxN + 1];
  __shared__ int stage[kStageInts];
  __shared__ int t_src[kUcMaxRows], t_dst[kUcMaxRows];
  for (int i = threadIdx.x; i <= D.N; i += kUcThreads) svp[i] = W.vprefix[i];
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < D.N * (D.L + 1); i += kUcThreads) exp_off[i] = W.exp_off[i];
  __syncthreads();
  int lo, hi;
  block_range(svp[D.N], lo, hi);
  const UnpackStage S = unpack_stage<kUcThreads>(D, W, svp, stage, lo, hi);
  const int n16 = D.H / 16;                                    // payload units per row
  const int rchunk = kUcThreads * kUcUnroll / n16;             // whole rows per chunk (n16 >= 8)
  const int dr1 = kUcThreads / n16, dc1 = kUcThreads % n16;   // per-slot advance of (row, column)
  const int r0 = threadIdx.x / n16, c0 = threadIdx.x % n16;
  const v4u* __restrict__ qs = reinterpret_cast<const v4u*>(recv_q);
  v4u* __restrict__ qd = reinterpret_cast<v4u*>(x_q);
  const bool scales16 = (D.NB & 3) == 0;
  for (int g0 = lo; g0 < hi; g0 += rchunk) {
    const int nr = min(rchunk, hi - g0);
    for (int r = threadIdx.x; r < nr; r += kUcThreads) {
      int src, dst;
      unpack_row(D, W, S, svp, g0 + r, row_src, src, dst);
      t_src[r] = dst >= 0 ? src : -1;
      t_dst[r] = dst;
    }
    __syncthreads();
    if (x_q != nullptr) {
      v4u v[kUcUnroll];
      int dst[kUcUnroll];
      int r = r0, c = c0;
#pragma unroll
      for (int u = 0; u < kUcUnroll; ++u) {
        dst[u] = -1;
        if (r < nr) {
          const int sr = t_src[r];
          if (sr >= 0) {
            dst[u] = t_dst[r];
            v[u] = ld16(qs + (int64_t)sr * n16 + c);
          }
        }
        r += dr1;
        c += dc1;
        if (c >= n16) {
          c -= n16;
          ++r;
        }
      }
      c = c0;
#pragma unroll
      for (int u = 0; u < kUcUnroll; ++u) {
        if (dst[u] >= 0) st16(qd + (int64_t)dst[u] * n16 + c, v[u]);
        c += dc1;
        if (c >= n16) c -= n16;
      }
      // Scales: NB floats per row, as 16-byte units where rows are whole units.
      if (scales16) {
        const int s16 = D.NB / 4;
        for (int f = threadIdx.x; f < nr * s16; f += kUcThreads) {
          const int rr = f / s16, cc = f - rr * s16;
          if (t_src[rr] >= 0)
            st16(reinterpret_cast<v4u*>(x_s + (int64_t)t_dst[rr] * D.NB) + cc,
                 ld16(reinterpret_cast<const v4u*>(recv_s + (int64_t)t_src[rr] * D.NB) + cc));
        }
      } else {
        for (int f = threadIdx.x; f < nr * D.NB; f += kUcThreads) {
          const int rr = f / D.NB, cc = f - rr * D.NB;
          if (t_src[rr] >= 0) x_s[(int64_t)t_dst[rr] * D.NB + cc] = recv_s[(int64_t)t_src[rr] * D.NB + cc];
        }
      }
    }
    __syncthreads();
  }
}

// Slices of its hidden dimension each token is split into: doubled while
// there are fewer work items than the GPU holds waves (about 32 per CU), so
// small batches still keep enough loads and stores in flight.
static int pack_slices(const Dims& D, int cus, bool payload) {
  const int64_t tokens = (int64_t)D.N * D.T;
  const int passes = (D.H + kPackCols - 1) / kPackCols;
  const int64_t wave_slots = (int64_t)cus * 32;
  int sl = 1;
  if (payload)
    while (sl * 2 <= passes && tokens * sl * 2 <= wave_slots) sl *= 2;
  return sl;
}

int launch_pack(const Dims& D0, const Ws& W, const uint16_t* x, const int* idx, int* send_pos, uint8_t* q_out,
                float* s_out, int* row_src, int* exp_off, int cus, hipStream_t st) {
  if (D0.N * D0.T == 0) return MOE_OK;
  Dims D = D0;
  D.slices = pack_slices(D, cus, x != nullptr);
  const int grid = stream_grid(kPackShape, cus, (int64_t)D.N * D.T * D.slices, kPkWaves);
  if (row_src)
    return launch("k_pack_direct", k_pack_direct, dim3(grid), dim3(kPkThreads), 0, st, D, W, x, idx, send_pos, q_out,
                  s_out, row_src, exp_off);
  return launch("k_pack", k_pack, dim3(grid), dim3(kPkThreads), 0, st, D, W, x, idx, send_pos, q_out, s_out);
}

int launch_unpack(const Dims& D, const Ws& W, const uint8_t* recv_q, const float* recv_s, uint8_t* x_q, float* x_s,
                  int* exp_off, int* row_src, int cus, hipStream_t st) {
  const int64_t need = ((int64_t)D.rows * (D.H / 16) + kUcThreads * kUcUnroll - 1) / (kUcThreads * kUcUnroll);
  const int grid = (int)(need < cus ? (need < 1 ? 1 : need) : cus);
  return launch("k_unpack", k_unpack, dim3(grid), dim3(kUcThreads), 0, st, D, W, recv_q, recv_s, x_q, x_s, exp_off,
                row_src);
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
  size_t lds = count_lds_bytes(D.E);
  lds = lds > cross_ll_lds_bytes(D.E) ? lds : cross_ll_lds_bytes(D.E);
  lds = lds > pack_lds_bytes(D.NB) ? lds : pack_lds_bytes(D.NB);
  if (direct) lds = lds > column_ll_lds_bytes(D.N, D.E) ? lds : column_ll_lds_bytes(D.N, D.E);
  const void* kernel = direct ? reinterpret_cast<const void*>(k_dispatch_ll_direct)
                              : reinterpret_cast<const void*>(k_dispatch_ll);
  const int layout_wgs = D.N + 1 + (direct ? D.N : 0);
  // Packers: as many as the k_pack grid would have, but no more than fit on
  // the GPU beside the layout workgroups, so no packer starts late.  The
  // direct form needs packers without tokens too (they write row_src).
  int npack = 0;
  if (x || direct) {
    const int resident = cus * ll_blocks_per_cu(kernel, lds) - layout_wgs;
    npack = stream_grid(kPackShape, cus, (int64_t)D.N * D.T * D.slices, kPkWaves);
    if (resident >= 1 && npack > resident) npack = resident;
  }
  if (direct)
    return launch("k_dispatch_ll_direct", k_dispatch_ll_direct, dim3(layout_wgs + npack), dim3(kThreads), lds, st, D,
                  W, x, idx, send_pos, q_out, s_out, row_src, exp_off, npack);
  return launch("k_dispatch_ll", k_dispatch_ll, dim3(layout_wgs + npack), dim3(kThreads), lds, st, D, W, x, idx,
                send_pos, q_out, s_out, npack);
}

}  // namespace moe
