// Internal definitions shared by the HIP translation units of libmoe_ep.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <tuple>
#include <utility>

#include "moe_ep.h"

namespace moe {

// Launch `k` on `st` and return the launch's own status (hipLaunchKernel
// reports it directly, so an earlier error left by another library in the
// same thread is neither reported nor cleared).
template <typename... KArgs, typename... Args>
int launch(const char* name, void (*k)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t st,
           Args&&... args) {
  std::tuple<KArgs...> vals(std::forward<Args>(args)...);
  void* ptrs[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
  std::apply([&](auto&... v) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&v)), ...);
  }, vals);
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, ptrs, lds, st);
  if (e != hipSuccess) {
    fprintf(stderr, "libmoe_ep: launching %s failed: %s (%d)\n", name, hipGetErrorString(e), (int)e);
    return MOE_EHIP;
  }
  return MOE_OK;
}

constexpr int kWave = 64;            // CDNA wavefront width
constexpr int kWavesPerBlock = 4;    // 256-thread workgroups everywhere
constexpr int kThreads = kWave * kWavesPerBlock;
constexpr int kMaxN = 256;
constexpr int kMaxE = 1024;
constexpr int kMaxK = 64;
constexpr int kMaxH = 32768;
constexpr int kScaleBlock = 128;     // elements per fp32 scale
// Routing chunk: slots of one rank handled by one workgroup of the count
// kernel; every wave takes a contiguous quarter, 64 slots per batch.  The
// chunk is 256..4096 slots, chosen per shape so that small batches still
// spread over several workgroups per rank.
constexpr int kMinChunk = 256;
constexpr int kMaxChunk = 4096;
constexpr int kMaxBatches = kMaxChunk / kWavesPerBlock / kWave;

// Problem sizes derived once on the host.
struct Dims {
  int N, T, H, E, k;
  int L;        // experts per rank
  int TK;       // slots per rank = T*k
  int C;        // routing chunk, slots
  int B;        // routing chunks per rank
  int NB;       // scale blocks per row = H/128
  int slices;   // single-launch pack work items per token (1 = whole row per wave)
  int R;        // fixed region rows, 0 = packed
  int Ce;       // early (private) rows per sender in each fixed region, 0 = none
  int rows;     // rows of every receive / expert-major array
  int64_t bound;  // N*T*max(k, L)
};

// Workspace tables, all int32 unless noted.
struct Ws {
  uint32_t *err;      // sticky MOE_FLAG_* word
  int *blk;           // [N][B][E] chunk counts, then chunk base positions
  int *cnt;           // [N][E]
  int *send_off;      // [N][E+1]
  int *recv_off;      // [N(dest)][N(src)+1]
  int *recv_total;    // [N]
  int *base;          // [N+1] first physical row of each region
  int *vprefix;       // [N+1] running total of rows written per region
  int *exp_off;       // [N][L+1]
  int *src_in_exp;    // [N+1][E] rows of expert e from sources before s
  int *local;         // [N][T*k] rank of each slot inside its chunk (several chunks per rank)
  int2 *umap;         // [rows] per valid expert-major row (region order): {source-major row or -1, physical row}
  // Exchange area of the single-launch dispatch, present only when every
  // rank's slots fit one routing chunk.  Each entry is an 8-byte pair
  // (tag << 32 | value), published and read with single-copy-atomic stores
  // and loads at agent scope, so a reader that sees the tag of the current
  // call also sees that call's value and needs no fence.
  uint32_t *ctl;      // [kCtlGroups + 1][kCtlStride]: per-group finish counter and call number, then the
                      // count of finished groups
  uint64_t *tpos;     // [N*T*k] send positions
  uint64_t *toff;     // [N][N+1] send_off[s][d*L], [s][N] = valid slots of s
  uint64_t *tcnt;     // [N][E] counts
  uint64_t *trel;     // [N][N] N*C + recv_off[d][s] - C - send_off[s][d*L] (C early rows)
  uint64_t *tbase;    // [N] region bases
  uint64_t *tcdone;   // [N][kReadyStride]: rank s's count work is published (early rows)
  uint64_t *tcold;    // [N][kReadyStride]: the column of destination d is published (value: rows d receives)
  // Direct form only (rows stored at their expert-major rows):
  uint64_t *temr;     // [N][E] base[d] + exp_off[d][l] + src_in_exp[s][e] - send_off[s][e], e = d*L + l
  uint64_t *tlim;     // [N][N] fixed regions: sender positions of s below this fit region d
};

// Completion words (tcdone, tcold) sit one per 64-byte line.
constexpr int kReadyStride = 8;

// Control words of the single-launch dispatch.  Workgroup b belongs to group
// b % kCtlGroups; each group has its own 64-byte line holding the number of
// its workgroups that have finished and its copy of the call number (calls
// completed on this workspace), so no single address takes one atomic per
// workgroup.  Line kCtlGroups counts the groups that have finished.
constexpr int kCtlGroups = 16;
constexpr int kCtlStride = 16;   // uint32 words per line

// Tag of call number `epoch`: the top bit is set, so no plain table entry
// (non-negative, or -1) and no zeroed word ever looks like a tag.
__device__ __forceinline__ uint32_t epoch_tag(uint32_t epoch) { return 0x80000000u | (epoch % 0x7FFFFFFFu); }

__device__ __forceinline__ void tag_put(uint64_t* p, uint32_t tag, int v) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | (uint32_t)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t tag_load(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_ok(uint64_t u, uint32_t tag) { return (uint32_t)(u >> 32) == tag; }

// Upper bound on polls of one value; about a second at the longest, after
// which the reader gives up, sets MOE_FLAG_TIMEOUT and drops what depended
// on the value, so every wait ends.
constexpr int kSpinLimit = 1 << 21;

// Wait for a tagged value; false after kSpinLimit polls.
__device__ __forceinline__ bool tag_wait(const uint64_t* p, uint32_t tag, int* v) {
  uint64_t u = tag_load(p);
  for (int it = 0; !tag_ok(u, tag); ++it) {
    if (it == kSpinLimit) return false;
    __builtin_amdgcn_s_sleep(2);
    u = tag_load(p);
  }
  *v = (int)(uint32_t)u;
  return true;
}

// ------------------------------------------------------------------ helpers

// One DPP move inside rows of 16 lanes; all lanes active.
template <int Ctrl>
__device__ __forceinline__ int dpp_mov(int v) {
  return __builtin_amdgcn_update_dpp(0, v, Ctrl, 0xF, 0xF, false);
}
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror: lane i <-> 7-i inside 8 lanes

// Max over each aligned group of 8 lanes, for non-negative float bit
// patterns compared as integers (exact for finite values).
__device__ __forceinline__ int max8_lanes(int v) {
  v = max(v, dpp_mov<kDppQuadXor1>(v));
  v = max(v, dpp_mov<kDppQuadXor2>(v));
  v = max(v, dpp_mov<kDppHalfMirror>(v));
  return v;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) & 0x8000u) | 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Row inside region d of block index u of source s's rows for d (u =
// send_pos - send_off[s][d*L]), given recv_off[d][s]: the sender's early
// rows first, then its share of the region's common part.
__device__ __forceinline__ int region_row(const Dims& D, int s, int u, int recv_off_ds) {
  return u < D.Ce ? s * D.Ce + u : D.N * D.Ce + recv_off_ds + (u - D.Ce);
}

// ------------------------------------------------------------------ streaming rows
//
// The row kernels move gigabytes once, so every bulk access is a 16-byte
// non-temporal load or store.  Most run in the one-shot form below (short
// workgroups taking consecutive tiles); the send-side partial sums from 16384
// tokens give each workgroup a contiguous range instead.
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// Non-temporal on both sides: 3-4% faster than plain accesses on the row
// kernels, and the fastest of the cache-policy combinations on a copy.
__device__ __forceinline__ v4u ld16(const v4u* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st16(v4u* p, v4u v) { __builtin_nontemporal_store(v, p); }

// This workgroup's share [lo, hi) of n items split evenly over the grid.
__device__ __forceinline__ void block_range(int n, int& lo, int& hi) {
  lo = (int)((int64_t)n * blockIdx.x / gridDim.x);
  hi = (int)((int64_t)n * (blockIdx.x + 1) / gridDim.x);
}

// One-shot row kernels: one 16-byte unit per thread.  A workgroup of
// kOsThreads threads takes a tile of consecutive units of the flat (row,
// column) unit space, and tiles go to workgroups in index order.  The
// dispatcher starts workgroups in index order and each lives briefly, so the
// workgroups resident at any moment cover a compact, moving window of rows,
// which keeps HBM pages open for all CUs at once.  Plain streams in this form
// measured 6.5 TB/s for a copy, 6.8 for writes and 7.1 for reads on MI355X,
// against 4.7, 4.1 and 6.1 with one contiguous chunk per workgroup (one box,
// one process), and a row permutation driven by a real routing copied at 6.3.
constexpr int kOsThreads = 256;
constexpr int64_t kOsMaxGrid = 16000000;   // workgroups per launch: keeps grid.x * 256 below 2^32

inline int os_grid(int64_t units, int per_wg = kOsThreads) {
  const int64_t t = (units + per_wg - 1) / per_wg;
  return (int)(t < 1 ? 1 : (t < kOsMaxGrid ? t : kOsMaxGrid));
}

// Tile starting at unit u0 of a flat space of rows of `per` units: the
// tile's first row g0, and this thread's unit's row g and column c.  One
// 64-bit division per tile (wave-uniform) and a 32-bit one only where the
// thread's unit lies past the tile's first row.
__device__ __forceinline__ void os_tile_pos(int64_t u0, int per, int& g0, int& g, int& c) {
  g0 = (int)(u0 / per);
  c = (int)(u0 - (int64_t)g0 * per) + (int)threadIdx.x;
  g = g0;
  if (c >= per) {
    const int q = c / per;
    g += q;
    c -= q * per;
  }
}

// Largest i in [0, n) with a[i*stride] <= v, for non-decreasing a with a[0] <= v.
template <class P>
__device__ __forceinline__ int floor_index(P a, int n, int v, int stride = 1) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a[(int64_t)mid * stride] <= v) lo = mid; else hi = mid;
  }
  return lo;
}

// Launchers (one per translation unit that owns the kernels).
int launch_route(const Dims& D, const Ws& W, const int* idx, int* send_pos, hipStream_t st);
// row_src == nullptr: into the source-major receive regions (q_out, s_out =
// recv_q, recv_s); otherwise straight into the expert-major rows (q_out,
// s_out = x_q, x_s), also writing row_src and exp_off.
int launch_pack(const Dims& D, const Ws& W, const uint16_t* x, const int* idx, int* send_pos, uint8_t* q_out,
                float* s_out, int* row_src, int* exp_off, int cus, hipStream_t st);
int launch_unpack(const Dims& D, const Ws& W, const uint8_t* recv_q, const float* recv_s, uint8_t* x_q, float* x_s,
                  int* exp_off, int* row_src, int cus, hipStream_t st);
int launch_comb_send(const Dims& D, const Ws& W, const uint16_t* y, const int* row_src, uint16_t* comb, int cus,
                     hipStream_t st);
int launch_comb_recv(const Dims& D, const uint16_t* comb, const int* send_pos, const float* w, uint16_t* out, int cus,
                     hipStream_t st);
int launch_comb_pull(const Dims& D, const Ws& W, const uint16_t* y, const int* idx, const int* send_pos,
                     const float* w, uint16_t* out, int cus, hipStream_t st);
// row_src == nullptr: into the receive regions (q_out, s_out = recv_q,
// recv_s); otherwise the direct form, into the expert-major rows (x_q, x_s),
// also writing row_src and exp_off.
int launch_dispatch_ll(const Dims& D, const Ws& W, const uint16_t* x, const int* idx, int* send_pos,
                       uint8_t* q_out, float* s_out, int* row_src, int* exp_off, int cus, hipStream_t st);
int launch_comb_send_partial(const Dims& D, const Ws& W, const uint16_t* y, const int* idx, const int* send_pos,
                             const float* w, uint16_t* comb, int cus, hipStream_t st);
int launch_comb_recv_partial(const Dims& D, const Ws& W, const uint16_t* comb, const int* idx, const int* send_pos,
                             uint16_t* out, int cus, hipStream_t st);
int launch_fill_u32(uint32_t* p, uint32_t v, int n, hipStream_t st);

}  // namespace moe
