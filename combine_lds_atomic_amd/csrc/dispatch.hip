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
//             source-major receive region.
#include "moe_internal.h"

// fp32 -> e4m3fn conversion.  Both variants give the same bytes on the
// whole input domain (every bfloat16 pair x <= amax), which the exhaustive
// sweep test checks against the oracle:
//   MOE_PACK_CVT 0: round with integer operations on the float's bits;
//                1: v_cvt_pk_fp8_f32 (on gfx950 it converts to OCP e4m3fn,
//                   round to nearest even), two values per instruction.
#ifndef MOE_PACK_CVT
#define MOE_PACK_CVT 1
#endif
#ifndef MOE_PACK_PASSES
#define MOE_PACK_PASSES 4
#endif

namespace moe {

constexpr int kPkWaves = kPackShape.waves, kPkThreads = kPackShape.threads();
constexpr int kUpWaves = kUnpackShape.waves, kUpThreads = kUnpackShape.threads();
constexpr int kPackCols = kWave * 16;         // elements one wave covers per pass (16 per lane)
constexpr int kPackPasses = MOE_PACK_PASSES;  // passes whose loads are issued together

// Four quotients x[i] / scale (IEEE division) packed as e4m3fn bytes,
// little end first.
__device__ __forceinline__ uint32_t quant4(const float* v, float scale) {
  float q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = v[i] / scale;
#if MOE_PACK_CVT
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w, true);
  return (uint32_t)w;
#else
  return f32_to_e4m3fn(q[0]) | (f32_to_e4m3fn(q[1]) << 8) | (f32_to_e4m3fn(q[2]) << 16) |
         (f32_to_e4m3fn(q[3]) << 24);
#endif
}

// Work item = (token, slice): slice sl of a token covers passes
// [sl*pps, (sl+1)*pps) of 1024 elements, pps = ceil(passes / slices).
__global__ __launch_bounds__(kPkThreads) void k_pack(Dims D, Ws W, const uint16_t* __restrict__ x,
                                                     const int* __restrict__ idx, int* __restrict__ send_pos,
                                                     uint8_t* __restrict__ recv_q, float* __restrict__ recv_s) {
  __shared__ float sscale[kPkWaves][kMaxNB];
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int passes = (D.H + kPackCols - 1) / kPackCols;
  const int pps = (passes + D.slices - 1) / D.slices;
  int lo, hi;
  block_range(D.N * D.T * D.slices, lo, hi);
  for (int item = lo + wv; item < hi; item += kPkWaves) {
    const int tok = item / D.slices, sl = item - tok * D.slices;
    const int s = tok / D.T, t = tok - s * D.T;
    // Lane j < k resolves slot j.  With one routing chunk per rank the count
    // kernel already wrote the final position; otherwise it left the rank
    // inside the chunk, and the chunk's base for the expert completes it.
    int row = -1;
    if (lane < D.k) {
      const int i = t * D.k + lane;
      const int64_t slot = (int64_t)s * D.TK + i;
      const int e = idx[slot];
      if (e >= 0 && e < D.E) {
        int sp;
        if (D.B > 1) {
          sp = W.local[slot] + W.blk[((int64_t)s * D.B + i / D.C) * D.E + e];
          if (sl == 0) send_pos[slot] = sp;
        } else {
          sp = send_pos[slot];
        }
        const int d = e / D.L;
        const int r = W.recv_off[d * (D.N + 1) + s] + sp - W.send_off[s * (D.E + 1) + d * D.L];
        const int pr = W.base[d] + r;
        if ((D.R == 0 || r < D.R) && r >= 0 && pr < D.rows) row = pr;
      }
    }
    if (x == nullptr) continue;

    const uint16_t* xr = x + (int64_t)tok * D.H;
    const int h0 = sl * pps * kPackCols, h1 = min(D.H, (sl + 1) * pps * kPackCols);
    for (int c0 = h0; c0 < h1; c0 += kPackCols * kPackPasses) {
      // Issue the loads of several passes before any math.
      v4u a[kPackPasses], b[kPackPasses];
#pragma unroll
      for (int p = 0; p < kPackPasses; ++p) {
        const int col = c0 + p * kPackCols + lane * 16;
        const bool act = col < h1;
        a[p] = act ? ld16(reinterpret_cast<const v4u*>(xr + col)) : v4u{0, 0, 0, 0};
        b[p] = act ? ld16(reinterpret_cast<const v4u*>(xr + col + 8)) : v4u{0, 0, 0, 0};
      }
#pragma unroll
      for (int p = 0; p < kPackPasses; ++p) {
        if (c0 + p * kPackCols >= h1) break;
        const int col = c0 + p * kPackCols + lane * 16;   // this lane's 16 elements
        const bool act = col < h1;                          // whole 8-lane groups drop out together
        float v[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = bf16_lo(a[p][i]);
          v[2 * i + 1] = bf16_hi(a[p][i]);
          v[8 + 2 * i] = bf16_lo(b[p][i]);
          v[8 + 2 * i + 1] = bf16_hi(b[p][i]);
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
        if (act && (lane & 7) == 0) sscale[wv][col / kScaleBlock] = amax != 0.0f ? scale : 0.0f;
        for (int j = 0; j < D.k; ++j) {
          const int rj = __builtin_amdgcn_readlane(row, j);
          if (rj >= 0 && act) st16(reinterpret_cast<v4u*>(recv_q + (int64_t)rj * D.H + col), q);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    for (int bi = h0 / kScaleBlock + lane; bi < h1 / kScaleBlock; bi += kWave) {
      const float sc = sscale[wv][bi];
      for (int j = 0; j < D.k; ++j) {
        const int rj = __builtin_amdgcn_readlane(row, j);
        if (rj >= 0) recv_s[(int64_t)rj * D.NB + bi] = sc;
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

constexpr int kRowsPerPass = 8;   // rows whose metadata one wave resolves at once

__global__ __launch_bounds__(kUpThreads) void k_unpack(Dims D, Ws W, const uint8_t* __restrict__ recv_q,
                                                       const float* __restrict__ recv_s, uint8_t* __restrict__ x_q,
                                                       float* __restrict__ x_s, int* __restrict__ exp_off,
                                                       int* __restrict__ row_src) {
  __shared__ int svp[kMaxN + 1];
  for (int i = threadIdx.x; i <= D.N; i += kUpThreads) svp[i] = W.vprefix[i];
  if (blockIdx.x == 0)   // per-expert offsets for the grouped GEMM, as computed by the scan
    for (int i = threadIdx.x; i < D.N * (D.L + 1); i += kUpThreads) exp_off[i] = W.exp_off[i];
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int N = D.N, E = D.E, L = D.L;
  const bool scales16 = (D.NB & 3) == 0;   // scale rows are whole 16-byte units
  int lo, hi;
  block_range(svp[N], lo, hi);        // valid rows, in region order
  for (int g0 = lo + wv; g0 < hi; g0 += kUpWaves * kRowsPerPass) {
    int src = -1, dst = -1;
    const int g = g0 + lane * kUpWaves;
    if (lane < kRowsPerPass && g < hi) {
      const int d = floor_index(svp, N + 1, g);
      const int i = g - svp[d];                                  // expert-major row inside region d
      const int* eo = W.exp_off + d * (L + 1);
      const int l = min(floor_index(eo, L + 1, i), L - 1);
      const int e = d * L + l;
      const int u1 = i - eo[l];
      const int s = min(floor_index(W.src_in_exp + e, N + 1, u1, E), N - 1);
      const int u = u1 - W.src_in_exp[s * E + e];
      const int* so = W.send_off + s * (E + 1);
      const int j = W.recv_off[d * (N + 1) + s] + (so[e] - so[d * L]) + u;   // source-major row
      const int pd = W.base[d] + i;
      if (pd < D.rows) {
        dst = pd;
        const int ps = W.base[d] + j;
        const bool ok = (D.R == 0 || j < D.R) && j >= 0 && ps < D.rows;
        row_src[pd] = ok ? s * D.TK + so[e] + u : -1;
        if (ok) src = ps;
      }
    }
    if (x_q == nullptr) continue;   // layout only
    for (int r = 0; r < kRowsPerPass; ++r) {
      const int sr = __builtin_amdgcn_readlane(src, r);
      const int dr = __builtin_amdgcn_readlane(dst, r);
      if (sr < 0 || dr < 0) continue;
      wave_copy16<8>(reinterpret_cast<v4u*>(x_q + (int64_t)dr * D.H),
                     reinterpret_cast<const v4u*>(recv_q + (int64_t)sr * D.H), D.H / 16, lane);
      if (scales16) {
        const int n16 = D.NB / 4;
        if (lane < n16)
          st16(reinterpret_cast<v4u*>(x_s + (int64_t)dr * D.NB) + lane,
               ld16(reinterpret_cast<const v4u*>(recv_s + (int64_t)sr * D.NB) + lane));
        for (int c = lane + kWave; c < n16; c += kWave)
          st16(reinterpret_cast<v4u*>(x_s + (int64_t)dr * D.NB) + c,
               ld16(reinterpret_cast<const v4u*>(recv_s + (int64_t)sr * D.NB) + c));
      } else {
        for (int c = lane; c < D.NB; c += kWave) x_s[(int64_t)dr * D.NB + c] = recv_s[(int64_t)sr * D.NB + c];
      }
    }
  }
}

int launch_pack(const Dims& D0, const Ws& W, const uint16_t* x, const int* idx, int* send_pos, uint8_t* recv_q,
                float* recv_s, int cus, hipStream_t st) {
  if (D0.N * D0.T == 0) return MOE_OK;
  // Split tokens into slices of their hidden dimension while there are fewer
  // tokens than the GPU holds waves (about 32 per CU), so small batches still
  // keep enough loads and stores in flight.
  Dims D = D0;
  const int64_t tokens = (int64_t)D.N * D.T;
  const int passes = (D.H + kPackCols - 1) / kPackCols;
  const int64_t wave_slots = (int64_t)cus * 32;
  D.slices = 1;
  if (x != nullptr)
    while (D.slices * 2 <= passes && tokens * D.slices * 2 <= wave_slots) D.slices *= 2;
  const int grid = stream_grid(kPackShape, cus, tokens * D.slices, kPkWaves);
  return launch("k_pack", k_pack, dim3(grid), dim3(kPkThreads), 0, st, D, W, x, idx, send_pos, recv_q, recv_s);
}

int launch_unpack(const Dims& D, const Ws& W, const uint8_t* recv_q, const float* recv_s, uint8_t* x_q, float* x_s,
                  int* exp_off, int* row_src, int cus, hipStream_t st) {
  const int grid = stream_grid(kUnpackShape, cus, (int64_t)D.rows, kUpWaves);
  return launch("k_unpack", k_unpack, dim3(grid), dim3(kUpThreads), 0, st, D, W, recv_q, recv_s, x_q, x_s, exp_off,
                row_src);
}

}  // namespace moe
