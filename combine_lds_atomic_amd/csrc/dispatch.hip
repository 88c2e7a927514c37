// Dispatch data movement ("Enabling trillion-parameter models on AWS EFA",
// sections "Send and receive buffers", "Dispatch and combine", and
// "Evaluation: dispatch/combine latency" for the block-scaled fp8 payload).
//
//   k_pack    one wave per token: final slot positions, block-128 amax with
//             DPP, fp8 quantisation, and k 16-byte row stores straight into
//             the destination ranks' receive regions (the "remote write").
//   k_unpack  one wave per 8 expert-major rows: the receive side finds each
//             row's (expert, source) segment from the exchanged counts alone
//             and copies it out of the source-major receive region.
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(kThreads) void k_pack(Dims D, Ws W, const uint16_t* __restrict__ x,
                                                   const int* __restrict__ idx, int* __restrict__ send_pos,
                                                   uint8_t* __restrict__ recv_q, float* __restrict__ recv_s) {
  __shared__ float sscale[kWavesPerBlock][kMaxNB];
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int NT = D.N * D.T;
  for (int tok = blockIdx.x * kWavesPerBlock + wv; tok < NT; tok += gridDim.x * kWavesPerBlock) {
    const int s = tok / D.T, t = tok - s * D.T;
    // Lane j < k resolves slot j: position = chunk base of its expert + rank
    // inside the chunk (left in send_pos by the count kernel).
    int row = -1;
    if (lane < D.k) {
      const int i = t * D.k + lane;
      const int64_t slot = (int64_t)s * D.TK + i;
      const int e = idx[slot];
      if (e >= 0 && e < D.E) {
        const int sp = W.blk[((int64_t)s * D.B + i / kChunk) * D.E + e] + send_pos[slot];
        send_pos[slot] = sp;
        const int d = e / D.L;
        const int r = W.recv_off[d * (D.N + 1) + s] + sp - W.send_off[s * (D.E + 1) + d * D.L];
        const int pr = W.base[d] + r;
        if ((D.R == 0 || r < D.R) && r >= 0 && pr < D.rows) row = pr;
      }
    }
    if (x == nullptr) continue;

    const uint16_t* xr = x + (int64_t)tok * D.H;
    for (int c0 = 0; c0 < D.H; c0 += kWave * 16) {
      const int col = c0 + lane * 16;          // this lane's 16 elements
      const bool act = col < D.H;              // whole 8-lane groups drop out together
      uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
      if (act) {
        a = *reinterpret_cast<const uint4*>(xr + col);
        b = *reinterpret_cast<const uint4*>(xr + col + 8);
      }
      const uint32_t wds[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      float v[16];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[2 * i] = bf16_lo(wds[i]);
        v[2 * i + 1] = bf16_hi(wds[i]);
      }
      int am = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) am = max(am, (int)(__float_as_uint(v[i]) & 0x7FFFFFFFu));
      am = max8_lanes(am);                     // amax of the 128-element block
      const float amax = __uint_as_float((uint32_t)am);
      const float scale = amax / 448.0f;       // IEEE division, round to nearest even
      uint32_t q[4] = {0, 0, 0, 0};
      if (amax != 0.0f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          q[i] = f32_to_e4m3fn(v[4 * i] / scale) | (f32_to_e4m3fn(v[4 * i + 1] / scale) << 8) |
                 (f32_to_e4m3fn(v[4 * i + 2] / scale) << 16) | (f32_to_e4m3fn(v[4 * i + 3] / scale) << 24);
        }
      }
      if (act && (lane & 7) == 0) sscale[wv][col / kScaleBlock] = amax != 0.0f ? scale : 0.0f;
      const uint4 qv = make_uint4(q[0], q[1], q[2], q[3]);
      for (int j = 0; j < D.k; ++j) {
        const int rj = __builtin_amdgcn_readlane(row, j);
        if (rj >= 0 && act) *reinterpret_cast<uint4*>(recv_q + (int64_t)rj * D.H + col) = qv;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    for (int bi = lane; bi < D.NB; bi += kWave) {
      const float sc = sscale[wv][bi];
      for (int j = 0; j < D.k; ++j) {
        const int rj = __builtin_amdgcn_readlane(row, j);
        if (rj >= 0) recv_s[(int64_t)rj * D.NB + bi] = sc;
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

constexpr int kRowsPerWave = 8;

__global__ __launch_bounds__(kThreads) void k_unpack(Dims D, Ws W, const uint8_t* __restrict__ recv_q,
                                                     const float* __restrict__ recv_s, uint8_t* __restrict__ x_q,
                                                     float* __restrict__ x_s, int* __restrict__ exp_off,
                                                     int* __restrict__ row_src) {
  __shared__ int svp[kMaxN + 1];
  for (int i = threadIdx.x; i <= D.N; i += kThreads) svp[i] = W.vprefix[i];
  if (blockIdx.x == 0)   // per-expert offsets for the grouped GEMM, as computed by the scan
    for (int i = threadIdx.x; i < D.N * (D.L + 1); i += kThreads) exp_off[i] = W.exp_off[i];
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int total = svp[D.N];
  const int N = D.N, E = D.E, L = D.L;
  for (int g0 = (blockIdx.x * kWavesPerBlock + wv) * kRowsPerWave; g0 < total;
       g0 += gridDim.x * kWavesPerBlock * kRowsPerWave) {
    int src = -1, dst = -1;
    if (lane < kRowsPerWave && g0 + lane < total) {
      const int g = g0 + lane;
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
    for (int r = 0; r < kRowsPerWave; ++r) {
      const int sr = __builtin_amdgcn_readlane(src, r);
      const int dr = __builtin_amdgcn_readlane(dst, r);
      if (sr < 0 || dr < 0) continue;
      wave_copy16<8>(reinterpret_cast<uint4*>(x_q + (int64_t)dr * D.H),
                     reinterpret_cast<const uint4*>(recv_q + (int64_t)sr * D.H), D.H / 16, lane);
      for (int c = lane; c < D.NB; c += kWave) x_s[(int64_t)dr * D.NB + c] = recv_s[(int64_t)sr * D.NB + c];
    }
  }
}

int launch_pack(const Dims& D, const Ws& W, const uint16_t* x, const int* idx, int* send_pos, uint8_t* recv_q,
                float* recv_s, int grid, hipStream_t st) {
  if (D.N * D.T == 0) return MOE_OK;
  return launch("k_pack", k_pack, dim3(grid), dim3(kThreads), 0, st, D, W, x, idx, send_pos, recv_q, recv_s);
}

int launch_unpack(const Dims& D, const Ws& W, const uint8_t* recv_q, const float* recv_s, uint8_t* x_q, float* x_s,
                  int* exp_off, int* row_src, int grid, hipStream_t st) {
  return launch("k_unpack", k_unpack, dim3(grid), dim3(kThreads), 0, st, D, W, recv_q, recv_s, x_q, x_s, exp_off,
                row_src);
}

}  // namespace moe
