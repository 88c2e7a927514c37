// Combine ("Enabling trillion-parameter models on AWS EFA": section
// "Introduction" -- combine returns the processed rows to their source and
// forms each token's weighted average; section "Dispatch and combine" --
// routing is already known from dispatch, rows go back with one contiguous
// write per peer and the receive side accumulates them into the output).
//
//   k_comb_send  one wave per 8 expert-major rows: comb[row_src[i]] = y[i]
//   k_comb_recv  one wave per token: fp32 sum over slots of w * y, bf16 out
//   k_copy16     plain streaming copy (measurement aid)
#include "moe_internal.h"

namespace moe {

constexpr int kCombRowsPerWave = 8;

__global__ __launch_bounds__(kThreads) void k_comb_send(Dims D, Ws W, const uint16_t* __restrict__ y,
                                                        const int* __restrict__ row_src, uint16_t* __restrict__ comb) {
  __shared__ int svp[kMaxN + 1];
  __shared__ int sbase[kMaxN + 1];
  for (int i = threadIdx.x; i <= D.N; i += kThreads) {
    svp[i] = W.vprefix[i];
    sbase[i] = W.base[i];
  }
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int total = svp[D.N];
  const int ncomb = D.N * D.TK;
  for (int g0 = (blockIdx.x * kWavesPerBlock + wv) * kCombRowsPerWave; g0 < total;
       g0 += gridDim.x * kWavesPerBlock * kCombRowsPerWave) {
    int src = -1, dst = -1;
    if (lane < kCombRowsPerWave && g0 + lane < total) {
      const int g = g0 + lane;
      int lo = 0, hi = D.N + 1;   // region of valid row g
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (svp[mid] <= g) lo = mid; else hi = mid;
      }
      const int p = sbase[lo] + (g - svp[lo]);
      if (p < D.rows) {
        const int rs = row_src[p];
        if (rs >= 0 && rs < ncomb) {
          src = p;
          dst = rs;
        }
      }
    }
    for (int r = 0; r < kCombRowsPerWave; ++r) {
      const int sr = __builtin_amdgcn_readlane(src, r);
      const int dr = __builtin_amdgcn_readlane(dst, r);
      if (sr < 0) continue;
      wave_copy16<8>(reinterpret_cast<uint4*>(comb + (int64_t)dr * D.H),
                      reinterpret_cast<const uint4*>(y + (int64_t)sr * D.H), D.H / 8, lane);
    }
  }
}

// acc = fl(acc + fl(w * y)) in slot order, never fused into an FMA.
__device__ __forceinline__ void acc_row8(float* acc, float w, const uint4& v) {
#pragma clang fp contract(off)
  const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float p0 = w * bf16_lo(wd[i]);
    const float p1 = w * bf16_hi(wd[i]);
    acc[2 * i] = acc[2 * i] + p0;
    acc[2 * i + 1] = acc[2 * i + 1] + p1;
  }
}

constexpr int kSlotGroup = 8;

__global__ __launch_bounds__(kThreads) void k_comb_recv(Dims D, const uint16_t* __restrict__ comb,
                                                        const int* __restrict__ send_pos,
                                                        const float* __restrict__ topk_w, uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int NT = D.N * D.T;
  for (int tok = blockIdx.x * kWavesPerBlock + wv; tok < NT; tok += gridDim.x * kWavesPerBlock) {
    const int s = tok / D.T;
    int row = -1;
    float wt = 0.0f;
    if (lane < D.k) {
      const int sp = send_pos[(int64_t)tok * D.k + lane];
      wt = topk_w[(int64_t)tok * D.k + lane];
      if (sp >= 0 && sp < D.TK) row = s * D.TK + sp;
    }
    uint16_t* orow = out + (int64_t)tok * D.H;
    for (int col = lane * 8; col < D.H; col += kWave * 8) {
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
      for (int j0 = 0; j0 < D.k; j0 += kSlotGroup) {
        uint4 v[kSlotGroup];
        int rr[kSlotGroup];
#pragma unroll
        for (int jj = 0; jj < kSlotGroup; ++jj) {
          const int j = j0 + jj;
          rr[jj] = j < D.k ? __builtin_amdgcn_readlane(row, j) : -1;
          if (rr[jj] >= 0) v[jj] = *reinterpret_cast<const uint4*>(comb + (int64_t)rr[jj] * D.H + col);
        }
#pragma unroll
        for (int jj = 0; jj < kSlotGroup; ++jj) {
          const int j = j0 + jj;
          const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wt), j < D.k ? j : 0));
          if (rr[jj] >= 0) acc_row8(acc, wj, v[jj]);
        }
      }
      uint4 o;
      o.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
      o.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
      o.z = f32_to_bf16_rne(acc[4]) | (f32_to_bf16_rne(acc[5]) << 16);
      o.w = f32_to_bf16_rne(acc[6]) | (f32_to_bf16_rne(acc[7]) << 16);
      *reinterpret_cast<uint4*>(orow + col) = o;
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_copy16(uint4* __restrict__ dst, const uint4* __restrict__ src, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

int launch_comb_send(const Dims& D, const Ws& W, const uint16_t* y, const int* row_src, uint16_t* comb, int grid,
                     hipStream_t st) {
  if (D.N * D.TK == 0) return MOE_OK;
  return launch("k_comb_send", k_comb_send, dim3(grid), dim3(kThreads), 0, st, D, W, y, row_src, comb);
}

int launch_comb_recv(const Dims& D, const uint16_t* comb, const int* send_pos, const float* w, uint16_t* out, int grid,
                     hipStream_t st) {
  if (D.N * D.T == 0) return MOE_OK;
  return launch("k_comb_recv", k_comb_recv, dim3(grid), dim3(kThreads), 0, st, D, comb, send_pos, w, out);
}

int launch_copy(void* dst, const void* src, int64_t n16, int grid, hipStream_t st) {
  if (n16 == 0) return MOE_OK;
  return launch("k_copy16", k_copy16, dim3(grid), dim3(kThreads), 0, st, reinterpret_cast<uint4*>(dst),
                reinterpret_cast<const uint4*>(src), n16);
}

}  // namespace moe
