// Host side of the C ABI declared in include/moe_ep.h: argument checks,
// workspace carving, grid sizing and launches on the caller's stream.
#include <mutex>

#include "moe_internal.h"

namespace moe {

__global__ void k_fill_u32(uint32_t* __restrict__ p, uint32_t v, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = v;
}

int launch_fill_u32(uint32_t* p, uint32_t v, int n, hipStream_t st) {
  return launch("k_fill_u32", k_fill_u32, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, st, p, v, n);
}

__global__ void k_copy_u32(uint32_t* __restrict__ dst, const uint32_t* __restrict__ src) { *dst = *src; }

namespace {

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shape checks shared by every entry point; fills the derived sizes.
int make_dims(const moe_shape* sh, Dims* D) {
  if (!sh) return MOE_ENULL;
  const moe_shape& s = *sh;
  if (s.early_rows < 0) return MOE_EINVAL;
  if (s.early_rows > 0 && (s.region_rows == 0 || (int64_t)s.N * s.early_rows > s.region_rows)) return MOE_EINVAL;
  if (s.N < 1 || s.N > kMaxN) return MOE_EINVAL;
  if (s.T < 0) return MOE_EINVAL;
  if (s.H < kScaleBlock || s.H > kMaxH || s.H % kScaleBlock) return MOE_EINVAL;
  if (s.E < 1 || s.E > kMaxE || s.E % s.N) return MOE_EINVAL;
  if (s.k < 1 || s.k > kMaxK || s.k > s.E) return MOE_EINVAL;
  if (s.region_rows < 0) return MOE_EINVAL;
  const int64_t tk = (int64_t)s.T * s.k;
  const int64_t slots = tk * s.N;
  if (slots > INT32_MAX) return MOE_ERANGE;
  const int64_t rows = s.region_rows ? (int64_t)s.N * s.region_rows : slots;
  if (rows > INT32_MAX) return MOE_ERANGE;
  D->N = s.N;
  D->T = s.T;
  D->H = s.H;
  D->E = s.E;
  D->k = s.k;
  D->L = s.E / s.N;
  D->TK = (int)tk;
  // A rank that fits one chunk (<= 4096 slots) gets exactly one, so the count
  // kernel finishes its positions; larger ranks get the smallest power-of-two
  // chunk (256..4096 slots) that keeps their chunks at 32 or fewer.
  int C = kMinChunk;
  if (tk <= kMaxChunk) {
    while (C < tk) C *= 2;
  } else {
    while (C < kMaxChunk && (tk + C - 1) / C > 32) C *= 2;
  }
  D->C = C;
  D->B = (int)((tk + C - 1) / C);
  D->NB = s.H / kScaleBlock;
  D->R = (int)s.region_rows;
  D->Ce = s.early_rows;
  D->rows = (int)rows;
  D->bound = (int64_t)s.N * s.T * (s.k > D->L ? s.k : D->L);
  return MOE_OK;
}

constexpr size_t kAlign = 256;
inline size_t up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// Carve the workspace; returns its total size.  ws may be NULL (sizing only).
// tables_only: only what the multi-launch direct dispatch uses (no unpack
// row map, no exchange area of the single-launch calls).
size_t carve(const Dims& D, void* ws, Ws* W, bool tables_only = false) {
  char* b = static_cast<char*>(ws);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    char* p = b ? b + o : nullptr;
    o += up(bytes);
    return p;
  };
  char* hdr = take(kAlign);
  W->err = reinterpret_cast<uint32_t*>(hdr);
  W->blk = reinterpret_cast<int*>(take(sizeof(int) * (size_t)D.N * D.B * D.E));
  W->cnt = reinterpret_cast<int*>(take(sizeof(int) * (size_t)D.N * D.E));
  W->send_off = reinterpret_cast<int*>(take(sizeof(int) * (size_t)D.N * (D.E + 1)));
  W->recv_off = reinterpret_cast<int*>(take(sizeof(int) * (size_t)D.N * (D.N + 1)));
  W->recv_total = reinterpret_cast<int*>(take(sizeof(int) * (size_t)D.N));
  W->base = reinterpret_cast<int*>(take(sizeof(int) * (size_t)(D.N + 1)));
  W->vprefix = reinterpret_cast<int*>(take(sizeof(int) * (size_t)(D.N + 1)));
  W->exp_off = reinterpret_cast<int*>(take(sizeof(int) * (size_t)D.N * (D.L + 1)));
  W->src_in_exp = reinterpret_cast<int*>(take(sizeof(int) * (size_t)(D.N + 1) * D.E));
  W->local = reinterpret_cast<int*>(take(D.B > 1 ? sizeof(int) * (size_t)D.N * D.TK : 0));
  W->umap = reinterpret_cast<int2*>(take(tables_only ? 0 : sizeof(int2) * (size_t)D.rows));
  // Exchange area of the single-launch dispatch (one routing chunk per rank
  // only), last so that moe_workspace_init clears it with the header.
  const bool ll = D.B == 1 && !tables_only;
  auto take64 = [&](size_t n) { return reinterpret_cast<uint64_t*>(take(ll ? sizeof(uint64_t) * n : 0)); };
  W->ctl = reinterpret_cast<uint32_t*>(take(ll ? sizeof(uint32_t) * (kCtlGroups + 1) * kCtlStride : 0));
  W->tpos = take64((size_t)D.N * D.TK);
  W->toff = take64((size_t)D.N * (D.N + 1));
  W->tcnt = take64((size_t)D.N * D.E);
  W->trel = take64((size_t)D.N * D.N);
  W->tbase = take64((size_t)D.N);
  W->tcdone = take64((size_t)D.N * kReadyStride);
  W->temr = take64((size_t)D.N * D.E);
  W->tlim = take64((size_t)D.N * D.N);
  W->tcold = take64((size_t)D.N * kReadyStride);
  return o;
}


// Compute units of the current device, cached per device.
int device_cus() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> g(mu);
  if (!cache[dev]) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

inline Ws W_of(const Dims& D, void* ws) {
  Ws W;
  carve(D, ws, &W);
  return W;
}

// The workspace of moe_dispatch_direct_noalloc: a file-scope device array,
// one copy on every GPU the library runs on, held until the process ends.
// Host code never uses the array's name as an address: the device address
// comes from hipGetSymbolAddress, once per device (scratch_address).
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of the current device's `scratch`, looked up on the first
// call on that device (with the device current) and kept per device.
int scratch_address(void** out) {
  static std::mutex mu;
  static void* cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_EHIP;
  std::lock_guard<std::mutex> g(mu);
  if (!cache[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      fprintf(stderr, "libmoe_ep: hipGetSymbolAddress(scratch) failed on device %d: %s\n", dev,
              hipGetErrorString(e));
      return MOE_EHIP;
    }
    cache[dev] = p;
  }
  *out = cache[dev];
  return MOE_OK;
}

// The direct dispatch on a carved workspace: routing, then the pack into the
// expert-major rows (or, without tokens, only the layout).
int direct_dispatch(const Dims& D, const Ws& W, const uint16_t* tokens, const int32_t* topk_idx, uint8_t* x_q,
                    float* x_s, int32_t* send_pos, int32_t* exp_off, int32_t* row_src, hipStream_t st) {
  int rc = launch_route(D, W, topk_idx, send_pos, st);
  if (rc) return rc;
  if (D.T == 0)   // the layout-only receive half writes exp_off
    return launch_unpack(D, W, nullptr, nullptr, nullptr, nullptr, exp_off, row_src, device_cus(), st);
  return launch_pack(D, W, tokens, topk_idx, send_pos, x_q, x_s, row_src, exp_off, device_cus(), st);
}

// Host checks of moe_dispatch_direct's arguments (the workspace apart).
int direct_args(const Dims& D, const uint16_t* tokens, const int32_t* topk_idx, const uint8_t* x_q, const float* x_s,
                const int32_t* send_pos, const int32_t* exp_off, const int32_t* row_src) {
  if (!exp_off) return MOE_ENULL;
  if (!aligned(exp_off, 4)) return MOE_EALIGN;
  if (D.T == 0) return MOE_OK;   // empty arrays may be NULL
  if (!topk_idx || !send_pos || !row_src) return MOE_ENULL;
  if (tokens && (!x_q || !x_s)) return MOE_ENULL;
  if (!aligned(topk_idx, 4) || !aligned(send_pos, 4) || !aligned(row_src, 4)) return MOE_EALIGN;
  if (tokens && (!aligned(tokens, 16) || !aligned(x_q, 16) || !aligned(x_s, 4))) return MOE_EALIGN;
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

int64_t moe_recv_rows(const moe_shape* shape) {
  Dims D;
  const int rc = make_dims(shape, &D);
  return rc ? rc : D.rows;
}

int64_t moe_workspace_bytes(const moe_shape* shape) {
  Dims D;
  const int rc = make_dims(shape, &D);
  if (rc) return rc;
  Ws W;
  return (int64_t)carve(D, nullptr, &W);
}

int moe_workspace_init(const moe_shape* shape, void* ws, void* stream) {
  Dims D;
  int rc = make_dims(shape, &D);
  if (rc) return rc;
  if (!ws) return MOE_ENULL;
  if (!aligned(ws, kAlign)) return MOE_EALIGN;
  hipStream_t st = as_stream(stream);
  rc = launch_fill_u32(static_cast<uint32_t*>(ws), 0u, (int)(kAlign / sizeof(uint32_t)), st);
  if (rc || D.B != 1) return rc;
  Ws W;
  const size_t total = carve(D, ws, &W);
  const size_t x0 = static_cast<size_t>(reinterpret_cast<char*>(W.ctl) - static_cast<char*>(ws));
  return launch_fill_u32(W.ctl, 0u, (int)((total - x0) / sizeof(uint32_t)), st);
}

int moe_dispatch_send(const moe_shape* shape, const uint16_t* tokens, const int32_t* topk_idx, uint8_t* recv_q,
                      float* recv_s, int32_t* send_pos, void* ws, void* stream) {
  Dims D;
  int rc = make_dims(shape, &D);
  if (rc) return rc;
  if (!ws) return MOE_ENULL;
  if (!aligned(ws, kAlign)) return MOE_EALIGN;
  if (D.T == 0) return launch_route(D, W_of(D, ws), topk_idx, send_pos, as_stream(stream));   // empty arrays may be NULL
  if (!topk_idx || !send_pos) return MOE_ENULL;
  if (tokens && (!recv_q || !recv_s)) return MOE_ENULL;
  if (!aligned(ws, kAlign) || !aligned(topk_idx, 4) || !aligned(send_pos, 4)) return MOE_EALIGN;
  if (tokens && (!aligned(tokens, 16) || !aligned(recv_q, 16) || !aligned(recv_s, 4))) return MOE_EALIGN;
  Ws W;
  carve(D, ws, &W);
  hipStream_t st = as_stream(stream);
  rc = launch_route(D, W, topk_idx, send_pos, st);
  if (rc) return rc;
  return launch_pack(D, W, tokens, topk_idx, send_pos, recv_q, recv_s, nullptr, nullptr, device_cus(), st);
}

int moe_dispatch_direct(const moe_shape* shape, const uint16_t* tokens, const int32_t* topk_idx, uint8_t* x_q,
                        float* x_s, int32_t* send_pos, int32_t* exp_off, int32_t* row_src, void* ws, void* stream) {
  Dims D;
  int rc = make_dims(shape, &D);
  if (rc) return rc;
  if (!ws) return MOE_ENULL;
  if (!aligned(ws, kAlign)) return MOE_EALIGN;
  rc = direct_args(D, tokens, topk_idx, x_q, x_s, send_pos, exp_off, row_src);
  if (rc) return rc;
  return direct_dispatch(D, W_of(D, ws), tokens, topk_idx, x_q, x_s, send_pos, exp_off, row_src, as_stream(stream));
}

int moe_dispatch_direct_noalloc(const moe_shape* shape, const uint16_t* tokens, const int32_t* topk_idx,
                                uint8_t* x_q, float* x_s, int32_t* send_pos, int32_t* exp_off, int32_t* row_src,
                                uint32_t* flags, void* stream) {
  Dims D;
  int rc = make_dims(shape, &D);
  if (rc) return rc;
  Ws W;
  const size_t need = carve(D, nullptr, &W, true);
  if (need > kScratchBytes) {
    fprintf(stderr, "libmoe_ep: moe_dispatch_direct_noalloc needs %zu bytes of routing tables for this shape, "
                    "more than its %zu-byte scratch\n", need, kScratchBytes);
    return MOE_ERANGE;
  }
  if (!flags) return MOE_ENULL;
  if (!aligned(flags, 4)) return MOE_EALIGN;
  rc = direct_args(D, tokens, topk_idx, x_q, x_s, send_pos, exp_off, row_src);
  if (rc) return rc;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc) return rc;
  carve(D, ws, &W, true);
  hipStream_t st = as_stream(stream);
  // The error word starts at zero for this call (a fill kernel rather than a
  // memset, so the call can be captured in a graph).
  rc = launch_fill_u32(W.err, 0u, 1, st);
  if (rc) return rc;
  rc = direct_dispatch(D, W, tokens, topk_idx, x_q, x_s, send_pos, exp_off, row_src, st);
  if (rc) return rc;
  return launch("k_copy_u32", k_copy_u32, dim3(1), dim3(1), 0, st, flags, static_cast<const uint32_t*>(W.err));
}

int moe_dispatch_send_ll(const moe_shape* shape, const uint16_t* tokens, const int32_t* topk_idx, uint8_t* recv_q,
                         float* recv_s, int32_t* send_pos, void* ws, void* stream) {
  Dims D;
  int rc = make_dims(shape, &D);
  if (rc) return rc;
  if (!ws) return MOE_ENULL;
  if (!aligned(ws, kAlign)) return MOE_EALIGN;
  if (D.T == 0) return launch_route(D, W_of(D, ws), topk_idx, send_pos, as_stream(stream));   // nothing to exchange
  if (D.B != 1) return MOE_EINVAL;   // more than one routing chunk per rank
  if (!topk_idx || !send_pos) return MOE_ENULL;
  if (tokens && (!recv_q || !recv_s)) return MOE_ENULL;
  if (!aligned(topk_idx, 4) || !aligned(send_pos, 4)) return MOE_EALIGN;
  if (tokens && (!aligned(tokens, 16) || !aligned(recv_q, 16) || !aligned(recv_s, 4))) return MOE_EALIGN;
  return launch_dispatch_ll(D, W_of(D, ws), tokens, topk_idx, send_pos, recv_q, recv_s, nullptr, nullptr,
                            device_cus(), as_stream(stream));
}

int moe_dispatch_direct_ll(const moe_shape* shape, const uint16_t* tokens, const int32_t* topk_idx, uint8_t* x_q,
                           float* x_s, int32_t* send_pos, int32_t* exp_off, int32_t* row_src, void* ws,
                           void* stream) {
  Dims D;
  int rc = make_dims(shape, &D);
  if (rc) return rc;
  if (!ws || !exp_off) return MOE_ENULL;
  if (!aligned(ws, kAlign) || !aligned(exp_off, 4)) return MOE_EALIGN;
  hipStream_t st = as_stream(stream);
  Ws W;
  carve(D, ws, &W);
  if (D.T == 0) {   // nothing to exchange; empty arrays may be NULL
    rc = launch_route(D, W, topk_idx, send_pos, st);
    return rc ? rc : launch_unpack(D, W, nullptr, nullptr, nullptr, nullptr, exp_off, row_src, device_cus(), st);
  }
  if (D.B != 1) return MOE_EINVAL;   // more than one routing chunk per rank
  if (!topk_idx || !send_pos || !row_src) return MOE_ENULL;
  if (tokens && (!x_q || !x_s)) return MOE_ENULL;
  if (!aligned(topk_idx, 4) || !aligned(send_pos, 4) || !aligned(row_src, 4)) return MOE_EALIGN;
  if (tokens && (!aligned(tokens, 16) || !aligned(x_q, 16) || !aligned(x_s, 4))) return MOE_EALIGN;
  return launch_dispatch_ll(D, W, tokens, topk_idx, send_pos, x_q, x_s, row_src, exp_off, device_cus(), st);
}

int moe_dispatch_recv(const moe_shape* shape, const uint8_t* recv_q, const float* recv_s, const void* ws,
                      uint8_t* x_q, float* x_s, int32_t* exp_off, int32_t* row_src, void* stream) {
  Dims D;
  int rc = make_dims(shape, &D);
  if (rc) return rc;
  if (!ws || !exp_off || (!row_src && D.T > 0)) return MOE_ENULL;
  const bool payload = recv_q || recv_s || x_q || x_s;
  if (payload && D.T > 0 && (!recv_q || !recv_s || !x_q || !x_s)) return MOE_ENULL;
  if (!aligned(ws, kAlign) || !aligned(exp_off, 4) || !aligned(row_src, 4)) return MOE_EALIGN;
  if (payload && (!aligned(recv_q, 16) || !aligned(x_q, 16) || !aligned(recv_s, 4) || !aligned(x_s, 4)))
    return MOE_EALIGN;
  Ws W;
  carve(D, const_cast<void*>(ws), &W);
  return launch_unpack(D, W, recv_q, recv_s, x_q, x_s, exp_off, row_src, device_cus(), as_stream(stream));
}

int moe_combine_send(const moe_shape* shape, const uint16_t* y_em, const int32_t* row_src, const void* ws,
                     uint16_t* comb, void* stream) {
  Dims D;
  int rc = make_dims(shape, &D);
  if (rc) return rc;
  if (!ws) return MOE_ENULL;
  if (D.T == 0) return MOE_OK;
  if (!y_em || !row_src || !comb) return MOE_ENULL;
  if (!aligned(y_em, 16) || !aligned(comb, 16) || !aligned(row_src, 4) || !aligned(ws, kAlign)) return MOE_EALIGN;
  Ws W;
  carve(D, const_cast<void*>(ws), &W);
  return launch_comb_send(D, W, y_em, row_src, comb, device_cus(), as_stream(stream));
}

int moe_combine_recv(const moe_shape* shape, const uint16_t* comb, const int32_t* send_pos, const float* topk_w,
                     uint16_t* out, void* stream) {
  Dims D;
  int rc = make_dims(shape, &D);
  if (rc) return rc;
  if (D.T == 0) return MOE_OK;
  if (!comb || !send_pos || !topk_w || !out) return MOE_ENULL;
  if (!aligned(comb, 16) || !aligned(out, 16) || !aligned(send_pos, 4) || !aligned(topk_w, 4)) return MOE_EALIGN;
  return launch_comb_recv(D, comb, send_pos, topk_w, out, device_cus(),
                          as_stream(stream));
}

int moe_combine_pull(const moe_shape* shape, const uint16_t* y_em, const int32_t* topk_idx, const int32_t* send_pos,
                     const float* topk_w, const void* ws, uint16_t* out, void* stream) {
  Dims D;
  int rc = make_dims(shape, &D);
  if (rc) return rc;
  if (!ws) return MOE_ENULL;
  if (!aligned(ws, kAlign)) return MOE_EALIGN;
  if (D.T == 0) return MOE_OK;
  if (!y_em || !topk_idx || !send_pos || !topk_w || !out) return MOE_ENULL;
  if (!aligned(y_em, 16) || !aligned(out, 16) || !aligned(topk_idx, 4) || !aligned(send_pos, 4) ||
      !aligned(topk_w, 4))
    return MOE_EALIGN;
  Ws W;
  carve(D, const_cast<void*>(ws), &W);
  return launch_comb_pull(D, W, y_em, topk_idx, send_pos, topk_w, out, device_cus(), as_stream(stream));
}

int moe_combine_send_partial(const moe_shape* shape, const uint16_t* y_em, const int32_t* topk_idx,
                             const int32_t* send_pos, const float* topk_w, const void* ws, uint16_t* comb,
                             void* stream) {
  Dims D;
  int rc = make_dims(shape, &D);
  if (rc) return rc;
  if (!ws) return MOE_ENULL;
  if (!aligned(ws, kAlign)) return MOE_EALIGN;
  if (D.T == 0) return MOE_OK;
  if (!y_em || !topk_idx || !send_pos || !topk_w || !comb) return MOE_ENULL;
  if (!aligned(y_em, 16) || !aligned(comb, 16) || !aligned(topk_idx, 4) || !aligned(send_pos, 4) ||
      !aligned(topk_w, 4))
    return MOE_EALIGN;
  return launch_comb_send_partial(D, W_of(D, const_cast<void*>(ws)), y_em, topk_idx, send_pos, topk_w, comb,
                                  device_cus(), as_stream(stream));
}

int moe_combine_recv_partial(const moe_shape* shape, const uint16_t* comb, const int32_t* topk_idx,
                             const int32_t* send_pos, const void* ws, uint16_t* out, void* stream) {
  Dims D;
  int rc = make_dims(shape, &D);
  if (rc) return rc;
  if (!ws) return MOE_ENULL;
  if (!aligned(ws, kAlign)) return MOE_EALIGN;
  if (D.T == 0) return MOE_OK;
  if (!comb || !topk_idx || !send_pos || !out) return MOE_ENULL;
  if (!aligned(comb, 16) || !aligned(out, 16) || !aligned(topk_idx, 4) || !aligned(send_pos, 4)) return MOE_EALIGN;
  return launch_comb_recv_partial(D, W_of(D, const_cast<void*>(ws)), comb, topk_idx, send_pos, out, device_cus(),
                                  as_stream(stream));
}

int moe_status(void* ws, void* stream, uint32_t* flags) {
  if (!ws || !flags) return MOE_ENULL;
  if (!aligned(ws, kAlign)) return MOE_EALIGN;
  hipStream_t st = as_stream(stream);
  uint32_t h = 0;
  if (hipMemcpyAsync(&h, ws, sizeof(h), hipMemcpyDeviceToHost, st) != hipSuccess) return MOE_EHIP;
  if (hipStreamSynchronize(st) != hipSuccess) return MOE_EHIP;
  int rc = launch_fill_u32(static_cast<uint32_t*>(ws), 0u, 1, st);
  if (rc) return rc;
  *flags = h;
  return MOE_OK;
}

int moe_layout_export(const moe_shape* shape, const void* ws, int32_t* cnt, int32_t* send_off, int32_t* recv_off,
                      int32_t* recv_total, int32_t* base, void* stream) {
  Dims D;
  int rc = make_dims(shape, &D);
  if (rc) return rc;
  if (!ws) return MOE_ENULL;
  if (!aligned(ws, kAlign)) return MOE_EALIGN;
  Ws W;
  carve(D, const_cast<void*>(ws), &W);
  hipStream_t st = as_stream(stream);
  struct Item {
    int32_t* dst;
    const int* src;
    size_t n;
  } items[] = {{cnt, W.cnt, (size_t)D.N * D.E},
               {send_off, W.send_off, (size_t)D.N * (D.E + 1)},
               {recv_off, W.recv_off, (size_t)D.N * (D.N + 1)},
               {recv_total, W.recv_total, (size_t)D.N},
               {base, W.base, (size_t)D.N + 1}};
  for (const Item& it : items) {
    if (!it.dst) continue;
    if (hipMemcpyAsync(it.dst, it.src, it.n * sizeof(int32_t), hipMemcpyDeviceToDevice, st) != hipSuccess)
      return MOE_EHIP;
  }
  return MOE_OK;
}

}  // extern "C"
