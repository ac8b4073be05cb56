// api.hip -- the C interface (include/flash_attn.h): argument validation,
// dispatch and status codes. Validation happens before any HIP call, so a
// rejected call launches nothing and writes nothing.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "flash_attn.h"
#include "fa_launch.h"

// Scratch of flash_attn_bwd_noalloc: the backward pass's row statistics (D,
// then LSE * log2(e)), 2 * B * H * N floats, in a fixed device array instead of
// a caller's buffer. Each device that loads the library holds its own copy
// until the process ends. Host code never uses the name `scratch` as an
// address (on the host it is only a stand-in for the device symbol): the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) float scratch[FA_NOALLOC_MAX_ROWS * 2];

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by both forward entry points. Returns FA_OK with *empty set
// when there is nothing to compute.
int validate(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int H, int N,
             int d, float scale, int dtype, bool* empty) {
  *empty = false;
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if (B == 0 || H == 0 || N == 0) {
    *empty = true;
    return FA_OK;
  }
  if (!q || !k || !v || !o) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  // One grid dimension of at most 2^32 work-items; element offsets in 64 bits.
  const int64_t bh = (int64_t)B * H;
  const int64_t rows = fa::flash_rows_per_block(dtype, d);
  const int64_t blocks = bh * ((N + rows - 1) / rows);
  if (blocks * 256 >= ((int64_t)1 << 32) || blocks > INT32_MAX) return FA_ERR_SHAPE;
  return FA_OK;
}

fa::AttnArgs make_args(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                       int d, float scale, int dtype, void* stream) {
  fa::AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.scale = scale;
  a.dtype = dtype;
  a.stream = static_cast<hipStream_t>(stream);
  return a;
}

// Device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept; nullptr if the lookup fails.
float* scratch_ptr(hipError_t* err) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* ptr[kMaxDevices] = {};
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    ptr[dev] = static_cast<float*>(p);
  }
  return ptr[dev];
}

// Bytes one head occupies in the three-pass workspace, or 0 on overflow.
size_t naive_head_bytes(int N, int dtype) {
  const unsigned __int128 n = (unsigned)N;
  const unsigned __int128 b = n * n * (unsigned)(4 + fa::elem_bytes(dtype));
  return b > (unsigned __int128)SIZE_MAX ? 0 : (size_t)b;
}

}  // namespace

extern "C" {

int flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   float scale, int dtype, void* stream) {
  bool empty;
  const int st = validate(q, k, v, o, lse, B, H, N, d, scale, dtype, &empty);
  if (st != FA_OK || empty) return st;
  const hipError_t e = fa::launch_flash(make_args(q, k, v, o, lse, B, H, N, d, scale, dtype, stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int flash_attn_fwd_causal(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                          int d, float scale, int dtype, void* stream) {
  bool empty;
  const int st = validate(q, k, v, o, lse, B, H, N, d, scale, dtype, &empty);
  if (st != FA_OK || empty) return st;
  const hipError_t e = fa::launch_flash_causal(make_args(q, k, v, o, lse, B, H, N, d, scale, dtype, stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// Every check of the backward entry points except their row-statistics
// scratch. Returns FA_OK with *empty set when there is nothing to compute.
static int validate_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                        int dtype, bool* empty) {
  const int st = validate(q, k, v, dq, lse, B, H, N, d, scale, dtype, empty);
  if (st != FA_OK || *empty) return st;
  if (!o || !dout || !lse || !dk || !dv) return FA_ERR_NULL;
  if (!aligned16(o) || !aligned16(dout) || !aligned16(dk) || !aligned16(dv)) return FA_ERR_ALIGN;
  return FA_OK;
}

// Launch of a validated backward pass with row-statistics scratch `delta`.
static int launch_bwd_checked(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H, int N,
                              int d, float scale, int dtype, void* stream, bool causal) {
  fa::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.scale = scale;
  a.dtype = dtype;
  a.stream = static_cast<hipStream_t>(stream);
  const hipError_t e = fa::launch_bwd(a, causal);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

static int flash_attn_bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dout,
                               const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H, int N,
                               int d, float scale, int dtype, void* stream, bool causal) {
  bool empty;
  const int st = validate_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, dtype, &empty);
  if (st != FA_OK || empty) return st;
  if (!delta) return FA_ERR_NULL;
  if (!aligned16(delta)) return FA_ERR_ALIGN;
  return launch_bwd_checked(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, scale, dtype, stream, causal);
}

int flash_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, float* delta, int B, int H, int N, int d, float scale, int dtype,
                   void* stream) {
  return flash_attn_bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, scale, dtype, stream, false);
}

int flash_attn_bwd_causal(const void* q, const void* k, const void* v, const void* o, const void* dout,
                          const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H, int N, int d,
                          float scale, int dtype, void* stream) {
  return flash_attn_bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, scale, dtype, stream, true);
}

int flash_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                           int dtype, void* stream) {
  // Every check of flash_attn_bwd except the caller's scratch pointer, then
  // the size limit of the fixed scratch; all before any HIP call.
  bool empty;
  const int st = validate_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, dtype, &empty);
  if (st != FA_OK || empty) return st;
  if ((int64_t)B * H * N > FA_NOALLOC_MAX_ROWS) return FA_ERR_TOO_LARGE;
  hipError_t e;
  float* delta = scratch_ptr(&e);
  if (!delta) return FA_ERR_HIP;
  return launch_bwd_checked(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, scale, dtype, stream, false);
}

size_t attn_naive_workspace_bytes(int B, int H, int N, int dtype) {
  if (B < 0 || H < 0 || N < 0) return 0;
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return 0;
  const size_t head = naive_head_bytes(N, dtype);
  const unsigned __int128 all = (unsigned __int128)head * (unsigned)B * (unsigned)H;
  return all > (unsigned __int128)SIZE_MAX ? 0 : (size_t)all;
}

int attn_naive_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  bool empty;
  const int st = validate(q, k, v, o, lse, B, H, N, d, scale, dtype, &empty);
  if (st != FA_OK || empty) return st;
  const size_t head = naive_head_bytes(N, dtype);
  if (head == 0 || fa::naive_max_heads_per_launch(N, d, dtype) < 1) return FA_ERR_SHAPE;
  if (!workspace) return FA_ERR_NULL;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  if (workspace_bytes < head) return FA_ERR_WORKSPACE;
  const hipError_t e =
      fa::launch_naive(make_args(q, k, v, o, lse, B, H, N, d, scale, dtype, stream), workspace, workspace_bytes);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid or too large shape";
    case FA_ERR_UNSUPPORTED: return "unsupported dtype or head size";
    case FA_ERR_ALIGN: return "pointer is not 16-byte aligned";
    case FA_ERR_WORKSPACE: return "workspace smaller than one head";
    case FA_ERR_SCALE: return "scale is not finite";
    case FA_ERR_HIP: return "HIP launch error";
    case FA_ERR_TOO_LARGE: return "B*H*N exceeds the fixed scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

}  // extern "C"
