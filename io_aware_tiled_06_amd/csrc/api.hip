// api.hip -- the C interface (include/flash_attn.h): argument validation,
// dispatch and status codes. Validation happens before any HIP call, so a
// rejected call launches nothing and writes nothing.
#include <math.h>
#include <stdint.h>

#include "flash_attn.h"
#include "fa_launch.h"

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

static int flash_attn_bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dout,
                               const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H, int N,
                               int d, float scale, int dtype, void* stream, bool causal) {
  bool empty;
  const int st = validate(q, k, v, dq, lse, B, H, N, d, scale, dtype, &empty);
  if (st != FA_OK || empty) return st;
  if (!o || !dout || !lse || !dk || !dv || !delta) return FA_ERR_NULL;
  if (!aligned16(o) || !aligned16(dout) || !aligned16(dk) || !aligned16(dv) || !aligned16(delta))
    return FA_ERR_ALIGN;
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
    default: return "unknown status";
  }
}

}  // extern "C"
