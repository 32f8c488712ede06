// C ABI of the attention library: argument validation (host only, before any
// HIP call), kernel selection and launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/fa.h"
#include "fa_launch.h"

namespace {

thread_local char g_hip_error[256] = "no HIP error recorded";

bool debug_sync() {
  static const bool on = [] {
    const char* e = std::getenv("FA_DEBUG");
    return e && e[0] && e[0] != '0';
  }();
  return on;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  std::snprintf(g_hip_error, sizeof g_hip_error, "HIP error %d: %s", (int)e, hipGetErrorString(e));
  return FA_ERR_HIP;
}

int finish(hipError_t e, void* stream) {
  if (e != hipSuccess) return hip_status(e);
  if (debug_sync()) {
    e = hipStreamSynchronize((hipStream_t)stream);
    if (e == hipSuccess) e = hipGetLastError();
    return hip_status(e);
  }
  return FA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_fwd(const void* q, const void* k, const void* v, const void* o, const void* lse, int B, int Hq,
              int Hkv, int N, int d, int causal, float scale, bool* empty) {
  if (B < 0 || N < 0 || Hq < 1 || Hkv < 1 || d < 1) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  // sizes must fit the kernels' 32-bit grid arithmetic
  if ((long long)B * Hq * ((N + 63) / 64) > 0x7fffffffLL) return FA_ERR_SHAPE;
  *empty = (B == 0 || N == 0);
  if (*empty) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int N,
           int d, int causal, float scale, void* stream) {
  bool empty = false;
  const int st = check_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, &empty);
  if (st != FA_OK || empty) return st;
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, d, causal != 0, scale, stream};
  return finish(fa::launch_fwd_bf16(a), stream);
}

int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int N,
              int d, int causal, float scale, int window, const float* alibi_slopes, void* stream) {
  bool empty = false;
  const int st = check_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, &empty);
  if (st != FA_OK) return st;
  if (window < 0) return FA_ERR_SHAPE;
  if (window > 0 && !causal) return FA_ERR_UNSUPPORTED;
  if (empty) return FA_OK;
  if (alibi_slopes && ((uintptr_t)alibi_slopes & 3u) != 0) return FA_ERR_ALIGN;
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, d, causal != 0, scale, stream, window, alibi_slopes};
  return finish(fa::launch_fwd_bf16(a), stream);
}

int fa_prefill_paged(const void* q, const void* kpages, const void* vpages, const int32_t* page_table,
                     const int32_t* ctx_lens, void* o, float* lse, int num_seqs, int Hq, int Hkv, int d, int chunk,
                     int page_size, int max_pages_per_seq, int num_pages, float scale, void* stream) {
  if (num_seqs < 0 || chunk < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_pages_per_seq < 1 || num_pages < 1)
    return FA_ERR_SHAPE;
  if ((long long)num_seqs * Hq * ((chunk + 255) / 256) > 0x7fffffffLL) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (page_size != 16) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if (num_seqs == 0 || chunk == 0) return FA_OK;
  if (!q || !kpages || !vpages || !page_table || !ctx_lens || !o || !lse) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(kpages) || !aligned16(vpages) || !aligned16(page_table) ||
      !aligned16(ctx_lens) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  fa::FwdArgs a{q, kpages, vpages, o, lse, num_seqs, Hq, Hkv, chunk, d, true, scale, stream};
  a.page_table = page_table;
  a.ctx_lens = ctx_lens;
  a.max_pages = max_pages_per_seq;
  return finish(fa::launch_prefill_paged(a), stream);
}

size_t fa_bwd_workspace_size(int B, int Hq, int Hkv, int N, int d) {
  if (B < 0 || N < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || (d != 64 && d != 128)) return 0;
  return fa::bwd_plan(B, Hq, Hkv, N, d).bytes;
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
           void* dk, void* dv, int B, int Hq, int Hkv, int N, int d, int causal, float scale, void* workspace,
           size_t workspace_bytes, void* stream) {
  bool empty = false;
  int st = check_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, &empty);
  if (st != FA_OK || empty) return st;
  if (!dout || !dq || !dk || !dv) return FA_ERR_NULL;
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv)) return FA_ERR_ALIGN;
  const fa::BwdPlan pl = fa::bwd_plan(B, Hq, Hkv, N, d);
  if (!workspace || workspace_bytes < pl.bytes) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  fa::BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, causal != 0, scale, workspace, stream};
  return finish(fa::launch_bwd_bf16(a), stream);
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int Hq, int Hkv,
               int N, int d, int causal, float scale, void* stream) {
  bool empty = false;
  const int st = check_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, &empty);
  if (st != FA_OK || empty) return st;
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, d, causal != 0, scale, stream};
  return finish(fa::launch_fwd_f32(a), stream);
}

size_t fa_decode_paged_workspace_size(int num_seqs, int Hq, int d, int max_pages_per_seq, int page_size) {
  if (num_seqs < 0 || Hq < 1 || max_pages_per_seq < 1) return 0;
  if (d != 64 && d != 128) return 0;
  if (page_size != 16) return 0;
  return fa::decode_workspace_bytes(num_seqs, Hq, d, max_pages_per_seq);
}

int fa_decode_paged(const void* q, const void* kpages, const void* vpages, const int32_t* page_table,
                    const int32_t* ctx_lens, void* o, float* lse, int num_seqs, int Hq, int Hkv, int d,
                    int page_size, int max_pages_per_seq, int num_pages, float scale, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_pages_per_seq < 1 || num_pages < 1)
    return FA_ERR_SHAPE;
  // grid: x = num_seqs * Hkv * ceil(G / heads per workgroup) <= num_seqs * Hq; y = splits
  if ((long long)num_seqs * Hq > 0x7fffffffLL || fa::decode_max_splits(max_pages_per_seq) > 65535)
    return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (page_size != 16) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if (num_seqs == 0) return FA_OK;
  if (!q || !kpages || !vpages || !page_table || !ctx_lens || !o || !lse) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(kpages) || !aligned16(vpages) || !aligned16(page_table) ||
      !aligned16(ctx_lens) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  const size_t need = fa::decode_workspace_bytes(num_seqs, Hq, d, max_pages_per_seq);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  fa::DecodeArgs a{q,  kpages, vpages, page_table, ctx_lens, o, lse, num_seqs, Hq, Hkv, d, page_size,
                   max_pages_per_seq, scale, workspace, stream};
  return finish(fa::launch_decode_paged(a), stream);
}

int fa_decode_paged_int8(const void* q, const int8_t* kpages, const float* kscale, const int8_t* vpages,
                         const float* vscale, const int32_t* page_table, const int32_t* ctx_lens, void* o, float* lse,
                         int num_seqs, int Hq, int Hkv, int d, int page_size, int group, int max_pages_per_seq,
                         int num_pages, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_pages_per_seq < 1 || num_pages < 1)
    return FA_ERR_SHAPE;
  if ((long long)num_seqs * Hq > 0x7fffffffLL || fa::decode_max_splits(max_pages_per_seq) > 65535)
    return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (page_size != 16 || group != 32) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if (num_seqs == 0) return FA_OK;
  if (!q || !kpages || !kscale || !vpages || !vscale || !page_table || !ctx_lens || !o || !lse) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(kpages) || !aligned16(vpages) || !aligned16(page_table) || !aligned16(ctx_lens) ||
      !aligned16(o) || !aligned16(lse) || ((uintptr_t)kscale & 3u) || ((uintptr_t)vscale & 3u))
    return FA_ERR_ALIGN;
  const size_t need = fa::decode_workspace_bytes(num_seqs, Hq, d, max_pages_per_seq);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  fa::DecodeArgs a{q,  kpages, vpages, page_table, ctx_lens, o, lse, num_seqs, Hq, Hkv, d, page_size,
                   max_pages_per_seq, scale, workspace, stream};
  a.kscale = kscale;
  a.vscale = vscale;
  return finish(fa::launch_decode_paged(a), stream);
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid shape (negative size, Hq not a multiple of Hkv, or too large)";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension (64 or 128) or page size (16)";
    case FA_ERR_SCALE: return "scale is not finite";
    case FA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case FA_ERR_WORKSPACE: return "decode workspace is NULL or too small";
    case FA_ERR_HIP: return g_hip_error;
    default: return "unknown status";
  }
}

}  // extern "C"
