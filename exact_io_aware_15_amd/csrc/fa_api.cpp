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

// A dispatch of `blocks` workgroups of `threads` threads fits the launch limits.
bool fits(long long blocks, int threads) { return blocks >= 1 && blocks <= fa::kMaxWorkItems / threads; }

// The bf16 kernels address one (batch, head) slice of N x d elements through a
// buffer descriptor whose byte range is a 32-bit value.
bool slice_fits(long long N, int d, int elem) { return N * d * elem <= 0xffffffffLL; }

long long cdiv(long long a, long long b) { return (a + b - 1) / b; }

// Checks in a fixed order: sizes (FA_ERR_SHAPE, including the kernels' launch
// limits), head dimension, scale, then pointers.
int check_fwd_args(int B, int Hq, int Hkv, int N, int d, int causal, float scale) {
  if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || d < 1) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  return FA_OK;
}

int check_fwd_ptrs(const void* q, const void* k, const void* v, const void* o, const void* lse) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  return FA_OK;
}

// Size limits of the bf16 forward kernel (fa_fwd, fa_fwd_ex).
int check_fwd_bf16_sizes(int B, int Hq, int N, int d) {
  if (!slice_fits(N, d, 2)) return FA_ERR_SHAPE;
  if (!fits((long long)B * Hq * cdiv(N, fa::kGeomFwdRows), fa::kGeomFwdThreads)) return FA_ERR_SHAPE;
  return FA_OK;
}

// Decode split grid: num_seqs * Hkv * ceil(G / 4) <= num_seqs * Hq workgroups along x,
// splits along y (at most 65535).
int check_decode_sizes(int num_seqs, int Hq, int max_pages_per_seq) {
  if ((long long)max_pages_per_seq * 16 > 0x7fffffffLL) return FA_ERR_SHAPE;
  const long long splits = fa::decode_max_splits(max_pages_per_seq);
  if (splits > 65535) return FA_ERR_SHAPE;
  if (!fits((long long)num_seqs * Hq * splits, fa::kGeomDecThreads)) return FA_ERR_SHAPE;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int N,
           int d, int causal, float scale, void* stream) {
  int st = check_fwd_args(B, Hq, Hkv, N, d, causal, scale);
  if (st == FA_OK) st = check_fwd_bf16_sizes(B, Hq, N, d);
  if (st == FA_OK) st = check_fwd_ptrs(q, k, v, o, lse);
  if (st != FA_OK) return st;
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, d, causal != 0, scale, stream};
  return finish(fa::launch_fwd_bf16(a), stream);
}

size_t fa_fwd_splitk_workspace_size(int B, int Hq, int N, int d, int causal) {
  if (B < 1 || Hq < 1 || N < 1 || (d != 64 && d != 128) || (causal != 0 && causal != 1)) return 0;
  return fa::fwd_split_plan(B, Hq, N, d, causal != 0).bytes;
}

int fa_fwd_splitk(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int N,
                  int d, int causal, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_fwd_args(B, Hq, Hkv, N, d, causal, scale);
  if (st == FA_OK) st = check_fwd_bf16_sizes(B, Hq, N, d);
  if (st == FA_OK) st = check_fwd_ptrs(q, k, v, o, lse);
  if (st != FA_OK) return st;
  const fa::SplitPlan pl = fa::fwd_split_plan(B, Hq, N, d, causal != 0);
  // the merge grid: one 256-thread workgroup per 1024 / d rows of every (head, query block)
  if (!fits((long long)B * Hq * pl.nqb * (fa::kGeomFwdRows / (1024 / d)), 256)) return FA_ERR_SHAPE;
  if (pl.bytes > 0) {
    if (!workspace || workspace_bytes < pl.bytes) return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_ALIGN;
  }
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, d, causal != 0, scale, stream};
  a.workspace = workspace;
  return finish(fa::launch_fwd_splitk(a), stream);
}

int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int N,
              int d, int causal, float scale, int window, const float* alibi_slopes, void* stream) {
  if (window < 0) return FA_ERR_SHAPE;
  int st = check_fwd_args(B, Hq, Hkv, N, d, causal, scale);
  if (st == FA_OK) st = check_fwd_bf16_sizes(B, Hq, N, d);
  if (st != FA_OK) return st;
  if (window > 0 && !causal) return FA_ERR_UNSUPPORTED;
  st = check_fwd_ptrs(q, k, v, o, lse);
  if (st != FA_OK) return st;
  if (alibi_slopes && ((uintptr_t)alibi_slopes & 3u) != 0) return FA_ERR_ALIGN;
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, d, causal != 0, scale, stream, window, alibi_slopes};
  return finish(fa::launch_fwd_bf16(a), stream);
}

int fa_prefill_paged(const void* q, const void* kpages, const void* vpages, const int32_t* page_table,
                     const int32_t* ctx_lens, void* o, float* lse, int num_seqs, int Hq, int Hkv, int d, int chunk,
                     int page_size, int max_pages_per_seq, int num_pages, float scale, void* stream) {
  if (num_seqs < 1 || chunk < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_pages_per_seq < 1 || num_pages < 1)
    return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (page_size != 16) return FA_ERR_UNSUPPORTED;
  // a chunk lies inside its sequence's cache, which the page table bounds
  if ((long long)max_pages_per_seq * page_size > 0x7fffffffLL || chunk > max_pages_per_seq * page_size)
    return FA_ERR_SHAPE;
  if (!fits((long long)num_seqs * Hq * cdiv(chunk, fa::kGeomFwdRows), fa::kGeomFwdThreads)) return FA_ERR_SHAPE;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if (!q || !kpages || !vpages || !page_table || !ctx_lens || !o || !lse) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(kpages) || !aligned16(vpages) || !aligned16(page_table) ||
      !aligned16(ctx_lens) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  fa::FwdArgs a{q, kpages, vpages, o, lse, num_seqs, Hq, Hkv, chunk, d, true, scale, stream};
  a.page_table = page_table;
  a.ctx_lens = ctx_lens;
  a.max_pages = max_pages_per_seq;
  a.num_pages = num_pages;
  return finish(fa::launch_prefill_paged(a), stream);
}

size_t fa_bwd_workspace_size(int B, int Hq, int Hkv, int N, int d) {
  if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || (d != 64 && d != 128)) return 0;
  return fa::bwd_plan(B, Hq, Hkv, N, d).bytes;
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
           void* dk, void* dv, int B, int Hq, int Hkv, int N, int d, int causal, float scale, void* workspace,
           size_t workspace_bytes, void* stream) {
  int st = check_fwd_args(B, Hq, Hkv, N, d, causal, scale);
  if (st != FA_OK) return st;
  // the four kernels' dispatch sizes: one row per d/8 lanes (delta), 256-row dQ and
  // 128-key dK/dV workgroups, one element per lane (partial-sum reduction)
  const fa::BwdPlan pl = fa::bwd_plan(B, Hq, Hkv, N, d);
  if (!slice_fits(N, d, 2) || !fits(cdiv((long long)B * Hq * N * (d / 8), 256), 256) ||
      !fits((long long)B * Hq * cdiv(N, fa::kGeomDqRows), fa::kGeomDqThreads) ||
      !fits((long long)B * Hkv * pl.nchunks * cdiv(N, fa::kGeomDkdvRows), fa::kGeomDkdvThreads) ||
      !fits(cdiv((long long)B * Hkv * N * d, 256), 256))
    return FA_ERR_SHAPE;
  st = check_fwd_ptrs(q, k, v, o, lse);
  if (st != FA_OK) return st;
  if (!dout || !dq || !dk || !dv) return FA_ERR_NULL;
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv)) return FA_ERR_ALIGN;
  if (!workspace || workspace_bytes < pl.bytes) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  fa::BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, causal != 0, scale, workspace, stream};
  return finish(fa::launch_bwd_bf16(a), stream);
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int Hq, int Hkv,
               int N, int d, int causal, float scale, void* stream) {
  int st = check_fwd_args(B, Hq, Hkv, N, d, causal, scale);
  if (st != FA_OK) return st;
  const int rows = fa::kGeomF32Threads / (d / 16);
  if (!fits((long long)B * Hq * cdiv(N, rows), fa::kGeomF32Threads)) return FA_ERR_SHAPE;
  st = check_fwd_ptrs(q, k, v, o, lse);
  if (st != FA_OK) return st;
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, d, causal != 0, scale, stream};
  return finish(fa::launch_fwd_f32(a), stream);
}

size_t fa_decode_paged_workspace_size(int num_seqs, int Hq, int d, int max_pages_per_seq, int page_size) {
  if (num_seqs < 1 || Hq < 1 || max_pages_per_seq < 1) return 0;
  if (d != 64 && d != 128) return 0;
  if (page_size != 16) return 0;
  return fa::decode_workspace_bytes(num_seqs, Hq, d, max_pages_per_seq);
}

int fa_decode_paged(const void* q, const void* kpages, const void* vpages, const int32_t* page_table,
                    const int32_t* ctx_lens, void* o, float* lse, int num_seqs, int Hq, int Hkv, int d,
                    int page_size, int max_pages_per_seq, int num_pages, float scale, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (num_seqs < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_pages_per_seq < 1 || num_pages < 1)
    return FA_ERR_SHAPE;
  if (check_decode_sizes(num_seqs, Hq, max_pages_per_seq) != FA_OK) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (page_size != 16) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if (!q || !kpages || !vpages || !page_table || !ctx_lens || !o || !lse) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(kpages) || !aligned16(vpages) || !aligned16(page_table) ||
      !aligned16(ctx_lens) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  const size_t need = fa::decode_workspace_bytes(num_seqs, Hq, d, max_pages_per_seq);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  fa::DecodeArgs a{q,  kpages, vpages, page_table, ctx_lens, o, lse, num_seqs, Hq, Hkv, d, page_size,
                   max_pages_per_seq, num_pages, scale, workspace, stream};
  return finish(fa::launch_decode_paged(a), stream);
}

int fa_decode_paged_int8(const void* q, const int8_t* kpages, const float* kscale, const int8_t* vpages,
                         const float* vscale, const int32_t* page_table, const int32_t* ctx_lens, void* o, float* lse,
                         int num_seqs, int Hq, int Hkv, int d, int page_size, int group, int max_pages_per_seq,
                         int num_pages, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_pages_per_seq < 1 || num_pages < 1)
    return FA_ERR_SHAPE;
  if (check_decode_sizes(num_seqs, Hq, max_pages_per_seq) != FA_OK) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (page_size != 16 || group != 32) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if (!q || !kpages || !kscale || !vpages || !vscale || !page_table || !ctx_lens || !o || !lse) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(kpages) || !aligned16(vpages) || !aligned16(page_table) || !aligned16(ctx_lens) ||
      !aligned16(o) || !aligned16(lse) || ((uintptr_t)kscale & 3u) || ((uintptr_t)vscale & 3u))
    return FA_ERR_ALIGN;
  const size_t need = fa::decode_workspace_bytes(num_seqs, Hq, d, max_pages_per_seq);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  fa::DecodeArgs a{q,  kpages, vpages, page_table, ctx_lens, o, lse, num_seqs, Hq, Hkv, d, page_size,
                   max_pages_per_seq, num_pages, scale, workspace, stream};
  a.kscale = kscale;
  a.vscale = vscale;
  return finish(fa::launch_decode_paged(a), stream);
}

int fa_decode_paged_noalloc(const void* q, const void* kpages, const void* vpages, const int32_t* page_table,
                            const int32_t* ctx_lens, void* o, float* lse, int num_seqs, int Hq, int Hkv, int d,
                            int page_size, int max_pages_per_seq, int num_pages, float scale, void* stream) {
  if (num_seqs < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_pages_per_seq < 1 || num_pages < 1)
    return FA_ERR_SHAPE;
  if (check_decode_sizes(num_seqs, Hq, max_pages_per_seq) != FA_OK) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (page_size != 16) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if (!q || !kpages || !vpages || !page_table || !ctx_lens || !o || !lse) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(kpages) || !aligned16(vpages) || !aligned16(page_table) ||
      !aligned16(ctx_lens) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  if (fa::decode_workspace_bytes(num_seqs, Hq, d, max_pages_per_seq) > fa::kNoAllocScratchBytes)
    return FA_ERR_SCRATCH;
  void* ws = nullptr;
  const hipError_t e = fa::noalloc_scratch(stream, &ws);
  if (e != hipSuccess) return hip_status(e);
  fa::DecodeArgs a{q,  kpages, vpages, page_table, ctx_lens, o, lse, num_seqs, Hq, Hkv, d, page_size,
                   max_pages_per_seq, num_pages, scale, ws, stream};
  return finish(fa::launch_decode_paged(a), stream);
}

size_t fa_decode_paged_noalloc_max_scratch(void) { return fa::kNoAllocScratchBytes; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid shape (a size below 1, Hq not a multiple of Hkv, or too large for the kernels)";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension (64 or 128) or page size (16)";
    case FA_ERR_SCALE: return "scale is not finite";
    case FA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case FA_ERR_WORKSPACE: return "decode workspace is NULL or too small";
    case FA_ERR_HIP: return g_hip_error;
    case FA_ERR_SCRATCH:
      return "sizes need more than the library's fixed device scratch (fa_decode_paged_noalloc_max_scratch bytes)";
    default: return "unknown status";
  }
}

}  // extern "C"
