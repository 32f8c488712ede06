// Internal host-side interface between the C ABI (fa_api.cpp) and the kernel
// translation units.  Arguments reaching these launchers are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <algorithm>
#include <stddef.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, N, d;
  bool causal;
  float scale;
  void* stream;
  int window = 0;                 // bf16 only: keys j >= i - window + 1 (0: none)
  const float* slopes = nullptr;  // bf16 only: ALiBi slope per query head, or none
  // chunked prefill over a paged cache (launch_prefill_paged): B = sequences, N = chunk
  // length, k/v = page pools [pages][Hkv][16][d]
  const int32_t* page_table = nullptr;
  const int32_t* ctx_lens = nullptr;
  int max_pages = 0;
  int num_pages = 0;              // pages in each pool (page ids are clamped below it)
  void* workspace = nullptr;      // split-K forward (launch_fwd_splitk): fp32 partials
};

struct DecodeArgs {
  const void* q;
  const void* kpages;
  const void* vpages;
  const int32_t* page_table;
  const int32_t* ctx_lens;
  void* o;
  float* lse;
  int S, Hq, Hkv, d, page_size, max_pages, num_pages;
  float scale;
  void* workspace;
  void* stream;
  // INT8 cache (fa_decode_paged_int8): kpages/vpages hold int8, with one fp32 scale
  // per (page, head, token, 32 channels) in kscale/vscale; nullptr = bf16 cache
  const float* kscale = nullptr;
  const float* vscale = nullptr;
};

// Workgroup geometry of the kernels, shared with the host-side validation: a
// dispatch's total work-item count (workgroups x threads) must stay below 2^31.
// Each kernel source checks its own constants against these.
constexpr int kGeomFwdRows = 256;     // bf16 forward: query rows per workgroup
constexpr int kGeomFwdThreads = 512;
constexpr int kGeomF32Threads = 256;  // fp32 forward: d / 16 lanes per row, so 256 / (d / 16) rows
constexpr int kGeomDecThreads = 256;  // decode split kernel (the merge kernel has d threads)
constexpr int kGeomDqRows = 256;      // backward dQ: query rows per workgroup
constexpr int kGeomDqThreads = 512;
constexpr int kGeomDkdvRows = 128;    // backward dK/dV: keys per workgroup
constexpr int kGeomDkdvThreads = 512;
constexpr long long kMaxWorkItems = 0x7fffffffLL;

// Pages handled by one split of the paged decode.  The workspace size depends on it.
#ifndef FA_DECODE_PAGES_PER_SPLIT
#define FA_DECODE_PAGES_PER_SPLIT 128
#endif
constexpr int kDecodePagesPerSplit = FA_DECODE_PAGES_PER_SPLIT;

inline int decode_max_splits(int max_pages) {
  return (max_pages + kDecodePagesPerSplit - 1) / kDecodePagesPerSplit;
}
// Workspace: o partials [S][Hq][splits][d] fp32, then lse partials [S][Hq][splits] fp32.
inline size_t decode_workspace_bytes(int S, int Hq, int d, int max_pages) {
  const size_t splits = (size_t)decode_max_splits(max_pages);
  const size_t o_bytes = (size_t)S * Hq * splits * d * sizeof(float);
  const size_t l_bytes = (size_t)S * Hq * splits * sizeof(float);
  return ((o_bytes + 255) / 256) * 256 + l_bytes;
}

// Split-K forward plan (fa_fwd_splitk).  When a launch has fewer (256-row query block,
// head) items than kSplitTargetItems workgroups (256: the MI355X compute units), the
// key tiles of each block are cut into chunks of T tiles, T the smallest value (at
// least 4) that keeps the item count within the target; blocks with more than one
// chunk leave fp32 (O, lse) partials in the workspace for a merge.  Otherwise nothing is
// split (T = the longest block's tile count) and no workspace is needed.
// Workspace: O partials [B*Hq][query blocks][smax][256][d] fp32 (padded to 256 B), then
// per partial row m + log2 of its fp32 probability sum, then m + log2 of the sum of
// its bf16-rounded probabilities (each [B*Hq][query blocks][smax][256] fp32).
constexpr int kSplitTargetItems = 256;
inline int fwd_key_tiles(int N, int d, bool causal, int qb) {
  const int bc = d == 64 ? 128 : 64;
  const long long kend = causal ? std::min<long long>(N, (long long)(qb + 1) * kGeomFwdRows) : N;
  return (int)((kend + bc - 1) / bc);
}
struct SplitPlan {
  int T, smax, nqb;
  long long items;
  size_t o_bytes, bytes;
};
inline SplitPlan fwd_split_plan(int B, int Hq, int N, int d, bool causal) {
  SplitPlan p;
  p.nqb = (N + kGeomFwdRows - 1) / kGeomFwdRows;
  const long long BH = (long long)B * Hq;
  const int maxt = fwd_key_tiles(N, d, causal, p.nqb - 1);
  auto items_for = [&](int T) {
    long long n = 0;
    for (int qb = 0; qb < p.nqb; ++qb) n += (fwd_key_tiles(N, d, causal, qb) + T - 1) / T;
    return n * BH;
  };
  p.T = maxt;
  if (BH * p.nqb < kSplitTargetItems) {
    for (int T = std::min(4, maxt); T < maxt; ++T)
      if (items_for(T) <= kSplitTargetItems) {
        p.T = T;
        break;
      }
  }
  p.smax = (maxt + p.T - 1) / p.T;
  p.items = items_for(p.T);
  if (p.smax > 1) {
    const size_t rows = (size_t)BH * p.nqb * p.smax * kGeomFwdRows;
    p.o_bytes = (rows * d * sizeof(float) + 255) / 256 * 256;
    p.bytes = p.o_bytes + 2 * rows * sizeof(float);
  } else {
    p.o_bytes = 0;
    p.bytes = 0;
  }
  return p;
}

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  int B, Hq, Hkv, N, d;
  bool causal;
  float scale;
  void* workspace;
  void* stream;
};

// Backward launch plan.  dK/dV workgroups cover 128 keys of one K/V head; when
// there are fewer than 512 of them, the query heads of each group are split into
// chunks (each workgroup one chunk) whose fp32 partial sums are added at the end.
// Workspace: D = rowsum(dO * O) [B][Hq][N] fp32 and L2 = L * log2(e) [B][Hq][N]
// fp32 (each padded to 256 B), then the dK and dV partials [chunks][B][Hkv][N][d]
// fp32 each when chunks > 1.
struct BwdPlan {
  int nchunks, heads_per_chunk;
  size_t l2_offset, part_offset, part_elems, bytes;
};
inline BwdPlan bwd_plan(int B, int Hq, int Hkv, int N, int d) {
  BwdPlan p;
  const long long nkb = (N + 127) / 128;
  const long long base = (long long)B * Hkv * nkb;
  const int G = Hq / Hkv;
  int nch = 1;
  if (base > 0 && base < 512) nch = (int)((512 + base - 1) / base);
  if (nch > G) nch = G;
  p.heads_per_chunk = (G + nch - 1) / nch;
  p.nchunks = (G + p.heads_per_chunk - 1) / p.heads_per_chunk;
  p.l2_offset = (((size_t)B * Hq * N * sizeof(float)) + 255) / 256 * 256;
  p.part_offset = 2 * p.l2_offset;
  p.part_elems = p.nchunks > 1 ? (size_t)p.nchunks * B * Hkv * N * d : 0;
  p.bytes = p.part_offset + 2 * p.part_elems * sizeof(float);
  return p;
}

hipError_t launch_fwd_bf16(const FwdArgs& a);
hipError_t launch_fwd_splitk(const FwdArgs& a);
hipError_t launch_prefill_paged(const FwdArgs& a);
hipError_t launch_bwd_bf16(const BwdArgs& a);
hipError_t launch_fwd_f32(const FwdArgs& a);
hipError_t launch_decode_paged(const DecodeArgs& a);

// Allocation-free decode: the library's own device scratch replaces the workspace.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;  // 32 MiB per GPU
// Device address of the scratch on the stream's GPU (looked up once per device).
hipError_t noalloc_scratch(void* stream, void** ptr);

}  // namespace fa
