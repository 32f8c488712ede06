// Internal host-side interface between the C ABI (fa_api.cpp) and the kernel
// translation units.  Arguments reaching these launchers are already validated.
#pragma once

#include <hip/hip_runtime.h>
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
};

struct DecodeArgs {
  const void* q;
  const void* kpages;
  const void* vpages;
  const int32_t* page_table;
  const int32_t* ctx_lens;
  void* o;
  float* lse;
  int S, Hq, Hkv, d, page_size, max_pages;
  float scale;
  void* workspace;
  void* stream;
  // INT8 cache (fa_decode_paged_int8): kpages/vpages hold int8, with one fp32 scale
  // per (page, head, token, 32 channels) in kscale/vscale; nullptr = bf16 cache
  const float* kscale = nullptr;
  const float* vscale = nullptr;
};

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
hipError_t launch_prefill_paged(const FwdArgs& a);
hipError_t launch_bwd_bf16(const BwdArgs& a);
hipError_t launch_fwd_f32(const FwdArgs& a);
hipError_t launch_decode_paged(const DecodeArgs& a);

}  // namespace fa
