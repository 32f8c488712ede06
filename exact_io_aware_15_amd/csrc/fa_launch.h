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

hipError_t launch_fwd_bf16(const FwdArgs& a);
hipError_t launch_fwd_f32(const FwdArgs& a);
hipError_t launch_decode_paged(const DecodeArgs& a);

}  // namespace fa
