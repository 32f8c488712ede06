// Split-K paged-KV decode: one query token per sequence attends its whole
// cached context, which lives in fixed 16-token pages reached through a page
// table ("Phase 08 -- Inference Optimization at Depth", Concepts list: KV cache,
// paged attention; Lab 03 steps 1 and 4).
//
// Phase 1 (decode_split_kernel): one workgroup per (split of 128 pages, K/V head,
// sequence) serves up to HB query heads of that K/V head's group, so each K/V
// page is read from HBM once for the whole group.  The split index is the slow
// grid dimension: workgroups are dealt round-robin to the 8 XCDs by linear id, so
// each XCD gets an even share of (sequence, head) pairs at every split index
// (with the split fastest, an XCD would only ever see splits j and j + 8, and
// the early splits, active for every sequence, would pile onto a few XCDs).
// The split's page ids are read once, one per lane, and taken from that
// register wave-uniformly.  Its 4 waves take the split's pages two at a time,
// round-robin.  In a wave, lane l holds tokens 2*(l/8) and
// 2*(l/8)+1 of each page and the d columns {8*(l%8) + 64*c .. +8}; each (page,
// head) block is 4 KB contiguous, so every 16-byte load instruction covers 8
// whole 128-byte row segments.  The next page pair is fetched while the current
// one is consumed.  Scores: bf16 pair dot products (v_dot2c_f32_bf16, fp32
// accumulation) then a 3-step DPP sum over the 8 lanes of a token.  The
// wave keeps the online-softmax state (running max m, sum l, unnormalised
// accumulator) of the "Phase 08" Lab 01 recurrence, rescaling only when a head's
// max grows.  Tokens at or past ctx_len get probability 0 and their V rows are
// zeroed before use, so NaN in unused slots cannot leak (0 * NaN).  The waves'
// states are merged through LDS and the split writes (o_c normalised, lse_c).
//
// Phase 2 (decode_merge_kernel): per (sequence, query head) combine the splits:
// L = log sum_c exp(lse_c), O = sum_c exp(lse_c - L) o_c.
#include <mutex>
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"


namespace fa {
namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kPage = 16;
constexpr int kDecWaves = 4;
constexpr int kDecThreads = kDecWaves * 64;
static_assert(kDecThreads == kGeomDecThreads, "host-side launch limits assume this workgroup size");

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// Page id of split page idx (wave-uniform, 0 <= idx < kDecodePagesPerSplit): lane i
// of register r holds page p_begin + 64 r + i; read back with readlane.
template <int R>
__device__ __forceinline__ int page_id_of(const int (&lane_pid)[R], int idx) {
  int id = __builtin_amdgcn_readlane(lane_pid[0], idx & 63);
#pragma unroll
  for (int r = 1; r < R; ++r)
    if ((idx >> 6) == r) id = __builtin_amdgcn_readlane(lane_pid[r], idx & 63);
  return id;
}

// This lane's K and V data of one (page, K/V head) block of BYTES bytes: NV 16-byte
// loads at byte offsets off[i], non-temporal (each page is read once per call).  The
// buffer descriptor spans the block, or nothing when the page lies past the split:
// such loads return zeros without touching memory, so the loop's loads stay
// unconditional (the compiler never has to drain the other buffer's loads early)
// without fetching any page twice.
template <int NV, typename T>
__device__ __forceinline__ void load_block(const void* kblk, const void* vblk, uint32_t bytes, const int (&off)[NV],
                                           T (&kd)[NV], T (&vd)[NV]) {
  const auto krs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(kblk), (short)0, bytes, 0x00020000);
  const auto vrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(vblk), (short)0, bytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int o = off[i];
    if constexpr (sizeof(T) == 16) {
      kd[i] = __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(krs, o, 0, 2));
      vd[i] = __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(vrs, o, 0, 2));
    } else if constexpr (sizeof(T) == 8) {
      kd[i] = __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(krs, o, 0, 2));
      vd[i] = __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(vrs, o, 0, 2));
    } else {
      kd[i] = __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(krs, o, 0, 2));
      vd[i] = __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(vrs, o, 0, 2));
    }
  }
}

template <int D, int HB>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ KPg, const uint16_t* __restrict__ VPg,
    const int32_t* __restrict__ table, const int32_t* __restrict__ ctx, float* __restrict__ ws_o,
    float* __restrict__ ws_l, int Hq, int Hkv, int max_pages, int num_pages, int max_splits, int nhb, float c) {
  constexpr int CPL = D / 64;  // 8-column chunks per token per lane
  constexpr int DL = CPL * 8;  // d columns per lane
  constexpr int PP = 2;        // pages consumed per wave iteration
  __shared__ float sm_m[kDecWaves][HB];
  __shared__ float sm_l[kDecWaves][HB];
  __shared__ float sm_lr[kDecWaves][HB];
  __shared__ float sm_acc[kDecWaves][HB][D];

  const int split = blockIdx.y;
  const int hb = blockIdx.x % nhb;
  const int g = (blockIdx.x / nhb) % Hkv;
  const int s = blockIdx.x / (nhb * Hkv);
  const int G = Hq / Hkv;
  // device-side sizes are clamped to the buffers the host described: the context to
  // the page table's row, page ids to the pools (out-of-range values give wrong
  // output, never an access outside the buffers)
  const int n = min(max(ctx[s], 0), max_pages * kPage);
  const int npages = (n + kPage - 1) / kPage;
  const int p_begin = split * kDecodePagesPerSplit;
  if (p_begin >= npages) return;  // this split has no tokens: nothing is written or read later
  const int p_end = min(npages, p_begin + kDecodePagesPerSplit);

  const int tid = threadIdx.x;
  // wave index made provably wave-uniform, so page indices derived from it stay in
  // scalar registers (the page-id readlane below needs a uniform lane index)
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int tg = lane >> 3;  // token pair within the page
  const int dg = lane & 7;   // column group

  // query heads served: h = g*G + hb*HB + hh, valid while hb*HB + hh < G.
  // q stays packed bf16 (two columns per register) for the dot2 score products.
  uint32_t qp[HB][DL / 2];
  float qscale[HB];
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    const int hl = hb * HB + hh;
    const bool ok = hl < G;
    const uint16_t* qrow = Q + ((size_t)s * Hq + g * G + (ok ? hl : 0)) * D;
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
      const u32x4 x = ldg16(qrow + (dg + 8 * cc) * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) qp[hh][cc * 4 + e] = ok ? x[e] : 0u;
    }
    qscale[hh] = c;
  }

  // online-softmax state per served head: running max (log2 units), sums of the
  // fp32 probabilities (for L) and of their bf16 roundings (for O), and the
  // unnormalised output accumulator for this lane's d columns
  float m_run[HB], l_run[HB], l_rnd[HB], acc[HB][DL];
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    m_run[hh] = -INFINITY;
    l_run[hh] = 0.f;
    l_rnd[hh] = 0.f;
#pragma unroll
    for (int i = 0; i < DL; ++i) acc[hh][i] = 0.f;
  }

  // page ids of this split, lane i of register r holding page p_begin + 64 r + i;
  // read back with readlane at a wave-uniform index
  constexpr int kIdRegs = (kDecodePagesPerSplit + 63) / 64;
  const int32_t* trow = table + (size_t)s * max_pages;
  int lane_pid[kIdRegs];
#pragma unroll
  for (int r = 0; r < kIdRegs; ++r) {
    const int pg = p_begin + 64 * r + (tid & 63);
    const int id = pg < p_end ? trow[pg] : 0;
    lane_pid[r] = (unsigned)id < (unsigned)num_pages ? id : num_pages - 1;
  }
  const size_t head_off = (size_t)g * kPage * D;
  const size_t page_stride = (size_t)Hkv * kPage * D;
  // this lane's byte offsets in a (page, head) block: tokens 2 tg + j, columns (dg + 8 cc) * 8 ..
  int boff[2 * CPL];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) boff[j * CPL + cc] = ((2 * tg + j) * D + (dg + 8 * cc) * 8) * 2;

  // Two register buffers (A, B) of one page pair each, used alternately: the pair
  // after next is fetched into the buffer just consumed, so one pair is always in
  // flight while the other is processed (no register copies that would force a
  // wait on outstanding loads).  A page past this split's end (the second page of an
  // odd last pair, or the prefetch after a wave's last pair) gets an empty buffer
  // descriptor: its loads return zeros without a memory access, and consume() treats
  // its tokens as invalid.
  u32x4 ka[PP][2 * CPL], va[PP][2 * CPL];
  u32x4 kb[PP][2 * CPL], vb[PP][2 * CPL];
  auto fetch = [&](int p0, u32x4 (&kd)[PP][2 * CPL], u32x4 (&vd)[PP][2 * CPL]) {
#pragma unroll
    for (int pp = 0; pp < PP; ++pp) {
      const int p = p0 + pp;
      const bool valid = p < p_end;
      const size_t base = (size_t)page_id_of(lane_pid, min(p, p_end - 1) - p_begin) * page_stride + head_off;
      load_block<2 * CPL>(KPg + base, VPg + base, valid ? kPage * D * 2 : 0, boff, kd[pp], vd[pp]);
    }
  };
  auto consume = [&](int p, u32x4 (&kc)[PP][2 * CPL], u32x4 (&vc)[PP][2 * CPL]) {
    // scores: this lane's 2 tokens of each page of the pair, every served head
    float sc[PP][2][HB];
#pragma unroll
    for (int pp = 0; pp < PP; ++pp)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int tok = (p + pp) * kPage + 2 * tg + j;
        const bool valid = tok < n && p + pp < p_end;
#pragma unroll
        for (int hh = 0; hh < HB; ++hh) {
          float part = 0.f;
#pragma unroll
          for (int cc = 0; cc < CPL; ++cc)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              part = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kc[pp][j * CPL + cc][e]), as_bf16x2(qp[hh][cc * 4 + e]),
                                                     part, false);
          part = sum8(part) * qscale[hh];
          sc[pp][j][hh] = valid ? part : -INFINITY;
        }
      }
    // online softmax state update (wave-uniform max per head)
    bool grow = false;
    float mnew[HB];
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      float pm = fmaxf(fmaxf(sc[0][0][hh], sc[0][1][hh]), fmaxf(sc[1][0][hh], sc[1][1][hh]));
      pm = max_stride8(pm);
      mnew[hh] = fmaxf(m_run[hh], pm);
      grow |= mnew[hh] > m_run[hh];
    }
    if (grow) {
#pragma unroll
      for (int hh = 0; hh < HB; ++hh) {
        const float alpha = exp2_fast(m_run[hh] - mnew[hh]);
        l_run[hh] *= alpha;
        l_rnd[hh] *= alpha;
#pragma unroll
        for (int i = 0; i < DL; ++i) acc[hh][i] *= alpha;
        m_run[hh] = mnew[hh];
      }
    }
    // the sequence's last page may hold slots past ctx_len (and a redirected page
    // is a duplicate): zero their V so that 0 * NaN cannot occur
    if ((p + PP) * kPage > n || p + PP > p_end) {
#pragma unroll
      for (int pp = 0; pp < PP; ++pp)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const bool valid = (p + pp) * kPage + 2 * tg + j < n && p + pp < p_end;
#pragma unroll
          for (int cc = 0; cc < CPL; ++cc)
#pragma unroll
            for (int e = 0; e < 4; ++e) vc[pp][j * CPL + cc][e] = valid ? vc[pp][j * CPL + cc][e] : 0u;
        }
    }
    // O += P V as bf16 pair dot products over the lane's two tokens: P packed as
    // (p(t0), p(t1)) per head, V repacked as (V[t0][d], V[t1][d]) per column.  O is
    // later divided by the sum of these rounded probabilities, L uses the fp32 sum.
    const bf16x2 ones = as_bf16x2(0x3f803f80u);
#pragma unroll
    for (int pp = 0; pp < PP; ++pp) {
      uint32_t ppair[HB];
#pragma unroll
      for (int hh = 0; hh < HB; ++hh) {
        const float p0 = (sc[pp][0][hh] == -INFINITY) ? 0.f : exp2_fast(sc[pp][0][hh] - m_run[hh]);
        const float p1 = (sc[pp][1][hh] == -INFINITY) ? 0.f : exp2_fast(sc[pp][1][hh] - m_run[hh]);
        l_run[hh] += p0 + p1;
        ppair[hh] = pack_bf16x2(p0, p1);
        l_rnd[hh] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(ppair[hh]), ones, l_rnd[hh], false);
      }
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w0 = vc[pp][cc][e], w1 = vc[pp][CPL + cc][e];
          const uint32_t lo = __builtin_amdgcn_perm(w1, w0, 0x05040100u);  // (w0.lo, w1.lo)
          const uint32_t hi = __builtin_amdgcn_perm(w1, w0, 0x07060302u);  // (w0.hi, w1.hi)
#pragma unroll
          for (int hh = 0; hh < HB; ++hh) {
            acc[hh][cc * 8 + 2 * e] =
                __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(ppair[hh]), as_bf16x2(lo), acc[hh][cc * 8 + 2 * e], false);
            acc[hh][cc * 8 + 2 * e + 1] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(ppair[hh]), as_bf16x2(hi),
                                                                          acc[hh][cc * 8 + 2 * e + 1], false);
          }
        }
    }
  };

  // wave w takes page pairs p_begin + PP*(w + 4i), i = 0, 1, ...
  constexpr int kStride = PP * kDecWaves;
  int p = p_begin + PP * w;
  if (p < p_end) fetch(p, ka, va);
  while (p < p_end) {
    fetch(p + kStride, kb, vb);
    consume(p, ka, va);
    p += kStride;
    if (p >= p_end) break;
    fetch(p + kStride, ka, va);
    consume(p, kb, vb);
    p += kStride;
  }

  // combine the 8 token-pair lanes of each column group, then the 4 waves
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    l_run[hh] = sum_stride8(l_run[hh]);
    l_rnd[hh] = sum_stride8(l_rnd[hh]);
#pragma unroll
    for (int i = 0; i < DL; ++i) acc[hh][i] = sum_stride8(acc[hh][i]);
  }
  if (lane < 8) {
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      if (lane == 0) {
        sm_m[w][hh] = m_run[hh];
        sm_l[w][hh] = l_run[hh];
        sm_lr[w][hh] = l_rnd[hh];
      }
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc)
#pragma unroll
        for (int e = 0; e < 8; ++e) sm_acc[w][hh][(dg + 8 * cc) * 8 + e] = acc[hh][cc * 8 + e];
    }
  }
  __syncthreads();
  for (int i = tid; i < HB * D; i += kDecThreads) {
    const int hh = i / D, d = i % D;
    const int hl = hb * HB + hh;
    if (hl >= G) continue;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) M = fmaxf(M, sm_m[ww][hh]);
    float wsum = 0.f, rsum = 0.f, o = 0.f;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) {
      const float mw = sm_m[ww][hh];
      const float f = (mw == -INFINITY) ? 0.f : exp2_fast(mw - M);
      wsum += f * sm_l[ww][hh];
      rsum += f * sm_lr[ww][hh];
      o += f * sm_acc[ww][hh][d];
    }
    const size_t slot = ((size_t)s * Hq + g * G + hl) * max_splits + split;
    ws_o[slot * D + d] = o / rsum;
    if (d == 0) ws_l[slot] = M + log2_fast(wsum);  // log2 units
  }
}


// ---------------------------------------------------------------------------
// INT8 group-scaled KV cache (screna.ai KV-cache quantization block: 8-bit cache
// with group-wise scales).  K/V pages hold int8 values, one fp32 scale per
// (page, K/V head, token, 32 consecutive channels); the value is int8 * scale.
// Same grid, page-id register and ping-pong buffers as decode_split_kernel, one page
// per wave iteration; lane l holds tokens 2(l/8), 2(l/8)+1 and channels
// (l%8)*CH .. +CH (one 32-channel group), CH = D/8.
//  - Keys: byte b enters as the fp16 value 1024 + (b + 128), built by one byte permute per channel pair (b ^ 0x80 as the
//    low byte under a 0x64 high byte), against q converted exactly to fp16 under a power-of-two scale per head.  Then
//    q.k = sum q_c (1152 + b_c) - 1152 sum q_c, with fp16 pair dot products and fp32 sums (the products are exact): the
//    key offset is removed algebraically.
//  - Values: the signed byte b enters as the bf16 value b (at most 8 significant bits: the upper half of its fp32
//    conversion, one sign-extending instruction), so O += (p s) b per group with bf16 pair dot products and exact
//    products.  p s enters P V rounded to bf16; O and L are normalised by the fp32 sum of the probabilities.  (fp16
//    would bound p s to its range, which arbitrary scales need not respect.)
//  - Softmax: each lane keeps its own running maximum of the raw scores q.k * kscale (the factor k = |scale| log2(e)
//    times the head's q unscale enters the exponent's fused multiply-add), raised only when a score passes it by more
//    than 8 / k, so probabilities stay at most 2^8 and no per-page reduction across lanes is needed.  The lanes'
//    maxima are combined once, after the loop.
template <int CH>
struct I8Vec;
template <>
struct I8Vec<16> {
  typedef u32x4 T;
};
template <>
struct I8Vec<8> {
  typedef u32x2 T;
};

// Keeps the compiler from re-fusing a product into the following cross-lane add
// (it would otherwise recompute the product in an fmac beside a DPP move).
__device__ __forceinline__ float opaque(float x) {
  asm("" : "+v"(x));
  return x;
}

template <int D, int HB>
__global__ __launch_bounds__(kDecThreads) void decode_split_int8_kernel(
    const uint16_t* __restrict__ Q, const int8_t* __restrict__ KQ, const float* __restrict__ KS,
    const int8_t* __restrict__ VQ, const float* __restrict__ VS, const int32_t* __restrict__ table,
    const int32_t* __restrict__ ctx, float* __restrict__ ws_o, float* __restrict__ ws_l, int Hq, int Hkv,
    int max_pages, int num_pages, int max_splits, int nhb, float c) {
  constexpr int CH = D / 8;           // channels per lane
  constexpr int NG = D / 32;          // scale groups per token
  constexpr int NW = CH / 4;          // 32-bit words per token per lane
  constexpr int PP = 1;               // pages consumed per wave iteration
  constexpr float kGrow = 8.f;        // log2 units a score may exceed the running max by
  typedef typename I8Vec<CH>::T vec_t;
  __shared__ float sm_m[kDecWaves][HB];
  __shared__ float sm_l[kDecWaves][HB];
  __shared__ float sm_acc[kDecWaves][HB][D];

  const int split = blockIdx.y;
  const int hb = blockIdx.x % nhb;
  const int g = (blockIdx.x / nhb) % Hkv;
  const int s = blockIdx.x / (nhb * Hkv);
  const int G = Hq / Hkv;
  // device-side sizes are clamped to the buffers the host described: the context to
  // the page table's row, page ids to the pools (out-of-range values give wrong
  // output, never an access outside the buffers)
  const int n = min(max(ctx[s], 0), max_pages * kPage);
  const int npages = (n + kPage - 1) / kPage;
  const int p_begin = split * kDecodePagesPerSplit;
  if (p_begin >= npages) return;
  const int p_end = min(npages, p_begin + kDecodePagesPerSplit);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int tg = lane >> 3;
  const int dg = lane & 7;
  const int grp = dg * CH / 32;       // the lane's scale group

  // q as fp16 channel pairs (the score dot2 operands) for the lane's channels.  Each
  // head's q is scaled by a power of two that puts its largest magnitude in
  // [2^13, 2^14), so every bf16 value converts to fp16 exactly (11 significant bits),
  // and negated when the softmax scale is negative, so that k >= 0.  qsum = 1152 *
  // sum q removes the key offset (see above).
  const float cabs = fabsf(c);
  const float csgn = c < 0.f ? -1.f : 1.f;
  uint32_t qp[HB][CH / 2];
  float qsum[HB], kh[HB], grow_by[HB];
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    const int hl = hb * HB + hh;
    const bool ok = hl < G;
    const uint16_t* qrow = Q + ((size_t)s * Hq + g * G + (ok ? hl : 0)) * D + dg * CH;
    uint32_t raw[CH / 2];
    float mx = 0.f;
#pragma unroll
    for (int e = 0; e < CH / 8; ++e) {
      const u32x4 x = ldg16(qrow + e * 8);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        raw[e * 4 + k] = ok ? x[k] : 0u;
        mx = fmaxf(mx, fmaxf(fabsf(bf16lo_to_f32(raw[e * 4 + k])), fabsf(bf16hi_to_f32(raw[e * 4 + k]))));
      }
    }
    mx = fmaxf(mx, dpp<0xB1>(mx));  // max over the head's 8 channel-group lanes
    mx = fmaxf(mx, dpp<0x4E>(mx));
    mx = fmaxf(mx, dpp<0x141>(mx));
    const int ex = min(max(__builtin_amdgcn_frexp_expf(mx), -100), 128);  // mx in [2^(ex-1), 2^ex)
    const float up = csgn * ldexpf(1.f, 14 - ex);
    kh[hh] = cabs * ldexpf(1.f, ex - 14);
    grow_by[hh] = kGrow / kh[hh];  // +inf when k = 0: the first maximum is kept
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < CH / 2; ++i) {
      const f32x2 v = {bf16lo_to_f32(raw[i]) * up, bf16hi_to_f32(raw[i]) * up};
      const f16x2 h = __builtin_convertvector(v, f16x2);
      qp[hh][i] = __builtin_bit_cast(uint32_t, h);
      sum += (float)h[0] + (float)h[1];
    }
    qsum[hh] = 1152.f * sum;
  }

  // per lane: running max of the raw scores, the score that triggers a rescale, -max*k,
  // the fp32 probability sum, the offset correction and the unnormalised output
  float m_run[HB], thr[HB], nmk[HB], l_run[HB], acc[HB][CH];
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    m_run[hh] = -INFINITY;
    thr[hh] = -INFINITY;
    nmk[hh] = 0.f;
    l_run[hh] = 0.f;
#pragma unroll
    for (int i = 0; i < CH; ++i) acc[hh][i] = 0.f;
  }

  constexpr int kIdRegs = (kDecodePagesPerSplit + 63) / 64;
  const int32_t* trow = table + (size_t)s * max_pages;
  int lane_pid[kIdRegs];
#pragma unroll
  for (int r = 0; r < kIdRegs; ++r) {
    const int pg = p_begin + 64 * r + (tid & 63);
    const int id = pg < p_end ? trow[pg] : 0;
    lane_pid[r] = (unsigned)id < (unsigned)num_pages ? id : num_pages - 1;
  }
  // this lane's byte offsets in a (page, head) block of int8 values and of scales
  int boff[2], soff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    boff[j] = (2 * tg + j) * D + dg * CH;
    soff[j] = ((2 * tg + j) * NG + grp) * 4;
  }
  // as in decode_split_kernel: a page past the split gets empty buffer descriptors
  vec_t ka[PP][2], va[PP][2], kb[PP][2], vb[PP][2];
  float ksa[PP][2], vsa[PP][2], ksb[PP][2], vsb[PP][2];
  // pages p_begin .. p_full - 1 hold 16 tokens of the context each; a sequence's last
  // page may hold fewer (only in its last split)
  const int p_full = min(p_end, n / kPage);
  // fetch pages p0 .. p0 + PP - 1 (those at or past lim get empty descriptors)
  auto fetch = [&](int p0, int lim, vec_t (&kd)[PP][2], vec_t (&vd)[PP][2], float (&ksd)[PP][2],
                   float (&vsd)[PP][2]) {
#pragma unroll
    for (int pp = 0; pp < PP; ++pp) {
      const int p = p0 + pp;
      const bool valid = p < lim;
      const size_t head = (size_t)page_id_of(lane_pid, min(p, p_end - 1) - p_begin) * Hkv + g;
      load_block<2>(KQ + head * kPage * D, VQ + head * kPage * D, valid ? kPage * D : 0, boff, kd[pp], vd[pp]);
      load_block<2>(KS + head * kPage * NG, VS + head * kPage * NG, valid ? kPage * NG * 4 : 0, soff, ksd[pp],
                    vsd[pp]);
    }
  };
  // FULL: every token of the pages lies inside the context, so the per-token validity
  // selects are left out
  auto consume = [&](auto full, int p, vec_t (&kc)[PP][2], vec_t (&vc)[PP][2], float (&ksc)[PP][2],
                     float (&vsc)[PP][2]) {
    constexpr bool FULL = decltype(full)::value;
    float sc[PP][2][HB];  // raw scores (q.k * kscale), -inf past the context
#pragma unroll
    for (int pp = 0; pp < PP; ++pp)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bool valid = FULL || ((p + pp) * kPage + 2 * tg + j < n && p + pp < p_end);
        // key byte b as the fp16 value 1024 + (b + 128): the unsigned byte b ^ 0x80
        // becomes the low byte of an fp16 whose high byte is 0x64 (one byte permute per
        // channel pair); the products with fp16 q are exact in the fp32 sums
        uint32_t up[CH / 2];
#pragma unroll
        for (int e = 0; e < NW; ++e) {
          const uint32_t x = kc[pp][j][e] ^ 0x80808080u;
          up[2 * e] = __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u);
          up[2 * e + 1] = __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u);
        }
#pragma unroll
        for (int hh = 0; hh < HB; ++hh) {
          float part = -qsum[hh];
#pragma unroll
          for (int i = 0; i < CH / 2; ++i)
            part = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, qp[hh][i]), __builtin_bit_cast(f16x2, up[i]), part,
                                          false);
          // lanes l and l ^ 1 hold halves of one scale group (CH = 16) or of its first
          // half (CH = 8): add them, apply the token's group scale, finish the sum
          part += dpp<0xB1>(part);
          part = opaque(part * ksc[pp][j]);
          part += dpp<0x4E>(part);
          part += dpp<0x141>(part);
          sc[pp][j][hh] = valid ? part : -INFINITY;
        }
      }
    // raise a lane's max (and rescale its sums) only where a score passes the threshold
    bool grow = false;
    float pm[HB];
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      pm[hh] = fmaxf(sc[0][0][hh], sc[0][1][hh]);
#pragma unroll
      for (int pp = 1; pp < PP; ++pp) pm[hh] = fmaxf(pm[hh], fmaxf(sc[pp][0][hh], sc[pp][1][hh]));
      grow |= pm[hh] > thr[hh];
    }
    if (grow) {
#pragma unroll
      for (int hh = 0; hh < HB; ++hh) {
        if (pm[hh] > thr[hh]) {
          const float alpha = m_run[hh] == -INFINITY ? 0.f : exp2_fast((m_run[hh] - pm[hh]) * kh[hh]);
          l_run[hh] *= alpha;
#pragma unroll
          for (int i = 0; i < CH; ++i) acc[hh][i] *= alpha;
          m_run[hh] = pm[hh];
          thr[hh] = pm[hh] + grow_by[hh];
          nmk[hh] = -pm[hh] * kh[hh];
        }
      }
    }
#pragma unroll
    for (int pp = 0; pp < PP; ++pp) {
      // channel c of the two tokens as one bf16 pair: a signed byte has at most 8
      // significant bits, so its fp32 conversion (one instruction, sign-extending the
      // byte) is exact in the upper half, which one byte permute per pair moves into place
      uint32_t vp[CH];
#pragma unroll
      for (int e = 0; e < NW; ++e) {
        const uint32_t x0 = vc[pp][0][e], x1 = vc[pp][1][e];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          vp[4 * e + k] = __builtin_amdgcn_perm(__float_as_uint((float)(signed char)(x1 >> (8 * k))),
                                                __float_as_uint((float)(signed char)(x0 >> (8 * k))), 0x07060302u);
      }
      const bool v0 = FULL || ((p + pp) * kPage + 2 * tg < n && p + pp < p_end);
      const bool v1 = FULL || ((p + pp) * kPage + 2 * tg + 1 < n && p + pp < p_end);
      // invalid tokens (possibly NaN scales) contribute exactly nothing
      const float s0 = v0 ? vsc[pp][0] : 0.f, s1 = v1 ? vsc[pp][1] : 0.f;
#pragma unroll
      for (int hh = 0; hh < HB; ++hh) {
        const float p0 = v0 ? exp2_fast(fmaf(sc[pp][0][hh], kh[hh], nmk[hh])) : 0.f;
        const float p1 = v1 ? exp2_fast(fmaf(sc[pp][1][hh], kh[hh], nmk[hh])) : 0.f;
        l_run[hh] += p0 + p1;
        const uint32_t ps = pack_bf16x2(p0 * s0, p1 * s1);
#pragma unroll
        for (int i = 0; i < CH; ++i)
          acc[hh][i] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(ps), as_bf16x2(vp[i]), acc[hh][i], false);
      }
    }
  };

  // wave w takes pages p_begin + PP (w + 4 i): whole pages in the loop, then the
  // sequence's partial last page (or the pages of a partial group) after it
  constexpr int kStride = PP * kDecWaves;
  int p = p_begin + PP * w;
  if (p + PP <= p_full) fetch(p, p_full, ka, va, ksa, vsa);
  while (p + PP <= p_full) {
    fetch(p + kStride, p_full, kb, vb, ksb, vsb);
    consume(std::true_type{}, p, ka, va, ksa, vsa);
    p += kStride;
    if (p + PP > p_full) break;
    fetch(p + kStride, p_full, ka, va, ksa, vsa);
    consume(std::true_type{}, p, kb, vb, ksb, vsb);
    p += kStride;
  }
  if (p < p_end) {
    fetch(p, p_end, ka, va, ksa, vsa);
    consume(std::false_type{}, p, ka, va, ksa, vsa);
  }

  // bring the 8 token-pair lanes to a common max, remove the byte offset, combine the
  // lanes, then the 4 waves (in log2 units)
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    const float mw = max_stride8(m_run[hh]);
    const float f = m_run[hh] == -INFINITY ? 0.f : exp2_fast((m_run[hh] - mw) * kh[hh]);
    l_run[hh] = sum_stride8(l_run[hh] * f);
#pragma unroll
    for (int i = 0; i < CH; ++i) acc[hh][i] = sum_stride8(acc[hh][i] * f);
    m_run[hh] = mw == -INFINITY ? -INFINITY : mw * kh[hh];
  }
  if (lane < 8) {
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      if (lane == 0) {
        sm_m[w][hh] = m_run[hh];
        sm_l[w][hh] = l_run[hh];
      }
#pragma unroll
      for (int i = 0; i < CH; ++i) sm_acc[w][hh][dg * CH + i] = acc[hh][i];
    }
  }
  __syncthreads();
  for (int i = tid; i < HB * D; i += kDecThreads) {
    const int hh = i / D, d = i % D;
    const int hl = hb * HB + hh;
    if (hl >= G) continue;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) M = fmaxf(M, sm_m[ww][hh]);
    float wsum = 0.f, o = 0.f;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) {
      const float mw = sm_m[ww][hh];
      const float f = (mw == -INFINITY) ? 0.f : exp2_fast(mw - M);
      wsum += f * sm_l[ww][hh];
      o += f * sm_acc[ww][hh][d];
    }
    const size_t slot = ((size_t)s * Hq + g * G + hl) * max_splits + split;
    ws_o[slot * D + d] = o / wsum;
    if (d == 0) ws_l[slot] = M + log2_fast(wsum);
  }
}

template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(const float* __restrict__ ws_o,
                                                         const float* __restrict__ ws_l,
                                                         const int32_t* __restrict__ ctx,
                                                         uint16_t* __restrict__ O, float* __restrict__ Lse,
                                                         int Hq, int max_pages, int max_splits) {
  const int s = blockIdx.x / Hq;
  const int h = blockIdx.x % Hq;
  const int d = threadIdx.x;
  const int n = min(ctx[s], max_pages * kPage);  // as in the split kernels
  const size_t out = ((size_t)s * Hq + h);
  if (n <= 0) {
    O[out * D + d] = 0;
    if (d == 0) Lse[out] = -INFINITY;
    return;
  }
  const int nsplit = ((n + kPage - 1) / kPage + kDecodePagesPerSplit - 1) / kDecodePagesPerSplit;
  const float* lp = ws_l + out * max_splits;
  const float* op = ws_o + out * max_splits * D;
  float M = -INFINITY;
  for (int c = 0; c < nsplit; ++c) M = fmaxf(M, lp[c]);
  float wsum = 0.f, o = 0.f;
  for (int c = 0; c < nsplit; ++c) {
    const float f = exp2_fast(lp[c] - M);
    wsum += f;
    o += f * op[(size_t)c * D + d];
  }
  O[out * D + d] = __builtin_bit_cast(uint16_t, to_bf16(o / wsum));
  if (d == 0) Lse[out] = (M + log2_fast(wsum)) * kLn2;
}

template <int D, int HB>
hipError_t launch_split(const DecodeArgs& a, float* ws_o, float* ws_l, int max_splits) {
  const int G = a.Hq / a.Hkv;
  const int nhb = (G + HB - 1) / HB;
  const dim3 grid((unsigned)(a.S * a.Hkv * nhb), (unsigned)max_splits);
  hipLaunchKernelGGL((decode_split_kernel<D, HB>), grid, dim3(kDecThreads), 0, (hipStream_t)a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.kpages, (const uint16_t*)a.vpages, a.page_table,
                     a.ctx_lens, ws_o, ws_l, a.Hq, a.Hkv, a.max_pages, a.num_pages, max_splits, nhb, a.scale * kLog2e);
  return hipGetLastError();
}

template <int D, int HB>
hipError_t launch_split_int8(const DecodeArgs& a, float* ws_o, float* ws_l, int max_splits) {
  const int G = a.Hq / a.Hkv;
  const int nhb = (G + HB - 1) / HB;
  const dim3 grid((unsigned)(a.S * a.Hkv * nhb), (unsigned)max_splits);
  hipLaunchKernelGGL((decode_split_int8_kernel<D, HB>), grid, dim3(kDecThreads), 0, (hipStream_t)a.stream,
                     (const uint16_t*)a.q, (const int8_t*)a.kpages, a.kscale, (const int8_t*)a.vpages, a.vscale,
                     a.page_table, a.ctx_lens, ws_o, ws_l, a.Hq, a.Hkv, a.max_pages, a.num_pages, max_splits,
                     nhb, a.scale * kLog2e);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a) {
  const int max_splits = decode_max_splits(a.max_pages);
  float* ws_o = (float*)a.workspace;
  const size_t o_bytes = (size_t)a.S * a.Hq * max_splits * D * sizeof(float);
  float* ws_l = (float*)((uint8_t*)a.workspace + ((o_bytes + 255) / 256) * 256);
  const int G = a.Hq / a.Hkv;
  hipError_t e;
  if (a.kscale != nullptr) {
    if (G <= 1) e = launch_split_int8<D, 1>(a, ws_o, ws_l, max_splits);
    else if (G <= 2) e = launch_split_int8<D, 2>(a, ws_o, ws_l, max_splits);
    else e = launch_split_int8<D, 4>(a, ws_o, ws_l, max_splits);
  } else if (G <= 1) e = launch_split<D, 1>(a, ws_o, ws_l, max_splits);
  else if (G <= 2) e = launch_split<D, 2>(a, ws_o, ws_l, max_splits);
  else e = launch_split<D, 4>(a, ws_o, ws_l, max_splits);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)(a.S * a.Hq)), dim3(D), 0, (hipStream_t)a.stream,
                     ws_o, ws_l, a.ctx_lens, (uint16_t*)a.o, a.lse, a.Hq, a.max_pages, max_splits);
  return hipGetLastError();
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

// Device scratch of the allocation-free decode (fa_decode_paged_noalloc): the split
// partials live here instead of in a caller workspace.  One copy per GPU, held until
// the process ends; every call on a GPU shares it, so overlapping calls on one GPU
// race.  The split kernels write every partial the merge kernel reads in the same
// call, so nothing needs clearing between calls.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t launch_decode_paged(const DecodeArgs& a) {
  return a.d == 64 ? launch_d<64>(a) : launch_d<128>(a);
}

// Device address of this GPU's scratch copy.  The array's name is a host-side
// stand-in, not a device address, so the address is looked up once per device
// (with that device current) and cached; kernels only ever get the cached pointer.
hipError_t noalloc_scratch(void* stream, void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int sdev = dev;
  if (stream != nullptr) {
    hipDevice_t d = 0;
    e = hipStreamGetDevice((hipStream_t)stream, &d);
    if (e != hipSuccess) return e;
    sdev = (int)d;
  }
  if (sdev < 0 || sdev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[sdev] == nullptr) {
    if (sdev != dev && (e = hipSetDevice(sdev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (sdev != dev) {
      const hipError_t e2 = hipSetDevice(dev);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[sdev] = p;
  }
  *ptr = g_scratch_ptr[sdev];
  return hipSuccess;
}

}  // namespace fa
