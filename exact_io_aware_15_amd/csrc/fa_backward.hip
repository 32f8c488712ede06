// Exact-attention backward on gfx950 matrix cores: dQ, dK, dV from Q, K, V, the
// forward's O and per-row logsumexp L, and the upstream gradient dO.
//
// "Phase 08 -- Inference Optimization at Depth", Concepts list (the FlashAttention
// backward needs only O and L, never the N x N matrix) and Lab 01 step 6 (the
// optional backward pass).  The pages give no formulas; the kernels evaluate the
// standard chain rule through the softmax, recomputing P tile by tile from Q, K
// and the stored L instead of reading it:
//
//   D   = rowsum(dO * O)                     (bwd_delta_kernel)
//   P   = exp(scale * Q K^T - L)             (masked entries 0)
//   dP  = dO V^T,   dS = P * (dP - D)
//   dQ  = scale * dS K                       (bwd_dq_kernel: one pass over K/V per query block)
//   dV  = P^T dO,   dK = scale * dS^T Q      (bwd_dkdv_kernel: one pass over Q/dO per key block)
//
// Both main kernels run eight waves per workgroup (two per SIMD) and stream the
// other operand in 64-row tiles through two LDS buffers, copied HBM -> LDS with the LDS-destination bit of 128-bit buffer loads
// (rows past N read as zero), rows unpadded with XOR-swizzled 16-byte chunks.
// Every product runs on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  The dQ
// kernel computes S^T and dP^T with a lane per query row (so the row's L and D sit
// in one register), like the forward, and accumulates dQ^T = K^T dS^T reading K^T
// fragments with ds_read_b64_tr_b16.  The dK/dV kernel computes S and dP with a lane
// per key and accumulates dV = P^T dO and dK = dS^T Q reading dO and Q through the
// transposing reads; at d = 128 its V^T fragments come from the key block's V rows in
// LDS.  It streams each head's unmasked row tiles first and the few that need masking
// (the causal diagonal, the ragged end) last, each group through code of its own.
// Grouped query heads: a K/V head's gradients sum over the query
// heads of its group; when there are too few (key block, K/V head) pairs to fill
// the GPU (multi-query), the group's heads are split into chunks whose fp32 partial
// sums a last kernel adds up.
#include <climits>
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kBwdWaves = 4;                 // dK/dV: key groups of 32 per workgroup
constexpr int kKvWaves = 8;                  // dK/dV waves: two per key group (row halves), two per SIMD
constexpr int kBwdThreads = kKvWaves * 64;
#ifndef FA_BWD_DQ_WAVES
#define FA_BWD_DQ_WAVES 8
#endif
constexpr int kDqWaves = FA_BWD_DQ_WAVES;    // dQ: two waves per SIMD
constexpr int kWaveRows = 32;                // query rows (dQ) or keys (dK/dV) per wave
constexpr int kBlockRows = kBwdWaves * kWaveRows;  // 128 keys per dK/dV workgroup
constexpr int kDqRows = kDqWaves * kWaveRows;      // 256 query rows per dQ workgroup
constexpr int kTile = 64;                    // rows of the streamed operand per tile
static_assert(kDqRows == kGeomDqRows && kDqWaves * 64 == kGeomDqThreads && kBlockRows == kGeomDkdvRows &&
                  kBwdThreads == kGeomDkdvThreads,
              "host-side launch limits assume this geometry");

template <int D, int W = kBwdWaves>
struct BLay {
  static constexpr int ROWB = D * 2;              // bytes per row
  static constexpr int CPR = ROWB / 16;           // 16-byte chunks per row
  static constexpr int RPB = 1024 / ROWB;         // rows per 1 KB block
  static constexpr int TBYTES = kTile * ROWB;     // one tile
  static constexpr int BPW = TBYTES / 1024 / W;  // 1 KB blocks copied per wave (W waves)
  static_assert(BPW * W * 1024 == TBYTES, "tile copy must split evenly over the waves");
  // physical chunk = logical chunk ^ swz(row); depends on row & 15 only.  Tiles are
  // read both ways: by rows (b128, 16 consecutive rows at one logical chunk: swz must
  // be one-to-one over those rows, per LDS bank half at d = 64) and transposed (per
  // 32-lane half, 4 consecutive rows x one aligned 4-chunk window: swz must move each
  // of the 4 rows, per bank half at d = 64, to a different window).
  __host__ __device__ static constexpr int swz(int r) {
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
};

typedef short s16x8 __attribute__((ext_vector_type(8)));

// HBM -> LDS copy of tile rows r0 .. r0+63 of one (batch, head) slice by W waves:
// this wave's 1 KB blocks w, w + W, ...  Block w + Wi lies W KB after block w in
// both HBM and LDS and the swizzle repeats with that period, so one per-lane
// offset cp serves all.
template <int D, int W = kBwdWaves>
__device__ __forceinline__ void copy_tile(uint8_t* dst, const void* base, uint32_t bytes, uint32_t cp, int r0, int w) {
  using L = BLay<D, W>;
  constexpr uint32_t kStride = W * 1024;
  static_assert((kStride / L::ROWB) % 16 == 0, "swizzle must repeat every W blocks");
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
  const uint32_t off = (uint32_t)r0 * L::ROWB + cp;
#pragma unroll
  for (int i = 0; i < L::BPW; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (FA_LDS void*)(dst + w * 1024 + i * kStride), 16, off, i * kStride,
                                             0, 0);
}

// 64 fp32 row values (L or D) of rows r0 .. r0+63 into dst; lanes 0..15 of the
// calling wave, rows past N read as zero.
__device__ __forceinline__ void copy_rowvals(float* dst, const float* base, int N, int r0, int lane) {
  if (lane < 16) {
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, (uint32_t)N * 4, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (FA_LDS void*)dst, 16, (uint32_t)r0 * 4 + lane * 16, 0, 0, 0);
  }
}

// Lane's byte offset for copying block w of a tile (row w*RPB + lane/CPR, swizzled chunk).
template <int D, int W = kBwdWaves>
__device__ __forceinline__ uint32_t copy_offset(int w, int lane) {
  using L = BLay<D, W>;
  const int r = w * L::RPB + lane / L::CPR;
  return r * L::ROWB + (((lane % L::CPR) ^ L::swz(r)) << 4);
}

// Offsets of the transposing fragment reads X^T[d][rows] from a row-major tile:
// for d block db, the lower (rows R0 + 4hi + 0..3) and upper (R0 + 8 + 4hi + 0..3)
// reads of a 16-row group R0 (R0 a multiple of 16).  Source lane li of 16-lane
// group grp reads row 4hi + li/4 (+8) and d = 32db + 16(grp&1) + 4(li&3) .. +3.
template <int D>
__device__ __forceinline__ void tr_offsets(int lane, int (&tlo)[D / 32], int (&thi)[D / 32]) {
  using L = BLay<D>;
  const int hi = lane >> 5, grp = lane >> 4, li = lane & 15;
  const int vr = 4 * hi + (li >> 2);
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int lc = 4 * db + 2 * (grp & 1) + ((li & 3) >> 1);
    tlo[db] = vr * L::ROWB + ((lc ^ L::swz(vr)) << 4) + (li & 1) * 8;
    thi[db] = (vr + 8) * L::ROWB + ((lc ^ L::swz(vr + 8)) << 4) + (li & 1) * 8;
  }
}

__device__ __forceinline__ bf16x8 tr_frag(const uint8_t* base, int lo, int up) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(base + lo));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(base + up));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// Scheduling pattern for a run of `mfmas` MFMAs that each consume `reads` LDS
// reads: keep the reads of `ahead` MFMAs in flight ahead of their use.
template <int mfmas, int reads, int id, int ahead>
__device__ __forceinline__ void sched_reads_ahead() {
  constexpr int pre = ahead < mfmas ? ahead : mfmas;
  __builtin_amdgcn_sched_group_barrier(0x100, pre * reads, id);
#pragma unroll
  for (int i = 0; i < mfmas - pre; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, id);
    __builtin_amdgcn_sched_group_barrier(0x100, reads, id);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, pre, id);
}

// ---------------------------------------------------------------------------
// D = rowsum(dO * O): D/8 lanes per row, 16-byte loads, DPP reduction.  The same
// pass writes L2 = L * log2(e), the row's logsumexp in base 2, which the dK/dV
// kernel subtracts per element.
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
                                                        const float* __restrict__ Lse, float* __restrict__ Dlt,
                                                        float* __restrict__ L2, long long rows) {
  constexpr int LPR = D / 8;  // lanes per row: 16 (d128) or 8 (d64)
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = gid / LPR;
  const int c = (int)(gid % LPR);
  float acc = 0.f;
  if (row < rows) {
    const u32x4 o = ld16(O + row * D + c * 8);
    const u32x4 g = ld16(dO + row * D + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = __builtin_fmaf(bf16lo_to_f32(o[e]), bf16lo_to_f32(g[e]), acc);
      acc = __builtin_fmaf(bf16hi_to_f32(o[e]), bf16hi_to_f32(g[e]), acc);
    }
  }
  acc = sum8(acc);                         // lanes l ^ 1, 2, 4
  if (LPR == 16) acc += dpp<0x128>(acc);   // and l ^ 8 (row_ror:8 inside 16-lane rows)
  if (row < rows && c == 0) {
    Dlt[row] = acc;
    L2[row] = Lse[row] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (128-row query block, query head, batch), four waves of 32
// rows.  K and V tiles of 64 keys stream through LDS (two buffers each).
// LDS reads kept ahead of the MFMAs (measured per kernel and head dim)
template <int D>
constexpr int ahead_dq() { return D == 64 ? 6 : 4; }
template <int D>
constexpr int ahead_dkdv() { return D == 64 ? 6 : 4; }
// dK/dV at d = 128 keeps the key block's V rows in LDS instead of registers: the 32
// registers freed keep the kernel within its 256 without spills
template <int D>
constexpr bool kVinLds = D == 128;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kDqWaves * 64, 1) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ Lse, const float* __restrict__ Dlt,
    uint16_t* __restrict__ dQ, int B, int Hq, int Hkv, int N, float cs /* scale * log2 e */, float scale) {
  using L = BLay<D, kDqWaves>;
  constexpr int KK = D / 16, DB = D / 32;
  constexpr int kAhead = ahead_dq<D>();
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * L::TBYTES];  // K[2], V[2]

  const int nqb = (N + kDqRows - 1) / kDqRows;
  const int BH = B * Hq;
  const int qb = CAUSAL ? (nqb - 1 - (int)(blockIdx.x / BH)) : (int)(blockIdx.x / BH);  // heaviest first
  const int bh = blockIdx.x % BH;
  const int b = bh / Hq, h = bh % Hq;
  const int g = h / (Hq / Hkv);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int rw0 = qb * kDqRows + w * kWaveRows;
  const int qrow = rw0 + l32;
  const bool row_ok = qrow < N;

  const size_t qoff = (size_t)(b * Hq + h) * N;
  const uint16_t* kbase = K + (size_t)(b * Hkv + g) * N * D;
  const uint16_t* vbase = V + (size_t)(b * Hkv + g) * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;

  // Q and dO rows as B operands (Q^T, dO^T fragments): row qrow, d = kk*16 + hi*8 .. +8
  bf16x8 qf[KK], gf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (row_ok) {
      x = ld16(Q + (qoff + qrow) * D + kk * 16 + hi * 8);
      y = ld16(dO + (qoff + qrow) * D + kk * 16 + hi * 8);
    }
    qf[kk] = __builtin_bit_cast(bf16x8, x);
    gf[kk] = __builtin_bit_cast(bf16x8, y);
  }
  // the row's statistics: P = exp2(cs * s - l2); rows past N get P = 0
  const float l2 = row_ok ? Lse[qoff + qrow] * kLog2e : INFINITY;
  const float dl = row_ok ? Dlt[qoff + qrow] : 0.f;

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  int roff[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) roff[kk] = l32 * L::ROWB + (((2 * kk + hi) ^ L::swz(l32)) << 4);
  int tlo[DB], thi[DB];
  tr_offsets<D>(lane, tlo, thi);
  const uint32_t cp = copy_offset<D, kDqWaves>(w, lane);

  const int kend = CAUSAL ? min(N, (qb + 1) * kDqRows) : N;
  const int ntiles = (kend + kTile - 1) / kTile;

  if (ntiles > 0) {
    copy_tile<D, kDqWaves>(smem, kbase, head_bytes, cp, 0, w);
    copy_tile<D, kDqWaves>(smem + 2 * L::TBYTES, vbase, head_bytes, cp, 0, w);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  for (int t0 = 0; t0 < ntiles; t0 += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = t0 + u;
      if (t >= ntiles) break;
      const int j0 = t * kTile;
      if (t + 1 < ntiles) {
        copy_tile<D, kDqWaves>(smem + (1 - u) * L::TBYTES, kbase, head_bytes, cp, j0 + kTile, w);
        copy_tile<D, kDqWaves>(smem + (3 - u) * L::TBYTES, vbase, head_bytes, cp, j0 + kTile, w);
      }
      debug_copy_fence();
      const bool skip = CAUSAL && (j0 > rw0 + kWaveRows - 1);
      // restrict LDS tile pointers: the copy in flight writes only the other buffer,
      // so the reads need not wait for it (the compiler otherwise waits for all
      // outstanding copies before the first LDS read that might alias them)
      auto tile = [&](const uint8_t* __restrict__ kb, const uint8_t* __restrict__ vb) {
        // S^T = K Q^T and dP^T = V dO^T; lane holds keys a*32 + 8(r/4) + 4hi + r%4 of its row
        f32x16 s[2], dp[2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            s[a][r] = 0.f;
            dp[a][r] = 0.f;
          }
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
          for (int a = 0; a < 2; ++a) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kb + a * 32 * L::ROWB + roff[kk]);
            s[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s[a], 0, 0, 0);
          }
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
          for (int a = 0; a < 2; ++a) {
            const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vb + a * 32 * L::ROWB + roff[kk]);
            dp[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, gf[kk], dp[a], 0, 0, 0);
          }
        sched_reads_ahead<4 * KK, 1, 0, kAhead>();
        debug_read_fence();
        // exponents cs * s - l2 in place; masked keys (after the row, or past N) get
        // -inf in a branch that only tiles on the diagonal or past N take (the empty
        // asm keeps it a branch; selected into every tile the masking would cost
        // three VALU operations per entry)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[a][r] = __builtin_fmaf(s[a][r], cs, -l2);
        const bool need_mask = CAUSAL ? (j0 + kTile - 1 > rw0) : (j0 + kTile > N);
        if (need_mask) {
          float ninf;
          asm volatile("v_mov_b32 %0, 0xff800000" : "=v"(ninf));
          const int lim = (CAUSAL ? qrow - j0 : N - 1 - j0) - 4 * hi;
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (a * 32 + 8 * (r >> 2) + (r & 3) > lim) s[a][r] = ninf;
        }
        // dS^T = P^T * (dP^T - D)
        bf16x8 dsb[2][2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            u32x4 pk;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              float d2[2];
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                const int r = h2 * 8 + 2 * j + e;
                d2[e] = exp2_fast(s[a][r]) * (dp[a][r] - dl);
              }
              pk[j] = pack_bf16x2(d2[0], d2[1]);
            }
            dsb[a][h2] = __builtin_bit_cast(bf16x8, pk);
          }
        // dQ^T += K^T dS^T
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const uint8_t* grp0 = kb + (a * 32 + h2 * 16) * L::ROWB;
              acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag(grp0, tlo[db], thi[db]), dsb[a][h2], acc[db],
                                                                0, 0, 0);
            }
        sched_reads_ahead<4 * DB, 2, 1, kAhead>();
        debug_read_fence();
      };
      if (!skip) tile(smem + u * L::TBYTES, smem + (2 + u) * L::TBYTES);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile t+1 has landed
      __syncthreads();
    }
  }

  // dQ = scale * (dQ^T)^T: lane holds d = db*32 + 8*g4 + 4*hi + 0..3 of its row
  if (row_ok) {
    uint16_t* out = dQ + (qoff + qrow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        u32x2 w2;
        w2[0] = pack_bf16x2(acc[db][4 * g4 + 0] * scale, acc[db][4 * g4 + 1] * scale);
        w2[1] = pack_bf16x2(acc[db][4 * g4 + 2] * scale, acc[db][4 * g4 + 3] * scale);
        *reinterpret_cast<u32x2*>(out + db * 32 + 8 * g4 + 4 * hi) = w2;
      }
  }
}

// Source of the dK/dV kernel's streamed items.  Each query head of the chunk has
// row tiles t_first .. nt-1.  Only its first n_lead tiles (on the causal diagonal of
// the key block) and, when N is not a multiple of the tile, its last tile need masking;
// the nu tiles between need none.  Items 0 .. n_un-1 are the unmasked tiles of every
// head (head-major), the remaining items the nm masked tiles of every head.
struct ItemSrc {
  const uint16_t* Q;
  const uint16_t* dO;
  const float* L2;
  const float* Dlt;
  int b, Hq, N, h_begin, t_first, nt, n_lead, nu, nm, n_un;
  uint32_t head_bytes, cp;
  int w, lane;
};

// (query head, row tile) of item i.  The unmasked tiles of a head are taken from the
// last one down: every key block of the head then streams the same Q/dO rows at about
// the same time (a causal block's first rows are its own, its last ones everybody's),
// so the blocks of a head that run together on an XCD share them through its L2.
__device__ __forceinline__ void item_pos(const ItemSrc& s, int item, int& h, int& t) {
  if (item < s.n_un) {
    h = item / s.nu;
    t = s.t_first + s.n_lead + (s.nu - 1 - item % s.nu);
  } else {
    const int j = item - s.n_un;
    h = j / s.nm;
    const int k = j % s.nm;
    t = k < s.n_lead ? s.t_first + k : s.nt - 1;
  }
  h += s.h_begin;
}

// Start the HBM -> LDS copies of one item into buffer buf: its Q and dO tiles
// (all waves) and the 64 rows' L (wave 0) and D (wave 1).
template <int D>
__device__ __forceinline__ void issue_item(const ItemSrc& s, uint8_t* qdst, uint8_t* gdst, float (*rowv)[2][kTile],
                                           int item, int buf) {
  using L = BLay<D>;
  int h, t;
  item_pos(s, item, h, t);
  const int r0 = t * kTile;
  const size_t qo = (size_t)(s.b * s.Hq + h) * s.N;
  copy_tile<D, kKvWaves>(qdst, s.Q + qo * D, s.head_bytes, s.cp, r0, s.w);
  copy_tile<D, kKvWaves>(gdst, s.dO + qo * D, s.head_bytes, s.cp, r0, s.w);
  if (s.w == 0) copy_rowvals(rowv[buf][0], s.L2 + qo, s.N, r0, s.lane);
  if (s.w == 1) copy_rowvals(rowv[buf][1], s.Dlt + qo, s.N, r0, s.lane);
}

// One streamed item (a query head's 64-row Q/dO tile with its rows' L2 and D) of
// the dK/dV kernel for this wave's 32 keys, rows 32*rh .. +32 of the tile (rh, the
// wave's row half, is already in the lane offsets roff, tlo, thi and rvo): S = Q K^T,
// dP = dO V^T, P, dS, then dV += P^T dO and dK += dS^T Q.  MASK: the item may need
// masking for some wave (need_mask: for this one); without it no masking code is
// emitted.  RP / RF are the LDS pointer types (restrict or plain, chosen by the kernel).
template <int D, bool CAUSAL, bool MASK, typename RP, typename RF>
__device__ __forceinline__ void dkdv_tile(RP qb_, RP gb_, RF lrow, RF drow, bool need_mask, int rbase, int kw0, int N,
                                          float cs, const int (&roff)[D / 16], const int (&tlo)[D / 32],
                                          const int (&thi)[D / 32], int rvo, const bf16x8 (&kf)[D / 16],
                                          const bf16x8 (&vf)[D / 16], RP vrows, f32x16 (&dka)[D / 32],
                                          f32x16 (&dva)[D / 32]) {
  using L = BLay<D>;
  constexpr int KK = D / 16, DB = D / 32;
  constexpr int kAhead = ahead_dkdv<D>();
  const int lane = (int)__lane_id(), l32 = lane & 31, hi = lane >> 5;
  // S = Q K^T and dP = dO V^T for rows 8(r/4) + 4hi + r%4 of the half
  f32x16 s, dp;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s[r] = 0.f;
    dp[r] = 0.f;
  }
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const bf16x8 qa = *reinterpret_cast<const bf16x8*>(qb_ + roff[kk]);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[kk], s, 0, 0, 0);
  }
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const bf16x8 ga = *reinterpret_cast<const bf16x8*>(gb_ + roff[kk]);
    // V^T fragment: from registers, or (kVinLds) from the key block's V rows in LDS
    bf16x8 vk;
    if constexpr (kVinLds<D>)
      vk = *reinterpret_cast<const bf16x8*>(vrows + l32 * L::ROWB + (((2 * kk + hi) ^ L::swz(l32)) << 4));
    else
      vk = vf[kk];
    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vk, dp, 0, 0, 0);
  }
  sched_reads_ahead<2 * KK, kVinLds<D> ? 2 : 1, 2, kAhead>();
  debug_read_fence();
  bf16x8 pb[2], dsb[2];
  if constexpr (D == 64) {
    // exponents s * cs - L2 in place (L2 = L log2 e); masked entries (key after the
    // row, or row past N) get -inf in a branch that only diagonal and tail tiles take
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // rows 8j + 4hi .. +4
      const f32x4 lv = *reinterpret_cast<const f32x4*>(reinterpret_cast<const uint8_t*>(lrow) + rvo + 32 * j);
#pragma unroll
      for (int i = 0; i < 4; ++i) s[4 * j + i] = __builtin_fmaf(s[4 * j + i], cs, -lv[i]);
    }
    if (MASK && need_mask) {
      // the empty asm keeps this a branch (selected into every tile, the masking
      // would cost four VALU operations per entry); -inf is made here rather than
      // held in a register across the loop
      float ninf;
      asm volatile("v_mov_b32 %0, 0xff800000" : "=v"(ninf));
      const int mlo = CAUSAL ? kw0 + l32 - rbase - 4 * hi : INT_MIN;
      const int mhi = N - rbase - 4 * hi;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 8 * (r / 4) + r % 4;  // row of entry r, less rbase + 4hi
        if (c < mlo || c >= mhi) s[r] = ninf;
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      u32x4 pk, dk;
#pragma unroll
      for (int q4 = 0; q4 < 2; ++q4) {
        const int j = 2 * s2 + q4;
        const f32x4 dv = *reinterpret_cast<const f32x4*>(reinterpret_cast<const uint8_t*>(drow) + rvo + 32 * j);
        float pv[4], dsv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[i] = exp2_fast(s[4 * j + i]);
          dsv[i] = pv[i] * (dp[4 * j + i] - dv[i]);
        }
        pk[2 * q4] = pack_bf16x2(pv[0], pv[1]);
        pk[2 * q4 + 1] = pack_bf16x2(pv[2], pv[3]);
        dk[2 * q4] = pack_bf16x2(dsv[0], dsv[1]);
        dk[2 * q4 + 1] = pack_bf16x2(dsv[2], dsv[3]);
      }
      pb[s2] = __builtin_bit_cast(bf16x8, pk);
      dsb[s2] = __builtin_bit_cast(bf16x8, dk);
    }
  } else {
    // d = 128 has no registers to spare for values held across a branch: P and dS
    // are made four rows at a time, the mask as a select
    const int key = kw0 + l32;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      u32x4 pk, dk;
#pragma unroll
      for (int q4 = 0; q4 < 2; ++q4) {
        const int j = 2 * s2 + q4;  // rows 8j + 4hi .. +4
        const f32x4 lv = *reinterpret_cast<const f32x4*>(reinterpret_cast<const uint8_t*>(lrow) + rvo + 32 * j);
        const f32x4 dv = *reinterpret_cast<const f32x4*>(reinterpret_cast<const uint8_t*>(drow) + rvo + 32 * j);
        float pv[4], dsv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float p = exp2_fast(__builtin_fmaf(s[4 * j + i], cs, -lv[i]));
          const int row = rbase + 8 * j + 4 * hi + i;
          if (MASK && need_mask && ((CAUSAL && key > row) || row >= N)) p = 0.f;
          pv[i] = p;
          dsv[i] = p * (dp[4 * j + i] - dv[i]);
        }
        pk[2 * q4] = pack_bf16x2(pv[0], pv[1]);
        pk[2 * q4 + 1] = pack_bf16x2(pv[2], pv[3]);
        dk[2 * q4] = pack_bf16x2(dsv[0], dsv[1]);
        dk[2 * q4 + 1] = pack_bf16x2(dsv[2], dsv[3]);
      }
      pb[s2] = __builtin_bit_cast(bf16x8, pk);
      dsb[s2] = __builtin_bit_cast(bf16x8, dk);
    }
  }
  // dV += P^T dO, dK += dS^T Q over the 32 rows (two 16-row steps)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int r0g = 16 * s2 * L::ROWB;
      dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pb[s2], tr_frag(gb_ + r0g, tlo[db], thi[db]), dva[db], 0, 0, 0);
      dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dsb[s2], tr_frag(qb_ + r0g, tlo[db], thi[db]), dka[db], 0, 0, 0);
    }
  sched_reads_ahead<4 * DB, 2, 3, kAhead>();
  debug_read_fence();
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (128-key block, K/V head, batch, chunk of the group's
// query heads), four key groups of 32 keys with two waves each: the waves of a
// group take the two 32-row halves of every 64-row tile and keep partial dK, dV,
// summed through LDS at the end.  For every query head of the chunk, Q and dO tiles
// of 64 rows (and the rows' L and D) stream through LDS (two buffers).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dlt,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, float* __restrict__ partK, float* __restrict__ partV,
    int B, int Hq, int Hkv, int N, int heads_per_chunk, int nchunks, float cs, float scale) {
  using L = BLay<D>;
  constexpr int KK = D / 16, DB = D / 32;
  constexpr int kAhead = ahead_dkdv<D>();
  // Q and dO tiles, two buffers each.  At d = 128 the four are separate arrays, so the
  // compiler can tell a tile's reads from the next item's copies into the other
  // buffers and does not wait for those copies mid-tile; at d = 64 one array (with
  // that wait) measured faster.
  constexpr bool kSplitBufs = D == 128;
  // row values first: their addresses then fit the 16-bit offset of an LDS read
  __shared__ __attribute__((aligned(16))) float rowv[2][2][kTile];  // [buffer][L2, D][row]
  __shared__ __attribute__((aligned(16))) uint8_t sm0[kSplitBufs ? L::TBYTES : 4 * L::TBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t sm1[kSplitBufs ? L::TBYTES : 16];
  __shared__ __attribute__((aligned(16))) uint8_t sm2[kSplitBufs ? L::TBYTES : 16];
  __shared__ __attribute__((aligned(16))) uint8_t sm3[kSplitBufs ? L::TBYTES : 16];
  __shared__ __attribute__((aligned(16))) uint8_t smv[kVinLds<D> ? kBlockRows * L::ROWB : 16];  // V rows (kVinLds)
  uint8_t* const smq0 = sm0;
  uint8_t* const smq1 = kSplitBufs ? sm1 : sm0 + L::TBYTES;
  uint8_t* const smg0 = kSplitBufs ? sm2 : sm0 + 2 * L::TBYTES;
  uint8_t* const smg1 = kSplitBufs ? sm3 : sm0 + 3 * L::TBYTES;

  const int G = Hq / Hkv;
  const int per_kb = B * Hkv * nchunks;
  const int kb = blockIdx.x / per_kb;  // key blocks in order: the first have the most rows (causal)
  const int rem = blockIdx.x % per_kb;
  const int chunk = rem % nchunks;
  const int bg = rem / nchunks;
  const int b = bg / Hkv, g = bg % Hkv;
  const int h_begin = g * G + chunk * heads_per_chunk;
  const int nh = min(heads_per_chunk, (g + 1) * G - h_begin);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = w & (kBwdWaves - 1);  // key group
  const int rh = w / kBwdWaves;        // row half of every 64-row tile
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int kw0 = kb * kBlockRows + kg * kWaveRows;  // this wave's first key
  const int key = kw0 + l32;

  const size_t kvoff = (size_t)(b * Hkv + g) * N;
  // K and V rows as B operands (K^T, V^T fragments): key, d = kk*16 + hi*8 .. +8
  bf16x8 kf[KK], vf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (key < N) {
      x = ld16(K + (kvoff + key) * D + kk * 16 + hi * 8);
      if (!kVinLds<D>) y = ld16(V + (kvoff + key) * D + kk * 16 + hi * 8);
    }
    kf[kk] = __builtin_bit_cast(bf16x8, x);
    vf[kk] = __builtin_bit_cast(bf16x8, y);
  }
  // kVinLds: the group's 32 V rows (key-major, 16-byte chunks swizzled like the Q
  // tiles, so the fragment reads of 16 consecutive keys are conflict-free); each of
  // the group's two waves stores half of the chunks.  The first barrier below orders
  // these writes before any read.
  if constexpr (kVinLds<D>) {
#pragma unroll
    for (int k2 = 0; k2 < KK / 2; ++k2) {
      const int kk = rh * (KK / 2) + k2;
      u32x4 y = {0u, 0u, 0u, 0u};
      if (key < N) y = ld16(V + (kvoff + key) * D + kk * 16 + hi * 8);
      *reinterpret_cast<u32x4*>(smv + (kg * kWaveRows + l32) * L::ROWB + (((2 * kk + hi) ^ L::swz(l32)) << 4)) = y;
    }
  }
  f32x16 dka[DB], dva[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dka[db][r] = 0.f;
      dva[db][r] = 0.f;
    }

  // lane offsets into the tiles, rows of this wave's half (adding 32 rows keeps the
  // swizzle, which depends on the row's low four bits)
  const int half = rh * kWaveRows * L::ROWB;
  int roff[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) roff[kk] = half + l32 * L::ROWB + (((2 * kk + hi) ^ L::swz(l32)) << 4);
  int tlo[DB], thi[DB];
  tr_offsets<D>(lane, tlo, thi);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    tlo[db] += half;
    thi[db] += half;
  }
  const int rvo = (rh * kWaveRows + 4 * hi) * 4;  // byte offset of the lane's first row value
  const uint32_t cp = copy_offset<D, kKvWaves>(w, lane);
  const uint32_t head_bytes = (uint32_t)N * D * 2;

  // (head, row tile) items in order; causal: rows before the block's first key are skipped
  const int nt = (N + kTile - 1) / kTile;
  const int t_first = CAUSAL ? (kb * kBlockRows) / kTile : 0;
  const int per_head = nt - t_first;
  const int n_lead = CAUSAL ? min(2, per_head) : 0;
  const int tail = (N % kTile != 0 && per_head > n_lead) ? 1 : 0;
  const int nu = per_head - n_lead - tail, nm = n_lead + tail;
  const int n_un = nh * nu;
  const int total = nh * per_head;

  const ItemSrc src{Q, dO, L2, Dlt, b, Hq, N, h_begin, t_first, nt, n_lead, nu, nm, n_un, head_bytes, cp, w, lane};
  if (total > 0) issue_item<D>(src, smq0, smg0, rowv, 0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();

  // restrict LDS pointers at d = 128 (see the tile buffers above)
  using RP = std::conditional_t<kSplitBufs, const uint8_t* __restrict__, const uint8_t*>;
  using RF = std::conditional_t<kSplitBufs, const float* __restrict__, const float*>;
  // one item in buffer u (= item parity): start the next item's copies, process this
  // one, wait for the next to land
  auto step = [&](auto mask_c, auto u_c, int item) {
    constexpr bool MASK = decltype(mask_c)::value;
    constexpr int u = decltype(u_c)::value;
    if (item + 1 < total) issue_item<D>(src, u ? smq0 : smq1, u ? smg0 : smg1, rowv, item + 1, 1 - u);
    debug_copy_fence();
    int h, t;
    item_pos(src, item, h, t);
    const int rbase = t * kTile + rh * kWaveRows;  // the half's rows: rbase + 8j + 4hi + i
    // causal: a tile whose last row precedes the wave's first key adds nothing (only
    // masked items can be such tiles)
    const bool skip = MASK && CAUSAL && (rbase + kWaveRows - 1 < kw0);
    if (!skip) {
      // the lane's entry is valid for key <= row < N
      const bool need_mask = (CAUSAL && rbase < kw0 + kWaveRows - 1) || (rbase + kWaveRows > N);
      dkdv_tile<D, CAUSAL, MASK, RP, RF>(u ? smq1 : smq0, u ? smg1 : smg0, rowv[u][0], rowv[u][1], need_mask, rbase, kw0,
                                         N, cs, roff, tlo, thi, rvo, kf, vf, smv + kg * kWaveRows * L::ROWB, dka, dva);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  };
  using F = std::false_type;
  using T = std::true_type;
  using U0 = std::integral_constant<int, 0>;
  using U1 = std::integral_constant<int, 1>;
  // the unmasked items, then the masked ones (item i always uses buffer i & 1)
  for (int i0 = 0; i0 < n_un; i0 += 2) {
    step(F{}, U0{}, i0);
    if (i0 + 1 < n_un) step(F{}, U1{}, i0 + 1);
  }
  int i1 = n_un;
  if (i1 < total && (i1 & 1)) step(T{}, U1{}, i1++);
  for (; i1 < total; i1 += 2) {
    step(T{}, U0{}, i1);
    if (i1 + 1 < total) step(T{}, U1{}, i1 + 1);
  }

  // the two row halves of each key group are summed through LDS (the first tile
  // buffer is free now: 16 KB per pass, one 32-column block of dK or dV per pass);
  // the first half writes
  {
    float* rbuf = reinterpret_cast<float*>(sm0);
#pragma unroll
    for (int pass = 0; pass < 2 * DB; ++pass) {
      f32x16& acc = pass < DB ? dka[pass] : dva[pass - DB];
      if (rh == 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) rbuf[(kg * 16 + r) * 64 + lane] = acc[r];
      }
      __syncthreads();
      if (rh == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] += rbuf[(kg * 16 + r) * 64 + lane];
      }
      __syncthreads();
    }
  }
  if (rh != 0) return;
  // lane holds keys kw0 + 8(r/4) + 4hi + r%4 at d = db*32 + l32
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int kr = kw0 + 8 * (r >> 2) + 4 * hi + (r & 3);
    if (kr >= N) continue;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const size_t idx = (kvoff + kr) * D + db * 32 + l32;
      if (nchunks == 1) {
        dK[idx] = __builtin_bit_cast(uint16_t, to_bf16(dka[db][r] * scale));
        dV[idx] = __builtin_bit_cast(uint16_t, to_bf16(dva[db][r]));
      } else {
        const size_t pidx = (size_t)chunk * B * Hkv * N * D + idx;
        partK[pidx] = dka[db][r] * scale;
        partV[pidx] = dva[db][r];
      }
    }
  }
}

// Sum of the head-chunk partials of dK and dV, rounded to bf16.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const float* __restrict__ partK, const float* __restrict__ partV,
                                                         uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
                                                         long long n, int nchunks) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float sk = 0.f, sv = 0.f;
  for (int c = 0; c < nchunks; ++c) {
    sk += partK[(size_t)c * n + i];
    sv += partV[(size_t)c * n + i];
  }
  dK[i] = __builtin_bit_cast(uint16_t, to_bf16(sk));
  dV[i] = __builtin_bit_cast(uint16_t, to_bf16(sv));
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_t(const BwdArgs& a) {
  hipStream_t st = (hipStream_t)a.stream;
  const BwdPlan pl = bwd_plan(a.B, a.Hq, a.Hkv, a.N, a.d);
  float* dlt = (float*)a.workspace;
  float* l2 = (float*)((uint8_t*)a.workspace + pl.l2_offset);
  float* partK = (float*)((uint8_t*)a.workspace + pl.part_offset);
  float* partV = partK + pl.part_elems;
  const long long rows = (long long)a.B * a.Hq * a.N;
  constexpr int LPR = D / 8;
  hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)((rows * LPR + 255) / 256)), dim3(256), 0, st,
                     (const uint16_t*)a.o, (const uint16_t*)a.dout, a.lse, dlt, l2, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float cs = a.scale * kLog2e;
  const int nqb_dq = (a.N + kDqRows - 1) / kDqRows;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)(nqb_dq * a.B * a.Hq)), dim3(kDqWaves * 64), 0, st,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout, a.lse,
                     dlt, (uint16_t*)a.dq, a.B, a.Hq, a.Hkv, a.N, cs, a.scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nkb = (a.N + kBlockRows - 1) / kBlockRows;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)(nkb * a.B * a.Hkv * pl.nchunks)),
                     dim3(kBwdThreads), 0, st, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (const uint16_t*)a.dout, l2, dlt, (uint16_t*)a.dk, (uint16_t*)a.dv, partK, partV, a.B, a.Hq,
                     a.Hkv, a.N, pl.heads_per_chunk, pl.nchunks, cs, a.scale);
  e = hipGetLastError();
  if (e != hipSuccess || pl.nchunks == 1) return e;
  const long long n = (long long)a.B * a.Hkv * a.N * D;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, partK, partV,
                     (uint16_t*)a.dk, (uint16_t*)a.dv, n, pl.nchunks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a) {
  if (a.d == 64) return a.causal ? launch_bwd_t<64, true>(a) : launch_bwd_t<64, false>(a);
  return a.causal ? launch_bwd_t<128, true>(a) : launch_bwd_t<128, false>(a);
}

}  // namespace fa
