// bf16 exact-attention forward on gfx950 matrix cores.
//
// The FlashAttention forward of "Phase 08 -- Inference Optimization at Depth"
// (Concepts list: online softmax, FlashAttention tiling, causal tiles handled
// apart; Lab 01 steps 2 and 4) with the query-block parallelism of getnybble
// "Inference Optimization -- Advanced", question 5, and the grouped K/V heads of
// the screna.ai MHA/MQA/GQA block.
//
// Work decomposition: one item per (256-row query block, query head, batch), taken by
// a workgroup of 8 waves (two per SIMD); the plain forward runs one persistent
// workgroup per compute unit over a static list of items (fwd_bf16_persistent_kernel),
// the windowed, ALiBi and paged forms one workgroup per item, and the split-K form one
// workgroup per chunk of an item's key tiles.  Each wave owns 32 query rows and keeps their Q
// fragments in registers for the whole pass.  K/V are streamed in tiles of 64
// keys (128 at d = 64) through two LDS buffers: the next tile is copied
// HBM -> LDS by 128-bit buffer loads with the LDS-destination bit (no staging
// registers; rows past N read as zero) while the current one is consumed.  Rows are stored unpadded
// with their 16-byte chunks XOR-swizzled by row, so the b128 K reads and the
// transposing V reads both hit distinct LDS banks.  Per tile and wave:
//   S^T = K Q^T  with v_mfma_f32_32x32x16_bf16 (K from LDS is the A operand, so
//                every lane ends up holding 16 keys of one query row),
//   online softmax in the log2 domain (row max over the lane's keys plus one
//                permlane32 swap; exp2 with scale*log2e folded into one FMA),
//   O^T += V^T P^T with the same MFMA; V^T fragments come straight from the
//                row-major LDS tile through ds_read_b64_tr_b16, and P stays in
//                the registers the S MFMA produced (the key order inside a
//                16-key step is permuted identically on both operands).
// The two waves sharing a SIMD interleave one's exponentials with the other's
// matrix instructions.
//
// Rescaling (the running-max recurrence): the max m used in the exponentials is
// raised only when a row's tile max exceeds it by more than kRescaleThreshold
// (log2 units), and then O and the sums are multiplied by exp2(m_old - m_new);
// otherwise the previous m is kept, so probabilities stay below 2^threshold and
// the vector-ALU rescale of O is skipped.  The same m is used for O, l and L,
// so this computes the same exact attention.  O is normalised by the sum of the
// bf16-rounded probabilities that actually entered the P V product (one bf16
// dot2 per pair), so O is a weighted mean with consistent weights; L uses the
// fp32 sum of the unrounded probabilities.
//
// Causal: tiles wholly above a wave's rows are skipped, tiles crossing the
// diagonal (or the ragged end of the sequence) take the masked path, every other
// tile runs mask-free; no tile past the block's last row is ever loaded.
// Only O (bf16) and L (fp32) are written.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kRowsPerWave = 32;            // one 32-row MFMA block per wave
#ifndef FA_PREFILL_WAVES
#define FA_PREFILL_WAVES 8
#endif
constexpr int kWaves = FA_PREFILL_WAVES;    // waves per workgroup (8: two per SIMD)
constexpr int kThreads = kWaves * 64;
constexpr int kBR = kWaves * kRowsPerWave;  // 256 query rows per workgroup
static_assert(kBR == kGeomFwdRows && kThreads == kGeomFwdThreads, "host-side launch limits assume this geometry");
constexpr float kRescaleThreshold = 8.0f;   // log2 units: probabilities stay <= 256
constexpr int kPrefetch = 4;                // LDS fragment reads kept ahead of the MFMAs
#ifndef FA_PREFILL_STAGES
#define FA_PREFILL_STAGES 2
#endif
constexpr int kStages = FA_PREFILL_STAGES;  // K/V tiles resident in LDS (copies run kStages-1 ahead)

template <int D>
struct Lay {
  static constexpr int ROWB = D * 2;            // bytes per K/V row in LDS (unpadded)
  static constexpr int CPR = ROWB / 16;         // 16-byte chunks per row
  static constexpr int RPB = 1024 / ROWB;       // rows per 1 KB wave copy (64 lanes x 16 B)
  // Keys per tile: 64 at d = 128 (two 32-key MFMA blocks), 128 at d = 64, where a
  // tile's matrix work per key is half as large and the wider tile halves the
  // barriers and copy waits per key.
  static constexpr int BC = D == 64 ? 128 : 64;
  static constexpr int NA = BC / 32;            // 32-key MFMA blocks per tile
  static constexpr int TBYTES = BC * ROWB;      // one tensor tile
  static constexpr int BLOCKS = TBYTES / 1024;  // 1 KB copies per tensor tile
  static constexpr int BPW = BLOCKS / kWaves;   // ... per wave
  static_assert(BPW * kWaves == BLOCKS, "tile copy must split evenly over the waves");
  // Chunk swizzles (physical chunk = logical chunk ^ swz(row)).
  // K: the 16 rows read together by a b128 instruction land on 16 distinct
  //    16-byte bank groups.
  __host__ __device__ static constexpr int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  // V: each 16-lane group of a transposing read touches 4 rows x 32 bytes; the
  //    swizzle moves whole 32-byte pairs so the 8 (row, pair) accesses of a
  //    32-lane half are bank-disjoint.
  __host__ __device__ static constexpr int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

__device__ __forceinline__ u32x4 ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

typedef short s16x8 __attribute__((ext_vector_type(8)));

// s_waitcnt vmcnt(n * L): wait until at most n tiles' worth (L loads each) of this
// wave's HBM -> LDS copies are outstanding.  n is 0 .. kStages-2.
template <int L>
__device__ __forceinline__ void wait_vmem_tiles(int n) {
  static_assert(L * (kStages - 2) < 64, "vmcnt field is 6 bits");
  auto enc = [](int v) { return 0x0F70 | (v & 15) | ((v >> 4) << 14); };
  if (kStages > 3 && n >= 2) {
    __builtin_amdgcn_s_waitcnt(enc(2 * L));
  } else if (kStages > 2 && n == 1) {
    __builtin_amdgcn_s_waitcnt(enc(L));
  } else {
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }
}

// Per-wave state carried across tiles.
template <int D>
struct WaveState {
  static constexpr int KK = D / 16;
  static constexpr int DB = D / 32;
  bf16x8 qf[KK];     // Q^T fragments (B operand)
  f32x16 oacc[DB];   // O^T accumulators: lane holds row l%32, 16 d values per block
  float m_run;       // max used in the exponentials (log2 units)
  float l_exact;     // this lane's partial sum of fp32 probabilities (for L)
  float l_round;     // ... of the bf16-rounded probabilities (for O)
};

// Row max of one tile's scores (masked where needed), in log2 units.
// lim: largest key offset (within the tile, minus the lane's 4*hi) that is visible.
template <bool MASK, int NA>
__device__ __forceinline__ float tile_rowmax(f32x16 (&s)[NA], int lim, float c) {
  float mx = -INFINITY;
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (MASK) {
        const int koff = a * 32 + 8 * (r >> 2) + (r & 3);
        s[a][r] = (koff <= lim) ? s[a][r] : -INFINITY;
      }
      mx = fmaxf(mx, s[a][r]);
    }
  mx = max_xor32(mx);
  return mx * c;  // c > 0, so -inf stays -inf
}

// Same with the mask applied only when need_mask (wave-uniform) is set: one code
// path for masked and unmasked tiles, so the accumulators are not copied between
// two register assignments where the paths would rejoin.
template <int NA>
__device__ __forceinline__ float tile_rowmax_rt(f32x16 (&s)[NA], int lim, float c, bool need_mask) {
  if (need_mask) {
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int koff = a * 32 + 8 * (r >> 2) + (r & 3);
        s[a][r] = (koff <= lim) ? s[a][r] : -INFINITY;
      }
  }
  return tile_rowmax<false>(s, lim, c);
}

// Raise the running max of rows whose tile max exceeds it by more than the
// threshold, rescaling O and the sums.  Wave-uniform branch.
// SAFE: a row may still be at m_run = -inf when another row of the wave grows (only
// with a sliding window); its factor is then 0 (its O and sums are still zero).
template <int D, bool SAFE = false>
__device__ __forceinline__ void maybe_rescale(WaveState<D>& st, float mt) {
  const bool grow = mt > st.m_run + kRescaleThreshold;
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
    const float mnew = fmaxf(st.m_run, mt);
    float alpha = exp2_fast(st.m_run - mnew);  // m_run = -inf, mnew finite -> 0
    if (SAFE && st.m_run == -INFINITY) alpha = 0.f;
    st.l_exact *= alpha;
    st.l_round *= alpha;
#pragma unroll
    for (int db = 0; db < WaveState<D>::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.oacc[db][r] *= alpha;
    st.m_run = mnew;
  }
}

// exp2 of the scores against the running max, packed to bf16 as the B operand of
// the P V product; fp32 and bf16-rounded row sums.  Masked scores are -inf and
// c > 0, so their probability is exactly 0.
// SAFE: the row may not have seen a visible key yet (m_run = -inf, possible only
// with a sliding window); its masked scores then give exp2(-inf - 0) = 0.
// REL: the scores already are log2-domain logits relative to the running max, so
// the probabilities are their plain exponentials.
template <int D, bool SAFE = false, bool REL = false>
__device__ __forceinline__ void softmax_pack(const f32x16 (&s)[Lay<D>::NA], WaveState<D>& st, float c,
                                             bf16x8 (&pb)[Lay<D>::NA][2]) {
  const float m = (SAFE && st.m_run == -INFINITY) ? 0.f : st.m_run;
  const bf16x2 ones = as_bf16x2(0x3f803f80u);
  float psum = 0.f, rsum = 0.f;
#pragma unroll
  for (int a = 0; a < Lay<D>::NA; ++a)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      u32x4 pk;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = REL ? exp2_fast(s[a][h2 * 8 + 2 * j]) : exp2_fast(__builtin_fmaf(s[a][h2 * 8 + 2 * j], c, -m));
        const float p1 =
            REL ? exp2_fast(s[a][h2 * 8 + 2 * j + 1]) : exp2_fast(__builtin_fmaf(s[a][h2 * 8 + 2 * j + 1], c, -m));
        psum += p0;
        psum += p1;
        const uint32_t w2 = pack_bf16x2(p0, p1);
        rsum = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w2), ones, rsum, false);
        pk[j] = w2;
      }
      pb[a][h2] = __builtin_bit_cast(bf16x8, pk);
    }
  st.l_exact += psum;
  st.l_round += rsum;
}

// Causal ALiBi's key term as a rank-one MFMA update: A rows (keys a*32 + l32) hold
// slope2/c times the key's offset in the tile, split into three bf16 parts (k = 0..2),
// and B columns hold ones there, so the product adds slope2 * offset / c to every
// score of that key.  Lanes of the upper half hold zeros (k = 8..15).
struct AlibiExt {
  bf16x8 a[4];  // one per 32-key block of the tile (two or four used)
  bf16x8 b;
};

// EXT: sliding window and/or ALiBi.  The scores are first turned into log2-domain
// logits x = s*c - slope2*|i - j| (slope2 = ALiBi slope * log2 e; base = i - j0 - 4hi,
// so i - j = base - koff), masked on both sides (lo <= koff <= lim), then fed to
// the same online softmax with unit scale.
// kb and vb are restrict: the copies in flight during a tile only write the other
// LDS slot (every read of a slot follows the wait and barrier that end the slot's
// copy), which lets the compiler drop the wait for all outstanding HBM -> LDS
// copies that it would otherwise put before the first transposing V read.
// RTMASK: plain path with the mask decided at run time by need_mask.
// SPLIT (causal ALiBi, wave-uniform): the probabilities enter the P V product as two
// bf16 parts, bf16(p) and bf16(p - bf16(p)), one MFMA each.  Used on the tiles nearest
// a wave's diagonal, where steep slopes put almost all of a row's weight on a few
// keys: the rounding of those few weights to bf16 (2^-9 relative) would otherwise
// reach O directly, while over many keys the roundings average out.
template <int D, bool MASK, bool EXT, bool LIN = false, bool RTMASK = false, bool SPLIT = false>
__device__ __forceinline__ void process_tile(WaveState<D>& st, const uint8_t* __restrict__ kb,
                                             const uint8_t* __restrict__ vb,
                                             const int (&koff)[D / 16], const int (&voff)[D / 32], int lim,
                                             int l32, float c, int lo = 0, float base = 0.f, float slope2 = 0.f,
                                             const AlibiExt* ax = nullptr, bool need_mask = false) {
  using LY = Lay<D>;
  constexpr int KK = D / 16;
  constexpr int DB = D / 32;
  constexpr int NA = LY::NA;

  // ---- scores S^T = K Q^T; K fragment: key a*32 + l32, d = kk*16 + hi*8 .. +8
  f32x16 sc[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[a][r] = 0.f;
  if constexpr (EXT && LIN) {
#pragma unroll
    for (int a = 0; a < NA; ++a) sc[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ax->a[a], ax->b, sc[a], 0, 0, 0);
  }
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kb + (a * 32 + l32) * LY::ROWB + koff[kk]);
      sc[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, st.qf[kk], sc[a], 0, 0, 0);
    }
  // schedule: kPrefetch fragment reads in flight ahead of the MFMA that consumes them
  if constexpr (EXT && LIN) __builtin_amdgcn_sched_group_barrier(0x008, NA, 0);  // the ALiBi updates first
  __builtin_amdgcn_sched_group_barrier(0x100, kPrefetch, 0);  // LDS reads
#pragma unroll
  for (int i = 0; i < NA * KK - kPrefetch; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, kPrefetch, 0);
  debug_read_fence();

  // ---- online softmax
  bf16x8 pb[NA][2];
  bf16x8 pbl[NA][2];  // SPLIT: second bf16 parts
  if constexpr (EXT && LIN) {
    // Causal: a visible key never lies after its row, so the ALiBi term
    // -slope2 |i - j| = slope2 (kofs + 4hi) - slope2 (base + 4hi) is affine in the key
    // offset.  The MFMA update above already added slope2 (kofs + 4hi) / c to the
    // scores.  The logits are taken relative to ref (the running max; 0 before the
    // row's first visible key): y = s' c - (slope2 (base + 4hi) + ref).  When the max
    // is raised they are shifted to the new one, so the probabilities are plain exp2(y).
    const float ref = st.m_run == -INFINITY ? 0.f : st.m_run;
    const float nb = -__builtin_fmaf(slope2, base + (float)(4 * (int)(__lane_id() >> 5)), ref);
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kofs = a * 32 + 8 * (r >> 2) + (r & 3);
        const float y = __builtin_fmaf(sc[a][r], c, nb);
        sc[a][r] = (!MASK || (kofs <= lim && kofs >= lo)) ? y : -INFINITY;
      }
    const float mt = tile_rowmax<false>(sc, 0, 1.f) + ref;  // tile max in absolute units
    const bool grow = mt > st.m_run + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float mnew = fmaxf(st.m_run, mt);
      float alpha = exp2_fast(st.m_run - mnew);
      if (st.m_run == -INFINITY) alpha = 0.f;
      st.l_exact *= alpha;
      st.l_round *= alpha;
#pragma unroll
      for (int db = 0; db < WaveState<D>::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.oacc[db][r] *= alpha;
      st.m_run = mnew;
      const float sh = mnew == -INFINITY ? 0.f : mnew - ref;
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[a][r] -= sh;
    }
    softmax_pack<D, true, true>(sc, st, 1.f, pb);
    if constexpr (SPLIT) {
      // the second bf16 part of each probability (p = exp2(y), as in softmax_pack)
      const bf16x2 ones = as_bf16x2(0x3f803f80u);
      float rlo = 0.f;
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const u32x4 hk = __builtin_bit_cast(u32x4, pb[a][h2]);
          u32x4 lk;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float p0 = exp2_fast(sc[a][h2 * 8 + 2 * j]);
            const float p1 = exp2_fast(sc[a][h2 * 8 + 2 * j + 1]);
            const uint32_t hw = hk[j];
            lk[j] = pack_bf16x2(p0 - bf16lo_to_f32(hw), p1 - bf16hi_to_f32(hw));
            rlo = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(lk[j]), ones, rlo, false);
          }
          pbl[a][h2] = __builtin_bit_cast(bf16x8, lk);
        }
      st.l_round += rlo;
    }
  } else if constexpr (EXT) {
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kofs = a * 32 + 8 * (r >> 2) + (r & 3);
        const float x = __builtin_fmaf(sc[a][r], c, -slope2 * fabsf(base - (float)kofs));
        sc[a][r] = (!MASK || (kofs <= lim && kofs >= lo)) ? x : -INFINITY;
      }
    const float mt = tile_rowmax<false>(sc, 0, 1.f);
    maybe_rescale<D, true>(st, mt);
    softmax_pack<D, true>(sc, st, 1.f, pb);
  } else {
    const float mt = RTMASK ? tile_rowmax_rt(sc, lim, c, need_mask) : tile_rowmax<MASK>(sc, lim, c);
    maybe_rescale<D>(st, mt);
    softmax_pack<D>(sc, st, c, pb);
  }

  // ---- O^T += V^T P^T.  V^T fragment for (a, h2, db): keys a*32 + h2*16 + 4*hi +
  // {0..3, 8..11}, d = db*32 + l32, via two transposing reads of 4 keys each
  // (voff[db] holds this lane's row-in-group and swizzled chunk offset).
  // (scheduling fence: the V fragment reads are not hoisted into the score phase,
  // where their registers would push the wave past its 256-register budget)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint8_t* p1 = vb + (a * 32 + h2 * 16) * LY::ROWB + voff[db];
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(p1));
        const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(p1 + 8 * LY::ROWB));
        const s16x8 cat = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
        st.oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cat), pb[a][h2],
                                                              st.oacc[db], 0, 0, 0);
      }
  // same schedule for the V fragments (two transposing reads per MFMA)
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPrefetch, 1);
#pragma unroll
  for (int i = 0; i < 2 * NA * DB - kPrefetch; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, kPrefetch, 1);
  debug_read_fence();
  if constexpr (EXT && LIN) {
    if constexpr (SPLIT) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const uint8_t* p1 = vb + (a * 32 + h2 * 16) * LY::ROWB + voff[db];
            const s16x4 vlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(p1));
            const s16x4 vup = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(p1 + 8 * LY::ROWB));
            const s16x8 cat = __builtin_shufflevector(vlo, vup, 0, 1, 2, 3, 4, 5, 6, 7);
            st.oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cat), pbl[a][h2],
                                                                  st.oacc[db], 0, 0, 0);
          }
    }
  }
}

// HBM -> LDS copy of one K/V tile into buffer buf: this wave's 1 KB blocks
// w, w + 8, ... of each tensor; kcp/vcp are the lane's byte offsets within the
// tile's rows (swizzle included), to which the tile's first-row offset is added.
// The buffer descriptors span one head's K (V) rows, so rows past N read as zero.
template <int D>
__device__ __forceinline__ void copy_tile(uint8_t* smem, const void* kbase, const void* vbase, uint32_t head_bytes,
                                          const uint32_t* kcp, const uint32_t* vcp,
                                          int j0, int buf, int w) {
  using LY = Lay<D>;
  const auto krs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(kbase), (short)0, head_bytes, 0x00020000);
  const auto vrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(vbase), (short)0, head_bytes, 0x00020000);
  // LDS slots: K tiles in slots 0 .. kStages-1, V tiles in slots kStages .. 2*kStages-1
  uint8_t* kb = smem + buf * LY::TBYTES;
  uint8_t* vb = smem + (kStages + buf) * LY::TBYTES;
  const uint32_t base = (uint32_t)j0 * LY::ROWB;
#pragma unroll
  for (int i = 0; i < LY::BPW; ++i) {
    const int blk = w + kWaves * i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (FA_LDS void*)(kb + blk * 1024), 16, base + kcp[i], 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (FA_LDS void*)(vb + blk * 1024), 16, base + vcp[i], 0, 0, 0);
  }
}

// PAGED: chunked prefill over a paged cache.  B counts sequences and N is the
// chunk length C; sequence s holds ctxl[s] >= C cached tokens in 16-token pages
// (K, V are the page pools [pages][Hkv][16][D], table the page table), the chunk
// rows sit at positions ctxl[s] - C + r and the attention is causal in positions.
// HBM -> LDS copy of one K/V tile (keys j0 .. j0+BC-1, BC/16 16-token pages) from the
// page pools, into buffer buf with the same swizzled layout as copy_tile.  Each 1 KB
// block lies in one page (slot rows pr0 .. pr0 + RPB - 1); its buffer descriptor
// spans only the page's valid slots (below nk), so slots past the context -- and
// whole pages past it, whose table entries are never read -- land as zeros.
template <int D>
__device__ __forceinline__ void copy_tile_paged(uint8_t* smem, const uint16_t* kpool, const uint16_t* vpool,
                                                const int32_t* trow, int nk, int num_pages, int Hkv, int g, int j0,
                                                int buf, int w, int lane) {
  using LY = Lay<D>;
  uint8_t* kb = smem + buf * LY::TBYTES;
  uint8_t* vb = smem + (kStages + buf) * LY::TBYTES;
#pragma unroll
  for (int i = 0; i < LY::BPW; ++i) {
    const int blk = w + kWaves * i;
    const int r0 = blk * LY::RPB;                 // tile row of the block's first row
    const int tp = (j0 + r0) / 16;                // logical page
    // wave-uniform by construction; kept in scalar registers so that the buffer
    // descriptors are too (a vector clamp here made the compiler wrap every copy in
    // a loop over distinct descriptor values)
    const int valid = __builtin_amdgcn_readfirstlane(min(max(nk - tp * 16, 0), 16));
    const int id = valid > 0 ? trow[tp] : 0;
    const int pid = (unsigned)id < (unsigned)num_pages ? id : num_pages - 1;  // ids stay inside the pools
    const size_t head = ((size_t)pid * Hkv + g) * 16 * D;
    const auto krs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kpool + head), (short)0,
                                                       (uint32_t)valid * LY::ROWB, 0x00020000);
    const auto vrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vpool + head), (short)0,
                                                       (uint32_t)valid * LY::ROWB, 0x00020000);
    const int r = r0 + lane / LY::CPR;            // tile row this lane copies
    const int pc = lane % LY::CPR;
    const uint32_t ko = (r % 16) * LY::ROWB + ((pc ^ LY::swz_k(r)) << 4);
    const uint32_t vo = (r % 16) * LY::ROWB + ((pc ^ LY::swz_v(r)) << 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (FA_LDS void*)(kb + blk * 1024), 16, ko, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (FA_LDS void*)(vb + blk * 1024), 16, vo, 0, 0, 0);
  }
}

// Page ids of one K/V tile of the paged cache (keys j0 .. j0 + BC - 1), one per lane:
// lane i holds the table entry of page j0 / 16 + i.  One vector load through a buffer
// descriptor spanning the sequence's pages with tokens, so lanes past them read 0.
// The loop loads the ids a tile ahead of the copy that uses them, so the copy does not
// wait for a page-table read.
template <int D>
__device__ __forceinline__ int load_tile_page_ids(const int32_t* trow, int nk, int j0, int lane) {
  const uint32_t bytes = (uint32_t)((nk + 15) / 16) * 4;
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(trow), (short)0, bytes, 0x00020000);
  return (int)__builtin_amdgcn_raw_buffer_load_b32(rs, (j0 / 16 + lane) * 4, 0, 0);
}

// copy_tile_paged with the tile's page ids already in a register (load_tile_page_ids).
template <int D>
__device__ __forceinline__ void copy_tile_paged_ids(uint8_t* smem, const uint16_t* kpool, const uint16_t* vpool,
                                                    int idv, int nk, int num_pages, int Hkv, int g, int j0, int buf,
                                                    int w, int lane) {
  using LY = Lay<D>;
  uint8_t* kb = smem + buf * LY::TBYTES;
  uint8_t* vb = smem + (kStages + buf) * LY::TBYTES;
#pragma unroll
  for (int i = 0; i < LY::BPW; ++i) {
    const int blk = w + kWaves * i;
    const int r0 = blk * LY::RPB;
    const int tp = (j0 + r0) / 16;
    const int valid = __builtin_amdgcn_readfirstlane(min(max(nk - tp * 16, 0), 16));
    const int id = __builtin_amdgcn_readlane(idv, r0 / 16);  // j0 is a multiple of 16
    const int pid = (unsigned)id < (unsigned)num_pages ? id : num_pages - 1;
    const size_t head = ((size_t)pid * Hkv + g) * 16 * D;
    const auto krs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kpool + head), (short)0,
                                                       (uint32_t)valid * LY::ROWB, 0x00020000);
    const auto vrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vpool + head), (short)0,
                                                       (uint32_t)valid * LY::ROWB, 0x00020000);
    const int r = r0 + lane / LY::CPR;
    const int pc = lane % LY::CPR;
    const uint32_t ko = (r % 16) * LY::ROWB + ((pc ^ LY::swz_k(r)) << 4);
    const uint32_t vo = (r % 16) * LY::ROWB + ((pc ^ LY::swz_v(r)) << 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (FA_LDS void*)(kb + blk * 1024), 16, ko, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (FA_LDS void*)(vb + blk * 1024), 16, vo, 0, 0, 0);
  }
}

template <int D, bool CAUSAL, bool EXT, bool PAGED>
__global__ __launch_bounds__(kThreads, 8 / kWaves) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ Lse, int B, int Hq, int Hkv, int N,
    float c /* |scale| * log2(e), > 0 */, uint32_t qsign /* 0x80008000 if scale < 0 */,
    int window /* EXT: keys j >= i - window + 1 only (0: none) */, const float* __restrict__ slopes /* EXT: ALiBi */,
    const int32_t* __restrict__ table /* PAGED */, const int32_t* __restrict__ ctxl /* PAGED */,
    int max_pages /* PAGED */, int num_pages /* PAGED */, int split_tiles /* split-K: key tiles per chunk */,
    float* __restrict__ ws_o /* split-K: O partials */, float* __restrict__ ws_l /* split-K: lse partials */,
    int smax /* split-K: chunk slots per block */, int ws_rows /* split-K: rows of partials */) {
  using LY = Lay<D>;
  constexpr int KK = D / 16;
  constexpr int DB = D / 32;
  // The plain instantiation (no window, ALiBi or paging) is the split-K forward: each
  // workgroup takes one chunk of split_tiles key tiles of a (query block, head); a block
  // cut into several chunks leaves fp32 (O, lse) partials for fwd_split_merge_kernel.
  constexpr bool SPLIT = !EXT && !PAGED;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStages * LY::TBYTES];

  const int nqb = (N + kBR - 1) / kBR;
  const int G = Hq / Hkv;
  // Work order: (query block, batch, K/V head, query head in group), causal blocks
  // heaviest first; paged: (sequence, K/V head, query block, query head in group).
  // The workgroups that read the same K/V (the G query heads of a group, and when
  // paged also the chunk's query blocks) are consecutive in that order.  Workgroups
  // are dealt to the 8 XCDs round-robin by linear index, so runs of S consecutive
  // items are handed to one XCD and their K/V tiles are fetched from HBM once into
  // that XCD's L2.  Runs go to the XCDs in snake order (round k of runs: XCD x takes
  // run 8k + x, or 8k + 7 - x when k is odd): a run can be a whole causal query block
  // (S = 32 with one K/V head), and dealing the heaviest runs to the same XCDs every
  // round would leave the others idle at the end.  Slot s of XCD x takes item
  // c S + s % S, with run c from round k = s / S.  A ragged tail of fewer than 8 S
  // items keeps the plain order.
  const int S = PAGED ? G * nqb : G;
  int item = (int)blockIdx.x;
  if (!SPLIT && item < (int)(gridDim.x / (8 * S)) * 8 * S) {
    const int x = item & 7, slot = item >> 3, k = slot / S;
    item = (8 * k + ((k & 1) ? 7 - x : x)) * S + slot % S;
  }
  int qb, b, h;
  int split = 0, nsplit = 1;
  if constexpr (SPLIT) {
    // heaviest blocks first (causal); per block its chunks, per chunk the heads
    const int BH = B * Hq;
    qb = 0;
    for (int r = 0; r < nqb; ++r) {
      qb = CAUSAL ? nqb - 1 - r : r;
      const int kend_q = CAUSAL ? min(N, (qb + 1) * kBR) : N;
      nsplit = ((kend_q + LY::BC - 1) / LY::BC + split_tiles - 1) / split_tiles;
      if (item < nsplit * BH) break;
      item -= nsplit * BH;
    }
    split = item / BH;
    b = (item % BH) / Hq;
    h = (item % BH) % Hq;
  } else if constexpr (PAGED) {
    const int per_seq = Hkv * nqb * G;
    b = item / per_seq;
    const int r = item % per_seq;
    const int gg = r / (nqb * G), r2 = r % (nqb * G);
    qb = nqb - 1 - r2 / G;
    h = gg * G + r2 % G;
  } else {
    const int BH = B * Hq;
    qb = CAUSAL ? (nqb - 1 - item / BH) : item / BH;
    const int bh = item % BH;
    b = bh / Hq;
    h = bh % Hq;
  }
  const int g = h / G;

  const int tid = threadIdx.x;
  // paged: a wave-uniform index keeps each copy's page id (read back from a lane) and
  // its buffer descriptors in scalar registers
  const int w = PAGED ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;  // which half of the wave
  const int grp = lane >> 4, li = lane & 15;
  const int rw0 = qb * kBR + w * kRowsPerWave;
  const int qrow = rw0 + l32;

  const uint16_t* qbase = Q + ((size_t)(b * Hq + h) * N) * D;
  const uint16_t* kbase = K + (PAGED ? 0 : ((size_t)(b * Hkv + g) * N) * D);
  const uint16_t* vbase = V + (PAGED ? 0 : ((size_t)(b * Hkv + g) * N) * D);
  // keys and the position of query row 0 (the chunk's first token when paged)
  // (paged: the context is clamped to [chunk, page-table row], so a wrong device-side
  // value gives wrong output but every access stays inside the buffers)
  const int Nk = PAGED ? min(max(ctxl[b], N), max_pages * 16) : N;
  const int poff = PAGED ? Nk - N : 0;
  const int rw0p = rw0 + poff;
  const int qrowp = qrow + poff;
  const int32_t* trow = PAGED ? table + (size_t)b * max_pages : nullptr;

  WaveState<D> st;
  // Q fragments (B operand of S^T = K Q^T): row qrow, d = kk*16 + hi*8 .. +8
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qrow < N) x = ld_global16(qbase + (size_t)qrow * D + kk * 16 + hi * 8);
    x ^= qsign;
    st.qf[kk] = __builtin_bit_cast(bf16x8, x);
  }
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.oacc[db][r] = 0.f;
  st.m_run = -INFINITY;
  st.l_exact = 0.f;
  st.l_round = 0.f;

  // loop-invariant LDS byte offsets of this lane's fragment reads
  int koff[KK], voff[DB];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) koff[kk] = ((2 * kk + hi) ^ LY::swz_k(l32)) << 4;
  {
    const int vr = 4 * hi + (li >> 2);  // row within a 16-key step (the +8 read keeps the swizzle)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int lc = 4 * db + 2 * (grp & 1) + ((li & 3) >> 1);
      voff[db] = vr * LY::ROWB + ((lc ^ LY::swz_v(vr)) << 4) + (li & 1) * 8;
    }
  }

  const int kend = CAUSAL ? min(Nk, poff + (qb + 1) * kBR) : Nk;
  int ntiles = (kend + LY::BC - 1) / LY::BC;
  // sliding window: tiles wholly left of the block's first row's window are never loaded
  int t_begin = (EXT && window > 0) ? max(0, poff + qb * kBR - window + 1) / LY::BC : 0;
  if constexpr (SPLIT) {
    t_begin = split * split_tiles;
    ntiles = min(ntiles, t_begin + split_tiles);
  }
  const float slope2 = (EXT && slopes != nullptr) ? slopes[h] * kLog2e : 0.f;
  AlibiExt ax;
  if constexpr (EXT && CAUSAL) {
    // slope2 / c per unit of key offset (c > 0; with a zero scale c is tiny and the
    // scores' own term vanishes against the bias, as it does in exact arithmetic)
    const float ks = slope2 / c;
    auto rb = [](float x) { return __uint_as_float((uint32_t)__builtin_bit_cast(uint16_t, to_bf16(x)) << 16); };
#pragma unroll
    for (int a = 0; a < LY::NA; ++a) {
      u32x4 wv = {0u, 0u, 0u, 0u};
      if (hi == 0) {
        const float v = ks * (float)(a * 32 + l32);
        const float h0 = rb(v), h1 = rb(v - h0), h2 = rb(v - h0 - h1);
        wv[0] = pack_bf16x2(h0, h1);
        wv[1] = pack_bf16x2(h2, 0.f);
      }
      ax.a[a] = __builtin_bit_cast(bf16x8, wv);
    }
    u32x4 wb = {0u, 0u, 0u, 0u};
    if (hi == 0) {
      wb[0] = pack_bf16x2(1.f, 1.f);
      wb[1] = pack_bf16x2(1.f, 0.f);
    }
    ax.b = __builtin_bit_cast(bf16x8, wb);
  }

  // ---- HBM -> LDS copies of one K/V tile (buffer loads with the LDS bit).  Wave w
  // copies 1 KB blocks w, w + 8, ... of each tensor; lane l of a block writes
  // physical chunk l % CPR of row blk*RPB + l / CPR, which holds logical chunk
  // (l % CPR) ^ swz(row).  Rows past N lie past the buffer end and read as zero.
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  uint32_t kcp[LY::BPW], vcp[LY::BPW];
#pragma unroll
  for (int i = 0; i < LY::BPW; ++i) {
    const int blk = w + kWaves * i;
    const int r = blk * LY::RPB + lane / LY::CPR;
    const int pc = lane % LY::CPR;
    kcp[i] = r * LY::ROWB + ((pc ^ LY::swz_k(r)) << 4);
    vcp[i] = r * LY::ROWB + ((pc ^ LY::swz_v(r)) << 4);
  }
  // LDS ring of kStages tiles: tile t lives in slot t % kStages, and the copy of
  // tile t + kStages - 1 is started at the top of iteration t into the slot that
  // tile t - 1 used (every wave finished it before the previous barrier).  Each
  // wave waits only for the copies of the tile needed next (vmcnt counts this
  // wave's outstanding loads in issue order), so a copy has kStages - 1 tile-times
  // to arrive from HBM.
  constexpr int kLoadsPerTile = 2 * LY::BPW;
  // Tile order: left to right, except with causal ALiBi, whose bias grows toward
  // the diagonal: walking the tiles from the diagonal leftward sets each row's
  // running max on its first tile, where a left-to-right walk raises it (and
  // rescales O) on most tiles of the steeper heads.  Loop index t then stands for
  // the tile ntiles - 1 - (t - t_begin).
  const bool rev = EXT && CAUSAL && slopes != nullptr;
  constexpr int kAhead = (kStages - 1) * LY::BC;  // key distance of the tile copied ahead
#pragma unroll
  for (int p = 0; p < kStages - 1; ++p)
    if (t_begin + p < ntiles) {
      if constexpr (PAGED)
        copy_tile_paged<D>(smem, K, V, trow, Nk, num_pages, Hkv, g, (rev ? ntiles - 1 - p : t_begin + p) * LY::BC, p, w, lane);
      else
        copy_tile<D>(smem, kbase, vbase, head_bytes, kcp, vcp, (rev ? ntiles - 1 - p : t_begin + p) * LY::BC, p, w);
    }
  // paged: the page ids of the first tile copied inside the loops
  int idv = 0;
  if constexpr (PAGED) idv = load_tile_page_ids<D>(trow, Nk, (t_begin + kStages - 1) * LY::BC, lane);
  wait_vmem_tiles<kLoadsPerTile>(min(kStages - 2, ntiles - 1 - t_begin));  // the first tile has landed
  __syncthreads();

  int ndone = 0;  // tiles this wave has processed (EXT)
  int t_start = t_begin;
  if constexpr (PAGED) {
    // Causal in positions: every row of the block sees every key of the tiles below
    // t_m, so those tiles run through the unmasked body in a loop of their own.  With
    // both bodies in one loop the register allocator kept the O accumulators in two
    // places and copied them in and out on every unmasked tile of this instantiation.
    static_assert(!PAGED || CAUSAL, "the paged forward is causal");
    const int t_m = min(ntiles, (poff + qb * kBR + 1) / LY::BC);
    const int t_split = t_begin + max(0, (t_m - t_begin) / kStages) * kStages;
    for (int t0 = t_begin; t0 < t_split; t0 += kStages) {
#pragma unroll
      for (int u = 0; u < kStages; ++u) {
        const int t = t0 + u;
        const int j0 = t * LY::BC;
        if (t + kStages - 1 < ntiles) {
          copy_tile_paged_ids<D>(smem, K, V, idv, Nk, num_pages, Hkv, g, j0 + kAhead, (u + kStages - 1) % kStages, w,
                                 lane);
          idv = load_tile_page_ids<D>(trow, Nk, j0 + kAhead + LY::BC, lane);  // covered by the end-of-tile wait
        }
        debug_copy_fence();
        process_tile<D, false, false>(st, smem + u * LY::TBYTES, smem + (kStages + u) * LY::TBYTES, koff, voff,
                                      qrowp - j0 - 4 * hi, l32, c);
        wait_vmem_tiles<kLoadsPerTile>(max(0, min(kStages - 2, ntiles - 2 - t)));
        __syncthreads();
      }
    }
    t_start = t_split;
  }
  // The loop is unrolled by kStages so every slot index, and with it every LDS
  // address offset, is a compile-time constant.
  for (int t0 = t_start; t0 < ntiles; t0 += kStages) {
#pragma unroll
    for (int u = 0; u < kStages; ++u) {
      const int t = t0 + u;
      if (t >= ntiles) break;
      const int j0 = rev ? (ntiles - 1 - (t - t_begin)) * LY::BC : t * LY::BC;
      if (t + kStages - 1 < ntiles) {
        if constexpr (PAGED) {
          copy_tile_paged_ids<D>(smem, K, V, idv, Nk, num_pages, Hkv, g, j0 + kAhead, (u + kStages - 1) % kStages, w,
                                 lane);
          idv = load_tile_page_ids<D>(trow, Nk, j0 + kAhead + LY::BC, lane);  // covered by the end-of-tile wait
        } else
          copy_tile<D>(smem, kbase, vbase, head_bytes, kcp, vcp, rev ? j0 - kAhead : j0 + kAhead,
                       (u + kStages - 1) % kStages, w);
      }
      debug_copy_fence();

      const bool left_of_window = EXT && window > 0 && (j0 + LY::BC - 1 < rw0p - window + 1);
      const bool skip = (CAUSAL && (j0 > rw0p + kRowsPerWave - 1)) || left_of_window;
      if (!skip) {
        const bool need_mask = (CAUSAL ? (j0 + LY::BC - 1 > rw0p) : (j0 + LY::BC > Nk)) ||
                               (EXT && window > 0 && j0 < rw0p + kRowsPerWave - window);
        // causal: key j0 + koff visible iff koff + 4*hi <= qrow - j0 (keys past N
        // only reach rows >= N, which are never stored); otherwise iff key < N
        const int lim = (CAUSAL ? qrowp - j0 : Nk - 1 - j0) - 4 * hi;
        const uint8_t* kb = smem + u * LY::TBYTES;
        const uint8_t* vb = smem + (kStages + u) * LY::TBYTES;
        if constexpr (EXT) {
          // window: key visible iff koff + 4*hi >= qrow - window + 1 - j0
          const int lo = window > 0 ? qrowp - window + 1 - j0 - 4 * hi : -LY::BC;
          const float base = (float)(qrowp - j0 - 4 * hi);
          // causal ALiBi: the first two tiles a wave takes (its diagonal tile and the one
          // left of it, in the diagonal-first order) carry P in two bf16 parts
          const bool split = rev && ndone < 2;
          ++ndone;
          // the two-part tiles are instantiations of their own, so the other tiles carry
          // no code or registers for the second part
          if (CAUSAL && split) {
            if constexpr (CAUSAL) {
              if (need_mask)
                process_tile<D, true, true, true, false, true>(st, kb, vb, koff, voff, lim, l32, c, lo, base, slope2,
                                                               &ax);
              else
                process_tile<D, false, true, true, false, true>(st, kb, vb, koff, voff, lim, l32, c, lo, base,
                                                                slope2, &ax);
            }
          } else if (need_mask) {
            process_tile<D, true, true, CAUSAL>(st, kb, vb, koff, voff, lim, l32, c, lo, base, slope2, &ax);
          } else {
            process_tile<D, false, true, CAUSAL>(st, kb, vb, koff, voff, lim, l32, c, lo, base, slope2, &ax);
          }
        } else {
          if constexpr (!CAUSAL) {
            // only a ragged last tile is masked
            process_tile<D, false, false, false, true>(st, kb, vb, koff, voff, lim, l32, c, 0, 0.f, 0.f, nullptr,
                                                       need_mask);
          } else if (need_mask) {
            process_tile<D, true, false>(st, kb, vb, koff, voff, lim, l32, c);
          } else {
            process_tile<D, false, false>(st, kb, vb, koff, voff, lim, l32, c);
          }
        }
      }

      // tile t + 1 must have landed; the copies of later tiles may still be in flight
      wait_vmem_tiles<kLoadsPerTile>(max(0, min(kStages - 2, ntiles - 2 - t)));
      __syncthreads();
    }
  }

  // ---- epilogue: O = O / l_round (bf16), L = (m + log2 l_exact) ln 2
  const float lr = sum_xor32(st.l_round);
  const float le = sum_xor32(st.l_exact);
  if (SPLIT && nsplit > 1) {
    // this chunk's partial: O / l_round, m + log2 l_exact and m + log2 l_round (log2 units)
    // in fp32; a row with no visible key in the chunk leaves O = 0 and -inf
    const float pinv = lr > 0.f ? 1.f / lr : 0.f;
    if (qrow < N) {
      const size_t slot = (((size_t)(b * Hq + h) * nqb + qb) * smax + split) * kBR + (qrow - qb * kBR);
      float* orow = ws_o + slot * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 v4 = {st.oacc[db][4 * g4 + 0] * pinv, st.oacc[db][4 * g4 + 1] * pinv,
                            st.oacc[db][4 * g4 + 2] * pinv, st.oacc[db][4 * g4 + 3] * pinv};
          *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * g4 + 4 * hi) = v4;
        }
      if (hi == 0) {
        ws_l[slot] = le > 0.f ? st.m_run + log2_fast(le) : -INFINITY;
        ws_l[(size_t)ws_rows + slot] = lr > 0.f ? st.m_run + log2_fast(lr) : -INFINITY;
      }
    }
    return;
  }
  const float inv = 1.f / lr;
  if (qrow < N) {
    uint16_t* orow = O + ((size_t)(b * Hq + h) * N + qrow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * hi;
        u32x2 w2;
        w2[0] = pack_bf16x2(st.oacc[db][4 * g4 + 0] * inv, st.oacc[db][4 * g4 + 1] * inv);
        w2[1] = pack_bf16x2(st.oacc[db][4 * g4 + 2] * inv, st.oacc[db][4 * g4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d0) = w2;
      }
    if (hi == 0) Lse[(size_t)(b * Hq + h) * N + qrow] = (st.m_run + log2_fast(le)) * kLn2;
  }
}

// Persistent form of the plain forward (no window, no ALiBi, not paged): one workgroup
// per compute unit walks a static list of the (query block, batch, head) items.  The
// work per item and the results are those of fwd_bf16_kernel; what changes is the
// cost between items.  During an item's last tile the workgroup already copies the next
// item's first K/V tile into the LDS slot the previous tile freed, and it loads the next
// Q fragments (into the registers of the current ones, dead after the last tile) before
// the epilogue's stores, so the next item starts on data that has landed instead of
// paying the HBM round trip, and no workgroup launch sits between items.  (Loading the
// next Q during the last tile instead, into 32 registers of its own, measured 2-6%
// slower than no prefetch at all.)
// Schedule: the items are the grid of fwd_bf16_kernel in its work order (heaviest
// causal blocks first, runs of the G query heads sharing K/V dealt to one XCD in snake
// order).  Workgroup p takes virtual index r P + p in even rounds r and the mirrored slot
// of its own XCD, r P + 8 (P/8 - 1 - p/8) + p % 8, in odd ones: with P a multiple of 8,
// every index a workgroup takes lies on the XCD it runs on (workgroups are dealt to the
// XCDs round-robin), and the alternating direction pairs heavy causal blocks with light
// ones (c3: every workgroup gets 66 tiles).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_persistent_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ Lse, int B, int Hq, int Hkv, int N,
    float c /* |scale| * log2(e), > 0 */, uint32_t qsign /* 0x80008000 if scale < 0 */, int nitems) {
  using LY = Lay<D>;
  constexpr int KK = D / 16;
  constexpr int DB = D / 32;
  static_assert(kStages == 2, "the cross-item prefetch assumes a two-slot ring");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStages * LY::TBYTES];

  const int nqb = (N + kBR - 1) / kBR;
  const int G = Hq / Hkv;
  const int P = (int)gridDim.x, pw = (int)blockIdx.x;
  const int BH = B * Hq;
  // item of round r for this workgroup, or -1
  auto item_of = [&](int r) -> int {
    int vb;
    if (!(r & 1)) vb = r * P + pw;
    else if ((P & 7) == 0) vb = r * P + 8 * (P / 8 - 1 - pw / 8) + (pw & 7);
    else vb = r * P + P - 1 - pw;
    if (vb >= nitems) return -1;
    int item = vb;
    if (item < (nitems / (8 * G)) * 8 * G) {
      const int x = item & 7, slot = item >> 3, k = slot / G;
      item = (8 * k + ((k & 1) ? 7 - x : x)) * G + slot % G;
    }
    return item;
  };

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int grp = lane >> 4, li = lane & 15;

  // loop-invariant LDS byte offsets of this lane's fragment reads and copies
  int koff[KK], voff[DB];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) koff[kk] = ((2 * kk + hi) ^ LY::swz_k(l32)) << 4;
  {
    const int vr = 4 * hi + (li >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int lc = 4 * db + 2 * (grp & 1) + ((li & 3) >> 1);
      voff[db] = vr * LY::ROWB + ((lc ^ LY::swz_v(vr)) << 4) + (li & 1) * 8;
    }
  }
  uint32_t kcp[LY::BPW], vcp[LY::BPW];
#pragma unroll
  for (int i = 0; i < LY::BPW; ++i) {
    const int blk = w + kWaves * i;
    const int r = blk * LY::RPB + lane / LY::CPR;
    const int pc = lane % LY::CPR;
    kcp[i] = r * LY::ROWB + ((pc ^ LY::swz_k(r)) << 4);
    vcp[i] = r * LY::ROWB + ((pc ^ LY::swz_v(r)) << 4);
  }
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  constexpr int kLoadsPerTile = 2 * LY::BPW;

  // item coordinates: query block, batch, query head, K/V head
  struct Coord {
    int qb, b, h, g;
  };
  auto coord_of = [&](int item) -> Coord {
    Coord k;
    k.qb = CAUSAL ? (nqb - 1 - item / BH) : item / BH;
    const int bh = item % BH;
    k.b = bh / Hq;
    k.h = bh % Hq;
    k.g = k.h / G;
    return k;
  };
  auto kv_base = [&](const Coord& k, const uint16_t* T) { return T + ((size_t)(k.b * Hkv + k.g) * N) * D; };
  // Q fragments (B operand of S^T = K Q^T) of wave w: row qb*kBR + w*32 + l32,
  // d = kk*16 + hi*8 .. +8 (rows past N read as zero)
  auto load_q = [&](const Coord& k, bf16x8 (&qf)[KK]) {
    const int qrow = k.qb * kBR + w * kRowsPerWave + l32;
    const uint16_t* qbase = Q + ((size_t)(k.b * Hq + k.h) * N) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qrow < N) x = ld_global16(qbase + (size_t)qrow * D + kk * 16 + hi * 8);
      x ^= qsign;
      qf[kk] = __builtin_bit_cast(bf16x8, x);
    }
  };

  int r = 0;
  int item = item_of(0);
  if (item < 0) return;
  Coord cur = coord_of(item);
  WaveState<D> st;
  load_q(cur, st.qf);
  copy_tile<D>(smem, kv_base(cur, K), kv_base(cur, V), head_bytes, kcp, vcp, 0, 0, w);
  wait_vmem_tiles<kLoadsPerTile>(0);
  __syncthreads();

  while (true) {
    const int nitem = item_of(r + 1);
    const Coord nxt = coord_of(nitem >= 0 ? nitem : item);
    bool prefetched = false;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) st.oacc[db][rr] = 0.f;
    st.m_run = -INFINITY;
    st.l_exact = 0.f;
    st.l_round = 0.f;

    const int rw0 = cur.qb * kBR + w * kRowsPerWave;
    const int qrow = rw0 + l32;
    const uint16_t* kbase = kv_base(cur, K);
    const uint16_t* vbase = kv_base(cur, V);
    const int kend = CAUSAL ? min(N, (cur.qb + 1) * kBR) : N;
    const int ntiles = (kend + LY::BC - 1) / LY::BC;

    for (int t0 = 0; t0 < ntiles; t0 += kStages) {
#pragma unroll
      for (int u = 0; u < kStages; ++u) {
        const int t = t0 + u;
        if (t >= ntiles) break;
        const int j0 = t * LY::BC;
        if (t + 1 < ntiles) {
          copy_tile<D>(smem, kbase, vbase, head_bytes, kcp, vcp, j0 + LY::BC, (u + 1) % kStages, w);
        } else if (u == kStages - 1 && nitem >= 0) {
          // last tile, in slot 1: slot 0 is free for the next item's first tile
          copy_tile<D>(smem, kv_base(nxt, K), kv_base(nxt, V), head_bytes, kcp, vcp, 0, 0, w);
          prefetched = true;
        }
        debug_copy_fence();

        const bool skip = CAUSAL && (j0 > rw0 + kRowsPerWave - 1);
        if (!skip) {
          const bool need_mask = CAUSAL ? (j0 + LY::BC - 1 > rw0) : (j0 + LY::BC > N);
          const int lim = (CAUSAL ? qrow - j0 : N - 1 - j0) - 4 * hi;
          const uint8_t* kb = smem + u * LY::TBYTES;
          const uint8_t* vb = smem + (kStages + u) * LY::TBYTES;
          if constexpr (!CAUSAL) {
            process_tile<D, false, false, false, true>(st, kb, vb, koff, voff, lim, l32, c, 0, 0.f, 0.f, nullptr,
                                                       need_mask);
          } else if (need_mask) {
            process_tile<D, true, false>(st, kb, vb, koff, voff, lim, l32, c);
          } else {
            process_tile<D, false, false>(st, kb, vb, koff, voff, lim, l32, c);
          }
        }
        // the next tile (of this item, or the next item's first) must have landed
        wait_vmem_tiles<kLoadsPerTile>(0);
        __syncthreads();
      }
    }

    // the next item's Q (the fragments of this one are dead after the last tile), in
    // flight during the epilogue
    if (nitem >= 0) load_q(nxt, st.qf);
    // ---- epilogue: O = O / l_round (bf16), L = (m + log2 l_exact) ln 2
    {
      const float lr = sum_xor32(st.l_round);
      const float le = sum_xor32(st.l_exact);
      const float inv = 1.f / lr;
      if (qrow < N) {
        uint16_t* orow = O + ((size_t)(cur.b * Hq + cur.h) * N + qrow) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int d0 = db * 32 + 8 * g4 + 4 * hi;
            u32x2 w2;
            w2[0] = pack_bf16x2(st.oacc[db][4 * g4 + 0] * inv, st.oacc[db][4 * g4 + 1] * inv);
            w2[1] = pack_bf16x2(st.oacc[db][4 * g4 + 2] * inv, st.oacc[db][4 * g4 + 3] * inv);
            *reinterpret_cast<u32x2*>(orow + d0) = w2;
          }
        if (hi == 0) Lse[(size_t)(cur.b * Hq + cur.h) * N + qrow] = (st.m_run + log2_fast(le)) * kLn2;
      }
    }
    if (nitem < 0) break;
    if (!prefetched) {
      // the last tile sat in slot 0 (odd tile count): copy the next item's first tile now
      copy_tile<D>(smem, kv_base(nxt, K), kv_base(nxt, V), head_bytes, kcp, vcp, 0, 0, w);
      debug_copy_fence();
      wait_vmem_tiles<kLoadsPerTile>(0);
      __syncthreads();
    }
    cur = nxt;
    item = nitem;
    ++r;
  }
}

template <int D, bool CAUSAL, bool EXT, bool PAGED = false>
hipError_t launch(const FwdArgs& a) {
  const int nqb = (a.N + kBR - 1) / kBR;
  const dim3 grid((unsigned)(nqb * a.B * a.Hq));
  // scores are used as s * c with c > 0; a zero scale becomes a tiny positive c,
  // which leaves every unmasked exponential exactly 1 and masked ones exactly 0
  float c = fabsf(a.scale) * kLog2e;
  if (!(c > 1e-30f)) c = 1e-30f;
  const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, EXT, PAGED>), grid, dim3(kThreads), 0, (hipStream_t)a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o,
                     a.lse, a.B, a.Hq, a.Hkv, a.N, c, qsign, a.window, a.slopes, a.page_table, a.ctx_lens,
                     a.max_pages, a.num_pages, 0, nullptr, nullptr, 1, 0);
  return hipGetLastError();
}

// Sum of the chunk partials of the blocks the split-K plan cut (the decode's
// log-sum-exp merge).  O = sum_c r_c O_c / sum_c r_c with r_c = exp2(lr_c - max lr), lr_c
// the log2 of chunk c's sum of bf16-rounded probabilities: O_c was normalised by that
// sum, so this is exactly the one-pass O (the sum of the rounded weights times V, over
// their sum).  L = (max le + log2 sum_c exp2(le_c - max le)) ln 2 from the fp32 sums.
// One workgroup per RPP rows of a (head, query block) (RPP = 1024 / d: a thread per four
// channels of a row); blocks left whole wrote O and L themselves.
template <int D>
constexpr int kMergeRows = 1024 / D;
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_split_merge_kernel(const float* __restrict__ ws_o,
                                                              const float* __restrict__ ws_l, uint16_t* __restrict__ O,
                                                              float* __restrict__ Lse, int N, int nqb, int split_tiles,
                                                              int smax, int ws_rows) {
  const float* __restrict__ ws_r = ws_l + ws_rows;
  using LY = Lay<D>;
  constexpr int TPR = D / 4;             // threads per row (four channels each)
  constexpr int RPP = kMergeRows<D>;     // rows per workgroup
  constexpr int PPB = kBR / RPP;         // workgroups per query block
  const int blk = blockIdx.x / PPB, part = blockIdx.x % PPB;
  const int bh = blk / nqb, qb = blk % nqb;
  const int kend = CAUSAL ? min(N, (qb + 1) * kBR) : N;
  const int nsplit = ((kend + LY::BC - 1) / LY::BC + split_tiles - 1) / split_tiles;
  if (nsplit <= 1) return;
  const int tid = threadIdx.x, rr = tid / TPR, c4 = (tid % TPR) * 4;
  const size_t slot0 = ((size_t)bh * nqb + qb) * smax;
  {
    const int r = part * RPP + rr, row = qb * kBR + r;
    if (row >= N) return;
    float Me = -INFINITY, Mr = -INFINITY;
    for (int c = 0; c < nsplit; ++c) {
      Me = fmaxf(Me, ws_l[(slot0 + c) * kBR + r]);
      Mr = fmaxf(Mr, ws_r[(slot0 + c) * kBR + r]);
    }
    float esum = 0.f, rsum = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < nsplit; ++c) {
      const float le = ws_l[(slot0 + c) * kBR + r], lr = ws_r[(slot0 + c) * kBR + r];
      esum += le == -INFINITY ? 0.f : exp2_fast(le - Me);
      const float wc = lr == -INFINITY ? 0.f : exp2_fast(lr - Mr);
      rsum += wc;
      o += wc * *reinterpret_cast<const f32x4*>(ws_o + ((slot0 + c) * kBR + r) * D + c4);
    }
    const float inv = rsum > 0.f ? 1.f / rsum : 0.f;
    u32x2 w2;
    w2[0] = pack_bf16x2(o[0] * inv, o[1] * inv);
    w2[1] = pack_bf16x2(o[2] * inv, o[3] * inv);
    *reinterpret_cast<u32x2*>(O + ((size_t)bh * N + row) * D + c4) = w2;
    if (c4 == 0) Lse[(size_t)bh * N + row] = esum > 0.f ? (Me + log2_fast(esum)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_split(const FwdArgs& a) {
  const SplitPlan pl = fwd_split_plan(a.B, a.Hq, a.N, a.d, a.causal);
  float c = fabsf(a.scale) * kLog2e;
  if (!(c > 1e-30f)) c = 1e-30f;
  const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
  float* wso = pl.smax > 1 ? (float*)a.workspace : nullptr;
  float* wsl = pl.smax > 1 ? (float*)((uint8_t*)a.workspace + pl.o_bytes) : nullptr;
  const int ws_rows = pl.smax > 1 ? a.B * a.Hq * pl.nqb * pl.smax * kBR : 0;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, false, false>), dim3((unsigned)pl.items), dim3(kThreads), 0,
                     (hipStream_t)a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (uint16_t*)a.o, a.lse, a.B, a.Hq, a.Hkv, a.N, c, qsign, 0, nullptr, nullptr, nullptr, 0, 0,
                     pl.T, wso, wsl, pl.smax, ws_rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.smax <= 1) return e;
  hipLaunchKernelGGL((fwd_split_merge_kernel<D, CAUSAL>),
                     dim3((unsigned)(a.B * a.Hq * pl.nqb * (kBR / kMergeRows<D>))), dim3(256), 0,
                     (hipStream_t)a.stream, wso, wsl, (uint16_t*)a.o, a.lse, a.N, pl.nqb, pl.T, pl.smax, ws_rows);
  return hipGetLastError();
}

// Compute units of the stream's device (one persistent workgroup each), cached per
// device.
int compute_units() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

template <int D, bool CAUSAL>
hipError_t launch_persistent(const FwdArgs& a) {
  const int nqb = (a.N + kBR - 1) / kBR;
  const int nitems = nqb * a.B * a.Hq;
  const int P = min(nitems, compute_units());
  float c = fabsf(a.scale) * kLog2e;
  if (!(c > 1e-30f)) c = 1e-30f;
  const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((fwd_bf16_persistent_kernel<D, CAUSAL>), dim3((unsigned)P), dim3(kThreads), 0,
                     (hipStream_t)a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (uint16_t*)a.o, a.lse, a.B, a.Hq, a.Hkv, a.N, c, qsign, nitems);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_splitk(const FwdArgs& a) {
  if (a.d == 64) return a.causal ? launch_split<64, true>(a) : launch_split<64, false>(a);
  return a.causal ? launch_split<128, true>(a) : launch_split<128, false>(a);
}

hipError_t launch_prefill_paged(const FwdArgs& a) {
  return a.d == 64 ? launch<64, true, false, true>(a) : launch<128, true, false, true>(a);
}

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  if (a.window > 0 || a.slopes != nullptr) {
    if (a.d == 64) return a.causal ? launch<64, true, true>(a) : launch<64, false, true>(a);
    return a.causal ? launch<128, true, true>(a) : launch<128, false, true>(a);
  }
  if (a.d == 64) return a.causal ? launch_persistent<64, true>(a) : launch_persistent<64, false>(a);
  return a.causal ? launch_persistent<128, true>(a) : launch_persistent<128, false>(a);
}

}  // namespace fa
