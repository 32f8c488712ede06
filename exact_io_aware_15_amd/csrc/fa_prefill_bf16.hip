// bf16 exact-attention forward on gfx950 matrix cores.
//
// The FlashAttention forward of "Phase 08 -- Inference Optimization at Depth"
// (Concepts list: online softmax, FlashAttention tiling, causal tiles handled
// apart; Lab 01 steps 2 and 4) with the query-block parallelism of getnybble
// "Inference Optimization -- Advanced", question 5, and the grouped K/V heads of
// the screna.ai MHA/MQA/GQA block.
//
// Work decomposition: one workgroup of 4 waves (one per SIMD) per (256-row query
// block, query head, batch).  Each wave owns 64 query rows as two 32-row MFMA
// blocks and keeps their Q fragments in registers for the whole pass.  K/V are
// streamed in tiles of 64 keys through two LDS buffers: the next tile is copied
// HBM -> LDS by 128-bit buffer loads with the LDS-destination bit (no staging
// registers; rows past N read as zero) while the current one is consumed.  Rows
// are stored unpadded with their 16-byte chunks XOR-swizzled by row, so both the
// b128 K reads and the transposing V reads hit distinct LDS banks.  Per tile and wave:
//   S^T = K Q^T  with v_mfma_f32_32x32x16_bf16 (K from LDS is the A operand, so
//                every lane ends up holding 16 keys of one query row),
//   online softmax in the log2 domain (row max over the lane's keys plus one
//                permlane32 swap; exp2 with scale*log2e folded into one FMA),
//   O^T += V^T P^T with the same MFMA; V^T fragments come straight from the
//                row-major LDS tile through ds_read_b64_tr_b16, and P stays in
//                the registers the S MFMA produced (the key order inside a
//                16-key step is permuted identically on both operands).
// The two row blocks are software-pipelined inside the wave: the S MFMAs of block
// 1 are issued next to the softmax arithmetic of block 0, and the PV MFMAs of
// block 0 next to the softmax of block 1, so the matrix cores and the vector ALU
// work at the same time.
//
// Rescaling follows the running-max recurrence exactly: a row's m rises to its
// tile max whenever that is larger, and O and l are multiplied by exp(m_old -
// m_new).  The multiply is skipped, wave-wide, on tiles where no row's max grew
// (then every factor would be 1).  The largest score of a tile that sets m gets
// probability exactly 1, which keeps the bf16 rounding of P off the dominant key.
//
// Causal: tiles wholly above a wave's rows are skipped, tiles crossing the
// diagonal (or the ragged end of the sequence) take the masked path, every other
// tile runs mask-free; no tile past the block's last row is ever loaded.
// Only O (bf16) and L (fp32) are written.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kRB = 1;                      // 32-row MFMA blocks per wave
constexpr int kRowsPerWave = 32 * kRB;
constexpr int kWaves = 8;                   // two waves per SIMD
constexpr int kThreads = kWaves * 64;
constexpr int kBR = kWaves * kRowsPerWave;  // 256 query rows per workgroup
constexpr int kBC = 64;                     // keys per tile (two 32-key MFMA blocks)

template <int D>
struct Lay {
  static constexpr int ROWB = D * 2;            // bytes per K/V row in LDS (unpadded)
  static constexpr int CPR = ROWB / 16;         // 16-byte chunks per row
  static constexpr int RPB = 1024 / ROWB;       // rows per 1 KB wave copy (64 lanes x 16 B)
  static constexpr int TBYTES = kBC * ROWB;     // one tensor tile
  static constexpr int BUF = 2 * TBYTES;        // K tile then V tile
  static constexpr int BLOCKS = TBYTES / 1024;  // 1 KB copies per tensor tile
  static constexpr int BPW = BLOCKS / kWaves;   // ... per wave
  // chunk swizzles: physical chunk = logical chunk ^ swz(row)
  __device__ static constexpr int swz_k(int r) { return r & (CPR - 1); }
  __device__ static constexpr int swz_v(int r) { return (r & (CPR / 2 - 1)) << 1; }
};

__device__ __forceinline__ u32x4 ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

typedef short s16x8 __attribute__((ext_vector_type(8)));

// Per-wave state carried across tiles.
template <int D>
struct WaveState {
  static constexpr int KK = D / 16;
  static constexpr int DB = D / 32;
  bf16x8 qf[kRB][KK];     // Q^T fragments (B operand), one per 32-row block
  f32x16 oacc[kRB][DB];   // O^T accumulators: lane holds row l%32, 16 d values per block
  float m_run[kRB];       // max used in the exponentials (log2 units)
  float l_run[kRB];       // partial row sums of this lane's keys
};

// Masked max of one row block's scores; returns the tile max in log2 units.
template <bool MASK, bool CAUSAL>
__device__ __forceinline__ float tile_rowmax(f32x16 (&s)[2], int j0, int qrow, int hi, int N, float c) {
  float mx = -INFINITY;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (MASK) {
        const int key = j0 + a * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        const bool vis = key < N && (!CAUSAL || key <= qrow);
        s[a][r] = vis ? s[a][r] : -INFINITY;
      }
      mx = fmaxf(mx, s[a][r]);
    }
  mx = max_xor32(mx);
  return (mx == -INFINITY) ? -INFINITY : mx * c;
}

// Raise the running max of rows whose tile max exceeds it, rescaling that row
// block's O and l.  Wave-uniform branch: skipped when no row of the wave grew.
template <int D>
__device__ __forceinline__ void maybe_rescale(WaveState<D>& st, int rb, float mt) {
  const bool grow = mt > st.m_run[rb];
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
    const float mnew = fmaxf(st.m_run[rb], mt);
    const float alpha = exp2_fast(st.m_run[rb] - mnew);  // m_run = -inf -> 0
    st.l_run[rb] *= alpha;
#pragma unroll
    for (int db = 0; db < WaveState<D>::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.oacc[rb][db][r] *= alpha;
    st.m_run[rb] = mnew;
  }
}

// exp2 of the row block's scores against the running max, fp32 row sum, bf16 pack.
template <bool MASK>
__device__ __forceinline__ void softmax_pack(const f32x16 (&s)[2], float m, float c, float& l,
                                             bf16x8 (&pb)[2][2]) {
  const float mref = (m == -INFINITY) ? 0.f : m;
  float psum = 0.f;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      u32x4 pk;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x0 = s[a][st * 8 + 2 * j], x1 = s[a][st * 8 + 2 * j + 1];
        float p0 = exp2_fast(__builtin_fmaf(x0, c, -mref));
        float p1 = exp2_fast(__builtin_fmaf(x1, c, -mref));
        if (MASK) {
          p0 = (x0 == -INFINITY) ? 0.f : p0;
          p1 = (x1 == -INFINITY) ? 0.f : p1;
        }
        psum += p0;
        psum += p1;
        pk[j] = pack_bf16x2(p0, p1);
      }
      pb[a][st] = __builtin_bit_cast(bf16x8, pk);
    }
  l += psum;
}

template <int D, bool MASK, bool CAUSAL>
__device__ __forceinline__ void process_tile(WaveState<D>& st, const uint8_t* kb, const uint8_t* vb, int j0,
                                             int rw0, int lane, int N, float c) {
  using LY = Lay<D>;
  constexpr int KK = D / 16;
  constexpr int DB = D / 32;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // K fragments (A operand of S^T = K Q^T): key a*32 + l32, d = kk*16 + hi*8 .. +8
  auto kfrag = [&](int a, int kk) {
    const int r = a * 32 + l32;
    return *reinterpret_cast<const bf16x8*>(kb + r * LY::ROWB + (((2 * kk + hi) ^ LY::swz_k(r)) << 4));
  };
  // V^T fragments (A operand of O^T = V^T P^T) through the transposing LDS read:
  // keys a*32 + s2*16 + 4*hi + {0..3, 8..11}, d = db*32 + l32
  const int grp = lane >> 4, li = lane & 15;
  auto vaddr = [&](int r, int lc, int inner) {
    return vb + r * LY::ROWB + ((lc ^ LY::swz_v(r)) << 4) + inner;
  };
  auto vfrag = [&](int a, int s2, int db) {
    // source lane li reads 8 bytes of row kb1 + li/4 at d = dbase + 4*(li%4)
    const int r = a * 32 + s2 * 16 + 4 * hi + (li >> 2);
    const int lc = (db * 32 + (grp & 1) * 16) / 8 + ((li & 3) >> 1);
    const int inner = (li & 1) * 8;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(vaddr(r, lc, inner)));
    const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(vaddr(r + 8, lc, inner)));
    const s16x8 cat = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, cat);
  };

  // ---- scores S^T = K Q^T for every row block
  f32x16 sc[kRB][2];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[rb][a][r] = 0.f;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const bf16x8 kf = kfrag(a, kk);
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
        sc[rb][a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, st.qf[rb][kk], sc[rb][a], 0, 0, 0);
    }

  // ---- online softmax per row block
  bf16x8 pb[kRB][2][2];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const float mt = tile_rowmax<MASK, CAUSAL>(sc[rb], j0, rw0 + 32 * rb + l32, hi, N, c);
    maybe_rescale<D>(st, rb, mt);
    softmax_pack<MASK>(sc[rb], st.m_run[rb], c, st.l_run[rb], pb[rb]);
  }

  // ---- O^T += V^T P^T
  // (scheduling fence: the V fragment reads are not hoisted into the score phase,
  // where their registers would push the wave past its 256-register budget)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 vf = vfrag(a, s2, db);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
          st.oacc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[rb][a][s2], st.oacc[rb][db], 0, 0, 0);
      }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ Lse, int B, int Hq, int Hkv, int N,
    float c /* |scale| * log2(e) */, uint32_t qsign /* 0x80008000 if scale < 0 */) {
  using LY = Lay<D>;
  constexpr int KK = D / 16;
  constexpr int DB = D / 32;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * LY::BUF];

  const int nqb = (N + kBR - 1) / kBR;
  const int BH = B * Hq;
  // causal: heaviest query blocks are dispatched first
  const int qb = CAUSAL ? (nqb - 1 - (int)(blockIdx.x / BH)) : (int)(blockIdx.x / BH);
  const int bh = blockIdx.x % BH;
  const int b = bh / Hq, h = bh % Hq;
  const int g = h / (Hq / Hkv);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;  // which half of the wave
  const int rw0 = qb * kBR + w * kRowsPerWave;

  const uint16_t* qbase = Q + ((size_t)(b * Hq + h) * N) * D;
  const uint16_t* kbase = K + ((size_t)(b * Hkv + g) * N) * D;
  const uint16_t* vbase = V + ((size_t)(b * Hkv + g) * N) * D;

  WaveState<D> st;
  // Q fragments (B operand of S^T = K Q^T): row rw0 + rb*32 + l32, d = kk*16 + hi*8 .. +8
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int row = rw0 + rb * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row < N) x = ld_global16(qbase + (size_t)row * D + kk * 16 + hi * 8);
      x ^= qsign;
      st.qf[rb][kk] = __builtin_bit_cast(bf16x8, x);
    }
  }
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.oacc[rb][db][r] = 0.f;
    st.m_run[rb] = -INFINITY;
    st.l_run[rb] = 0.f;
  }

  const int kend = CAUSAL ? min(N, (qb + 1) * kBR) : N;
  const int ntiles = (kend + kBC - 1) / kBC;

  // ---- HBM -> LDS copies of one K/V tile (buffer loads with the LDS bit).  Wave w
  // copies 1 KB blocks w, w + 4, ... of each tensor; lane l of a block writes
  // physical chunk l % CPR of row blk*RPB + l / CPR, which holds logical chunk
  // (l % CPR) ^ swz(row).  Out-of-range rows (key >= N) read as zero.
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, head_bytes, 0x00020000);
  auto copy_tile = [&](int j0, int buf) {
    uint8_t* kb = smem + buf * LY::BUF;
    uint8_t* vb = kb + LY::TBYTES;
#pragma unroll
    for (int i = 0; i < LY::BPW; ++i) {
      const int blk = w + kWaves * i;
      const int r = blk * LY::RPB + lane / LY::CPR;
      const int pc = lane % LY::CPR;
      const uint32_t row_off = (uint32_t)(j0 + r) * (D * 2);
      // a row past N gets an offset past the buffer end, so the copy writes zeros
      const uint32_t koff = (j0 + r < N) ? row_off + ((pc ^ LY::swz_k(r)) << 4) : head_bytes;
      const uint32_t voff = (j0 + r < N) ? row_off + ((pc ^ LY::swz_v(r)) << 4) : head_bytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (FA_LDS void*)(kb + blk * 1024), 16, koff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (FA_LDS void*)(vb + blk * 1024), 16, voff, 0, 0, 0);
    }
  };

  copy_tile(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies have landed
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int j0 = t * kBC;
    // the other buffer was last read in tile t - 1, which every wave has finished
    if (t + 1 < ntiles) copy_tile(j0 + kBC, buf ^ 1);

    const bool skip = CAUSAL && (j0 > rw0 + kRowsPerWave - 1);
    if (!skip) {
      const bool need_mask = (CAUSAL && (j0 + kBC - 1 > rw0)) || (j0 + kBC > N);
      const uint8_t* kb = smem + buf * LY::BUF;
      const uint8_t* vb = kb + LY::TBYTES;
      if (need_mask)
        process_tile<D, true, CAUSAL>(st, kb, vb, j0, rw0, lane, N, c);
      else
        process_tile<D, false, CAUSAL>(st, kb, vb, j0, rw0, lane, N, c);
    }

    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
  }

  // ---- epilogue: O = O / l (bf16), L = (m + log2 l) ln 2
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const float lt = sum_xor32(st.l_run[rb]);
    const float inv = 1.f / lt;
    const int row = rw0 + rb * 32 + l32;
    if (row < N) {
      uint16_t* orow = O + ((size_t)(b * Hq + h) * N + row) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = db * 32 + 8 * g4 + 4 * hi;
          u32x2 w2;
          w2[0] = pack_bf16x2(st.oacc[rb][db][4 * g4 + 0] * inv, st.oacc[rb][db][4 * g4 + 1] * inv);
          w2[1] = pack_bf16x2(st.oacc[rb][db][4 * g4 + 2] * inv, st.oacc[rb][db][4 * g4 + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + d0) = w2;
        }
      if (hi == 0) Lse[(size_t)(b * Hq + h) * N + row] = (st.m_run[rb] + log2_fast(lt)) * kLn2;
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a) {
  const int nqb = (a.N + kBR - 1) / kBR;
  const dim3 grid((unsigned)(nqb * a.B * a.Hq));
  const float c = fabsf(a.scale) * kLog2e;
  const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), grid, dim3(kThreads), 0, (hipStream_t)a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o,
                     a.lse, a.B, a.Hq, a.Hkv, a.N, c, qsign);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  if (a.d == 64) return a.causal ? launch<64, true>(a) : launch<64, false>(a);
  return a.causal ? launch<128, true>(a) : launch<128, false>(a);
}

}  // namespace fa
