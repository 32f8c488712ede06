// bf16 exact-attention forward on gfx950 matrix cores.
//
// The FlashAttention forward of "Phase 08 -- Inference Optimization at Depth"
// (Concepts list: online softmax, FlashAttention tiling, causal tiles handled
// apart; Lab 01 steps 2 and 4) with the query-block parallelism of getnybble
// "Inference Optimization -- Advanced", question 5, and the grouped K/V heads of
// the screna.ai MHA/MQA/GQA block.
//
// Work decomposition: one workgroup of 4 waves per (256-row query block, query
// head, batch).  Each wave owns 64 query rows and keeps its Q fragments in
// registers for the whole pass.  K/V are streamed in tiles of 64 keys through
// two LDS buffers (the next tile is fetched with 128-bit global loads while the
// current one is consumed).  Per tile and wave:
//   S^T = K Q^T  with v_mfma_f32_32x32x16_bf16 (K from LDS is the A operand, so
//                every lane ends up holding 16 keys of one query row),
//   online softmax in the log2 domain (row max over the lane's 16 keys plus one
//                permlane32 swap; exp2 with scale*log2e folded into one FMA),
//   O^T += V^T P^T with the same MFMA; V^T fragments come straight from the
//                row-major LDS tile through ds_read_b64_tr_b16, and P stays in
//                the registers the S MFMA produced (the key order inside a
//                16-key step is permuted identically on both operands).
// Causal: tiles wholly above a wave's rows are skipped, tiles crossing the
// diagonal take the masked path, every other tile runs mask-free; no tile past
// the block's last row is ever loaded.  Only O (bf16) and L (fp32) are written.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 64;           // two 32-row MFMA blocks
constexpr int kBR = kWaves * kRowsPerWave;  // 256 query rows per workgroup
constexpr int kBC = 64;                     // keys per tile (two 32-key MFMA blocks)

template <int D>
struct Lay {
  static constexpr int KP = D * 2 + 16;  // K row pitch in bytes (b128 reads conflict-free)
  static constexpr int VP = D * 2 + 32;  // V row pitch in bytes (transposed b64 reads)
  static constexpr int KBYTES = kBC * KP;
  static constexpr int VBYTES = kBC * VP;
  static constexpr int BUF = KBYTES + VBYTES;
  static constexpr int CH = kBC * D / 8 / kThreads;  // 16-byte chunks per thread per tensor
};

__device__ __forceinline__ u32x4 ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ Lse, int B, int Hq, int Hkv, int N,
    float c /* |scale| * log2(e) */, uint32_t qsign /* 0x80008000 if scale < 0 */) {
  using LY = Lay<D>;
  constexpr int KK = D / 16;  // 16-wide d steps of the S MFMA
  constexpr int DB = D / 32;  // 32-wide d blocks of the O accumulator
  constexpr int CH = LY::CH;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * LY::BUF];

  const int nqb = (N + kBR - 1) / kBR;
  const int BH = B * Hq;
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

  // ---- Q fragments (B operand of S^T = K Q^T): row rw0 + rb*32 + l32, d = kk*16 + hi*8 .. +8
  bf16x8 qf[2][KK];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = rw0 + rb * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row < N) x = ld_global16(qbase + (size_t)row * D + kk * 16 + hi * 8);
      x ^= qsign;
      qf[rb][kk] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x16 oacc[2][DB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[rb][db][r] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  const int kend = CAUSAL ? min(N, (qb + 1) * kBR) : N;
  const int ntiles = (kend + kBC - 1) / kBC;

  // ---- global -> register staging of one K/V tile
  u32x4 kst[CH], vst[CH];
  auto fetch = [&](int j0) {
#pragma unroll
    for (int c2 = 0; c2 < CH; ++c2) {
      const int idx = c2 * kThreads + tid;
      const int r = idx / (D / 8), col = (idx % (D / 8)) * 8;
      const int key = j0 + r;
      u32x4 zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
      if (key < N) {
        zk = ld_global16(kbase + (size_t)key * D + col);
        zv = ld_global16(vbase + (size_t)key * D + col);
      }
      kst[c2] = zk;
      vst[c2] = zv;
    }
  };
  auto stash = [&](int buf) {
    uint8_t* kb = smem + buf * LY::BUF;
    uint8_t* vb = kb + LY::KBYTES;
#pragma unroll
    for (int c2 = 0; c2 < CH; ++c2) {
      const int idx = c2 * kThreads + tid;
      const int r = idx / (D / 8), col = (idx % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(kb + r * LY::KP + col * 2) = kst[c2];
      *reinterpret_cast<u32x4*>(vb + r * LY::VP + col * 2) = vst[c2];
    }
  };

  fetch(0);
  stash(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int j0 = t * kBC;
    const bool has_next = t + 1 < ntiles;
    if (has_next) fetch(j0 + kBC);

    const bool skip = CAUSAL && (j0 > rw0 + kRowsPerWave - 1);
    if (!skip) {
      const bool need_mask = (CAUSAL && (j0 + kBC - 1 > rw0)) || (j0 + kBC > N);
      const uint8_t* kb = smem + buf * LY::BUF;
      const uint8_t* vb = kb + LY::KBYTES;

      // ---- S^T = K Q^T : sacc[kb][rb], lane holds keys kb*32 + 8*(r/4) + 4*hi + r%4 of row l32
      f32x16 sacc[2][2];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[a][rb][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kb + (a * 32 + l32) * LY::KP + kk * 32 + hi * 16);
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            sacc[a][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[rb][kk], sacc[a][rb], 0, 0, 0);
        }
      }

      // ---- online softmax (log2 domain), P packed to bf16 as the B operand of the PV MFMA
      bf16x8 pb[2][2][2];  // [key block][16-key step][row block]
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int qrow = rw0 + rb * 32 + l32;
        float mx = -INFINITY;
        if (need_mask) {
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = j0 + a * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
              const bool vis = key < N && (!CAUSAL || key <= qrow);
              sacc[a][rb][r] = vis ? sacc[a][rb][r] : -INFINITY;
              mx = fmaxf(mx, sacc[a][rb][r]);
            }
        } else {
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[a][rb][r]);
        }
        mx = max_xor32(mx);
        const float mt = (mx == -INFINITY) ? -INFINITY : mx * c;
        const float mnew = fmaxf(m_run[rb], mt);
        const float mref = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = exp2_fast(m_run[rb] - mref);
        float psum = 0.f;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            bf16x8 pk;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float s = sacc[a][rb][st * 8 + j];
              float p = exp2_fast(__builtin_fmaf(s, c, -mref));
              if (need_mask) p = (s == -INFINITY) ? 0.f : p;
              psum += p;
              pk[j] = to_bf16(p);
            }
            pb[a][st][rb] = pk;
          }
        l_run[rb] = l_run[rb] * alpha + psum;
        m_run[rb] = mnew;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[rb][db][r] *= alpha;
      }

      // ---- O^T += V^T P^T
      const int grp = lane >> 4, li = lane & 15;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int kb1 = a * 32 + st * 16 + 4 * hi;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int dbase = db * 32 + (grp & 1) * 16;
            const uint8_t* p1 = vb + (kb1 + (li >> 2)) * LY::VP + (dbase + 4 * (li & 3)) * 2;
            const uint8_t* p2 = p1 + 8 * LY::VP;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(p1));
            const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(p2));
            const s16x4 both_lo = lo, both_hi = up;
            typedef short s16x8 __attribute__((ext_vector_type(8)));
            const s16x8 cat = __builtin_shufflevector(both_lo, both_hi, 0, 1, 2, 3, 4, 5, 6, 7);
            const bf16x8 vf = __builtin_bit_cast(bf16x8, cat);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
              oacc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[a][st][rb], oacc[rb][db], 0, 0, 0);
          }
        }
    }

    if (has_next) stash(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O / l (bf16), L = (m + log2 l) ln 2
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float lt = sum_xor32(l_run[rb]);
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
          w2[0] = pack_bf16x2(oacc[rb][db][4 * g4 + 0] * inv, oacc[rb][db][4 * g4 + 1] * inv);
          w2[1] = pack_bf16x2(oacc[rb][db][4 * g4 + 2] * inv, oacc[rb][db][4 * g4 + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + d0) = w2;
        }
      if (hi == 0) Lse[(size_t)(b * Hq + h) * N + row] = (m_run[rb] + log2_fast(lt)) * kLn2;
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
