// fp32 exact-attention forward (no downcast anywhere).
//
// The FlashAttention forward of "Phase 08 -- Inference Optimization at Depth"
// (Concepts list: online softmax, tiling; Lab 01 steps 2 and 4), in fp32: Q rows
// are split into blocks of 64, K/V are streamed through LDS in tiles of 64 keys,
// and each query row keeps a running max m, running sum l and an unnormalised
// output accumulator that is rescaled by exp(m_old - m_new) per tile.  Causal
// tiles entirely above the diagonal are never loaded.  Only O and L are written.
//
// Four waves per workgroup share each K/V tile in LDS.  Each query row is shared
// by TPR = d/16 lanes, each owning 16 of its d columns: a dot product is 16 FMAs
// per lane plus two (d = 64) or three (d = 128) DPP additions across the row's
// lanes, and the P V update is 16 FMAs per lane and key.  A workgroup holds
// 4*64/TPR rows (64 at d = 64, 32 at d = 128), and the per-lane work is a quarter
// (an eighth) of a whole-row thread's, so short sequences still keep many waves busy.  This path exists for fp32
// inputs, whose sizes in practice are small; it uses VALU FMAs, not matrix cores.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kKeys = 64;    // keys per tile (B_c)
constexpr int kDH = 16;      // head-dim columns owned by one lane
constexpr int kWavesF = 4;   // waves per workgroup
constexpr int kThreadsF = 64 * kWavesF;
static_assert(kThreadsF == kGeomF32Threads, "host-side launch limits assume this workgroup size");

template <int D>
struct F32Lay {
  static constexpr int TPR = D / kDH;    // lanes per query row
  static constexpr int ROWS = kThreadsF / TPR;  // query rows per workgroup (B_r)
};

// Sum over the TPR lanes of a row (aligned groups of 4 or 8).
template <int TPR>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (TPR == 8) return sum8(x);
  x += dpp<0xB1>(x);
  return x + dpp<0x4E>(x);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreadsF) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ L, int Hq, int Hkv, int N, float c /* scale*log2e */) {
  constexpr int TPR = F32Lay<D>::TPR;
  constexpr int kRows = F32Lay<D>::ROWS;
  __shared__ float4 ks[kKeys][D / 4];
  __shared__ float4 vs[kKeys][D / 4];

  const int nqb = (N + kRows - 1) / kRows;
  const int bh = blockIdx.x / nqb;
  // heaviest causal blocks first
  const int qb = CAUSAL ? (nqb - 1 - (blockIdx.x % nqb)) : (blockIdx.x % nqb);
  const int b = bh / Hq, h = bh % Hq;
  const int g = h / (Hq / Hkv);
  const int tid = threadIdx.x;
  const int row = qb * kRows + tid / TPR;
  const int part = tid % TPR;  // this lane's 16 columns: part*16 .. part*16+15
  const bool row_ok = row < N;

  const float* qp = Q + (((size_t)(b * Hq + h) * N) + (row_ok ? row : 0)) * D + part * kDH;
  const float4* kb = reinterpret_cast<const float4*>(K + ((size_t)(b * Hkv + g) * N) * D);
  const float4* vb = reinterpret_cast<const float4*>(V + ((size_t)(b * Hkv + g) * N) * D);

  float q[kDH], o[kDH];
#pragma unroll
  for (int i = 0; i < kDH; ++i) {
    q[i] = row_ok ? qp[i] * c : 0.f;  // scores kept in log2 units: s2 = scale*log2e*(q.k)
    o[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  const int kend = CAUSAL ? min(N, (qb + 1) * kRows) : N;
  for (int j0 = 0; j0 < kend; j0 += kKeys) {
    __syncthreads();
    for (int e = tid; e < kKeys * D / 4; e += kThreadsF) {
      const int r = e / (D / 4), col = e % (D / 4);
      const bool ok = j0 + r < N;
      ks[r][col] = ok ? kb[(size_t)(j0 + r) * (D / 4) + col] : make_float4(0.f, 0.f, 0.f, 0.f);
      vs[r][col] = ok ? vb[(size_t)(j0 + r) * (D / 4) + col] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
    float s[kKeys];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int i4 = 0; i4 < kDH / 4; ++i4) {
        const float4 k4 = ks[j][part * (kDH / 4) + i4];
        acc = __builtin_fmaf(q[4 * i4 + 0], k4.x, acc);
        acc = __builtin_fmaf(q[4 * i4 + 1], k4.y, acc);
        acc = __builtin_fmaf(q[4 * i4 + 2], k4.z, acc);
        acc = __builtin_fmaf(q[4 * i4 + 3], k4.w, acc);
      }
      acc = row_sum<TPR>(acc);  // every lane of the row now holds the full dot product
      const int key = j0 + j;
      const bool vis = key < N && (!CAUSAL || key <= row);
      s[j] = vis ? acc : -INFINITY;
      tmax = fmaxf(tmax, s[j]);
    }
    const float mnew = fmaxf(m, tmax);
    const float mref = (mnew == -INFINITY) ? 0.f : mnew;
    const float alpha = exp2_fast(m - mref);  // m = -inf -> 0
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      s[j] = exp2_fast(s[j] - mref);
      psum += s[j];
    }
    l = l * alpha + psum;
#pragma unroll
    for (int i = 0; i < kDH; ++i) o[i] *= alpha;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
#pragma unroll
      for (int i4 = 0; i4 < kDH / 4; ++i4) {
        const float4 v4 = vs[j][part * (kDH / 4) + i4];
        o[4 * i4 + 0] = __builtin_fmaf(s[j], v4.x, o[4 * i4 + 0]);
        o[4 * i4 + 1] = __builtin_fmaf(s[j], v4.y, o[4 * i4 + 1]);
        o[4 * i4 + 2] = __builtin_fmaf(s[j], v4.z, o[4 * i4 + 2]);
        o[4 * i4 + 3] = __builtin_fmaf(s[j], v4.w, o[4 * i4 + 3]);
      }
    }
    m = mnew;
  }
  if (!row_ok) return;
  const float inv = 1.f / l;
  float* op = O + (((size_t)(b * Hq + h) * N) + row) * D + part * kDH;
#pragma unroll
  for (int i = 0; i < kDH; i += 4) {
    float4 w = make_float4(o[i] * inv, o[i + 1] * inv, o[i + 2] * inv, o[i + 3] * inv);
    *reinterpret_cast<float4*>(op + i) = w;
  }
  if (part == 0) L[(size_t)(b * Hq + h) * N + row] = (m + log2_fast(l)) * kLn2;
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a) {
  const int nqb = (a.N + F32Lay<D>::ROWS - 1) / F32Lay<D>::ROWS;
  const dim3 grid((unsigned)(nqb * a.B * a.Hq));
  const dim3 block(kThreadsF);
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), grid, block, 0, (hipStream_t)a.stream,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse,
                     a.Hq, a.Hkv, a.N, a.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a) {
  if (a.d == 64) return a.causal ? launch<64, true>(a) : launch<64, false>(a);
  return a.causal ? launch<128, true>(a) : launch<128, false>(a);
}

}  // namespace fa
