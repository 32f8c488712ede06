// fp32 exact-attention forward (no downcast anywhere).
//
// The FlashAttention forward of "Phase 08 -- Inference Optimization at Depth"
// (Concepts list: online softmax, tiling; Lab 01 steps 2 and 4), in fp32: Q rows
// are split into blocks of 64, K/V are streamed through LDS in tiles of 64 keys,
// and each query row keeps a running max m, running sum l and an unnormalised
// output accumulator that is rescaled by exp(m_old - m_new) per tile.  Causal
// tiles entirely above the diagonal are never loaded.  Only O and L are written.
//
// One thread owns 64 of the d columns of one query row (d = 64: one thread per
// row; d = 128: two threads per row that combine their partial dot products with
// one DPP exchange).  This path exists for fp32 inputs, whose sizes in practice
// are small; it uses VALU FMAs, not matrix cores.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kRows = 64;    // query rows per workgroup (B_r)
constexpr int kKeys = 64;    // keys per tile (B_c)
constexpr int kDH = 64;      // head-dim columns owned by one thread

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kRows * (D / kDH)) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ L, int Hq, int Hkv, int N, float c /* scale*log2e */) {
  constexpr int TPR = D / kDH;  // threads per row
  __shared__ float ks[kKeys][D];
  __shared__ float vs[kKeys][D];

  const int nqb = (N + kRows - 1) / kRows;
  const int bh = blockIdx.x / nqb;
  // heaviest causal blocks first
  const int qb = CAUSAL ? (nqb - 1 - (blockIdx.x % nqb)) : (blockIdx.x % nqb);
  const int b = bh / Hq, h = bh % Hq;
  const int g = h / (Hq / Hkv);
  const int tid = threadIdx.x;
  const int row = qb * kRows + tid / TPR;
  const int half = tid % TPR;
  const bool row_ok = row < N;

  const float* qp = Q + (((size_t)(b * Hq + h) * N) + (row_ok ? row : 0)) * D + half * kDH;
  const float* kb = K + ((size_t)(b * Hkv + g) * N) * D;
  const float* vb = V + ((size_t)(b * Hkv + g) * N) * D;

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
    for (int e = tid; e < kKeys * D; e += kRows * TPR) {
      const int r = e / D, col = e % D;
      const bool ok = j0 + r < N;
      ks[r][col] = ok ? kb[(size_t)(j0 + r) * D + col] : 0.f;
      vs[r][col] = ok ? vb[(size_t)(j0 + r) * D + col] : 0.f;
    }
    __syncthreads();
    float s[kKeys];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < kDH; ++i) acc = __builtin_fmaf(q[i], ks[j][half * kDH + i], acc);
      if (TPR == 2) acc += dpp<0xB1>(acc);  // partner thread (l ^ 1) holds the other half
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
      for (int i = 0; i < kDH; ++i) o[i] = __builtin_fmaf(s[j], vs[j][half * kDH + i], o[i]);
    }
    m = mnew;
  }
  if (!row_ok) return;
  const float inv = 1.f / l;
  float* op = O + (((size_t)(b * Hq + h) * N) + row) * D + half * kDH;
#pragma unroll
  for (int i = 0; i < kDH; i += 4) {
    float4 w = make_float4(o[i] * inv, o[i + 1] * inv, o[i + 2] * inv, o[i + 3] * inv);
    *reinterpret_cast<float4*>(op + i) = w;
  }
  if (half == 0) L[(size_t)(b * Hq + h) * N + row] = (m + log2_fast(l)) * kLn2;
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a) {
  const int nqb = (a.N + kRows - 1) / kRows;
  const dim3 grid((unsigned)(nqb * a.B * a.Hq));
  const dim3 block(kRows * (D / kDH));
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
