// Multi-head attention forward in fp32 (the fp32 reference-precision path).
//
// Same method as the bf16 kernel -- the tiled online softmax of "TileLang
// study notes" (section "FlashAttention implementation") with base-2
// exponentials after folding scale*log2(e) ("TileLang programming model and
// FlashMLA", section 3.1) -- but every product and sum is an fp32 VALU FMA,
// for callers that need fp32 accuracy rather than MFMA throughput.
//
// One wave per workgroup, one query row per lane; K/V tiles of 32 keys are
// staged in LDS and read by all lanes as broadcasts. The running max is
// raised exactly (no threshold) so the result follows the recurrence step
// for step.
#include "device_common.h"
#include "launch.h"

namespace tattn {

struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int Sq, Skv;
  float c;  // scale * log2(e)
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) void mha_fwd_f32_kernel(F32Args a) {
  constexpr int BC = 32;
  __shared__ f32x4 ks[BC * D / 4];
  __shared__ f32x4 vs[BC * D / 4];

  const int lane = threadIdx.x;
  const int bh = blockIdx.x;
  const int Sq = a.Sq, Skv = a.Skv;
  const int row = blockIdx.y * 64 + lane;
  const bool valid = row < Sq;
  const float* kp = a.k + (size_t)bh * Skv * D;
  const float* vp = a.v + (size_t)bh * Skv * D;

  f32x4 q[D / 4], o[D / 4];
  {
    const f32x4* qr = (const f32x4*)(a.q + ((size_t)bh * Sq + (valid ? row : 0)) * D);
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
      q[i] = valid ? qr[i] : f32x4{0.f, 0.f, 0.f, 0.f};
      o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  float m = -INFINITY, l = 0.f;
  const int lim = CAUSAL ? min(Skv - 1, row + Skv - Sq) : Skv - 1;
  int kv_end = Skv;
  if (CAUSAL) {
    const int last = min((int)blockIdx.y * 64 + 63, Sq - 1);
    kv_end = max(0, min(Skv, last + Skv - Sq + 1));
  }

  for (int t0 = 0; t0 < kv_end; t0 += BC) {
    __syncthreads();
    for (int e = lane; e < BC * D / 4; e += 64) {
      const int r = e / (D / 4), c4 = e - r * (D / 4);
      const int gr = min(t0 + r, Skv - 1);
      ks[e] = ((const f32x4*)(kp + (size_t)gr * D))[c4];
      vs[e] = ((const f32x4*)(vp + (size_t)gr * D))[c4];
    }
    __syncthreads();

    float s[BC];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < D / 4; ++i) acc += q[i] * ks[j * (D / 4) + i];
      const float dot = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      s[j] = (t0 + j <= lim) ? dot * a.c : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    if (mx > m) {
      const float alpha = exp2f(m - mx);  // m = -inf gives 0
      l *= alpha;
#pragma unroll
      for (int i = 0; i < D / 4; ++i) o[i] *= alpha;
      m = mx;
    }
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      const float p = s[j] == -INFINITY ? 0.f : exp2f(s[j] - m);
      l += p;
#pragma unroll
      for (int i = 0; i < D / 4; ++i) o[i] += p * vs[j * (D / 4) + i];
    }
  }

  if (valid) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    f32x4* orow = (f32x4*)(a.o + ((size_t)bh * Sq + row) * D);
#pragma unroll
    for (int i = 0; i < D / 4; ++i) orow[i] = o[i] * inv;
    a.lse[(size_t)bh * Sq + row] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_f32(const F32Args& a, int n_bh, hipStream_t stream) {
  const dim3 grid(n_bh, (a.Sq + 63) / 64);
  hipLaunchKernelGGL((mha_fwd_f32_kernel<D, CAUSAL>), grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_mha_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                              int B, int H, int Sq, int Skv, int D, bool causal, float scale,
                              hipStream_t stream) {
  F32Args a{q, k, v, o, lse, Sq, Skv, scale * kLog2e};
  const int n_bh = B * H;
  if (D == 128) return causal ? launch_f32<128, true>(a, n_bh, stream) : launch_f32<128, false>(a, n_bh, stream);
  return causal ? launch_f32<64, true>(a, n_bh, stream) : launch_f32<64, false>(a, n_bh, stream);
}

}  // namespace tattn
