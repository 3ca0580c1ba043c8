// Multi-head attention forward in fp32 (the fp32 reference-precision path).
//
// Same method as the bf16 kernel -- the tiled online softmax of "TileLang
// study notes" (section "FlashAttention implementation") with base-2
// exponentials after folding scale*log2(e) ("TileLang programming model and
// FlashMLA", section 3.1) -- but every product and sum is an fp32 VALU FMA,
// for callers that need fp32 accuracy rather than MFMA throughput.
//
// Four waves per workgroup; each query row is spread over R = 8 neighbouring
// lanes (lane r of a row owns the 16-byte chunks r, r + 8, ... of the row),
// so a wave holds 8 rows and a workgroup 32. K/V tiles of 32 keys are staged
// in LDS; at each key the 8 lanes of a row read 8 consecutive chunks of the
// key row (one 128-byte run, the same for every row of the wave), form
// partial dot products and sum them over the row's lanes with three DPP
// steps. Each lane keeps the row's running max and sum (identical across the
// row's lanes) and its own slice of the output. The running max is raised
// exactly (no threshold) so the result follows the recurrence step for step.
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

constexpr int kF32R = 8;                 // lanes per query row
constexpr int kF32NW = 4;                // waves per workgroup
constexpr int kF32Rows = 64 / kF32R * kF32NW;  // query rows per workgroup

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kF32NW) void mha_fwd_f32_kernel(F32Args a) {
  constexpr int BC = 32;
  constexpr int C4 = D / 4;         // 16-byte chunks per row
  constexpr int CL = C4 / kF32R;    // chunks per lane
  static_assert(C4 % kF32R == 0, "row chunks must split over the row's lanes");
  __shared__ f32x4 ks[BC * C4];
  __shared__ f32x4 vs[BC * C4];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int sub = lane & (kF32R - 1);
  const int bh = blockIdx.x;
  const int Sq = a.Sq, Skv = a.Skv;
  const int row0 = blockIdx.y * kF32Rows;
  const int row = row0 + (t >> 3);
  const bool valid = row < Sq;
  const float* kp = a.k + (size_t)bh * Skv * D;
  const float* vp = a.v + (size_t)bh * Skv * D;

  f32x4 q[CL], o[CL];
  {
    const f32x4* qr = (const f32x4*)(a.q + ((size_t)bh * Sq + (valid ? row : 0)) * D);
#pragma unroll
    for (int i = 0; i < CL; ++i) {
      q[i] = valid ? qr[sub + kF32R * i] : f32x4{0.f, 0.f, 0.f, 0.f};
      o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  float m = -INFINITY, l = 0.f;
  const int lim = CAUSAL ? min(Skv - 1, row + Skv - Sq) : Skv - 1;
  int kv_end = Skv;
  if (CAUSAL) {
    const int last = min(row0 + kF32Rows - 1, Sq - 1);
    kv_end = max(0, min(Skv, last + Skv - Sq + 1));
  }

  for (int t0 = 0; t0 < kv_end; t0 += BC) {
    __syncthreads();
    for (int e = t; e < BC * C4; e += 64 * kF32NW) {
      const int r = e / C4, c4 = e - r * C4;
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
      for (int i = 0; i < CL; ++i) acc += q[i] * ks[j * C4 + sub + kF32R * i];
      const float dot = octet_sum((acc[0] + acc[1]) + (acc[2] + acc[3]));
      s[j] = (t0 + j <= lim) ? dot * a.c : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    if (mx > m) {
      const float alpha = exp2f(m - mx);  // m = -inf gives 0
      l *= alpha;
#pragma unroll
      for (int i = 0; i < CL; ++i) o[i] *= alpha;
      m = mx;
    }
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      const float p = s[j] == -INFINITY ? 0.f : exp2f(s[j] - m);
      l += p;
#pragma unroll
      for (int i = 0; i < CL; ++i) o[i] += p * vs[j * C4 + sub + kF32R * i];
    }
  }

  if (valid) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    f32x4* orow = (f32x4*)(a.o + ((size_t)bh * Sq + row) * D);
#pragma unroll
    for (int i = 0; i < CL; ++i) orow[sub + kF32R * i] = o[i] * inv;
    if (sub == 0) a.lse[(size_t)bh * Sq + row] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_f32(const F32Args& a, int n_bh, hipStream_t stream) {
  const dim3 grid(n_bh, (a.Sq + kF32Rows - 1) / kF32Rows);
  hipLaunchKernelGGL((mha_fwd_f32_kernel<D, CAUSAL>), grid, dim3(64 * kF32NW), 0, stream, a);
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
