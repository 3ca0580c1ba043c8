// Multi-head attention forward, bf16 inputs, fp32 accumulation, gfx950.
//
// Method: the tiled online-softmax attention of "TileLang study notes"
// (section "FlashAttention implementation": per query tile, loop over K/V
// tiles, S = scale*Q*K^T, running row max m and sum l, rescale of the output
// accumulator, O = acc / l), with the exponentials taken in base 2 after
// folding scale*log2(e) into one multiply, as "TileLang programming model and
// FlashMLA" (section 3.1) does. The K/V tile loop is software pipelined over
// two LDS stages (section 2.2 there).
//
// gfx950 mapping (one workgroup = NW waves = NW*QB*32 query rows):
//  * S^T = K * Q^T on v_mfma_f32_32x32x16_bf16. Q^T is the B operand and is
//    loaded once into registers; K comes from LDS as the A operand. With S
//    transposed, lane l owns query column l%32 and 16 of the 32 keys of each
//    key block, so a row max / row sum is an in-lane reduction plus one
//    v_permlane32_swap with lane l ^ 32.
//  * O^T = V^T * P^T: the P^T B operand is the S^T accumulator itself,
//    exponentiated and rounded to bf16 in place (its key order matches the
//    A operand's); V^T is read from the row-major V tile by
//    ds_read_b64_tr_b16. O^T keeps lane l on query l%32, so the rescale and
//    the final 1/l are per-lane multiplies.
//  * K/V tiles move HBM -> LDS with global_load_lds_dwordx4 (no VGPR round
//    trip) into an XOR-swizzled layout, double buffered; one barrier per
//    tile.
//  * The running max is only raised when a new score exceeds it by more than
//    2^8 (in base-2 units), so the O rescale runs on few tiles; every
//    exponential stays <= 2^8 and the result is unchanged (both O and l are
//    taken relative to the same m).
//  * Workgroup -> tile order: the hardware hands workgroup i to XCD i % 8;
//    all query tiles of a (batch, head) are sent to one XCD so its K/V stays
//    in that XCD's L2, and causal launches run the longest tiles first.
#include "device_common.h"
#include "launch.h"

namespace tattn {

struct MhaArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int Sq, Skv;
  int n_bh;
  int n_qtiles;
  float c;    // scale * log2(e)
  int remap;  // n_bh % 8 == 0: XCD-grouped order
};

template <int D, int NW, int QB, int BC, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1))) void mha_fwd_bf16_kernel(MhaArgs a) {
  constexpr int BR = NW * QB * 32;
  constexpr int CPR = D / 8;   // 16-byte chunks per row
  constexpr int KS = D / 16;   // MFMA k-steps of Q*K^T
  constexpr int DB = D / 32;   // 32-wide blocks of the head dimension
  constexpr int KB = BC / 32;  // 32-key blocks per tile
  constexpr int TILE = BC * D * 2;
  constexpr int LOADS = BC * CPR / (64 * NW);
  static_assert(BC * CPR % (64 * NW) == 0, "tile must split into whole wave loads");
  constexpr float TAU = 8.0f;

  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hi = lane >> 5;      // wave half
  const int col = lane & 31;     // query column owned by the lane

  int bh, qt;
  {
    const int i = blockIdx.x;
    int rank;
    if (a.remap) {
      const int nbh_x = a.n_bh >> 3, local = i >> 3, xcd = i & 7;
      rank = local / nbh_x;
      bh = xcd * nbh_x + (local - rank * nbh_x);
    } else {
      rank = i / a.n_bh;
      bh = i - rank * a.n_bh;
    }
    qt = CAUSAL ? a.n_qtiles - 1 - rank : rank;
  }

  const int Sq = a.Sq, Skv = a.Skv;
  const int q0 = qt * BR;
  const int wrow0 = q0 + wave * QB * 32;
  const uint16_t* qp = a.q + (size_t)bh * Sq * D;
  const uint16_t* kp = a.k + (size_t)bh * Skv * D;
  const uint16_t* vp = a.v + (size_t)bh * Skv * D;
  const float c = a.c;

  int kv_end = Skv;
  if (CAUSAL) {
    const int last = min(q0 + BR, Sq) - 1;
    kv_end = max(0, min(Skv, last + Skv - Sq + 1));
  }
  const int nt = (kv_end + BC - 1) / BC;

  auto issue = [&](int t, int stage) {
    char* kl = smem + stage * 2 * TILE;
    char* vl = kl + TILE;
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
      const int slot = (n * NW + wave) * 64 + lane;
      const int row = slot / CPR;
      const int chunk = swz<CPR>(row, slot % CPR);
      int gr = t * BC + row;
      gr = gr < Skv ? gr : Skv - 1;
      const size_t off = (size_t)gr * D + chunk * 8;
      load_lds16(kp + off, kl + (n * NW + wave) * 1024);
      load_lds16(vp + off, vl + (n * NW + wave) * 1024);
    }
  };

  if (nt > 0) issue(0, 0);

  // Q^T fragments (B operand), loaded once.
  bf16x8 qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wrow0 + qb * 32 + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x = {0, 0, 0, 0};
      if (row < Sq) x = *(const u32x4*)(qp + (size_t)row * D + ks * 16 + hi * 8);
      qf[qb][ks] = as_bf16x8(x);
    }
  }

  f32x16 oacc[DB][QB];
  float m[QB], lsum[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    lsum[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db][qb] = f32x16{};
  }

  for (int t = 0; t < nt; ++t) {
    const int st = t & 1;
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    barrier();
    if (t + 1 < nt) issue(t + 1, st ^ 1);
    const char* kl = smem + st * 2 * TILE;
    const char* vl = kl + TILE;

    // ---- S^T = K * Q^T (all K fragments of a key block are read before its MFMAs)
    f32x16 s[KB][QB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int row = kb * 32 + col;
      bf16x8 kf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[ks] = as_bf16x8(lds_read128(kl + (row * CPR + swz<CPR>(row, ks * 2 + hi)) * 16));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma32(kf[ks], qf[qb][ks], s[kb][qb]);
      // keep the KS operand reads of this key block ahead of its MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, KS * QB, 0);
    }

    // ---- masks (tail keys, causal diagonal)
    const int kv0 = t * BC;
    const bool need_mask = (kv0 + BC > Skv) || (CAUSAL && kv0 + BC - 1 > wrow0 + Skv - Sq);
    if (need_mask) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int lim = CAUSAL ? min(Skv - 1, wrow0 + qb * 32 + col + Skv - Sq) : Skv - 1;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int j = kv0 + kb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
            if (j > lim) s[kb][qb][i] = -INFINITY;
          }
      }
    }

    // ---- online softmax; P^T fragments in bf16
    bf16x8 pf[KB][2][QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][qb][i]);
      mx = max_halves(mx) * c;
      const bool raise = mx - m[qb] > TAU;  // false when mx == -inf
      if (__builtin_amdgcn_ballot_w64(raise)) {
        const float alpha = raise ? fast_exp2(m[qb] - mx) : 1.f;
        m[qb] = raise ? mx : m[qb];
        lsum[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db][qb] *= alpha;
      }
      const float mc = m[qb] == -INFINITY ? 0.f : m[qb];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          float p[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            p[j] = fast_exp2(fmaf(s[kb][qb][half * 8 + j], c, -mc));
            lsum[qb] += p[j];
          }
          u32x4 w = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                     pack_bf16x2(p[6], p[7])};
          pf[kb][half][qb] = as_bf16x8(w);
        }
    }

    // ---- O^T += V^T * P^T; the transposing reads of d-block db+1 are in
    // flight while the MFMAs of d-block db run.
    {
      const int g = (lane >> 4) & 1, s16 = lane & 15;
      const int rsub = 4 * hi + (s16 >> 2);
      const uint32_t vbase = lds_addr(vl);
      auto vread = [&](int db, u32x2 (&r)[KB * 4]) {
        const int d = db * 32 + 16 * g + 4 * (s16 & 3);
        const int chunk = d >> 3, boff = (d & 7) * 2;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int rr = kb * 32 + half * 16 + 8 * e + rsub;
              r[(kb * 2 + half) * 2 + e] =
                  lds_read_tr16_async<0>(vbase + (rr * CPR + swz<CPR>(rr, chunk)) * 16 + boff);
            }
      };
      u32x2 vr[2][KB * 4];
      vread(0, vr[0]);
      wait_lds_tied(vr[0]);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        if (db + 1 < DB) vread(db + 1, vr[(db + 1) & 1]);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int x = (kb * 2 + half) * 2;
            const bf16x8 vf = cat_tr(vr[db & 1][x], vr[db & 1][x + 1]);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = mfma32(vf, pf[kb][half][qb], oacc[db][qb]);
          }
        if (db + 1 < DB) wait_lds_tied(vr[(db + 1) & 1]);
      }
    }
  }

  // ---- epilogue: O = acc / l (bf16), LSE = (m + log2 l) * ln 2
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = sum_halves(lsum[qb]);
    const int row = wrow0 + qb * 32 + col;
    if (row < Sq) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      uint16_t* orow = a.o + ((size_t)bh * Sq + row) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + 8 * g4 + 4 * hi;
          u32x2 w = {pack_bf16x2(oacc[db][qb][g4 * 4 + 0] * inv, oacc[db][qb][g4 * 4 + 1] * inv),
                     pack_bf16x2(oacc[db][qb][g4 * 4 + 2] * inv, oacc[db][qb][g4 * 4 + 3] * inv)};
          *(u32x2*)(orow + d) = w;
        }
      if (hi == 0) a.lse[(size_t)bh * Sq + row] = l > 0.f ? (m[qb] + __log2f(l)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, int NW, int QB, int BC, bool CAUSAL>
static hipError_t launch_one(const MhaArgs& a, hipStream_t stream) {
  constexpr int BR = NW * QB * 32;
  constexpr size_t lds = 2 * 2 * (size_t)BC * D * 2;
  auto kern = mha_fwd_bf16_kernel<D, NW, QB, BC, CAUSAL>;
  // Thread-safe one-time opt-in to more than the default dynamic LDS.
  static const hipError_t attr_err =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr_err != hipSuccess) return attr_err;
  MhaArgs b = a;
  b.n_qtiles = (a.Sq + BR - 1) / BR;
  const long long grid = (long long)b.n_qtiles * a.n_bh;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  b.remap = (a.n_bh % 8) == 0;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NW * 64), lds, stream, b);
  return hipGetLastError();
}

hipError_t launch_mha_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int Sq, int Skv, int D, bool causal, float scale,
                               hipStream_t stream) {
  MhaArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.Sq = Sq;
  a.Skv = Skv;
  a.n_bh = B * H;
  a.c = scale * kLog2e;
  if (D == 128) {
    return causal ? launch_one<128, 4, 1, 64, true>(a, stream) : launch_one<128, 4, 1, 64, false>(a, stream);
  }
  return causal ? launch_one<64, 4, 1, 64, true>(a, stream) : launch_one<64, 4, 1, 64, false>(a, stream);
}

}  // namespace tattn
