// Multi-head attention forward, bf16 inputs, fp32 accumulation, gfx950.
//
// Method: the tiled online-softmax attention of "TileLang study notes"
// (section "FlashAttention implementation": per query tile, loop over K/V
// tiles, S = scale*Q*K^T, running row max m and sum l, rescale of the output
// accumulator, O = acc / l), with the exponentials taken in base 2 after
// folding scale*log2(e) into one multiply, as "TileLang programming model and
// FlashMLA" (section 3.1) does. The K/V tile loop is software pipelined over
// LDS stages (section 2.2 there).
//
// gfx950 mapping (one workgroup = NW waves = NW*32 query rows, two waves per
// SIMD):
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
//  * K/V tiles of 64 keys move HBM -> LDS with global_load_lds_dwordx4 (no
//    VGPR round trip) into an XOR-swizzled layout, through a ring of three
//    stages; one barrier per tile. Every LDS address is a per-lane base plus
//    an instruction offset (stage, key block, row half).
//  * The two waves of a SIMD run offset by a phase: waves 0..NW/2-1 run
//    scores(t), softmax(t), P*V(t) after barrier t; waves NW/2.. run
//    softmax(t-1), P*V(t-1), scores(t), so one wave's VALU phase overlaps the
//    other's MFMA phases. Tiles that need masks (causal diagonal, ragged
//    tail) run in step afterwards.
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

template <int D, int NW, int BC, int NSTAGE, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void mha_fwd_bf16_kernel(MhaArgs a) {
  constexpr int BR = NW * 32;      // query rows per workgroup (32 per wave)
  constexpr int CPR = D / 8;       // 16-byte chunks per row
  constexpr int RS = D * 2;        // row stride in bytes
  constexpr int KS = D / 16;       // MFMA k-steps of Q*K^T
  constexpr int DB = D / 32;       // 32-wide blocks of the head dimension
  constexpr int KB = BC / 32;      // 32-key blocks per tile
  constexpr int TILE = BC * RS;    // bytes of one K or V tile
  constexpr int VREG = NSTAGE * TILE;  // V tiles follow the NSTAGE K tiles
  constexpr int LOADS = BC * CPR / (64 * NW);
  constexpr int LPT = 2 * LOADS;   // loads per wave per tile (K and V)
  static_assert(BC * CPR % (64 * NW) == 0, "tile must split into whole wave loads");
  static_assert(NSTAGE * TILE <= 65536, "LDS offsets must fit the 16-bit instruction offset");
  static_assert(NSTAGE == 3, "three LDS stages: the lagging wave group reads tile t-1 after barrier t");
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
  const int wrow0 = q0 + wave * 32;
  const uint16_t* qp = a.q + (size_t)bh * Sq * D;
  const char* kp = (const char*)(a.k + (size_t)bh * Skv * D);
  const char* vp = (const char*)(a.v + (size_t)bh * Skv * D);
  const float c = a.c;

  int kv_end = Skv;
  if (CAUSAL) {
    const int last = min(q0 + BR, Sq) - 1;
    kv_end = max(0, min(Skv, last + Skv - Sq + 1));
  }
  const int nt = (kv_end + BC - 1) / BC;
  // last key this wave's rows can see (causal); tiles past it are skipped
  const int wave_kv_last = CAUSAL ? min(wrow0 + 31, Sq - 1) + Skv - Sq : Skv - 1;

  // Lane-dependent LDS address parts. The XOR swizzle touches only the low
  // 4 chunk bits and depends only on the low 4 row bits, so the key block,
  // row half, K/V choice and stage are immediate offsets.
  const uint32_t smem0 = lds_addr(smem);
  uint32_t kbase[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kbase[ks] = smem0 + col * RS + 16 * swz<CPR>(col, 2 * ks + hi);
  uint32_t vbase[2][DB];
  {
    const int gq = (lane >> 4) & 1, s16 = lane & 15;
    const int x = 2 * gq + ((s16 & 3) >> 1), boff = 8 * (s16 & 1);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int rr = 8 * e + 4 * hi + (s16 >> 2);
#pragma unroll
      for (int db = 0; db < DB; ++db) vbase[e][db] = smem0 + VREG + rr * RS + 16 * swz<CPR>(rr, db * 4 + x) + boff;
    }
  }

  // Tile t -> stage ST: wave loads n cover chunk slots (n*NW + wave)*64 + lane.
  auto issue = [&](int t, auto STc) {
    constexpr int ST = decltype(STc)::value;
    const int lim = Skv - 1 - t * BC;  // >= 0: tile t has a visible key
    const char* kt = kp + (size_t)t * BC * RS;
    const char* vt = vp + (size_t)t * BC * RS;
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
      const int slot = (n * NW + wave) * 64 + lane;
      const int row = slot / CPR;
      const uint32_t off = (uint32_t)(min(row, lim) * RS + 16 * swz<CPR>(row, slot % CPR));
      const uint32_t dst = smem0 + ST * TILE + (n * NW + wave) * 1024;
      load_lds16_asm(kt + off, dst);
      load_lds16_asm(vt + off, dst + VREG);
    }
  };

  if (nt > 0) issue(0, std::integral_constant<int, 0>{});

  // Q^T fragments (B operand), loaded once.
  bf16x8 qf[KS];
  {
    const int row = wrow0 + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x = {0, 0, 0, 0};
      if (row < Sq) x = *(const u32x4*)(qp + (size_t)row * D + ks * 16 + hi * 8);
      qf[ks] = as_bf16x8(x);
    }
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m = -INFINITY, lsum = 0.f;

  // ---- the three phases of one tile (stage ST):
  //   M1: S^T = K*Q^T (MFMA), V: masks + online softmax (VALU), M2: O^T += V^T*P^T (MFMA)
  auto m1 = [&](auto STc, f32x16 (&s)[KB]) {
    constexpr int ST = decltype(STc)::value;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s[kb] = f32x16{};
    // k-steps in groups of 2; inside a group the key blocks alternate, so
    // consecutive MFMAs never depend on each other
    static_for<KS / 2>([&](auto Gc) {
      constexpr int g = decltype(Gc)::value;
      bf16x8 kf[2][KB];
      static_for<2>([&](auto Uc) {
        static_for<KB>([&](auto KBc) {
          kf[Uc][KBc] = as_bf16x8(lds_read128(
              (const void*)(uintptr_t)(kbase[2 * g + Uc] + ST * TILE + decltype(KBc)::value * 32 * RS)));
        });
      });
      static_for<2>([&](auto Uc) {
        static_for<KB>([&](auto KBc) { s[KBc] = mfma32(kf[Uc][KBc], qf[2 * g + Uc], s[KBc]); });
      });
    });
  };

  auto vphase = [&](int t, f32x16 (&s)[KB], bf16x8 (&pf)[KB][2], auto MASKEDc) {
    const int kv0 = t * BC;
    if constexpr (decltype(MASKEDc)::value) {
      const int lim = CAUSAL ? min(Skv - 1, wrow0 + col + Skv - Sq) : Skv - 1;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kv0 + kb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3) > lim) s[kb][i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = max_halves(mx) * c;
    const bool raise = mx - m > TAU;  // false when mx == -inf
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float alpha = raise ? fast_exp2(m - mx) : 1.f;
      m = raise ? mx : m;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    }
    const float mc = m == -INFINITY ? 0.f : m;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          p[j] = fast_exp2(fmaf(s[kb][half * 8 + j], c, -mc));
          lsum += p[j];
        }
        u32x4 w = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                   pack_bf16x2(p[6], p[7])};
        pf[kb][half] = as_bf16x8(w);
      }
  };

  auto m2 = [&](auto STc, const bf16x8 (&pf)[KB][2]) {
    constexpr int ST = decltype(STc)::value;
    // for each 16-key slice: read the V^T fragments of all d-blocks, then one
    // MFMA per d-block (independent accumulators back to back)
    static_for<KB * 2>([&](auto SC) {
      constexpr int kb = decltype(SC)::value / 2, half = decltype(SC)::value % 2;
      constexpr int off = ST * TILE + kb * 32 * RS + half * 16 * RS;
      bf16x8 vf[DB];
      static_for<DB>([&](auto DBc) {
        const u32x2 r0 = lds_read_tr16<off>(vbase[0][DBc]);
        const u32x2 r1 = lds_read_tr16<off>(vbase[1][DBc]);
        vf[DBc] = cat_tr(r0, r1);
      });
      static_for<DB>([&](auto DBc) { oacc[DBc] = mfma32(vf[DBc], pf[kb][half], oacc[DBc]); });
    });
  };

  // Two wave groups share each SIMD: group 0 (waves 0..NW/2-1) runs
  // M1(t) V(t) M2(t) after barrier t; group 1 runs V(t-1) M2(t-1) M1(t).
  // Each group's VALU phase then overlaps the other group's MFMA phases.
  // Tile t-1 stays readable until barrier t+1 because the ring has three
  // stages and the refill issued at barrier t targets stage (t+1) % 3.
  const bool lag = wave >= NW / 2;
  f32x16 s_cur[KB];   // scores of the tile in flight (group 1: of tile t-1 across the barrier)

  // One tile step of a group; LAG is a compile-time copy per group so the
  // two groups' loops are allocated independently.
  auto tile = [&](int t, auto STc, auto LAGc, bool& pending) {
    constexpr int ST = decltype(STc)::value;
    constexpr int SP = (ST + NSTAGE - 1) % NSTAGE;  // stage of tile t-1
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    barrier();
    if (t + 1 < nt) issue(t + 1, std::integral_constant<int, (ST + 1) % NSTAGE>{});
    if constexpr (!decltype(LAGc)::value) {
      bf16x8 pf[KB][2];
      m1(STc, s_cur);
      vphase(t, s_cur, pf, std::false_type{});
      m2(STc, pf);
    } else {
      if (pending) {
        bf16x8 pf[KB][2];
        vphase(t - 1, s_cur, pf, std::false_type{});
        m2(std::integral_constant<int, SP>{}, pf);
      }
      pending = true;
      m1(STc, s_cur);
    }
  };

  // Tiles [0, t_plain) need no mask for any wave of the workgroup; they run
  // unrolled over the LDS stages with the two groups offset. The rest
  // (causal diagonal, ragged tail) run in step, masked, after group 1 has
  // finished its pending tile.
  int t_plain = Skv / BC;
  if (CAUSAL) t_plain = min(t_plain, max(0, (q0 + Skv - Sq + 1) / BC));
  t_plain = min(t_plain, nt);
  const int t_main = t_plain - t_plain % NSTAGE;
  auto run = [&](auto LAGc) {
    bool pending = false;
    for (int t = 0; t < t_main; t += NSTAGE)
      static_for<NSTAGE>([&](auto STc) { tile(t + decltype(STc)::value, STc, LAGc, pending); });
    if constexpr (decltype(LAGc)::value) {
      if (pending) {  // tile t_main - 1 sits in stage NSTAGE - 1
        bf16x8 pf[KB][2];
        vphase(t_main - 1, s_cur, pf, std::false_type{});
        m2(std::integral_constant<int, NSTAGE - 1>{}, pf);
      }
    }
  };
  if (lag) run(std::true_type{});
  else run(std::false_type{});
  int t = t_main;

  // the remaining tiles run without the lag (both groups in step)
  auto tile_step = [&](int tt, auto STc) {
    constexpr int ST = decltype(STc)::value;
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    barrier();
    if (tt + 1 < nt) issue(tt + 1, std::integral_constant<int, (ST + 1) % NSTAGE>{});
    if (CAUSAL && tt * BC > wave_kv_last) return;
    bf16x8 pf[KB][2];
    m1(STc, s_cur);
    vphase(tt, s_cur, pf, std::true_type{});
    m2(STc, pf);
  };
  for (; t < nt; ++t) {
    const int st = t % NSTAGE;
    if (st == 0) tile_step(t, std::integral_constant<int, 0>{});
    else if (st == 1) tile_step(t, std::integral_constant<int, 1>{});
    else tile_step(t, std::integral_constant<int, 2>{});
  }

  // ---- epilogue: O = acc / l (bf16), LSE = (m + log2 l) * ln 2
  {
    const float l = sum_halves(lsum);
    const int row = wrow0 + col;
    if (row < Sq) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      uint16_t* orow = a.o + ((size_t)bh * Sq + row) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + 8 * g4 + 4 * hi;
          u32x2 w = {pack_bf16x2(oacc[db][g4 * 4 + 0] * inv, oacc[db][g4 * 4 + 1] * inv),
                     pack_bf16x2(oacc[db][g4 * 4 + 2] * inv, oacc[db][g4 * 4 + 3] * inv)};
          *(u32x2*)(orow + d) = w;
        }
      if (hi == 0) a.lse[(size_t)bh * Sq + row] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, int NW, int BC, bool CAUSAL>
static hipError_t launch_one(const MhaArgs& a, hipStream_t stream) {
  constexpr int BR = NW * 32;
  constexpr int NSTAGE = 3;
  constexpr size_t lds = 2 * (size_t)NSTAGE * BC * D * 2;
  auto kern = mha_fwd_bf16_kernel<D, NW, BC, NSTAGE, CAUSAL>;
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
  if (D == 128) return causal ? launch_one<128, 8, 64, true>(a, stream) : launch_one<128, 8, 64, false>(a, stream);
  return causal ? launch_one<64, 8, 64, true>(a, stream) : launch_one<64, 8, 64, false>(a, stream);
}

}  // namespace tattn
