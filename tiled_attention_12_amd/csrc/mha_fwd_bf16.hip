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
// gfx950 mapping (one workgroup = NW waves = NW*32 query rows; the dense
// launch has 8 waves, two per SIMD, except on small launches, below):
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
//  * Each wave runs one tile behind itself: after barrier t it forms the
//    scores of tile t on the MFMAs while the VALU exponentiates the scores of
//    tile t-1 (instruction groups interleaved with sched_group_barrier), then
//    accumulates P*V of tile t-1. These tiles are exponentiated against tile
//    0's max without forming their own maxima; after the item each wave
//    checks l and O for overflow and, if one is found, writes its rows again
//    with an exact fp32 online softmax. Tiles that need masks (causal
//    diagonal, ragged tail) run unpipelined afterwards with the exact step.
//  * Exact step: the running max is only raised when a new score exceeds it
//    by more than 2^8 (in base-2 units), so the O rescale runs on few tiles;
//    every exponential stays <= 2^8 and the result is unchanged (both O and l
//    are taken relative to the same m). Masks take one bit mask of the
//    visible keys per 32-key block, then a one-bit extract and a bitfield
//    select per score.
//  * Small dense launches (fewer 256-row items than compute units; without a
//    mask, at most half as many) run the same steps in 4-wave workgroups of
//    128 rows, two per compute unit: half-height items shorten the longest
//    item and spread over more compute units. Their ring holds two K and two
//    V stages (64 KB): the pipelined steps refill K of tile t+1 and V of tile
//    t at barrier t, so V is loaded one step after its K, while its P*V is
//    still a step away.
//  * Windows and block masks run a separate walk: 4-wave workgroups of 128
//    rows (two 64-row mask blocks), 32-key tiles, three or four workgroups
//    per compute unit, visiting only the tiles some row sees and the mask
//    keeps, every visited tile through the exact step.
//  * Persistent grid: as many workgroups as fit on the compute units loop
//    over work items (one NW*32-row query tile of one (batch, head) each).
//    The hardware hands workgroup i to XCD i % 8 and item i runs on XCD i % 8
//    too: all query tiles of a (batch, head) go to one XCD so its K/V stays
//    in that XCD's L2. Causal items are taken longest first, and each
//    workgroup's passes alternate direction so long and short tiles pair up.
#include "device_common.h"
#include "launch.h"

// K/V ring depth of the 8-wave dense kernel and the window/mask walk: 3
// (prefetch one tile ahead) or 4 (two tiles ahead); the 4-wave dense kernel
// keeps two K and two V stages
#ifndef TATTN_MHA_STAGES
#define TATTN_MHA_STAGES 3
#endif
// VALU instructions scheduled between consecutive score MFMAs
#ifndef TATTN_VALU_PER_MFMA
#define TATTN_VALU_PER_MFMA 3
#endif


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
  int H;      // query heads
  int group;  // query heads per KV head
  int window; // key window half-width (0: none)
  const uint8_t* bmask;  // [B, H, nqb, nkb] per 64x64 block, or null
  int nqb, nkb;
  int n_items;  // n_qtiles * n_bh
};

// Block size of the block mask: 64 query rows x 64 keys (one key tile; each
// wave's 32 rows lie inside one query block).
constexpr int kMaskBlock = 64;

// Waves per SIMD: for the 4-wave window/mask walk four at head width 64 and
// three at 128 (that many workgroups per compute unit, within the 128 or 168
// registers it leaves each wave), two for the others.
template <int D, int NW, bool EXT>
constexpr int kWavesPerSimd = (EXT && NW == 4) ? (D == 64 ? 4 : 3) : 2;

// The 4-wave walk at head width 128 takes the lane id through an opaque copy
// per work item, so its lane-dependent addresses are recomputed per item
// instead of being held across items: that keeps it within 168 registers
// (held, they spilled and were reloaded from scratch at every item start).
// The other instantiations keep them, which measured faster for them.
template <int D, int NW, bool EXT>
constexpr bool kLanePerItem = EXT && NW == 4 && D == 128;

template <int D, int NW, int BC, int NSTAGE, bool CAUSAL, bool EXT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<D, NW, EXT>, kWavesPerSimd<D, NW, EXT>))) void mha_fwd_bf16_kernel(MhaArgs a) {
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
  // Tile t+PF is loaded while tile t is scored and tile t-1 accumulated, so
  // the ring needs PF + 2 stages.
  // The dense 4-wave shape refills K and V one step apart (K of tile t+1 and
  // V of tile t at barrier t), so two stages of each suffice.
  constexpr bool SKV = !EXT && NW == 4;
  constexpr int PF = SKV ? 1 : NSTAGE - 2;
  static_assert(PF == 1 || PF == 2, "prefetch distance 1 or 2");
  static_assert(!SKV || NSTAGE == 2, "split refills: two K and two V stages");
  constexpr int UN = NSTAGE % 2 == 0 ? NSTAGE : 2 * NSTAGE;  // unroll: stages x score sets
  constexpr float TAU = 8.0f;

  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int lane0 = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hi0 = lane0 >> 5;    // wave half
  const int col0 = lane0 & 31;   // query column owned by the lane

  // One work item = one (batch*head, BR-row query tile). The grid is
  // persistent (as many workgroups as fit on the compute units at once);
  // item i runs where workgroup i would: on XCD i % 8.
  auto process = [&](const int i) {
    int lane = lane0, hi = hi0, col = col0;
    if constexpr (kLanePerItem<D, NW, EXT>) {
      asm volatile("" : "+v"(lane));
      hi = lane >> 5;
      col = lane & 31;
    }
    int bh, qt;
    {
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
    // query head h of batch b reads KV head h / group
    const int bq = bh / a.H, hq = bh - bq * a.H;
    const size_t kvh = (size_t)bq * (a.H / a.group) + hq / a.group;
    const char* kp = (const char*)(a.k + kvh * Skv * D);
    const char* vp = (const char*)(a.v + kvh * Skv * D);
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

    // Tile t -> stage ST: wave loads n cover chunk slots (n*NW + wave)*64 + lane;
    // WH selects the K (1) and/or V (2) half.
    auto issue_kv = [&](int t, auto STc, auto WHc) {
      constexpr int ST = decltype(STc)::value;
      constexpr int WH = decltype(WHc)::value;
      const int lim = Skv - 1 - t * BC;  // >= 0: tile t has a visible key
      const char* kt = kp + (size_t)t * BC * RS;
      const char* vt = vp + (size_t)t * BC * RS;
#pragma unroll
      for (int n = 0; n < LOADS; ++n) {
        const int slot = (n * NW + wave) * 64 + lane;
        const int row = slot / CPR;
        const uint32_t off = (uint32_t)(min(row, lim) * RS + 16 * swz<CPR>(row, slot % CPR));
        const uint32_t dst = smem0 + ST * TILE + (n * NW + wave) * 1024;
        if constexpr ((WH & 1) != 0) load_lds16_sbase(kt, off, dst);
        if constexpr ((WH & 2) != 0) load_lds16_sbase(vt, off, dst + VREG);
      }
    };
    using OnlyK = std::integral_constant<int, 1>;
    using OnlyV = std::integral_constant<int, 2>;
    auto issue = [&](int t, auto STc) { issue_kv(t, STc, std::integral_constant<int, 3>{}); };

    // Tiles 0 .. t_main-1 need no mask (the pipelined part of the dense path).
    auto first_masked_tile = [&]() {
      int t = Skv / BC;
      if (CAUSAL) t = min(t, max(0, (q0 + Skv - Sq + 1) / BC));
      return min(t, nt);
    };
    if constexpr (SKV) {
      // V of tile 0 follows at its barrier, unless no tile is pipelined
      if (0 < nt) {
        if (first_masked_tile() > 0) issue_kv(0, std::integral_constant<int, 0>{}, OnlyK{});
        else issue(0, std::integral_constant<int, 0>{});
      }
    } else if constexpr (!EXT) {
      static_for<PF>([&](auto Ic) {
        if (decltype(Ic)::value < nt) issue(decltype(Ic)::value, Ic);
      });
    }
    // wait until this wave's loads of tile t have landed (tiles up to
    // t + PF - 1 may still be in flight)
    auto wait_tile = [&](int t) {
      if constexpr (PF == 2) {
        if (t + 1 < nt) {
          wait_vmcnt<LPT>();
          return;
        }
      }
      wait_vmcnt<0>();
    };

    // Q^T fragments (B operand), loaded once. The wave's 32 rows first come
    // into LDS, whole rows per load, through ring stages 1 and 2 (unused
    // until the first barrier of the item: K side for the first half of the
    // waves, V side for the rest), laid out like a K tile so the fragment
    // reads use the K-operand addresses. Rows past Sq repeat row Sq - 1;
    // their results are never written.
    bf16x8 qf[KS];
    constexpr bool QSTAGE = PF == 1;
    auto load_q_staged = [&]() {
      const uint32_t qb = smem0 + (wave < NW / 2 ? TILE + wave * (32 * RS) : VREG + TILE + (wave - NW / 2) * (32 * RS));
      constexpr int QL = 32 * CPR / 64;
#pragma unroll
      for (int n = 0; n < QL; ++n) {
        const int slot = n * 64 + lane;
        const int r = slot / CPR;
        const int grow = min(wrow0 + r, Sq - 1);
        load_lds16_asm((const char*)(qp + (size_t)grow * D) + 16 * swz<CPR>(r, slot % CPR), qb + n * 1024);
      }
      wait_vmcnt<0>();
      asm volatile("" ::: "memory");
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[ks] = as_bf16x8(lds_read128((const void*)(uintptr_t)(kbase[ks] - smem0 + qb)));
    };
    if constexpr (QSTAGE) {
      // the window/mask path stages Q after issuing its first tile
      if constexpr (!EXT) load_q_staged();
    } else {
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
      // consecutive MFMAs never depend on each other. The K fragments of group
      // g+1 are read while group g's MFMAs run.
      auto rd = [&](auto Gc, bf16x8 (&kf)[2][KB]) {
        constexpr int g = decltype(Gc)::value;
        static_for<2>([&](auto Uc) {
          static_for<KB>([&](auto KBc) {
            kf[Uc][KBc] = as_bf16x8(lds_read128(
                (const void*)(uintptr_t)(kbase[2 * g + Uc] + ST * TILE + decltype(KBc)::value * 32 * RS)));
          });
        });
      };
      bf16x8 kf[2][2][KB];
      rd(std::integral_constant<int, 0>{}, kf[0]);
      static_for<KS / 2>([&](auto Gc) {
        constexpr int g = decltype(Gc)::value;
        if constexpr (g + 1 < KS / 2) rd(std::integral_constant<int, g + 1>{}, kf[(g + 1) % 2]);
        static_for<2>([&](auto Uc) {
          static_for<KB>([&](auto KBc) { s[KBc] = mfma32(kf[g % 2][Uc][KBc], qf[2 * g + Uc], s[KBc]); });
        });
      });
    };

    // V, first part: masks, tile max, and (rarely) raising the running max
    auto vmax = [&](int t, f32x16 (&s)[KB], auto MASKEDc) {
      const int kv0 = t * BC;
      if constexpr (decltype(MASKEDc)::value) {
        // key j is visible to this lane's row when lo <= j <= lim
        const int pos = wrow0 + col + Skv - Sq;
        int lim = CAUSAL ? min(Skv - 1, pos) : Skv - 1;
        int lo = 0;
        if constexpr (EXT) {
          if (a.window > 0) {
            lim = min(lim, pos + a.window - 1);
            lo = pos - a.window;
          }
        }
        // Score i of key block kb sits at key b + p_i, b = kv0 + 32*kb + 4*hi,
        // p_i = 8*(i>>2) + (i&3) <= 27. One bit mask per block marks the
        // visible offsets lo-b .. lim-b; each score then costs a sign-extended
        // one-bit extract and a bitfield select against -inf.
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int b = kv0 + kb * 32 + 4 * hi;
          const int up = min(max(lim - b, -1), 30) + 1;
          const int dn = min(max(lo - b, 0), 31);
          const uint32_t vis = ((1u << up) - 1u) & (~0u << dn);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const uint32_t keep = (uint32_t)__builtin_amdgcn_sbfe((int)vis, 8 * (i >> 2) + (i & 3), 1);
            s[kb][i] = __uint_as_float((__float_as_uint(s[kb][i]) & keep) | (~keep & 0xff800000u));
          }
        }
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
    };
    // V, second part: exponentials, row sums, P^T in bf16
    auto vexp = [&](const f32x16 (&s)[KB], bf16x8 (&pf)[KB][2]) {
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
    auto vphase = [&](int t, f32x16 (&s)[KB], bf16x8 (&pf)[KB][2], auto MASKEDc) {
      vmax(t, s, MASKEDc);
      vexp(s, pf);
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

    bool redo_rows = false;  // this wave's rows need the exact recompute
    if constexpr (EXT) {
      // Sliding window and/or block mask: the workgroup walks only the key
      // tiles that some of its rows can see and that the block mask keeps,
      // one tile in flight; a wave whose own rows see nothing of a tile (or
      // whose query block masks it) skips that tile's arithmetic. Every such
      // tile is masked per element (window edges, causal diagonal, tail).
      const int W = a.window;
      const int off = Skv - Sq;
      const int last_row = min(q0 + BR, Sq) - 1;
      int lo = 0, hi = Skv;
      if (CAUSAL) hi = min(hi, last_row + off + 1);
      if (W > 0) {
        lo = max(0, q0 + off - W);
        hi = min(hi, last_row + off + W);
      }
      const int t_first = lo / BC;
      const int t_end = hi > lo ? (hi + BC - 1) / BC : t_first;
      const int wlast = min(wrow0 + 31, Sq - 1);
      int wlo = 0, whi = Skv;
      if (CAUSAL) whi = min(whi, wlast + off + 1);
      if (W > 0) {
        wlo = max(0, wrow0 + off - W);
        whi = min(whi, wlast + off + W);
      }
      const bool wave_rows = wrow0 < Sq;
      const uint8_t* mrow = a.bmask ? a.bmask + (size_t)bh * a.nqb * a.nkb : nullptr;
      const int qb_first = q0 / kMaskBlock, qb_last = last_row / kMaskBlock, qb_w = wrow0 / kMaskBlock;
      auto active = [&](int t) {
        if (!mrow) return true;
        int any = 0;
        for (int qb = qb_first; qb <= qb_last; ++qb) any |= mrow[qb * a.nkb + t * BC / kMaskBlock];
        return any != 0;
      };
      auto next_active = [&](int t) {
        do { ++t; } while (t < t_end && !active(t));
        return t;
      };
      f32x16 sx[KB];
      int cur = t_first;
      if (cur < t_end && !active(cur)) cur = next_active(cur);
      if (cur < t_end) {
        issue(cur, std::integral_constant<int, 0>{});
        if constexpr (QSTAGE) load_q_staged();
      }
      for (int cnt = 0; cur < t_end; ++cnt) {
        // mask bytes are read before the next refill is issued, so waiting for
        // them never waits for that refill
        const int nxt = next_active(cur);
        const bool wact = wave_rows && cur * BC < whi && (cur + 1) * BC > wlo &&
                          (!mrow || mrow[qb_w * a.nkb + cur * BC / kMaskBlock] != 0);
        const int st = cnt % NSTAGE;
        static_for<NSTAGE>([&](auto STc) {
          constexpr int ST = decltype(STc)::value;
          if (st != ST) return;
          wait_vmcnt<0>();
          wait_lgkmcnt0();
          barrier();
          if (nxt < t_end) issue(nxt, std::integral_constant<int, (ST + 1) % NSTAGE>{});
          if (wact) {
            bf16x8 pf[KB][2];
            m1(STc, sx);
            vphase(cur, sx, pf, std::true_type{});
            m2(STc, pf);
          }
        });
        cur = nxt;
      }
    } else {
      // Every wave runs one tile behind itself: after barrier t it forms the
      // scores of tile t (MFMA) while it exponentiates those of tile t-1 (VALU),
      // then accumulates P*V of tile t-1, and the refill of tile t+PF is in
      // flight. The scores alternate between two register sets; the loop is
      // unrolled over UN tiles (a multiple of both the stage count and 2) so
      // every stage offset and register set is a compile-time constant. The
      // refill issued at barrier t targets stage (t+PF) % NSTAGE, last read by
      // P*V of tile t-2 before that barrier.
      //
      // These steps take the running max from tile 0 only and exponentiate the
      // later tiles against it without forming their tile maxima: the same
      // softmax as long as nothing overflows (a later score would have to
      // exceed the reference by about 2^7 base-2 units). The epilogue checks
      // l and O for that and, if needed, runs the item again with the exact
      // step (tile max, threshold raise, O rescale) on every tile.
      f32x16 sb[2][KB];
      f32x16 (&s_cur)[KB] = sb[0];
      const int t_main = first_masked_tile();
      if (t_main > 0) {
        wait_tile(0);
        wait_lgkmcnt0();
        barrier();
        if constexpr (SKV) {
          if (1 < nt) issue_kv(1, std::integral_constant<int, 1>{}, OnlyK{});
          issue_kv(0, std::integral_constant<int, 0>{}, OnlyV{});
        } else if (PF < nt) {
          issue(PF, std::integral_constant<int, PF % NSTAGE>{});
        }
        m1(std::integral_constant<int, 0>{}, sb[0]);
        // the reference: tile 0's max (no key of a pipelined tile is masked,
        // so it is finite for every row)
        vmax(0, sb[0], std::false_type{});
        for (int t0 = 0; t0 + 1 < t_main; t0 += UN) {
          static_for<UN>([&](auto Uc) {
            constexpr int U = decltype(Uc)::value + 1;          // tile t0 + U
            constexpr int ST = U % NSTAGE, SP = (U - 1) % NSTAGE;
            constexpr int BN = U % 2, BP = (U - 1) % 2;
            const int t = t0 + U;
            if (t >= t_main) return;  // the last pass may end early
            wait_tile(t);
            wait_lgkmcnt0();
            barrier();
            if constexpr (SKV) {
              if (t + 1 < nt) issue_kv(t + 1, std::integral_constant<int, (ST + 1) % NSTAGE>{}, OnlyK{});
              issue_kv(t, std::integral_constant<int, ST>{}, OnlyV{});
            } else if (t + PF < nt) {
              issue(t + PF, std::integral_constant<int, (ST + PF) % NSTAGE>{});
            }
            bf16x8 pf[KB][2];
            vexp(sb[BP], pf);
            m1(std::integral_constant<int, ST>{}, sb[BN]);
            m2(std::integral_constant<int, SP>{}, pf);
            // MFMAs of the scores alternate with the exponentials' VALU work,
            // each group of K-fragment reads one step ahead; then P*V.
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * 2 * KB, 0);
            static_for<KS * KB>([&](auto Ic) {
              constexpr int i = decltype(Ic)::value;
              constexpr int ahead = 2 * 2 * KB;  // reads issued before MFMA i
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, TATTN_VALU_PER_MFMA, 0);
              if constexpr (i % (2 * KB) == 2 * KB - 1 && i + 1 + ahead <= KS * KB)
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * KB, 0);
            });
            static_for<KB * 2>([&](auto) {
              __builtin_amdgcn_sched_group_barrier(0x100, 2 * DB, 0);
              __builtin_amdgcn_sched_group_barrier(0x008, DB, 0);
            });
          });
        }
        if constexpr (SKV) {
          // V of tile t_main - 1 was issued at that tile's barrier; from here
          // on K and V of a tile are loaded together, so V of tile t_main
          // follows now
          wait_vmcnt<0>();
          wait_lgkmcnt0();
          barrier();
          if (t_main < nt) {
            if (t_main % 2 == 0) issue_kv(t_main, std::integral_constant<int, 0>{}, OnlyV{});
            else issue_kv(t_main, std::integral_constant<int, 1>{}, OnlyV{});
          }
        }
        // tile t_main - 1 still needs its softmax and P*V; its stage and
        // score set follow from its position in the unrolled pass
        const int r_last = (t_main - 1) % UN;
        static_for<UN>([&](auto Rc) {
          constexpr int R = decltype(Rc)::value;
          if (r_last != R) return;
          bf16x8 pf[KB][2];
          vphase(t_main - 1, sb[R % 2], pf, std::false_type{});
          m2(std::integral_constant<int, R % NSTAGE>{}, pf);
        });
      }

      // the remaining tiles (causal diagonal, ragged tail) run masked, in order
      auto tile_step = [&](int tt, auto STc) {
        constexpr int ST = decltype(STc)::value;
        wait_tile(tt);
        wait_lgkmcnt0();
        barrier();
        if (tt + PF < nt) issue(tt + PF, std::integral_constant<int, (ST + PF) % NSTAGE>{});
        if (CAUSAL && tt * BC > wave_kv_last) return;
        bf16x8 pf[KB][2];
        m1(STc, s_cur);
        vphase(tt, s_cur, pf, std::true_type{});
        m2(STc, pf);
      };
      for (int t = t_main; t < nt; ++t) {
        const int st = t % NSTAGE;
        static_for<NSTAGE>([&](auto STc) {
          if (st == decltype(STc)::value) tile_step(t, STc);
        });
      }

      // Overflow check of the first run: l of this lane below 2^100 and every
      // O accumulator finite (x*0 is NaN for x = inf or NaN). A wave that
      // fails it writes its rows once more after the epilogue, exactly.
      {
        float fin = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) fin = fmaf(oacc[db][i], 0.f, fin);
        redo_rows = __builtin_amdgcn_ballot_w64(!(lsum <= 0x1p100f) || !(fin == 0.f)) != 0;
      }
    }

    // ---- epilogue: O = acc / l (bf16), LSE = (m + log2 l) * ln 2. The
    // wave's 32 rows go through LDS (the ring is free once every wave has
    // passed the barrier below) so each store writes whole, contiguous rows.
    {
      const float l = sum_halves(lsum);
      const int row = wrow0 + col;
      const float inv = l > 0.f ? 1.f / l : 0.f;
      constexpr int SRS = RS + 16;  // staging row stride (padded)
      static_assert(NW * 32 * SRS <= 2 * NSTAGE * TILE, "staging fits the ring");
      typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
      typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
      // (addresses from an opaque copy of the lane id, so the compiler does
      // not compute them before the tile loop and hold them across it)
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const uint32_t stg = lds_addr(smem) + wave * 32 * SRS;
      const uint32_t wr = stg + (ln & 31) * SRS + 8 * (ln >> 5);
      barrier();
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + 8 * g4;
          *(lds_u32x2*)(uintptr_t)(wr + d * 2) =
              u32x2{pack_bf16x2(oacc[db][g4 * 4 + 0] * inv, oacc[db][g4 * 4 + 1] * inv),
                    pack_bf16x2(oacc[db][g4 * 4 + 2] * inv, oacc[db][g4 * 4 + 3] * inv)};
        }
      // each store: 64 lanes x 16 bytes = 64 / CPR whole rows
      constexpr int RPS = 64 / CPR;
      const int rsub = ln / CPR, csub = ln % CPR;
#pragma unroll
      for (int r0 = 0; r0 < 32; r0 += RPS) {
        const int rr = r0 + rsub;
        const u32x4 v = *(const lds_u32x4*)(uintptr_t)(stg + rr * SRS + 16 * csub);
        // streaming stores: the output is not read again by this kernel
        if (wrow0 + rr < Sq)
          __builtin_nontemporal_store(v, (u32x4*)(a.o + ((size_t)bh * Sq + wrow0 + rr) * D + 8 * csub));
      }
      if (row < Sq && hi == 0) a.lse[(size_t)bh * Sq + row] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
    }

    // ---- exact recompute of this wave's 32 rows, for a wave whose check
    // failed: fp32 online softmax with the exact running max, K and V read
    // straight from global memory, 8 lanes per row (lane r of a row owns the
    // 16-byte chunks r, r + 8, ...), 8 rows at a time; the results replace
    // what the epilogue wrote. Slow, and only taken when a later score
    // exceeds tile 0's max by about 2^7 base-2 units.
    if (redo_rows) {
      wait_vmcnt<0>();  // the epilogue's stores of these rows come first
      constexpr int CL = CPR / 8;  // chunks per lane
      const int sub = lane & 7;
      for (int pass = 0; pass < 4; ++pass) {
        const int r = wrow0 + 8 * pass + (lane >> 3);
        const int rc = min(r, Sq - 1);
        const int lim = CAUSAL ? min(Skv - 1, rc + Skv - Sq) : Skv - 1;
        int lim_w = lim;  // the pass's last key: the largest limit of its rows
#pragma unroll
        for (int off = 8; off < 64; off <<= 1) lim_w = max(lim_w, __shfl_xor(lim_w, off));
        float qv[CL][8], ov[CL][8];
#pragma unroll
        for (int ci = 0; ci < CL; ++ci) {
          const u32x4 w = *(const u32x4*)(qp + (size_t)rc * D + 8 * (sub + 8 * ci));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            qv[ci][2 * e] = __uint_as_float(w[e] << 16);
            qv[ci][2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
            ov[ci][2 * e] = ov[ci][2 * e + 1] = 0.f;
          }
        }
        float mr = -INFINITY, lr = 0.f;
        for (int j = 0; j <= lim_w; ++j) {
          const uint16_t* kr = (const uint16_t*)kp + (size_t)j * D;
          const uint16_t* vr = (const uint16_t*)vp + (size_t)j * D;
          float dot = 0.f;
#pragma unroll
          for (int ci = 0; ci < CL; ++ci) {
            const u32x4 w = *(const u32x4*)(kr + 8 * (sub + 8 * ci));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              dot = fmaf(qv[ci][2 * e], __uint_as_float(w[e] << 16), dot);
              dot = fmaf(qv[ci][2 * e + 1], __uint_as_float(w[e] & 0xffff0000u), dot);
            }
          }
          dot = octet_sum(dot);
          if (j > lim) continue;
          const float sc = dot * c;
          if (sc > mr) {
            const float alpha = fast_exp2(mr - sc);  // 0 for mr = -inf
            lr *= alpha;
#pragma unroll
            for (int ci = 0; ci < CL; ++ci)
#pragma unroll
              for (int e = 0; e < 8; ++e) ov[ci][e] *= alpha;
            mr = sc;
          }
          const float p = fast_exp2(sc - mr);
          lr += p;
#pragma unroll
          for (int ci = 0; ci < CL; ++ci) {
            const u32x4 w = *(const u32x4*)(vr + 8 * (sub + 8 * ci));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              ov[ci][2 * e] = fmaf(p, __uint_as_float(w[e] << 16), ov[ci][2 * e]);
              ov[ci][2 * e + 1] = fmaf(p, __uint_as_float(w[e] & 0xffff0000u), ov[ci][2 * e + 1]);
            }
          }
        }
        if (r < Sq) {
          const float inv = lr > 0.f ? 1.f / lr : 0.f;
#pragma unroll
          for (int ci = 0; ci < CL; ++ci) {
            const u32x4 w = {pack_bf16x2(ov[ci][0] * inv, ov[ci][1] * inv), pack_bf16x2(ov[ci][2] * inv, ov[ci][3] * inv),
                             pack_bf16x2(ov[ci][4] * inv, ov[ci][5] * inv), pack_bf16x2(ov[ci][6] * inv, ov[ci][7] * inv)};
            *(u32x4*)(a.o + ((size_t)bh * Sq + r) * D + 8 * (sub + 8 * ci)) = w;
          }
          if (sub == 0) a.lse[(size_t)bh * Sq + r] = lr > 0.f ? (mr + __log2f(lr)) * kLn2 : -INFINITY;
        }
      }
    }
  };

  // Items of XCD x are x + 8*local (local < L); workgroup w (XCD w % 8, the
  // j-th of J there) takes local j, 2J-1-j, 2J+j, ... so that consecutive
  // passes pair long causal tiles with short ones. Without the XCD order,
  // workgroup w takes items w, w + G, ...
  const int G = gridDim.x;
  const int xq = blockIdx.x & 7, jq = blockIdx.x >> 3, J = G >> 3, L = a.n_items >> 3;
  for (int k = 0;; ++k) {
    int item = -1;
    if (a.remap) {
      if (k * J >= L) break;
      const int local = (k & 1) ? (k + 1) * J - 1 - jq : k * J + jq;
      if (local < L) item = xq + 8 * local;
    } else {
      item = blockIdx.x + k * G;
      if (item >= a.n_items) break;
    }
    if (item >= 0) process(item);
    // every wave is done with the LDS ring before the next item refills it
    wait_lgkmcnt0();
    barrier();
  }
}

template <int D, int NW, int BC, bool CAUSAL, bool EXT>
static hipError_t launch_one(const MhaArgs& a, int n_cu, hipStream_t stream) {
  constexpr int BR = NW * 32;
  constexpr int NSTAGE = (!EXT && NW == 4) ? 2 : TATTN_MHA_STAGES;
  // the K and V rings
  constexpr size_t lds = 2 * (size_t)NSTAGE * BC * D * 2;
  static_assert(lds <= 160 * 1024, "LDS budget");
  auto kern = mha_fwd_bf16_kernel<D, NW, BC, NSTAGE, CAUSAL, EXT>;
  // Thread-safe one-time opt-in to more than the default dynamic LDS.
  static const hipError_t attr_err =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr_err != hipSuccess) return attr_err;
  MhaArgs b = a;
  b.n_qtiles = (a.Sq + BR - 1) / BR;
  const long long items = (long long)b.n_qtiles * a.n_bh;
  if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  b.n_items = (int)items;
  b.remap = (a.n_bh % 8) == 0 && n_cu >= 8;
  // as many workgroups per compute unit as LDS and the waves per SIMD allow
  // (one for 8-wave workgroups); a multiple of 8 for the XCD order
  constexpr int WG_REG = 4 * kWavesPerSimd<D, NW, EXT> / NW;
  constexpr int OCC = (int)(160 * 1024 / lds) < WG_REG ? (int)(160 * 1024 / lds) : WG_REG;
  static_assert(OCC >= 1, "one workgroup must fit");
  const long long slots = (long long)n_cu * OCC;
  long long grid = items < slots ? items : slots;
  if (b.remap) grid = (grid / 8) * 8;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NW * 64), lds, stream, b);
  return hipGetLastError();
}

hipError_t launch_mha_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int Hkv, int Sq, int Skv, int D, bool causal, int window,
                               const uint8_t* block_mask, float scale, int n_cu, int dense_waves,
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
  a.H = H;
  a.group = H / Hkv;
  a.window = window;
  a.bmask = block_mask;
  a.nqb = (Sq + kMaskBlock - 1) / kMaskBlock;
  a.nkb = (Skv + kMaskBlock - 1) / kMaskBlock;
  const bool ext = window > 0 || block_mask != nullptr;
  // Windows and block masks run on 4-wave workgroups of 128 rows (two 64-row
  // mask blocks) with 32-key tiles, three or four per compute unit, so one
  // workgroup's loads, item start and output stores overlap the others'
  // arithmetic, and a mask block's kept tiles are walked with fewer idle
  // waves than a 256-row workgroup's four blocks would leave.
  if (ext) {
    static_assert(kMaskBlock % 32 == 0, "mask blocks hold whole 32-key tiles");
    if (D == 128) return causal ? launch_one<128, 4, 32, true, true>(a, n_cu, stream) : launch_one<128, 4, 32, false, true>(a, n_cu, stream);
    return causal ? launch_one<64, 4, 32, true, true>(a, n_cu, stream) : launch_one<64, 4, 32, false, true>(a, n_cu, stream);
  }
  // Dense: 8-wave workgroups of 256 rows, one per CU. When the launch has
  // fewer 256-row items than CUs, 4-wave workgroups of 128 rows (two per CU)
  // instead: causally, half-height items halve the longest item; without a
  // mask only when at most half the CUs would be busy (each 4-wave workgroup
  // then has its CU to itself; two sharing one are ~16 % slower per row).
  const long long items8 = (long long)a.n_bh * ((Sq + 255) / 256);
  bool four = causal ? items8 < n_cu : 2 * items8 <= n_cu;
  if (dense_waves == 4 || dense_waves == 8) four = dense_waves == 4;
  if (four) {
    if (D == 128) return causal ? launch_one<128, 4, 64, true, false>(a, n_cu, stream) : launch_one<128, 4, 64, false, false>(a, n_cu, stream);
    return causal ? launch_one<64, 4, 64, true, false>(a, n_cu, stream) : launch_one<64, 4, 64, false, false>(a, n_cu, stream);
  }
  if (D == 128) return causal ? launch_one<128, 8, 64, true, false>(a, n_cu, stream) : launch_one<128, 8, 64, false, false>(a, n_cu, stream);
  return causal ? launch_one<64, 8, 64, true, false>(a, n_cu, stream) : launch_one<64, 8, 64, false, false>(a, n_cu, stream);
}

}  // namespace tattn
