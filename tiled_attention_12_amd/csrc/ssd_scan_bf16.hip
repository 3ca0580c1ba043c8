// Mamba-2 state-space scan (chunk state + state passing + chunk scan in one
// pass), bf16 inputs and output, fp32 state and accumulation, gfx950.
//
// Method: the chunked form of Mamba-2's scalar-decay state-space layer, the
// linear-attention workload of "TileLang paper summary" (appendix A.4: the
// chunk-scan and chunk-state functions), walked in tiles of 64 steps as the
// Mamba scan sketch of "From FlashAttention to general kernels" (section 4)
// does. Per (batch b, head h), with Acs the running sum of dt*A inside a
// chunk:
//   y_t   = exp(Acs_t) * prev . C_t + sum_{s<=t} (C_t . B_s) exp(Acs_t - Acs_s) dt_s x_s
//   state = exp(Acs_last) * prev + sum_s exp(Acs_last - Acs_s) dt_s x_s (outer) B_s
// where prev is the state entering the chunk.
//
// gfx950 mapping:
//  * One workgroup walks all chunks of two heads of one batch that share a
//    B/C group (two teams of 4 waves; one team when heads per group is odd).
//    The state of each head stays in its team's MFMA accumulators for the
//    whole sequence, so HBM sees x, dt, B, C once and y once: no chunk states
//    or carried states ever leave the chip.
//  * Everything is transposed so each MFMA result feeds the next one without
//    a register shuffle: G^T = B * C^T (scores of step t against step s),
//    y^T = prev * C^T + x^T * G^T, state^T += (B^T scaled) * x, all on
//    v_mfma_f32_32x32x16_bf16. x^T and B^T operands come from the row-major
//    LDS tiles through ds_read_b64_tr_b16. G and the bf16 copy of the state
//    pass between the waves of a team through LDS.
//  * x, B, C (16-byte rows pieces) and dt move HBM -> LDS with
//    global_load_lds into a two-stage ring (XOR-swizzled rows); the loads of
//    chunk c+1 are in flight while chunk c computes. Two barriers per chunk.
//  * The heads of one batch go to one XCD (workgroup i runs on XCD i % 8), so
//    B and C, shared by every head of a group, are fetched from HBM once per
//    XCD and then hit in its L2.
#include "device_common.h"
#include "launch.h"

namespace tattn {

struct SsdArgs {
  const uint16_t* x;
  const float* dt;
  const float* A;
  const uint16_t* B;
  const uint16_t* C;
  uint16_t* y;
  const float* init_state;
  float* final_state;
  int Bt, L, H, G;
  int n_items;
  int remap;
};

namespace {

constexpr int kQ = 64;   // chunk length
constexpr int kP = 64;   // head dimension
constexpr int kN = 128;  // state dimension

// LDS layout: two stages of [B | C | x per team | dt per team], then per team
// the bf16 state [p][n] and G [t][s], then per-wave scratch floats.
template <int TEAMS>
struct SsdLds {
  static constexpr int BOFF = 0;
  static constexpr int COFF = kQ * kN * 2;
  static constexpr int XOFF = 2 * kQ * kN * 2;
  static constexpr int DTOFF = XOFF + TEAMS * kQ * kP * 2;
  static constexpr int STAGE = DTOFF + TEAMS * kQ * 4;
  static constexpr int STATE = 2 * STAGE;
  static constexpr int GREG = STATE + TEAMS * kP * kN * 2;
  static constexpr int SCR = GREG + TEAMS * kQ * kQ * 2;
  static constexpr int SCR_WAVE = 3 * kQ * 4;  // acs (base-2 units), dt, coef
  static constexpr int TOTAL = SCR + 4 * TEAMS * SCR_WAVE;
  static_assert(STAGE % 16 == 0, "stage alignment for the direct loads");
};

// inclusive prefix sum over the 64 lanes (row shifts inside 16-lane rows,
// then the two row broadcasts)
__device__ __forceinline__ float wave_prefix_sum(float v) {
#define TATTN_DPP(ctrl, rmask) \
  __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, rmask, 0xf, true))
  v += TATTN_DPP(0x111, 0xf);  // row_shr:1
  v += TATTN_DPP(0x112, 0xf);  // row_shr:2
  v += TATTN_DPP(0x114, 0xf);  // row_shr:4
  v += TATTN_DPP(0x118, 0xf);  // row_shr:8
  v += TATTN_DPP(0x142, 0xa);  // row_bcast:15 into rows 1 and 3
  v += TATTN_DPP(0x143, 0xc);  // row_bcast:31 into rows 2 and 3
#undef TATTN_DPP
  return v;
}

__device__ __forceinline__ void load_lds4_asm(const void* gptr, uint32_t lds_base_uniform) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
               :: "v"(gptr), "s"(lds_base_uniform) : "memory", "m0");
}

// streaming (non-temporal) 16-byte store: y is not read again by the scan
__device__ __forceinline__ void store16_asm(void* gptr, u32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off nt" :: "v"(gptr), "v"(v) : "memory");
}

// bf16 pair * (c0, c1), rounded back to bf16
__device__ __forceinline__ uint32_t scale_bf16x2(uint32_t w, float c0, float c1) {
  const float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xffff0000u);
  return pack_bf16x2(lo * c0, hi * c1);
}

}  // namespace

template <int TEAMS>
__global__ __launch_bounds__(256 * TEAMS) void ssd_scan_bf16_kernel(SsdArgs a) {
  using Lds = SsdLds<TEAMS>;
  constexpr int NW = 4 * TEAMS;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int team = wave >> 2, tw = wave & 3;
  const int l32 = lane & 31, hh = lane >> 5;

  // item -> (batch, first head); consecutive items share one XCD
  const int item = blockIdx.x;
  const int lin = a.remap ? (item & 7) * (a.n_items >> 3) + (item >> 3) : item;
  const int hpairs = a.H / TEAMS;
  const int b = lin / hpairs;
  const int h0 = (lin - b * hpairs) * TEAMS;
  const int h = h0 + team;
  const int g = h0 / (a.H / a.G);
  const int L = a.L, H = a.H, G = a.G;
  const float a2 = a.A[h] * kLog2e;
  const int nc = (L + kQ - 1) / kQ;

  const uint32_t smem0 = lds_addr(smem);
  const uint32_t state0 = smem0 + Lds::STATE + team * (kP * kN * 2);
  const uint32_t g0 = smem0 + Lds::GREG + team * (kQ * kQ * 2);
  float* scr = (float*)(smem + Lds::SCR + wave * Lds::SCR_WAVE);
  float* sc_acs = scr;
  float* sc_dt = scr + kQ;
  float* sc_coef = scr + 2 * kQ;

  // ---- direct HBM -> LDS loads of chunk c into stage ST
  const char* xg = (const char*)a.x;
  const char* bg = (const char*)a.B;
  const char* cg = (const char*)a.C;
  auto issue = [&](int c, int ST) {
    const int t0 = c * kQ;
    const int lim = min(kQ - 1, L - 1 - t0);
    const uint32_t st = smem0 + ST * Lds::STAGE;
    const size_t rowg0 = (size_t)b * L + t0;
#pragma unroll
    for (int n = 0; n < 16 / NW; ++n) {
      const int slot = (n * NW + wave) * 64 + lane;
      const int row = slot >> 4, pc = slot & 15;
      const size_t off = ((rowg0 + min(row, lim)) * G + g) * (kN * 2) + 16 * swz<16>(row, pc);
      load_lds16_asm(bg + off, st + Lds::BOFF + (n * NW + wave) * 1024);
      load_lds16_asm(cg + off, st + Lds::COFF + (n * NW + wave) * 1024);
    }
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int slot = (n * 4 + tw) * 64 + lane;
      const int row = slot >> 3, pc = slot & 7;
      const size_t off = ((rowg0 + min(row, lim)) * H + h) * (kP * 2) + 16 * swz<8>(row, pc);
      load_lds16_asm(xg + off, st + Lds::XOFF + team * (kQ * kP * 2) + (n * 4 + tw) * 1024);
    }
    if (tw == 0) {
      const float* src = a.dt + ((rowg0 + min(lane, lim)) * H + h);
      load_lds4_asm(src, st + Lds::DTOFF + team * (kQ * 4));
    }
  };

  // ---- lane address parts
  // tr reads: lane m of its 16-lane group addresses row base + m/4, column
  // 4*(m%4) of a 16-column group; the 8 values a lane receives are k = 8*hh + 0..7
  const int m16 = lane & 15, g16 = (lane >> 4) & 1;
  uint32_t btr[2], xtr[2][2];  // [e] for B (n block = tw); [pb][e] for x
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int r = 8 * hh + 4 * e + (m16 >> 2);  // row inside a 16-row k block
    const int cb = 4 * tw + 2 * g16 + ((m16 & 3) >> 1);
    btr[e] = Lds::BOFF + r * (kN * 2) + 16 * swz<16>(r, cb) + 8 * (m16 & 1);
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      const int cx = 4 * pb + 2 * g16 + ((m16 & 3) >> 1);
      xtr[pb][e] = Lds::XOFF + team * (kQ * kP * 2) + r * (kP * 2) + 16 * swz<8>(r, cx) + 8 * (m16 & 1);
    }
  }
  // this wave's tiles: G^T (sb, tb) for tw < 3; y^T (pb, tb); state^T n block tw
  const int gsb = tw == 2 ? 1 : 0, gtb = tw == 0 ? 0 : 1;
  const int ypb = tw & 1, ytb = tw >> 1;

  // ---- state: fp32 accumulators st[pb] = state^T rows n = 32*tw + 8j + 4hh + i, column p = 32*pb + l32
  f32x16 st[2];
  const size_t sbase = ((size_t)b * H + h) * kP * kN;
#pragma unroll
  for (int pb = 0; pb < 2; ++pb) {
    if (a.init_state) {
      const float* src = a.init_state + sbase + (size_t)(32 * pb + l32) * kN + 32 * tw + 4 * hh;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 v = *(const f32x4*)(src + 8 * j);
#pragma unroll
        for (int i = 0; i < 4; ++i) st[pb][4 * j + i] = v[i];
      }
    } else {
      st[pb] = f32x16{};
    }
  }
  // bf16 copy of the state in LDS, [p][n] rows of 256 bytes
  auto write_state = [&]() {
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      const int p = 32 * pb + l32;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x2 v = {pack_bf16x2(st[pb][4 * j], st[pb][4 * j + 1]),
                         pack_bf16x2(st[pb][4 * j + 2], st[pb][4 * j + 3])};
        const uint32_t ad = state0 + p * (kN * 2) + 16 * swz<16>(p, 4 * tw + j) + 8 * hh;
        *(__attribute__((address_space(3))) u32x2*)(uintptr_t)ad = v;
      }
    }
  };
  write_state();

  if (nc > 0) issue(0, 0);

  for (int c = 0; c < nc; ++c) {
    const int ST = c & 1;
    const uint32_t stg = smem0 + ST * Lds::STAGE;
    const int t0 = c * kQ;
    // chunk c's loads have landed once only the previous chunk's (at most 2)
    // y stores may still be in flight (vector memory operations complete in
    // order)
    if (c == 0) wait_vmcnt<0>(); else wait_vmcnt<2>();
    wait_lgkmcnt0();
    barrier();
    if (c + 1 < nc) issue(c + 1, ST ^ 1);

    // ---- phase 1: running sum of dt*A (base-2 units) over the chunk
    float dtv = *(const float*)(smem + ST * Lds::STAGE + Lds::DTOFF + team * (kQ * 4) + 4 * lane);
    if (t0 + lane >= L) dtv = 0.f;
    const float acs = wave_prefix_sum(dtv * a2);
    const float last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acs), 63));
    sc_acs[lane] = acs;
    sc_dt[lane] = dtv;
    sc_coef[lane] = fast_exp2(last - acs) * dtv;

    // ---- phase 2: G^T tile (gsb, gtb) = (B C^T) * decay * dt_s, causal, -> LDS G[t][s]
    if (tw < 3) {
      f32x16 acc = f32x16{};
      const int s = 32 * gsb + l32, t = 32 * gtb + l32;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const bf16x8 af = as_bf16x8(lds_read128((const void*)(uintptr_t)(
            stg + Lds::BOFF + s * (kN * 2) + 16 * swz<16>(s, 2 * kb + hh))));
        const bf16x8 bfr = as_bf16x8(lds_read128((const void*)(uintptr_t)(
            stg + Lds::COFF + t * (kN * 2) + 16 * swz<16>(t, 2 * kb + hh))));
        acc = mfma32(af, bfr, acc);
      }
      const float acs_t = sc_acs[t];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int s0 = 32 * gsb + 8 * j + 4 * hh;
        const f32x4 as4 = *(const f32x4*)(sc_acs + s0);
        const f32x4 ds4 = *(const f32x4*)(sc_dt + s0);
        float gv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float d = fminf(acs_t - as4[i], 0.f);
          gv[i] = (s0 + i <= t) ? acc[4 * j + i] * fast_exp2(d) * ds4[i] : 0.f;
        }
        const u32x2 v = {pack_bf16x2(gv[0], gv[1]), pack_bf16x2(gv[2], gv[3])};
        const uint32_t ad = g0 + t * (kQ * 2) + 16 * swz<8>(t, 4 * gsb + j) + 8 * hh;
        *(__attribute__((address_space(3))) u32x2*)(uintptr_t)ad = v;
      }
    }

    // ---- phase 3: y^T tile (ypb, ytb) = exp(Acs_t) * prev C^T
    f32x16 yacc = f32x16{};
    {
      const int p = 32 * ypb + l32, t = 32 * ytb + l32;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const bf16x8 af = as_bf16x8(lds_read128((const void*)(uintptr_t)(
            state0 + p * (kN * 2) + 16 * swz<16>(p, 2 * kb + hh))));
        const bf16x8 bfr = as_bf16x8(lds_read128((const void*)(uintptr_t)(
            stg + Lds::COFF + t * (kN * 2) + 16 * swz<16>(t, 2 * kb + hh))));
        yacc = mfma32(af, bfr, yacc);
      }
      const float sc = fast_exp2(sc_acs[t]);
#pragma unroll
      for (int i = 0; i < 16; ++i) yacc[i] *= sc;
    }

    // ---- phase 4: state^T = exp(Acs_last) state^T + (B^T * coef) x
    bf16x8 xf[2][4];
    {
      const float dec = fast_exp2(last);
#pragma unroll
      for (int pb = 0; pb < 2; ++pb)
#pragma unroll
        for (int i = 0; i < 16; ++i) st[pb][i] *= dec;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const uint32_t kofs = kb * 16;  // 16 rows per k block
        u32x2 w0 = lds_read_tr16<0>(stg + btr[0] + kofs * (kN * 2));
        u32x2 w1 = lds_read_tr16<0>(stg + btr[1] + kofs * (kN * 2));
#pragma unroll
        for (int pb = 0; pb < 2; ++pb) {
          const u32x2 x0 = lds_read_tr16<0>(stg + xtr[pb][0] + kofs * (kP * 2));
          const u32x2 x1 = lds_read_tr16<0>(stg + xtr[pb][1] + kofs * (kP * 2));
          xf[pb][kb] = cat_tr(x0, x1);
        }
        const f32x4 c0 = *(const f32x4*)(sc_coef + 16 * kb + 8 * hh);
        const f32x4 c1 = *(const f32x4*)(sc_coef + 16 * kb + 8 * hh + 4);
        w0[0] = scale_bf16x2(w0[0], c0[0], c0[1]);
        w0[1] = scale_bf16x2(w0[1], c0[2], c0[3]);
        w1[0] = scale_bf16x2(w1[0], c1[0], c1[1]);
        w1[1] = scale_bf16x2(w1[1], c1[2], c1[3]);
        const bf16x8 wf = cat_tr(w0, w1);
#pragma unroll
        for (int pb = 0; pb < 2; ++pb) st[pb] = mfma32(wf, xf[pb][kb], st[pb]);
      }
    }

    wait_lgkmcnt0();
    barrier();

    // ---- phase 5: y^T += x^T G^T, store y; then the new state's bf16 copy
    {
      const int t = 32 * ytb + l32;
      // (the x fragment index stays a compile-time constant)
      auto pv = [&](auto PBc) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          if (kb >= 2 && ytb == 0) break;
          const bf16x8 gf = as_bf16x8(lds_read128((const void*)(uintptr_t)(
              g0 + t * (kQ * 2) + 16 * swz<8>(t, 2 * kb + hh))));
          yacc = mfma32(xf[decltype(PBc)::value][kb], gf, yacc);
        }
      };
      if (ypb) pv(std::integral_constant<int, 1>{}); else pv(std::integral_constant<int, 0>{});
      // The wave's 32x32 block of y goes through the team's x tile of this
      // stage (no wave reads it after the barrier that follows the state
      // update; the next loads into this stage wait for the barrier at the
      // top of the next chunk), rows [t][p] with 16-byte chunk c of row t at
      // position c ^ (t & 7); each store then writes 64-byte row pieces. A
      // wave reads back only its own block, so no barrier is needed here.
      typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
      typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
      const uint32_t ys = stg + Lds::XOFF + team * (kQ * kP * 2);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int cch = 4 * ypb + j;
        *(lds_u32x2*)(uintptr_t)(ys + t * (kP * 2) + 16 * (cch ^ (t & 7)) + 8 * hh) =
            u32x2{pack_bf16x2(yacc[4 * j], yacc[4 * j + 1]), pack_bf16x2(yacc[4 * j + 2], yacc[4 * j + 3])};
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int tr = 32 * ytb + 16 * k + (lane >> 2);
        const int cc = 4 * ypb + (lane & 3);
        const u32x4 v = *(const lds_u32x4*)(uintptr_t)(ys + tr * (kP * 2) + 16 * (cc ^ (tr & 7)));
        if (t0 + tr < L)
          store16_asm((char*)a.y + (((size_t)b * L + t0 + tr) * H + h) * (kP * 2) + 16 * cc, v);
      }
    }
    write_state();
  }

  if (a.final_state) {
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      float* dst = a.final_state + sbase + (size_t)(32 * pb + l32) * kN + 32 * tw + 4 * hh;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 v = {st[pb][4 * j], st[pb][4 * j + 1], st[pb][4 * j + 2], st[pb][4 * j + 3]};
        *(f32x4*)(dst + 8 * j) = v;
      }
    }
  }
}

template <int TEAMS>
static hipError_t launch_ssd(const SsdArgs& a0, hipStream_t stream) {
  constexpr int lds = SsdLds<TEAMS>::TOTAL;
  static_assert(lds <= 160 * 1024, "LDS budget");
  auto kern = ssd_scan_bf16_kernel<TEAMS>;
  static const hipError_t attr_err =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr_err != hipSuccess) return attr_err;
  SsdArgs a = a0;
  const long long items = (long long)a.Bt * (a.H / TEAMS);
  if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  a.n_items = (int)items;
  a.remap = (a.n_items % 8) == 0;
  hipLaunchKernelGGL(kern, dim3((unsigned)a.n_items), dim3(256 * TEAMS), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_ssd_scan_bf16(const void* x, const float* dt, const float* A, const void* B, const void* C,
                                void* y, const float* init_state, float* final_state, int Bt, int L, int H,
                                int G, hipStream_t stream) {
  if (Bt == 0 || H == 0) return hipSuccess;
  SsdArgs a;
  a.x = (const uint16_t*)x;
  a.dt = dt;
  a.A = A;
  a.B = (const uint16_t*)B;
  a.C = (const uint16_t*)C;
  a.y = (uint16_t*)y;
  a.init_state = init_state;
  a.final_state = final_state;
  a.Bt = Bt;
  a.L = L;
  a.H = H;
  a.G = G;
  a.n_items = 0;
  a.remap = 0;
  if (L == 0 && !final_state) return hipSuccess;
  return ((H / G) % 2 == 0) ? launch_ssd<2>(a, stream) : launch_ssd<1>(a, stream);
}

}  // namespace tattn
