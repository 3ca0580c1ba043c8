// MLA decode forward (one query position per batch), bf16 in, fp32 accumulate.
//
// Method: the FlashMLA decode kernel of "TileLang programming model and
// FlashMLA" -- the query heads of a batch share one KV head; each KV tile is
// staged in fast memory once, scores are the sum of the latent product
// (Q * KV^T) and the rotary product (Q_pe * K_pe^T) (section 2.2), the
// softmax is max-subtracted base-2 with the scale folded in and a running
// log-sum (section 3.1), and the tile loop is software pipelined (section
// 2.2). The values are the latent rows themselves, so one LDS tile serves
// as both keys and values.
//
// Three kernels:
//  1. plan:    tile_ptr[b] = number of 32-key tiles in batches before b (a
//              separate launch for many batches; below kFusedPlanMax batches
//              every split workgroup forms it in LDS and workgroup 0 writes it
//              out for the merge).
//  2. split:   one persistent workgroup per compute unit takes an equal,
//              contiguous slice of the packed tile range (a slice may span
//              batches) and, for each batch it touches, writes the
//              normalised partial output O_s (bf16) and its log-sum-exp lse_s
//              (fp32) into slot (slice + batch), which is unique per piece.
//  3. combine: for every (batch, head), lse = ln sum_s exp(lse_s) and
//              O = sum_s exp(lse_s - lse) * O_s, rounded to bf16. This merge
//              is exact: each O_s is normalised by its own exp(lse_s).
//  Slices are numbered so that consecutive slices run on the same XCD (the
//  hardware hands workgroup i to XCD i % 8): the pieces of one batch then
//  share that XCD's L2 for Q.
//
// gfx950 mapping of the split kernel: 4 waves x 32 heads (H = 128), one wave
// per SIMD; wave w holds Q^T of its heads in registers (B operand, 36
// k-steps of 16) and the O^T accumulator (16 blocks of 32 latent columns) in
// the accumulation registers, which it fills. Per 32-key tile:
// S^T = KV * Q^T + K_pe * Q_pe^T with the tile read from LDS as the A operand
// (v_mfma_f32_32x32x16_bf16, the score accumulator pinned to ordinary
// VGPRs), the online softmax in lane-per-head form, and O^T += KV^T * P^T
// with KV^T read by ds_read_b64_tr_b16 from the same tile. The tile loop is
// software pipelined: step i scores tile i and runs its softmax, then
// accumulates P*V of tile i-1. Tiles arrive by global_load_lds_dwordx4
// through a 4-stage LDS ring with two tiles in flight; latent rows are
// padded in LDS so both read patterns are conflict-free with one base
// register each.
#include <mutex>

#include "device_common.h"
#include "launch.h"

namespace tattn {

constexpr int kDl = 512;     // latent width
constexpr int kDr = 64;      // rotary width
constexpr int kBK = 32;      // keys per tile
constexpr int kRowL = kDl * 2 + 48;   // latent row stride in LDS (1 KB + 48 B of padding)
constexpr int kTileL = kBK * kRowL;
constexpr int kTileR = kBK * kDr * 2;
constexpr int kStage = kTileL + kTileR;
// Up to this many batches the split kernel forms the tile prefix itself (in
// LDS beside the ring) instead of a separate plan launch.
constexpr int kFusedPlanMax = 1024;

struct MlaArgs {
  const uint16_t* q;
  const uint16_t* qpe;
  const uint16_t* kv;
  const uint16_t* kpe;
  uint16_t* o;
  float* lse;
  const int32_t* indptr;
  int B, H;
  float c;          // scale * log2(e)
  int* tile_ptr;    // [B + 1]
  float* part_lse;     // [(P + B) * H]
  uint16_t* part_o;    // [(P + B) * H * 512] bf16
};

// Slice index of physical workgroup w: consecutive slices on one XCD.
__device__ __forceinline__ int slice_of(int w, int P) {
  return (P & 7) ? w : (w & 7) * (P >> 3) + (w >> 3);
}

__device__ __forceinline__ int batch_tiles(const int32_t* indptr, int b) {
  const int len = indptr[b + 1] - indptr[b];
  return len > 0 ? (len + kBK - 1) / kBK : 0;
}

// Workgroup w of P takes global tiles [start(w), start(w + 1)).
__device__ __forceinline__ int split_start(int w, int T, int P) {
  return (int)(((long long)w * T) / P);
}

// The workgroup whose slice holds global tile g (0 <= g < T): the largest w
// with floor(w*T/P) <= g, i.e. w*T < (g+1)*P, i.e. ceil((g+1)*P/T) - 1.
__device__ __forceinline__ int split_owner(int g, int T, int P) {
  return (int)((((long long)g + 1) * P - 1) / T);
}

__global__ __launch_bounds__(1024) void mla_plan_kernel(MlaArgs a) {
  __shared__ int sums[1024];
  const int B = a.B;
  const int t = threadIdx.x;
  const int per = (B + 1023) / 1024;
  const int b0 = min(B, t * per), b1 = min(B, b0 + per);
  int local = 0;
  for (int b = b0; b < b1; ++b) local += batch_tiles(a.indptr, b);
  sums[t] = local;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = t >= off ? sums[t - off] : 0;
    __syncthreads();
    sums[t] += add;
    __syncthreads();
  }
  int run = t > 0 ? sums[t - 1] : 0;
  for (int b = b0; b < b1; ++b) {
    a.tile_ptr[b] = run;
    run += batch_tiles(a.indptr, b);
  }
  if (t == 1023) a.tile_ptr[B] = sums[1023];
}

// Combine: one workgroup of 256 threads per (batch, 8 heads); thread t owns
// head 8*blockIdx.y + t/32 and latent columns 16*(t%32) .. +15. Pieces of
// empty slices between the two owners wrote nothing and are skipped. The
// merge keeps a running maximum of the pieces' log-sum-exps, so the loads of
// up to four pieces are issued together.
__global__ __launch_bounds__(256) void mla_combine_kernel(MlaArgs a, int P) {
  constexpr int MP = 4;
  const int b = blockIdx.x;
  const int H = a.H;
  const int h = blockIdx.y * 8 + (threadIdx.x >> 5);
  const int c0 = 16 * (threadIdx.x & 31);
  const int T = a.tile_ptr[a.B];
  const int g0 = a.tile_ptr[b], g1 = a.tile_ptr[b + 1];
  if (h >= H) return;
  if (g0 >= g1) {  // a batch without keys: O = 0, LSE = -inf
    uint16_t* orow = a.o + ((size_t)b * H + h) * kDl + c0;
    *(u32x4*)orow = u32x4{0u, 0u, 0u, 0u};
    *(u32x4*)(orow + 8) = u32x4{0u, 0u, 0u, 0u};
    if ((threadIdx.x & 31) == 0) a.lse[(size_t)b * H + h] = -INFINITY;
    return;
  }
  const int w0 = split_owner(g0, T, P), w1 = split_owner(g1 - 1, T, P);
  // Slice v covers tiles [floor(v*T/P), floor((v+1)*T/P)); the bounds are
  // stepped from w0 as v*T = q*P + r (T = tq*P + tr), so no slice costs a
  // division (these are wave-uniform, and 64-bit divisions on the shared
  // scalar unit had made this kernel scalar-bound).
  const int tq = T / P, tr = T - tq * P;
  int q, r;
  {
    const long long vt = (long long)w0 * T;
    q = (int)(vt / P);
    r = (int)(vt - (long long)q * P);
  }
  float mx = -INFINITY, tot = 0.f;
  f32x4 acc[4] = {};
  for (int v0 = w0; v0 <= w1; v0 += MP) {
    float ls[MP];
    u32x4 x[MP][2];
#pragma unroll
    for (int k = 0; k < MP; ++k) {
      const int v = v0 + k;
      int q1 = q + tq, r1 = r + tr;
      if (r1 >= P) {
        r1 -= P;
        ++q1;
      }
      const bool nonempty = q1 != q;  // floor((v+1)*T/P) != floor(v*T/P)
      q = q1;
      r = r1;
      ls[k] = -INFINITY;
      x[k][0] = x[k][1] = u32x4{0u, 0u, 0u, 0u};
      if (v <= w1 && nonempty) {
        const size_t slot = (size_t)v + b;
        ls[k] = a.part_lse[slot * H + h];
        const u32x4* src = (const u32x4*)(a.part_o + (slot * H + h) * kDl + c0);
        x[k][0] = src[0];
        x[k][1] = src[1];
      }
    }
    float mn = mx;
#pragma unroll
    for (int k = 0; k < MP; ++k) mn = fmaxf(mn, ls[k]);
    if (mn == -INFINITY) continue;
    const float sc = mx == -INFINITY ? 0.f : __expf(mx - mn);  // rescale of what was merged so far
    tot *= sc;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] *= sc;
    mx = mn;
#pragma unroll
    for (int k = 0; k < MP; ++k) {
      const float wt = ls[k] == -INFINITY ? 0.f : __expf(ls[k] - mx);
      tot += wt;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * i + q / 2][2 * (q % 2)] += wt * __uint_as_float(x[k][i][q] << 16);
          acc[2 * i + q / 2][2 * (q % 2) + 1] += wt * __uint_as_float(x[k][i][q] & 0xffff0000u);
        }
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  uint16_t* orow = a.o + ((size_t)b * H + h) * kDl + c0;
  u32x4 o0 = {pack_bf16x2(acc[0][0] * inv, acc[0][1] * inv), pack_bf16x2(acc[0][2] * inv, acc[0][3] * inv),
              pack_bf16x2(acc[1][0] * inv, acc[1][1] * inv), pack_bf16x2(acc[1][2] * inv, acc[1][3] * inv)};
  u32x4 o1 = {pack_bf16x2(acc[2][0] * inv, acc[2][1] * inv), pack_bf16x2(acc[2][2] * inv, acc[2][3] * inv),
              pack_bf16x2(acc[3][0] * inv, acc[3][1] * inv), pack_bf16x2(acc[3][2] * inv, acc[3][3] * inv)};
  *(u32x4*)orow = o0;
  *(u32x4*)(orow + 8) = o1;
  if ((threadIdx.x & 31) == 0) a.lse[(size_t)b * H + h] = tot > 0.f ? mx + __logf(tot) : -INFINITY;
}

// S += A * B on v_mfma_f32_32x32x16_bf16 with the accumulator pinned to
// VGPRs (inline asm): the score tile then never competes with O for the
// accumulation registers, which O fills, and no accumulator is moved
// between the two register files inside the tile loop. LAST appends the
// wait states a VALU access to the result needs after the final MFMA of a
// chain (the compiler does not see this MFMA). For the same reason no wait
// states protect the A and B operands: an MFMA of the chain may read them
// some clocks after it issues, so no VALU instruction may run between these
// MFMAs (the compiler could give its result a register an MFMA has yet to
// read); the only writes there are the next K fragments' LDS reads, whose
// data lands long after.
template <bool FIRST, bool LAST>
__device__ __forceinline__ void mfma32_v(f32x16& s, bf16x8 a, bf16x8 b) {
  if constexpr (FIRST && LAST)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 4" : "=v"(s) : "v"(a), "v"(b));
  else if constexpr (FIRST)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(s) : "v"(a), "v"(b));
  else if constexpr (LAST)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(s) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a), "v"(b));
}

template <int NW, int NSTAGE, bool FUSE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_split_kernel(MlaArgs a) {
  constexpr int KS = (kDl + kDr) / 16;          // 36 k-steps of the score product
  constexpr int KSL = kDl / 16;                 // 32 of them on the latent part
  constexpr int DB = kDl / 32;                  // 16 output blocks
  constexpr int LAT_LOADS = kBK / NW;           // one 1 KB latent row per wave load
  constexpr int PE_LOADS = kBK * (kDr / 8) / (64 * NW);
  constexpr int LPT = LAT_LOADS + PE_LOADS;     // loads per wave per tile
  constexpr int PF = NSTAGE - 2;                // tiles in flight ahead of the scored one
  static_assert(kBK * (kDr / 8) % (64 * NW) == 0, "rotary tile must split into wave loads");
  static_assert(PF * LPT < 64, "vmcnt range");
  static_assert(PF == 1 || PF == 2, "ring of 3 or 4 stages");
  constexpr float TAU = 8.0f;

  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hi = lane >> 5, col = lane & 31;
  const int H = a.H;
  // heads past H (the last wave's padding when H is not a multiple of 32)
  // compute on head H-1's query and store nothing
  const int head = wave * 32 + col;
  const int qhead = min(head, H - 1);
  const float c = a.c;
  const uint32_t smem0 = lds_addr(smem);

  // Lane-dependent LDS offsets inside a stage. Latent rows are padded to
  // kRowL bytes, so each latent read is one base register plus an
  // instruction offset: the score operand (key row col, 16-byte chunk
  // 2*ks + hi; 16 consecutive rows at one chunk hit 16 distinct 4-bank
  // groups) and the transposing reads of the value operand (a 16-lane group
  // reads 32 bytes from each of four consecutive key rows, 48 bytes of bank
  // offset apart). The rotary rows keep the XOR swizzle of their loads.
  const uint32_t kb_off = (uint32_t)(col * kRowL + 16 * hi);
  uint32_t pb_off[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) pb_off[r] = kTileL + col * 128 + 16 * swz<8>(col, 2 * r + hi);
  const uint32_t tb_off =
      (uint32_t)((4 * hi + ((lane & 15) >> 2)) * kRowL + 32 * ((lane >> 4) & 1) + 8 * (lane & 3));

  // Tile prefix: tile_ptr[b] = tiles of batches before b. With FUSE the
  // workgroup forms it in LDS (and workgroup 0 also writes it out for the
  // merge kernel); otherwise the plan kernel has written it.
  typedef __attribute__((address_space(3))) int lds_int;
  lds_int* tp_lds = (lds_int*)(uintptr_t)(smem0 + NSTAGE * kStage);
  if constexpr (FUSE) {
    const int B = a.B, nthr = NW * 64, t = threadIdx.x;
    const int per = (B + nthr - 1) / nthr;
    const int b0 = min(B, t * per), b1 = min(B, b0 + per);
    int local = 0;
    for (int bb = b0; bb < b1; ++bb) local += batch_tiles(a.indptr, bb);
    // inclusive scan of the per-thread counts (Hillis-Steele in LDS)
    lds_int* sc = tp_lds + kFusedPlanMax + 1;
    sc[t] = local;
    __syncthreads();
    for (int off = 1; off < nthr; off <<= 1) {
      const int add = t >= off ? sc[t - off] : 0;
      __syncthreads();
      sc[t] += add;
      __syncthreads();
    }
    int run = t > 0 ? sc[t - 1] : 0;
    for (int bb = b0; bb < b1; ++bb) {
      tp_lds[bb] = run;
      run += batch_tiles(a.indptr, bb);
    }
    if (t == nthr - 1) tp_lds[B] = sc[nthr - 1];
    __syncthreads();
    if (blockIdx.x == 0)
      for (int bb = t; bb <= B; bb += nthr) a.tile_ptr[bb] = tp_lds[bb];
  }
  auto tile_ptr = [&](int i) -> int {
    if constexpr (FUSE) return tp_lds[i];
    else return a.tile_ptr[i];
  };

  const int P = gridDim.x, w = slice_of(blockIdx.x, P);
  const int T = tile_ptr(a.B);
  int g = split_start(w, T, P);
  const int gend = split_start(w + 1, T, P);
  if (g >= gend) return;

  int b;
  {
    int lo = 0, up = a.B;  // tile_ptr[lo] <= g < tile_ptr[up]
    while (up - lo > 1) {
      const int mid = (lo + up) >> 1;
      if (tile_ptr(mid) <= g) lo = mid; else up = mid;
    }
    b = lo;
  }

  while (true) {
    const int tb = tile_ptr(b);
    const int seg_end = min(gend, tile_ptr(b + 1));
    const int t0 = g - tb, nt = seg_end - g;
    const int kv_lo = a.indptr[b];
    const int kv_hi = a.indptr[b + 1];

    // all waves are done with the LDS ring of the previous piece
    wait_lgkmcnt0();
    barrier();

    // Tile i of this piece -> LDS stage i % NSTAGE. A latent load of a wave
    // covers one whole key row (rows past the batch repeat its last row, so
    // the prologue may load tiles past the piece's end); rotary loads cover
    // 8 rows with the chunk order swizzled on the global side.
    auto issue = [&](int i) {
      char* sl = smem + (i % NSTAGE) * kStage;
      const int key0 = kv_lo + (t0 + i) * kBK;
#pragma unroll
      for (int n = 0; n < LAT_LOADS; ++n) {
        const int row = n * NW + wave;
        const int gr = min(key0 + row, kv_hi - 1);
        load_lds16_sbase(a.kv + (size_t)gr * kDl, 16 * lane, lds_addr(sl + row * kRowL));
      }
      // rotary rows relative to the tile's first row (clamped like the latent rows)
      const int rbase = min(key0, kv_hi - 1);
#pragma unroll
      for (int n = 0; n < PE_LOADS; ++n) {
        const int slot = (n * NW + wave) * 64 + lane;
        const int row = slot >> 3;
        const uint32_t voff = (uint32_t)(min(row, kv_hi - 1 - rbase) * (kDr * 2) + swz<8>(row, slot & 7) * 16);
        load_lds16_sbase(a.kpe + (size_t)rbase * kDr, voff, lds_addr(sl + kTileL + (n * NW + wave) * 1024));
      }
    };
#pragma unroll
    for (int i = 0; i < PF; ++i) issue(i);

    // Q^T fragments of this wave's heads (after the first tiles' loads, so
    // they travel together)
    bf16x8 qf[KS];
    {
      const uint16_t* qr = a.q + ((size_t)b * H + qhead) * kDl + hi * 8;
      const uint16_t* pr = a.qpe + ((size_t)b * H + qhead) * kDr + hi * 8;
#pragma unroll
      for (int ks = 0; ks < KSL; ++ks) qf[ks] = as_bf16x8(*(const u32x4*)(qr + ks * 16));
#pragma unroll
      for (int ks = KSL; ks < KS; ++ks) qf[ks] = as_bf16x8(*(const u32x4*)(pr + (ks - KSL) * 16));
    }

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    float m = -INFINITY, lsum = 0.f;

    // ---- S^T = KV * Q^T + K_pe * Q_pe^T of the tile in stage st, the
    // operand reads six k-steps ahead of their MFMAs
    auto score = [&](int st, f32x16& s) {
      const uint32_t kb = smem0 + (uint32_t)(st * kStage) + kb_off;
      const uint32_t pb = smem0 + (uint32_t)(st * kStage);
      constexpr int AHEAD = 6;
      auto kread = [&](auto KSc) -> u32x4 {
        constexpr int ks = decltype(KSc)::value;
        if constexpr (ks < KSL) return lds_read128_async<32 * ks>(kb);
        else return lds_read128_async<0>(pb + pb_off[ks - KSL]);
      };
      u32x4 kr[AHEAD];
      static_for<AHEAD>([&](auto KSc) { kr[decltype(KSc)::value] = kread(KSc); });
      static_for<KS>([&](auto KSc) {
        constexpr int ks = decltype(KSc)::value, slot = ks % AHEAD;
        constexpr int later = (KS - 1 - ks) < (AHEAD - 1) ? (KS - 1 - ks) : (AHEAD - 1);
        wait_lds_tied_n4<later>(kr[slot]);
        mfma32_v<ks == 0, ks == KS - 1>(s, as_bf16x8(kr[slot]), qf[ks]);
        if constexpr (ks + AHEAD < KS) kr[slot] = kread(std::integral_constant<int, ks + AHEAD>{});
      });
    };
    // ---- online softmax (lane = head): the running max is raised only past
    // the threshold (then alpha < 1 rescales l here and O by the caller),
    // P^T in bf16, row sums from the unrounded P
    auto softmax = [&](const f32x16& s, bf16x8 (&pf)[2], bool& raised, float& alpha) {
      float mx = -INFINITY;
#pragma unroll
      for (int i2 = 0; i2 < 16; ++i2) mx = fmaxf(mx, s[i2]);
      mx = max_halves(mx) * c;
      raised = mx - m > TAU;  // false when mx == -inf
      alpha = raised ? fast_exp2(m - mx) : 1.f;
      m = raised ? mx : m;
      lsum *= alpha;
      const float mc = m == -INFINITY ? 0.f : m;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          p[j] = fast_exp2(fmaf(s[half * 8 + j], c, -mc));
          lsum += p[j];
        }
        u32x4 x = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                   pack_bf16x2(p[6], p[7])};
        pf[half] = as_bf16x8(x);
      }
    };
    // ---- O^T += KV^T * P^T for the tile in stage st (KV^T by transposing
    // reads of the same latent rows), half 0 of every d-block, then half 1;
    // the reads of four steps are in flight
    auto pv = [&](int st, const bf16x8 (&pf)[2]) {
      const uint32_t vb = smem0 + (uint32_t)(st * kStage) + tb_off;
      constexpr int NSTEP = 2 * DB;
      constexpr int AHEAD = 4;
      auto vread = [&](auto SC, u32x2 (&r)[2]) {
        constexpr int stp = decltype(SC)::value, half = stp / DB, db = stp % DB;
        constexpr int off = half * 16 * kRowL + db * 64;
        r[0] = lds_read_tr16_async<off>(vb);
        r[1] = lds_read_tr16_async<off + 8 * kRowL>(vb);
      };
      u32x2 vr[AHEAD][2];
      static_for<AHEAD>([&](auto SC) { vread(SC, vr[decltype(SC)::value]); });
      static_for<NSTEP>([&](auto SC) {
        constexpr int stp = decltype(SC)::value, half = stp / DB, db = stp % DB;
        constexpr int slot = stp % AHEAD;
        constexpr int later = (NSTEP - 1 - stp) < (AHEAD - 1) ? (NSTEP - 1 - stp) : (AHEAD - 1);
        wait_lds_tied_n<2 * later>(vr[slot][0], vr[slot][1]);
        oacc[db] = mfma32(cat_tr(vr[slot][0], vr[slot][1]), pf[half], oacc[db]);
        if constexpr (stp + AHEAD < NSTEP) vread(std::integral_constant<int, stp + AHEAD>{}, vr[slot]);
      });
    };
    // ---- the rare O rescale after a raise, in place in the accumulation
    // registers (wait states first: the last P*V MFMA wrote them)
    auto rescale = [&](bool raised, float alpha) {
      if (__builtin_amdgcn_ballot_w64(raised)) {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" ::: "memory");
        static_for<DB>([&](auto DBc) { scale_acc16(oacc[DBc], alpha); });
      }
    };
    // the piece's last tile may be partial: keys past the batch score -inf
    auto tail_mask = [&](int i, f32x16& s) {
      const int nvalid = min(kBK, kv_hi - (kv_lo + (t0 + i) * kBK));
      if (nvalid < kBK) {
#pragma unroll
        for (int i2 = 0; i2 < 16; ++i2)
          if (8 * (i2 >> 2) + 4 * hi + (i2 & 3) >= nvalid) s[i2] = -INFINITY;
      }
    };
    // tile i in LDS, every wave past P*V of tile i-2 (so the refill of
    // tile i+PF may overwrite its stage), then that refill issued
    auto wait_tile = [&](int i) {
      // the tiles issued before step i are 0 .. max(PF-1, min(i+PF-1, nt-1))
      const int last = max(PF - 1, min(i + PF - 1, nt - 1));
      if (last > i) wait_vmcnt<LPT>();
      else wait_vmcnt<0>();
      barrier();
      if (i + PF < nt) issue(i + PF);
    };

    // Software pipeline over the piece's tiles: step i scores tile i, runs
    // its softmax and then accumulates P*V of tile i-1 (whose P the previous
    // step produced), so the MFMAs of one tile's product follow the VALU
    // work of the other's without waiting for it. O is rescaled after P*V
    // of tile i-1 when tile i raised the running max.
    bf16x8 pf_prev[2];
    {
      wait_tile(0);
      f32x16 s;
      score(0, s);
      if (nt == 1) tail_mask(0, s);
      bool raised;
      float alpha;
      softmax(s, pf_prev, raised, alpha);  // O is still zero: nothing to rescale
    }
    auto step = [&](int i, auto LASTc) {
      wait_tile(i);
      f32x16 s;
      score(i % NSTAGE, s);
      if constexpr (decltype(LASTc)::value) tail_mask(i, s);
      bf16x8 pf[2];
      bool raised;
      float alpha;
      softmax(s, pf, raised, alpha);
      pv((i - 1) % NSTAGE, pf_prev);
      rescale(raised, alpha);
      pf_prev[0] = pf[0];
      pf_prev[1] = pf[1];
    };
    for (int i = 1; i + 1 < nt; ++i) step(i, std::false_type{});
    if (nt > 1) step(nt - 1, std::true_type{});
    pv((nt - 1) % NSTAGE, pf_prev);

    // ---- normalised partial of this piece -> slot (workgroup + batch). The
    // rows go through LDS (the ring is free once every wave has passed the
    // barrier below) so that each store writes one whole 1 KB head row.
    {
      const float l = sum_halves(lsum);
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const size_t slot = (size_t)w + b;
      constexpr int SRS = kDl * 2 + 16;  // staging row stride (padded)
      static_assert(NW * 32 * SRS <= NSTAGE * kStage, "staging fits the ring");
      typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
      typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
      const uint32_t stg = smem0 + wave * 32 * SRS;
      wait_vmcnt<0>();  // the prologue may have loaded tiles past the piece's end
      barrier();
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + 8 * g4 + 4 * hi;
          *(lds_u32x2*)(uintptr_t)(stg + col * SRS + d * 2) =
              u32x2{pack_bf16x2(oacc[db][g4 * 4] * inv, oacc[db][g4 * 4 + 1] * inv),
                    pack_bf16x2(oacc[db][g4 * 4 + 2] * inv, oacc[db][g4 * 4 + 3] * inv)};
        }
      uint16_t* po = a.part_o + (slot * H + wave * 32) * kDl + 8 * lane;
      const int rows = min(32, H - wave * 32);  // this wave's heads below H
#pragma unroll 8
      for (int r = 0; r < 32; ++r)
        if (r < rows) *(u32x4*)(po + (size_t)r * kDl) = *(const lds_u32x4*)(uintptr_t)(stg + r * SRS + 16 * lane);
      if (hi == 0 && head < H) a.part_lse[slot * H + head] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
    }

    g = seg_end;
    if (g >= gend) break;
    do { ++b; } while (tile_ptr(b + 1) <= g);
  }
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t mla_workspace_bytes(int B, int H, int n_split) {
  const size_t slots = (size_t)n_split + B;
  return align256((size_t)(B + 1) * 4) + align256(slots * H * 4) + slots * H * kDl * 2;
}

template <int NW, int NSTAGE, bool FUSE>
static hipError_t launch_split(const MlaArgs& a, int n_split, hipStream_t stream) {
  // ring, then (fused plan) the tile prefix and the scan scratch
  constexpr size_t lds = (size_t)NSTAGE * kStage + (size_t)(kFusedPlanMax + 1 + NW * 64) * 4;
  static_assert(lds <= 160 * 1024, "LDS budget");
  auto kern = mla_split_kernel<NW, NSTAGE, FUSE>;
  static const hipError_t attr_err =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr_err != hipSuccess) return attr_err;
  hipLaunchKernelGGL(kern, dim3(n_split), dim3(NW * 64), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_mla_decode(const void* q, const void* q_pe, const void* kv, const void* k_pe,
                             void* o, float* lse, int B, int H, const int32_t* kv_indptr,
                             float scale, int n_split, void* workspace, hipStream_t stream) {
  MlaArgs a{};
  a.q = (const uint16_t*)q;
  a.qpe = (const uint16_t*)q_pe;
  a.kv = (const uint16_t*)kv;
  a.kpe = (const uint16_t*)k_pe;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.indptr = kv_indptr;
  a.B = B;
  a.H = H;
  a.c = scale * kLog2e;
  char* ws = (char*)workspace;
  const size_t slots = (size_t)n_split + B;
  const size_t ints = align256((size_t)(B + 1) * 4);
  a.tile_ptr = (int*)ws;
  a.part_lse = (float*)(ws + ints);
  a.part_o = (uint16_t*)(ws + ints + align256(slots * H * 4));

  hipError_t e = hipSuccess;
  const bool fuse = B < kFusedPlanMax;
  if (!fuse) {
    hipLaunchKernelGGL(mla_plan_kernel, dim3(1), dim3(1024), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // 32 heads per wave: 4 waves above 64 heads, 2 above 32, else 1
  if (H > 64) e = fuse ? launch_split<4, 4, true>(a, n_split, stream) : launch_split<4, 4, false>(a, n_split, stream);
  else if (H > 32) e = fuse ? launch_split<2, 4, true>(a, n_split, stream) : launch_split<2, 4, false>(a, n_split, stream);
  else e = fuse ? launch_split<1, 3, true>(a, n_split, stream) : launch_split<1, 3, false>(a, n_split, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_combine_kernel, dim3(B, (H + 7) / 8), dim3(256), 0, stream, a, n_split);
  return hipGetLastError();
}

// ---- static workspace of mla_decode_noalloc
//
// kNoAllocScratchBytes of device memory in the library's own code object,
// one copy per GPU the library runs on, held until the process ends. In
// host code `scratch` names a host-side stand-in, not the device array: its
// device address comes from hipGetSymbolAddress, looked up once per device
// with that device current and kept here; only that address is passed on.
// Nothing in the workspace needs to start at zero (every slot the merge
// reads was written by the same call), so the calls clear nothing.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

hipError_t mla_noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 256;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace tattn
