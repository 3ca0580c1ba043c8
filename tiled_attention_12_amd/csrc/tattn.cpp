// C ABI of libtattn.so: argument validation, dispatch to the gfx950
// launchers, the per-device workspace of the split decode. See
// include/tattn.h for the contract of every entry point.
#include "tattn.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "launch.h"

#define TATTN_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kMaxSeq = 1 << 30;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int status_of(hipError_t e) {
  if (e == hipSuccess) return TATTN_OK;
  if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) return TATTN_ERR_OOM;
  return TATTN_ERR_HIP;
}

// Compute-unit count of the current device (cached per device ordinal).
int current_device_cus(int* cus) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return TATTN_ERR_HIP;
  static std::mutex mu;
  static int cache[256] = {0};
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 256 && cache[dev] > 0) {
    *cus = cache[dev];
    return TATTN_OK;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return TATTN_ERR_HIP;
  if (dev < 256) cache[dev] = n;
  *cus = n;
  return TATTN_OK;
}

int have_device() {
  int dev = -1;
  return (hipGetDevice(&dev) == hipSuccess && dev >= 0) ? TATTN_OK : TATTN_ERR_HIP;
}

// Decode workspaces: one per (device, stream), up to kWsSlots streams per
// device, each grown (never shrunk) to the largest size a call on that
// stream has needed and kept until the process ends. A call on the slot's
// own stream needs no ordering against the slot's earlier calls (stream
// order gives it). Only a slot that passes to another stream (every slot
// taken) needs its last call's completion: `done` is recorded after a call
// whenever more than one slot is in use, and the new stream waits for it;
// a slot whose last call came while it was the only slot in use has no
// such event, and its takeover waits on the host for the device to finish
// (the one case where a call blocks the host; slots are never released, so
// only a device's first slot can be in that state, and only once). With a single stream no
// event is recorded or waited for. A buffer that has to grow is not freed at
// once: it is retired with an event recorded on the calling stream, after
// its last use, and freed by a later call once that event has completed.
struct Workspace {
  hipStream_t stream = nullptr;
  bool used = false;
  void* ptr = nullptr;
  size_t bytes = 0;
  hipEvent_t done = nullptr;
  bool recorded = false;  // `done` marks the slot's last call
  unsigned long long last_use = 0;
};
struct Retired {
  void* ptr;
  hipEvent_t done;
};
constexpr int kWsSlots = 8;
struct DeviceWorkspaces {
  Workspace slot[kWsSlots];
  std::vector<Retired> retired;
  unsigned long long clock = 0;
};

std::mutex g_ws_mu;
DeviceWorkspaces g_ws[256];

// Frees retired buffers whose last kernels have completed (never waits).
void free_retired(DeviceWorkspaces& d) {
  size_t keep = 0;
  for (size_t i = 0; i < d.retired.size(); ++i) {
    Retired& r = d.retired[i];
    if (hipEventQuery(r.done) == hipSuccess) {
      (void)hipFree(r.ptr);
      (void)hipEventDestroy(r.done);
    } else {
      d.retired[keep++] = r;
    }
  }
  d.retired.resize(keep);
  (void)hipGetLastError();  // a not-ready query is not an error of this call
}

// The slot of `s` on this device: its own, else an unused one, else the
// least recently used one (whose stream the call then waits for).
Workspace& slot_for(DeviceWorkspaces& d, hipStream_t s) {
  Workspace* lru = &d.slot[0];
  for (Workspace& w : d.slot) {
    if (w.used && w.stream == s) return w;
    if (w.last_use < lru->last_use) lru = &w;
  }
  for (Workspace& w : d.slot)
    if (!w.used) {
      w.used = true;
      w.stream = s;
      return w;
    }
  lru->stream = s;
  return *lru;
}

// Workgroup shape of the dense prefill: TATTN_MHA_WAVES = 4 or 8 forces it
// (a test hook: both shapes must give the same result); otherwise the
// launcher picks it from the launch size.
int mha_dense_waves() {
  if (const char* v = std::getenv("TATTN_MHA_WAVES")) {
    const long n = std::strtol(v, nullptr, 10);
    if (n == 4 || n == 8) return (int)n;
  }
  return 0;
}

// Shared validation of the two MHA entry points. Returns TATTN_OK with
// *nothing = true when there is no work.
int check_mha(const void* q, const void* k, const void* v, const void* o, const void* lse, int B, int H,
              int Sq, int Skv, int D, int causal, float scale, bool* nothing) {
  *nothing = false;
  if (B < 0 || H < 0 || Sq < 0 || Skv < 0) return TATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return TATTN_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return TATTN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return TATTN_ERR_UNSUPPORTED;
  if (B == 0 || H == 0 || Sq == 0) {
    *nothing = true;
    return TATTN_OK;
  }
  if (!q || !o || !lse || (Skv > 0 && (!k || !v))) return TATTN_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(o, 16) || !aligned(lse, 4) || (Skv > 0 && (!aligned(k, 16) || !aligned(v, 16))))
    return TATTN_ERR_ALIGN;
  if (Sq > kMaxSeq || Skv > kMaxSeq) return TATTN_ERR_UNSUPPORTED;
  const long long n_bh = (long long)B * H;
  if (n_bh > INT_MAX || n_bh * ((Sq + 31) / 32) > INT_MAX) return TATTN_ERR_UNSUPPORTED;
  return TATTN_OK;
}

}  // namespace

TATTN_API int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Sq,
                       int Skv, int D, int causal, float scale, void* stream) {
  bool nothing = false;
  int st = check_mha(q, k, v, o, lse, B, H, Sq, Skv, D, causal, scale, &nothing);
  if (st != TATTN_OK || nothing) return st;
  int cus = 0;
  if ((st = current_device_cus(&cus)) != TATTN_OK) return st;
  return status_of(tattn::launch_mha_fwd_bf16(q, k, v, o, lse, B, H, H, Sq, Skv, D, causal != 0, 0, nullptr,
                                              scale, cus, mha_dense_waves(), (hipStream_t)stream));
}

TATTN_API int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                          int Hkv, int Sq, int Skv, int D, int causal, int window, const uint8_t* block_mask,
                          float scale, void* stream) {
  if (Hkv < 1 && !(B == 0 || H == 0)) return TATTN_ERR_INVALID_ARG;
  if (Hkv > 0 && H % Hkv != 0) return TATTN_ERR_INVALID_ARG;
  if (window < 0) return TATTN_ERR_INVALID_ARG;
  if (window > kMaxSeq) return TATTN_ERR_UNSUPPORTED;
  bool nothing = false;
  int st = check_mha(q, k, v, o, lse, B, H, Sq, Skv, D, causal, scale, &nothing);
  if (st != TATTN_OK || nothing) return st;
  int cus = 0;
  if ((st = current_device_cus(&cus)) != TATTN_OK) return st;
  return status_of(tattn::launch_mha_fwd_bf16(q, k, v, o, lse, B, H, Hkv, Sq, Skv, D, causal != 0, window,
                                              block_mask, scale, cus, mha_dense_waves(), (hipStream_t)stream));
}

TATTN_API int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
                           int Sq, int Skv, int D, int causal, float scale, void* stream) {
  bool nothing = false;
  int st = check_mha(q, k, v, o, lse, B, H, Sq, Skv, D, causal, scale, &nothing);
  if (st != TATTN_OK || nothing) return st;
  if ((Sq + 63) / 64 > 65535) return TATTN_ERR_UNSUPPORTED;
  if ((st = have_device()) != TATTN_OK) return st;
  return status_of(tattn::launch_mha_fwd_f32(q, k, v, o, lse, B, H, Sq, Skv, D, causal != 0, scale,
                                             (hipStream_t)stream));
}

// Number of split workgroups of the MLA decode: the device's compute units,
// or TATTN_MLA_SPLITS when set to a positive count (a test hook: the result
// must not depend on how the keys are split).
static int mla_splits(int cus) {
  if (const char* v = std::getenv("TATTN_MLA_SPLITS")) {
    const long n = std::strtol(v, nullptr, 10);
    if (n > 0 && n <= 65536) return (int)n;
  }
  return cus;
}

// Shared validation of the two MLA entry points. Returns TATTN_OK with
// *nothing = true when there is no work.
static int check_mla(const void* q, const void* q_pe, const void* kv, const void* k_pe, const void* o,
                     const void* lse, int B, int H, const int32_t* kv_indptr, float scale, bool* nothing) {
  *nothing = false;
  if (B < 0 || H < 0) return TATTN_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return TATTN_ERR_INVALID_ARG;
  if (B == 0) {
    *nothing = true;
    return TATTN_OK;
  }
  if (H < 1 || H > 128) return TATTN_ERR_UNSUPPORTED;
  // kv and k_pe may be null when no batch has keys (N = 0): the kernels read
  // key rows only inside the ranges kv_indptr gives
  if (!q || !q_pe || !o || !lse || !kv_indptr) return TATTN_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(q_pe, 16) || !aligned(kv, 16) || !aligned(k_pe, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(kv_indptr, 4))
    return TATTN_ERR_ALIGN;
  if ((long long)B * H > INT_MAX || B > (1 << 24)) return TATTN_ERR_UNSUPPORTED;
  return TATTN_OK;
}

TATTN_API int mla_decode(const void* q, const void* q_pe, const void* kv, const void* k_pe, void* o, float* lse,
                         int B, int H, const int32_t* kv_indptr, float scale, void* stream) {
  bool nothing = false;
  int st = check_mla(q, q_pe, kv, k_pe, o, lse, B, H, kv_indptr, scale, &nothing);
  if (st != TATTN_OK || nothing) return st;
  int cus = 0;
  if ((st = current_device_cus(&cus)) != TATTN_OK) return st;
  const int n_split = mla_splits(cus);
  const size_t bytes = tattn::mla_workspace_bytes(B, H, n_split);
  if (const char* cap = std::getenv("TATTN_WS_LIMIT_BYTES")) {
    if (bytes > (size_t)std::strtoull(cap, nullptr, 10)) return TATTN_ERR_OOM;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) return TATTN_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  std::lock_guard<std::mutex> lock(g_ws_mu);
  DeviceWorkspaces& d = g_ws[dev];
  free_retired(d);
  int in_use = 0;
  bool own = false, any_free = false;
  for (const Workspace& x : d.slot) {
    in_use += x.used;
    own |= x.used && x.stream == s;
    any_free |= !x.used;
  }
  const bool takeover = !own && !any_free;  // the slot passes from another stream
  if (!own) ++in_use;
  Workspace& w = slot_for(d, s);
  w.last_use = ++d.clock;
  if (!w.done && hipEventCreateWithFlags(&w.done, hipEventDisableTiming) != hipSuccess) {
    w.done = nullptr;
    return TATTN_ERR_HIP;
  }
  if (takeover) {
    // after the slot's last call on its previous stream
    if (w.recorded) {
      if (hipStreamWaitEvent(s, w.done, 0) != hipSuccess) return TATTN_ERR_HIP;
    } else if (hipDeviceSynchronize() != hipSuccess) {
      return TATTN_ERR_HIP;
    }
  }
  if (w.bytes < bytes) {
    void* p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess || !p) {
      (void)hipGetLastError();
      return TATTN_ERR_OOM;
    }
    if (w.ptr) {
      // the old buffer's last use is ordered before this point of stream s
      // (same stream, or the takeover's wait above): an event recorded here
      // completes after it
      hipEvent_t ret = nullptr;
      if (hipEventCreateWithFlags(&ret, hipEventDisableTiming) != hipSuccess) {
        (void)hipFree(p);
        return TATTN_ERR_HIP;
      }
      if (hipEventRecord(ret, s) != hipSuccess) {
        (void)hipEventDestroy(ret);
        (void)hipFree(p);
        return TATTN_ERR_HIP;
      }
      d.retired.push_back({w.ptr, ret});
    }
    w.ptr = p;
    w.bytes = bytes;
  }
  const hipError_t e =
      tattn::launch_mla_decode(q, q_pe, kv, k_pe, o, lse, B, H, kv_indptr, scale, n_split, w.ptr, s);
  // another stream may take this slot over only when several are in use
  hipError_t er = hipSuccess;
  w.recorded = false;
  if (in_use > 1) {
    er = hipEventRecord(w.done, s);
    w.recorded = er == hipSuccess;
  }
  if (e != hipSuccess) return status_of(e);
  return status_of(er);
}

TATTN_API int mla_decode_noalloc(const void* q, const void* q_pe, const void* kv, const void* k_pe, void* o,
                                 float* lse, int B, int H, const int32_t* kv_indptr, float scale, void* stream) {
  bool nothing = false;
  int st = check_mla(q, q_pe, kv, k_pe, o, lse, B, H, kv_indptr, scale, &nothing);
  if (st != TATTN_OK || nothing) return st;
  int cus = 0;
  if ((st = current_device_cus(&cus)) != TATTN_OK) return st;
  const int n_split = mla_splits(cus);
  if (tattn::mla_workspace_bytes(B, H, n_split) > tattn::kNoAllocScratchBytes) return TATTN_ERR_SCRATCH;
  void* ws = nullptr;
  const hipError_t e = tattn::mla_noalloc_scratch(&ws);
  if (e != hipSuccess) return status_of(e);
  return status_of(tattn::launch_mla_decode(q, q_pe, kv, k_pe, o, lse, B, H, kv_indptr, scale, n_split, ws,
                                            (hipStream_t)stream));
}

TATTN_API int ssd_scan(const void* x, const float* dt, const float* A, const void* B, const void* C, void* y,
                       const float* init_state, float* final_state, int batch, int seqlen, int heads,
                       int groups, int headdim, int dstate, void* stream) {
  if (batch < 0 || seqlen < 0 || heads < 0 || groups < 0 || headdim < 0 || dstate < 0)
    return TATTN_ERR_INVALID_ARG;
  if (heads > 0 && (groups < 1 || heads % groups != 0)) return TATTN_ERR_INVALID_ARG;
  if (headdim != 64 || dstate != 128) return TATTN_ERR_UNSUPPORTED;
  if (batch == 0 || heads == 0) return TATTN_OK;
  if (seqlen == 0 && !final_state) return TATTN_OK;
  if (!A || (seqlen > 0 && (!x || !dt || !B || !C || !y))) return TATTN_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(y, 16) || !aligned(init_state, 16) ||
      !aligned(final_state, 16) || !aligned(dt, 4) || !aligned(A, 4))
    return TATTN_ERR_ALIGN;
  if ((long long)batch * heads > INT_MAX) return TATTN_ERR_UNSUPPORTED;
  if ((double)batch * seqlen * heads * headdim >= 4.6e18) return TATTN_ERR_UNSUPPORTED;
  if (final_state && init_state) {
    const uintptr_t bytes = (uintptr_t)batch * heads * headdim * dstate * 4;
    const uintptr_t f = (uintptr_t)final_state, i = (uintptr_t)init_state;
    if (f < i + bytes && i < f + bytes) return TATTN_ERR_INVALID_ARG;
  }
  int st = have_device();
  if (st != TATTN_OK) return st;
  return status_of(tattn::launch_ssd_scan_bf16(x, dt, A, B, C, y, init_state, final_state, batch, seqlen,
                                               heads, groups, (hipStream_t)stream));
}

TATTN_API const char* tattn_status_str(int status) {
  switch (status) {
    case TATTN_OK: return "ok";
    case TATTN_ERR_INVALID_ARG: return "invalid argument";
    case TATTN_ERR_UNSUPPORTED: return "unsupported shape or parameter";
    case TATTN_ERR_ALIGN: return "pointer misaligned";
    case TATTN_ERR_OOM: return "device workspace allocation failed";
    case TATTN_ERR_HIP: return "HIP runtime error or no usable device";
    case TATTN_ERR_SCRATCH: return "request needs more than the static scratch of mla_decode_noalloc";
    default: return "unknown status";
  }
}
