// Internal launchers called by the C ABI layer (tattn.cpp). Each enqueues
// its kernels on `stream` and returns the launch status; arguments are
// already validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tattn {

// K and V hold Hkv heads (H a multiple of Hkv); window 0 means no window;
// block_mask is null or a device [B, H, ceil(Sq/64), ceil(Skv/64)] byte mask;
// n_cu is the device's compute-unit count (the persistent grid size);
// dense_waves 4 or 8 forces the workgroup shape of the dense path, anything
// else leaves the choice to the launch size.
hipError_t launch_mha_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int Hkv, int Sq, int Skv, int D, bool causal, int window,
                               const uint8_t* block_mask, float scale, int n_cu, int dense_waves,
                               hipStream_t stream);

hipError_t launch_mha_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                              int B, int H, int Sq, int Skv, int D, bool causal, float scale,
                              hipStream_t stream);

// Bytes of device workspace mla_decode needs for B batches and H heads when
// split over `n_split` workgroups.
size_t mla_workspace_bytes(int B, int H, int n_split);

// Size of the static workspace of mla_decode_noalloc, and its device
// address on the current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
hipError_t mla_noalloc_scratch(void** ptr);

hipError_t launch_mla_decode(const void* q, const void* q_pe, const void* kv, const void* k_pe,
                             void* o, float* lse, int B, int H, const int32_t* kv_indptr,
                             float scale, int n_split, void* workspace, hipStream_t stream);

// Mamba-2 state-space scan: x [Bt, L, H, 64] bf16, dt [Bt, L, H] fp32,
// A [H] fp32, B/C [Bt, L, G, 128] bf16 -> y [Bt, L, H, 64] bf16; the initial
// and final states [Bt, H, 64, 128] fp32 may be null.
hipError_t launch_ssd_scan_bf16(const void* x, const float* dt, const float* A, const void* B, const void* C,
                                void* y, const float* init_state, float* final_state, int Bt, int L, int H,
                                int G, hipStream_t stream);

}  // namespace tattn
