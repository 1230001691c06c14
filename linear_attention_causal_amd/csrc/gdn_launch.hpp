// Host-side launchers of the libgdn kernels.  Arguments have been validated
// by the C ABI layer (abi.hip) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>

#include "gdn.h"

namespace gdn {

hipError_t launch_conv_update(const gdn_geometry& g, const gdn_layer_weights& w,
                              const gdn_state_pool& pool, const int32_t* slot_idx,
                              int B, const void* qkv_in, float* qkv_out,
                              hipStream_t stream);

hipError_t launch_decode(const gdn_geometry& g, const gdn_layer_weights& w,
                         const gdn_state_pool& pool, const int32_t* slot_idx, int B,
                         const float* qkv, const void* z, const void* a,
                         const void* b, void* y, float* o_raw, hipStream_t stream);

// Workspace bytes of the fused step for up to B rows (any call with B' <= B
// fits).
size_t decode_workspace_bytes(const gdn_geometry& g, long long B);

// Library-held workspace of gdn_decode_step_noalloc: size, and the current
// device's copy (address taken and array cleared on first use per device).
constexpr size_t kStaticScratchBytes = GDN_NOALLOC_WORKSPACE_BYTES;
hipError_t static_scratch(void** ptr, hipStream_t stream);

hipError_t launch_decode_step(const gdn_geometry& g, const gdn_layer_weights& w,
                              const gdn_state_pool& pool, const int32_t* slot_idx, int B,
                              const void* qkv_in, const void* z, const void* a, const void* b,
                              void* y, float* o_raw, void* workspace, hipStream_t stream);

// Token-indexed scratch layout of the chunkwise prefill (see prefill.hip).
size_t prefill_scratch_bytes(const gdn_geometry& g, long long total_tokens,
                             long long num_seqs);

hipError_t launch_prefill(const gdn_geometry& g, const gdn_layer_weights& w,
                          const gdn_state_pool& pool, const int32_t* cu_seqlens,
                          const int32_t* cu_seqlens_host, int max_len, long long total_tokens,
                          const int32_t* slot_idx, const uint8_t* has_init, int N,
                          const void* qkv_in, const void* z, const void* a,
                          const void* b, void* y, float* o_raw, void* scratch,
                          hipStream_t stream);

// One weight of a projection launch: w [N][K] bf16, y [M][ldy] bf16.
// tile0 is filled in by launch_linear.
constexpr int kMaxLinearOuts = 4;
struct LinearOut {
  const __bf16* w;
  __bf16* y;
  int N, ldy, tile0;
};
// Kernel and workgroup tile (rows x columns) launch_linear uses.
struct LinearPlan {
  enum Kind { kStream, kTile } kind;
  int rows, cols;
};
LinearPlan linear_plan(int M, const LinearOut* outs, int count);
hipError_t launch_linear(const void* x, int M, int K, int ldx, const LinearOut* outs, int count,
                         hipStream_t stream);

// Device-side check of a slot index: result[0] = GDN_OK or GDN_E_SLOT,
// result[1] = the smallest offending row (INT32_MAX when none).
hipError_t launch_check_slots(const int32_t* slot, int B, int num_slots, int32_t* result,
                              hipStream_t stream);

hipError_t launch_compact(const gdn_geometry& g, const gdn_state_pool* pools, int L,
                          const int32_t* src, const int32_t* dst, int n,
                          hipStream_t stream);

}  // namespace gdn
