// D2D compaction of slot-indexed state on retire (pegainfer issue #1001,
// Splits, "TP CUDA Graph": slot-indexed recurrent/conv state, D2D compaction
// on retire).  One launch covers every (layer, pair): slot dst[i] of each
// layer's pools receives a bit-exact copy of slot src[i].  The host has
// checked that the source and destination sets are disjoint and that the
// destinations are distinct, so every 16-byte unit is written by exactly one
// thread and no copy reads a unit another copy writes.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int kCompactLayersPerLaunch = 32;
constexpr int kCompactThreads = 256;
constexpr int kCompactUnroll = 4;  // 16-byte units per thread

struct CompactParams {
  const int32_t* src;
  const int32_t* dst;
  size_t rec_units;   // 16-byte units of one slot's recurrent state
  size_t conv_units;  // 16-byte units of one slot's conv window
  int num_slots;      // device-side guard: pairs outside [0, num_slots) are skipped
  char* rec[kCompactLayersPerLaunch];
  char* conv[kCompactLayersPerLaunch];
};

// grid: x = pieces of one slot, y = pair, z = layer within this launch
__global__ __launch_bounds__(kCompactThreads) void compact_kernel(CompactParams p) {
  const int pair = blockIdx.y, layer = blockIdx.z;
  const int si = p.src[pair], di = p.dst[pair];
  if (si < 0 || si >= p.num_slots || di < 0 || di >= p.num_slots) return;
  const size_t s = (size_t)si, d = (size_t)di;
  const size_t total = p.rec_units + p.conv_units;
  const size_t base = (size_t)blockIdx.x * kCompactThreads * kCompactUnroll + threadIdx.x;
  u32x4 v[kCompactUnroll];
  const u32x4* from[kCompactUnroll];
  u32x4* to[kCompactUnroll];
#pragma unroll
  for (int k = 0; k < kCompactUnroll; ++k) {
    const size_t u = base + (size_t)k * kCompactThreads;
    from[k] = nullptr;
    to[k] = nullptr;
    if (u < p.rec_units) {
      from[k] = reinterpret_cast<const u32x4*>(p.rec[layer]) + s * p.rec_units + u;
      to[k] = reinterpret_cast<u32x4*>(p.rec[layer]) + d * p.rec_units + u;
    } else if (u < total) {
      const size_t c = u - p.rec_units;
      from[k] = reinterpret_cast<const u32x4*>(p.conv[layer]) + s * p.conv_units + c;
      to[k] = reinterpret_cast<u32x4*>(p.conv[layer]) + d * p.conv_units + c;
    }
  }
#pragma unroll
  for (int k = 0; k < kCompactUnroll; ++k)
    if (from[k]) v[k] = __builtin_nontemporal_load(from[k]);
#pragma unroll
  for (int k = 0; k < kCompactUnroll; ++k)
    if (to[k]) __builtin_nontemporal_store(v[k], to[k]);
}

hipError_t launch_compact(const gdn_geometry& g, const gdn_state_pool* pools, int L,
                          const int32_t* src, const int32_t* dst, int n,
                          hipStream_t stream) {
  const size_t C = 2 * (size_t)g.num_k_heads * g.head_k_dim +
                   (size_t)g.num_v_heads * g.head_v_dim;
  const size_t ebytes = g.act_dtype == GDN_BF16 ? 2 : 4;
  CompactParams p;
  p.src = src;
  p.dst = dst;
  p.rec_units = (size_t)g.num_v_heads * g.head_k_dim * g.head_v_dim * 4 / 16;
  p.conv_units = (size_t)g.conv_kernel * C * ebytes / 16;
  p.num_slots = pools[0].num_slots;
  const size_t per_block = (size_t)kCompactThreads * kCompactUnroll;
  const unsigned pieces = (unsigned)((p.rec_units + p.conv_units + per_block - 1) / per_block);
  for (int l0 = 0; l0 < L; l0 += kCompactLayersPerLaunch) {
    const int nl = L - l0 < kCompactLayersPerLaunch ? L - l0 : kCompactLayersPerLaunch;
    for (int i = 0; i < kCompactLayersPerLaunch; ++i) {
      p.rec[i] = i < nl ? reinterpret_cast<char*>(pools[l0 + i].recurrent) : nullptr;
      p.conv[i] = i < nl ? static_cast<char*>(pools[l0 + i].conv) : nullptr;
    }
    compact_kernel<<<dim3(pieces, n, nl), kCompactThreads, 0, stream>>>(p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gdn
