// Device-side check of a device-resident slot index (the counterpart of the
// host checks made when a call is given slot_idx_host): every entry is either
// negative (a padding row) or in [0, num_slots), and no non-negative slot is
// named twice.  Two launches, both capturable in a graph: the first sets the
// result to "valid", the second compares every pair of rows through LDS
// tiles and records a violation with atomics.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int kSlotTile = 256;

__global__ __launch_bounds__(64) void slots_init_kernel(int32_t* result) {
  if (threadIdx.x == 0) {
    result[0] = GDN_OK;
    result[1] = 0x7fffffff;
  }
}

// One workgroup per tile pair (I, J), J >= I, of 256 rows each: thread t
// takes row i = 256 I + t and compares its slot with every row j > i of
// block J (tile I itself also range-checks its rows).  A violation at row j
// (a slot out of range, or one that an earlier row already names) lowers
// result[1] to j and sets result[0].
__global__ __launch_bounds__(kSlotTile) void slots_check_kernel(const int32_t* slot, int B,
                                                                int num_slots, int nb,
                                                                int32_t* result) {
  __shared__ int32_t sj[kSlotTile];
  // tile pair from the linear block id: row I holds nb - I pairs
  long long rem = blockIdx.x;
  int I = 0;
  while (rem >= nb - I) {
    rem -= nb - I;
    ++I;
  }
  const int J = I + (int)rem;
  const int t = threadIdx.x;
  const int j_load = J * kSlotTile + t;
  sj[t] = j_load < B ? slot[j_load] : -1;
  __syncthreads();
  const int i = I * kSlotTile + t;
  if (i >= B) return;
  const int si = slot[i];
  int bad = 0x7fffffff;
  if (I == J && si >= num_slots) bad = i;
  if (si >= 0) {
    const int j0 = J * kSlotTile;
    const int jn = min(kSlotTile, B - j0);
    for (int q = 0; q < jn; ++q)
      if (j0 + q > i && sj[q] == si) {
        bad = min(bad, j0 + q);
        break;   // the first repeat of row i's slot in this tile
      }
  }
  if (bad != 0x7fffffff) {
    atomicMin(&result[1], bad);
    __hip_atomic_store(&result[0], (int32_t)GDN_E_SLOT, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

hipError_t launch_check_slots(const int32_t* slot, int B, int num_slots, int32_t* result,
                              hipStream_t stream) {
  slots_init_kernel<<<1, 64, 0, stream>>>(result);
  if (B > 0) {
    const long long nb = (B + kSlotTile - 1) / kSlotTile;
    const long long pairs = nb * (nb + 1) / 2;
    slots_check_kernel<<<dim3((unsigned)pairs), kSlotTile, 0, stream>>>(slot, B, num_slots,
                                                                       (int)nb, result);
  }
  return hipGetLastError();
}

}  // namespace gdn
