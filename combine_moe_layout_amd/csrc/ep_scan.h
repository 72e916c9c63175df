// ep_scan.h -- a workgroup-wide exclusive scan over an LDS array, shared by the
// one-launch layout kernels (ep_fused.hip, ep_group.hip).
#pragma once
#include "ep_device.h"

namespace ep {

// Exclusive scan of n <= EP_MAX_EXPERTS values in LDS (in place into out),
// returning the total; every thread of the block calls it (the block is whole
// waves).  Its two barriers also order any LDS writes made before the call.
__device__ __forceinline__ int32_t block_exclusive_scan(const int32_t* in, int32_t* out, int n,
                                                      int32_t* s_wave) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int waves = (blockDim.x + kWave - 1) / kWave;
  const int per = (n + blockDim.x - 1) / blockDim.x;
  const int first = tid * per;
  int32_t mine = 0;
  for (int i = 0; i < per; ++i)
    if (first + i < n) mine += in[first + i];
  const int32_t incl = wave_inclusive_sum(mine);
  if (lane == kWave - 1) s_wave[wave] = incl;
  __syncthreads();
  int32_t before = 0, total = 0;
  for (int w = 0; w < waves; ++w) {
    before += w < wave ? s_wave[w] : 0;
    total += s_wave[w];
  }
  int32_t run = before + incl - mine;
  for (int i = 0; i < per; ++i) {
    if (first + i < n) {
      const int32_t v = in[first + i];
      out[first + i] = run;
      run += v;
    }
  }
  __syncthreads();
  return total;
}

}  // namespace ep
