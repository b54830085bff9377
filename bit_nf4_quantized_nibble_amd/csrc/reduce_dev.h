// reduce_dev.h -- the reduction of the skinny rank-product kernel's per-slice
// partial sums, as a device function of the workgroup index, so that it can run
// in its own launch (lora.hip) or ride on another launch of the same workgroup
// size (the dequantize kernels, quant.hip).  RedJob / RedJobs are in common.h.
#pragma once

#include "common.h"

namespace qnf4 {

// Reductions of per-slice partial sums (see SkRed), one thread per element of a
// rows x width grid (rows: P, or ldt with a transposed output; width: R, or ldcd
// with a padded cd output); workgroups [0, nblk of job 0) take job 0, the next
// nblk of job 1 job 1, and so on.  32-bit indexing (the launcher checks the sizes).
template <int CD>
__device__ __forceinline__ void skreduce_block(const RedJobs& js, uint32_t blk) {
  int w = 0;
  uint32_t b = blk;
#pragma unroll
  for (int k = 0; k < kRedJobs - 1; ++k)
    if (w == k && b >= js.j[k].nblk) {
      b -= js.j[k].nblk;
      w = k + 1;
    }
  const RedJob& j = js.j[w];
  const uint32_t idx = b * kRedThreads + threadIdx.x;
  if (idx >= j.rows * j.width) return;
  const uint32_t pr = idx / j.width, t = idx - pr * j.width;
  if (pr >= j.P) {  // zero columns P .. ldt-1 of the transposed copies
    if (t < j.R) {
      if (j.outt) store_cd<CD>(j.outt, (int64_t)(t * j.ldt + pr), 0.f);
      if (j.side_t) store_cd<CD>(j.side_t, (int64_t)(t * j.ldt + pr), 0.f);
    }
    return;
  }
  if (t >= j.R) {  // width > R only with a padded cd output
    store_cd<CD>(j.outcd, (int64_t)(pr * j.ldcd + t), 0.f);
    return;
  }
  // slices in groups of 8, every load of a group issued before its first add
  // (slices past S read slice 0 and are dropped; without a side input the side load
  // reads the first partial sum); the sum runs in slice order
  const float sv = *(j.side ? j.side + pr * j.R + t : j.part);
  float sum = 0.f;
  for (int z0 = 0; z0 < (int)j.S; z0 += 8) {  // S <= kRedMaxS
    float v[8];
#pragma unroll
    for (int z = 0; z < 8; ++z)
      v[z] = j.part[((uint32_t)(z0 + z < (int)j.S ? z0 + z : 0) * j.P + pr) * kRedBR + t];
#pragma unroll
    for (int z = 0; z < 8; ++z) sum += z0 + z < (int)j.S ? v[z] : 0.f;
  }
  if (j.out32) j.out32[j.trans ? t * j.P + pr : pr * j.R + t] = sum * j.sc32;
  if (j.outcd) store_cd<CD>(j.outcd, (int64_t)(pr * j.ldcd + t), sum * j.sccd);
  if (j.outt) store_cd<CD>(j.outt, (int64_t)(t * j.ldt + pr), sum * j.sccd);
  if (j.side_t) store_cd<CD>(j.side_t, (int64_t)(t * j.ldt + pr), sv);
}

}  // namespace qnf4
