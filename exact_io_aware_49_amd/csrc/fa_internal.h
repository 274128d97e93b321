// fa_internal.h -- host-side launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

// Backward with query heads sharing K/V heads: the workgroups that own a block
// of 128 keys run over every query head of the group.  When there are too few
// such blocks to fill the GPU (B * Hkv * ceil(N/128) below 512), the group's
// query heads are split over up to `group` workgroups per key block; each
// writes float32 partial dK/dV and a reduction kernel sums them.
inline int bwd_splits(long long nkvh, int N, int group) {
  const long long blocks = nkvh * (((long long)N + 127) / 128);
  long long s = (512 + blocks - 1) / blocks;
  if (s > group) s = group;
  if (s < 1) s = 1;
  return (int)s;
}
// float offset of the partial area in the workspace (after D and lse*log2e,
// rounded up to 256 bytes)
inline size_t bwd_partial_offset_floats(long long nqh, int N) {
  const size_t bytes = 2 * (size_t)nqh * (size_t)N * sizeof(float);
  return ((bytes + 255) & ~(size_t)255) / sizeof(float);
}

// Each launcher enqueues its kernels on `stream` and returns hipGetLastError().
// Arguments are already validated by the C ABI layer.  H is the number of
// query heads; `group` query heads share one K/V head (H / group K/V heads).
hipError_t launch_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                           int group, int N, int d, bool causal, float scale, hipStream_t stream);
hipError_t launch_fwd_f32(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                          int group, int N, int d, bool causal, float scale, hipStream_t stream);
hipError_t launch_bwd_bf16(const void *q, const void *k, const void *v, const void *o, const void *dout,
                           const float *lse, void *dq, void *dk, void *dv, float *dsum, int B, int H, int group,
                           int N, int d, bool causal, float scale, hipStream_t stream);

}  // namespace fa
