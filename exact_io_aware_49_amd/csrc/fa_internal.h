// fa_internal.h -- host-side launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

// Each launcher enqueues its kernels on `stream` and returns hipGetLastError().
// Arguments are already validated by the C ABI layer.
hipError_t launch_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                           int N, int d, bool causal, float scale, hipStream_t stream);
hipError_t launch_fwd_f32(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                          int N, int d, bool causal, float scale, hipStream_t stream);
hipError_t launch_bwd_bf16(const void *q, const void *k, const void *v, const void *o, const void *dout,
                           const float *lse, void *dq, void *dk, void *dv, float *dsum, int B, int H, int N,
                           int d, bool causal, float scale, hipStream_t stream);

}  // namespace fa
