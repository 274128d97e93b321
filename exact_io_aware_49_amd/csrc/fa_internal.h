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

// Attention of Nq query rows against a key/value cache (fa_decode): one wave
// per (batch, K/V head, block of 32 query rows, key range of `chunk` keys);
// the key range is split until there are about 2048 waves (at least 256 keys
// each; 2048 long ranges beat 4096 shorter ones by 15% at B=16, 8 K/V heads,
// an 8K cache: fewer partials to merge and less start-up per wave).  The workspace holds float32 partial O [B*Hq*Nq][nsplit][d] and,
// 256-byte aligned after it, partial lse [B*Hq*Nq][nsplit].
struct DecodePlan {
  int nrb;                      // blocks of 32 query rows per (batch, K/V head)
  int nsplit;                   // key ranges per row block
  int chunk;                    // keys per range (multiple of 32)
  long long nwaves;
  size_t lpart_offset_floats;   // start of the lse partials in the workspace
  size_t bytes;                 // workspace size
};
inline DecodePlan decode_plan(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
  DecodePlan p;
  const long long rows = (long long)(Hq / Hkv) * Nq;
  p.nrb = (int)((rows + 31) / 32);
  const long long base = (long long)B * Hkv * p.nrb;
  long long s = (2048 + base - 1) / base;
  const long long most = ((long long)Nk + 255) / 256;
  if (s > most) s = most;
  if (s < 1) s = 1;
  const long long chunk = (((long long)Nk + s - 1) / s + 31) / 32 * 32;
  s = ((long long)Nk + chunk - 1) / chunk;
  p.nsplit = (int)s;
  p.chunk = (int)chunk;
  p.nwaves = base * s;
  const size_t nrows = (size_t)B * (size_t)Hq * (size_t)Nq;
  const size_t obytes = nrows * (size_t)s * (size_t)d * sizeof(float);
  p.lpart_offset_floats = ((obytes + 255) & ~(size_t)255) / sizeof(float);
  p.bytes = (p.lpart_offset_floats * sizeof(float) + nrows * (size_t)s * sizeof(float) + 255) & ~(size_t)255;
  return p;
}

// Each launcher enqueues its kernels on `stream` and returns hipGetLastError().
// Arguments are already validated by the C ABI layer.  H is the number of
// query heads; `group` query heads share one K/V head (H / group K/V heads).
hipError_t launch_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                           int group, int N, int d, bool causal, float scale, hipStream_t stream);
hipError_t launch_fwd_bf16_r64(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                               int group, int N, bool causal, float scale, hipStream_t stream);
hipError_t launch_fwd_fp8(const void *q, const void *k, const void *v, float q_scale, float k_scale, float v_scale,
                          void *o, float *lse, int B, int H, int group, int N, int d, bool causal, float scale,
                          hipStream_t stream);
hipError_t launch_fwd_f32(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                          int group, int N, int d, bool causal, float scale, hipStream_t stream);
hipError_t launch_bwd_bf16(const void *q, const void *k, const void *v, const void *o, const void *dout,
                           const float *lse, void *dq, void *dk, void *dv, float *dsum, int B, int H, int group,
                           int N, int d, bool causal, float scale, hipStream_t stream);

hipError_t launch_decode_bf16(const void *q, const void *k, const void *v, const int *kv_lens, void *o, float *lse,
                              float *ws, int B, int Hq, int Hkv, int Nq, int Nk, int d, bool causal, float scale,
                              hipStream_t stream);

}  // namespace fa
