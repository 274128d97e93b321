// fa_internal.h -- host-side launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>

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

// Attention of Nq query rows against a key/value cache (fa_decode).  A
// segment is one block of up to 32 query rows (the (query head, query) pairs
// of one K/V head's group) of one sequence.  The decode kernel runs at most
// kDecodeMaxWaves waves, each over an equal share of the list of 32-key tiles
// of all segments, and writes a float32 partial result per (wave w, segment s)
// pair it touches at slot w + s (distinct for every pair, below
// kDecodeMaxWaves + segments).  Workspace layout (each part 256-byte aligned):
// partial O [slots][rpb][d], partial lse [slots][rpb], and per segment the
// first and last wave that handled it (int32 pairs).
constexpr long long kDecodeMaxWaves = 2048;

struct DecodePlan {
  int nrb;                // blocks of 32 query rows per (sequence, K/V head)
  int rpb;                // rows stored per partial: min(32, group * Nq)
  long long segments;     // B * Hkv * nrb
  size_t lpart_offset;    // byte offsets in the workspace
  size_t segw_offset;
  size_t bytes;           // workspace size
};
inline DecodePlan decode_plan(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
  (void)Nk;
  DecodePlan p;
  const long long rows = (long long)(Hq / Hkv) * Nq;
  p.nrb = (int)((rows + 31) / 32);
  p.rpb = (int)(rows < 32 ? rows : 32);
  p.segments = (long long)B * Hkv * p.nrb;
  const size_t slots = (size_t)kDecodeMaxWaves + (size_t)p.segments;
  auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t obytes = align(slots * (size_t)p.rpb * (size_t)d * sizeof(float));
  const size_t lbytes = align(slots * (size_t)p.rpb * sizeof(float));
  p.lpart_offset = obytes;
  p.segw_offset = obytes + lbytes;
  p.bytes = p.segw_offset + align(2 * (size_t)p.segments * sizeof(int));
  return p;
}

// Compute units of the current device (looked up once per device; 256 if the
// query fails).
int cu_count();

// Round length for map_block_balanced: a causal grid of `blocks` workgroups of
// `kernel` that the device holds all at once (at most the kernel's resident
// workgroups per CU times the CU count, and whole rounds over the 8 XCDs) gets
// its XCD's CU count; any other grid gets 0 (map_block's order).  `per_cu`
// caches the kernel's resident workgroups per CU (0 = not looked up yet).
template <typename Kernel>
int snake_round(Kernel kernel, int threads, long long blocks, std::atomic<int> &per_cu) {
  int r = per_cu.load(std::memory_order_relaxed);
  if (r == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&r, kernel, threads, 0) != hipSuccess || r < 1) r = 1;
    per_cu.store(r, std::memory_order_relaxed);
  }
  const int cus = cu_count();
  if (cus % 8 != 0 || blocks % 8 != 0 || blocks > (long long)r * cus) return 0;
  return cus / 8;
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
                              void *ws, int B, int Hq, int Hkv, int Nq, int Nk, int d, bool causal, float scale,
                              hipStream_t stream);

}  // namespace fa
