// fa_api.cpp -- the C ABI of libfa.so: argument validation and dispatch.
//
// Every argument is checked before any HIP call, so a rejected call enqueues
// nothing and touches no device state.  The launchers behind this layer live in
// the .hip files; they report launch errors via hipGetLastError, mapped here to
// FA_ERR_HIP.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cmath>
#include <mutex>

#include "fa.h"
#include "fa_internal.h"

namespace {

constexpr int kVersion = 10000;  // 1.0.0

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_common(int B, int H, int N, int d, int causal, float scale, int dtype) {
  if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED_DTYPE;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_BAD_SHAPE;
  if (d != 32 && d != 64 && d != 96 && d != 128 && d != 256) return FA_ERR_UNSUPPORTED_HEAD_DIM;
  // head dims 32, 96 and 256: bf16 only
  if ((d == 32 || d == 96 || d == 256) && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED_HEAD_DIM;
  // B*H*N rows must stay below 2^55 (so B*H*N*d < 2^62), and the launch grids
  // (at most one workgroup per 64 rows of each head) must fit in 2^31 - 1.
  const unsigned long long bh = (unsigned long long)B * (unsigned long long)H;
  if (bh > (1ull << 55) / (unsigned long long)N) return FA_ERR_BAD_SHAPE;
  if (bh * (((unsigned long long)N + 63) / 64) > 0x7fffffffull) return FA_ERR_BAD_SHAPE;
  // one head's [N, d] slab is addressed through 32-bit buffer offsets
  const unsigned long long esize = (dtype == FA_DTYPE_F32) ? 4ull : 2ull;
  if ((unsigned long long)N * (unsigned long long)d * esize >= (1ull << 31)) return FA_ERR_BAD_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_BAD_ARGUMENT;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_BAD_SCALE;
  return FA_OK;
}

// Hq query heads over Hkv >= 1 K/V heads in contiguous groups
int check_heads(int Hq, int Hkv) {
  if (Hkv < 1 || Hq < 1 || Hq % Hkv != 0) return FA_ERR_BAD_SHAPE;
  return FA_OK;
}

// Decode: Nq query rows of B*Hq heads against a [B, Hkv, Nk, d] cache
int check_decode(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale, int dtype) {
  if (dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED_DTYPE;
  if (B < 1 || Nq < 1 || Nk < 1) return FA_ERR_BAD_SHAPE;
  if (check_heads(Hq, Hkv) != FA_OK) return FA_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
  const unsigned long long lim = 1ull << 55;
  if ((unsigned long long)B * (unsigned long long)Hkv > lim / (unsigned long long)Nk) return FA_ERR_BAD_SHAPE;
  if ((unsigned long long)B * (unsigned long long)Hq > lim / (unsigned long long)Nq) return FA_ERR_BAD_SHAPE;
  if ((unsigned long long)Nk * (unsigned long long)d * 2ull >= (1ull << 31)) return FA_ERR_BAD_SHAPE;
  if ((unsigned long long)Hq / Hkv * (unsigned long long)Nq > 0x7fffffffull) return FA_ERR_BAD_SHAPE;
  const fa::DecodePlan p = fa::decode_plan(B, Hq, Hkv, Nq, Nk, d);
  if (p.segments > (1LL << 30)) return FA_ERR_BAD_SHAPE;               // segment numbers (and pairs) fit in int32
  if ((long long)B * Hq * Nq > 0x7fffffffLL) return FA_ERR_BAD_SHAPE;  // up to one merge workgroup per query row
  if (causal != 0 && causal != 1) return FA_ERR_BAD_ARGUMENT;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_BAD_SCALE;
  return FA_OK;
}

// ---- static scratch for fa_bwd_noalloc -----------------------------------
// The backward's per-row workspace (D and lse * log2 e, two float32 per query
// row) for callers that cannot allocate.  Every GPU the library runs on holds
// its own copy of this array until the process ends.  Host code never passes
// the array's name to a kernel: it is a host-side stand-in, not a device
// address.  Its device address is looked up once per device with
// hipGetSymbolAddress and kept in scratch_ptr.
constexpr size_t kScratchBytes = size_t(16) << 20;  // 16 MiB: up to 2^21 query rows
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> scratch_ptr[kMaxDevices];
std::mutex scratch_mutex;

// Device address of `scratch` on the current device, or nullptr if the lookup
// failed (or the device index is out of range).
void *scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void *p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  p = scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

namespace fa {

// Compute units of the current device, looked up once per device.
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace fa

extern "C" {

int fa_version(void) { return kVersion; }

const char *fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL_POINTER: return "FA_ERR_NULL_POINTER: a required pointer is NULL";
    case FA_ERR_BAD_SHAPE: return "FA_ERR_BAD_SHAPE: B, H and N must be >= 1, the tensor size must fit, and the query heads must split evenly over the K/V heads";
    case FA_ERR_UNSUPPORTED_HEAD_DIM: return "FA_ERR_UNSUPPORTED_HEAD_DIM: head dim d must be 64 or 128 (also 32, 96, 256 for the bf16 forward and backward, 256 for the FP8 forward)";
    case FA_ERR_UNSUPPORTED_DTYPE: return "FA_ERR_UNSUPPORTED_DTYPE: dtype not supported by this entry point";
    case FA_ERR_BAD_SCALE: return "FA_ERR_BAD_SCALE: scale must be finite and > 0";
    case FA_ERR_MISALIGNED: return "FA_ERR_MISALIGNED: tensor pointers must be 16-byte aligned";
    case FA_ERR_WORKSPACE_TOO_SMALL: return "FA_ERR_WORKSPACE_TOO_SMALL: workspace missing or below fa_bwd_workspace_size()";
    case FA_ERR_BAD_ARGUMENT: return "FA_ERR_BAD_ARGUMENT: causal must be 0 or 1";
    case FA_ERR_HIP: return "FA_ERR_HIP: a HIP launch or runtime call failed";
    case FA_ERR_SCRATCH_TOO_SMALL: return "FA_ERR_SCRATCH_TOO_SMALL: fa_bwd_noalloc needs more than its 16 MiB static scratch (B*H*N above 2^21)";
    default: return "unknown fa status code";
  }
}

int fa_fwd_gqa(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq, int Hkv, int N,
               int d, int causal, float scale, int dtype, void *stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_POINTER;
  int st = check_common(B, Hq, N, d, causal, scale, dtype);
  if (st == FA_OK) st = check_heads(Hq, Hkv);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_MISALIGNED;
  const int group = Hq / Hkv;
  hipError_t e;
  if (dtype == FA_DTYPE_BF16)
    e = fa::launch_fwd_bf16(q, k, v, o, lse, B, Hq, group, N, d, causal == 1, scale, (hipStream_t)stream);
  else
    e = fa::launch_fwd_f32(q, k, v, o, lse, B, Hq, group, N, d, causal == 1, scale, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int N, int d,
           int causal, float scale, int dtype, void *stream) {
  return fa_fwd_gqa(q, k, v, o, lse, B, H, H, N, d, causal, scale, dtype, stream);
}

int fa_fwd_fp8(const void *q, const void *k, const void *v, float q_scale, float k_scale, float v_scale, void *o,
               float *lse, int B, int Hq, int Hkv, int N, int d, int causal, float scale, void *stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_POINTER;
  int st = check_common(B, Hq, N, d, causal, scale, FA_DTYPE_BF16);
  if (st == FA_OK) st = check_heads(Hq, Hkv);
  if (st != FA_OK) return st;
  if (d != 64 && d != 128 && d != 256) return FA_ERR_UNSUPPORTED_HEAD_DIM;
  for (float x : {q_scale, k_scale, v_scale})
    if (!std::isfinite(x) || !(x > 0.f)) return FA_ERR_BAD_SCALE;
  const float c = q_scale * k_scale * scale;
  if (!std::isnormal(c) || !std::isnormal(c * 1.4426950408889634f)) return FA_ERR_BAD_SCALE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_MISALIGNED;
  hipError_t e = fa::launch_fwd_fp8(q, k, v, q_scale, k_scale, v_scale, o, lse, B, Hq, Hq / Hkv, N, d, causal == 1,
                                    scale, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_gqa_workspace_size(int B, int Hq, int Hkv, int N, int d, int dtype) {
  if (check_common(B, Hq, N, d, 0, 1.0f, dtype) != FA_OK || check_heads(Hq, Hkv) != FA_OK ||
      dtype != FA_DTYPE_BF16)
    return 0;
  // D_i and lse_i * log2(e), one float32 each per query row; with the query
  // heads of a group split over several workgroups, float32 partial dK and dV
  // per split
  const long long nqh = (long long)B * Hq;
  const long long nkvh = (long long)B * Hkv;
  size_t bytes = fa::bwd_partial_offset_floats(nqh, N) * sizeof(float);
  const int nsplit = fa::bwd_splits(nkvh, N, Hq / Hkv);
  if (nsplit > 1) bytes += 2 * (size_t)nsplit * (size_t)nkvh * (size_t)N * (size_t)d * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d, int dtype) {
  return fa_bwd_gqa_workspace_size(B, H, H, N, d, dtype);
}

int fa_bwd_gqa(const void *q, const void *k, const void *v, const void *o, const void *dout, const float *lse,
               void *dq, void *dk, void *dv, void *workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
               int N, int d, int causal, float scale, int dtype, void *stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL_POINTER;
  int st = check_common(B, Hq, N, d, causal, scale, dtype);
  if (st == FA_OK) st = check_heads(Hq, Hkv);
  if (st != FA_OK) return st;
  if (dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED_DTYPE;
  const size_t need = fa_bwd_gqa_workspace_size(B, Hq, Hkv, N, d, dtype);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(lse) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace))
    return FA_ERR_MISALIGNED;
  hipError_t e = fa::launch_bwd_bf16(q, k, v, o, dout, lse, dq, dk, dv, (float *)workspace, B, Hq, Hq / Hkv, N,
                                     d, causal == 1, scale, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout, const float *lse,
           void *dq, void *dk, void *dv, void *workspace, size_t workspace_bytes, int B, int H, int N, int d,
           int causal, float scale, int dtype, void *stream) {
  return fa_bwd_gqa(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, H, N, d, causal, scale,
                    dtype, stream);
}

size_t fa_bwd_noalloc_scratch_bytes(void) { return kScratchBytes; }

int fa_bwd_noalloc(const void *q, const void *k, const void *v, const void *o, const void *dout, const float *lse,
                   void *dq, void *dk, void *dv, int B, int H, int N, int d, int causal, float scale, int dtype,
                   void *stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL_POINTER;
  int st = check_common(B, H, N, d, causal, scale, dtype);
  if (st != FA_OK) return st;
  if (dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED_DTYPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(lse) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_MISALIGNED;
  // one query head per K/V head: the workspace is D and lse * log2 e only
  if (fa_bwd_gqa_workspace_size(B, H, H, N, d, dtype) > kScratchBytes) return FA_ERR_SCRATCH_TOO_SMALL;
  void *ws = scratch_on_current_device();
  if (!ws) return FA_ERR_HIP;
  hipError_t e = fa::launch_bwd_bf16(q, k, v, o, dout, lse, dq, dk, dv, (float *)ws, B, H, 1, N, d, causal == 1,
                                     scale, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_decode_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d, int dtype) {
  if (check_decode(B, Hq, Hkv, Nq, Nk, d, 0, 1.0f, dtype) != FA_OK) return 0;
  return fa::decode_plan(B, Hq, Hkv, Nq, Nk, d).bytes;
}

int fa_decode(const void *q, const void *k, const void *v, const int *kv_lens, void *o, float *lse, void *workspace,
              size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
              int dtype, void *stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_POINTER;
  int st = check_decode(B, Hq, Hkv, Nq, Nk, d, causal, scale, dtype);
  if (st != FA_OK) return st;
  const size_t need = fa::decode_plan(B, Hq, Hkv, Nq, Nk, d).bytes;
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) || !aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(kv_lens) & 3u) != 0)
    return FA_ERR_MISALIGNED;
  hipError_t e = fa::launch_decode_bf16(q, k, v, kv_lens, o, lse, workspace, B, Hq, Hkv, Nq, Nk, d,
                                        causal == 1, scale, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
