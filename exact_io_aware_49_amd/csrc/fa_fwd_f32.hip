// fa_fwd_f32.hip -- exact-attention forward in float32 (vector ALU) for gfx950.
//
// Same tiled, online-softmax scheme as the bf16 kernel ("FlashAttention (DE)",
// sections "Tiling und blockweise Verarbeitung" and "Online-Softmax-Berechnung"),
// but every product and sum is a float32 FMA so the result stays within float32
// rounding of the exact value.  This path serves small float32 problems; it is
// latency-bound rather than throughput-bound, so it favours simplicity.
//
// One workgroup (4 waves) owns 4 ROWS query rows, ROWS per wave.  Per K/V tile
// of 64 keys: lane j of a wave computes the ROWS scores of key j against its
// wave's rows (Q rows are LDS broadcasts, K row j is a padded LDS row), the row
// maxima are wave reductions, P goes through a small per-wave LDS buffer, and
// each lane accumulates output columns (lane, lane + 64) of its rows.  A wave
// walks its rows one after the other, so few rows per wave (many workgroups)
// suit small problems: ROWS is 1, 2 or 4, the smallest that keeps the grid at
// or below 512 workgroups (4 beyond).  Each row's arithmetic is the same for any
// ROWS, so the results do not depend on it.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int F_BC = 64;  // keys per tile

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <int D, bool CAUSAL, int ROWS>
__global__ void __launch_bounds__(256)
fa_fwd_f32_kernel(const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
                  float *__restrict__ O, float *__restrict__ LSE, int N, int group, float scale) {
  constexpr int F_ROWS = ROWS;     // query rows per wave
  constexpr int F_BR = 4 * ROWS;  // query rows per workgroup
  constexpr int KS = D + 4;  // padded K row (floats)
  constexpr int CPL = D / 64;  // output columns per lane
  __shared__ __align__(16) float Qs[F_BR * D];
  __shared__ __align__(16) float Ks[F_BC * KS];
  __shared__ __align__(16) float Vs[F_BC * D];
  __shared__ __align__(16) float Ps[4 * F_ROWS * F_BC];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nqb = (N + F_BR - 1) / F_BR;
  const int bh = blockIdx.x / nqb;
  const int qb = blockIdx.x % nqb;
  const size_t head_off = (size_t)bh * N * D;           // query head: Q, O
  const size_t kv_off = (size_t)(bh / group) * N * D;   // its K/V head (group query heads share one)
  const int q0 = qb * F_BR;
  const int qw0 = q0 + wave * F_ROWS;

  // Q tile -> LDS (rows beyond N are zero)
  for (int e = tid; e < F_BR * D / 4; e += 256) {
    const int r = e / (D / 4), c4 = e % (D / 4);
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    if (q0 + r < N) v = *reinterpret_cast<const floatx4 *>(Q + head_off + (size_t)(q0 + r) * D + 4 * c4);
    *reinterpret_cast<floatx4 *>(Qs + r * D + 4 * c4) = v;
  }

  float m[F_ROWS], lp[F_ROWS], acc[F_ROWS][CPL];
#pragma unroll
  for (int i = 0; i < F_ROWS; ++i) {
    m[i] = -INFINITY;
    lp[i] = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[i][c] = 0.f;
  }

  int ntiles = (N + F_BC - 1) / F_BC;
  if (CAUSAL) ntiles = min(ntiles, (min(q0 + F_BR, N) - 1) / F_BC + 1);

  for (int t = 0; t < ntiles; ++t) {
    const int kb = t * F_BC;
    __syncthreads();  // previous tile fully consumed
    for (int e = tid; e < F_BC * D / 4; e += 256) {
      const int r = e / (D / 4), c4 = e % (D / 4);
      floatx4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (kb + r < N) {
        kv = *reinterpret_cast<const floatx4 *>(K + kv_off + (size_t)(kb + r) * D + 4 * c4);
        vv = *reinterpret_cast<const floatx4 *>(V + kv_off + (size_t)(kb + r) * D + 4 * c4);
      }
      *reinterpret_cast<floatx4 *>(Ks + r * KS + 4 * c4) = kv;
      *reinterpret_cast<floatx4 *>(Vs + r * D + 4 * c4) = vv;
    }
    __syncthreads();

    if (CAUSAL && kb > qw0 + F_ROWS - 1) continue;  // whole tile above this wave's rows

    // scores of key (kb + lane) against the wave's F_ROWS (1, 2 or 4) rows
    float s[F_ROWS];
#pragma unroll
    for (int i = 0; i < F_ROWS; ++i) s[i] = 0.f;
    for (int c = 0; c < D; c += 4) {
      const floatx4 kv = *reinterpret_cast<const floatx4 *>(Ks + lane * KS + c);
#pragma unroll
      for (int i = 0; i < F_ROWS; ++i) {
        const floatx4 qv = *reinterpret_cast<const floatx4 *>(Qs + (wave * F_ROWS + i) * D + c);
        s[i] = __builtin_fmaf(qv[0], kv[0], s[i]);
        s[i] = __builtin_fmaf(qv[1], kv[1], s[i]);
        s[i] = __builtin_fmaf(qv[2], kv[2], s[i]);
        s[i] = __builtin_fmaf(qv[3], kv[3], s[i]);
      }
    }
    const int key = kb + lane;
    float *Pw = Ps + wave * F_ROWS * F_BC;
#pragma unroll
    for (int i = 0; i < F_ROWS; ++i) {
      float x = s[i] * scale;
      if (key >= N || (CAUSAL && key > qw0 + i)) x = -INFINITY;
      const float mt = wave_max(x);
      const float mn = fmaxf(m[i], mt);
      const float alpha = (m[i] == -INFINITY) ? 0.f : expf(m[i] - mn);
      const float p = (mn == -INFINITY) ? 0.f : expf(x - mn);
      m[i] = (mn == -INFINITY) ? m[i] : mn;
      lp[i] = lp[i] * alpha + p;
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[i][c] *= alpha;
      Pw[i * F_BC + lane] = p;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    for (int j = 0; j < F_BC; j += 4) {
      float vv[4][CPL];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int c = 0; c < CPL; ++c) vv[u][c] = Vs[(j + u) * D + lane + 64 * c];
#pragma unroll
      for (int i = 0; i < F_ROWS; ++i) {
        const floatx4 pv = *reinterpret_cast<const floatx4 *>(Pw + i * F_BC + j);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          acc[i][c] = __builtin_fmaf(pv[0], vv[0][c], acc[i][c]);
          acc[i][c] = __builtin_fmaf(pv[1], vv[1][c], acc[i][c]);
          acc[i][c] = __builtin_fmaf(pv[2], vv[2][c], acc[i][c]);
          acc[i][c] = __builtin_fmaf(pv[3], vv[3][c], acc[i][c]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
  }

#pragma unroll
  for (int i = 0; i < F_ROWS; ++i) {
    const int row = qw0 + i;
    const float l = wave_sum(lp[i]);
    if (row < N) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) O[head_off + (size_t)row * D + lane + 64 * c] = acc[i][c] / l;
      if (lane == 0) LSE[(size_t)bh * N + row] = m[i] + logf(l);
    }
  }
}

template <int D, bool CAUSAL, int ROWS>
hipError_t launch_rows(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int group,
                       int N, float scale, hipStream_t stream) {
  const long long blocks = (long long)((N + 4 * ROWS - 1) / (4 * ROWS)) * B * H;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fa_fwd_f32_kernel<D, CAUSAL, ROWS>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const float *)q, (const float *)k, (const float *)v, (float *)o, lse, N, group, scale);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int group,
                  int N, float scale, hipStream_t stream) {
  // smallest rows-per-wave whose grid stays at or below 512 workgroups
  // (measured: B1 H2 N128 d64 29 -> 6 us with 1 row; B2 H4 N1024 d128 best at 4)
  const long long bh = (long long)B * H;
  if (bh * ((N + 3) / 4) <= 512) return launch_rows<D, CAUSAL, 1>(q, k, v, o, lse, B, H, group, N, scale, stream);
  if (bh * ((N + 7) / 8) <= 512) return launch_rows<D, CAUSAL, 2>(q, k, v, o, lse, B, H, group, N, scale, stream);
  return launch_rows<D, CAUSAL, 4>(q, k, v, o, lse, B, H, group, N, scale, stream);
}

}  // namespace

hipError_t launch_fwd_f32(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                          int group, int N, int d, bool causal, float scale, hipStream_t stream) {
  if (d == 64) return causal ? launch<64, true>(q, k, v, o, lse, B, H, group, N, scale, stream)
                             : launch<64, false>(q, k, v, o, lse, B, H, group, N, scale, stream);
  return causal ? launch<128, true>(q, k, v, o, lse, B, H, group, N, scale, stream)
                : launch<128, false>(q, k, v, o, lse, B, H, group, N, scale, stream);
}

}  // namespace fa
