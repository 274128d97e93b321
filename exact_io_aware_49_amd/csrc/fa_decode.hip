// fa_decode.hip -- attention of a few new query rows against a key/value cache.
//
// The serving case of the pages' "Spezialisierte Lösungen" ("FlashAttention
// (DE)", section "Evolution und Weiterentwicklungen": FlashInfer streams the
// KV cache during generation).  Nq query rows per sequence (the last Nq
// positions) attend to the first L_b rows of the sequence's cache.  With
// little query work per byte of cache, the kernel is bound by reading K and V
// once from HBM, so the cache is split into key ranges spread over many
// waves, and a second kernel merges the partial results with the online-
// softmax rule (lse = ln sum_s e^lse_s, O = sum_s e^(lse_s - lse) O_s).
//
// fa_decode_kernel: one wave per (batch, K/V head, block of 32 query rows,
// key range).  The rows of a block are the (query head, query) pairs of the
// K/V head's group, so grouped heads share each K/V byte.  The four waves of
// a workgroup are independent (no barriers): each streams its own 32-key K
// and V tiles into its own double-buffered LDS area with buffer_load ... lds,
// computes S^T = K Q^T and O^T += V^T P^T on bf16 matrix cores exactly as the
// forward does, and writes a float32 (O, lse) partial for its key range.
// fa_decode_merge_kernel: one workgroup per query row.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

template <int D>
struct DecCfg {
  static constexpr int BC = 32;              // keys per tile
  static constexpr int KSTEPS = D / 16;      // MFMA k-steps over the head dim
  static constexpr int CT = D / 32;          // 32-column output tiles
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int RB = 2 * D;           // bytes per row
  static constexpr int RPI = 1024 / RB;      // rows per wave-wide 16-byte load
  static constexpr int TB = BC * RB;         // bytes per tile
  static constexpr int LPT = TB / 1024;      // wave-wide loads per tile and tensor
  static constexpr int WAVE_LDS = 4 * TB;    // K0, K1, V0, V1
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256)
fa_decode_kernel(const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K, const __bf16 *__restrict__ V,
                 const int *__restrict__ kv_lens, float *__restrict__ Opart, float *__restrict__ Lpart, int Hq,
                 int Hkv, int Nq, int Nk, int nrb, int nsplit, int chunk, long long nwaves, float scale_log2e) {
  using C = DecCfg<D>;
  constexpr int TB = C::TB;
  constexpr int RB = C::RB;
  __shared__ __align__(1024) unsigned char smem[4 * C::WAVE_LDS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const long long wid = (long long)blockIdx.x * 4 + wave;
  if (wid >= nwaves) return;  // the waves share no barrier
  // wid = ((b * Hkv + hk) * nrb + rb) * nsplit + split
  const int split = (int)(wid % nsplit);
  long long rest = wid / nsplit;
  const int rb = (int)(rest % nrb);
  rest /= nrb;
  const int hk = (int)(rest % Hkv);
  const int b = (int)(rest / Hkv);
  const int group = Hq / Hkv;

  int len = kv_lens ? kv_lens[b] : Nk;
  len = min(max(len, 0), Nk);
  const int k0 = split * chunk;
  const int k1 = min(k0 + chunk, len);
  const int ntiles = (k1 > k0) ? (k1 - k0 + C::BC - 1) / C::BC : 0;

  // this lane's query row: (query head g of the group, query i)
  const int row = rb * 32 + l32;
  const bool row_ok = row < group * Nq;
  const int g = row_ok ? row / Nq : 0;
  const int qi = row_ok ? row - g * Nq : 0;
  const int hq = hk * group + g;
  const long long orow = ((long long)b * Hq + hq) * Nq + qi;  // output row
  const int pos = len - Nq + qi;                             // the query's position in the sequence

  bf16x8 qf[C::KSTEPS];
  {
    const __bf16 *qrow = Q + orow * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks)
      qf[ks] = as_bf16x8(row_ok ? ld16(qrow + 16 * ks) : u32x4{0, 0, 0, 0});
  }

  unsigned char *wl = smem + wave * C::WAVE_LDS;  // this wave's K0, K1, V0, V1
  const size_t kv_off = ((size_t)b * Hkv + hk) * (size_t)Nk * D;
  const uint32_t head_bytes = (uint32_t)Nk * RB;  // rows past the cache read as zero
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + kv_off, head_bytes);
  const int ld_row = lane / C::CPR;
  const int ld_chunk = lane % C::CPR;
  auto issue = [&](int t, int buf) {
    const int r0 = k0 + t * C::BC;
#pragma unroll
    for (int u = 0; u < C::LPT; ++u) {
      const int row0 = u * C::RPI;
      const int r = row0 + ld_row;
      load_lds16(krs, wl + buf * TB + row0 * RB, (uint32_t)(r0 + r) * RB + 16u * (ld_chunk ^ swz_k<D>(r)));
      load_lds16(vrs, wl + (2 + buf) * TB + row0 * RB, (uint32_t)(r0 + r) * RB + 16u * (ld_chunk ^ swz_v<D>(r)));
    }
  };

  // per-lane LDS addresses: score A operand (K row swap_bits23(l32), chunk 2 ks + half)
  // and transposed V reads (as in the forward)
  const uint32_t wbase = lds_addr(wl);
  uint32_t kaddr[C::KSTEPS];
  {
    const int r = swap_bits23(l32);
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) kaddr[ks] = wbase + r * RB + 16 * ((2 * ks + half) ^ swz_k<D>(r));
  }
  uint32_t vaddr[C::CT][2];
  {
    const int rlo = 8 * half + ((lane & 15) >> 2);
    const int tq = lane & 3;
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
      const int ch = 4 * ct + 2 * ((lane >> 4) & 1) + (tq >> 1);
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int r = rlo + 4 * hi;
        vaddr[ct][hi] = wbase + 2 * TB + r * RB + 16 * (ch ^ swz_v<D>(r)) + 8 * (tq & 1);
      }
    }
  }

  floatx16 oacc[C::CT];
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) oacc[ct] = floatx16{0};
  float m_run = -INFINITY;  // running maximum of the raw scores of this row
  float l_part = 0.f;       // this lane's part of the exponential sum

  auto tile = [&](auto bufc, int t) {
    constexpr int BUF = decltype(bufc)::value;
    if (t + 1 < ntiles) {
      issue(t + 1, BUF ^ 1);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * C::LPT) : "memory");  // tile t has landed
    } else {
      wait_vmem();
    }
    // S^T of the 32 keys of tile t: lane = query row, registers = keys
    floatx16 s = floatx16{0};
    {
      u32x4 a[C::KSTEPS];
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) a[ks] = ds_read_b128_at<BUF * TB>(kaddr[ks]);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) {
        redefine(a[ks]);
        s = mfma32x32x16(as_bf16x8(a[ks]), qf[ks], s);
      }
    }
    const int kb = k0 + t * C::BC;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kb + 16 * (r >> 3) + 8 * half + (r & 7);
      if (key >= k1 || (CAUSAL && key > pos)) s[r] = -INFINITY;
    }
    float mloc = max3f(s[0], s[1], s[2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) mloc = max3f(mloc, s[r], s[r + 1]);
    mloc = fmaxf(mloc, s[15]);
    // (uniform across the wave: a row that has seen no visible key yet has
    // m = -inf, gets alpha = 0 and P = 0, and keeps O = 0, l = 0)
    const float m_new = fmaxf(m_run, max_with_partner(mloc));
    const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2((m_run - m_new) * scale_log2e);
    l_part *= alpha;
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[ct][r] *= alpha;
    m_run = m_new;
    const float mc = (m_new == -INFINITY) ? 0.f : m_new * scale_log2e;
    static_for<2>([&](auto mcc) {
      constexpr int M = decltype(mcc)::value;  // keys 16 M .. 16 M + 15 of the tile
      u32x4 pw;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = fast_exp2(__builtin_fmaf(s[8 * M + 2 * i], scale_log2e, -mc));
        const float p1 = fast_exp2(__builtin_fmaf(s[8 * M + 2 * i + 1], scale_log2e, -mc));
        pw[i] = pack_bf16x2(p0, p1);
        l_part = add_bf16_pair(pw[i], l_part);
      }
      constexpr int OFF = BUF * TB + 16 * M * RB;
#pragma unroll
      for (int ct = 0; ct < C::CT; ++ct) {
        u32x2 lo = ds_read_tr16_at<OFF>(vaddr[ct][0]);
        u32x2 hi = ds_read_tr16_at<OFF>(vaddr[ct][1]);
        lds_wait(lo, hi);
        const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
        oacc[ct] = mfma32x32x16(as_bf16x8(av), as_bf16x8(pw), oacc[ct]);
      }
    });
  };

  if (ntiles > 0) issue(0, 0);
  for (int t = 0; t < ntiles; t += 2) {
    tile(std::integral_constant<int, 0>{}, t);
    if (t + 1 < ntiles) tile(std::integral_constant<int, 1>{}, t + 1);
  }

  // partial result of this key range: O normalised by its own sum, lse in natural log
  const float l_tot = sum_with_partner(l_part);
  if (row_ok) {
    const bool any = l_tot > 0.f;
    const float inv = any ? 1.f / l_tot : 0.f;
    float *op = Opart + (orow * nsplit + split) * D;
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const floatx4 w = {oacc[ct][4 * j] * inv, oacc[ct][4 * j + 1] * inv, oacc[ct][4 * j + 2] * inv,
                           oacc[ct][4 * j + 3] * inv};
        *reinterpret_cast<floatx4 *>(op + 32 * ct + 8 * j + 4 * half) = w;
      }
    if (half == 0) Lpart[orow * nsplit + split] = any ? (m_run * scale_log2e + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// Merge the nsplit partials of each query row: lse = m + ln sum_s e^(lse_s - m),
// O = sum_s e^(lse_s - lse) O_s.  A row no split saw gets O = 0, lse = -inf.
// One workgroup per row: the weights go through LDS, then each thread sums
// 8 columns over a strided subset of the splits and the subsets are added in
// a fixed order, so the result is bitwise reproducible.
template <int D>
__global__ void __launch_bounds__(256)
fa_decode_merge_kernel(const float *__restrict__ Opart, const float *__restrict__ Lpart, __bf16 *__restrict__ O,
                       float *__restrict__ LSE, int nsplit) {
  constexpr int C8 = D / 8;          // 8-column chunks per row
  constexpr int SG = 256 / C8;       // split groups
  __shared__ float red[256];
  __shared__ floatx4 part[SG][C8][2];
  const int tid = threadIdx.x;
  const long long row = blockIdx.x;
  const float *lp = Lpart + row * nsplit;
  // ---- maximum and sum of e^(lse_s - m) over the splits
  float m = -INFINITY;
  for (int s = tid; s < nsplit; s += 256) m = fmaxf(m, lp[s]);
  red[tid] = m;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  m = red[0];
  __syncthreads();
  float sum = 0.f;
  if (m != -INFINITY)
    for (int s = tid; s < nsplit; s += 256) sum += expf(lp[s] - m);
  red[tid] = sum;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  sum = red[0];
  // ---- weighted sum of the partial rows
  const int c8 = tid % C8;
  const int sg = tid / C8;
  floatx4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
  if (m != -INFINITY) {
    for (int s = sg; s < nsplit; s += SG) {
      const float w = expf(lp[s] - m);
      const float *op = Opart + (row * nsplit + s) * D + 8 * c8;
      a += w * *reinterpret_cast<const floatx4 *>(op);
      b += w * *reinterpret_cast<const floatx4 *>(op + 4);
    }
  }
  part[sg][c8][0] = a;
  part[sg][c8][1] = b;
  __syncthreads();
  if (tid < C8) {
    floatx4 ta = {0, 0, 0, 0}, tb = {0, 0, 0, 0};
    for (int g = 0; g < SG; ++g) {
      ta += part[g][tid][0];
      tb += part[g][tid][1];
    }
    if (m != -INFINITY) {
      ta /= sum;
      tb /= sum;
    }
    const u32x4 w = {pack_bf16x2(ta[0], ta[1]), pack_bf16x2(ta[2], ta[3]), pack_bf16x2(tb[0], tb[1]),
                     pack_bf16x2(tb[2], tb[3])};
    *reinterpret_cast<u32x4 *>(O + row * D + 8 * tid) = w;
    if (tid == 0) LSE[row] = (m == -INFINITY) ? -INFINITY : m + logf(sum);
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const void *q, const void *k, const void *v, const int *kv_lens, void *o, float *lse, float *ws,
                  int B, int Hq, int Hkv, int Nq, int Nk, float scale, hipStream_t stream) {
  const DecodePlan p = decode_plan(B, Hq, Hkv, Nq, Nk, D);
  float *opart = ws;
  float *lpart = ws + p.lpart_offset_floats;
  const long long blocks = (p.nwaves + 3) / 4;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fa_decode_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, kv_lens, opart, lpart, Hq, Hkv, Nq,
                     Nk, p.nrb, p.nsplit, p.chunk, p.nwaves, scale * kLog2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long nrows = (long long)B * Hq * Nq;
  if (nrows > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fa_decode_merge_kernel<D>), dim3((unsigned)nrows), dim3(256), 0, stream,
                     (const float *)opart, (const float *)lpart, (__bf16 *)o, lse, p.nsplit);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const void *q, const void *k, const void *v, const int *kv_lens, void *o, float *lse,
                              float *ws, int B, int Hq, int Hkv, int Nq, int Nk, int d, bool causal, float scale,
                              hipStream_t stream) {
  if (d == 64)
    return causal ? launch<64, true>(q, k, v, kv_lens, o, lse, ws, B, Hq, Hkv, Nq, Nk, scale, stream)
                  : launch<64, false>(q, k, v, kv_lens, o, lse, ws, B, Hq, Hkv, Nq, Nk, scale, stream);
  return causal ? launch<128, true>(q, k, v, kv_lens, o, lse, ws, B, Hq, Hkv, Nq, Nk, scale, stream)
                : launch<128, false>(q, k, v, kv_lens, o, lse, ws, B, Hq, Hkv, Nq, Nk, scale, stream);
}

}  // namespace fa
