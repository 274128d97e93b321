// fa_bwd_bf16.hip -- exact-attention backward with recomputation, bf16 on gfx950.
//
// Training keeps only the per-row log-sum-exp from the forward and recomputes
// the score blocks here (Dutch glossary page "FlashAttention", section
// "Hoe werkt het?", bullet "Herberekening").  The gradients are the calculus of
// the attention equation ("FlashAttention (DE)", section "Problematik der
// Standard-Attention") for L = sum(dO * O):
//   P = exp(scale S - lse),  dV = P^T dO,  dP = dO V^T,  D_i = dO_i . O_i,
//   dS = P (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Two kernels, no atomics:
//   fa_bwd_dq_kernel   -- owns 128 query rows (32 per wave).  Computes D for its
//                         rows (stored for the second kernel), then streams K/V
//                         tiles: S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T.
//                         Lane = query row, so lse and D are per-lane scalars.
//   fa_bwd_dkdv_kernel -- owns 128 keys (32 per wave), K and V rows held in
//                         registers.  Streams query tiles: S = Q K^T, dP = dO V^T,
//                         dS, dV^T += dO^T P, dK^T += Q^T dS.  Lane = key.
// The second product of each kernel needs its streamed operand transposed
// (K^T, dO^T, Q^T); those copies are written to LDS by the staging threads,
// with the 4x8 register transpose of fa_device.h.  P and dS go straight from
// the accumulator registers of the first products into the B operand of the
// second ones (row order fixed by swap_bits23), so they never touch LDS.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

// ============================================================== dQ kernel
template <int D>
struct DqCfg {
  static constexpr int BR = 128;              // query rows per workgroup
  static constexpr int BC = 64;               // keys per tile
  static constexpr int NKT = BC / 32;
  static constexpr int KSTEPS = D / 16;
  static constexpr int CT = D / 32;
  static constexpr int RSTRIDE = D + 8;       // K and V rows in LDS
  static constexpr int TSTRIDE = BC + 8;      // K^T rows in LDS
  static constexpr int KT_ELEMS = BC * RSTRIDE;
  static constexpr int KTT_ELEMS = D * TSTRIDE;
  static constexpr int STAGE = 2 * KT_ELEMS + KTT_ELEMS;
  static constexpr int UNITS = (BC / 4) * (D / 8);  // 4x8 blocks per operand tile
  static constexpr int MINW = (D == 64) ? 2 : 1;
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256, DqCfg<D>::MINW)
fa_bwd_dq_kernel(const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K, const __bf16 *__restrict__ V,
                 const __bf16 *__restrict__ Og, const __bf16 *__restrict__ dO, const float *__restrict__ LSE,
                 __bf16 *__restrict__ dQ, float *__restrict__ Dsum, int N, float scale_log2e, float scale) {
  using C = DqCfg<D>;
  __shared__ __align__(16) __bf16 smem[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int nqb = (N + C::BR - 1) / C::BR;
  const int bh = blockIdx.x % (gridDim.x / nqb);
  const int qb = CAUSAL ? (nqb - 1 - blockIdx.x / (gridDim.x / nqb)) : (blockIdx.x / (gridDim.x / nqb));
  const size_t head_off = (size_t)bh * N * D;
  const int q0 = qb * C::BR;
  const int qw0 = q0 + 32 * wave;
  const int my_q = qw0 + l32;
  const bool q_ok = my_q < N;

  // ---- Q and dO rows as B operands; D_i = dO_i . O_i from the same slots
  bf16x8 qf[C::KSTEPS], dof[C::KSTEPS];
  float dpart = 0.f;
  {
    const size_t roff = head_off + (size_t)(q_ok ? my_q : 0) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      const u32x4 z = {0, 0, 0, 0};
      const u32x4 qv = q_ok ? ld16(Q + roff + 16 * ks) : z;
      const u32x4 dv = q_ok ? ld16(dO + roff + 16 * ks) : z;
      const u32x4 ov = q_ok ? ld16(Og + roff + 16 * ks) : z;
      qf[ks] = as_bf16x8(qv);
      dof[ks] = as_bf16x8(dv);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        dpart = __builtin_fmaf(bf16lo_to_f32(dv[w]), bf16lo_to_f32(ov[w]), dpart);
        dpart = __builtin_fmaf(bf16hi_to_f32(dv[w]), bf16hi_to_f32(ov[w]), dpart);
      }
    }
  }
  const float drow = sum_with_partner(dpart);
  const float lse2 = q_ok ? LSE[(size_t)bh * N + my_q] * kLog2e : 0.f;
  if (q_ok && half == 0) Dsum[(size_t)bh * N + my_q] = drow;

  int ntiles = (N + C::BC - 1) / C::BC;
  if (CAUSAL) ntiles = min(ntiles, (min(q0 + C::BR, N) - 1) / C::BC + 1);

  // ---- staging: K unit (rows + transposed) and V unit (rows) per thread
  const bool do_k = (C::UNITS == 256) || (tid < 128);
  const bool do_v = (C::UNITS == 256) || (tid >= 128);
  const int unit = (C::UNITS == 256) ? tid : (tid & 127);
  const int u_kq = unit % (C::BC / 4);
  const int u_g = unit / (C::BC / 4);
  const __bf16 *Kh = K + head_off;
  const __bf16 *Vh = V + head_off;
  u32x4 kblk[4], vblk[4];

  auto load_tile = [&](int t) {
    const int kb = t * C::BC;
    if (do_k) load_block4x8(kblk, Kh, kb + 4 * u_kq, N, D, u_g);
    if (do_v) load_block4x8(vblk, Vh, kb + 4 * u_kq, N, D, u_g);
  };
  auto store_tile = [&](int buf) {
    __bf16 *Ks = smem + buf * C::STAGE;
    __bf16 *Vs = Ks + C::KT_ELEMS;
    __bf16 *KTs = Vs + C::KT_ELEMS;
    if (do_k) {
      store_block_rows(Ks, C::RSTRIDE, 4 * u_kq, u_g, kblk);
      store_block_transposed(KTs, C::TSTRIDE, 4 * u_kq, u_g, kblk);
    }
    if (do_v) store_block_rows(Vs, C::RSTRIDE, 4 * u_kq, u_g, vblk);
  };

  floatx16 dqacc[C::CT];
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) dqacc[ct] = floatx16{0};

  load_tile(0);
  store_tile(0);
  __syncthreads();
  const int arow = swap_bits23(l32);

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const bool prefetch = (t + 1) < ntiles;
    if (prefetch) load_tile(t + 1);
    const int kb = t * C::BC;
    if (!CAUSAL || kb <= qw0 + 31) {
      const __bf16 *Ks = smem + buf * C::STAGE;
      const __bf16 *Vs = Ks + C::KT_ELEMS;
      const __bf16 *KTs = Vs + C::KT_ELEMS;
      floatx16 s[C::NKT], dp[C::NKT];
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt) {
        s[kt] = floatx16{0};
        dp[kt] = floatx16{0};
        const __bf16 *krow = Ks + (32 * kt + arow) * C::RSTRIDE + 8 * half;
        const __bf16 *vrow = Vs + (32 * kt + arow) * C::RSTRIDE + 8 * half;
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
          s[kt] = mfma32x32x16(as_bf16x8(ld16(krow + 16 * ks)), qf[ks], s[kt]);
          dp[kt] = mfma32x32x16(as_bf16x8(ld16(vrow + 16 * ks)), dof[ks], dp[kt]);
        }
      }
      const bool need_mask = (CAUSAL && (kb + C::BC - 1 > qw0)) || (kb + C::BC > N);
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          float d8[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int r = 8 * m + i;
            float p = fast_exp2(__builtin_fmaf(s[kt][r], scale_log2e, -lse2));
            if (need_mask) {
              const int key = kb + 32 * kt + 16 * m + 8 * half + i;
              if (key >= N || (CAUSAL && key > my_q)) p = 0.f;
            }
            d8[i] = p * (dp[kt][r] - drow);
          }
          const bf16x8 dsb = to_bf16x8(d8[0], d8[1], d8[2], d8[3], d8[4], d8[5], d8[6], d8[7]);
          const int key_off = 32 * kt + 16 * m + 8 * half;
#pragma unroll
          for (int ct = 0; ct < C::CT; ++ct) {
            const bf16x8 a = as_bf16x8(ld16(KTs + (32 * ct + l32) * C::TSTRIDE + key_off));
            dqacc[ct] = mfma32x32x16(a, dsb, dqacc[ct]);
          }
        }
      }
    }
    if (prefetch) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (q_ok) {
    __bf16 *row = dQ + head_off + (size_t)my_q * D;
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack_bf16x2(dqacc[ct][4 * g + 0] * scale, dqacc[ct][4 * g + 1] * scale);
        w[1] = pack_bf16x2(dqacc[ct][4 * g + 2] * scale, dqacc[ct][4 * g + 3] * scale);
        st8(row + 32 * ct + 8 * g + 4 * half, w);
      }
    }
  }
}

// ============================================================== dK/dV kernel
template <int D>
struct DkvCfg {
  static constexpr int BKV = 128;             // keys per workgroup
  static constexpr int BQ = 64;               // query rows per tile
  static constexpr int NQT = BQ / 32;
  static constexpr int KSTEPS = D / 16;
  static constexpr int CT = D / 32;
  static constexpr int RSTRIDE = D + 8;       // Q and dO rows in LDS
  static constexpr int TSTRIDE = BQ + 8;      // Q^T and dO^T rows in LDS
  static constexpr int R_ELEMS = BQ * RSTRIDE;
  static constexpr int T_ELEMS = D * TSTRIDE;
  static constexpr int STAGE = 2 * R_ELEMS + 2 * T_ELEMS + 2 * BQ * 2;  // + lse, D as float
  static constexpr int UNITS = (BQ / 4) * (D / 8);
  static constexpr int MINW = (D == 64) ? 2 : 1;
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256, DkvCfg<D>::MINW)
fa_bwd_dkdv_kernel(const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K, const __bf16 *__restrict__ V,
                   const __bf16 *__restrict__ dO, const float *__restrict__ LSE,
                   const float *__restrict__ Dsum, __bf16 *__restrict__ dK, __bf16 *__restrict__ dV, int N,
                   float scale_log2e, float scale) {
  using C = DkvCfg<D>;
  __shared__ __align__(16) __bf16 smem[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int nkb = (N + C::BKV - 1) / C::BKV;
  const int nbh = gridDim.x / nkb;
  const int bh = blockIdx.x % nbh;
  const int kblk = blockIdx.x / nbh;  // ascending: with a causal mask the first blocks have the most work
  const size_t head_off = (size_t)bh * N * D;
  const int kb0 = kblk * C::BKV;
  const int kw0 = kb0 + 32 * wave;
  const int my_k = kw0 + l32;
  const bool k_ok = my_k < N;

  bf16x8 kf[C::KSTEPS], vf[C::KSTEPS];
  {
    const size_t roff = head_off + (size_t)(k_ok ? my_k : 0) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      const u32x4 z = {0, 0, 0, 0};
      kf[ks] = as_bf16x8(k_ok ? ld16(K + roff + 16 * ks) : z);
      vf[ks] = as_bf16x8(k_ok ? ld16(V + roff + 16 * ks) : z);
    }
  }

  const int nqt_all = (N + C::BQ - 1) / C::BQ;
  const int qt0 = CAUSAL ? (kb0 / C::BQ) : 0;

  const bool do_q = (C::UNITS == 256) || (tid < 128);
  const bool do_o = (C::UNITS == 256) || (tid >= 128);
  const int unit = (C::UNITS == 256) ? tid : (tid & 127);
  const int u_kq = unit % (C::BQ / 4);
  const int u_g = unit / (C::BQ / 4);
  const __bf16 *Qh = Q + head_off;
  const __bf16 *dOh = dO + head_off;
  const float *Lh = LSE + (size_t)bh * N;
  const float *Dh = Dsum + (size_t)bh * N;
  u32x4 qblk[4], oblk[4];
  float lsv = 0.f;

  auto load_tile = [&](int t) {
    const int qs = t * C::BQ;
    if (do_q) load_block4x8(qblk, Qh, qs + 4 * u_kq, N, D, u_g);
    if (do_o) load_block4x8(oblk, dOh, qs + 4 * u_kq, N, D, u_g);
    if (tid < C::BQ) {
      const int q = qs + tid;
      lsv = (q < N) ? Lh[q] * kLog2e : INFINITY;  // rows past N get P = 0
    } else if (tid < 2 * C::BQ) {
      const int q = qs + tid - C::BQ;
      lsv = (q < N) ? Dh[q] : 0.f;
    }
  };
  auto store_tile = [&](int buf) {
    __bf16 *Qs = smem + buf * C::STAGE;
    __bf16 *dOs = Qs + C::R_ELEMS;
    __bf16 *QTs = dOs + C::R_ELEMS;
    __bf16 *dOTs = QTs + C::T_ELEMS;
    float *stat = reinterpret_cast<float *>(dOTs + C::T_ELEMS);  // [0, BQ): lse*log2e, [BQ, 2BQ): D
    if (do_q) {
      store_block_rows(Qs, C::RSTRIDE, 4 * u_kq, u_g, qblk);
      store_block_transposed(QTs, C::TSTRIDE, 4 * u_kq, u_g, qblk);
    }
    if (do_o) {
      store_block_rows(dOs, C::RSTRIDE, 4 * u_kq, u_g, oblk);
      store_block_transposed(dOTs, C::TSTRIDE, 4 * u_kq, u_g, oblk);
    }
    if (tid < 2 * C::BQ) stat[tid] = lsv;
  };

  floatx16 dkacc[C::CT], dvacc[C::CT];
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) {
    dkacc[ct] = floatx16{0};
    dvacc[ct] = floatx16{0};
  }

  const int arow = swap_bits23(l32);
  if (qt0 < nqt_all) {
    load_tile(qt0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = qt0; t < nqt_all; ++t) {
    const int buf = (t - qt0) & 1;
    const bool prefetch = (t + 1) < nqt_all;
    if (prefetch) load_tile(t + 1);
    const int qs = t * C::BQ;
    if (!CAUSAL || qs + C::BQ - 1 >= kw0) {
      const __bf16 *Qs = smem + buf * C::STAGE;
      const __bf16 *dOs = Qs + C::R_ELEMS;
      const __bf16 *QTs = dOs + C::R_ELEMS;
      const __bf16 *dOTs = QTs + C::T_ELEMS;
      const float *stat = reinterpret_cast<const float *>(dOTs + C::T_ELEMS);
      const bool need_mask = (CAUSAL && qs < kw0 + 31) || (kb0 + C::BKV > N);
#pragma unroll
      for (int qt = 0; qt < C::NQT; ++qt) {
        floatx16 s = floatx16{0}, dp = floatx16{0};
        const __bf16 *qrow = Qs + (32 * qt + arow) * C::RSTRIDE + 8 * half;
        const __bf16 *orow = dOs + (32 * qt + arow) * C::RSTRIDE + 8 * half;
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
          s = mfma32x32x16(as_bf16x8(ld16(qrow + 16 * ks)), kf[ks], s);
          dp = mfma32x32x16(as_bf16x8(ld16(orow + 16 * ks)), vf[ks], dp);
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int qoff = 32 * qt + 16 * m + 8 * half;  // tile-local query of register 8m
          const floatx4 l0 = *reinterpret_cast<const floatx4 *>(stat + qoff);
          const floatx4 l1 = *reinterpret_cast<const floatx4 *>(stat + qoff + 4);
          const floatx4 d0 = *reinterpret_cast<const floatx4 *>(stat + C::BQ + qoff);
          const floatx4 d1 = *reinterpret_cast<const floatx4 *>(stat + C::BQ + qoff + 4);
          float p8[8], s8[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float lq = (i < 4) ? l0[i] : l1[i - 4];
            const float dq = (i < 4) ? d0[i] : d1[i - 4];
            const int r = 8 * m + i;
            float p = fast_exp2(__builtin_fmaf(s[r], scale_log2e, -lq));
            if (need_mask) {
              const int q = qs + qoff + i;
              if (!k_ok || (CAUSAL && q < my_k)) p = 0.f;
            }
            p8[i] = p;
            s8[i] = p * (dp[r] - dq);
          }
          const bf16x8 pb = to_bf16x8(p8[0], p8[1], p8[2], p8[3], p8[4], p8[5], p8[6], p8[7]);
          const bf16x8 sb = to_bf16x8(s8[0], s8[1], s8[2], s8[3], s8[4], s8[5], s8[6], s8[7]);
#pragma unroll
          for (int ct = 0; ct < C::CT; ++ct) {
            const bf16x8 ao = as_bf16x8(ld16(dOTs + (32 * ct + l32) * C::TSTRIDE + qoff));
            const bf16x8 aq = as_bf16x8(ld16(QTs + (32 * ct + l32) * C::TSTRIDE + qoff));
            dvacc[ct] = mfma32x32x16(ao, pb, dvacc[ct]);
            dkacc[ct] = mfma32x32x16(aq, sb, dkacc[ct]);
          }
        }
      }
    }
    if (prefetch) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (k_ok) {
    __bf16 *krow = dK + head_off + (size_t)my_k * D;
    __bf16 *vrow = dV + head_off + (size_t)my_k * D;
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 wk, wv;
        wk[0] = pack_bf16x2(dkacc[ct][4 * g + 0] * scale, dkacc[ct][4 * g + 1] * scale);
        wk[1] = pack_bf16x2(dkacc[ct][4 * g + 2] * scale, dkacc[ct][4 * g + 3] * scale);
        wv[0] = pack_bf16x2(dvacc[ct][4 * g + 0], dvacc[ct][4 * g + 1]);
        wv[1] = pack_bf16x2(dvacc[ct][4 * g + 2], dvacc[ct][4 * g + 3]);
        st8(krow + 32 * ct + 8 * g + 4 * half, wk);
        st8(vrow + 32 * ct + 8 * g + 4 * half, wv);
      }
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const void *q, const void *k, const void *v, const void *o, const void *dout,
                  const float *lse, void *dq, void *dk, void *dv, float *dsum, int B, int H, int N, float scale,
                  hipStream_t stream) {
  const long long nbh = (long long)B * H;
  const long long gq = nbh * ((N + DqCfg<D>::BR - 1) / DqCfg<D>::BR);
  const long long gk = nbh * ((N + DkvCfg<D>::BKV - 1) / DkvCfg<D>::BKV);
  if (gq > 0x7fffffffLL || gk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const float c = scale * kLog2e;
  hipLaunchKernelGGL((fa_bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)gq), dim3(256), 0, stream,
                     (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, (const __bf16 *)o,
                     (const __bf16 *)dout, lse, (__bf16 *)dq, dsum, N, c, scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)gk), dim3(256), 0, stream,
                     (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, (const __bf16 *)dout, lse,
                     (const float *)dsum, (__bf16 *)dk, (__bf16 *)dv, N, c, scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const void *q, const void *k, const void *v, const void *o, const void *dout,
                           const float *lse, void *dq, void *dk, void *dv, float *dsum, int B, int H, int N,
                           int d, bool causal, float scale, hipStream_t stream) {
  if (d == 64)
    return causal ? launch<64, true>(q, k, v, o, dout, lse, dq, dk, dv, dsum, B, H, N, scale, stream)
                  : launch<64, false>(q, k, v, o, dout, lse, dq, dk, dv, dsum, B, H, N, scale, stream);
  return causal ? launch<128, true>(q, k, v, o, dout, lse, dq, dk, dv, dsum, B, H, N, scale, stream)
                : launch<128, false>(q, k, v, o, dout, lse, dq, dk, dv, dsum, B, H, N, scale, stream);
}

}  // namespace fa
