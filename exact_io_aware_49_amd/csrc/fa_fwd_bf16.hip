// fa_fwd_bf16.hip -- fused exact-attention forward for bf16 on gfx950 matrix cores.
//
// What is computed: O = softmax(scale * Q K^T) V and lse = ln sum_j exp(scale q_i.k_j)
// ("FlashAttention (DE)", section "Problematik der Standard-Attention").  How:
// the IO-aware scheme of sections "Tiling und blockweise Verarbeitung",
// "Online-Softmax-Berechnung" and "Zusammenfassen von Operationen in einem
// CUDA-Kernel": one workgroup owns a block of query rows, keeps them in
// registers, streams K/V tiles through LDS, updates a running row maximum and
// exponential sum per row, and writes only O and lse.  The N x N scores never
// leave registers.
//
// Mapping to one workgroup (4 waves, 256 threads), BR = 128 query rows:
//   * Each wave owns 32 query rows.  Its Q rows sit in VGPRs as the B operand
//     of S^T = K Q^T (lane = query row, 8 consecutive head-dim slots per lane).
//   * A K/V tile of BC keys (BC = 64 for d = 128, 128 for d = 64) is staged per
//     iteration: K row-major in LDS (padded rows), V transposed in LDS so that
//     the values of one head-dim column for consecutive keys are contiguous.
//     Staging is double-buffered: the global loads of tile j+1 are issued before
//     tile j is computed and land in LDS after it.
//   * S^T tiles (32 keys x 32 queries) are computed with v_mfma_f32_32x32x16_bf16.
//     The result leaves each lane holding one query row and 16 of its keys per
//     tile; the other 16 sit in the lane 32 away.  The row maximum therefore
//     needs one cross-half exchange per tile.
//   * P = 2^(S c - m c) with c = scale * log2(e) (one FMA + one v_exp_f32 per
//     score), rounded to bf16, is directly the B operand of O^T += V^T P^T, so P
//     never touches LDS.  O^T accumulates in registers: lane = query row.
//   * The running maximum is only moved when the tile maximum exceeds it by more
//     than 2^8 in exp2 units.  Both O and the exponential sum are expressed
//     relative to the same reference, so the final O / l is unchanged; values
//     stay below 2^8 times the row sum, far from float32 overflow.
//   * Causal: tiles entirely above the diagonal are never loaded; a wave whose
//     rows are all above a tile skips its math; only diagonal and ragged tiles
//     pay for masking.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

template <int D>
struct FwdCfg {
  static constexpr int BR = 128;                  // query rows per workgroup
  static constexpr int BC = (D == 128) ? 64 : 128; // keys per tile
  static constexpr int NKT = BC / 32;             // 32-key score tiles per K/V tile
  static constexpr int KSTEPS = D / 16;           // MFMA k-steps over the head dim
  static constexpr int CT = D / 32;               // 32-column output tiles
  static constexpr int KSTRIDE = D + 8;           // bf16 elements per K row in LDS
  static constexpr int VSTRIDE = BC + 8;          // bf16 elements per V^T row in LDS
  static constexpr int KTILE = BC * KSTRIDE;      // bf16 elements per K buffer
  static constexpr int VTILE = D * VSTRIDE;       // bf16 elements per V^T buffer
  static constexpr int KVEC = BC * D / 8 / 256;   // 16-byte K vectors per thread per tile (= 4)
  static constexpr int KQUADS = BC / 4;           // 4-key groups for the V transpose
};

// Map the linear workgroup id to (batch*head, query block).  Workgroups are
// dispatched round-robin over the 8 XCDs; grouping consecutive ids of one XCD
// onto the same heads keeps a head's K/V in that XCD's L2.  Causal launches
// run the heaviest query blocks (most key tiles) first.
__device__ __forceinline__ void map_block(int bid, int nqb, int nbh, bool causal, int &bh, int &qb) {
  const int total = nqb * nbh;
  int id = bid;
  if ((total & 7) == 0) {
    const int per_xcd = total >> 3;
    id = (bid & 7) * per_xcd + (bid >> 3);
  }
  if (causal) {
    // within each XCD's contiguous range, order by descending query block
    const int per_xcd = ((total & 7) == 0) ? (total >> 3) : total;
    const int base = (id / per_xcd) * per_xcd;
    const int local = id - base;
    // heads covered by this range (per_xcd is a multiple of nqb when nbh % 8 == 0)
    if (per_xcd % nqb == 0) {
      const int heads_here = per_xcd / nqb;
      const int qrank = local / heads_here;
      bh = base / nqb + (local % heads_here);
      qb = nqb - 1 - qrank;
      return;
    }
    bh = id / nqb;
    qb = nqb - 1 - (id % nqb);
    return;
  }
  bh = id / nqb;
  qb = id % nqb;
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 2)
fa_fwd_bf16_kernel(const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K,
                   const __bf16 *__restrict__ V, __bf16 *__restrict__ O, float *__restrict__ LSE,
                   int N, int nbh, float scale_log2e, float scale) {
  using C = FwdCfg<D>;
  __shared__ __align__(16) __bf16 smem[2 * (C::KTILE + C::VTILE)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int nqb = (N + C::BR - 1) / C::BR;
  int bh, qb;
  map_block(blockIdx.x, nqb, nbh, CAUSAL, bh, qb);

  const size_t head_off = (size_t)bh * (size_t)N * D;
  const __bf16 *Qh = Q + head_off;
  const __bf16 *Kh = K + head_off;
  const __bf16 *Vh = V + head_off;

  const int q0 = qb * C::BR;              // first query row of the workgroup
  const int qw0 = q0 + wave * 32;         // first query row of this wave
  const int my_q = qw0 + l32;             // this lane's query row

  // ---- Q fragments: B operand, lane = query row, slots = d in [16*ks + 8*half, +8)
  bf16x8 qf[C::KSTEPS];
  {
    const bool ok = my_q < N;
    const __bf16 *qrow = Qh + (size_t)(ok ? my_q : 0) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      u32x4 v = ok ? ld16(qrow + 16 * ks) : u32x4{0, 0, 0, 0};
      qf[ks] = as_bf16x8(v);
    }
  }

  // ---- number of key tiles this workgroup visits
  const int ntiles_all = (N + C::BC - 1) / C::BC;
  int ntiles = ntiles_all;
  if (CAUSAL) {
    const int last_q = min(q0 + C::BR, N) - 1;
    ntiles = min(ntiles_all, last_q / C::BC + 1);
  }

  // ---- staging helpers: thread t owns KVEC K vectors and one 4x8 V block per tile
  const int k_g = tid % (D / 8);          // 16-byte column group of K
  const int k_r = tid / (D / 8);          // first K row; rows k_r + (256/(D/8))*u
  constexpr int K_ROWSTEP = 256 / (D / 8);
  const int v_kq = tid % C::KQUADS;       // key quad of V
  const int v_g = tid / C::KQUADS;        // 8-wide head-dim group of V

  u32x4 kreg[C::KVEC];
  u32x4 vreg[4];

  auto load_tile = [&](int t) {
    const int kb = t * C::BC;
#pragma unroll
    for (int u = 0; u < C::KVEC; ++u) {
      const int r = kb + k_r + K_ROWSTEP * u;
      kreg[u] = (r < N) ? ld16(Kh + (size_t)r * D + 8 * k_g) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = kb + 4 * v_kq + u;
      vreg[u] = (r < N) ? ld16(Vh + (size_t)r * D + 8 * v_g) : u32x4{0, 0, 0, 0};
    }
  };

  auto store_tile = [&](int buf) {
    __bf16 *Ks = smem + buf * (C::KTILE + C::VTILE);
    __bf16 *Vt = Ks + C::KTILE;
#pragma unroll
    for (int u = 0; u < C::KVEC; ++u) st16(Ks + (k_r + K_ROWSTEP * u) * C::KSTRIDE + 8 * k_g, kreg[u]);
    // 4 keys x 8 columns -> 8 rows of V^T, 4 keys each (8 bytes)
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      // column 2p (low halves) and 2p+1 (high halves) of the four key rows
      const uint32_t a0 = vreg[0][p], a1 = vreg[1][p], a2 = vreg[2][p], a3 = vreg[3][p];
      u32x2 lo, hi;
      lo[0] = __builtin_amdgcn_perm(a1, a0, 0x05040100u);
      lo[1] = __builtin_amdgcn_perm(a3, a2, 0x05040100u);
      hi[0] = __builtin_amdgcn_perm(a1, a0, 0x07060302u);
      hi[1] = __builtin_amdgcn_perm(a3, a2, 0x07060302u);
      st8(Vt + (8 * v_g + 2 * p) * C::VSTRIDE + 4 * v_kq, lo);
      st8(Vt + (8 * v_g + 2 * p + 1) * C::VSTRIDE + 4 * v_kq, hi);
    }
  };

  floatx16 oacc[C::CT];
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) oacc[ct] = floatx16{0};
  float m_ref = -INFINITY;  // running maximum of raw scores (q.k, unscaled)
  float l_part = 0.f;       // this lane's part of the running exponential sum

  load_tile(0);
  store_tile(0);
  __syncthreads();

  // A-operand row for the score tile: K row swap_bits23(l32) of each 32-key tile
  const int krow_perm = swap_bits23(l32);

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const bool prefetch = (t + 1) < ntiles;
    if (prefetch) load_tile(t + 1);

    const int kb = t * C::BC;
    const bool wave_active = !CAUSAL || (kb <= qw0 + 31);
    if (wave_active) {
      const __bf16 *Ks = smem + buf * (C::KTILE + C::VTILE);
      const __bf16 *Vt = Ks + C::KTILE;

      // ---- S^T = K Q^T for NKT tiles of 32 keys
      floatx16 s[C::NKT];
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt) {
        s[kt] = floatx16{0};
        const __bf16 *krow = Ks + (32 * kt + krow_perm) * C::KSTRIDE + 8 * half;
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
          bf16x8 a = as_bf16x8(ld16(krow + 16 * ks));
          s[kt] = mfma32x32x16(a, qf[ks], s[kt]);
        }
      }

      // ---- masking (diagonal and ragged tiles only)
      const bool need_mask = (CAUSAL && (kb + C::BC - 1 > qw0)) || (kb + C::BC > N);
      if (need_mask) {
#pragma unroll
        for (int kt = 0; kt < C::NKT; ++kt) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb + 32 * kt + 16 * (r >> 3) + 8 * half + (r & 7);
            const bool hide = (key >= N) || (CAUSAL && key > my_q);
            if (hide) s[kt][r] = -INFINITY;
          }
        }
      }

      // ---- row maximum of this tile (lane holds 16*NKT keys, partner lane the rest)
      float mloc = s[0][0];
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, s[kt][r]);
      const float m_tile = fmaxf(mloc, swap_halves(mloc));
      const float m_new = fmaxf(m_ref, m_tile);

      // ---- move the reference maximum only when the scores outgrow it by > 2^8
      const bool grow = (m_new - m_ref) * scale_log2e > 8.0f;
      if (__ballot(grow) != 0) {
        const float alpha = (m_ref == -INFINITY) ? 0.f : fast_exp2((m_ref - m_new) * scale_log2e);
        m_ref = (m_new == -INFINITY) ? m_ref : m_new;
        l_part *= alpha;
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[ct][r] *= alpha;
      }
      const float mc = (m_ref == -INFINITY) ? 0.f : m_ref * scale_log2e;

      // ---- P = 2^(S c - m c), its row sum, and O^T += V^T P^T
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          float p[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            p[i] = fast_exp2(__builtin_fmaf(s[kt][8 * m + i], scale_log2e, -mc));
            l_part += p[i];
          }
          const bf16x8 pb = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
          const int key_off = 32 * kt + 16 * m + 8 * half;
#pragma unroll
          for (int ct = 0; ct < C::CT; ++ct) {
            bf16x8 a = as_bf16x8(ld16(Vt + (32 * ct + l32) * C::VSTRIDE + key_off));
            oacc[ct] = mfma32x32x16(a, pb, oacc[ct]);
          }
        }
      }
    }

    if (prefetch) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, lse = (m c + log2 l) ln 2
  const float l_tot = l_part + swap_halves(l_part);
  if (my_q < N) {
    const float inv = 1.f / l_tot;
    __bf16 *orow = O + head_off + (size_t)my_q * D;
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[ct][4 * g + 0] * inv, oacc[ct][4 * g + 1] * inv);
        w[1] = pack_bf16x2(oacc[ct][4 * g + 2] * inv, oacc[ct][4 * g + 3] * inv);
        st8(orow + 32 * ct + 8 * g + 4 * half, w);
      }
    }
    if (half == 0) {
      LSE[(size_t)bh * N + my_q] = (m_ref * scale_log2e + __log2f(l_tot)) * kLn2;
    }
  }
  (void)scale;
}

template <int D, bool CAUSAL>
hipError_t launch(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int N,
                  float scale, hipStream_t stream) {
  using C = FwdCfg<D>;
  const int nbh = B * H;
  const int nqb = (N + C::BR - 1) / C::BR;
  const long long blocks = (long long)nqb * nbh;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, (__bf16 *)o, lse, N, nbh,
                     scale * kLog2e, scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                           int N, int d, bool causal, float scale, hipStream_t stream) {
  if (d == 64) return causal ? launch<64, true>(q, k, v, o, lse, B, H, N, scale, stream)
                             : launch<64, false>(q, k, v, o, lse, B, H, N, scale, stream);
  return causal ? launch<128, true>(q, k, v, o, lse, B, H, N, scale, stream)
                : launch<128, false>(q, k, v, o, lse, B, H, N, scale, stream);
}

}  // namespace fa
