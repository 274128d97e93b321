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
//   fa_bwd_dq_kernel   -- owns 128 query rows (256 at d = 128; 32 per wave).  Computes D for its
//                         rows and stores D and lse*log2(e) for the second kernel,
//                         then streams K/V tiles of 64 keys:
//                         S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T.
//                         Lane = query row, so lse and D are per-lane scalars.
//   fa_bwd_dkdv_kernel -- (d = 32, 64, 96, 256) owns 128 keys (32 per wave), K and V rows
//                         held in registers.  Streams Q/dO tiles of 64 queries:
//                         S = Q K^T, dP = dO V^T, dS, dV^T += dO^T P, dK^T += Q^T dS.
//                         Lane = key.
//   fa_bwd_dkdv_pair_kernel -- (d = 128) the same work for 128 keys split over
//                         8 waves in pairs that share a SIMD and a 32-key group:
//                         one wave computes S, P and dV (K rows in registers),
//                         its partner dP, dS and dK (V rows in registers), with
//                         P passed through LDS.  One wave per key group would
//                         need about 330 registers at d = 128 (one wave per
//                         SIMD, nothing to hide its latencies); a pair needs
//                         under 256 each, so two waves share every SIMD.
// Streamed tiles go from HBM straight into LDS (buffer_load ... lds, double
// buffered) as row-major tiles whose 16-byte chunks are XOR-permuted per row.
// Each tile is read twice from that single copy: as rows (ds_read_b128, the A
// operand of the first products) and transposed (ds_read_b64_tr_b16, the A
// operand of the second products).  P and dS go straight from the accumulator
// registers of the first products into the B operand of the second ones (row
// order fixed by swap_bits23); only the pair kernel also hands P (float32) to
// the partner wave through LDS.  Masked scores are set to -inf in a pass before
// the exponentials (P = 0 exactly), which keeps the exponential code one
// branch-free block.  At d = 256 the one-wave kernel runs as two launches, one
// for dV and one for dK (one wave cannot hold both accumulators there).
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

template <int D>
struct BwdCfg {
  static constexpr int TROWS = 64;            // rows of a streamed tile
  static constexpr int KSTEPS = D / 16;
  static constexpr int CT = D / 32;
  // LDS rows are DL columns wide: d = 96 sits in a 128-column layout whose last
  // four 16-byte chunks read as zero
  static constexpr int DL = (D == 96) ? 128 : D;
  static constexpr int CPR = DL / 8;          // 16-byte chunks per LDS row
  static constexpr int RB = 2 * DL;           // bytes per LDS row
  static constexpr int RBG = 2 * D;           // bytes per row in global memory
  static constexpr int RPI = 1024 / RB;       // rows per wave-wide 16-byte load
  static constexpr int TB = TROWS * RB;       // bytes per tile
  static constexpr int LPW = TB / 1024 / 4;   // loads per wave per tile
};

// One 64-row tile of a [N, D] head slab (rows r0 .. r0+63) into LDS at `dst`,
// split over the 4 waves; rows past N read as zero.
template <int D, int NW = 4>
__device__ __forceinline__ void issue_tile(__amdgpu_buffer_rsrc_t rs, unsigned char *dst, int r0, int wave,
                                           int lane) {
  using C = BwdCfg<D>;
  constexpr int LPW = C::TB / 1024 / NW;  // loads per wave
#pragma unroll
  for (int u = 0; u < LPW; ++u) {
    const int row0 = (wave * LPW + u) * C::RPI;
    const int row = row0 + lane / C::CPR;
    const int c = (lane % C::CPR) ^ swz_rt<C::DL>(row);
    uint32_t g = (uint32_t)(r0 + row) * C::RBG + 16u * c;
    if constexpr (C::DL != D)
      if (c >= D / 8) g = 0x80000000u;  // padding chunk: past the buffer, reads zero
    load_lds16(rs, dst + row0 * C::RB, g);
  }
}

// Per-lane byte offsets of the two read patterns of a tile.
//  rows : A operand of a 32x32x16 MFMA over 32 tile rows 32*sub + swap_bits23(l32),
//         k-step ks -> logical chunk 2*ks + half.  Add 32*sub*RB for sub-tile `sub`.
//  trans: transposed read (ds_read_b64_tr_b16) of rows 16*ch + 8*half + (l&15)/4 (+4 for
//         the high half), columns 32*ct + 16*((l>>4)&1) + 4*(l&3).  Add 16*ch*RB.
template <int D>
struct TileOffsets {
  int rows[D / 16];
  uint32_t trans[D / 32][2];
  __device__ __forceinline__ void init(int lane, uint32_t trans_base) {
    using C = BwdCfg<D>;
    const int half = lane >> 5;
    const int r = swap_bits23(lane & 31);
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) rows[ks] = r * C::RB + 16 * ((2 * ks + half) ^ swz_rt<C::DL>(r));
    const int rlo = 8 * half + ((lane & 15) >> 2);
    const int tq = lane & 3;
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
      const int ch = 4 * ct + 2 * ((lane >> 4) & 1) + (tq >> 1);
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int rr = rlo + 4 * hi;
        trans[ct][hi] = trans_base + rr * C::RB + 16 * (ch ^ swz_rt<C::DL>(rr)) + 8 * (tq & 1);
      }
    }
  }
};

// acc[ct] += A^T(ct) * b, where A^T(ct) is the transposed read of the tile at
// LDS displacement OFF (buffer base + 16*ch*RB) for 32-column group ct.
template <int D, int OFF>
__device__ __forceinline__ void mfma_transposed(floatx16 (&acc)[D / 32], const TileOffsets<D> &to,
                                                const bf16x8 &b) {
  if constexpr (D / 32 % 2 == 1) {  // an odd column group count: the last one alone
    constexpr int c = D / 32 - 1;
    constexpr int HI = OFF & ~0xffff;
    constexpr int LO = OFF & 0xffff;
    u32x2 l0 = ds_read_tr16_at<LO>(to.trans[c][0] + HI);
    u32x2 h0 = ds_read_tr16_at<LO>(to.trans[c][1] + HI);
    lds_wait(l0, h0);
    const u32x4 a0 = {l0[0], l0[1], h0[0], h0[1]};
    acc[c] = mfma32x32x16(as_bf16x8(a0), b, acc[c]);
  }
#pragma unroll
  for (int c2 = 0; c2 + 1 < D / 32; c2 += 2) {
    // the instruction's offset field holds 16 bits; larger displacements go into the address
    constexpr int HI = OFF & ~0xffff;
    constexpr int LO = OFF & 0xffff;
    u32x2 l0 = ds_read_tr16_at<LO>(to.trans[c2][0] + HI);
    u32x2 h0 = ds_read_tr16_at<LO>(to.trans[c2][1] + HI);
    u32x2 l1 = ds_read_tr16_at<LO>(to.trans[c2 + 1][0] + HI);
    u32x2 h1 = ds_read_tr16_at<LO>(to.trans[c2 + 1][1] + HI);
    lds_wait(l0, h0, l1, h1);
    const u32x4 a0 = {l0[0], l0[1], h0[0], h0[1]};
    const u32x4 a1 = {l1[0], l1[1], h1[0], h1[1]};
    acc[c2] = mfma32x32x16(as_bf16x8(a0), b, acc[c2]);
    acc[c2 + 1] = mfma32x32x16(as_bf16x8(a1), b, acc[c2 + 1]);
  }
}

// Store a [32 rows x D] fp32 accumulator as float32 times `mul` (same register
// layout as store_rows_bf16 below).
template <int D>
__device__ __forceinline__ void store_rows_f32(float *row, const floatx16 (&acc)[D / 32], float mul, int half) {
#pragma unroll
  for (int ct = 0; ct < D / 32; ++ct) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const floatx4 w = {acc[ct][4 * g + 0] * mul, acc[ct][4 * g + 1] * mul, acc[ct][4 * g + 2] * mul,
                         acc[ct][4 * g + 3] * mul};
      *reinterpret_cast<floatx4 *>(row + 32 * ct + 8 * g + 4 * half) = w;
    }
  }
}

// Store a [32 rows x D] fp32 accumulator (lane = row l32, register r of column
// tile ct = column 32*ct + 8*(r/4) + 4*half + r%4) as bf16 times `mul`.
template <int D>
__device__ __forceinline__ void store_rows_bf16(__bf16 *row, const floatx16 (&acc)[D / 32], float mul, int half) {
#pragma unroll
  for (int ct = 0; ct < D / 32; ++ct) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = pack_bf16x2(acc[ct][4 * g + 0] * mul, acc[ct][4 * g + 1] * mul);
      w[1] = pack_bf16x2(acc[ct][4 * g + 2] * mul, acc[ct][4 * g + 3] * mul);
      st8(row + 32 * ct + 8 * g + 4 * half, w);
    }
  }
}

// ============================================================== dQ kernel
// waves per dQ workgroup: 8 at d = 128 (one K/V tile in LDS serves 256 query rows,
// 1-2% faster than 4), 4 otherwise
template <int D> constexpr int dq_waves() { return (D == 128) ? 8 : 4; }
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(64 * dq_waves<D>(), (D == 256) ? 1 : 8 / dq_waves<D>())
fa_bwd_dq_kernel(const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K, const __bf16 *__restrict__ V,
                 const __bf16 *__restrict__ Og, const __bf16 *__restrict__ dO, const float *__restrict__ LSE,
                 __bf16 *__restrict__ dQ, float *__restrict__ Dsum, float *__restrict__ Lse2, int N,
                 int group, float scale_log2e, float scale, int xcd_round) {
  using C = BwdCfg<D>;
  constexpr int TB = C::TB;
  constexpr int RB = C::RB;
  constexpr int NW = dq_waves<D>();
  constexpr int BR = 32 * NW;  // query rows per workgroup
  // LDS: K tiles at [0, TB), [TB, 2TB); V tiles at [2TB, 3TB), [3TB, 4TB)
  __shared__ __align__(1024) unsigned char smem[4 * TB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int nqb = (N + BR - 1) / BR;
  const int nbh = gridDim.x / nqb;
  int bh, qb;
  // same-head blocks share an XCD's L2
  if (CAUSAL && xcd_round > 0) map_block_balanced(blockIdx.x, nqb, nbh, xcd_round, bh, qb);
  else map_block(blockIdx.x, nqb, nbh, CAUSAL, bh, qb);
  const size_t head_off = (size_t)bh * N * D;
  const int q0 = qb * BR;
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
  if (q_ok && half == 0) {
    Dsum[(size_t)bh * N + my_q] = drow;
    Lse2[(size_t)bh * N + my_q] = lse2;
  }

  int ntiles = (N + 63) / 64;
  if (CAUSAL) ntiles = min(ntiles, (min(q0 + BR, N) - 1) / 64 + 1);

  const uint32_t head_bytes = (uint32_t)N * C::RBG;
  const size_t kv_off = (size_t)(bh / group) * N * D;  // the K/V head this query head reads
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + kv_off, head_bytes);
  TileOffsets<D> to;
  to.init(lane, lds_addr(smem));  // transposed reads are of the K tiles

  floatx16 dqacc[C::CT];
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) dqacc[ct] = floatx16{0};

  auto step = [&](auto bufc, int t) {
    constexpr int BUF = decltype(bufc)::value;
    wait_vmem();
    __syncthreads();  // tile t is in LDS for everyone; tile t-1 is no longer read
    if (t + 1 < ntiles) {
      issue_tile<D, NW>(krs, smem + (BUF ^ 1) * TB, (t + 1) * 64, wave, lane);
      issue_tile<D, NW>(vrs, smem + (2 + (BUF ^ 1)) * TB, (t + 1) * 64, wave, lane);
    }
    const int kb = t * 64;
    if (CAUSAL && kb > qw0 + 31) return;  // every key of the tile is above this wave's rows
    const unsigned char *Ks = smem + BUF * TB;
    const unsigned char *Vs = smem + (2 + BUF) * TB;
    const bool need_mask = (CAUSAL && (kb + 63 > qw0)) || (kb + 64 > N);
    static_for<2>([&](auto ktc) {
      constexpr int KT = decltype(ktc)::value;
      floatx16 s = floatx16{0}, dp = floatx16{0};
      {
        bf16x8 a[C::KSTEPS], b[C::KSTEPS];
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
          a[ks] = as_bf16x8(ld16(Ks + to.rows[ks] + 32 * KT * RB));
          b[ks] = as_bf16x8(ld16(Vs + to.rows[ks] + 32 * KT * RB));
        }
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
          s = mfma32x32x16(a[ks], qf[ks], s);
          dp = mfma32x32x16(b[ks], dof[ks], dp);
        }
      }
      // masked keys get a score of -inf, so P = 2^-inf = 0 exactly; done as a
      // pass of its own so the exponentials below stay one branch-free block
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + 32 * KT + 16 * (r >> 3) + 8 * half + (r & 7);
          if (key >= N || (CAUSAL && key > my_q)) s[r] = -INFINITY;
        }
      }
      static_for<2>([&](auto mc) {
        constexpr int M = decltype(mc)::value;
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float d2[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int r = 8 * M + 2 * i + e;
            const float p = fast_exp2(__builtin_fmaf(s[r], scale_log2e, -lse2));
            d2[e] = p * (dp[r] - drow);
          }
          w[i] = pack_bf16x2(d2[0], d2[1]);
        }
        mfma_transposed<D, BUF * TB + 16 * (2 * KT + M) * RB>(dqacc, to, as_bf16x8(w));
      });
    });
  };

  issue_tile<D, NW>(krs, smem, 0, wave, lane);
  issue_tile<D, NW>(vrs, smem + 2 * TB, 0, wave, lane);
  for (int t = 0; t < ntiles; t += 2) {
    step(std::integral_constant<int, 0>{}, t);
    if (t + 1 < ntiles) step(std::integral_constant<int, 1>{}, t + 1);
  }

  if (q_ok) store_rows_bf16<D>(dQ + head_off + (size_t)my_q * D, dqacc, scale, half);
}

// ============================================================== dK/dV kernel
// WHAT: 3 = dK and dV, 1 = dV only, 2 = dK only (head dim 256 runs the two
// halves as separate launches: one wave cannot hold both accumulators there)
template <int D, bool CAUSAL, int WHAT = 3>
__global__ void __launch_bounds__(256, (D == 256) ? 1 : (D == 96) ? 2 : 3)
fa_bwd_dkdv_kernel(const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K, const __bf16 *__restrict__ V,
                   const __bf16 *__restrict__ dO, const float *__restrict__ Dsum, const float *__restrict__ Lse2,
                   __bf16 *__restrict__ dK, __bf16 *__restrict__ dV, float *__restrict__ part, int N, int group,
                   int nsplit, float scale_log2e, float scale, int xcd_round) {
  using C = BwdCfg<D>;
  constexpr int TB = C::TB;
  constexpr int RB = C::RB;
  constexpr int BKV = 128;                  // keys per workgroup
  constexpr int STAGE = 2 * TB + 1024;      // Q tile, dO tile, lse*log2e[64], D[64]
  __shared__ __align__(1024) unsigned char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int nkb = (N + BKV - 1) / BKV;
  const int nkvh = gridDim.x / (nkb * nsplit);  // K/V heads
  int vh, rb;
  // same-head blocks share an XCD's L2
  if (CAUSAL && xcd_round > 0) map_block_balanced(blockIdx.x, nkb, nkvh * nsplit, xcd_round, vh, rb);
  else map_block(blockIdx.x, nkb, nkvh * nsplit, CAUSAL, vh, rb);
  // the query heads of a K/V head's group may be split over nsplit workgroups,
  // each writing a float32 partial dK/dV that a reduction kernel sums
  const int bh = vh / nsplit;
  const int split = vh - bh * nsplit;
  // with a causal mask the lowest key blocks have the most work: run them first
  const int kblk = CAUSAL ? (nkb - 1 - rb) : rb;
  // bh is a K/V head; query heads bh * group .. bh * group + group - 1 read it
  const size_t head_off = (size_t)bh * N * D;
  const int kb0 = kblk * BKV;
  const int kw0 = kb0 + 32 * wave;
  const int my_k = kw0 + l32;
  const bool k_ok = my_k < N;

  constexpr bool DO_K = (WHAT & 2) != 0;
  constexpr bool DO_V = (WHAT & 1) != 0;
  bf16x8 kf[C::KSTEPS], vf[C::KSTEPS];
  {
    const size_t roff = head_off + (size_t)(k_ok ? my_k : 0) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      const u32x4 z = {0, 0, 0, 0};
      kf[ks] = as_bf16x8(k_ok ? ld16(K + roff + 16 * ks) : z);
      if constexpr (DO_K) vf[ks] = as_bf16x8(k_ok ? ld16(V + roff + 16 * ks) : z);
    }
  }

  const int nqt = (N + 63) / 64;
  const int qt0 = CAUSAL ? (kb0 / 64) : 0;

  const uint32_t head_bytes = (uint32_t)N * C::RBG;
  // query heads g0 .. g1-1 of the group are this workgroup's share
  const int g0 = (int)((long long)split * group / nsplit);
  const int g1 = (int)((long long)(split + 1) * group / nsplit);
  __amdgpu_buffer_rsrc_t qrs, ors, lrs, drs;  // the current query head's Q, dO, lse*log2e, D
  TileOffsets<D> to;
  to.init(lane, lds_addr(smem));  // transposed reads of the Q tile; the dO tile is TB further

  auto issue = [&](int t, int stage) {
    unsigned char *base = smem + stage * STAGE;
    issue_tile<D>(qrs, base, t * 64, wave, lane);
    issue_tile<D>(ors, base + TB, t * 64, wave, lane);
    if (wave == 0) load_lds4(lrs, base + 2 * TB, (uint32_t)(t * 64 + lane) * 4u);
    if (wave == 1) load_lds4(drs, base + 2 * TB + 256, (uint32_t)(t * 64 + lane) * 4u);
  };

  floatx16 dkacc[C::CT], dvacc[C::CT];
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) {
    dkacc[ct] = floatx16{0};
    dvacc[ct] = floatx16{0};
  }

  auto step = [&](auto bufc, int t) {
    constexpr int BUF = decltype(bufc)::value;
    wait_vmem();
    __syncthreads();
    if (t + 1 < nqt) issue(t + 1, BUF ^ 1);
    const int qs = t * 64;
    if (CAUSAL && qs + 63 < kw0) return;  // every query of the tile is before this wave's keys
    const unsigned char *Qs = smem + BUF * STAGE;
    const unsigned char *Os = Qs + TB;
    const float *lst = reinterpret_cast<const float *>(Qs + 2 * TB);
    const bool need_mask = (CAUSAL && qs < kw0 + 31) || (qs + 64 > N) || (kb0 + BKV > N);
    static_for<2>([&](auto qtc) {
      constexpr int QT = decltype(qtc)::value;
      floatx16 s = floatx16{0}, dp = floatx16{0};
      // operand rows in groups of RCH k-steps (all at once below d = 256)
      constexpr int RCH = (D == 256) ? 4 : C::KSTEPS;
#pragma unroll
      for (int k0 = 0; k0 < C::KSTEPS; k0 += RCH) {
        bf16x8 a[RCH], b[RCH];
#pragma unroll
        for (int i = 0; i < RCH; ++i) {
          a[i] = as_bf16x8(ld16(Qs + to.rows[k0 + i] + 32 * QT * RB));
          if constexpr (DO_K) b[i] = as_bf16x8(ld16(Os + to.rows[k0 + i] + 32 * QT * RB));
        }
#pragma unroll
        for (int i = 0; i < RCH; ++i) {
          s = mfma32x32x16(a[i], kf[k0 + i], s);
          if constexpr (DO_K) dp = mfma32x32x16(b[i], vf[k0 + i], dp);
        }
      }
      // masked (query, key) pairs get a score of -inf, so P = 0 exactly; a pass
      // of its own keeps the exponentials below one branch-free block
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = qs + 32 * QT + 16 * (r >> 3) + 8 * half + (r & 7);
          if (q >= N || !k_ok || (CAUSAL && q < my_k)) s[r] = -INFINITY;
        }
      }
      static_for<2>([&](auto mc) {
        constexpr int M = decltype(mc)::value;
        const int qoff = 32 * QT + 16 * M + 8 * half;  // tile-local query of register 8M
        const floatx4 l0 = *reinterpret_cast<const floatx4 *>(lst + qoff);
        const floatx4 l1 = *reinterpret_cast<const floatx4 *>(lst + qoff + 4);
        floatx4 d0 = floatx4{0}, d1 = floatx4{0};
        if constexpr (DO_K) {
          d0 = *reinterpret_cast<const floatx4 *>(lst + 64 + qoff);
          d1 = *reinterpret_cast<const floatx4 *>(lst + 64 + qoff + 4);
        }
        u32x4 pw, sw;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float p2[2], s2[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int j = 2 * i + e;
            const float lq = (j < 4) ? l0[j] : l1[j - 4];
            const float dq = (j < 4) ? d0[j] : d1[j - 4];
            const float p = fast_exp2(__builtin_fmaf(s[8 * M + j], scale_log2e, -lq));
            p2[e] = p;
            s2[e] = p * (dp[8 * M + j] - dq);
          }
          pw[i] = pack_bf16x2(p2[0], p2[1]);
          sw[i] = pack_bf16x2(s2[0], s2[1]);
        }
        constexpr int OFFQ = BUF * STAGE + 16 * (2 * QT + M) * RB;
        if constexpr (DO_V) mfma_transposed<D, OFFQ + TB>(dvacc, to, as_bf16x8(pw));  // dV^T += dO^T P
        if constexpr (DO_K) mfma_transposed<D, OFFQ>(dkacc, to, as_bf16x8(sw));       // dK^T += Q^T dS
      });
    });
  };

  for (int g = g0; g < g1; ++g) {
    const size_t hq = (size_t)bh * group + g;  // query head
    qrs = make_rsrc(Q + hq * N * D, head_bytes);
    ors = make_rsrc(dO + hq * N * D, head_bytes);
    lrs = make_rsrc(Lse2 + hq * N, (uint32_t)N * 4u);
    drs = make_rsrc(Dsum + hq * N, (uint32_t)N * 4u);
    if (g > g0) __syncthreads();  // every wave is done with the previous head's tiles
    issue(qt0, 0);
    for (int t = qt0; t < nqt; t += 2) {
      step(std::integral_constant<int, 0>{}, t);
      if (t + 1 < nqt) step(std::integral_constant<int, 1>{}, t + 1);
    }
  }

  if (k_ok) {
    if (nsplit == 1) {
      if constexpr (DO_K) store_rows_bf16<D>(dK + head_off + (size_t)my_k * D, dkacc, scale, half);
      if constexpr (DO_V) store_rows_bf16<D>(dV + head_off + (size_t)my_k * D, dvacc, 1.0f, half);
    } else {  // partials [2][nsplit][K/V heads][N][D]: dK (scaled) then dV
      const size_t per = (size_t)nkvh * N * D;
      const size_t off = (size_t)split * per + head_off + (size_t)my_k * D;
      if constexpr (DO_K) store_rows_f32<D>(part + off, dkacc, scale, half);
      if constexpr (DO_V) store_rows_f32<D>(part + (size_t)nsplit * per + off, dvacc, 1.0f, half);
    }
  }
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(512, 1)
fa_bwd_dkdv_pair_kernel(const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K, const __bf16 *__restrict__ V,
                   const __bf16 *__restrict__ dO, const float *__restrict__ Dsum, const float *__restrict__ Lse2,
                   __bf16 *__restrict__ dK, __bf16 *__restrict__ dV, float *__restrict__ part, int N, int group,
                   int nsplit, float scale_log2e, float scale, int xcd_round) {
  using C = BwdCfg<D>;
  constexpr int TB = C::TB;
  constexpr int RB = C::RB;
  constexpr int BKV = 128;                  // keys per workgroup: 4 groups of 32
  constexpr int STAGE = 2 * TB + 1024;      // Q tile, dO tile, lse*log2e[64], D[64]
  constexpr int PBUF = 2 * STAGE;           // P exchange: [sub-tile 2][key group 4][half 2][2][64 lanes x 16 B]
  __shared__ __align__(1024) unsigned char smem[2 * STAGE + 32768];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // waves w and w + 4 share a SIMD and a key group: role 0 (w < 4) forms P and
  // accumulates dV, role 1 forms dS from the P of its partner and accumulates dK
  const int role = wave >> 2;
  const int kg = wave & 3;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int nkb = (N + BKV - 1) / BKV;
  const int nkvh = gridDim.x / (nkb * nsplit);  // K/V heads
  int vh, rb;
  // same-head blocks share an XCD's L2
  if (CAUSAL && xcd_round > 0) map_block_balanced(blockIdx.x, nkb, nkvh * nsplit, xcd_round, vh, rb);
  else map_block(blockIdx.x, nkb, nkvh * nsplit, CAUSAL, vh, rb);
  // the query heads of a K/V head's group may be split over nsplit workgroups,
  // each writing a float32 partial dK/dV that a reduction kernel sums
  const int bh = vh / nsplit;
  const int split = vh - bh * nsplit;
  // with a causal mask the lowest key blocks have the most work: run them first
  const int kblk = CAUSAL ? (nkb - 1 - rb) : rb;
  // bh is a K/V head; query heads bh * group .. bh * group + group - 1 read it
  const size_t head_off = (size_t)bh * N * D;
  const int kb0 = kblk * BKV;
  const int kw0 = kb0 + 32 * kg;
  const int my_k = kw0 + l32;
  const bool k_ok = my_k < N;

  // B operand of the first products: K rows (role 0, S = Q K^T) or V rows (role 1, dP = dO V^T)
  bf16x8 bf[C::KSTEPS];
  {
    const __bf16 *src = (role == 0) ? K : V;
    const size_t roff = head_off + (size_t)(k_ok ? my_k : 0) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) bf[ks] = as_bf16x8(k_ok ? ld16(src + roff + 16 * ks) : u32x4{0, 0, 0, 0});
  }

  const int nqt = (N + 63) / 64;
  const int qt0 = CAUSAL ? (kb0 / 64) : 0;

  const uint32_t head_bytes = (uint32_t)N * C::RBG;
  // query heads g0 .. g1-1 of the group are this workgroup's share
  const int g0 = (int)((long long)split * group / nsplit);
  const int g1 = (int)((long long)(split + 1) * group / nsplit);
  __amdgpu_buffer_rsrc_t qrs, ors, lrs, drs;  // the current query head's Q, dO, lse*log2e, D
  // transposed reads of the second products: the dO tile (role 0, dV^T += dO^T P)
  // or the Q tile (role 1, dK^T += Q^T dS), which is TB before it
  TileOffsets<D> to;
  to.init(lane, lds_addr(smem) + (role == 0 ? TB : 0));

  auto issue = [&](int t, int stage) {
    unsigned char *base = smem + stage * STAGE;
    issue_tile<D, 8>(qrs, base, t * 64, wave, lane);
    issue_tile<D, 8>(ors, base + TB, t * 64, wave, lane);
    if (wave == 0) load_lds4(lrs, base + 2 * TB, (uint32_t)(t * 64 + lane) * 4u);
    if (wave == 1) load_lds4(drs, base + 2 * TB + 256, (uint32_t)(t * 64 + lane) * 4u);
  };

  floatx16 acc[C::CT];  // dV^T (role 0) or dK^T (role 1), lane = key
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) acc[ct] = floatx16{0};

  auto step = [&](auto bufc, int t) {
    constexpr int BUF = decltype(bufc)::value;
    wait_vmem();
    __syncthreads();
    if (t + 1 < nqt) issue(t + 1, BUF ^ 1);
    const int qs = t * 64;
    // every query of the tile is before this key group's keys: nothing to do,
    // but the workgroup barrier below is still passed
    const bool active = !(CAUSAL && qs + 63 < kw0);
    const unsigned char *Qs = smem + BUF * STAGE;
    const float *lst = reinterpret_cast<const float *>(Qs + 2 * TB);
    const bool need_mask = (CAUSAL && qs < kw0 + 31) || (qs + 64 > N) || (kb0 + BKV > N);

    // ---- first products for both 32-query sub-tiles: S (role 0) or dP (role 1)
    floatx16 first[2];
    if (active) {
      const unsigned char *As = Qs + role * TB;  // Q rows or dO rows
      static_for<2>([&](auto qtc) {
        constexpr int QT = decltype(qtc)::value;
        floatx16 a = floatx16{0};
        bf16x8 r[C::KSTEPS];
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) r[ks] = as_bf16x8(ld16(As + to.rows[ks] + 32 * QT * RB));
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) a = mfma32x32x16(r[ks], bf[ks], a);
        first[QT] = a;
      });
    }
    u32x4 pw[2][2];  // role 0: P of (sub-tile, half) as bf16, lane = key, 8 queries
    if (role == 0 && active) {
      // masked (query, key) pairs get a score of -inf, so P = 0 exactly; a pass
      // of its own keeps the exponentials below one branch-free block
      if (need_mask) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int q = qs + 32 * qt + 16 * (r >> 3) + 8 * half + (r & 7);
            if (q >= N || !k_ok || (CAUSAL && q < my_k)) first[qt][r] = -INFINITY;
          }
      }
      static_for<2>([&](auto qtc) {
        constexpr int QT = decltype(qtc)::value;
        static_for<2>([&](auto mc) {
          constexpr int M = decltype(mc)::value;
          const int qoff = 32 * QT + 16 * M + 8 * half;  // tile-local query of register 8M
          const floatx4 l0 = *reinterpret_cast<const floatx4 *>(lst + qoff);
          const floatx4 l1 = *reinterpret_cast<const floatx4 *>(lst + qoff + 4);
          float pf[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float p2[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int j = 2 * i + e;
              const float lq = (j < 4) ? l0[j] : l1[j - 4];
              const float p = fast_exp2(__builtin_fmaf(first[QT][8 * M + j], scale_log2e, -lq));
              p2[e] = p;
              pf[j] = p;
            }
            pw[QT][M][i] = pack_bf16x2(p2[0], p2[1]);
          }
          // float32 P for the partner's dS, in two 16-byte halves
          unsigned char *slot = smem + PBUF + ((QT * 4 + kg) * 2 + M) * 2048 + lane * 16;
          *reinterpret_cast<floatx4 *>(slot) = floatx4{pf[0], pf[1], pf[2], pf[3]};
          *reinterpret_cast<floatx4 *>(slot + 1024) = floatx4{pf[4], pf[5], pf[6], pf[7]};
        });
      });
    }
    if (role == 1 && active) {
      // dP - D now, while the partner still forms P: after the barrier the dS
      // wave is the critical path and only has to multiply by P
      static_for<2>([&](auto qtc) {
        constexpr int QT = decltype(qtc)::value;
        static_for<2>([&](auto mc) {
          constexpr int M = decltype(mc)::value;
          const int qoff = 32 * QT + 16 * M + 8 * half;
          const floatx4 d0 = *reinterpret_cast<const floatx4 *>(lst + 64 + qoff);
          const floatx4 d1 = *reinterpret_cast<const floatx4 *>(lst + 64 + qoff + 4);
#pragma unroll
          for (int j = 0; j < 8; ++j) first[QT][8 * M + j] -= (j < 4) ? d0[j] : d1[j - 4];
        });
      });
    }
    __syncthreads();  // P of every key group is in LDS
    if (!active) return;
    // B operands of the second products: P (role 0) or dS (role 1).  Only these
    // differ between the roles; the products themselves are one code path, so
    // the accumulator is not copied where the two roles' branches meet.
    u32x4 bop[2][2];
    if (role == 0) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int m = 0; m < 2; ++m) bop[qt][m] = pw[qt][m];
    } else {
      static_for<2>([&](auto qtc) {
        constexpr int QT = decltype(qtc)::value;
        static_for<2>([&](auto mc) {
          constexpr int M = decltype(mc)::value;
          const unsigned char *slot = smem + PBUF + ((QT * 4 + kg) * 2 + M) * 2048 + lane * 16;
          const floatx4 p0 = *reinterpret_cast<const floatx4 *>(slot);
          const floatx4 p1 = *reinterpret_cast<const floatx4 *>(slot + 1024);
          u32x4 sw;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float s2[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int j = 2 * i + e;
              const float p = (j < 4) ? p0[j] : p1[j - 4];
              s2[e] = p * first[QT][8 * M + j];  // P (dP - D)
            }
            sw[i] = pack_bf16x2(s2[0], s2[1]);
          }
          bop[QT][M] = sw;
        });
      });
    }
    // dV^T += dO^T P (role 0) or dK^T += Q^T dS (role 1)
    static_for<2>([&](auto qtc) {
      constexpr int QT = decltype(qtc)::value;
      static_for<2>([&](auto mc) {
        constexpr int M = decltype(mc)::value;
        constexpr int OFFQ = BUF * STAGE + 16 * (2 * QT + M) * RB;
        mfma_transposed<D, OFFQ>(acc, to, as_bf16x8(bop[QT][M]));
      });
    });
  };

  for (int g = g0; g < g1; ++g) {
    const size_t hq = (size_t)bh * group + g;  // query head
    qrs = make_rsrc(Q + hq * N * D, head_bytes);
    ors = make_rsrc(dO + hq * N * D, head_bytes);
    lrs = make_rsrc(Lse2 + hq * N, (uint32_t)N * 4u);
    drs = make_rsrc(Dsum + hq * N, (uint32_t)N * 4u);
    if (g > g0) __syncthreads();  // every wave is done with the previous head's tiles
    issue(qt0, 0);
    for (int t = qt0; t < nqt; t += 2) {
      step(std::integral_constant<int, 0>{}, t);
      if (t + 1 < nqt) step(std::integral_constant<int, 1>{}, t + 1);
    }
  }

  if (k_ok) {
    if (nsplit == 1) {
      if (role == 0) store_rows_bf16<D>(dV + head_off + (size_t)my_k * D, acc, 1.0f, half);
      else store_rows_bf16<D>(dK + head_off + (size_t)my_k * D, acc, scale, half);
    } else {  // partials [2][nsplit][K/V heads][N][D]: dK (scaled) then dV
      const size_t per = (size_t)nkvh * N * D;
      const size_t off = (size_t)split * per + head_off + (size_t)my_k * D;
      if (role == 0) store_rows_f32<D>(part + (size_t)nsplit * per + off, acc, 1.0f, half);
      else store_rows_f32<D>(part + off, acc, scale, half);
    }
  }
}

// ============================================================== split reduction
// dK and dV as bf16 from the float32 partials of the workgroups that shared a
// K/V head's query heads: out[e] = sum over splits j = 0, 1, ... in that order,
// so the result is bitwise reproducible.  One thread per 8 elements.
__global__ void __launch_bounds__(256)
fa_bwd_reduce_kernel(const float *__restrict__ part, __bf16 *__restrict__ dK, __bf16 *__restrict__ dV,
                     long long count, int nsplit) {
  const long long chunks = count / 8;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= 2 * chunks) return;
  const int which = i >= chunks;  // 0: dK, 1: dV
  const long long e = (i - which * chunks) * 8;
  const float *p = part + (size_t)which * nsplit * count + e;
  floatx4 a = *reinterpret_cast<const floatx4 *>(p);
  floatx4 b = *reinterpret_cast<const floatx4 *>(p + 4);
  for (int j = 1; j < nsplit; ++j) {
    a += *reinterpret_cast<const floatx4 *>(p + (size_t)j * count);
    b += *reinterpret_cast<const floatx4 *>(p + (size_t)j * count + 4);
  }
  const u32x4 w = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
  *reinterpret_cast<u32x4 *>((which ? dV : dK) + e) = w;
}

template <int D, bool CAUSAL>
hipError_t launch(const void *q, const void *k, const void *v, const void *o, const void *dout,
                  const float *lse, void *dq, void *dk, void *dv, float *ws, int B, int H, int group, int N,
                  float scale, hipStream_t stream) {
  const long long nbh = (long long)B * H;          // query heads
  const long long nkvh = nbh / group;              // K/V heads
  const int nsplit = bwd_splits(nkvh, N, group);
  const long long gq = nbh * ((N + 32 * dq_waves<D>() - 1) / (32 * dq_waves<D>()));
  const long long gk = nkvh * nsplit * ((N + 127) / 128);
  if (gq > 0x7fffffffLL || gk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const float c = scale * kLog2e;
  float *dsum = ws;
  float *lse2 = ws + (size_t)nbh * N;
  float *part = (nsplit > 1) ? ws + bwd_partial_offset_floats(nbh, N) : nullptr;
  // causal grids the device holds all at once: the snake order of map_block_balanced
  int rq = 0, rk = 0;
  if constexpr (CAUSAL) {
    static std::atomic<int> per_cu_q{0}, per_cu_k{0};
    rq = snake_round(fa_bwd_dq_kernel<D, CAUSAL>, 64 * dq_waves<D>(), gq, per_cu_q);
    if constexpr (D == 128) rk = snake_round(fa_bwd_dkdv_pair_kernel<D, CAUSAL>, 512, gk, per_cu_k);
    else if constexpr (D != 256) rk = snake_round(fa_bwd_dkdv_kernel<D, CAUSAL>, 256, gk, per_cu_k);
  }
  hipLaunchKernelGGL((fa_bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)gq), dim3(64 * dq_waves<D>()), 0, stream,
                     (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, (const __bf16 *)o,
                     (const __bf16 *)dout, lse, (__bf16 *)dq, dsum, lse2, N, group, c, scale, rq);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (D != 128 && D != 256)
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)gk), dim3(256), 0, stream,
                       (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, (const __bf16 *)dout,
                       (const float *)dsum, (const float *)lse2, (__bf16 *)dk, (__bf16 *)dv, part, N, group,
                       nsplit, c, scale, rk);
  else if constexpr (D == 256) {
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, CAUSAL, 1>), dim3((unsigned)gk), dim3(256), 0, stream,
                       (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, (const __bf16 *)dout,
                       (const float *)dsum, (const float *)lse2, (__bf16 *)dk, (__bf16 *)dv, part, N, group,
                       nsplit, c, scale, rk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, CAUSAL, 2>), dim3((unsigned)gk), dim3(256), 0, stream,
                       (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, (const __bf16 *)dout,
                       (const float *)dsum, (const float *)lse2, (__bf16 *)dk, (__bf16 *)dv, part, N, group,
                       nsplit, c, scale, rk);
  }
  else
    hipLaunchKernelGGL((fa_bwd_dkdv_pair_kernel<D, CAUSAL>), dim3((unsigned)gk), dim3(512), 0, stream,
                       (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, (const __bf16 *)dout,
                       (const float *)dsum, (const float *)lse2, (__bf16 *)dk, (__bf16 *)dv, part, N, group,
                       nsplit, c, scale, rk);
  if (nsplit == 1) return hipGetLastError();
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long count = nkvh * (long long)N * D;
  const long long threads = 2 * (count / 8);
  hipLaunchKernelGGL(fa_bwd_reduce_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                     (const float *)part, (__bf16 *)dk, (__bf16 *)dv, count, nsplit);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const void *q, const void *k, const void *v, const void *o, const void *dout,
                           const float *lse, void *dq, void *dk, void *dv, float *ws, int B, int H, int group,
                           int N, int d, bool causal, float scale, hipStream_t stream) {
  if (d == 96)
    return causal ? launch<96, true>(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, group, N, scale, stream)
                  : launch<96, false>(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, group, N, scale, stream);
  if (d == 32)
    return causal ? launch<32, true>(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, group, N, scale, stream)
                  : launch<32, false>(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, group, N, scale, stream);
  if (d == 64)
    return causal ? launch<64, true>(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, group, N, scale, stream)
                  : launch<64, false>(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, group, N, scale, stream);
  if (d == 128)
    return causal ? launch<128, true>(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, group, N, scale, stream)
                  : launch<128, false>(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, group, N, scale, stream);
  return causal ? launch<256, true>(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, group, N, scale, stream)
                : launch<256, false>(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, group, N, scale, stream);
}

}  // namespace fa
