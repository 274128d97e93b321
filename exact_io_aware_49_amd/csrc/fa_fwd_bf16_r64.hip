// fa_fwd_bf16_r64.hip -- bf16 attention forward at head dim 128 with 64 query
// rows per wave.
//
// What is computed is the same as in fa_fwd_bf16.hip: O = softmax(scale Q K^T) V
// and lse = ln sum_j exp(scale q_i.k_j) ("FlashAttention (DE)", section
// "Problematik der Standard-Attention"), by the tiled online-softmax scheme of
// sections "Tiling und blockweise Verarbeitung", "Online-Softmax-Berechnung"
// and "Zusammenfassen von Operationen in einem CUDA-Kernel".
//
// Why a second kernel: with 32 query rows per wave, every 32x32x16 matrix
// product reads its 1 KB K or V^T operand from LDS for 32 rows only, and at
// full matrix-core rate the LDS pipe would be about 80% busy.  Here a wave
// owns 64 query rows (two 32-row blocks) and every K or V^T fragment it reads
// from LDS feeds two products, one per block, which halves the LDS bytes per
// flop.  The register cost (Q of 64 rows: 64 registers; O^T of 64 rows: 128)
// leaves room for one wave per SIMD only.  Q lives in AGPRs (pinned there by
// empty asm statements; a matrix product reads its B operand from AGPRs
// directly); this source is built with the VGPR form of the MFMA instructions,
// so the scores and the output accumulators are VGPRs and the vector code
// reads the scores without copying them out of AGPRs (in the AGPR form every
// tile copied all 32 score registers per lane, 1% slower).
//
// Mapping: 4 waves (one per SIMD), 256 query rows per workgroup; wave w owns
// rows [64 w, 64 w + 64) of the block as blocks r = 0, 1 of 32 rows.
//   * K/V tiles of 32 keys stream HBM -> LDS by buffer_load ... lds into rings
//     of four slots, each slot its own LDS array.  The loop is unrolled by four
//     so every slot index is a compile-time constant: the compiler then knows
//     which array each in-flight transfer writes, schedules the LDS reads
//     itself and never waits for a transfer into another slot.  K(t+4) and
//     V(t+3) are issued at step t; one workgroup barrier per tile.
//   * Step t:
//       phase A: S(t+1) = K(t+1) Q^T (16 products)   || P of keys 16..31 of
//                tile t, and the V^T fragments of tile t are read
//       phase B: O^T += V(t)^T P(t)^T (16 products) || P of keys 0..15 of
//                tile t+1, and the K fragments of tile t+2 are read
//     so the single wave of a SIMD always has independent vector work to
//     issue between its matrix products.
//   * The reference maximum is tile 0's row maximum and stays put while the
//     probabilities stay finite: they keep their relative precision at any
//     magnitude, and O and l share the reference, so O / l is exact either
//     way.  Only a chunk whose row sum exceeds 2^64 moves it (a rare branch
//     that rescales O and l and recomputes the tile's P), so no tile after
//     the first needs a row maximum.
//   * Causal: tiles above the diagonal of every row of the workgroup are never
//     loaded; a wave past its last tile only helps load; the diagonal and
//     ragged tiles are masked.
//
// Operand layouts are those of fa_fwd_bf16.hip: K rows enter the score
// product in swap_bits23 order, so eight consecutive accumulator registers hold
// eight consecutive keys and P goes straight from the accumulators into the B
// operand of the value product; V^T is read with ds_read_b64_tr_b16.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

template <int D>
struct R64Cfg {
  static constexpr int NW = 4;                    // waves per workgroup (one per SIMD)
  static constexpr int BR = 64 * NW;              // query rows per workgroup
  static constexpr int BC = 32;                   // keys per tile
  static constexpr int KS = D / 16;               // k-steps of the score product
  static constexpr int CT = D / 32;               // 32-column output tiles
  static constexpr int RB = D * 2;                // bytes per K/V row
  static constexpr int TB = BC * RB;              // bytes per K or V tile
  static constexpr int CPR = D / 8;               // 16-byte chunks per row
  static constexpr int RPI = 1024 / RB;           // rows per wave-wide 16-byte load
  static constexpr int LPW = TB / 1024 / NW;      // loads per wave per tensor per tile
  // vector instructions the scheduler places after each matrix product: phase A
  // (score products) and phase B (value products).  One wave per SIMD issues
  // in order, and a product runs 32 cycles; measured best of 2..6 (phase A: 2 to 4
  // level; phase B: 3 is 2% slower, 5 level non-causal and 1% slower causal).
  static constexpr int VEC_A = 3;
  static constexpr int VEC_B = 4;
};

typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));

// ds_read_b64_tr_b16 from an LDS array (compiler-visible, so it is scheduled and
// counted like any LDS load)
__device__ __forceinline__ u32x2 tr16(const unsigned char *p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
  return __builtin_bit_cast(u32x2, r);
}
__device__ __forceinline__ u32x4 b128(const unsigned char *p) { return *reinterpret_cast<const u32x4 *>(p); }

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 1)
fa_fwd_r64_kernel(const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K, const __bf16 *__restrict__ V,
                  __bf16 *__restrict__ O, float *__restrict__ LSE, int N, int nbh, int group, float scale_log2e) {
  using C = R64Cfg<D>;
  constexpr int TB = C::TB;
  constexpr int RB = C::RB;
  // four K slots and four V slots, separate arrays (see the header comment)
  __shared__ __align__(1024) unsigned char ks0[TB], ks1[TB], ks2[TB], ks3[TB];
  __shared__ __align__(1024) unsigned char vs0[TB], vs1[TB], vs2[TB], vs3[TB];
  auto kslot = [&](auto jc) -> unsigned char * {
    constexpr int J = decltype(jc)::value & 3;
    if constexpr (J == 0) return ks0;
    else if constexpr (J == 1) return ks1;
    else if constexpr (J == 2) return ks2;
    else return ks3;
  };
  auto vslot = [&](auto jc) -> unsigned char * {
    constexpr int J = decltype(jc)::value & 3;
    if constexpr (J == 0) return vs0;
    else if constexpr (J == 1) return vs1;
    else if constexpr (J == 2) return vs2;
    else return vs3;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int nqb = (N + C::BR - 1) / C::BR;
  int bh, qb;
  map_block(blockIdx.x, nqb, nbh, CAUSAL, bh, qb);

  const size_t head_off = (size_t)bh * (size_t)N * D;
  const size_t kv_off = (size_t)(bh / group) * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * RB;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + kv_off, head_bytes);

  const int q0 = qb * C::BR;
  const int qw0 = q0 + 64 * wave;  // first query row of this wave
  int my_q[2];
  my_q[0] = qw0 + l32;
  my_q[1] = qw0 + 32 + l32;

  // ---- Q fragments of both blocks (B operand: lane = query row), kept in AGPRs
  bf16x8 qf[2][C::KS];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const bool ok = my_q[r] < N;
    const __bf16 *qrow = Q + head_off + (size_t)(ok ? my_q[r] : 0) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[r][ks] = as_bf16x8(ok ? ld16(qrow + 16 * ks) : u32x4{0, 0, 0, 0});
  }
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) asm volatile("" : "+a"(qf[r][ks]));

  const int ntiles_all = (N + C::BC - 1) / C::BC;
  int ntiles = ntiles_all;
  if (CAUSAL) ntiles = min(ntiles_all, (min(q0 + C::BR, N) - 1) / C::BC + 1);

  // ---- direct loads: wave w fills rows [(w LPW + u) RPI, + RPI) of a tile.
  // Tiles outside [0, ntiles) get an offset beyond the buffer (they read zero
  // and cost no memory traffic), so every step issues the same loads.
  const int ld_row_in = lane / C::CPR;
  const int ld_chunk = lane % C::CPR;
  auto issue = [&](__amdgpu_buffer_rsrc_t rs, bool is_k, int t, unsigned char *slot) {
#pragma unroll
    for (int u = 0; u < C::LPW; ++u) {
      const int row0 = (wave * C::LPW + u) * C::RPI;
      const int row = row0 + ld_row_in;
      const int sw = is_k ? swz_k<D>(row) : swz_v<D>(row);
      const uint32_t off = ((unsigned)t < (unsigned)ntiles)
                               ? (uint32_t)(t * C::BC + row) * RB + 16u * (uint32_t)(ld_chunk ^ sw)
                               : 0x80000000u;
      load_lds16(rs, slot + row0 * RB, off);
    }
  };

  // ---- per-lane LDS byte offsets within a tile
  int koff[C::KS];
  {
    const int r = swap_bits23(l32);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) koff[ks] = r * RB + 16 * ((2 * ks + half) ^ swz_k<D>(r));
  }
  int voff[C::CT][2];
  {
    const int rlo = 8 * half + ((lane & 15) >> 2);
    const int tq = lane & 3;
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
      const int ch = 4 * ct + 2 * ((lane >> 4) & 1) + (tq >> 1);
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int r = rlo + 4 * hi;
        voff[ct][hi] = r * RB + 16 * (ch ^ swz_v<D>(r)) + 8 * (tq & 1);
      }
    }
  }

  floatx16 oacc[2][C::CT];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) oacc[r][ct] = floatx16{0};
  float m_ref[2] = {-INFINITY, -INFINITY};  // reference maximum of raw scores, per block
  float l_part[2] = {0.f, 0.f};             // this lane's part of the exponential sum

  // Keys past N or (causal) past the row's own index get score -inf.
  auto mask_tile = [&](floatx16 &s, int t, int r) {
    const int kb = t * C::BC;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kb + 16 * (i >> 3) + 8 * half + (i & 7);
      if ((key >= N) || (CAUSAL && key > my_q[r])) s[i] = -INFINITY;
    }
  };
  // Row maximum of one block's (masked) tile of scores, both wave halves.
  auto tile_max = [&](const floatx16 &s) -> float {
    float m = max3f(s[0], s[1], s[2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) m = max3f(m, s[i], s[i + 1]);
    m = fmaxf(m, s[15]);
    return max_with_partner(m);
  };
  // P of one 16-key chunk m of scores s, rounded to bf16; lsum = the row sum of
  // the rounded values (this lane's eight)
  auto chunk_p = [&](const floatx16 &s, int m, float mcr, float &lsum) -> bf16x8 {
    u32x4 pw;
    lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p0 = fast_exp2(__builtin_fmaf(s[8 * m + 2 * i], scale_log2e, -mcr));
      const float p1 = fast_exp2(__builtin_fmaf(s[8 * m + 2 * i + 1], scale_log2e, -mcr));
      pw[i] = pack_bf16x2(p0, p1);
      lsum = add_bf16_pair(pw[i], lsum);
    }
    return as_bf16x8(pw);
  };
  auto mc_of = [&](int r) -> float { return (m_ref[r] == -INFINITY) ? 0.f : m_ref[r] * scale_log2e; };
  // Probabilities are taken against a reference that stays put: floating point
  // keeps their relative precision at any magnitude, so the reference only has
  // to keep them finite.  A chunk whose row sum leaves [0, 2^64] (or is not a
  // number) makes the wave move the reference of that block to the tile's
  // maximum, rescale what earlier tiles added and recompute the tile's P.
  constexpr float kPMax = 18446744073709551616.f;  // 2^64
  auto too_big = [&](float l) -> bool { return !(l <= kPMax); };

  u32x4 kf[C::KS];          // K fragments of the next tile (score A operands)
  u32x2 vf[2][C::CT][2];    // V^T fragments of this tile (two 16-key chunks)
  auto read_k = [&](const unsigned char *slot) {
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) kf[ks] = b128(slot + koff[ks]);
  };
  auto read_v = [&](const unsigned char *slot) {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) vf[cc][ct][hi] = tr16(slot + 16 * cc * RB + voff[ct][hi]);
  };

  // At the barrier of step t every wave has K(t+2) and V(t) in LDS once its own
  // transfers up to those have landed: the later ones, K(t+3), V(t+1) and
  // V(t+2) (LPW loads each), may still be in flight.
  constexpr int VM_AFTER = 3 * C::LPW;
  auto sync = [&]() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(VM_AFTER) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // ---- prologue: the transfers of steps -4 .. -1 (K(s+4), V(s+3) at step s)
  issue(krs, true, 0, kslot(I0{}));
  issue(vrs, false, -1, vslot(I3{}));
  issue(krs, true, 1, kslot(I1{}));
  issue(vrs, false, 0, vslot(I0{}));
  issue(krs, true, 2, kslot(I2{}));
  issue(vrs, false, 1, vslot(I1{}));
  issue(krs, true, 3, kslot(I3{}));
  issue(vrs, false, 2, vslot(I2{}));
  sync();  // K(0..2) and V(0)

  floatx16 sA[2], sB[2];
  read_k(kslot(I0{}));
  sA[0] = floatx16{0};
  sA[1] = floatx16{0};
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    sA[0] = mfma32x32x16(as_bf16x8(kf[ks]), qf[0][ks], sA[0]);
    sA[1] = mfma32x32x16(as_bf16x8(kf[ks]), qf[1][ks], sA[1]);
  }
  read_k(kslot(I1{}));  // the score operand of step 0
  bf16x8 pc0[2];        // P of keys 0..15 of the current tile
  float l0[2];          // their row sums
  // the reference: tile 0's row maximum
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    mask_tile(sA[r], 0, r);
    m_ref[r] = tile_max(sA[r]);
    pc0[r] = chunk_p(sA[r], 0, mc_of(r), l0[r]);
  }

  // One step (tile t, slot J = t mod 4).  MASK: tile t+1 may need masking.
  auto step = [&](auto jc, auto maskc, int t, floatx16 (&cur)[2], floatx16 (&nxt)[2]) {
    constexpr int J = decltype(jc)::value;
    sync();  // K(t+2) and V(t) are in LDS; slots of K(t) and V(t-1) are free
    issue(krs, true, t + 4, kslot(std::integral_constant<int, J>{}));
    issue(vrs, false, t + 3, vslot(std::integral_constant<int, J + 3>{}));
    read_v(vslot(std::integral_constant<int, J>{}));
    // ---- phase A: S(t+1) = K(t+1) Q^T || P of keys 16..31 of tile t
    nxt[0] = floatx16{0};
    nxt[1] = floatx16{0};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      nxt[0] = mfma32x32x16(as_bf16x8(kf[ks]), qf[0][ks], nxt[0]);
      nxt[1] = mfma32x32x16(as_bf16x8(kf[ks]), qf[1][ks], nxt[1]);
    }
    float l1[2];
    bf16x8 pc1[2];
    pc1[0] = chunk_p(cur[0], 1, mc_of(0), l1[0]);
    pc1[1] = chunk_p(cur[1], 1, mc_of(1), l1[1]);
    const bool big = too_big(l0[0]) || too_big(l0[1]) || too_big(l1[0]) || too_big(l1[1]);
#pragma unroll
    for (int i = 0; i < 2 * C::KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // a matrix product
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);        // an LDS read
      __builtin_amdgcn_sched_group_barrier(0x002, C::VEC_A, 0);  // vector work
    }
    if (__ballot(big) != 0) {
      // rare: move the reference of each block to this tile's maximum
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const float m_new = fmaxf(m_ref[r], tile_max(cur[r]));
        const float alpha = fast_exp2((m_ref[r] - m_new) * scale_log2e);
        m_ref[r] = m_new;
        l_part[r] *= alpha;
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[r][ct][i] *= alpha;
        pc0[r] = chunk_p(cur[r], 0, mc_of(r), l0[r]);
        pc1[r] = chunk_p(cur[r], 1, mc_of(r), l1[r]);
      }
    }
    l_part[0] += l0[0] + l1[0];
    l_part[1] += l0[1] + l1[1];
    // ---- phase B: O^T += V(t)^T P(t)^T || P of keys 0..15 of tile t+1
    read_k(kslot(std::integral_constant<int, J + 2>{}));
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
      const u32x4 a0 = {vf[0][ct][0][0], vf[0][ct][0][1], vf[0][ct][1][0], vf[0][ct][1][1]};
      oacc[0][ct] = mfma32x32x16(as_bf16x8(a0), pc0[0], oacc[0][ct]);
      oacc[1][ct] = mfma32x32x16(as_bf16x8(a0), pc0[1], oacc[1][ct]);
    }
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
      const u32x4 a1 = {vf[1][ct][0][0], vf[1][ct][0][1], vf[1][ct][1][0], vf[1][ct][1][1]};
      oacc[0][ct] = mfma32x32x16(as_bf16x8(a1), pc1[0], oacc[0][ct]);
      oacc[1][ct] = mfma32x32x16(as_bf16x8(a1), pc1[1], oacc[1][ct]);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      if constexpr (decltype(maskc)::value) mask_tile(nxt[r], t + 1, r);
      pc0[r] = chunk_p(nxt[r], 0, mc_of(r), l0[r]);
    }
#pragma unroll
    for (int i = 0; i < 4 * C::CT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i % 2 == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, C::VEC_B, 0);
    }
  };
  auto sync_step = [&](auto jc, int t) {
    constexpr int J = decltype(jc)::value;
    sync();
    issue(krs, true, t + 4, kslot(std::integral_constant<int, J>{}));
    issue(vrs, false, t + 3, vslot(std::integral_constant<int, J + 3>{}));
  };

  // tiles this wave has work in (causal rows see keys up to their own index),
  // rounded up to whole groups of four steps: the extra tiles are masked for
  // every row of the wave (past its diagonal, or past N) and contribute zero
  const int nact = CAUSAL ? min(ntiles, (qw0 + 63) / C::BC + 1) : ntiles;
  const int nact4 = (nact + 3) & ~3;
  const int ntot4 = (ntiles + 3) & ~3;
  // leading tiles no row of the wave masks
  const int nfull = CAUSAL ? min((qw0 + 1) / C::BC, N / C::BC) : N / C::BC;

  int t = 0;
  for (; t + 4 < nfull; t += 4) {
    step(I0{}, std::false_type{}, t, sA, sB);
    step(I1{}, std::false_type{}, t + 1, sB, sA);
    step(I2{}, std::false_type{}, t + 2, sA, sB);
    step(I3{}, std::false_type{}, t + 3, sB, sA);
  }
  for (; t < nact4; t += 4) {
    step(I0{}, std::true_type{}, t, sA, sB);
    step(I1{}, std::true_type{}, t + 1, sB, sA);
    step(I2{}, std::true_type{}, t + 2, sA, sB);
    step(I3{}, std::true_type{}, t + 3, sB, sA);
  }
  // the rest of the workgroup's tiles: this wave only helps load them
  for (; t < ntot4; t += 4) {
    sync_step(I0{}, t);
    sync_step(I1{}, t + 1);
    sync_step(I2{}, t + 2);
    sync_step(I3{}, t + 3);
  }
  // every transfer issued has landed before the workgroup ends (zero-range
  // transfers past the end still complete)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: O = O^T / l, lse = (m c + log2 l) ln 2
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const float l_tot = sum_with_partner(l_part[r]);
    if (my_q[r] < N) {
      const float inv = 1.f / l_tot;
      __bf16 *orow = O + head_off + (size_t)my_q[r] * D;
#pragma unroll
      for (int ct = 0; ct < C::CT; ++ct) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 w;
          w[0] = pack_bf16x2(oacc[r][ct][4 * g + 0] * inv, oacc[r][ct][4 * g + 1] * inv);
          w[1] = pack_bf16x2(oacc[r][ct][4 * g + 2] * inv, oacc[r][ct][4 * g + 3] * inv);
          st8(orow + 32 * ct + 8 * g + 4 * half, w);
        }
      }
      if (half == 0) LSE[(size_t)bh * N + my_q[r]] = (m_ref[r] * scale_log2e + __log2f(l_tot)) * kLn2;
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_r64(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int group,
                      int N, float scale, hipStream_t stream) {
  using C = R64Cfg<D>;
  const int nbh = B * H;
  const int nqb = (N + C::BR - 1) / C::BR;
  const long long blocks = (long long)nqb * nbh;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fa_fwd_r64_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(64 * C::NW), 0, stream,
                     (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, (__bf16 *)o, lse, N, nbh, group,
                     scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16_r64(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                               int group, int N, bool causal, float scale, hipStream_t stream) {
  return causal ? launch_r64<128, true>(q, k, v, o, lse, B, H, group, N, scale, stream)
                : launch_r64<128, false>(q, k, v, o, lse, B, H, group, N, scale, stream);
}

}  // namespace fa
