// fa_fwd_fp8.hip -- exact-attention forward with FP8 (OCP E4M3) inputs on gfx950.
//
// FlashAttention-3's FP8 mode ("FlashAttention (DE)", section "Evolution und
// Weiterentwicklungen", subsection "FlashAttention-3 (2024)") carried to the
// gfx950 FP8 matrix cores.  Q, K and V arrive as E4M3 codes with one float32
// scale per tensor (real value = code * scale); O is written in bf16, lse in
// float32.  The algorithm is the bf16 forward's: a workgroup of 4 waves owns
// 128 query rows, K/V tiles of 64 keys stream through LDS with buffer_load ...
// lds, the running maximum moves lazily (only when a tile's maximum exceeds it
// by more than 2^8 in exp2 units), and the next tile's scores are computed
// under the current tile's softmax.  What changes:
//   * S^T = K Q^T and O^T += V^T P^T run on v_mfma_scale_f32_32x32x64_f8f6f4
//     (E4M3 x E4M3, unit block scales): 64 head-dim or key values per MFMA,
//     twice the bf16 rate.  The per-tensor scales fold into the exponent
//     constant (q_scale * k_scale * scale * log2 e) and the final O scaling.
//   * P = 2^(S c - m c) (at most 2^8) is rounded to E4M3 for the P V product.
//     The row sum uses the same rounded values: one more MFMA multiplies an
//     all-ones operand by P^T, so every lane holds its row's sum.
//   * The contraction index of an MFMA is any fixed byte order shared by its
//     two operands.  The key order of one 64-key step is the order in which
//     the score accumulators hold their keys (byte t of lane half h is key
//     16 (t / 8) + 8 h + t % 8 of the tile), so P packs straight from the accumulators
//     and V^T is read from the row-major tile with ds_read_b64_tr_b8 (a lane
//     gets one column of 8 consecutive rows).
//   * LDS operand reads are ordinary loads (and the tr8 builtin), so the
//     compiler counts them and may move them ahead of their use.
//   * d = 256 runs one wave per SIMD (its 32 x 256 output accumulator lives in
//     AGPRs); d = 64 and 128 run two.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx16 mfma_fp8(const i32x8 &a, const i32x8 &b, const floatx16 &c) {
  // E4M3 x E4M3 (format codes 0, 0), block scale exponents 127 (2^0)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Two floats -> two E4M3 bytes in the low (HI = false) or high half of `old`.
template <bool HI>
__device__ __forceinline__ int pack_fp8x2(float a, float b, int old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

typedef int i32x2 __attribute__((ext_vector_type(2)));
// LDS reads the compiler can schedule and count (lgkmcnt) itself
__device__ __forceinline__ i32x2 lds_tr8(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2 *)(uintptr_t)addr);
}
__device__ __forceinline__ i32x4 lds_b128(uint32_t addr) {
  return *(const __attribute__((address_space(3))) i32x4 *)(uintptr_t)addr;
}

// LDS swizzles (16-byte chunk index ^ f(row)).  A 256-byte bank cycle holds
// 256 / D rows of a tile.  Score reads take one chunk of each of 16 rows, so
// fp8_swz_k spreads the rows of one cycle and the cycles over the chunks;
// transposed value reads take two adjacent chunks of each of 8 rows, so
// fp8_swz_v moves chunk pairs.  Both depend on row % 16 only, so tiles 16 rows
// apart share a pattern.
template <int D>
__device__ __forceinline__ int fp8_swz_k(int r) {
  return (r / (256 / D)) & (D / 16 - 1);
}
template <int D>
__device__ __forceinline__ int fp8_swz_v(int r) {
  return 2 * ((r / (256 / D)) & (D / 32 - 1));
}

template <int D>
struct Fp8Cfg {
  static constexpr int BR = 128;             // query rows per workgroup
  static constexpr int BC = 64;              // keys per tile
  static constexpr int NKT = BC / 32;        // 32-key score tiles per K/V tile
  static constexpr int KS8 = D / 64;         // MFMA k-steps over the head dim
  static constexpr int CT = D / 32;          // 32-column output tiles
  static constexpr int RB = D;               // bytes per row
  static constexpr int CPR = RB / 16;        // 16-byte chunks per row
  static constexpr int RPI = 1024 / RB;      // rows per wave-wide 16-byte load
  static constexpr int TB = BC * RB;         // bytes per tile
  static constexpr int LPW = TB / 1024 / 4;  // loads per wave per tensor per tile
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256, (D == 256) ? 1 : 2)
fa_fwd_fp8_kernel(const uint8_t *__restrict__ Q, const uint8_t *__restrict__ K, const uint8_t *__restrict__ V,
                  __bf16 *__restrict__ O, float *__restrict__ LSE, int N, int nbh, int group, float score_log2e,
                  float v_scale) {
  using C = Fp8Cfg<D>;
  constexpr int TB = C::TB;
  constexpr int RB = C::RB;
  // LDS: K buffers at [0, TB) and [TB, 2TB), V buffers at [2TB, 3TB) and [3TB, 4TB)
  __shared__ __align__(1024) unsigned char smem[4 * TB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int nqb = (N + C::BR - 1) / C::BR;
  int bh, qb;
  map_block(blockIdx.x, nqb, nbh, CAUSAL, bh, qb);
  const size_t head_off = (size_t)bh * (size_t)N * D;          // query head: Q, O
  const size_t kv_off = (size_t)(bh / group) * (size_t)N * D;  // its K/V head
  const uint32_t head_bytes = (uint32_t)N * RB;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + kv_off, head_bytes);

  const int q0 = qb * C::BR;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + l32;

  // ---- Q fragments: B operand, lane = query row, 32 bytes = d in [64 ks + 32 half, +32)
  i32x8 qf[C::KS8];
  {
    const bool ok = my_q < N;
    const uint8_t *qrow = Q + head_off + (size_t)(ok ? my_q : 0) * D + 32 * half;
#pragma unroll
    for (int ks = 0; ks < C::KS8; ++ks) {
      const u32x4 lo = ok ? ld16(qrow + 64 * ks) : u32x4{0, 0, 0, 0};
      const u32x4 hi = ok ? ld16(qrow + 64 * ks + 16) : u32x4{0, 0, 0, 0};
      qf[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  }

  const int ntiles_all = (N + C::BC - 1) / C::BC;
  int ntiles = ntiles_all;
  if (CAUSAL) ntiles = min(ntiles_all, (min(q0 + C::BR, N) - 1) / C::BC + 1);

  // ---- direct loads: wave w fills rows [(w*LPW + u)*RPI, +RPI) of a tile
  const int ld_row_in = lane / C::CPR;
  const int ld_chunk = lane % C::CPR;
  auto issue = [&](__amdgpu_buffer_rsrc_t rs, int t, int lds_off, auto isv) {
    constexpr bool IS_V = decltype(isv)::value;
#pragma unroll
    for (int u = 0; u < C::LPW; ++u) {
      const int row0 = (wave * C::LPW + u) * C::RPI;
      const int row = row0 + ld_row_in;
      const int ch = ld_chunk ^ (IS_V ? fp8_swz_v<D>(row) : fp8_swz_k<D>(row));
      const uint32_t g = (uint32_t)(t * C::BC + row) * RB + 16u * ch;
      load_lds16(rs, smem + lds_off + row0 * RB, g);
    }
  };
  auto issue_k = [&](int t, int lds_off) { issue(krs, t, lds_off, std::false_type{}); };
  auto issue_v = [&](int t, int lds_off) { issue(vrs, t, lds_off, std::true_type{}); };

  // ---- per-lane LDS addresses
  // score A operand: K row 32 kt + swap_bits23(l32), chunks 4 ks + 2 half + j (j = 0, 1)
  const uint32_t sbase = lds_addr(smem);
  uint32_t kaddr[C::KS8][2];
  {
    const int r = swap_bits23(l32);
#pragma unroll
    for (int ks = 0; ks < C::KS8; ++ks)
#pragma unroll
      for (int j = 0; j < 2; ++j) kaddr[ks][j] = sbase + r * RB + 16 * ((4 * ks + 2 * half + j) ^ fp8_swz_k<D>(r));
  }
  // value A operand: lane i = l % 16 of 16-lane group G = l / 16 reads row 8 half + i / 2 (+ 16 g)
  // at column 32 ct + 16 (G & 1) + 8 (i & 1); it receives column 32 ct + 16 (G & 1) + i of 8 rows
  uint32_t vaddr[C::CT];
  {
    const int i = lane & 15;
    const int cg = (lane >> 4) & 1;
    const int r = 8 * half + (i >> 1);
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct)
      vaddr[ct] = sbase + 2 * TB + r * RB + 16 * ((2 * ct + cg) ^ fp8_swz_v<D>(r)) + 8 * (i & 1);
  }

  floatx16 oacc[C::CT];
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) oacc[ct] = floatx16{0};
  int pw[8] = {0, 0, 0, 0, 0, 0, 0, 0};  // packed P, every byte rewritten per tile
  floatx16 lsum = floatx16{0};  // every register: this lane's row sum of the rounded P
  float m_ref = -INFINITY;      // reference maximum of the raw (unscaled) scores
  const i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838, 0x38383838, 0x38383838, 0x38383838};  // E4M3 1.0

  // S^T of 32-key sub-tile kt of the K tile at byte offset KOFF
  auto scores = [&](auto koffc, floatx16 (&s)[C::NKT]) {
    constexpr int KOFF = decltype(koffc)::value;
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt) s[kt] = floatx16{0};
    static_for<C::NKT>([&](auto ktc) {
      constexpr int KT = decltype(ktc)::value;
#pragma unroll
      for (int ks = 0; ks < C::KS8; ++ks) {
        const i32x4 lo = lds_b128(kaddr[ks][0] + KOFF + 32 * KT * RB);
        const i32x4 hi = lds_b128(kaddr[ks][1] + KOFF + 32 * KT * RB);
        const i32x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        s[KT] = mfma_fp8(a, qf[ks], s[KT]);
      }
    });
  };

  auto step = [&](auto bufc, int t, floatx16 (&cur)[C::NKT], floatx16 (&nxt)[C::NKT]) {
    constexpr int BUF = decltype(bufc)::value;
    wait_vmem();
    __syncthreads();  // K(t+1) and V(t) are in LDS; nobody reads K(t) or V(t-1) any more
    if (t + 2 < ntiles) issue_k(t + 2, BUF * TB);
    if (t + 1 < ntiles) issue_v(t + 1, (2 + (BUF ^ 1)) * TB);
    const int kb = t * C::BC;
    const bool act = !CAUSAL || (kb <= qw0 + 31);
    if (!act) return;
    // ---- masking (diagonal and ragged tiles only)
    const bool need_mask = (CAUSAL && (kb + C::BC - 1 > qw0)) || (kb + C::BC > N);
    if (need_mask) {
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + 32 * kt + 16 * (r >> 3) + 8 * half + (r & 7);
          if ((key >= N) || (CAUSAL && key > my_q)) cur[kt][r] = -INFINITY;
        }
    }
    float mloc = max3f(cur[0][0], cur[0][1], cur[0][2]);
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
      for (int r = (kt == 0 ? 3 : 0); r < 16; r += 2) {
        if (r + 1 < 16) mloc = max3f(mloc, cur[kt][r], cur[kt][r + 1]);
        else mloc = fmaxf(mloc, cur[kt][r]);
      }
    const float m_new = fmaxf(m_ref, max_with_partner(mloc));
    const bool grow = (m_new - m_ref) * score_log2e > 8.0f;
    if (__ballot(grow) != 0) {
      const float alpha = (m_ref == -INFINITY) ? 0.f : fast_exp2((m_ref - m_new) * score_log2e);
      m_ref = (m_new == -INFINITY) ? m_ref : m_new;
#pragma unroll
      for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[ct][r] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) lsum[r] *= alpha;
    }
    const float mc = (m_ref == -INFINITY) ? 0.f : m_ref * score_log2e;
    // ---- scores of tile t+1 (independent of the softmax below; the last tile's are discarded)
    scores(std::integral_constant<int, (BUF ^ 1) * TB>{}, nxt);
    // ---- P of tile t as E4M3, byte 16 kt + r = key 32 kt + 16 (r / 8) + 8 half + r % 8
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float p0 = fast_exp2(__builtin_fmaf(cur[kt][4 * w + 0], score_log2e, -mc));
        const float p1 = fast_exp2(__builtin_fmaf(cur[kt][4 * w + 1], score_log2e, -mc));
        const float p2 = fast_exp2(__builtin_fmaf(cur[kt][4 * w + 2], score_log2e, -mc));
        const float p3 = fast_exp2(__builtin_fmaf(cur[kt][4 * w + 3], score_log2e, -mc));
        pw[4 * kt + w] = pack_fp8x2<true>(p2, p3, pack_fp8x2<false>(p0, p1, pw[4 * kt + w]));
      }
    const i32x8 pb = {pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};
    // ---- O^T += V^T P^T (one 64-key step per column tile) and the row sum
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
      constexpr int VOFF = BUF * TB;
      const i32x2 g0 = lds_tr8(vaddr[ct] + VOFF);
      const i32x2 g1 = lds_tr8(vaddr[ct] + VOFF + 16 * RB);
      const i32x2 g2 = lds_tr8(vaddr[ct] + VOFF + 32 * RB);
      const i32x2 g3 = lds_tr8(vaddr[ct] + VOFF + 48 * RB);
      const i32x8 a = {g0[0], g0[1], g1[0], g1[1], g2[0], g2[1], g3[0], g3[1]};
      oacc[ct] = mfma_fp8(a, pb, oacc[ct]);
    }
    lsum = mfma_fp8(ones, pb, lsum);
  };

  // ---- prologue: K(0), V(0), K(1) in flight, then S of tile 0
  issue_k(0, 0);
  issue_v(0, 2 * TB);
  if (ntiles > 1) issue_k(1, TB);
  floatx16 sA[C::NKT], sB[C::NKT];
  wait_vmem();
  __syncthreads();
  scores(std::integral_constant<int, 0>{}, sA);

  for (int t = 0; t < ntiles; t += 2) {
    step(std::integral_constant<int, 0>{}, t, sA, sB);
    if (t + 1 < ntiles) step(std::integral_constant<int, 1>{}, t + 1, sB, sA);
  }

  // ---- epilogue: O = v_scale O^T / l, lse = (m c + log2 l) ln 2
  const float l_tot = lsum[0];
  if (my_q < N) {
    const float inv = v_scale / l_tot;
    __bf16 *orow = O + head_off + (size_t)my_q * D;
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[ct][4 * j + 0] * inv, oacc[ct][4 * j + 1] * inv);
        w[1] = pack_bf16x2(oacc[ct][4 * j + 2] * inv, oacc[ct][4 * j + 3] * inv);
        st8(orow + 32 * ct + 8 * j + 4 * half, w);
      }
    }
    if (half == 0) LSE[(size_t)bh * N + my_q] = (m_ref * score_log2e + __log2f(l_tot)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const void *q, const void *k, const void *v, float q_scale, float k_scale, float v_scale,
                  void *o, float *lse, int B, int H, int group, int N, float scale, hipStream_t stream) {
  using C = Fp8Cfg<D>;
  const int nbh = B * H;
  const int nqb = (N + C::BR - 1) / C::BR;
  const long long blocks = (long long)nqb * nbh;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fa_fwd_fp8_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const uint8_t *)q, (const uint8_t *)k, (const uint8_t *)v, (__bf16 *)o, lse, N, nbh, group,
                     q_scale * k_scale * scale * kLog2e, v_scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const void *q, const void *k, const void *v, float q_scale, float k_scale, float v_scale,
                          void *o, float *lse, int B, int H, int group, int N, int d, bool causal, float scale,
                          hipStream_t stream) {
  if (d == 256)
    return causal ? launch<256, true>(q, k, v, q_scale, k_scale, v_scale, o, lse, B, H, group, N, scale, stream)
                  : launch<256, false>(q, k, v, q_scale, k_scale, v_scale, o, lse, B, H, group, N, scale, stream);
  if (d == 64)
    return causal ? launch<64, true>(q, k, v, q_scale, k_scale, v_scale, o, lse, B, H, group, N, scale, stream)
                  : launch<64, false>(q, k, v, q_scale, k_scale, v_scale, o, lse, B, H, group, N, scale, stream);
  return causal ? launch<128, true>(q, k, v, q_scale, k_scale, v_scale, o, lse, B, H, group, N, scale, stream)
                : launch<128, false>(q, k, v, q_scale, k_scale, v_scale, o, lse, B, H, group, N, scale, stream);
}

}  // namespace fa
