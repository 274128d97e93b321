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
// Head dims 32, 64, 96, 128 and 256 (d = 96 in a 128-column LDS layout whose
// last four chunks read as zero).  At d = 256 a wave's Q fragments (64 registers),
// output accumulator (128) and two score tiles (64) leave no room for a second
// wave per SIMD or for a second LDS fragment set, so that instantiation runs
// one wave per SIMD and reads each chunk's fragments just before use.
//
// Mapping to one workgroup (4 waves and BR = 128 query rows; 8 waves and BR =
// 256 at d = 96 and 128, where one K/V tile then serves twice the rows):
//   * Each wave owns 32 query rows.  Its Q rows sit in VGPRs as the B operand
//     of S^T = K Q^T (lane = query row, 8 consecutive head-dim slots per lane).
//   * A K/V tile of BC = 64 keys goes from HBM
//     straight into LDS with buffer_load ... lds (no staging registers).  K runs
//     one tile ahead of V: while tile j's softmax and P V product run, the
//     scores of tile j+1 are already being computed from LDS, and K(j+2) and
//     V(j+1) are in flight (two K and two V buffers, 64 KB).  Rows past the end
//     of the sequence come back as zero from the buffer descriptor's range
//     check.  Tiles are row-major with the 16-byte chunks of each row XOR-
//     permuted by a function of the row, so the score reads (16 rows, one chunk)
//     and the transposed value reads (4 rows, 4 chunks) hit distinct banks.
//   * S^T tiles (32 keys x 32 queries) use v_mfma_f32_32x32x16_bf16; each lane
//     ends up with one query row and 16 of its keys per tile, the other 16 in
//     the lane 32 away, so the row maximum needs one v_permlane32_swap.
//   * P = 2^(S c - m c), c = scale * log2(e), is rounded to bf16 and used as the
//     B operand of O^T += V^T P^T directly from registers.  The V^T operand is
//     read from the row-major V tile with ds_read_b64_tr_b16.  The row sum adds
//     the same bf16 P values the product uses (v_dot2c_f32_bf16).
//   * The running maximum only moves when a tile's maximum exceeds it by more
//     than 2^8 in exp2 units; O and l share the reference, so O / l is
//     unchanged and every P stays below 2^8.
//   * A tile step runs in chunks of 16 keys; each chunk's LDS fragments (K
//     rows for the next tile's scores, V^T rows for this tile's product) are
//     read one chunk ahead into a second register set, so their latency runs
//     under the previous chunk's matrix products.
//   * Causal: tiles entirely above the diagonal are never loaded; a wave whose
//     rows are all above a tile skips its math; only diagonal and ragged tiles
//     pay for masking.  Heaviest row blocks are dispatched first; when the
//     whole grid is resident at once (B8 H12 N1024 d64: 768 workgroups, three
//     per CU) the odd dispatch rounds go lightest first, so each CU's three
//     blocks sum to 24-30 key tiles instead of 20-34 (per-workgroup timestamps;
//     that launch 27.1 -> 25.5 us).
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

// A causal d = 64 launch splits each workgroup's key range (SPLIT below) when
// it would otherwise have at most this many 128-row workgroups, i.e. no more
// than one per CU: there the unsplit launch runs one wave per SIMD through
// the longest blocks' 16+ key tiles.  Measured: B2 H3 N1000 15.6 -> 10.3 us;
// at 384 and more workgroups (B4/B8 H12 N1024) the split's 64 KB of LDS per
// workgroup (2 per CU instead of 3) costs more than it saves (B8: 25 -> 31 us).
constexpr long long SPLIT_MAX_WG = 256;

// Sequence lengths from which d = 128 launches use the 64-rows-per-wave kernel.
constexpr int R64_MIN_N = 4096;
constexpr int R64_MIN_N_CAUSAL = 16384;

template <int D>
struct FwdCfg {
  // waves per workgroup: 8 at d = 96 and 128 (one K/V tile in LDS serves 256
  // query rows, about 3% faster than 4 waves), 4 otherwise
  static constexpr int NWV = (D == 96 || D == 128) ? 8 : 4;
  static constexpr int BR = 32 * NWV;               // query rows per workgroup
  static constexpr int BC = 64;                     // keys per tile
  static constexpr int NKT = BC / 32;               // 32-key score tiles per K/V tile
  static constexpr int KSTEPS = D / 16;             // MFMA k-steps over the head dim
  static constexpr int CT = D / 32;                 // 32-column output tiles
  // LDS rows are DL columns wide: d = 96 sits in a 128-column layout whose last
  // four 16-byte chunks read as zero
  static constexpr int DL = (D == 96) ? 128 : D;
  static constexpr int CPR = DL / 8;                // 16-byte chunks per LDS row
  static constexpr int ROW_BYTES = DL * 2;          // bytes per LDS row
  static constexpr int GROW_BYTES = D * 2;          // bytes per row in global memory
  static constexpr int RPI = 1024 / ROW_BYTES;      // rows per wave-wide 16-byte load
  static constexpr int TILE_BYTES = BC * ROW_BYTES;
  static constexpr int LPW = TILE_BYTES / 1024 / NWV; // loads per wave per tensor per tile
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;
};


// SPLIT (causal d = 64 launches with few workgroups): a workgroup owns 64 query
// rows; waves 0-1 (one per 32 rows) take the lower half of the key tiles the
// rows see and waves 2-3 the upper half, each pair with its own LDS buffers, and
// the two partial results are merged at the end by the online-softmax rule
// (m = max(m0, m1), O and l rescaled by 2^((m_i - m) c)).  The last query blocks
// of a causal launch walk every key tile; splitting their keys halves that
// sequential chain when there are too few workgroups to hide it.
template <int D, bool CAUSAL, bool SPLIT>
__global__ void __launch_bounds__(64 * FwdCfg<D>::NWV, SPLIT ? 2 : ((D == 256) ? 1 : (D == 64) ? 3 : 8 / FwdCfg<D>::NWV))
fa_fwd_bf16_kernel(const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K,
                   const __bf16 *__restrict__ V, __bf16 *__restrict__ O, float *__restrict__ LSE,
                   int N, int nbh, int group, float scale_log2e, int xcd_round) {
  using C = FwdCfg<D>;
  static_assert(!SPLIT || (CAUSAL && C::NWV == 4), "the key split is built for 4-wave causal launches");
  constexpr int TB = C::TILE_BYTES;
  constexpr int RB = C::ROW_BYTES;
  constexpr int RG = SPLIT ? 2 : C::NWV;              // waves along the query rows
  constexpr int BRW = 32 * RG;                        // query rows per workgroup
  constexpr int LPW = C::TILE_BYTES / 1024 / RG;      // loads per wave per tensor per tile
  // LDS: K buffers at [0, TB) and [TB, 2TB), V buffers at [2TB, 3TB) and [3TB, 4TB);
  // with SPLIT a second such set at [4TB, 8TB) for the upper key half
  __shared__ __align__(1024) unsigned char smem[(SPLIT ? 8 : 4) * TB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int rg = SPLIT ? (wave & 1) : wave;  // 32-row group of this wave
  const int kh = SPLIT ? (wave >> 1) : 0;    // key half of this wave
  const int hb = kh * 4 * TB;                // LDS buffers of that key half

  const int nqb = (N + BRW - 1) / BRW;
  int bh, qb;
  if (CAUSAL && xcd_round > 0) map_block_balanced(blockIdx.x, nqb, nbh, xcd_round, bh, qb);
  else map_block(blockIdx.x, nqb, nbh, CAUSAL, bh, qb);

  const size_t head_off = (size_t)bh * (size_t)N * D;          // query head: Q, O
  const size_t kv_off = (size_t)(bh / group) * (size_t)N * D;  // its K/V head (group query heads share one)
  const uint32_t head_bytes = (uint32_t)N * C::GROW_BYTES;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + kv_off, head_bytes);

  const int q0 = qb * BRW;         // first query row of the workgroup
  const int qw0 = q0 + rg * 32;    // first query row of this wave
  const int my_q = qw0 + l32;      // this lane's query row

  // ---- Q fragments: B operand, lane = query row, slots = d in [16*ks + 8*half, +8)
  bf16x8 qf[C::KSTEPS];
  {
    const bool ok = my_q < N;
    const __bf16 *qrow = Q + head_off + (size_t)(ok ? my_q : 0) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) qf[ks] = as_bf16x8(ok ? ld16(qrow + 16 * ks) : u32x4{0, 0, 0, 0});
  }

  // ---- number of key tiles this workgroup visits
  const int ntiles_all = (N + C::BC - 1) / C::BC;
  int ntiles = ntiles_all;
  if (CAUSAL) ntiles = min(ntiles_all, (min(q0 + BRW, N) - 1) / C::BC + 1);
  // key tiles [t_lo, t_hi) of this wave's key half, visited in nsteps steps
  const int nsteps = SPLIT ? (ntiles + 1) / 2 : ntiles;
  const int t_lo = kh * nsteps;
  const int t_hi = SPLIT ? (kh ? ntiles : nsteps) : ntiles;

  // ---- direct loads: wave w fills rows [(w*LPW + u)*RPI, +RPI) of a tile
  const int ld_row_in = lane / C::CPR;
  const int ld_chunk = lane % C::CPR;
  // global byte offset of 16-byte chunk c of key row `row`; chunks past the row
  // (padding of a d = 96 layout) get an offset beyond the buffer, which reads zero
  auto goff = [&](int row, int c) -> uint32_t {
    if constexpr (C::DL != D)
      if (c >= D / 8) return 0x80000000u;
    return (uint32_t)row * C::GROW_BYTES + 16u * c;
  };
  auto issue_k = [&](int t, int lds_off) {
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const int row0 = (rg * LPW + u) * C::RPI;
      const int row = row0 + ld_row_in;
      load_lds16(krs, smem + hb + lds_off + row0 * RB, goff(t * C::BC + row, ld_chunk ^ swz_k<C::DL>(row)));
    }
  };
  auto issue_v = [&](int t, int lds_off) {
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const int row0 = (rg * LPW + u) * C::RPI;
      const int row = row0 + ld_row_in;
      load_lds16(vrs, smem + hb + lds_off + row0 * RB, goff(t * C::BC + row, ld_chunk ^ swz_v<C::DL>(row)));
    }
  };

  // ---- per-lane LDS offsets, hoisted out of the loop.  Rows 16 and 32 apart
  // share a swizzle, so tile/row/buffer displacements are compile-time constants.
  // score A operand: K row 32*kt + swap_bits23(l32), logical chunk 2*ks + half
  int koff[C::KSTEPS];
  {
    const int r = swap_bits23(l32);
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) koff[ks] = r * RB + 16 * ((2 * ks + half) ^ swz_k<C::DL>(r));
  }
  // value A operand (transposed read): lane j = l & 15 of its 16-lane group
  // addresses row key0 + (j >> 2), columns 32*ct + 16*((l >> 4) & 1) + 4*(j & 3)
  uint32_t voff[C::CT][2];
  {
    const uint32_t vb = lds_addr(smem) + hb + 2 * TB;
    const int rlo = 8 * half + ((lane & 15) >> 2);
    const int tq = lane & 3;
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
      const int ch = 4 * ct + 2 * ((lane >> 4) & 1) + (tq >> 1);
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int r = rlo + 4 * hi;
        voff[ct][hi] = vb + r * RB + 16 * (ch ^ swz_v<C::DL>(r)) + 8 * (tq & 1);
      }
    }
  }

  floatx16 oacc[C::CT];
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) oacc[ct] = floatx16{0};
  float m_ref = -INFINITY;  // running reference maximum of raw scores q.k
  float l_part = 0.f;       // this lane's part of the running exponential sum

  // S^T of one 32-key sub-tile, k-steps [k0, k0 + n) into acc
  auto qk_steps = [&](floatx16 &acc, const unsigned char *kbuf, int kt, int k0, int n) {
    bf16x8 a[C::KSTEPS];
#pragma unroll
    for (int i = 0; i < C::KSTEPS; ++i)
      if (i < n) a[i] = as_bf16x8(ld16(kbuf + koff[k0 + i] + 32 * kt * RB));
#pragma unroll
    for (int i = 0; i < C::KSTEPS; ++i)
      if (i < n) acc = mfma32x32x16(a[i], qf[k0 + i], acc);
  };

  constexpr int NCH = 2 * C::NKT;            // P chunks of 8 keys per lane per tile
  constexpr int QK_PER_CH = C::KSTEPS / 2;   // score MFMAs of the next tile per chunk

  // LDS fragments of one chunk: K rows for QK_PER_CH score k-steps of the next
  // tile and V^T rows for one 16-key slice of the current tile
  struct Frag {
    u32x4 k[QK_PER_CH];
    u32x2 v[C::CT][2];
  };
  const uint32_t kbase = lds_addr(smem) + hb;
  uint32_t kaddr[C::KSTEPS];
#pragma unroll
  for (int ks = 0; ks < C::KSTEPS; ++ks) kaddr[ks] = kbase + koff[ks];
  auto read_frag = [&](auto bufc, auto cc, Frag &f) {
    constexpr int BUF = decltype(bufc)::value;
    constexpr int CH = decltype(cc)::value;
    constexpr int first = CH * QK_PER_CH;
    constexpr int kt = first / C::KSTEPS;
    constexpr int k0 = first % C::KSTEPS;
    constexpr int KOFF = (BUF ^ 1) * TB + 32 * kt * RB;   // K buffer of tile t+1
    constexpr int VOFF = BUF * TB + (16 * CH) * RB;       // V buffer of tile t, rows 16 CH..
#pragma unroll
    for (int i = 0; i < QK_PER_CH; ++i) f.k[i] = ds_read_b128_at<KOFF>(kaddr[k0 + i]);
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
      f.v[ct][0] = ds_read_tr16_at<VOFF>(voff[ct][0]);
      f.v[ct][1] = ds_read_tr16_at<VOFF>(voff[ct][1]);
    }
  };
  auto frag_wait = [&](Frag &f) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < QK_PER_CH; ++i) redefine(f.k[i]);
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
      redefine(f.v[ct][0]);
      redefine(f.v[ct][1]);
    }
  };

  // Masked row maximum of one tile's scores, both halves of the wave combined.
  // Diagonal and ragged tiles get -inf at the keys a row must not see.
  auto tile_max = [&](floatx16 (&s)[C::NKT], int t) -> float {
    const int kb = t * C::BC;
    const bool need_mask = (CAUSAL && (kb + C::BC - 1 > qw0)) || (kb + C::BC > N);
    if (need_mask) {
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + 32 * kt + 16 * (r >> 3) + 8 * half + (r & 7);
          if ((key >= N) || (CAUSAL && key > my_q)) s[kt][r] = -INFINITY;
        }
    }
    float mloc = max3f(s[0][0], s[0][1], s[0][2]);
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
      for (int r = (kt == 0 ? 3 : 0); r < 16; r += 2) {
        if (r + 1 < 16) mloc = max3f(mloc, s[kt][r], s[kt][r + 1]);
        else mloc = fmaxf(mloc, s[kt][r]);
      }
    return max_with_partner(mloc);
  };
  // Only the mask of tile_max (used while the reference stays at the first tile's maximum).
  auto mask_only = [&](floatx16 (&s)[C::NKT], int t) {
    const int kb = t * C::BC;
    const bool need_mask = (CAUSAL && (kb + C::BC - 1 > qw0)) || (kb + C::BC > N);
    if (need_mask) {
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + 32 * kt + 16 * (r >> 3) + 8 * half + (r & 7);
          if ((key >= N) || (CAUSAL && key > my_q)) s[kt][r] = -INFINITY;
        }
    }
  };
  // At d = 64, 96 and 256 the maximum of tile t+1 is taken at the end of step t,
  // while that step's last matrix products still run, instead of after the
  // barrier that starts step t+1, where every wave of a SIMD would do it at
  // once with the matrix cores idle (1-4% faster there; at d = 32 and 128 no
  // gain).  mt carries it to the next step.  At d = 256 the move of the
  // reference maximum it may cause is made there too (REF_AT_TAIL).
  constexpr bool EARLY_MAX = (D == 64 || D == 96 || D == 256);
  constexpr bool REF_AT_TAIL = (D == 256);

  // Move the reference maximum only when a tile's scores outgrow it by more than
  // 2^8 (in exp2 units); O and l are rescaled with it.
  auto update_ref = [&](float m_tile) {
    const float m_new = fmaxf(m_ref, m_tile);
    const bool grow = (m_new - m_ref) * scale_log2e > 8.0f;
    if (__ballot(grow) != 0) {
      const float alpha = (m_ref == -INFINITY) ? 0.f : fast_exp2((m_ref - m_new) * scale_log2e);
      m_ref = (m_new == -INFINITY) ? m_ref : m_new;
      l_part *= alpha;
      if constexpr (D == 256) {
        // the accumulators live in AGPRs here; pinning them there at this point
        // keeps the compiler from copying all of them to VGPRs on every step
        // (outside this rarely taken branch) for the multiply below
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct) asm volatile("" : "+a"(oacc[ct]));
      }
#pragma unroll
      for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[ct][r] *= alpha;
    }
  };

  // One tile step.  BUF is the V buffer of tile t (and the K buffer of tile t).
  auto step = [&](auto fastc, auto bufc, int t, floatx16 (&cur)[C::NKT], floatx16 (&nxt)[C::NKT], float &mt) {
    constexpr bool FAST = decltype(fastc)::value;
    constexpr int BUF = decltype(bufc)::value;
    wait_vmem();
    __syncthreads();  // K(t+1) and V(t) are in LDS; nobody reads K(t) or V(t-1) any more
    if (t + 2 < t_hi) issue_k(t + 2, BUF * TB);
    if (t + 1 < t_hi) issue_v(t + 1, (2 + (BUF ^ 1)) * TB);

    const int kb = t * C::BC;
    const bool act = !CAUSAL || (kb <= qw0 + 31);

    Frag fa, fb;
    // fragments one chunk ahead at d = 64 and 128; at d = 256 a second set does not
    // fit, and at d = 32 a chunk has too little work to hide the reads behind
    constexpr bool AHEAD = (D == 64 || D == 96 || D == 128);
    if (AHEAD && act) read_frag(bufc, std::integral_constant<int, 0>{}, fa);
    float mc = 0.f;
    if (act) {
      // ---- row maximum of tile t (masked) and the reference maximum; with FAST
      // the reference stays at the first tile's maximum and only the mask is applied
      if constexpr (FAST) {
        if constexpr (!EARLY_MAX) mask_only(cur, t);
      } else if constexpr (!EARLY_MAX) {
        update_ref(tile_max(cur, t));
      } else if constexpr (!REF_AT_TAIL) {
        update_ref(mt);
      }
      mc = (m_ref == -INFINITY) ? 0.f : m_ref * scale_log2e;
    }

    // ---- P of tile t, O^T += V^T P^T, interleaved with S^T of tile t+1.
    // Chunk CH covers keys [16 CH, 16 CH + 16) of tile t (8 per lane) and
    // score k-steps [CH QK_PER_CH, +QK_PER_CH) of tile t+1.  Its LDS fragments
    // are read one chunk ahead, into the other of two register sets.
    auto chunk_p = [&](int kt, int m) -> bf16x8 {
      u32x4 pw;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = fast_exp2(__builtin_fmaf(cur[kt][8 * m + 2 * i], scale_log2e, -mc));
        const float p1 = fast_exp2(__builtin_fmaf(cur[kt][8 * m + 2 * i + 1], scale_log2e, -mc));
        pw[i] = pack_bf16x2(p0, p1);
        l_part = add_bf16_pair(pw[i], l_part);
      }
      return as_bf16x8(pw);
    };
    // (a wave that is active for tile t but not for t+1 -- the last tile, or
    // the causal diagonal -- computes scores it will not use; they are discarded)
    if (act) {
      static_for<NCH>([&](auto cc) {
        constexpr int CH = decltype(cc)::value;
        Frag &f = (CH % 2 == 0) ? fa : fb;
        Frag &g = (CH % 2 == 0) ? fb : fa;
        const bf16x8 pb = chunk_p(CH / 2, CH % 2);
        if constexpr (!AHEAD) read_frag(bufc, cc, f);
        frag_wait(f);
        if constexpr (AHEAD && CH + 1 < NCH) read_frag(bufc, std::integral_constant<int, CH + 1>{}, g);
        constexpr int first = CH * QK_PER_CH;
        constexpr int kt = first / C::KSTEPS;
        constexpr int k0 = first % C::KSTEPS;
        if constexpr (k0 == 0) nxt[kt] = floatx16{0};
#pragma unroll
        for (int i = 0; i < QK_PER_CH; ++i) nxt[kt] = mfma32x32x16(as_bf16x8(f.k[i]), qf[k0 + i], nxt[kt]);
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct) {
          const u32x4 av = {f.v[ct][0][0], f.v[ct][0][1], f.v[ct][1][0], f.v[ct][1][1]};
          oacc[ct] = mfma32x32x16(as_bf16x8(av), pb, oacc[ct]);
        }
      });
      if constexpr (EARLY_MAX) {
        const bool act1 = (t + 1 < t_hi) && (!CAUSAL || ((t + 1) * C::BC <= qw0 + 31));
        if (act1) {
          if constexpr (FAST) {
            mask_only(nxt, t + 1);
          } else {
            mt = tile_max(nxt, t + 1);
            if constexpr (REF_AT_TAIL) update_ref(mt);
          }
        }
      }
    }
  };

  // ---- prologue: K(t_lo), V(t_lo), K(t_lo+1) in flight, then S of tile t_lo
  // (an empty upper key half -- a block that sees one tile -- loads nothing).
  // The loop runs first with FAST: the reference maximum is the first tile's
  // row maximum and is never moved, so no later tile needs a row maximum
  // (probabilities keep their relative precision at any magnitude; O and l share
  // the reference).  If a row sum then exceeds 2^64 or O is not finite, the
  // workgroup runs the loop again with the moving reference.  Key-split (SPLIT)
  // launches, a few tiles per workgroup, use the moving reference directly.
  floatx16 sA[C::NKT], sB[C::NKT];
  auto run = [&](auto fastc) {
    constexpr bool FAST = decltype(fastc)::value;
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) oacc[ct] = floatx16{0};
    m_ref = -INFINITY;
    l_part = 0.f;
    if (t_lo < t_hi) {
      issue_k(t_lo, 0);
      issue_v(t_lo, 2 * TB);
    }
    if (t_lo + 1 < t_hi) issue_k(t_lo + 1, TB);
    wait_vmem();
    __syncthreads();
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt) {
      sA[kt] = floatx16{0};
      qk_steps(sA[kt], smem + hb, kt, 0, C::KSTEPS);
    }

    float mt = 0.f;
    if constexpr (FAST) {
      update_ref(tile_max(sA, t_lo));
    } else if constexpr (EARLY_MAX) {
      mt = tile_max(sA, t_lo);
      if constexpr (REF_AT_TAIL) update_ref(mt);
    }
    // (tiles at or past t_hi are above the diagonal of every row here, so the
    // causal test in step() leaves them inactive)
    for (int s = 0; s < nsteps; s += 2) {
      step(fastc, std::integral_constant<int, 0>{}, t_lo + s, sA, sB, mt);
      if (s + 1 < nsteps) step(fastc, std::integral_constant<int, 1>{}, t_lo + s + 1, sB, sA, mt);
    }
    // every LDS read of the loop was waited for inside its step; this wait makes
    // that visible to the static check of the generated code, which scans it in
    // text order (the loop's wait may be laid out before its last reads)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  if constexpr (SPLIT) {
    // small launches (a few tiles per workgroup): the moving reference directly
    run(std::false_type{});
  } else {
    run(std::true_type{});
    float osum = 0.f;
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) osum += oacc[ct][r];
    constexpr float kLMax = 18446744073709551616.f;  // 2^64
    const bool bad = !(l_part <= kLMax) || !(__builtin_fabsf(osum) <= 3.0e38f);
    if (__syncthreads_or(bad)) run(std::false_type{});
  }

  if constexpr (SPLIT) {
    // ---- merge the upper key half into the lower one: per lane its running
    // maximum, exponential sum and O^T registers, through LDS
    constexpr int XF = 2 + 16 * C::CT;  // floats per lane
    float *xs = reinterpret_cast<float *>(smem) + rg * XF * 64;
    __syncthreads();  // every wave is done reading K/V tiles
    if (kh == 1) {
      xs[lane] = m_ref;
      xs[64 + lane] = l_part;
#pragma unroll
      for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) xs[(2 + 16 * ct + r) * 64 + lane] = oacc[ct][r];
    }
    __syncthreads();
    if (kh == 1) return;
    const float m1 = xs[lane];
    const float m = fmaxf(m_ref, m1);
    const float a0 = (m_ref == -INFINITY) ? 0.f : fast_exp2((m_ref - m) * scale_log2e);
    const float a1 = (m1 == -INFINITY) ? 0.f : fast_exp2((m1 - m) * scale_log2e);
    l_part = a0 * l_part + a1 * xs[64 + lane];
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[ct][r] = a0 * oacc[ct][r] + a1 * xs[(2 + 16 * ct + r) * 64 + lane];
    if (m != -INFINITY) m_ref = m;
  }

  // ---- epilogue: O = O^T / l, lse = (m c + log2 l) ln 2
  const float l_tot = sum_with_partner(l_part);
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
    if (half == 0) LSE[(size_t)bh * N + my_q] = (m_ref * scale_log2e + __log2f(l_tot)) * kLn2;
  }
}

template <int D, bool CAUSAL, bool SPLIT = false>
hipError_t launch(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int group,
                  int N, float scale, hipStream_t stream) {
  using C = FwdCfg<D>;
  const int nbh = B * H;
  const int br = SPLIT ? 64 : C::BR;
  const int nqb = (N + br - 1) / br;
  const long long blocks = (long long)nqb * nbh;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // causal grids that are resident all at once: the snake order of map_block_balanced
  int xcd_round = 0;
  if (CAUSAL && !SPLIT) {
    static std::atomic<int> per_cu{0};
    xcd_round = snake_round(fa_fwd_bf16_kernel<D, CAUSAL, SPLIT>, 64 * C::NWV, blocks, per_cu);
  }
  hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, CAUSAL, SPLIT>), dim3((unsigned)blocks), dim3(64 * C::NWV), 0, stream,
                     (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, (__bf16 *)o, lse, N, nbh, group,
                     scale * kLog2e, xcd_round);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                           int group, int N, int d, bool causal, float scale, hipStream_t stream) {
  if (d == 96) return causal ? launch<96, true>(q, k, v, o, lse, B, H, group, N, scale, stream)
                             : launch<96, false>(q, k, v, o, lse, B, H, group, N, scale, stream);
  if (d == 32) return causal ? launch<32, true>(q, k, v, o, lse, B, H, group, N, scale, stream)
                             : launch<32, false>(q, k, v, o, lse, B, H, group, N, scale, stream);
  if (d == 64) {
    if (!causal) return launch<64, false>(q, k, v, o, lse, B, H, group, N, scale, stream);
    const long long wg128 = (long long)B * H * ((N + 127) / 128);
    if (wg128 <= SPLIT_MAX_WG) return launch<64, true, true>(q, k, v, o, lse, B, H, group, N, scale, stream);
    return launch<64, true>(q, k, v, o, lse, B, H, group, N, scale, stream);
  }
  if (d == 256) return causal ? launch<256, true>(q, k, v, o, lse, B, H, group, N, scale, stream)
                              : launch<256, false>(q, k, v, o, lse, B, H, group, N, scale, stream);
  // d = 128, long sequences: the kernel with 64 query rows per wave (fa_fwd_bf16_r64.hip),
  // 2-3% faster there; shorter and causal launches below 16K keep this kernel, whose
  // finer 32-row waves balance the causal diagonal better (the other kernel is 3%
  // slower at B2 H16 N4096 causal and at B8 H16 N1024)
  if (causal ? (N >= R64_MIN_N_CAUSAL) : (N >= R64_MIN_N))
    return launch_fwd_bf16_r64(q, k, v, o, lse, B, H, group, N, causal, scale, stream);
  return causal ? launch<128, true>(q, k, v, o, lse, B, H, group, N, scale, stream)
                : launch<128, false>(q, k, v, o, lse, B, H, group, N, scale, stream);
}

}  // namespace fa
