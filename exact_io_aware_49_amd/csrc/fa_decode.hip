// fa_decode.hip -- attention of a few new query rows against a key/value cache.
//
// The serving case of the pages' "Spezialisierte Lösungen" ("FlashAttention
// (DE)", section "Evolution und Weiterentwicklungen": FlashInfer streams the
// KV cache during generation).  Nq query rows per sequence (the last Nq
// positions) attend to the first L_b rows of the sequence's cache.  With
// little query work per byte of cache the kernel is bound by reading K and V
// once from HBM, and the work is laid out for that:
//
// A segment is one block of up to 32 query rows of one K/V head of one
// sequence: the (query head, query) pairs of the head's group, all against
// the same cache rows.  The 32-key tiles of all segments, segment after
// segment, form one list of T tiles.  fa_decode_kernel runs one wave per SIMD
// of the GPU (W waves, all resident at once; fewer when there are fewer than 8
// tiles per wave) and gives wave w the tiles [w T / W, (w+1) T / W) of that
// list: every wave streams the same number of tiles from the start of the
// kernel to its end, whatever the mix of cache lengths, so there are no gaps
// where waves end and new ones start up.  A wave's range crosses segment
// boundaries; at each boundary it writes a float32 (O, lse) partial for the
// rows of the segment it leaves and starts the next one, while its load
// pipeline keeps streaming across the boundary (the next segment's Q rows
// arrive through a fifth LDS buffer, ahead of its first tile).  The waves of
// a workgroup are independent (no barriers): each streams its own 32-key K
// and V tiles into its own double-buffered LDS area with buffer_load ... lds
// and computes S^T = K Q^T and O^T += V^T P^T on bf16 matrix cores exactly as
// the forward does.  Cache rows at or past a sequence's length are never
// read (the buffer range ends there and such rows load as zero).
//
// Partials are stored per (wave w, segment s) pair at slot w + s: along the
// tile list both w and s only grow and each new pair grows one of them, so
// w + s is distinct for every pair and below W + S.  The wave that handles a
// segment's first tile and the one that handles its last tile record their
// numbers; the merge kernel then combines the slots of those waves with the
// online-softmax rule (lse = ln sum e^lse_p, O = sum e^(lse_p - lse) O_p).
#include <atomic>

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
  static constexpr int TB = BC * RB;         // bytes per tile (and per 32 query rows)
  static constexpr int LPT = TB / 1024;      // wave-wide loads per tile and tensor
  static constexpr int WAVE_LDS = 5 * TB;    // K0, K1, V0, V1, the next segment's Q
};

// each wave in use gets at least this many tiles
constexpr int kMinTilesPerWave = 8;

__device__ __forceinline__ int seq_len(const int *lens, int b, int Nk) {
  const int l = lens ? lens[b] : Nk;
  return min(max(l, 0), Nk);
}

// Wave-uniform position in the tile list.
struct Cursor {
  int b, hk, rb;  // segment: row block rb of K/V head hk of sequence b
  int tile;       // tile within the segment
  int ntl;        // tiles of sequence b (each of its segments has this many)
  int len;        // cache rows of sequence b
};

// Cache lengths of 64 consecutive sequences, one per lane, for wave-uniform lookups.
struct LenChunk {
  int base;  // first sequence of the chunk
  int lens;  // this lane's: the length of sequence base + lane (0 past B)
};

__device__ __forceinline__ void load_chunk(LenChunk &lc, const int *lens, int base, int B, int Nk, int lane) {
  lc.base = base;
  lc.lens = (base + lane < B) ? seq_len(lens, base + lane, Nk) : 0;
}

// length of sequence b (wave-uniform); moves the chunk forward when b has left it
__device__ __forceinline__ int chunk_len(LenChunk &lc, const int *lens, int b, int B, int Nk, int lane) {
  if (b - lc.base >= 64) load_chunk(lc, lens, b & ~63, B, Nk, lane);
  return __builtin_amdgcn_readlane(lc.lens, b - lc.base);
}

// Next tile of the list (sequences without cache rows have no tiles and are
// skipped); past the last tile b becomes B.
__device__ __forceinline__ void advance(Cursor &c, LenChunk &lc, const int *lens, int B, int Hkv, int nrb, int Nk,
                                        int lane) {
  if (++c.tile < c.ntl) return;
  c.tile = 0;
  if (++c.rb < nrb) return;
  c.rb = 0;
  if (++c.hk < Hkv) return;
  c.hk = 0;
  while (++c.b < B) {
    c.len = chunk_len(lc, lens, c.b, B, Nk, lane);
    c.ntl = (c.len + 31) / 32;
    if (c.ntl > 0) return;
  }
}

__device__ __forceinline__ long long uniform_ll(long long x) {
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)x);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((unsigned long long)x >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

// sum over the wave, as a wave-uniform value
__device__ __forceinline__ long long wave_sum(long long x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return uniform_ll(x);
}

__device__ __forceinline__ long long wave_incl_scan(long long x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256)
fa_decode_kernel(const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K, const __bf16 *__restrict__ V,
                 const int *__restrict__ kv_lens, float *__restrict__ Opart, float *__restrict__ Lpart,
                 int *__restrict__ segw, int B, int Hq, int Hkv, int Nq, int Nk, int nrb, int rpb, int W,
                 float scale_log2e) {
  using C = DecCfg<D>;
  constexpr int TB = C::TB;
  constexpr int RB = C::RB;
  __shared__ __align__(1024) unsigned char smem[4 * C::WAVE_LDS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int w = blockIdx.x * 4 + wave;
  if (w >= W) return;  // the waves share no barrier
  const int group = Hq / Hkv;
  const int segs_b = Hkv * nrb;  // segments per sequence

  // ---- this wave's range [g0, g1) of the tile list
  auto tiles_of = [&](int b) -> long long {
    return b < B ? (long long)segs_b * ((seq_len(kv_lens, b, Nk) + 31) / 32) : 0;
  };
  long long T = 0;
  for (int c0 = 0; c0 < B; c0 += 64) T += wave_sum(tiles_of(c0 + lane));
  // waves in use: at most one per kMinTilesPerWave tiles, so that each has a
  // non-empty range and the merge no more partials than it needs
  long long Wu = T / kMinTilesPerWave;
  Wu = Wu < 1 ? 1 : (Wu > W ? W : Wu);
  if (w >= Wu) return;
  const long long g0 = uniform_ll((long long)w * T / Wu);
  const long long g1 = uniform_ll((long long)(w + 1) * T / Wu);
  if (g0 >= g1) return;
  // the sequence holding tile g0
  long long before = 0;
  int b0 = 0;
  for (int c0 = 0; c0 < B; c0 += 64) {
    const long long tb = tiles_of(c0 + lane);
    const long long incl = wave_incl_scan(tb, lane);
    const unsigned long long hit = __ballot(before + incl > g0);
    if (hit) {
      const int j = __builtin_ctzll(hit);
      b0 = c0 + j;
      before += uniform_ll(__shfl(incl - tb, j, 64));
      break;
    }
    before += uniform_ll(__shfl(incl, 63, 64));
  }
  Cursor ci;
  LenChunk lc;
  {
    ci.b = __builtin_amdgcn_readfirstlane(b0);
    load_chunk(lc, kv_lens, ci.b & ~63, B, Nk, lane);
    ci.len = chunk_len(lc, kv_lens, ci.b, B, Nk, lane);
    ci.ntl = (ci.len + 31) / 32;
    const int o = __builtin_amdgcn_readfirstlane((int)(g0 - before));  // tiles into sequence b0
    const int si = o / ci.ntl;
    ci.tile = o - si * ci.ntl;
    ci.hk = si / nrb;
    ci.rb = si - ci.hk * nrb;
  }
  Cursor cc = ci;  // the tile being computed; ci runs one tile ahead of it

  unsigned char *wl = smem + wave * C::WAVE_LDS;  // this wave's K0, K1, V0, V1, Q
  const int ld_row = lane / C::CPR;
  const int ld_chunk = lane % C::CPR;
  auto issue = [&](const Cursor &c, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const size_t kv_off = ((size_t)c.b * Hkv + c.hk) * (size_t)Nk * D;
    const uint32_t seq_bytes = (uint32_t)c.len * RB;  // rows past the sequence read as zero
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + kv_off, seq_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + kv_off, seq_bytes);
    const int r0 = c.tile * C::BC;
#pragma unroll
    for (int u = 0; u < C::LPT; ++u) {
      const int row0 = u * C::RPI;
      const int r = row0 + ld_row;
      load_lds16(krs, wl + BUF * TB + row0 * RB, (uint32_t)(r0 + r) * RB + 16u * (ld_chunk ^ swz_k<D>(r)));
      load_lds16(vrs, wl + (2 + BUF) * TB + row0 * RB, (uint32_t)(r0 + r) * RB + 16u * (ld_chunk ^ swz_v<D>(r)));
    }
  };
  // Q rows of segment c (the rows of a K/V head's group are consecutive in Q)
  auto issue_q = [&](const Cursor &c) {
    const int nv = min(32, group * Nq - c.rb * 32);
    const size_t q_off = (((size_t)c.b * Hq + (size_t)c.hk * group) * Nq + (size_t)c.rb * 32) * D;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + q_off, (uint32_t)nv * RB);
#pragma unroll
    for (int u = 0; u < C::LPT; ++u) {
      const int row0 = u * C::RPI;
      const int r = row0 + ld_row;
      load_lds16(qrs, wl + 4 * TB + row0 * RB, (uint32_t)r * RB + 16u * (ld_chunk ^ swz_k<D>(r)));
    }
  };

  // per-lane LDS addresses: score A operand (K row swap_bits23(l32), chunk 2 ks + half),
  // the Q operand (row l32) and the transposed V reads
  const uint32_t wbase = lds_addr(wl);
  uint32_t kaddr[C::KSTEPS];
  uint32_t qaddr[C::KSTEPS];
  {
    const int r = swap_bits23(l32);
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      kaddr[ks] = wbase + r * RB + 16 * ((2 * ks + half) ^ swz_k<D>(r));
      qaddr[ks] = wbase + l32 * RB + 16 * ((2 * ks + half) ^ swz_k<D>(l32));
    }
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

  bf16x8 qf[C::KSTEPS];
  floatx16 oacc[C::CT];
  float m_run = -INFINITY;  // running maximum of the raw scores of this row
  float l_part = 0.f;       // this lane's part of the exponential sum
  int pos = 0;              // this row's position in its sequence (causal)
  int kfree = 0;            // keys below this need no mask in any row of the segment

  auto tile = [&](auto bufc, long long g) {
    constexpr int BUF = decltype(bufc)::value;
    bool next_new_segment = false;
    if (g + 1 < g1) {
      advance(ci, lc, kv_lens, B, Hkv, nrb, Nk, lane);
      issue(ci, std::integral_constant<int, BUF ^ 1>{});
      next_new_segment = ci.tile == 0;
      // tile g (and the Q rows of its segment, loaded before it) have landed
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * C::LPT) : "memory");
    } else {
      wait_vmem();
    }
    if (g == g0 || cc.tile == 0) {
      // a new segment: its Q rows, its rows' positions, fresh accumulators
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) {
        u32x4 t = ds_read_b128_at<4 * TB>(qaddr[ks]);
        lds_wait(t);
        qf[ks] = as_bf16x8(t);
      }
      const int row = cc.rb * 32 + l32;
      pos = cc.len - Nq + (row % Nq);
      kfree = CAUSAL ? min(cc.len, cc.len - Nq + 1) : cc.len;
#pragma unroll
      for (int ct = 0; ct < C::CT; ++ct) oacc[ct] = floatx16{0};
      m_run = -INFINITY;
      l_part = 0.f;
    }
    // S^T of the 32 keys of tile g: lane = query row, registers = keys
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
    const int kb = cc.tile * C::BC;
    if (kb + C::BC > kfree) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb + 16 * (r >> 3) + 8 * half + (r & 7);
        if (key >= cc.len || (CAUSAL && key > pos)) s[r] = -INFINITY;
      }
    }
    float mloc = max3f(s[0], s[1], s[2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) mloc = max3f(mloc, s[r], s[r + 1]);
    mloc = fmaxf(mloc, s[15]);
    // (a row that has seen no visible key yet has m = -inf, gets alpha = 0
    // and P = 0, and keeps O = 0, l = 0)
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

    if (cc.tile == cc.ntl - 1 || g + 1 == g1) {
      // this wave's part of the segment ends: O normalised by its own sum, lse in natural log
      const int s_idx = (cc.b * Hkv + cc.hk) * nrb + cc.rb;
      const long long slot = (long long)w + s_idx;
      const int nv = min(32, group * Nq - cc.rb * 32);
      const float l_tot = sum_with_partner(l_part);
      if (l32 < nv) {
        const bool any = l_tot > 0.f;
        const float inv = any ? 1.f / l_tot : 0.f;
        float *op = Opart + (slot * rpb + l32) * D;
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const floatx4 v4 = {oacc[ct][4 * j] * inv, oacc[ct][4 * j + 1] * inv, oacc[ct][4 * j + 2] * inv,
                                oacc[ct][4 * j + 3] * inv};
            *reinterpret_cast<floatx4 *>(op + 32 * ct + 8 * j + 4 * half) = v4;
          }
        if (half == 0)
          Lpart[slot * rpb + l32] = any ? (m_run * scale_log2e + __log2f(l_tot)) * kLn2 : -INFINITY;
      }
    }
    if (lane == 0) {
      const int s_idx = (cc.b * Hkv + cc.hk) * nrb + cc.rb;
      if (cc.tile == 0) segw[2 * s_idx] = w;
      if (cc.tile == cc.ntl - 1) segw[2 * s_idx + 1] = w;
    }
    // the staging area is free again: bring in the next segment's Q rows
    if (next_new_segment) issue_q(ci);
    cc = ci;
  };

  issue_q(ci);
  issue(ci, std::integral_constant<int, 0>{});
  for (long long g = g0; g < g1; g += 2) {
    tile(std::integral_constant<int, 0>{}, g);
    if (g + 1 < g1) tile(std::integral_constant<int, 1>{}, g + 1);
  }
}

// Merge the partials of each query row, for segments with few partials.  One wave per row: the row's segment,
// its first and last wave, the largest lse over the slots, then lanes in 8
// groups sum e^(lse_p - m) O_p over every 8th slot (each lane D/8 columns) and
// the groups are added in a fixed order, so the result is bitwise
// reproducible.  A row whose sequence has no cache rows gets O = 0, lse = -inf.
template <int D>
__global__ void __launch_bounds__(256)
fa_decode_merge_kernel(const float *__restrict__ Opart, const float *__restrict__ Lpart,
                       const int *__restrict__ segw, const int *__restrict__ kv_lens, __bf16 *__restrict__ O,
                       float *__restrict__ LSE, int B, int Hq, int Hkv, int Nq, int Nk, int nrb, int rpb, int W) {
  constexpr int CPL = D / 8;  // columns per lane
  const int lane = threadIdx.x & 63;
  const int pg = lane >> 3;    // slot group
  const int cl = lane & 7;     // column block
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long long)B * Hq * Nq) return;
  const int qi = (int)(row % Nq);
  const long long bh = row / Nq;
  const int hq = (int)(bh % Hq);
  const int b = (int)(bh / Hq);
  const int group = Hq / Hkv;
  const int hk = hq / group;
  const int rig = (hq - hk * group) * Nq + qi;  // row within the K/V head's group
  const int rb = rig / 32;
  const int rin = rig - rb * 32;
  const int s_idx = (b * Hkv + hk) * nrb + rb;
  float acc[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) acc[j] = 0.f;
  float lse_out = -INFINITY;
  // the segment's first and last wave, loaded together with the sequence length
  // (one round trip; for an empty sequence they are stale and go unused)
  const int sw0 = segw[2 * s_idx], sw1 = segw[2 * s_idx + 1];
  if (seq_len(kv_lens, b, Nk) > 0) {
    // (clamped, so that no value can send a read outside the partial slots)
    const int wf = min(max(sw0, 0), W - 1);
    const int wl = min(max(sw1, wf), W - 1);
    const int np = wl - wf + 1;
    const float *lp = Lpart + ((long long)wf + s_idx) * rpb + rin;
    // each slot group: online-softmax merge of its slots (loads of all its
    // slots are independent of the arithmetic)
    float mg = -INFINITY, sg = 0.f;
    for (int p0 = pg; p0 < np; p0 += 32) {
      float L[4];
      floatx4 v[4][CPL / 4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int p = p0 + 8 * u;
        L[u] = -INFINITY;
#pragma unroll
        for (int j = 0; j < CPL / 4; ++j) v[u][j] = floatx4{0, 0, 0, 0};
        if (p < np) {
          L[u] = lp[(long long)p * rpb];
          const floatx4 *op = reinterpret_cast<const floatx4 *>(
              Opart + (((long long)wf + p + s_idx) * rpb + rin) * D + CPL * cl);
#pragma unroll
          for (int j = 0; j < CPL / 4; ++j) v[u][j] = op[j];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (L[u] > mg) {
          const float f = (mg == -INFINITY) ? 0.f : expf(mg - L[u]);
          sg *= f;
#pragma unroll
          for (int j = 0; j < CPL; ++j) acc[j] *= f;
          mg = L[u];
        }
        const float wgt = (L[u] == -INFINITY) ? 0.f : expf(L[u] - mg);
        sg += wgt;
#pragma unroll
        for (int j = 0; j < CPL / 4; ++j) {
          acc[4 * j] += wgt * v[u][j][0];
          acc[4 * j + 1] += wgt * v[u][j][1];
          acc[4 * j + 2] += wgt * v[u][j][2];
          acc[4 * j + 3] += wgt * v[u][j][3];
        }
      }
    }
    // combine the 8 groups in a fixed order
    float m = mg;
#pragma unroll
    for (int o = 8; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (m != -INFINITY) {
      const float f = (mg == -INFINITY) ? 0.f : expf(mg - m);
      float sum = sg * f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) acc[j] *= f;
#pragma unroll
      for (int o = 8; o < 64; o <<= 1) {
        sum += __shfl_xor(sum, o, 64);
#pragma unroll
        for (int j = 0; j < CPL; ++j) acc[j] += __shfl_xor(acc[j], o, 64);
      }
#pragma unroll
      for (int j = 0; j < CPL; ++j) acc[j] /= sum;
      lse_out = m + logf(sum);
    }
  }
  if (pg == 0) {
    u32x4 wv[CPL / 8];
#pragma unroll
    for (int j = 0; j < CPL / 8; ++j)
      wv[j] = u32x4{pack_bf16x2(acc[8 * j], acc[8 * j + 1]), pack_bf16x2(acc[8 * j + 2], acc[8 * j + 3]),
                    pack_bf16x2(acc[8 * j + 4], acc[8 * j + 5]), pack_bf16x2(acc[8 * j + 6], acc[8 * j + 7])};
    u32x4 *orow = reinterpret_cast<u32x4 *>(O + row * D + CPL * cl);
#pragma unroll
    for (int j = 0; j < CPL / 8; ++j) orow[j] = wv[j];
  }
  if (lane == 0) LSE[row] = lse_out;
}

// The same for segments with many partials (a few long sequences).  One workgroup per row: the row's
// segment and its first and last wave give the partial slots; 32 lane groups
// (8 per wave, each lane D/8 columns) merge every 32nd slot with the online-
// softmax rule, the groups of a wave combine through cross-lane sums and the
// four waves through LDS, always in the same order, so the result is bitwise
// reproducible.  A row whose sequence has no cache rows gets O = 0, lse = -inf.
template <int D>
__global__ void __launch_bounds__(256)
fa_decode_merge_wide_kernel(const float *__restrict__ Opart, const float *__restrict__ Lpart,
                       const int *__restrict__ segw, const int *__restrict__ kv_lens, __bf16 *__restrict__ O,
                       float *__restrict__ LSE, int B, int Hq, int Hkv, int Nq, int Nk, int nrb, int rpb, int W) {
  constexpr int CPL = D / 8;  // columns per lane
  __shared__ float red_m[4], red_s[4];
  __shared__ floatx4 red_acc[4][8][CPL / 4];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int grp = wv * 8 + (lane >> 3);  // slot group 0..31
  const int cl = lane & 7;               // column block
  const long long row = blockIdx.x;
  const int qi = (int)(row % Nq);
  const long long bh = row / Nq;
  const int hq = (int)(bh % Hq);
  const int b = (int)(bh / Hq);
  const int group = Hq / Hkv;
  const int hk = hq / group;
  const int rig = (hq - hk * group) * Nq + qi;  // row within the K/V head's group
  const int rb = rig / 32;
  const int rin = rig - rb * 32;
  const int s_idx = (b * Hkv + hk) * nrb + rb;
  float acc[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) acc[j] = 0.f;
  float mg = -INFINITY, sg = 0.f;
  // the segment's first and last wave, loaded together with the sequence length
  // (one round trip; for an empty sequence they are stale and go unused)
  const int sw0 = segw[2 * s_idx], sw1 = segw[2 * s_idx + 1];
  const bool any_rows = seq_len(kv_lens, b, Nk) > 0;
  if (any_rows) {
    // (clamped, so that no value can send a read outside the partial slots)
    const int wf = min(max(sw0, 0), W - 1);
    const int wl = min(max(sw1, wf), W - 1);
    const int np = wl - wf + 1;
    const float *lp = Lpart + ((long long)wf + s_idx) * rpb + rin;
    for (int p0 = grp; p0 < np; p0 += 128) {
      float L[4];
      floatx4 v[4][CPL / 4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int p = p0 + 32 * u;
        L[u] = -INFINITY;
#pragma unroll
        for (int j = 0; j < CPL / 4; ++j) v[u][j] = floatx4{0, 0, 0, 0};
        if (p < np) {
          L[u] = lp[(long long)p * rpb];
          const floatx4 *op = reinterpret_cast<const floatx4 *>(
              Opart + (((long long)wf + p + s_idx) * rpb + rin) * D + CPL * cl);
#pragma unroll
          for (int j = 0; j < CPL / 4; ++j) v[u][j] = op[j];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (L[u] > mg) {
          const float f = (mg == -INFINITY) ? 0.f : expf(mg - L[u]);
          sg *= f;
#pragma unroll
          for (int j = 0; j < CPL; ++j) acc[j] *= f;
          mg = L[u];
        }
        const float wgt = (L[u] == -INFINITY) ? 0.f : expf(L[u] - mg);
        sg += wgt;
#pragma unroll
        for (int j = 0; j < CPL / 4; ++j) {
          acc[4 * j] += wgt * v[u][j][0];
          acc[4 * j + 1] += wgt * v[u][j][1];
          acc[4 * j + 2] += wgt * v[u][j][2];
          acc[4 * j + 3] += wgt * v[u][j][3];
        }
      }
    }
    // combine the 8 groups of this wave
    float m = mg;
#pragma unroll
    for (int o = 8; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const float f = (mg == -INFINITY) ? 0.f : expf(mg - m);
    sg *= f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) acc[j] *= f;
#pragma unroll
    for (int o = 8; o < 64; o <<= 1) {
      sg += __shfl_xor(sg, o, 64);
#pragma unroll
      for (int j = 0; j < CPL; ++j) acc[j] += __shfl_xor(acc[j], o, 64);
    }
    mg = m;
  }
  // combine the four waves
  if (lane < 8) {
#pragma unroll
    for (int j = 0; j < CPL / 4; ++j)
      red_acc[wv][cl][j] = floatx4{acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]};
    if (lane == 0) {
      red_m[wv] = mg;
      red_s[wv] = sg;
    }
  }
  __syncthreads();
  if (wv != 0 || lane >= 8) return;
  float m = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
  float out[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) out[j] = 0.f;
  float lse_out = -INFINITY;
  if (any_rows && m != -INFINITY) {
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = (red_m[w] == -INFINITY) ? 0.f : expf(red_m[w] - m);
      sum += f * red_s[w];
#pragma unroll
      for (int j = 0; j < CPL / 4; ++j) {
        const floatx4 a = red_acc[w][cl][j];
        out[4 * j] += f * a[0];
        out[4 * j + 1] += f * a[1];
        out[4 * j + 2] += f * a[2];
        out[4 * j + 3] += f * a[3];
      }
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) out[j] /= sum;
    lse_out = m + logf(sum);
  }
  u32x4 *orow = reinterpret_cast<u32x4 *>(O + row * D + CPL * cl);
#pragma unroll
  for (int j = 0; j < CPL / 8; ++j)
    orow[j] = u32x4{pack_bf16x2(out[8 * j], out[8 * j + 1]), pack_bf16x2(out[8 * j + 2], out[8 * j + 3]),
                    pack_bf16x2(out[8 * j + 4], out[8 * j + 5]), pack_bf16x2(out[8 * j + 6], out[8 * j + 7])};
  if (lane == 0) LSE[row] = lse_out;
}

template <int D, bool CAUSAL>
hipError_t launch(const void *q, const void *k, const void *v, const int *kv_lens, void *o, float *lse, void *ws,
                  int B, int Hq, int Hkv, int Nq, int Nk, float scale, hipStream_t stream) {
  const DecodePlan p = decode_plan(B, Hq, Hkv, Nq, Nk, D);
  // one wave per SIMD: four per compute unit at d = 128 (one workgroup's 160 KB
  // of LDS), eight at d = 64 (two workgroups of 80 KB)
  long long W = (D == 64 ? 8LL : 4LL) * cu_count();
  if (W > kDecodeMaxWaves) W = kDecodeMaxWaves;
  const long long tmax = p.segments * (((long long)Nk + 31) / 32);
  if (W > tmax) W = tmax;
  unsigned char *base = static_cast<unsigned char *>(ws);
  float *opart = reinterpret_cast<float *>(base);
  float *lpart = reinterpret_cast<float *>(base + p.lpart_offset);
  int *segw = reinterpret_cast<int *>(base + p.segw_offset);
  hipLaunchKernelGGL((fa_decode_kernel<D, CAUSAL>), dim3((unsigned)((W + 3) / 4)), dim3(256), 0, stream,
                     (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, kv_lens, opart, lpart, segw, B, Hq, Hkv,
                     Nq, Nk, p.nrb, p.rpb, (int)W, scale * kLog2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long nrows = (long long)B * Hq * Nq;
  // about W / segments partials per segment: many of them get a workgroup per row
  if (W >= 32 * p.segments)
    hipLaunchKernelGGL((fa_decode_merge_wide_kernel<D>), dim3((unsigned)nrows), dim3(256), 0, stream,
                       (const float *)opart, (const float *)lpart, (const int *)segw, kv_lens, (__bf16 *)o, lse, B, Hq,
                       Hkv, Nq, Nk, p.nrb, p.rpb, (int)W);
  else
    hipLaunchKernelGGL((fa_decode_merge_kernel<D>), dim3((unsigned)((nrows + 3) / 4)), dim3(256), 0, stream,
                       (const float *)opart, (const float *)lpart, (const int *)segw, kv_lens, (__bf16 *)o, lse, B, Hq,
                       Hkv, Nq, Nk, p.nrb, p.rpb, (int)W);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const void *q, const void *k, const void *v, const int *kv_lens, void *o, float *lse,
                              void *ws, int B, int Hq, int Hkv, int Nq, int Nk, int d, bool causal, float scale,
                              hipStream_t stream) {
  if (d == 64)
    return causal ? launch<64, true>(q, k, v, kv_lens, o, lse, ws, B, Hq, Hkv, Nq, Nk, scale, stream)
                  : launch<64, false>(q, k, v, kv_lens, o, lse, ws, B, Hq, Hkv, Nq, Nk, scale, stream);
  return causal ? launch<128, true>(q, k, v, kv_lens, o, lse, ws, B, Hq, Hkv, Nq, Nk, scale, stream)
                : launch<128, false>(q, k, v, kv_lens, o, lse, ws, B, Hq, Hkv, Nq, Nk, scale, stream);
}

}  // namespace fa
