// Host check of the workgroup -> (head, row block) orders in fa_map.h, over a
// sweep of grid shapes.  Prints one line per violation and "ok N" at the end
// (N = grids checked), or "FAILED" and exit status 1.
//   * every (head, block) pair is taken by exactly one workgroup id;
//   * when the grid splits into whole heads per XCD (total % 8 == 0 and the
//     per-XCD share a multiple of the row blocks), a head's blocks all sit on
//     the XCD that ids of that residue go to (id % 8), and causal orders hand
//     out blocks heaviest first per XCD -- in every round for map_block, with
//     the odd full rounds reversed for map_block_balanced;
//   * the snake order does not widen the spread of per-position key-tile sums
//     for grids of up to three rounds (a CU at position p holds p, p+R, p+2R).
#include <cstdio>
#include <vector>

#include "fa_map.h"

static int fails = 0;
#define FAIL(...)                 \
  do {                            \
    if (fails < 40) {             \
      std::printf(__VA_ARGS__);   \
      std::printf("\n");          \
    }                             \
    ++fails;                      \
  } while (0)

static void check(int nqb, int nbh, bool causal, int round) {
  const int total = nqb * nbh;
  std::vector<int> seen(total, 0), bh_of(total), qb_of(total);
  for (int bid = 0; bid < total; ++bid) {
    int bh = -1, qb = -1;
    if (round >= 0) fa::map_block_balanced(bid, nqb, nbh, round, bh, qb);
    else fa::map_block(bid, nqb, nbh, causal, bh, qb);
    if (bh < 0 || bh >= nbh || qb < 0 || qb >= nqb) {
      FAIL("out of range: nqb %d nbh %d causal %d round %d bid %d -> (%d, %d)", nqb, nbh, causal, round, bid, bh, qb);
      return;
    }
    seen[bh * nqb + qb]++;
    bh_of[bid] = bh;
    qb_of[bid] = qb;
  }
  for (int i = 0; i < total; ++i)
    if (seen[i] != 1) {
      FAIL("pair (%d, %d) taken %d times: nqb %d nbh %d causal %d round %d", i / nqb, i % nqb, seen[i], nqb, nbh,
           causal, round);
      return;
    }
  const bool causal_order = causal || round >= 0;
  const int per_xcd = total / 8;
  if (total % 8 != 0 || per_xcd % nqb != 0) return;
  const int heads_here = per_xcd / nqb;
  for (int bid = 0; bid < total; ++bid)
    if (bh_of[bid] / heads_here != bid % 8)
      FAIL("head %d of bid %d not on XCD %d: nqb %d nbh %d round %d", bh_of[bid], bid, bid % 8, nqb, nbh, round);
  if (!causal_order) return;
  const int R = round > 0 ? round : per_xcd;
  for (int x = 0; x < 8; ++x)
    for (int local = 1; local < per_xcd; ++local) {
      const int r = local / R, r0 = (local - 1) / R;
      if (r != r0) continue;  // a new round
      const bool reversed = round > 0 && (r & 1) && (r + 1) * R <= per_xcd;
      const int a = qb_of[8 * (local - 1) + x], b = qb_of[8 * local + x];
      if (reversed ? (a > b) : (a < b))
        FAIL("order: nqb %d nbh %d round %d xcd %d local %d: %d then %d", nqb, nbh, round, x, local, a, b);
    }
  if (round > 0 && per_xcd <= 3 * round && per_xcd >= 2 * round) {
    // key tiles of a query block = its index + 1; spread of per-position sums
    auto spread = [&](bool snake) {
      int lo = 1 << 30, hi = 0;
      for (int x = 0; x < 8; ++x)
        for (int p = 0; p < round; ++p) {
          int sum = 0;
          for (int local = p; local < per_xcd; local += round) {
            int bh, qb;
            if (snake) fa::map_block_balanced(8 * local + x, nqb, nbh, round, bh, qb);
            else fa::map_block(8 * local + x, nqb, nbh, true, bh, qb);
            sum += qb + 1;
          }
          lo = sum < lo ? sum : lo;
          hi = sum > hi ? sum : hi;
        }
      return hi - lo;
    };
    if (spread(true) > spread(false))
      FAIL("snake widens the spread: nqb %d nbh %d round %d: %d > %d", nqb, nbh, round, spread(true), spread(false));
  }
}

int main() {
  int grids = 0;
  for (int nqb = 1; nqb <= 40; ++nqb)
    for (int nbh = 1; nbh <= 130; ++nbh) {
      check(nqb, nbh, false, -1);
      check(nqb, nbh, true, -1);
      for (int round : {0, 1, 4, 32})
        if (nqb * nbh <= 3 * 8 * 32 || round == 0) check(nqb, nbh, true, round);
      grids += 2;
    }
  // the named shapes: GPT-2 (8 blocks x 96 heads), the causal d=64 step (16 x 64), 32K causal (128 x 32)
  check(8, 96, true, 32);
  check(16, 64, true, 32);
  check(128, 32, true, -1);
  grids += 3;
  if (fails) {
    std::printf("FAILED: %d violations over %d grids\n", fails, grids);
    return 1;
  }
  std::printf("ok %d\n", grids);
  return 0;
}
