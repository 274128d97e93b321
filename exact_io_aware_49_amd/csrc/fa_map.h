// fa_map.h -- order in which a launch's workgroups take (head, row block)
// pairs.  Plain integer code, callable on the host as well, so a host test can
// check every grid shape for a one-to-one mapping.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

// Map the linear workgroup id to (batch*head, row block) for grids of
// nbh * nqb workgroups.  Workgroups are
// dispatched round-robin over the 8 XCDs; grouping consecutive ids of one XCD
// onto the same heads keeps a head's K/V in that XCD's L2.  Causal launches
// put the highest row blocks first (the heaviest for a query-block owner).
__host__ __device__ inline void map_block(int bid, int nqb, int nbh, bool causal, int &bh, int &qb) {
  const int total = nqb * nbh;
  int id = bid;
  if ((total & 7) == 0) {
    const int per_xcd = total >> 3;
    id = (bid & 7) * per_xcd + (bid >> 3);
  }
  if (causal) {
    const int per_xcd = ((total & 7) == 0) ? (total >> 3) : total;
    const int base = (id / per_xcd) * per_xcd;
    const int local = id - base;
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

// map_block for causal launches whose workgroups are all resident at once.
// Each XCD hands its workgroups to its compute units in rounds of `round`
// (its CU count), the same CU order every round, so a CU runs the workgroups at
// positions p, p + round, p + 2 round, ... of the XCD's list.  Heaviest first in
// every round would give the first CUs the heaviest block of every round; here
// the odd rounds run lightest first, so the blocks a CU holds together sum to
// about the same number of key tiles everywhere (a snake order).  round = 0, or
// a grid that does not split evenly over the XCDs, gives map_block's order.
__host__ __device__ inline void map_block_balanced(int bid, int nqb, int nbh, int round, int &bh, int &qb) {
  const int total = nqb * nbh;
  const int per_xcd = total >> 3;
  if (round <= 0 || (total & 7) != 0 || per_xcd % nqb != 0) {
    map_block(bid, nqb, nbh, true, bh, qb);
    return;
  }
  const int x = bid & 7;
  int local = bid >> 3;
  const int r = local / round;
  const int pos = local - r * round;
  if ((r & 1) && (r + 1) * round <= per_xcd) local = r * round + (round - 1 - pos);
  const int heads_here = per_xcd / nqb;
  bh = x * heads_here + local % heads_here;
  qb = nqb - 1 - local / heads_here;
}

}  // namespace fa
