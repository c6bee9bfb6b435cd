// Workgroup id -> (batch*head, query tiles) for the attention forward
// launches. Plain C++ (no HIP types) so that host tests can check it.
#pragma once

#if defined(__HIPCC__)
#define ATTN_HD __host__ __device__
#else
#define ATTN_HD
#endif

namespace attn {

constexpr int XCDS = 8;  // MI355X dies; workgroup ids are dealt round-robin over them

// Work orders of a single-pass launch.
//  ORDER_TILES: grid B*H*n_qtiles, the heaviest query tiles first across all
//    heads (longest-first packing of causal work).
//  ORDER_HEADS: grid B*H*n_qtiles; each XCD takes a contiguous range of the
//    head-major sequence of (head, query tile), so the workgroups resident on
//    an XCD share one or two heads' K/V in its L2.
//  ORDER_FOLDED (causal): grid B*H*ceil(n_qtiles/2); a workgroup takes query
//    tile n_qtiles-1-u and then its mirror u, so all workgroups fold the same
//    number of key tiles (n_qtiles + 1 pairs); (head, u) are dealt to XCDs in
//    head-major order as above.
// A split-KV launch uses ORDER_TILES with the run index varying fastest.
enum : int { ORDER_TILES = 0, ORDER_HEADS = 1, ORDER_FOLDED = 2 };

struct TileWork {
  int bh;         // batch*head index
  int qt_first;   // first query tile
  int qt_second;  // second query tile (ORDER_FOLDED), or -1
};

ATTN_HD inline int workgroups_per_head(int order, int n_qtiles) {
  return order == ORDER_FOLDED ? (n_qtiles + 1) / 2 : n_qtiles;
}

// bid in [0, BH * workgroups_per_head(order, n_qtiles)).
ATTN_HD inline TileWork work_of(int order, int bid, int BH, int n_qtiles) {
  TileWork w;
  w.qt_second = -1;
  if (order == ORDER_TILES) {
    w.qt_first = n_qtiles - 1 - bid / BH;
    w.bh = bid % BH;
    return w;
  }
  // XCD x receives ids x, x+8, x+16, ...: give it the x-th contiguous share.
  const int per_head = workgroups_per_head(order, n_qtiles);
  const int n = BH * per_head;
  const int x = bid % XCDS, i = bid / XCDS;
  const int rem = n % XCDS;
  const int pos = x * (n / XCDS) + (x < rem ? x : rem) + i;
  w.bh = pos / per_head;
  const int u = pos % per_head;
  w.qt_first = n_qtiles - 1 - u;
  if (order == ORDER_FOLDED && u != w.qt_first) w.qt_second = u;
  return w;
}

}  // namespace attn
