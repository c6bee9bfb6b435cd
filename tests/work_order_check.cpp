// Host check of the workgroup -> (head, query tile) maps of work_order.h.
// For each order and a range of head counts and tile counts: every (head,
// query tile) is covered exactly once; ORDER_TILES issues the heaviest tiles
// first; ORDER_FOLDED pairs tile t with its mirror n_qtiles-1-t, so every
// workgroup folds n_qtiles+1 causal tile pairs (the unpaired middle tile of
// an odd count excepted); under ORDER_HEADS and ORDER_FOLDED the ids one XCD
// receives (x, x+8, ...) walk the head-major sequence in steps of one.
#include <cstdio>
#include <vector>

#include "work_order.h"

using namespace attn;

static int bad = 0;
#define CHECK(cond, ...)                         \
  do {                                           \
    if (!(cond)) {                               \
      if (bad < 20) std::printf(__VA_ARGS__);    \
      ++bad;                                     \
    }                                            \
  } while (0)

int main() {
  const int bhs[] = {1, 2, 3, 7, 8, 9, 16, 31, 32, 128};
  const int nqs[] = {1, 2, 3, 4, 31, 32, 33, 64, 129};
  const int orders[] = {ORDER_TILES, ORDER_HEADS, ORDER_FOLDED};
  long cases = 0;
  for (int order : orders)
    for (int BH : bhs)
      for (int nq : nqs) {
        ++cases;
        const int per_head = workgroups_per_head(order, nq);
        const int n = BH * per_head;
        std::vector<int> seen((size_t)BH * nq, 0);
        int prev_qt = nq;
        for (int bid = 0; bid < n; ++bid) {
          const TileWork w = work_of(order, bid, BH, nq);
          CHECK(w.bh >= 0 && w.bh < BH, "order %d BH %d nq %d bid %d: head %d\n", order, BH, nq,
                bid, w.bh);
          CHECK(w.qt_first >= 0 && w.qt_first < nq, "order %d: qt_first %d\n", order, w.qt_first);
          if (w.bh < 0 || w.bh >= BH || w.qt_first < 0 || w.qt_first >= nq) continue;
          seen[(size_t)w.bh * nq + w.qt_first]++;
          if (order == ORDER_FOLDED) {
            if (w.qt_second >= 0) {
              CHECK(w.qt_second < w.qt_first && w.qt_first + w.qt_second == nq - 1,
                    "fold BH %d nq %d bid %d: tiles %d %d\n", BH, nq, bid, w.qt_first, w.qt_second);
              if (w.qt_second < nq) seen[(size_t)w.bh * nq + w.qt_second]++;
              // causal tile t folds t+1 pairs of 64-key tiles
              CHECK((w.qt_first + 1) + (w.qt_second + 1) == nq + 1, "fold work\n");
            } else {
              CHECK(2 * w.qt_first == nq - 1, "fold BH %d nq %d bid %d: lone tile %d\n", BH, nq,
                    bid, w.qt_first);
            }
          } else {
            CHECK(w.qt_second == -1, "order %d: second tile %d\n", order, w.qt_second);
          }
          if (order == ORDER_TILES) {
            CHECK(w.qt_first <= prev_qt, "tiles BH %d nq %d bid %d: not heaviest first\n", BH, nq,
                  bid);
            prev_qt = w.qt_first;
          }
        }
        for (size_t t = 0; t < seen.size(); ++t)
          CHECK(seen[t] == 1, "order %d BH %d nq %d: (head %zu, tile %zu) covered %d times\n",
                order, BH, nq, t / nq, t % nq, seen[t]);
        if (order != ORDER_TILES) {
          for (int x = 0; x < XCDS; ++x) {
            int prev = -1;
            for (int bid = x; bid < n; bid += XCDS) {
              const TileWork w = work_of(order, bid, BH, nq);
              const int pos = w.bh * per_head + (nq - 1 - w.qt_first);
              CHECK(prev < 0 || pos == prev + 1, "order %d BH %d nq %d xcd %d: %d after %d\n",
                    order, BH, nq, x, pos, prev);
              prev = pos;
            }
          }
        }
      }
  if (bad) {
    std::printf("FAIL: %d violations over %ld cases\n", bad, cases);
    return 1;
  }
  std::printf("ok: %ld cases\n", cases);
  return 0;
}
