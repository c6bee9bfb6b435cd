// Host check of the argument checks and launch geometry of the attention
// entry points (csrc/plan.h), meant to run under AddressSanitizer and
// UndefinedBehaviorSanitizer: status codes for valid and invalid arguments,
// workspace sizes against their closed form, grid sizes within one dispatch
// (blocks * threads < 2^32, bounded combine grid) or ATTN_ERR_SHAPE, and
// messages that stay inside a short buffer.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <limits>

#include "plan.h"

using namespace attn;

static int bad = 0;
static long checks = 0;
#define CHECK(cond, ...)                      \
  do {                                        \
    ++checks;                                 \
    if (!(cond)) {                            \
      if (bad < 30) std::printf(__VA_ARGS__); \
      ++bad;                                  \
    }                                         \
  } while (0)

// Fake, suitably aligned device addresses: the checks never dereference them.
static const void* P(uintptr_t off) { return reinterpret_cast<const void*>(0x7f0000000000ull + off); }

int main() {
  char buf[512];
  plan::Msg m{buf, sizeof(buf)};
  const void *q = P(0), *k = P(1 << 20), *v = P(2 << 20), *o = P(3 << 20);
  const float* lse = static_cast<const float*>(P(4 << 20));

  // valid calls
  const int Ss[] = {1, 2, 17, 127, 128, 129, 4096, 65535, 1 << 20, (1 << 23) - 1};
  for (int D : {64, 128})
    for (int S : Ss)
      for (int causal : {0, 1}) {
        if ((int64_t)S * D * 2 > INT_MAX) continue;
        const int rc = plan::check_args(q, k, v, o, lse, 1, 2, S, S, D, 0.125f, causal, m);
        CHECK(rc == ATTN_OK, "valid S=%d D=%d causal=%d rejected: %s\n", S, D, causal, buf);
      }

  // invalid calls, one defect each
  struct Bad {
    const void *q, *k, *v, *o;
    const float* lse;
    int B, H, Sq, Sk, D;
    float scale;
    int causal, status;
  };
  const float inf = std::numeric_limits<float>::infinity();
  const Bad cases[] = {
      {nullptr, k, v, o, lse, 1, 1, 8, 8, 64, 0.1f, 0, ATTN_ERR_NULL},
      {q, k, v, o, nullptr, 1, 1, 8, 8, 64, 0.1f, 0, ATTN_ERR_NULL},
      {q, k, v, o, lse, 0, 1, 8, 8, 64, 0.1f, 0, ATTN_ERR_SHAPE},
      {q, k, v, o, lse, 1, INT_MIN, 8, 8, 64, 0.1f, 0, ATTN_ERR_SHAPE},
      {q, k, v, o, lse, 1, 1, 0, 8, 64, 0.1f, 0, ATTN_ERR_SHAPE},
      {q, k, v, o, lse, 1, 1, 8, -5, 64, 0.1f, 0, ATTN_ERR_SHAPE},
      {q, k, v, o, lse, INT_MAX, INT_MAX, INT_MAX, INT_MAX, 128, 0.1f, 0, ATTN_ERR_SHAPE},
      {q, k, v, o, lse, 1, 1, 1 << 23, 1 << 23, 128, 0.1f, 0, ATTN_ERR_SHAPE},
      {q, k, v, o, lse, 1, 1, 8, 8, 96, 0.1f, 0, ATTN_ERR_UNSUPPORTED},
      {q, k, v, o, lse, 1, 1, 8, 8, INT_MIN, 0.1f, 0, ATTN_ERR_UNSUPPORTED},
      {P(8), k, v, o, lse, 1, 1, 8, 8, 64, 0.1f, 0, ATTN_ERR_ALIGN},
      {q, k, v, o, static_cast<const float*>(P(4 << 20 | 2)), 1, 1, 8, 8, 64, 0.1f, 0,
       ATTN_ERR_ALIGN},
      {q, k, v, o, lse, 1, 1, 8, 8, 64, 0.1f, 2, ATTN_ERR_ARG},
      {q, k, v, o, lse, 1, 1, 8, 8, 64, std::nanf(""), 0, ATTN_ERR_ARG},
      {q, k, v, o, lse, 1, 1, 8, 8, 64, -inf, 0, ATTN_ERR_ARG},
      {q, k, v, o, lse, 1, 1, 9, 8, 64, 0.1f, 1, ATTN_ERR_SHAPE},  // causal S_q > S_k
  };
  for (const Bad& c : cases) {
    buf[0] = '\0';
    const int rc = plan::check_args(c.q, c.k, c.v, c.o, c.lse, c.B, c.H, c.Sq, c.Sk, c.D,
                                    c.scale, c.causal, m);
    CHECK(rc == c.status, "B=%d H=%d Sq=%d Sk=%d D=%d: status %d, expected %d\n", c.B, c.H,
          c.Sq, c.Sk, c.D, rc, c.status);
    CHECK(buf[0] != '\0' && std::strlen(buf) < sizeof(buf), "no message for status %d\n", rc);
  }

  // a message longer than its buffer is truncated inside it
  char tiny[8];
  std::memset(tiny, 'x', sizeof(tiny));
  plan::fail(plan::Msg{tiny, sizeof(tiny)}, ATTN_ERR_ARG, "%s", "a message of many characters");
  CHECK(tiny[sizeof(tiny) - 1] == '\0', "truncated message not terminated\n");
  CHECK(plan::fail(plan::Msg{nullptr, 0}, ATTN_ERR_HIP, "ignored") == ATTN_ERR_HIP, "null sink\n");

  // workspace sizes: closed form, and 0 for bad arguments
  for (int D : {64, 128})
    for (int S : {1, 300, 4096, 1 << 20})
      for (int ns : {1, 2, 7, ATTN_MAX_SPLITS}) {
        const size_t got = plan::workspace_size(3, 5, S, D, ns);
        const size_t want = ns == 1 ? 0 : (size_t)ns * 3 * 5 * (size_t)S * (D + 1) * 4;
        CHECK(got == want, "workspace D=%d S=%d ns=%d: %zu vs %zu\n", D, S, ns, got, want);
      }
  CHECK(plan::workspace_size(1, 1, 8, 64, 0) == 0, "ns=0\n");
  CHECK(plan::workspace_size(1, 1, 8, 64, ATTN_MAX_SPLITS + 1) == 0, "ns too large\n");
  CHECK(plan::workspace_size(INT_MAX, INT_MAX, INT_MAX, 128, 64) == 0, "overflow\n");

  // launch geometry over a range of shapes
  long launches = 0;
  for (int D : {64, 128})
    for (int causal : {0, 1})
      for (int64_t BH : {1LL, 3LL, 8LL, 256LL, 16400LL, 1LL << 20})
        for (int S : {1, 129, 4096, 1 << 16, 1 << 20})
          for (int ns : {1, 2, 64}) {
            const double elems = (double)BH * S * D;
            if (elems >= 1099511627776.0) continue;
            const int B = (int)(BH >= 4 ? BH / 4 : BH), H = (int)(BH >= 4 ? 4 : 1);
            plan::Launch L{};
            buf[0] = '\0';
            const int rc = plan::make_launch(B, H, S, D, causal, ns, &L, m);
            ++launches;
            const int64_t nq = (S + 127) / 128;
            const int64_t per_head = L.order == ORDER_FOLDED ? (nq + 1) / 2 : nq;
            const int64_t blocks = (int64_t)B * H * per_head * ns;
            if (rc == ATTN_OK) {
              CHECK(L.blocks == blocks, "blocks %lld vs %lld\n", (long long)L.blocks,
                    (long long)blocks);
              CHECK(L.blocks * plan::THREADS <= plan::MAX_WORK_ITEMS, "grid too large\n");
              CHECK(L.n_qtiles == nq, "n_qtiles\n");
              // folded mirror pairs exactly for causal single passes whose
              // pairs fill the CUs (the three-wave routing reads folds())
              const bool want_fold = causal && ns == 1 &&
                                     (int64_t)B * H * ((nq + 1) / 2) >= plan::FOLD_MIN_WORKGROUPS;
              CHECK((L.order == ORDER_FOLDED) == want_fold &&
                        plan::folds(B, H, S, causal, ns) == want_fold,
                    "fold order B=%d H=%d S=%d causal=%d ns=%d\n", B, H, S, causal, ns);
              CHECK(ns == 1 || (L.combine_blocks >= 1 &&
                                L.combine_blocks <= plan::COMBINE_MAX_BLOCKS),
                    "combine grid %lld\n", (long long)L.combine_blocks);
              CHECK(ns > 1 || L.combine_blocks == 0, "combine grid without splits\n");
              if (ns > 1) {
                // wave-per-row combine exactly when a thread per row and 4
                // columns would not fill the CUs once; the grid covers every
                // row (or is capped and strides)
                const int64_t rows = (int64_t)B * H * S;
                const bool runs = rows * (D / 4) < plan::COMBINE_FILL_THREADS;
                CHECK(L.combine_runs == (runs ? 1 : 0), "combine form\n");
                const int64_t per = runs ? plan::COMBINE_THREADS / 64 : plan::COMBINE_THREADS;
                const int64_t items = runs ? rows : rows * (D / 4);
                const int64_t want = std::min<int64_t>((items + per - 1) / per,
                                                       plan::COMBINE_MAX_BLOCKS);
                CHECK(L.combine_blocks == want, "combine blocks %lld vs %lld\n",
                      (long long)L.combine_blocks, (long long)want);
              }
              CHECK(ns == 1 || L.order == ORDER_TILES, "split launches use ORDER_TILES\n");
              CHECK(causal || ns > 1 || L.order == ORDER_HEADS, "non-causal order\n");
            } else {
              CHECK(rc == ATTN_ERR_SHAPE && buf[0] != '\0', "make_launch status %d\n", rc);
              CHECK(blocks * plan::THREADS > plan::MAX_WORK_ITEMS,
                    "rejected a grid that fits: %lld blocks\n", (long long)blocks);
            }
          }

  if (bad) {
    std::printf("FAIL: %d of %ld checks (%ld launch shapes)\n", bad, checks, launches);
    return 1;
  }
  std::printf("ok: %ld checks (%ld launch shapes)\n", checks, launches);
  return 0;
}
