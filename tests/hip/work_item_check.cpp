// Host-side check of the forward/backward kernels' block -> work-item map
// (work_item in fa_fwd_kernel.hpp, compiled here for the host only): for many
// (heads, query tiles, splits, causal) shapes every block index must land on a
// distinct item and every item must be covered; both causal orders must hand
// each head's tiles on one XCD out longest first, and order 2 with whole heads per XCD each
// XCD's slots longest first across its heads.
// Prints "ok <shapes checked>" and exits 0, or names the first failing shape.
#include <cstdio>
#include <vector>

#include "fa_fwd_kernel.hpp"

int main() {
  int shapes = 0;
  for (int bh = 1; bh <= 70; ++bh)
    for (int nq : {1, 2, 3, 7, 16, 33})
      for (int splits : {1, 3})
        for (int causal = 0; causal < 3; ++causal) {
          const int per_head = nq * splits, total = bh * per_head;
          std::vector<int> seen(total, 0);
          std::vector<int> last_rank(8, -1), last_head_rank(8 * bh, -1);
          for (int bid = 0; bid < total; ++bid) {
            int h, t;
            fa::work_item(bid, total, per_head, causal, h, t);
            if (h < 0 || h >= bh || t < 0 || t >= per_head) {
              std::printf("out of range: bh=%d nq=%d splits=%d causal=%d bid=%d -> (%d, %d)\n", bh, nq,
                          splits, causal, bid, h, t);
              return 1;
            }
            ++seen[h * per_head + t];
            if (causal) {
              // a head's tiles on one XCD, in dispatch order: non-increasing query tile
              const int rank = per_head - 1 - t, key = 8 * h + (bid & 7);
              if (rank < last_head_rank[key]) {
                std::printf("head not longest-first: bh=%d nq=%d splits=%d causal=%d bid=%d\n", bh, nq,
                            splits, causal, bid);
                return 1;
              }
              last_head_rank[key] = rank;
            }
            if (causal == 2 && total % 8 == 0 && (total / 8) % per_head == 0) {
              // slots of one XCD in dispatch order: non-increasing query tile
              const int x = bid & 7, rank = per_head - 1 - t;
              if (rank < last_rank[x]) {
                std::printf("not longest-first: bh=%d nq=%d splits=%d bid=%d\n", bh, nq, splits, bid);
                return 1;
              }
              last_rank[x] = rank;
            }
          }
          for (int i = 0; i < total; ++i)
            if (seen[i] != 1) {
              std::printf("item %d covered %d times: bh=%d nq=%d splits=%d causal=%d\n", i, seen[i], bh, nq,
                          splits, causal);
              return 1;
            }
          ++shapes;
        }
  std::printf("ok %d\n", shapes);
  return 0;
}
