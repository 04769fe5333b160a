// Host driver for the key-chunk rules of fa_api_common.hpp: reads lines
// "wgs N causal cus" from stdin and prints, for each, the forward's split-KV
// chunks (fa_api::default_splits) and the backward dQ pass's chunks
// (fa_api::bwd_dq_splits, which ignores causal).
#include <cstdio>

#include "fa_api_common.hpp"

int main() {
  long long wgs, n, causal, cus;
  while (std::scanf("%lld %lld %lld %lld", &wgs, &n, &causal, &cus) == 4)
    std::printf("%d %d\n", fa_api::default_splits(wgs, n, causal != 0, cus), fa_api::bwd_dq_splits(wgs, n, cus));
  return 0;
}
