// Host driver for the key-chunk rules of fa_api_common.hpp: reads lines
// "wgs N causal cus fp8" from stdin and prints, for each, the forward's
// split-KV chunks (fa_api::default_splits) and the backward dQ pass's chunks
// (fa_api::bwd_dq_splits, which ignores causal and fp8).
#include <cstdio>

#include "fa_api_common.hpp"

int main() {
  long long wgs, n, causal, cus, fp8;
  while (std::scanf("%lld %lld %lld %lld %lld", &wgs, &n, &causal, &cus, &fp8) == 5)
    std::printf("%d %d\n", fa_api::default_splits(wgs, n, causal != 0, cus, fp8 != 0),
                fa_api::bwd_dq_splits(wgs, n, cus));
  return 0;
}
