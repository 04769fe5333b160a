// Host driver for fa_api::default_splits (fa_api_common.hpp): reads lines
// "wgs N causal cus" from stdin and prints the number of key chunks for each.
#include <cstdio>

#include "fa_api_common.hpp"

int main() {
  long long wgs, n, causal, cus;
  while (std::scanf("%lld %lld %lld %lld", &wgs, &n, &causal, &cus) == 4)
    std::printf("%d\n", fa_api::default_splits(wgs, n, causal != 0, cus));
  return 0;
}
