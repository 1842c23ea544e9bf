// Reads records (uint64 n, then n fp32 values) from the file argv[1] and
// prints, per record, the fp32 bits of the library's exact mean: the values'
// mantissas summed per exponent bucket (the double-quant kernel's first
// pass, written out here for the host) and mean_from_buckets.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "exact_mean.h"

int main(int argc, char** argv) {
  if (argc != 2) return 2;
  FILE* f = std::fopen(argv[1], "rb");
  if (!f) return 2;
  uint64_t n = 0;
  while (std::fread(&n, sizeof n, 1, f) == 1) {
    std::vector<float> v(n);
    if (n && std::fread(v.data(), sizeof(float), n, f) != n) return 3;
    unsigned long long bucket[qlora::kMeanBuckets] = {};
    for (uint64_t i = 0; i < n; ++i) {
      uint32_t bits;
      std::memcpy(&bits, &v[i], 4);
      const uint32_t e = (bits >> 23) & 0xFFu;
      const uint32_t b = e ? e : 1u;
      const unsigned long long m = (bits & 0x7FFFFFu) | (e ? 0x800000u : 0u);
      bucket[b] += m;
    }
    std::printf("%08x\n", qlora::mean_from_buckets(bucket, n));
  }
  std::fclose(f);
  return 0;
}
