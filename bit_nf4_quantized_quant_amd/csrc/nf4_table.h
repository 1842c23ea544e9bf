// The NF4 code table as passed to the kernels (plain data, host and device).
#pragma once

#include <cstdint>

namespace qlora {

// The 16 NF4 levels (fp32, ascending) and the 15 decision thresholds passed by
// value to every kernel that needs them.  thr[j] is the smallest fp32 number
// strictly above the midpoint of levels j and j+1, so for an fp32 quotient x
// the nearest level (the lower one on an exact tie) is #{ j : x >= thr[j] }.
struct Nf4Table {
  float level[16];
  float thr[15];
};

// The code tables the library knows (the C ABI's QLORA_TABLE_* values).
constexpr int kTableNf4 = 0, kTableUniform4 = 1, kTableFp4 = 2, kCodeTables = 3;

// Host: table `type` (0 <= type < kCodeTables), built once.  NF4 comes from
// the quantile construction.
const Nf4Table& code_table(int type);

// The thresholds by bucket, for a code search with one comparison: bucket q
// (0..32) is [q/16 - 1, (q+1)/16 - 1); it holds at most one threshold, thr[q]
// (+inf if none), and base[q] thresholds lie below it, so a quotient x in
// bucket q has code base[q] + (x >= thr[q]).  The bucket index may come from
// a rounded 16 x + 16: a quotient put one bucket off lies within 2^-23 of the
// shared edge, and since no threshold lies within 2^-20 of an edge, the code
// comes out the same.  ok = 0 if the table does not have these properties
// (the kernels then compare with all 15 thresholds).
struct Nf4Buckets {
  float thr[33];
  unsigned int base[33];
  int ok;
};

const Nf4Buckets& code_buckets(int type);

// The levels as the decode kernels feed them to bf16 dot products and matrix
// cores: bf16(kappa * L[i]), with the block sums scaled by 1/kappa at the end.
// kappa is the smallest integer in 1..64 for which every kappa * L[i] is a
// bf16 number (to 2^-20 relative) -- 15 for the uniform table, whose levels
// are odd multiples of 1/15, and 3 for FP4, whose levels are E2M1 values over
// 6 -- so those tables enter exactly; NF4's quantiles have no such multiple,
// kappa = 1, and the kernels take bf16(L).
struct DecodeLevels {
  uint16_t bf16[16];
  float kappa;
};

const DecodeLevels& decode_levels(int type);

}  // namespace qlora
