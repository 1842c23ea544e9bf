// The NF4 code table as passed to the kernels (plain data, host and device).
#pragma once

namespace qlora {

// The 16 NF4 levels (fp32, ascending) and the 15 decision thresholds passed by
// value to every kernel that needs them.  thr[j] is the smallest fp32 number
// strictly above the midpoint of levels j and j+1, so for an fp32 quotient x
// the nearest level (the lower one on an exact tie) is #{ j : x >= thr[j] }.
struct Nf4Table {
  float level[16];
  float thr[15];
};

// Host: the library's table, built once from the quantile construction.
const Nf4Table& nf4_table();

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

const Nf4Buckets& nf4_buckets();

// Each level split into two bf16 numbers, hi = bf16(L) and lo = bf16(L - hi),
// packed as hi | lo << 16.  hi + lo carries L to about 2^-17 relative, which
// lets the fused matrix kernels feed bf16 matrix cores with the levels and
// apply the per-block fp32 scale after the product.
struct Nf4HiLo {
  unsigned int word[16];
};

const Nf4HiLo& nf4_hilo();

}  // namespace qlora
