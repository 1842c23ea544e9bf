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

// Each level split into two bf16 numbers, hi = bf16(L) and lo = bf16(L - hi),
// packed as hi | lo << 16.  hi + lo carries L to about 2^-17 relative, which
// lets the fused matrix kernels feed bf16 matrix cores with the levels and
// apply the per-block fp32 scale after the product.
struct Nf4HiLo {
  unsigned int word[16];
};

const Nf4HiLo& nf4_hilo();

}  // namespace qlora
