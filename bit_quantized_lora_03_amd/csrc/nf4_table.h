// Host-side NF4 table (levels + decision thresholds); see nf4_table.cpp.
#pragma once

namespace qlora {

struct Nf4Table {
  float level[16];      // ascending, level[0] = -1, level[7] = 0, level[15] = 1
  float threshold[15];  // code(u) = #{i : u > threshold[i]}
};

// Built once (thread-safe) on first use.
const Nf4Table& nf4_table();

}  // namespace qlora
