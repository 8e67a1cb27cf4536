// Allocation of weighted items (sequence lengths, tree costs) to groups
// (micro-batches, data-parallel ranks): first-fit decreasing into the
// lightest group that fits, and k-way Karmarkar-Karp largest differencing
// with a fallback to FFD when a group exceeds the capacity.  Host only.
#pragma once

#include <cstdint>
#include <vector>

namespace pst {

enum PackStatus { kPackOk = 0, kPackInvalid = 1, kPackCapacity = 2 };

struct PackResult {
  std::vector<int32_t> group_of;  // group of every item
  int32_t n_groups = 0;
  bool fell_back = false;         // KK exceeded the capacity, FFD used instead
};

// values: n >= 1 non-negative weights; capacity > 0; min_groups >= 1 (at
// most n groups are ever formed); divisor >= 1.
PackStatus pack_ffd(const int64_t* values, int32_t n, int64_t capacity, int32_t min_groups,
                    int32_t divisor, PackResult* out);
PackStatus pack_kk(const int64_t* values, int32_t n, int64_t capacity, int32_t min_groups,
                   int32_t divisor, PackResult* out);
// Karmarkar-Karp into exactly k groups (k >= 1), numbered in ascending
// order of their sums.
void kk_partition(const int64_t* values, int32_t n, int32_t k, std::vector<int32_t>* group_of);

}  // namespace pst
