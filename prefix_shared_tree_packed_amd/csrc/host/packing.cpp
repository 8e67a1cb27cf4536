// FFD and Karmarkar-Karp allocation (article on AReaL's FFD/KK micro-batch
// packing: the FFD and KK sections, KK's implementation details and safety
// net).
//
// FFD: items in stable descending order; the first min_groups items open
// groups, every later item goes to the lightest group it fits (lowest index
// on ties) or opens a new one; a group count that is not a multiple of the
// divisor raises min_groups to the next multiple (never beyond the item
// count) and packs again.
//
// KK: every item is a partial partition ("state") of k subsets holding it
// alone.  A max-heap on spread (largest subset sum minus smallest; equal
// spreads pop in push order) yields two states, whose subsets are combined
// lightest-with-heaviest, until one state remains.
//
// A state stores only its non-empty subsets, each with its slot (its place
// in the ascending order of the k sums, empty subsets included), so memory
// is O(items) and a combination costs O(subsets it touches), not O(k).
// Subsets are linked lists of items, so joining two is O(1).  Slots
// reproduce a stable ascending sort of the k combined sums: zero sums keep
// their combined order, positive sums follow by (sum, combined position).
#include "packing.h"

#include <algorithm>
#include <functional>
#include <numeric>
#include <queue>
#include <utility>

namespace pst {
namespace {

PackStatus check_items(const int64_t* values, int32_t n, int64_t capacity, int32_t min_groups,
                       int32_t divisor) {
  if (!values || n < 1 || capacity <= 0 || min_groups < 1 || divisor < 1) return kPackInvalid;
  for (int32_t i = 0; i < n; ++i) {
    if (values[i] < 0) return kPackInvalid;
    if (values[i] > capacity) return kPackCapacity;
  }
  return kPackOk;
}

int32_t ffd_once(const int64_t* values, const std::vector<int32_t>& order, int64_t capacity,
                 int32_t min_groups, std::vector<int32_t>* group_of) {
  // the lightest group is the only candidate: if it has no room, none has
  using Group = std::pair<int64_t, int32_t>;  // (sum, index): lowest index on ties
  std::priority_queue<Group, std::vector<Group>, std::greater<Group>> light;
  int32_t n_groups = 0;
  for (int32_t i : order) {
    const int64_t v = values[i];
    if (n_groups >= min_groups && light.top().first + v <= capacity) {
      Group g = light.top();
      light.pop();
      g.first += v;
      (*group_of)[i] = g.second;
      light.push(g);
    } else {
      (*group_of)[i] = n_groups;
      light.push({v, n_groups++});
    }
  }
  return n_groups;
}

struct Subset {
  int32_t slot;  // place among the state's k subsets in ascending order of sum
  int64_t sum;
  int32_t head, tail;  // linked list of items through `next`
};

struct State {
  int64_t spread;
  int64_t seq;  // push order
  int32_t id;   // index into the state table
};

struct StateLess {
  bool operator()(const State& a, const State& b) const {
    if (a.spread != b.spread) return a.spread < b.spread;  // larger spread first
    return a.seq > b.seq;                                  // then earlier push
  }
};

}  // namespace

PackStatus pack_ffd(const int64_t* values, int32_t n, int64_t capacity, int32_t min_groups,
                    int32_t divisor, PackResult* out) {
  const PackStatus st = check_items(values, n, capacity, min_groups, divisor);
  if (st != kPackOk) return st;
  std::vector<int32_t> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return values[a] > values[b]; });
  out->group_of.assign(n, 0);
  out->fell_back = false;
  int32_t mg = std::min(min_groups, n);
  for (;;) {
    const int32_t g = ffd_once(values, order, capacity, mg, &out->group_of);
    out->n_groups = g;
    if (g % divisor == 0) break;
    const int64_t next = (static_cast<int64_t>(g) + divisor - 1) / divisor * divisor;
    if (next > n) break;
    mg = static_cast<int32_t>(next);
  }
  return kPackOk;
}

void kk_partition(const int64_t* values, int32_t n, int32_t k, std::vector<int32_t>* group_of) {
  std::vector<int32_t> next(n, -1);
  std::vector<std::vector<Subset>> states(n);  // non-empty subsets, ascending slot
  std::priority_queue<State, std::vector<State>, StateLess> heap;
  int64_t seq = 0;
  for (int32_t i = 0; i < n; ++i) {
    states[i].push_back({k - 1, values[i], i, i});
    heap.push({k > 1 ? values[i] : 0, seq++, i});
  }
  struct Pos {
    int32_t pos;  // place in the combined order
    int64_t sum;
    int32_t head, tail;
  };
  std::vector<Pos> comb;
  std::vector<int32_t> positive;
  while (heap.size() > 1) {
    const State a = heap.top();
    heap.pop();
    const State b = heap.top();
    heap.pop();
    const std::vector<Subset>& sa = states[a.id];
    const std::vector<Subset>& sb = states[b.id];
    // combined position p takes a's slot p and b's slot k-1-p; walk a's
    // slots upward and b's downward so positions come out ascending
    comb.clear();
    size_t ia = 0;
    size_t ib = sb.size();
    while (ia < sa.size() || ib > 0) {
      const int32_t pa = ia < sa.size() ? sa[ia].slot : k;
      const int32_t pb = ib > 0 ? k - 1 - sb[ib - 1].slot : k;
      Pos c{std::min(pa, pb), 0, -1, -1};
      if (pa == c.pos) {
        const Subset& x = sa[ia++];
        c.sum = x.sum;
        c.head = x.head;
        c.tail = x.tail;
      }
      if (pb == c.pos) {
        const Subset& y = sb[--ib];
        c.sum += y.sum;
        if (c.head < 0) {
          c.head = y.head;
        } else {
          next[c.tail] = y.head;
        }
        c.tail = y.tail;
      }
      comb.push_back(c);
    }
    // slots of a stable ascending sort of all k sums (absent positions are 0)
    positive.clear();
    for (int32_t j = 0; j < static_cast<int32_t>(comb.size()); ++j)
      if (comb[j].sum > 0) positive.push_back(j);
    std::sort(positive.begin(), positive.end(), [&](int32_t p, int32_t q) {
      return comb[p].sum != comb[q].sum ? comb[p].sum < comb[q].sum : p < q;
    });
    const int32_t n_pos = static_cast<int32_t>(positive.size());
    std::vector<Subset> out(comb.size());
    int32_t pos_before = 0;  // positive entries at smaller positions
    size_t w = 0;
    for (const Pos& c : comb) {  // zero sums: ascending position
      if (c.sum > 0) {
        ++pos_before;
        continue;
      }
      out[w++] = {c.pos - pos_before, 0, c.head, c.tail};
    }
    for (int32_t r = 0; r < n_pos; ++r) {
      const Pos& c = comb[positive[r]];
      out[w++] = {k - n_pos + r, c.sum, c.head, c.tail};
    }
    // zero sums took slots below k - n_pos in ascending order, positive sums
    // the slots above: `out` is already in slot order
    const int64_t hi = n_pos > 0 ? out.back().sum : 0;
    const int64_t lo = n_pos == k ? out.front().sum : 0;
    states[a.id].swap(out);
    std::vector<Subset>().swap(states[b.id]);
    heap.push({hi - lo, seq++, a.id});
  }
  group_of->assign(n, 0);
  for (const Subset& sub : states[heap.top().id])
    for (int32_t i = sub.head; i >= 0; i = (i == sub.tail) ? -1 : next[i]) (*group_of)[i] = sub.slot;
}

PackStatus pack_kk(const int64_t* values, int32_t n, int64_t capacity, int32_t min_groups,
                   int32_t divisor, PackResult* out) {
  const PackStatus st = check_items(values, n, capacity, min_groups, divisor);
  if (st != kPackOk) return st;
  int64_t total = 0;
  for (int32_t i = 0; i < n; ++i)
    if (__builtin_add_overflow(total, values[i], &total)) return kPackInvalid;
  int64_t k = std::max<int64_t>(min_groups, (total + capacity - 1) / capacity);
  k = std::max<int64_t>(k, 1);
  k = (k + divisor - 1) / divisor * divisor;
  k = std::min<int64_t>(k, n);
  kk_partition(values, n, static_cast<int32_t>(k), &out->group_of);
  std::vector<int64_t> sums(k, 0);
  for (int32_t i = 0; i < n; ++i) sums[out->group_of[i]] += values[i];
  if (*std::max_element(sums.begin(), sums.end()) > capacity) {
    const PackStatus f = pack_ffd(values, n, capacity, min_groups, divisor, out);
    out->fell_back = true;
    return f;
  }
  out->n_groups = static_cast<int32_t>(k);
  out->fell_back = false;
  return kPackOk;
}

}  // namespace pst
