// moe_sortnet.h -- the comparator network that sorts the eight keys a lane
// holds in the top-K selection: Batcher's odd-even merge sort for eight
// inputs (19 comparators, depth 6).  After comparator (i, j), element i holds
// the larger key and element j the smaller, so the network sorts in
// descending order.  Plain C++ (no HIP), so host tests read the same table.
#pragma once

namespace moe_impl {

constexpr int kSort8Comparators = 19;
constexpr unsigned char kSort8Net[kSort8Comparators][2] = {
    {0, 2}, {1, 3}, {4, 6}, {5, 7},   // sort pairs of pairs
    {0, 4}, {1, 5}, {2, 6}, {3, 7},   // merge the halves
    {0, 1}, {2, 3}, {4, 5}, {6, 7},
    {2, 4}, {3, 5},
    {1, 4}, {3, 6},
    {1, 2}, {3, 4}, {5, 6},
};

}  // namespace moe_impl
