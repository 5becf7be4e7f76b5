// XCD-aware order of a decode launch's work units (host and device code;
// the functions use no HIP API, so a host-only build of this header needs
// only __host__ and __device__ defined empty).
#pragma once

#include <stdint.h>

#include <algorithm>

namespace pa {

// XCD-aware order of a scheduled launch's single items.  The chip deals a
// launch's workgroups out to its 8 XCDs in turn (workgroup b runs on XCD
// b mod 8), and under a full-chip stream its odd XCDs read ~9% slower than
// its even ones (per-wave timestamps of the decode on several workloads and
// boxes), so with one unit (item, head group) per workgroup in item order the
// even XCDs finish first and the odd ones end the launch alone.  Here the
// units, longest first as the schedule lists them, go out in cycles of 84:
// ten rounds of one unit per XCD, then one more round for the even XCDs
// only, so the odd XCDs get 10 units for every 11 of the even ones, spread
// evenly over the launch; each XCD still takes its units longest first.
// The shared-prefix launch orders its group workgroups (first) the same way,
// then its single items after them.
// Position p of the items' region (global workgroup offset + p) runs unit
// xcd_order_unit(p, offset); positions whose unit is past the last are empty.
constexpr int kXcds = 8;
constexpr int kOddRounds = 10;   // rounds per cycle of an odd XCD
constexpr int kEvenRounds = 11;  // rounds per cycle of an even XCD
constexpr int kCycleUnits = kXcds * kOddRounds + (kXcds / 2) * (kEvenRounds - kOddRounds);

__host__ __device__ inline int xcd_order_unit(int p, int offset) {
  const int x = (offset + p) & (kXcds - 1);
  const int first = (x - offset) & (kXcds - 1);  // XCD x's first position
  const int k = (p - first) / kXcds;             // its k-th unit
  if (x & 1) {
    const int c = k / kOddRounds, r = k - c * kOddRounds;
    return c * kCycleUnits + r * kXcds + x;
  }
  const int c = k / kEvenRounds, r = k - c * kEvenRounds;
  return r < kOddRounds ? c * kCycleUnits + r * kXcds + x
                        : c * kCycleUnits + kXcds * kOddRounds + x / 2;
}

// The inverse: the position of unit u.
inline int64_t xcd_order_position(int64_t u, int64_t offset) {
  const int64_t c = u / kCycleUnits, j = u - c * kCycleUnits;
  int x;
  int64_t k;
  if (j < kXcds * kOddRounds) {
    x = int(j % kXcds);
    k = c * ((x & 1) ? kOddRounds : kEvenRounds) + j / kXcds;
  } else {
    x = int(2 * (j - kXcds * kOddRounds));
    k = c * kEvenRounds + kOddRounds;
  }
  const int first = int((int64_t(x) - offset) & (kXcds - 1));
  return first + kXcds * k;
}

// Positions (workgroups) of a launch of `units` units: one past the last
// unit's position over all XCDs.  An XCD's units are at most 12 apart in the
// unit order, so its last unit is among the last kCycleUnits.
inline int64_t xcd_order_positions(int64_t units, int64_t offset) {
  int64_t end = 0;
  for (int64_t u = std::max<int64_t>(0, units - kCycleUnits); u < units; ++u)
    end = std::max(end, xcd_order_position(u, offset) + 1);
  return end;
}

}  // namespace pa
