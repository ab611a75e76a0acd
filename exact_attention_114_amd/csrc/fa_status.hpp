// fa_status.hpp — state and host rules shared by the library's translation units.
#pragma once

#include <cstdint>

namespace fa {
// hipError_t of the last launch that failed on this thread (reported by fa_last_hip_error).
inline thread_local int last_hip_error = 0;

// Work order of banded and masked grids. Where tile lengths vary widely (causal-like bands: no
// left edge, and masked calls, whose hulls differ), the tiles of up to 4 (b, hkv) groups are
// interleaved, longest first, so that no group's long tiles start near the end of the grid.
// The groups taken together must keep their K and V within one XCD's 4 MiB L2 (more streams
// them from HBM again: 2.7x the reads on the GQA workload, 4 MiB per group), and their count
// must divide the groups so that every block is whole. Measured on MI355X against one group at
// a time: causal d = 64 N = 4096 4.7% faster (4 groups), N = 8192 1.9% (2 groups); a sliding
// window (near-equal lengths) was 2.4% slower interleaved and keeps one group. `unlimited` is
// the value of an edge without a limit.
inline int interleave_groups(int left, int right, int unlimited, bool masked, int64_t groups, int64_t Nk,
                             int64_t d) {
  const bool varied = (left == unlimited && right != unlimited) || masked;
  if (!varied) return 1;
  const int64_t kv_bytes = 2 * Nk * d * 2;  // K and V of one (b, hkv) in 16-bit
  for (int ilv = 4; ilv > 1; ilv /= 2)
    if (groups % ilv == 0 && ilv * kv_bytes <= ((int64_t)4 << 20)) return ilv;
  return 1;
}
}  // namespace fa
