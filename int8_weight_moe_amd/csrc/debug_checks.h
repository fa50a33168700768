// Host-side consistency checks of a permutation, run by the C ABI when the
// environment variable MOE_DEBUG is set (debug runs only: the arrays are first
// copied to the host). Plain C++ with no HIP dependency, so that the checks
// themselves can be exercised on the CPU.
//
// The permutation groups the T*K slots (slot s = t*K + k is token t's k-th
// expert choice) by expert:
//   offsets [E+1]  expert e owns sorted rows [offsets[e], offsets[e+1]);
//   sorted  [S]    the slot held by each sorted row (rows past offsets[E]: -1);
//   s2r     [S]    the sorted row of each slot (-1 for a slot not placed).
// Each check returns an empty string when it passes, else a message that
// names the first offending entry.
#pragma once

#include <stdint.h>
#include <stdio.h>

#include <string>
#include <vector>

namespace moe_debug {

inline std::string msg(const char* fmt, long a, long b = 0, long c = 0, long d = 0) {
  char buf[256];
  snprintf(buf, sizeof(buf), fmt, a, b, c, d);
  return buf;
}

// offsets[0] = 0, non-decreasing, offsets[E] <= S: every segment lies inside
// the S sorted rows.
inline std::string check_offsets(const int32_t* off, int E, long S) {
  if (off[0] != 0) return msg("expert_offsets[0] = %ld, expected 0", off[0]);
  for (int e = 0; e < E; ++e)
    if (off[e + 1] < off[e])
      return msg("expert_offsets decrease at expert %ld (%ld -> %ld)", e, off[e], off[e + 1]);
  if (off[E] > S) return msg("expert_offsets[E] = %ld exceeds the %ld slots", off[E], S);
  return "";
}

// The sorted rows below `rows` hold distinct slots in [0, S).
inline std::string check_sorted(const int32_t* sorted, long rows, long S) {
  std::vector<unsigned char> seen((size_t)S, 0);
  for (long r = 0; r < rows; ++r) {
    const long s = sorted[r];
    if (s < 0 || s >= S) return msg("sorted_slots[%ld] = %ld is outside [0, %ld)", r, s, S);
    if (seen[(size_t)s]) return msg("slot %ld is held by two sorted rows (the second: %ld)", s, r);
    seen[(size_t)s] = 1;
  }
  return "";
}

// Every slot_to_row entry is -1 or a row in [0, S).
inline std::string check_rows(const int32_t* s2r, long S) {
  for (long s = 0; s < S; ++s)
    if (s2r[s] < -1 || s2r[s] >= S) return msg("slot_to_row[%ld] = %ld is outside [-1, %ld)", s, s2r[s], S);
  return "";
}

// A permutation of the expert ids `ids` [S] as the library produces it: the
// checks above, every slot placed, each sorted row's slot routed to its
// segment's expert in ascending slot order, and slot_to_row the inverse of
// sorted_slots.
inline std::string check_permutation(const int32_t* ids, const int32_t* off, const int32_t* sorted,
                                     const int32_t* s2r, int E, long S) {
  long outside = 0, first = -1;
  for (long s = 0; s < S; ++s)
    if (ids[s] < 0 || ids[s] >= E) {
      if (first < 0) first = s;
      ++outside;
    }
  if (outside)
    return msg("%ld slots have an expert id outside [0, %ld) (first: slot %ld, id %ld)", outside, E, first,
               ids[first]);
  std::string m = check_offsets(off, E, S);
  if (m.empty() && off[E] != S) m = msg("expert_offsets[E] = %ld, expected all %ld slots", off[E], S);
  if (m.empty()) m = check_sorted(sorted, S, S);
  if (m.empty()) m = check_rows(s2r, S);
  if (!m.empty()) return m;
  for (int e = 0; e < E; ++e)
    for (long r = off[e]; r < off[e + 1]; ++r) {
      if (ids[sorted[r]] != e)
        return msg("sorted row %ld of expert %ld holds slot %ld, routed to expert %ld", r, e, sorted[r],
                   ids[sorted[r]]);
      if (r > off[e] && sorted[r] < sorted[r - 1])
        return msg("sorted rows %ld and %ld of expert %ld hold slots %ld out of ascending order", r - 1, r, e,
                   sorted[r]);
    }
  for (long r = 0; r < S; ++r)
    if (s2r[sorted[r]] != r) return msg("slot_to_row[%ld] = %ld, but the slot is held by sorted row %ld",
                                        sorted[r], s2r[sorted[r]], r);
  return "";
}

}  // namespace moe_debug
