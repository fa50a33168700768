// C entry points over the host-side permutation checks of the library
// (int8_weight_moe_amd/csrc/debug_checks.h), so that a CPU test can call them
// on hand-made arrays through ctypes. Each returns the check's message ("" = pass).
#include "../../int8_weight_moe_amd/csrc/debug_checks.h"

namespace {
std::string g_msg;
const char* keep(std::string m) {
  g_msg = std::move(m);
  return g_msg.c_str();
}
}  // namespace

extern "C" {
const char* chk_offsets(const int32_t* off, int E, long S) { return keep(moe_debug::check_offsets(off, E, S)); }
const char* chk_sorted(const int32_t* sorted, long rows, long S) {
  return keep(moe_debug::check_sorted(sorted, rows, S));
}
const char* chk_rows(const int32_t* s2r, long S) { return keep(moe_debug::check_rows(s2r, S)); }
const char* chk_permutation(const int32_t* ids, const int32_t* off, const int32_t* sorted, const int32_t* s2r, int E,
                            long S) {
  return keep(moe_debug::check_permutation(ids, off, sorted, s2r, E, S));
}
}
