// fa_status.hpp — state shared by the library's translation units.
#pragma once

namespace fa {
// hipError_t of the last launch that failed on this thread (reported by fa_last_hip_error).
inline thread_local int last_hip_error = 0;
}  // namespace fa
