// Counters of the host stand-ins in stubs.cpp.
#pragma once

namespace stub {
extern int launches;  // launcher calls since the program started
extern int overlaps;  // workspace regions found overwritten by another region
}  // namespace stub
