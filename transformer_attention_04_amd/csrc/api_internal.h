// Host-side helpers shared by the C-interface sources of libsdpa (not exported
// in include/sdpa.h).
#pragma once

#include "sdpa.h"

namespace sdpa {
// Records a printf-style message for sdpa_last_error() and returns st.
sdpa_status record_error(sdpa_status st, const char* fmt, ...);
}  // namespace sdpa
