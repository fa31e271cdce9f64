// host.h -- internal helpers shared by the host-side translation units
// (mllm.cpp, sched.cpp).  Not part of the C ABI.
#pragma once

#include "../../include/mllm.h"

namespace mllm {

// Record msg as this thread's last error and return st.
mllm_status host_fail(mllm_status st, const char *msg);
// Clear this thread's last error and return MLLM_OK.
mllm_status host_ok();

}  // namespace mllm
