// Host-side error state shared by the library's translation units: every
// entry point returns an asr_status code and leaves a message for
// asr_last_error() in a thread-local string.
#pragma once

#include <hip/hip_runtime.h>
#include <string>

namespace asr_host {

int fail(int status, const std::string& msg);  // records msg, returns status
int ok();                                      // clears the message, returns ASR_OK
int hip_fail(hipError_t e, const char* what);  // ASR_EHIP with the HIP error text

}  // namespace asr_host
