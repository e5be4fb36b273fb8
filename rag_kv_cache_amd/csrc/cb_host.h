// Host-side internals shared by the C-ABI sources of the library (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>

#include "../../include/cacheblend.h"

// Record the calling thread's error message (read by cb_last_error) and return st.
cb_status cbi_fail(cb_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// The context's compute stream, device and model description (ctx must be non-NULL).
hipStream_t cbi_compute_stream(const cb_ctx* ctx);
int cbi_device(const cb_ctx* ctx);
const cb_model_desc* cbi_desc(const cb_ctx* ctx);
