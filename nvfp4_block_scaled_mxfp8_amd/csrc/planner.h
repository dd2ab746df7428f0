// Host-planner entry points shared between the C ABI's source files (not part of the ABI).
#pragma once
#include "gmlp.h"

#include <stddef.h>

namespace gmlp {

// Sets the thread-local error text of gmlp_last_error() and returns st.
gmlp_status set_error(gmlp_status st, const char* fmt, ...);

// Workspace bytes gmlp_group_quantize needs for G groups (the split tables and the NVFP4 amax
// slots), without the slack gmlp_query_sizes adds.
size_t group_quantize_ws_need(int G);

// gmlp_group_quantize on a given workspace (launch counts reset as by the C ABI call).
gmlp_status group_quantize_on(const void* x, int64_t M, int64_t K, const int32_t* m_splits, int32_t G,
                              gmlp_recipe recipe, int32_t want_row, int32_t want_col, const gmlp_grouped_q* out,
                              void* ws, size_t ws_bytes, hipStream_t stream);

}  // namespace gmlp
