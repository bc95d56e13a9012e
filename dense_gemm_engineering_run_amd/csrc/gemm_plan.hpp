// gemm_plan.hpp -- host-side planning shared by the C ABI's entry points.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace mg {

// What gemm_run_ws would launch for these arguments with a workspace of
// ws_bytes bytes, after every argument check it runs (bar those on the
// workspace pointer): *config (-1 when nothing is launched), *need the bytes
// of workspace that config uses and *count_bytes how many of them, at the
// start, are arrival counters that must be zero when it starts.  Host only:
// no HIP call.  Returns a gemm_status_t.
int plan_ws(int64_t M, int64_t N, int64_t K, char a, char b, char c, int dtype, const void* A,
            const void* B, const void* C, int64_t lda, int64_t ldb, int64_t ldc, size_t ws_bytes,
            int config_id, int* config, uint64_t* need, uint64_t* count_bytes);

}  // namespace mg
