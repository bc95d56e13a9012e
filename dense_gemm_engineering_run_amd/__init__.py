"""MI355X (gfx950) dense GEMM engine: C = A * B^T on MFMA, behind a C ABI.

The compute runs in hand-written HIP kernels in libmi355_gemm.so; this package
is its Python binding (argument marshalling only) plus its build script.
"""
from ._binding import *  # noqa: F401,F403
from ._binding import (Epilogue, GemmError, gemm, gemm_config_describe, gemm_last_config,  # noqa: F401
                       gemm_load_tuning, gemm_num_configs, gemm_run, gemm_run_batched, gemm_run_config,
                       gemm_run_ex, gemm_run_ws, gemm_select_config, gemm_status_str, gemm_tuning_size,
                       gemm_workspace_size)
