"""MI355X-native KV-shared early-exit decoder (River-LLM) behind a C ABI.

The kernels and the scheduler live in libriver.so (HIP for gfx950, built by
``early_exit_kv_amd/build.py``); this package only marshals arguments.
"""
from .river import (  # noqa: F401
    EXPORTS, LINEAR_NAMES, RIVER_EXIT_COPY, RIVER_EXIT_INT4, RIVER_OPT_FORCE_E, RIVER_OPT_GRAPH,
    River, RiverConfig, RiverError, exit_bank_offsets, load_library, make_config, query_sizes,
    unpack_int4,
)
