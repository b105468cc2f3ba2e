"""Paged-KV attention step for AMD Instinct MI355X (gfx950).

The work happens in libpa.so (HIP kernels behind the C ABI of include/pa.h)
and libpa_sched.so (the host scheduler and block allocator of
include/pa_sched.h); this package only marshals arguments.  Importing it does not load the
library; the first call does, and raises if it has not been built.
"""
from ._lib import (  # noqa: F401
    EXPORTS, LIB_PATH, PA_BF16, PA_F32, TUNING, PAError, StepPlan, abi_version, alloc_workspace,
    NOALLOC_SCRATCH_BYTES, attention, attention_noalloc, attention_plan, attention_run,
    attention_workspace_bound, attention_workspace_size,
    build_step_metadata, compute_slot_mapping, copy_blocks, get_tuning, last_error, lib,
    rope_write_kv, set_profiling_events, set_tuning, status_str, swap_blocks, tuning,
    validate_metadata, write_kv,
)
from ._sched import SCHED_EXPORTS, SCHED_LIB_PATH, Scheduler, sched_lib  # noqa: F401,E402
