"""MI355X-native training update of a top-k mixture-of-experts feed-forward layer.

The update runs as one persistent HIP kernel behind the C ABI of
``include/moe_step.h``; ``binding`` exposes the same entry points to Python and
``layer.MoeLayerStep`` keeps the torch tensors of one layer's training state.
"""
from .binding import (  # noqa: F401
    MOE_RUN_APPLY, MOE_RUN_REFRESH_SHADOW, MOE_RUN_TRACE, MOE_RUN_ZERO_GRAD, MoeStepError, load_library,
    make_config, make_io, moe_step_check_config, moe_step_create, moe_step_destroy, moe_step_grid_size,
    moe_step_last_error, moe_step_param_count, moe_step_run, moe_step_status, moe_step_trace_words,
)
