"""H2O (Heavy-Hitter Oracle) KV-cache hot path for MI355X (gfx950).

The compute lives in libh2o.so (HIP kernels behind the C ABI of include/h2o.h);
this package holds the build step and a thin ctypes binding."""
from .binding import (  # noqa: F401
    H2OCache, H2OError, h2o_config, h2o_state, h2o_create, h2o_prefill, h2o_prefill_with_output,
    h2o_prefill_no_alloc, H2O_ERR_TOO_LARGE, H2O_NO_ALLOC_SCRATCH_BYTES,
    h2o_decode_step, h2o_decode_steps, h2o_query, h2o_launch_shape, h2o_steps_launch, h2o_destroy, load_library, status_string,
    H2O_OK, H2O_ERR_INVALID, H2O_ERR_UNSUPPORTED, H2O_ERR_STATE, H2O_ERR_OOM,
    H2O_ERR_HIP, H2O_F32, H2O_BF16, H2O_MAX_K, H2O_CACHE_INPUT, H2O_CACHE_E4M3,
    H2O_POLICY_H2O, H2O_POLICY_STATIC, H2O_POLICY_NAIVE, H2O_STEPS_AUTO, H2O_STEPS_PER_STEP, H2O_STEPS_PERSISTENT,
    H2O_STEPS_RESIDENT,
)
