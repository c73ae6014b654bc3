"""The largest budget k that h2o_create accepts for a launch shape, found by
asking the library (h2o_create with max_prompt = 0 and no split makes no HIP
call).  The create-time check and the kernels' LDS use must agree: the GPU
tests then run the decode at exactly that budget."""
from kv_cache_eviction_02_amd import binding as B


def largest_budget(head_dim, cache_dtype, waves, lo=1, hi=B.H2O_MAX_K):
    def ok(k):
        cfg = B.h2o_config(1, 2, head_dim, (k + 1) // 2, k // 2, 0, B.H2O_BF16, 0.0, 0, 0, waves, 1,
                           cache_dtype, 0, 0)
        fake = 0x10000
        st, ctx = B.h2o_create(cfg, B.h2o_state(fake, fake, fake, fake, fake, fake))
        if st == B.H2O_OK:
            B.h2o_destroy(ctx)
            return True
        assert st == B.H2O_ERR_UNSUPPORTED, st
        return False
    if ok(hi):
        return hi
    while hi - lo > 1:   # ok(lo) and not ok(hi)
        mid = (lo + hi) // 2
        if ok(mid):
            lo = mid
        else:
            hi = mid
    return lo
