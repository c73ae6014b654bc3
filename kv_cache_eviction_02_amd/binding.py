"""ctypes binding of libh2o (include/h2o.h), with the same call names.

Argument marshalling only: every step of the H2O path runs in the library's HIP
kernels.  torch supplies device buffers and the current HIP stream.  The
library must be built (``python -m kv_cache_eviction_02_amd.build``); loading
fails loudly when it is missing.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libh2o.so")

H2O_OK, H2O_ERR_INVALID, H2O_ERR_UNSUPPORTED, H2O_ERR_STATE, H2O_ERR_OOM, H2O_ERR_HIP, H2O_ERR_TOO_LARGE = range(7)
H2O_F32, H2O_BF16 = 0, 1
H2O_CACHE_INPUT, H2O_CACHE_E4M3 = 0, 1
H2O_POLICY_H2O, H2O_POLICY_STATIC, H2O_POLICY_NAIVE = 0, 1, 2
POLICIES = {"h2o": H2O_POLICY_H2O, "static": H2O_POLICY_STATIC, "naive": H2O_POLICY_NAIVE}
H2O_STEPS_AUTO, H2O_STEPS_PER_STEP, H2O_STEPS_PERSISTENT, H2O_STEPS_RESIDENT = 0, 1, 2, 3
STEPS_MODES = {"auto": H2O_STEPS_AUTO, "per_step": H2O_STEPS_PER_STEP, "persistent": H2O_STEPS_PERSISTENT,
               "resident": H2O_STEPS_RESIDENT}
H2O_MAX_K = 8192
H2O_MAX_PROMPT = 1 << 28
H2O_NO_ALLOC_SCRATCH_BYTES = 32 << 20

STATUS_NAMES = {
    H2O_OK: "H2O_OK",
    H2O_ERR_INVALID: "H2O_ERR_INVALID",
    H2O_ERR_UNSUPPORTED: "H2O_ERR_UNSUPPORTED",
    H2O_ERR_STATE: "H2O_ERR_STATE",
    H2O_ERR_OOM: "H2O_ERR_OOM",
    H2O_ERR_HIP: "H2O_ERR_HIP",
    H2O_ERR_TOO_LARGE: "H2O_ERR_TOO_LARGE",
}


class h2o_config(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("recent", ctypes.c_int32),
        ("heavy", ctypes.c_int32),
        ("max_prompt", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("start_pos", ctypes.c_int32),
        ("start_live", ctypes.c_int32),
        ("decode_waves", ctypes.c_int32),
        ("decode_split", ctypes.c_int32),
        ("cache_dtype", ctypes.c_int32),
        ("policy", ctypes.c_int32),
        ("steps_mode", ctypes.c_int32),
    ]


class h2o_state(ctypes.Structure):
    _fields_ = [
        ("k_slots", ctypes.c_void_p),
        ("v_slots", ctypes.c_void_p),
        ("score", ctypes.c_void_p),
        ("pos", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
    ]


class H2OError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


_lib = None


def load_library(path=LIB_PATH):
    """Load libh2o.so and declare the signatures; raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m kv_cache_eviction_02_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.h2o_create.argtypes = [ctypes.POINTER(h2o_config), ctypes.POINTER(h2o_state),
                               ctypes.POINTER(vp)]
    lib.h2o_create.restype = ctypes.c_int
    lib.h2o_prefill.argtypes = [vp, vp, vp, vp, i32, vp]
    lib.h2o_prefill.restype = ctypes.c_int
    lib.h2o_prefill_with_output.argtypes = [vp, vp, vp, vp, i32, vp, vp]
    lib.h2o_prefill_with_output.restype = ctypes.c_int
    lib.h2o_prefill_no_alloc.argtypes = [vp, vp, vp, vp, i32, vp, vp]
    lib.h2o_prefill_no_alloc.restype = ctypes.c_int
    lib.h2o_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    lib.h2o_decode_step.restype = ctypes.c_int
    lib.h2o_decode_steps.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp]
    lib.h2o_decode_steps.restype = ctypes.c_int
    lib.h2o_query.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.h2o_query.restype = ctypes.c_int
    lib.h2o_launch_shape.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.h2o_launch_shape.restype = ctypes.c_int
    lib.h2o_steps_launch.argtypes = [vp, i32, ctypes.POINTER(i32)]
    lib.h2o_steps_launch.restype = ctypes.c_int
    lib.h2o_destroy.argtypes = [vp]
    lib.h2o_destroy.restype = ctypes.c_int
    lib.h2o_status_string.argtypes = [ctypes.c_int]
    lib.h2o_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status):
    return load_library().h2o_status_string(status).decode()


def _check(status, where):
    if status != H2O_OK:
        raise H2OError(status, where)


# ---- raw calls, same names as the C ABI (pointers are ints) --------------------

def h2o_create(cfg: h2o_config, state: h2o_state):
    """Returns (status, ctx pointer or None)."""
    out = ctypes.c_void_p()
    st = load_library().h2o_create(ctypes.byref(cfg), ctypes.byref(state), ctypes.byref(out))
    return st, (out.value if st == H2O_OK else None)


def h2o_prefill(ctx, q, k, v, prompt_len, stream):
    return load_library().h2o_prefill(ctx, q, k, v, prompt_len, stream)


def h2o_prefill_with_output(ctx, q, k, v, prompt_len, out, stream):
    return load_library().h2o_prefill_with_output(ctx, q, k, v, prompt_len, out, stream)


def h2o_prefill_no_alloc(ctx, q, k, v, prompt_len, out, stream):
    return load_library().h2o_prefill_no_alloc(ctx, q, k, v, prompt_len, out, stream)


def h2o_decode_step(ctx, q, k_new, v_new, out, evicted_pos, stream):
    return load_library().h2o_decode_step(ctx, q, k_new, v_new, out, evicted_pos, stream)


def h2o_decode_steps(ctx, n_steps, q, k_new, v_new, out, evicted_pos, stream):
    return load_library().h2o_decode_steps(ctx, n_steps, q, k_new, v_new, out, evicted_pos, stream)


def h2o_query(ctx):
    t, n = ctypes.c_int32(), ctypes.c_int32()
    st = load_library().h2o_query(ctx, ctypes.byref(t), ctypes.byref(n))
    return st, t.value, n.value


def h2o_launch_shape(ctx):
    w, s = ctypes.c_int32(), ctypes.c_int32()
    st = load_library().h2o_launch_shape(ctx, ctypes.byref(w), ctypes.byref(s))
    return st, w.value, s.value


def h2o_steps_launch(ctx, n_steps):
    m = ctypes.c_int32()
    st = load_library().h2o_steps_launch(ctx, n_steps, ctypes.byref(m))
    return st, m.value


def h2o_destroy(ctx):
    return load_library().h2o_destroy(ctx)


# ---- torch-buffer convenience wrapper -------------------------------------------

class H2OCache:
    """A per-layer H2O KV cache on the current GPU.

    Owns the slot-layout state as torch tensors (k_slots, v_slots: [B, H, k, d]
    in the KV dtype; score: [B, H, k] float32; pos: [B, H, k] int32) and a
    library ctx bound to them.  ``prefill`` and ``step`` enqueue on torch's
    current stream and return without synchronising."""

    def __init__(self, batch, heads, head_dim, recent, heavy, max_prompt, dtype,
                 scale=0.0, device="cuda", decode_waves=0, start_pos=0, start_live=0,
                 state=None, decode_split=0, cache="input", policy="h2o", steps_mode="auto"):
        import torch
        self.torch = torch
        load_library()
        if dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("dtype must be torch.float32 or torch.bfloat16")
        if cache not in ("input", "e4m3"):
            raise ValueError("cache must be 'input' or 'e4m3'")
        if steps_mode not in STEPS_MODES:
            raise ValueError(f"steps_mode must be one of {sorted(STEPS_MODES)}")
        if policy not in POLICIES:
            raise ValueError(f"policy must be one of {sorted(POLICIES)}")
        self.policy = policy
        self.batch, self.heads, self.head_dim = batch, heads, head_dim
        self.recent, self.heavy, self.k = recent, heavy, recent + heavy
        self.dtype = dtype
        self.cache = cache
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        shape = (batch, heads, self.k, head_dim)
        slot_dtype = torch.uint8 if cache == "e4m3" else dtype
        if state is None:
            self.k_slots = torch.zeros(shape, dtype=slot_dtype, device=self.device)
            self.v_slots = torch.zeros(shape, dtype=slot_dtype, device=self.device)
            self.score = torch.zeros(shape[:3], dtype=torch.float32, device=self.device)
            self.pos = torch.full(shape[:3], -1, dtype=torch.int32, device=self.device)
            self.k_scale = self.v_scale = None
            if cache == "e4m3":
                self.k_scale = torch.zeros(shape[:3], dtype=torch.float32, device=self.device)
                self.v_scale = torch.zeros(shape[:3], dtype=torch.float32, device=self.device)
        else:
            self.k_slots, self.v_slots, self.score, self.pos = state[:4]
            self.k_scale, self.v_scale = (state[4], state[5]) if len(state) > 4 else (None, None)
        checks = [(self.k_slots, slot_dtype, shape), (self.v_slots, slot_dtype, shape),
                  (self.score, torch.float32, shape[:3]), (self.pos, torch.int32, shape[:3])]
        if cache == "e4m3":
            checks += [(self.k_scale, torch.float32, shape[:3]), (self.v_scale, torch.float32, shape[:3])]
        for t_, dt, shp in checks:
            if t_ is None or t_.dtype != dt or tuple(t_.shape) != shp or not t_.is_contiguous() \
                    or t_.device != self.device:
                raise ValueError("state tensors must be contiguous, on the device, with the "
                                 "layout's shapes and dtypes")
        self.cfg = h2o_config(batch, heads, head_dim, recent, heavy, max_prompt,
                              H2O_F32 if dtype == torch.float32 else H2O_BF16, scale,
                              start_pos, start_live, decode_waves, decode_split,
                              H2O_CACHE_E4M3 if cache == "e4m3" else H2O_CACHE_INPUT,
                              POLICIES[policy],
                              STEPS_MODES[steps_mode])
        self.state = h2o_state(self.k_slots.data_ptr(), self.v_slots.data_ptr(),
                               self.score.data_ptr(), self.pos.data_ptr(),
                               self.k_scale.data_ptr() if self.k_scale is not None else None,
                               self.v_scale.data_ptr() if self.v_scale is not None else None)
        st, ctx = h2o_create(self.cfg, self.state)
        _check(st, "h2o_create")
        self.ctx = ctx
        self.out = torch.empty((batch, heads, head_dim), dtype=torch.float32, device=self.device)
        self.evicted = torch.empty((batch, heads), dtype=torch.int32, device=self.device)

    def _stream(self):
        return self.torch.cuda.current_stream(self.device).cuda_stream

    def _input(self, x, shape, name):
        if x.dtype != self.dtype or tuple(x.shape) != shape or not x.is_contiguous() \
                or x.device != self.device:
            raise ValueError(f"{name}: expected contiguous {self.dtype} {shape} on {self.device}, "
                             f"got {x.dtype} {tuple(x.shape)} on {x.device}")
        return x.data_ptr()

    def _output(self, x, shape, dtype, name):
        if x.dtype != dtype or tuple(x.shape) != shape or not x.is_contiguous() or x.device != self.device:
            raise ValueError(f"{name}: expected contiguous {dtype} {shape} on {self.device}, "
                             f"got {x.dtype} {tuple(x.shape)} on {x.device}")
        return x.data_ptr()

    def prefill(self, q, k, v, output=False, out=None, no_alloc=False):
        """Seed the cache from a prompt [B, H, P, d].  With output=True (or an
        out tensor) also returns the prompt's attention output [B, H, P, d]
        float32.  no_alloc=True calls h2o_prefill_no_alloc (its scratch is the
        library's fixed buffer, not the ctx's)."""
        P = q.shape[2]
        shape = (self.batch, self.heads, P, self.head_dim)
        ptrs = [self._input(x, shape, n) for x, n in ((q, "q"), (k, "k"), (v, "v"))]
        if no_alloc:
            if output and out is None:
                out = self.torch.empty(shape, dtype=self.torch.float32, device=self.device)
            optr = None if out is None else self._output(out, shape, self.torch.float32, "out")
            _check(h2o_prefill_no_alloc(self.ctx, *ptrs, P, optr, self._stream()), "h2o_prefill_no_alloc")
            return out
        if not output and out is None:
            _check(h2o_prefill(self.ctx, *ptrs, P, self._stream()), "h2o_prefill")
            return None
        if out is None:
            out = self.torch.empty(shape, dtype=self.torch.float32, device=self.device)
        optr = self._output(out, shape, self.torch.float32, "out")
        _check(h2o_prefill_with_output(self.ctx, *ptrs, P, optr, self._stream()), "h2o_prefill_with_output")
        return out

    def step(self, q, k_new, v_new, out=None, evicted=None):
        """One decode step; returns (out [B, H, d] float32, evicted [B, H] int32).
        Without out / evicted arguments these are the cache's own buffers,
        overwritten by the next step: clone them to keep a step's results."""
        shape = (self.batch, self.heads, self.head_dim)
        ptrs = [self._input(x, shape, n) for x, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"))]
        out = self.out if out is None else out
        evicted = self.evicted if evicted is None else evicted
        optr = self._output(out, shape, self.torch.float32, "out")
        eptr = self._output(evicted, shape[:2], self.torch.int32, "evicted")
        _check(h2o_decode_step(self.ctx, *ptrs, optr, eptr, self._stream()), "h2o_decode_step")
        return out, evicted

    def steps(self, q, k_new, v_new, out=None, evicted=None):
        """n consecutive decode steps over known tokens: inputs [n, B, H, d];
        returns (out [n, B, H, d] float32, evicted [n, B, H] int32)."""
        n = q.shape[0]
        shape = (n, self.batch, self.heads, self.head_dim)
        ptrs = [self._input(x, shape, nm) for x, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"))]
        torch = self.torch
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=self.device)
        if evicted is None:
            evicted = torch.empty(shape[:3], dtype=torch.int32, device=self.device)
        optr = self._output(out, shape, torch.float32, "out")
        eptr = self._output(evicted, shape[:3], torch.int32, "evicted")
        _check(h2o_decode_steps(self.ctx, n, *ptrs, optr, eptr, self._stream()), "h2o_decode_steps")
        return out, evicted

    def position(self):
        st, t, n = h2o_query(self.ctx)
        _check(st, "h2o_query")
        return t, n

    def launch_shape(self):
        """(wavefronts per decode workgroup, workgroups per unit) chosen at creation."""
        st, w, sp = h2o_launch_shape(self.ctx)
        _check(st, "h2o_launch_shape")
        return w, sp

    def steps_launch(self, n_steps):
        """How steps() would launch n_steps steps now: "resident", "persistent" or "per_step"."""
        st, m = h2o_steps_launch(self.ctx, n_steps)
        _check(st, "h2o_steps_launch")
        return {v: k for k, v in STEPS_MODES.items()}[m]

    def close(self):
        if getattr(self, "ctx", None):
            # h2o_destroy frees the ctx's scratch: no enqueued call may still use it
            self.torch.cuda.synchronize(self.device)
            _check(h2o_destroy(self.ctx), "h2o_destroy")
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
