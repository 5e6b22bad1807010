"""ctypes binding of libspec.so: the C ABI of include/spec.h, same names.

Argument marshalling only; every step of the verify path runs in the HIP
library.  Importing this module fails loudly if the library is not built.
"""

import ctypes
import os
from ctypes import POINTER, byref, c_double, c_float, c_int32, c_int64, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspec.so")

SPEC_OK = 0
SPEC_E_INVAL = -1
SPEC_E_STATE = -2
SPEC_E_CAPACITY = -3
SPEC_E_HIP = -4
SPEC_E_UNSUPPORTED = -5
SPEC_DTYPE_FP32 = 0
SPEC_DTYPE_BF16 = 1
SPEC_LAYER_ATTN = 0
SPEC_LAYER_LR = 1
SPEC_WEIGHTS_NATIVE = 0
SPEC_WEIGHTS_W12 = 1
SPEC_WEIGHTS_W12_LOWP = 2
SPEC_MAX_LAYERS = 128

EXPORTS = [
    "spec_workspace_bytes", "spec_create", "spec_load_weights", "spec_prefill",
    "spec_verify", "spec_commit", "spec_release", "spec_request_state",
    "spec_force_root", "spec_set_fault", "spec_use_graphs", "spec_timing_enable",
    "spec_timing_read",
    "spec_destroy", "spec_last_error",
    "spec_acceptance_update", "spec_plan_drafts", "spec_verify_lowp", "spec_debug_flags",
    "spec_probe_read_bandwidth", "spec_probe_read_bandwidth_noalloc",
]


class spec_config(ctypes.Structure):
    _fields_ = [
        ("n_layers", c_int32), ("d_model", c_int32), ("n_heads", c_int32),
        ("n_kv_heads", c_int32), ("head_dim", c_int32), ("ffn_dim", c_int32),
        ("vocab", c_int32), ("dtype", c_int32), ("lr_state", c_int32),
        ("layer_kind", c_int32 * SPEC_MAX_LAYERS),
        ("rms_eps", c_float), ("rope_theta", c_float),
        ("max_requests", c_int32), ("max_ctx", c_int32), ("max_nodes", c_int32),
        ("max_rows", c_int32), ("prefill_chunk", c_int32), ("page_size", c_int32),
        ("weight_format", c_int32), ("kv_pages", c_int32),
    ]


class SpecError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libspec error {code}: {msg}")
        self.code = code


_lib = None


def lib():
    """Load libspec.so (once); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python tree_verification_spec_amd/build.py` (or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    P = POINTER
    i32p = P(c_int32)
    sig = {
        "spec_workspace_bytes": (c_size_t, [P(spec_config)]),
        "spec_create": (c_int32, [P(spec_config), c_void_p, c_size_t, c_void_p,
                                  P(c_void_p)]),
        "spec_load_weights": (c_int32, [c_void_p, c_int32, c_void_p, c_size_t, c_int32]),
        "spec_prefill": (c_int32, [c_void_p, c_int32, i32p, c_int32, i32p, c_void_p]),
        "spec_verify": (c_int32, [c_void_p, c_int32, i32p, i32p, i32p, i32p, i32p,
                                  i32p, i32p, c_void_p]),
        "spec_verify_lowp": (c_int32, [c_void_p, c_int32, i32p, i32p, i32p, i32p, i32p,
                                       i32p, i32p, c_void_p]),
        "spec_commit": (c_int32, [c_void_p, c_int32, i32p, i32p, i32p, i32p]),
        "spec_release": (c_int32, [c_void_p, c_int32]),
        "spec_request_state": (c_int32, [c_void_p, c_int32, i32p, i32p]),
        "spec_force_root": (c_int32, [c_void_p, c_int32, c_int32]),
        "spec_set_fault": (c_int32, [c_void_p, c_int32, c_float, c_int32]),
        "spec_use_graphs": (c_int32, [c_void_p, c_int32]),
        "spec_debug_flags": (c_int32, [c_void_p, c_int32]),
        "spec_timing_enable": (c_int32, [c_void_p, c_int32]),
        "spec_timing_read": (c_int32, [c_void_p, P(c_double), P(c_int64)]),
        "spec_destroy": (None, [c_void_p]),
        "spec_last_error": (ctypes.c_char_p, [c_void_p]),
        "spec_acceptance_update": (c_int32, [c_int32, i32p, i32p, c_float, P(c_float),
                                             P(c_float)]),
        "spec_plan_drafts": (c_int32, [c_int32, P(c_float), P(c_float), i32p, c_int32,
                                       c_float, c_int32, i32p]),
        "spec_probe_read_bandwidth": (c_int32, [c_void_p, c_size_t, c_int32, c_int32,
                                                c_int32, c_int32, c_void_p, c_void_p]),
        "spec_probe_read_bandwidth_noalloc": (c_int32, [c_void_p, c_size_t, c_int32, c_int32,
                                                        c_int32, c_int32, c_void_p, c_void_p]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _i32(seq):
    arr = (c_int32 * max(1, len(seq)))()
    for i, v in enumerate(seq):
        arr[i] = int(v)
    return arr


def _check(ctx, rc):
    if rc != SPEC_OK:
        raise SpecError(rc, spec_last_error(ctx))
    return rc


# ------------------------------------------------------------------ the ABI

def spec_workspace_bytes(cfg):
    return lib().spec_workspace_bytes(byref(cfg))


def spec_create(cfg, d_workspace, nbytes, hip_stream):
    out = c_void_p()
    rc = lib().spec_create(byref(cfg), c_void_p(d_workspace), nbytes,
                           c_void_p(hip_stream), byref(out))
    if rc != SPEC_OK:
        raise SpecError(rc, "spec_create failed (invalid config or workspace)")
    return out


def spec_load_weights(ctx, tensor_id, src_ptr, nbytes, src_on_device):
    return _check(ctx, lib().spec_load_weights(ctx, tensor_id, c_void_p(src_ptr),
                                               nbytes, int(src_on_device)))


def spec_prefill(ctx, req, prompt, d_logits=None):
    first = c_int32()
    p = _i32(prompt)
    _check(ctx, lib().spec_prefill(ctx, req, p, len(prompt), byref(first),
                                   c_void_p(d_logits or 0)))
    return first.value


def spec_verify(ctx, reqs, n_nodes, drafts, parents, max_nodes, d_logits=None,
                lowp=False):
    """Returns (paths: list of lists of draft indices, bonus: list).
    lowp: spec_verify_lowp (the 8-bit weight view; accepts nothing)."""
    n = len(reqs)
    slots = max_nodes - 1
    path = (c_int32 * max(1, n * slots))()
    plen = (c_int32 * n)()
    bonus = (c_int32 * n)()
    f = lib().spec_verify_lowp if lowp else lib().spec_verify
    _check(ctx, f(ctx, n, _i32(reqs), _i32(n_nodes), _i32(drafts), _i32(parents), path, plen,
                  bonus, c_void_p(d_logits or 0)))
    paths = [[path[r * slots + k] for k in range(plen[r])] for r in range(n)]
    return paths, list(bonus)


def spec_commit(ctx, reqs, paths, next_roots, max_nodes):
    n = len(reqs)
    slots = max_nodes - 1
    flat = [0] * max(1, n * slots)
    for r, p in enumerate(paths):
        for k, v in enumerate(p):
            flat[r * slots + k] = v
    return _check(ctx, lib().spec_commit(ctx, n, _i32(reqs), _i32(flat),
                                         _i32([len(p) for p in paths]),
                                         _i32(next_roots)))


def spec_release(ctx, req):
    return _check(ctx, lib().spec_release(ctx, req))


def spec_request_state(ctx, req):
    n, root = c_int32(), c_int32()
    rc = lib().spec_request_state(ctx, req, byref(n), byref(root))
    if rc != SPEC_OK:
        raise SpecError(rc, "request not active")
    return n.value, root.value


def spec_force_root(ctx, req, token):
    return _check(ctx, lib().spec_force_root(ctx, req, token))


def spec_set_fault(ctx, token, bias, after_position):
    return _check(ctx, lib().spec_set_fault(ctx, token, bias, after_position))


def spec_debug_flags(ctx, flags):
    return _check(ctx, lib().spec_debug_flags(ctx, flags))


def spec_use_graphs(ctx, enable):
    return _check(ctx, lib().spec_use_graphs(ctx, 1 if enable else 0))


def spec_timing_enable(ctx, cls):
    return _check(ctx, lib().spec_timing_enable(ctx, cls))


def spec_timing_read(ctx):
    ms, n = c_double(), c_int64()
    _check(ctx, lib().spec_timing_read(ctx, byref(ms), byref(n)))
    return ms.value, n.value


def _f32(seq):
    arr = (c_float * max(1, len(seq)))()
    for i, v in enumerate(seq):
        arr[i] = float(v)
    return arr


def spec_acceptance_update(offered, accepted, decay, succ, fail):
    """Decayed acceptance counts after one step (context-free); returns the
    new (succ, fail) lists."""
    n = len(offered)
    s, f = _f32(succ), _f32(fail)
    rc = lib().spec_acceptance_update(n, _i32(offered), _i32(accepted), decay, s, f)
    if rc:
        raise SpecError(rc, "spec_acceptance_update: invalid arguments")
    return list(s[:n]), list(f[:n])


def spec_plan_drafts(succ, fail, choices, min_prob, budget):
    """Per-request draft lengths under a shared node budget (context-free)."""
    n = len(succ)
    out = (c_int32 * max(1, n))()
    rc = lib().spec_plan_drafts(n, _f32(succ), _f32(fail), _i32(choices), len(choices),
                                min_prob, budget, out)
    if rc:
        raise SpecError(rc, "spec_plan_drafts: invalid arguments")
    return list(out[:n])


def spec_destroy(ctx):
    lib().spec_destroy(ctx)


def spec_last_error(ctx):
    s = lib().spec_last_error(ctx)
    return s.decode() if s else ""


def spec_probe_read_bandwidth(d_src, nbytes, grid, waves, depth, pattern, d_sink, stream):
    """Enqueue the streaming-read probe on `stream` (device pointers as ints)."""
    rc = lib().spec_probe_read_bandwidth(c_void_p(d_src), nbytes, grid, waves, depth,
                                         pattern, c_void_p(d_sink), c_void_p(stream))
    if rc != SPEC_OK:
        raise SpecError(rc, "spec_probe_read_bandwidth: invalid arguments or launch failure")


def spec_probe_read_bandwidth_noalloc(d_src, nbytes, grid, waves, depth, pattern, d_checksum,
                                      stream):
    """Enqueue the streaming-read probe with the library's own scratch; the
    XOR of every wavefront's checksum goes to d_checksum (one uint32)."""
    rc = lib().spec_probe_read_bandwidth_noalloc(c_void_p(d_src), nbytes, grid, waves, depth,
                                                 pattern, c_void_p(d_checksum),
                                                 c_void_p(stream))
    if rc != SPEC_OK:
        raise SpecError(rc, "spec_probe_read_bandwidth_noalloc: invalid arguments or launch "
                            "failure")
