"""ctypes binding for ``include/zero_flat.h``: same function names, argument
marshalling only.

Buffers may be given as torch tensors (their ``data_ptr()`` is passed) or as
integer device addresses.  ``stream`` defaults to torch's current HIP stream.
Every function raises ``ZeroError`` on a non-zero status.  There is no fallback:
if the shared library is missing, importing this module fails.
"""

import ctypes
import os

# torch brings its own HIP runtime.  Load it BEFORE the library so that the
# library's libamdhip64.so.7 dependency resolves to that same copy: two HIP
# runtimes in one process each open the device, and the second one sees none.
import torch  # noqa: F401

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "libzero_flat.so")

ZERO_OK = 0
ZERO_EINVAL = -1
ZERO_EALIAS = -2
ZERO_EHIP = -3
ZERO_ENOMEM = -4
ZERO_EIO = -5
ZERO_F16 = 1
ZERO_BF16 = 2
ZERO_MAX_RANKS = 1024
ZERO_MAX_ELEMS = 1 << 34
ZERO_FLAG_NONFINITE_GRAD = 1
ZERO_FLAG_NONFINITE_NORM = 2
ZERO_FLAG_NO_CONSTS = 4

# Every symbol include/zero_flat.h declares.
EXPORTED = (
    "zero_plan_create", "zero_plan_destroy", "zero_plan_info", "zero_plan_rank", "zero_plan_unit",
    "zero_plan_full_numel", "zero_plan_segments", "zero_model_state_bytes", "zero_comm_volume",
    "zero_workspace_bytes", "zero_reduce_shard", "zero_grad_norm", "zero_adam_step",
    "zero_gather_params", "zero_last_error", "zero_version",
    "zero_quant_code_bytes", "zero_quant_scale_count", "zero_quantize_blocks", "zero_dequantize_blocks",
    "zero_gather_dequant", "zero_cpu_adam_step", "zero_offload_adam_step", "zero_cpu_isa", "zero_cpu_set_isa",
    "zero_plan_reshard", "zero_ckpt_save", "zero_ckpt_load", "zero_adam_consts_fill", "zero_adam_step_consts",
    "zero_grad_norm_noalloc", "zero_reduce_owners", "zero_adam_step_owners", "zero_step_end",
    "zero_offload_create", "zero_offload_destroy", "zero_offload_begin", "zero_offload_end",
)
ZERO_QBLOCK = 256
ZERO_CPU_SCALAR = 0
ZERO_CPU_AVX2 = 1
ZERO_CPU_AVX512 = 2
ZERO_OFFLOAD_MIN_STAGING = 576
ZERO_LOC_DEVICE = 0
ZERO_LOC_HOST = 1
ZERO_CKPT_BLOCK = 262144
ZERO_CKPT_MIN_STAGING = 2 * 4 * ZERO_CKPT_BLOCK
ZERO_NOALLOC_MAX_ELEMS = 1 << 34
ZERO_NOALLOC_SCRATCH_BYTES = 16384 + 8 * (ZERO_NOALLOC_MAX_ELEMS // 2048)


class ZeroError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"[{code}] {message}")
        self.code = code


class zero_segment(ctypes.Structure):
    _fields_ = [("tensor", ctypes.c_int64), ("tensor_off", ctypes.c_int64),
                ("shard_off", ctypes.c_int64), ("len", ctypes.c_int64)]


class zero_reshard_segment(ctypes.Structure):
    _fields_ = [("old_rank", ctypes.c_int64), ("old_offset", ctypes.c_int64), ("new_offset", ctypes.c_int64),
                ("len", ctypes.c_int64)]


class zero_adam_hparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("inv_loss_scale", ctypes.c_float), ("step", ctypes.c_int64)]


class zero_step_state(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int64), ("applied", ctypes.c_int64), ("skipped", ctypes.c_int64),
                ("table_t0", ctypes.c_int64), ("last_flag", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class zero_adam_consts(ctypes.Structure):
    _fields_ = [(name, ctypes.c_float) for name in (
        "lr", "beta1", "beta2", "one_minus_beta1", "one_minus_beta2", "eps", "weight_decay", "inv_loss_scale",
        "bias_corr1", "bias_corr2")]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m zero_sharded_mixed_flat_amd.build`")

lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_sig = {
    "zero_plan_create": (_I, [ctypes.POINTER(_I64), _I, _I, _I, _I64, ctypes.POINTER(_P)]),
    "zero_plan_destroy": (None, [_P]),
    "zero_plan_info": (_I, [_P, ctypes.POINTER(_I), ctypes.POINTER(_I), ctypes.POINTER(_I),
                            ctypes.POINTER(_I)]),
    "zero_plan_rank": (_I, [_P, _I, ctypes.POINTER(_I64), ctypes.POINTER(_I64)]),
    "zero_plan_unit": (_I, [_P, _I, ctypes.POINTER(_I64), ctypes.POINTER(_I64), ctypes.POINTER(_I64),
                            ctypes.POINTER(_I64)]),
    "zero_plan_full_numel": (_I, [_P, ctypes.POINTER(_I64)]),
    "zero_plan_segments": (_I, [_P, ctypes.POINTER(_I64), _I, _I, ctypes.POINTER(zero_segment), _I,
                                ctypes.POINTER(_I)]),
    "zero_model_state_bytes": (_I, [ctypes.c_double, _I, _I, _I, ctypes.POINTER(ctypes.c_double)]),
    "zero_comm_volume": (_I, [ctypes.c_double, _I, _I, ctypes.POINTER(ctypes.c_double)]),
    "zero_workspace_bytes": (_I64, [_I64, _I]),
    "zero_reduce_shard": (_I, [ctypes.POINTER(_P), _I, _I64, _I, ctypes.c_float, _P, _P, _I64, _I, _P,
                               _P]),
    "zero_grad_norm": (_I, [_P, _I64, _I, ctypes.c_float, _P, _I64, _I, _P, _I, ctypes.c_float, _P, _P,
                            _P, _P]),
    "zero_grad_norm_noalloc": (_I, [_P, _I64, _I, ctypes.c_float, _P, _I, ctypes.c_float, _P, _P, _P, _P]),
    "zero_reduce_owners": (_I, [ctypes.POINTER(_P), _I, _I64, _I, _I64, _I, ctypes.c_float, _P, _I64, _P, _I64,
                                _P, _P]),
    "zero_adam_step_owners": (_I, [_P, _P, _P, _I64, _P, _I, _I64, _I64, _I, _P, _I64, _P, _P, _P, _P, _I64, _I,
                                   _P]),
    "zero_step_end": (_I, [_P, _P, _P]),
    "zero_adam_step": (_I, [_P, _P, _P, _P, _I, _I64, ctypes.POINTER(zero_adam_hparams), _P, _P, _P, _I,
                            _P]),
    "zero_gather_params": (_I, [_P, ctypes.POINTER(_P), _I, _I, _I, _P, _P, _I64, _P]),
    "zero_adam_consts_fill": (_I, [ctypes.POINTER(zero_adam_hparams), ctypes.POINTER(zero_adam_consts)]),
    "zero_adam_step_consts": (_I, [_P, _P, _P, _P, _I, _I64, _P, _P, _P, _P, _I, _P]),
    "zero_quant_code_bytes": (_I64, [_I64, _I]),
    "zero_quant_scale_count": (_I64, [_I64]),
    "zero_quantize_blocks": (_I, [_P, _I, _I64, _I, _P, _P, _P]),
    "zero_dequantize_blocks": (_I, [_P, _P, _I64, _I, _P, _I, _P]),
    "zero_gather_dequant": (_I, [_P, ctypes.POINTER(_P), ctypes.POINTER(_P), _I, _I, _I, _I, _P, _P, _I64, _P]),
    "zero_cpu_adam_step": (_I, [_P, _P, _P, _P, _I, _I64, ctypes.POINTER(zero_adam_hparams), ctypes.c_float, _I,
                                _P, _I, _I]),
    "zero_offload_adam_step": (_I, [_P, _P, _P, _P, _I, _I64, ctypes.POINTER(zero_adam_hparams), _P, _P, _P, _I,
                                    _P, _I64, _I, _P]),
    "zero_offload_create": (_I, [_I, ctypes.POINTER(_P)]),
    "zero_offload_destroy": (None, [_P]),
    "zero_offload_begin": (_I, [_P, _P, _P, _P, _P, _I, _I64, ctypes.POINTER(zero_adam_hparams), _P, _P, _I, _P,
                                _I64, _P, _I64, _P]),
    "zero_offload_end": (_I, [_P, _P, ctypes.POINTER(_I), _P]),
    "zero_plan_reshard": (_I, [_P, _P, _I, ctypes.POINTER(zero_reshard_segment), _I, ctypes.POINTER(_I)]),
    "zero_ckpt_save": (_I, [ctypes.c_char_p, _P, _I, _I64, _P, _P, _P, _I, _P, _I64, _P]),
    "zero_ckpt_load": (_I, [ctypes.POINTER(ctypes.c_char_p), _I, _P, _I, _P, _P, _P, _I, ctypes.POINTER(_I64), _P,
                            _I64, _P]),
    "zero_cpu_isa": (_I, []),
    "zero_cpu_set_isa": (_I, [_I]),
    "zero_last_error": (ctypes.c_char_p, []),
    "zero_version": (_I, []),
}
for _name, (_res, _args) in _sig.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def zero_last_error():
    return lib.zero_last_error().decode()


def zero_version():
    return lib.zero_version()


def _check(status):
    if status != ZERO_OK:
        raise ZeroError(status, zero_last_error())


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _need(x, nbytes, what):
    """A tensor argument must be a contiguous device tensor holding nbytes."""
    if x is None or isinstance(x, int) or nbytes <= 0:
        return
    if not x.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not x.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    have = x.numel() * x.element_size()
    if have < nbytes:
        raise ValueError(f"{what} holds {have} bytes, needs {nbytes}")


def _need_host(x, nbytes, what):
    """A tensor argument must be a contiguous host tensor holding nbytes."""
    if x is None or isinstance(x, int) or nbytes <= 0:
        return
    if x.is_cuda:
        raise ValueError(f"{what} must be a host tensor")
    if not x.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    have = x.numel() * x.element_size()
    if have < nbytes:
        raise ValueError(f"{what} holds {have} bytes, needs {nbytes}")


def _nbytes(x):
    if x is None:
        return 0
    if isinstance(x, int):
        raise TypeError("pass the workspace as a tensor (or give its size explicitly)")
    return x.numel() * x.element_size()


def _dtype(d):
    if isinstance(d, int):
        return d                      # validated by the library
    name = str(d)
    table = {"f16": ZERO_F16, "bf16": ZERO_BF16, "torch.float16": ZERO_F16,
             "torch.bfloat16": ZERO_BF16}
    if name in table:
        return table[name]
    raise ValueError(f"not a 16-bit dtype: {d!r}")


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


class PointerTable:
    """A host array of device pointers to a list of tensors, marshalled once.

    Entry points that take one buffer per rank accept a table in place of the
    list, which saves re-marshalling (and re-validating) the same pointers on
    every call.  The table keeps references to its tensors, so their memory
    stays valid while it lives.  Every tensor is checked against ``nbytes``
    (a contiguous device tensor holding at least that many bytes) when the
    table is built.
    """

    def __init__(self, tensors, nbytes, what="buffer"):
        self.tensors = list(tensors)
        for i, t in enumerate(self.tensors):
            _need(t, nbytes, f"{what} {i}")
        self.nbytes = int(nbytes)
        self.array = (_P * len(self.tensors))(*[_ptr(t) for t in self.tensors])

    def __len__(self):
        return len(self.tensors)


def _table(buffers, nbytes, what):
    """Pointer array for a list of tensors (validated) or a prebuilt PointerTable."""
    if isinstance(buffers, PointerTable):
        if buffers.nbytes < nbytes:
            raise ValueError(f"{what} table was validated for {buffers.nbytes} bytes per buffer, needs {nbytes}")
        return buffers.array
    for i, t in enumerate(buffers):
        _need(t, nbytes, f"{what} {i}")
    return (_P * len(buffers))(*[_ptr(t) for t in buffers])


# ---------------------------------------------------------------------------
# a0: partition
# ---------------------------------------------------------------------------

class Plan:
    """Owns a ``zero_plan*``; mirrors zero_plan_* as methods."""

    def __init__(self, unit_numels, nd, stage, align=8):
        self.handle = _P()
        sizes = (_I64 * len(unit_numels))(*[int(u) for u in unit_numels])
        handle = _P()
        _check(lib.zero_plan_create(sizes, len(unit_numels), int(nd), int(stage), int(align),
                                    ctypes.byref(handle)))
        self.handle = handle
        self._cache = {}

    def close(self):
        if self.handle and lib is not None:          # the module may be torn down first at exit
            lib.zero_plan_destroy(self.handle)
            self.handle = _P()

    def __del__(self):
        self.close()

    def info(self):
        if "info" not in self._cache:
            a, b, c, d = _I(), _I(), _I(), _I()
            _check(lib.zero_plan_info(self.handle, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c),
                                      ctypes.byref(d)))
            self._cache["info"] = {"n_units": a.value, "owners": b.value, "nd": c.value, "stage": d.value}
        return dict(self._cache["info"])

    def rank(self, rank):
        key = ("rank", int(rank))
        if key not in self._cache:
            s, r = _I64(), _I64()
            _check(lib.zero_plan_rank(self.handle, int(rank), ctypes.byref(s), ctypes.byref(r)))
            self._cache[key] = (s.value, r.value)
        return self._cache[key]

    def unit(self, unit):
        a, b, c, d = _I64(), _I64(), _I64(), _I64()
        _check(lib.zero_plan_unit(self.handle, int(unit), ctypes.byref(a), ctypes.byref(b),
                                  ctypes.byref(c), ctypes.byref(d)))
        return a.value, b.value, c.value, d.value

    def full_numel(self):
        if "full" not in self._cache:
            x = _I64()
            _check(lib.zero_plan_full_numel(self.handle, ctypes.byref(x)))
            self._cache["full"] = x.value
        return self._cache["full"]

    def segments(self, tensor_numels, rank):
        sizes = (_I64 * len(tensor_numels))(*[int(t) for t in tensor_numels])
        count = _I()
        _check(lib.zero_plan_segments(self.handle, sizes, len(tensor_numels), int(rank), None, 0,
                                      ctypes.byref(count)))
        out = (zero_segment * max(count.value, 1))()
        _check(lib.zero_plan_segments(self.handle, sizes, len(tensor_numels), int(rank), out,
                                      count.value, ctypes.byref(count)))
        return [(s.tensor, s.tensor_off, s.shard_off, s.len) for s in out[:count.value]]


def zero_plan_reshard(old_plan, new_plan, new_rank):
    """Runs (old_rank, old_offset, new_offset, len) filling new_rank's shard from the old shards."""
    count = _I()
    _check(lib.zero_plan_reshard(old_plan.handle, new_plan.handle, int(new_rank), None, 0, ctypes.byref(count)))
    out = (zero_reshard_segment * max(count.value, 1))()
    _check(lib.zero_plan_reshard(old_plan.handle, new_plan.handle, int(new_rank), out, count.value,
                                 ctypes.byref(count)))
    return [(s.old_rank, s.old_offset, s.new_offset, s.len) for s in out[:count.value]]


def zero_plan_create(unit_numels, nd, stage, align=8):
    return Plan(unit_numels, nd, stage, align)


# ---------------------------------------------------------------------------
# accounting and workspace
# ---------------------------------------------------------------------------

def zero_model_state_bytes(psi, nd, stage, k_bytes=12):
    out = ctypes.c_double()
    _check(lib.zero_model_state_bytes(float(psi), int(nd), int(stage), int(k_bytes), ctypes.byref(out)))
    return out.value


def zero_comm_volume(psi, nd, stage):
    out = ctypes.c_double()
    _check(lib.zero_comm_volume(float(psi), int(nd), int(stage), ctypes.byref(out)))
    return out.value


def zero_workspace_bytes(n, n_sets):
    b = lib.zero_workspace_bytes(int(n), int(n_sets))
    if b < 0:
        raise ZeroError(ZERO_EINVAL, zero_last_error())
    return b


# ---------------------------------------------------------------------------
# a1-a4
# ---------------------------------------------------------------------------

def zero_reduce_shard(contribs, n, dtype, inv_loss_scale, reduced_out, workspace, set_index, flag,
                      stream=None, workspace_bytes=None):
    ptrs = _table(contribs, 2 * n, "contribution")
    _need(reduced_out, 2 * n, "reduced_out")
    _need(flag, 4, "flag")
    wb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    _check(lib.zero_reduce_shard(ptrs, len(contribs), int(n), _dtype(dtype), float(inv_loss_scale),
                                 _ptr(reduced_out), _ptr(workspace), wb, int(set_index), _ptr(flag),
                                 _stream(stream)))


def zero_reduce_owners(contribs, n, owners, contrib_stride, dtype, inv_loss_scale, reduced_out, reduced_stride,
                       workspace, flag, stream=None, workspace_bytes=None):
    """``contribs``: one device tensor (or a PointerTable) per rank, each holding every owner's
    contribution from that rank (owner o's at element o * contrib_stride)."""
    span = (owners - 1) * contrib_stride + n if n > 0 else 0
    ptrs = _table(contribs, 2 * span, "contribution")
    _need(reduced_out, 2 * ((owners - 1) * reduced_stride + n) if n > 0 else 0, "reduced_out")
    _need(flag, 4, "flag")
    wb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    _check(lib.zero_reduce_owners(ptrs, len(contribs), int(n), int(owners), int(contrib_stride), _dtype(dtype),
                                  float(inv_loss_scale), _ptr(reduced_out), int(reduced_stride), _ptr(workspace), wb,
                                  _ptr(flag), _stream(stream)))


def step_state(first_step=1, table_t0=1):
    """A zero_step_state for the device (copy it into 40 device bytes)."""
    return zero_step_state(int(first_step), 0, 0, int(table_t0), 0, 0)


def zero_adam_step_owners(master, m, v, state_stride, grad, grad_dtype, grad_stride, n, owners, table_dev,
                          table_len, state_dev, coef, flag, param_out, param_stride, param_dtype, stream=None):
    ext = lambda stride, b: b * ((owners - 1) * stride + n) if n > 0 else 0
    for t, b, what in ((master, ext(state_stride, 4), "master"), (m, ext(state_stride, 4), "m"),
                       (v, ext(state_stride, 4), "v"), (grad, ext(grad_stride, 2), "grad"),
                       (param_out, ext(param_stride, 2), "param_out"), (coef, 4, "coef"), (flag, 4, "flag"),
                       (table_dev, table_len * ctypes.sizeof(zero_adam_consts), "table_dev"),
                       (state_dev, ctypes.sizeof(zero_step_state), "state_dev")):
        _need(t, b, what)
    _check(lib.zero_adam_step_owners(_ptr(master), _ptr(m), _ptr(v), int(state_stride), _ptr(grad),
                                     _dtype(grad_dtype), int(grad_stride), int(n), int(owners), _ptr(table_dev),
                                     int(table_len), _ptr(state_dev), _ptr(coef), _ptr(flag), _ptr(param_out),
                                     int(param_stride), _dtype(param_dtype), _stream(stream)))


def zero_step_end(flag, state_dev, stream=None):
    _need(flag, 4, "flag")
    _need(state_dev, ctypes.sizeof(zero_step_state), "state_dev")
    _check(lib.zero_step_end(_ptr(flag), _ptr(state_dev), _stream(stream)))


def zero_grad_norm(grad, n, dtype, inv_loss_scale, workspace, n_sets, extra_sumsq, n_extra, max_norm,
                   flag, norm_out, coef_out, stream=None, workspace_bytes=None):
    wb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    _need(grad, 2 * n, "grad")
    _need(extra_sumsq, 8 * n_extra, "extra_sumsq")
    for t, b, what in ((flag, 4, "flag"), (norm_out, 8, "norm_out"), (coef_out, 4, "coef_out")):
        _need(t, b, what)
    dt = _dtype(dtype) if grad is not None else 0
    _check(lib.zero_grad_norm(_ptr(grad), int(n), dt, float(inv_loss_scale), _ptr(workspace), wb,
                              int(n_sets), _ptr(extra_sumsq), int(n_extra), float(max_norm), _ptr(flag),
                              _ptr(norm_out), _ptr(coef_out), _stream(stream)))


def zero_grad_norm_noalloc(grad, n, dtype, inv_loss_scale, extra_sumsq, n_extra, max_norm, flag, norm_out,
                           coef_out, stream=None):
    _need(grad, 2 * n, "grad")
    _need(extra_sumsq, 8 * n_extra, "extra_sumsq")
    for t, b, what in ((flag, 4, "flag"), (norm_out, 8, "norm_out"), (coef_out, 4, "coef_out")):
        _need(t, b, what)
    dt = _dtype(dtype) if grad is not None else 0
    _check(lib.zero_grad_norm_noalloc(_ptr(grad), int(n), dt, float(inv_loss_scale), _ptr(extra_sumsq),
                                      int(n_extra), float(max_norm), _ptr(flag), _ptr(norm_out), _ptr(coef_out),
                                      _stream(stream)))


def adam_hparams(lr, beta1, beta2, eps, weight_decay, inv_loss_scale, step):
    return zero_adam_hparams(lr, beta1, beta2, eps, weight_decay, inv_loss_scale, int(step))


def zero_adam_step(master, m, v, grad, grad_dtype, n, hp, coef, flag, param_out, param_dtype,
                   stream=None):
    for t, b, what in ((master, 4 * n, "master"), (m, 4 * n, "m"), (v, 4 * n, "v"),
                       (grad, 2 * n, "grad"), (param_out, 2 * n, "param_out"), (coef, 4, "coef"),
                       (flag, 4, "flag")):
        _need(t, b, what)
    _check(lib.zero_adam_step(_ptr(master), _ptr(m), _ptr(v), _ptr(grad), _dtype(grad_dtype), int(n),
                              ctypes.byref(hp), _ptr(coef), _ptr(flag), _ptr(param_out),
                              _dtype(param_dtype), _stream(stream)))


def zero_adam_consts_fill(hp):
    """The fp32 scalars zero_adam_step derives from hp, as a zero_adam_consts (host)."""
    out = zero_adam_consts()
    _check(lib.zero_adam_consts_fill(ctypes.byref(hp), ctypes.byref(out)))
    return out


def zero_adam_step_consts(master, m, v, grad, grad_dtype, n, consts_dev, coef, flag, param_out, param_dtype,
                          stream=None):
    for t, b, what in ((master, 4 * n, "master"), (m, 4 * n, "m"), (v, 4 * n, "v"),
                       (grad, 2 * n, "grad"), (param_out, 2 * n, "param_out"), (coef, 4, "coef"),
                       (flag, 4, "flag"), (consts_dev, ctypes.sizeof(zero_adam_consts), "consts_dev")):
        _need(t, b, what)
    _check(lib.zero_adam_step_consts(_ptr(master), _ptr(m), _ptr(v), _ptr(grad), _dtype(grad_dtype), int(n),
                                     _ptr(consts_dev), _ptr(coef), _ptr(flag), _ptr(param_out), _dtype(param_dtype),
                                     _stream(stream)))


def zero_gather_params(plan, shards, unit_begin, unit_end, dtype, full, workspace=None, stream=None,
                       workspace_bytes=None):
    wb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    handle = plan.handle if isinstance(plan, Plan) else plan
    if isinstance(plan, Plan):
        info = plan.info()
        if len(shards) != info["owners"]:
            raise ValueError(f"need {info['owners']} shards, got {len(shards)}")
        shard_numel, _ = plan.rank(0)
        ptrs = _table(shards, 2 * shard_numel, "shard")
        _need(full, 2 * plan.full_numel(), "full")
    else:
        ptrs = _table(shards, 0, "shard")
    _check(lib.zero_gather_params(handle, ptrs, int(unit_begin), int(unit_end), _dtype(dtype),
                                  _ptr(full), _ptr(workspace), wb, _stream(stream)))


# ---------------------------------------------------------------------------
# block-quantised parameter gather
# ---------------------------------------------------------------------------

def zero_quant_code_bytes(n, bits):
    b = lib.zero_quant_code_bytes(int(n), int(bits))
    if b < 0:
        raise ZeroError(ZERO_EINVAL, zero_last_error())
    return b


def zero_quant_scale_count(n):
    c = lib.zero_quant_scale_count(int(n))
    if c < 0:
        raise ZeroError(ZERO_EINVAL, zero_last_error())
    return c


def zero_quantize_blocks(x, dtype, n, bits, codes, scales, stream=None):
    if n > 0 and bits in (8, 4):
        _need(x, 2 * n, "x")
        _need(codes, zero_quant_code_bytes(n, bits), "codes")
        _need(scales, 4 * zero_quant_scale_count(n), "scales")
    _check(lib.zero_quantize_blocks(_ptr(x), _dtype(dtype), int(n), int(bits), _ptr(codes), _ptr(scales),
                                    _stream(stream)))


def zero_dequantize_blocks(codes, scales, n, bits, y, dtype, stream=None):
    if n > 0 and bits in (8, 4):
        _need(codes, zero_quant_code_bytes(n, bits), "codes")
        _need(scales, 4 * zero_quant_scale_count(n), "scales")
        _need(y, 2 * n, "y")
    _check(lib.zero_dequantize_blocks(_ptr(codes), _ptr(scales), int(n), int(bits), _ptr(y), _dtype(dtype),
                                      _stream(stream)))


def zero_gather_dequant(plan, code_shards, scale_shards, unit_begin, unit_end, bits, dtype, full, workspace=None,
                        stream=None, workspace_bytes=None):
    wb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    handle = plan.handle if isinstance(plan, Plan) else plan
    code_bytes = scale_bytes = 0
    if isinstance(plan, Plan):
        owners = plan.info()["owners"]
        if len(code_shards) != owners or len(scale_shards) != owners:
            raise ValueError(f"need {owners} code and scale shards")
        shard_numel, _ = plan.rank(0)
        if bits in (8, 4):
            code_bytes = zero_quant_code_bytes(shard_numel, bits)
            scale_bytes = 4 * zero_quant_scale_count(shard_numel)
        _need(full, 2 * plan.full_numel(), "full")
    cp = _table(code_shards, code_bytes, "code shard")
    sp = _table(scale_shards, scale_bytes, "scale shard")
    _check(lib.zero_gather_dequant(handle, cp, sp, int(unit_begin), int(unit_end), int(bits), _dtype(dtype),
                                   _ptr(full), _ptr(workspace), wb, _stream(stream)))


# ---------------------------------------------------------------------------
# CPU-offloaded optimizer (ZeRO-Offload)
# ---------------------------------------------------------------------------

def zero_cpu_isa():
    return lib.zero_cpu_isa()


def zero_cpu_set_isa(isa):
    _check(lib.zero_cpu_set_isa(int(isa)))


def zero_cpu_adam_step(master, m, v, grad, grad_dtype, n, hp, coef, skip, param_out, param_dtype, n_threads):
    for t, b, what in ((master, 4 * n, "master"), (m, 4 * n, "m"), (v, 4 * n, "v"), (grad, 2 * n, "grad"),
                       (param_out, 2 * n, "param_out")):
        _need_host(t, b, what)
    _check(lib.zero_cpu_adam_step(_ptr(master), _ptr(m), _ptr(v), _ptr(grad), _dtype(grad_dtype), int(n),
                                  ctypes.byref(hp), float(coef), int(bool(skip)), _ptr(param_out),
                                  _dtype(param_dtype), int(n_threads)))


def zero_offload_adam_step(master, m, v, grad, grad_dtype, n, hp, coef, flag, param_out, param_dtype, staging,
                           n_threads, stream=None, staging_bytes=None):
    for t, b, what in ((master, 4 * n, "master"), (m, 4 * n, "m"), (v, 4 * n, "v")):
        _need_host(t, b, what)
    _need_host(staging, ZERO_OFFLOAD_MIN_STAGING, "staging")
    for t, b, what in ((grad, 2 * n, "grad"), (param_out, 2 * n, "param_out"), (coef, 4, "coef"),
                       (flag, 4, "flag")):
        _need(t, b, what)
    sb = _nbytes(staging) if staging_bytes is None else staging_bytes
    _check(lib.zero_offload_adam_step(_ptr(master), _ptr(m), _ptr(v), _ptr(grad), _dtype(grad_dtype), int(n),
                                      ctypes.byref(hp), _ptr(coef), _ptr(flag), _ptr(param_out),
                                      _dtype(param_dtype), _ptr(staging), int(sb), int(n_threads),
                                      _stream(stream)))


class Offload:
    """A zero_offload handle: the one-step-delayed host AdamW (begin / end)."""

    def __init__(self, n_threads):
        self.handle = _P()
        handle = _P()
        _check(lib.zero_offload_create(int(n_threads), ctypes.byref(handle)))
        self.handle = handle
        self._n = None                 # n of the update in flight
        self._keep = None              # buffers the update in flight uses

    def close(self):
        if self.handle and lib is not None:
            lib.zero_offload_destroy(self.handle)
            self.handle = _P()

    def __del__(self):
        self.close()

    def begin(self, master, m, v, grad, grad_dtype, n, hp, coef, flag, param_dtype, device_buffer, staging,
              stream=None, device_bytes=None, staging_bytes=None):
        for t, b, what in ((master, 4 * n, "master"), (m, 4 * n, "m"), (v, 4 * n, "v")):
            _need_host(t, b, what)
        _need_host(staging, ZERO_OFFLOAD_MIN_STAGING, "staging")
        for t, b, what in ((grad, 2 * n, "grad"), (coef, 4, "coef"), (flag, 4, "flag"),
                           (device_buffer, 4 * n, "device_buffer")):
            _need(t, b, what)
        db = _nbytes(device_buffer) if device_bytes is None else device_bytes
        sb = _nbytes(staging) if staging_bytes is None else staging_bytes
        _check(lib.zero_offload_begin(self.handle, _ptr(master), _ptr(m), _ptr(v), _ptr(grad), _dtype(grad_dtype),
                                      int(n), ctypes.byref(hp), _ptr(coef), _ptr(flag), _dtype(param_dtype),
                                      _ptr(device_buffer), int(db), _ptr(staging), int(sb), _stream(stream)))
        self._n = int(n)
        self._keep = (master, m, v, device_buffer, staging)

    def end(self, param_out, stream=None):
        """Finish the update in flight; returns True if it was applied."""
        if self._n is not None:
            _need(param_out, 2 * self._n, "param_out")
        applied = _I()
        rc = lib.zero_offload_end(self.handle, _ptr(param_out), ctypes.byref(applied), _stream(stream))
        if rc not in (ZERO_EINVAL, ZERO_EALIAS):    # the update has ended (applied, skipped or failed)
            self._n = None
            self._keep = None
        _check(rc)
        return bool(applied.value)

    @property
    def in_flight(self):
        return self._n is not None


# ---------------------------------------------------------------------------
# sharded checkpoints
# ---------------------------------------------------------------------------

def _location(tensors):
    devs = {t.is_cuda for t in tensors if t is not None and not isinstance(t, int)}
    if len(devs) > 1:
        raise ValueError("master, m and v must all be device tensors or all host tensors")
    return ZERO_LOC_DEVICE if devs == {True} else ZERO_LOC_HOST


def _check_state(plan, arrays, location):
    n, _ = plan.rank(0)
    for t, what in zip(arrays, ("master", "m", "v")):
        (_need if location == ZERO_LOC_DEVICE else _need_host)(t, 4 * n, what)


def zero_ckpt_save(path, plan, rank, step, master, m, v, staging, stream=None, location=None, staging_bytes=None):
    loc = _location((master, m, v)) if location is None else location
    _check_state(plan, (master, m, v), loc)
    _need_host(staging, ZERO_CKPT_MIN_STAGING, "staging")
    sb = _nbytes(staging) if staging_bytes is None else staging_bytes
    _check(lib.zero_ckpt_save(os.fsencode(path), plan.handle, int(rank), int(step), _ptr(master), _ptr(m), _ptr(v),
                              int(loc), _ptr(staging), int(sb), _stream(stream) if loc == ZERO_LOC_DEVICE else None))


def zero_ckpt_load(paths, plan, rank, master, m, v, staging, stream=None, location=None, staging_bytes=None):
    """Restores rank's shard under ``plan`` from every old rank's file; returns the saved step."""
    loc = _location((master, m, v)) if location is None else location
    _check_state(plan, (master, m, v), loc)
    _need_host(staging, ZERO_CKPT_MIN_STAGING, "staging")
    sb = _nbytes(staging) if staging_bytes is None else staging_bytes
    arr = (ctypes.c_char_p * len(paths))(*[os.fsencode(p) for p in paths])
    step = _I64()
    _check(lib.zero_ckpt_load(arr, len(paths), plan.handle, int(rank), _ptr(master), _ptr(m), _ptr(v), int(loc),
                              ctypes.byref(step), _ptr(staging), int(sb),
                              _stream(stream) if loc == ZERO_LOC_DEVICE else None))
    return step.value
