"""ctypes binding of ``include/ns.h``: argument marshalling only.

Python functions carry the C entry points' names. Torch supplies device memory
(tensors) and streams; every step of the path runs in the HIP library. The
library is loaded on first use and a missing build raises ``NSLibraryMissing``
(there is no fallback of any kind).
"""

from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnsq.so")

NS_BF16, NS_F32 = 0, 1
NS_MAX_DIMS, NS_MAX_SHARDS = 8, 64
STATUS = {
    0: "NS_OK", -1: "NS_ERR_INVALID_ARG", -2: "NS_ERR_NO_CANDIDATE", -3: "NS_ERR_HOME_RANGE",
    -4: "NS_ERR_SPLIT_SUM", -5: "NS_ERR_OVERFLOW", -6: "NS_ERR_PLAN_MISMATCH",
    -7: "NS_ERR_WORKSPACE", -8: "NS_ERR_DTYPE", -9: "NS_ERR_HIP",
}
EXPORTS = [
    "ns_last_error", "ns_version", "ns_plan", "ns_route_plan_create", "ns_route_plan_create_axis",
    "ns_route_plan_query",
    "ns_route_plan_upload", "ns_route_plan_destroy", "ns_pack_shards", "ns_unpack_shards",
    "ns_workspace_bytes", "ns_orthogonalize_batched", "ns_noalloc_init", "ns_orthogonalize_batched_noalloc",
    "ns_orthogonalize_strided", "ns_routed_workspace_bytes",
    "ns_orthogonalize_routed", "ns_gram_workspace_bytes", "ns_orthogonalize_gram", "ns_wave_plan", "ns_orthogonalize_waves", "ns_timing_enable",
    "ns_timing_read",
]


class NSLibraryMissing(ImportError):
    pass


class NSError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class ns_shape(ctypes.Structure):
    _fields_ = [("ndim", ctypes.c_int32), ("dims", ctypes.c_int64 * NS_MAX_DIMS)]


_P = ctypes.c_void_p
_I32, _I64, _U64, _F32, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "ns_last_error": (ctypes.c_char_p, []),
    "ns_version": (ctypes.c_char_p, []),
    "ns_plan": (_I32, [_I32, _P, _I32, _I32, _P, _P, _P, _P, _P]),
    "ns_route_plan_create": (_I32, [_I32, _P, _I32, _P, _P, _I32, ctypes.POINTER(_P)]),
    "ns_route_plan_create_axis": (_I32, [_I32, _P, _I32, _P, _P, _P, _I32, ctypes.POINTER(_P)]),
    "ns_route_plan_query": (_I32, [_P, _P, _P, _P, _P, _P, _P]),
    "ns_route_plan_upload": (_I32, [_P, _P, _P]),
    "ns_route_plan_destroy": (None, [_P]),
    "ns_pack_shards": (_I32, [_P, _P, _P, _P]),
    "ns_unpack_shards": (_I32, [_P, _P, _P, _P]),
    "ns_workspace_bytes": (_I32, [_I32, _P, _I32, _P, _P]),
    "ns_orthogonalize_batched": (_I32, [_I32, _P, _P, _P, _I32, _I32, _F32, _F32, _F32, _F32, _P, _P,
                                        _SZ, _P]),
    "ns_noalloc_init": (_I32, []),
    "ns_orthogonalize_batched_noalloc": (_I32, [_I32, _P, _P, _P, _I32, _I32, _F32, _F32, _F32, _F32, _P, _P]),
    "ns_orthogonalize_strided": (_I32, [_I32, _P, _P, _P, _P, _P, _I32, _I32, _F32, _F32, _F32, _F32, _P,
                                        _P, _SZ, _P]),
    "ns_routed_workspace_bytes": (_I32, [_P, _I32, _P, _P]),
    "ns_orthogonalize_routed": (_I32, [_P, _P, _P, _I32, _I32, _F32, _F32, _F32, _F32, _P, _P, _SZ, _P]),
    "ns_gram_workspace_bytes": (_I32, [_I32, _P, _I32, _P, _P]),
    "ns_orthogonalize_gram": (_I32, [_I32, _P, _P, _P, _I32, _I32, _F32, _F32, _F32, _F32, _F32, _P, _P, _SZ,
                                     _P]),
    "ns_wave_plan": (_I32, [_I32, _P, _P, _I32, _P, _P]),
    "ns_orthogonalize_waves": (_I32, [_I32, _P, _P, _P, _I32, _I32, _F32, _F32, _F32, _F32, _P, _I32, _P,
                                      _P, _SZ, _P]),
    "ns_timing_enable": (_I32, [_I32]),
    "ns_timing_read": (_I32, [_I32, _P, _P, _P]),
}

_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises NSLibraryMissing if it was never built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise NSLibraryMissing(
                    f"{LIB_PATH} not found: build it with `python -m newton_schulz_quintic_amd.build`")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGS.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
        return _lib


def _check(status: int) -> None:
    if status != 0:
        raise NSError(status, lib().ns_last_error().decode())


def _shapes(shapes):
    arr = (ns_shape * max(1, len(shapes)))()
    for i, s in enumerate(shapes):
        s = tuple(int(d) for d in s)
        if len(s) > NS_MAX_DIMS:
            raise ValueError(f"shape {s} has more than {NS_MAX_DIMS} dims")
        arr[i].ndim = len(s)
        for d, v in enumerate(s):
            arr[i].dims[d] = v
    return arr


def _arr(ctype, values):
    values = list(values)
    return (ctype * max(1, len(values)))(*values)


def _addr(x) -> int:
    return ctypes.addressof(x)


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _new_workspace(nbytes: int, device, stream):
    """A torch uint8 workspace for a call enqueued on ``stream``.

    torch's caching allocator ties a block to the stream that allocated it
    (the current stream). When the library's kernels run on another stream,
    the block is also recorded on that stream, so that dropping the returned
    workspace cannot hand its memory to new work before those kernels end.
    """
    import torch
    ws = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    if stream is not None:
        if isinstance(stream, torch.cuda.Stream):
            s = stream
        else:
            s = torch.cuda.ExternalStream(int(stream), device=ws.device)
        if s.cuda_stream != torch.cuda.current_stream(ws.device).cuda_stream:
            ws.record_stream(s)
    return ws


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def ns_last_error() -> str:
    return lib().ns_last_error().decode()


def ns_version() -> str:
    return lib().ns_version().decode()


def ns_plan(shapes, steps: int = 5, num_homes: int = 1, split_rows=None) -> dict:
    """Costs and LPT homes; see ns.h. Returns dict(cost, home, load, order)."""
    n = len(shapes)
    sh = _shapes(shapes)
    split = None
    if split_rows is not None:
        flat = [int(r) for row in split_rows for r in row]
        if len(flat) != n * num_homes:
            raise ValueError("split_rows must be n x num_homes")
        split = _arr(_I64, flat)
    cost, home, load, order = (_arr(_U64, [0] * n), _arr(_I32, [0] * n), _arr(_U64, [0] * num_homes),
                               _arr(_I32, [0] * n))
    _check(lib().ns_plan(n, _addr(sh), steps, num_homes, None if split is None else _addr(split),
                         _addr(cost), _addr(home), _addr(load), _addr(order)))
    return {"cost": list(cost)[:n], "home": list(home)[:n], "load": list(load)[:num_homes],
            "order": [i for i in list(order)[:n] if i >= 0]}


class RoutePlan:
    """Owns an ns_route_plan handle (destroyed with the object)."""

    def __init__(self, handle: int, n: int, num_shards: int, elem_bytes: int):
        self.handle = handle
        self.n, self.num_shards, self.elem_bytes = n, num_shards, elem_bytes
        self.device_table = None

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.ns_route_plan_destroy(self.handle)
            self.handle = None


def ns_route_plan_create(shapes, num_shards: int, split_rows, home, elem_bytes: int) -> RoutePlan:
    n = len(shapes)
    sh = _shapes(shapes)
    flat = [int(r) for row in split_rows for r in row]
    if len(flat) != n * num_shards:
        raise ValueError("split_rows must be n x num_shards")
    out = _P()
    split, homes = _arr(_I64, flat), _arr(_I32, home)     # held alive across the call
    _check(lib().ns_route_plan_create(n, _addr(sh), num_shards, _addr(split), _addr(homes),
                                      elem_bytes, ctypes.byref(out)))
    return RoutePlan(out.value, n, num_shards, elem_bytes)


def ns_route_plan_create_axis(shapes, num_shards: int, split_sizes, shard_dim, home,
                              elem_bytes: int) -> RoutePlan:
    """Route plan with tensor i split along shard_dim[i] (see ns.h)."""
    n = len(shapes)
    sh = _shapes(shapes)
    flat = [int(r) for row in split_sizes for r in row]
    if len(flat) != n * num_shards or len(shard_dim) != n:
        raise ValueError("split_sizes must be n x num_shards and shard_dim n long")
    out = _P()
    split, dims, homes = _arr(_I64, flat), _arr(_I32, shard_dim), _arr(_I32, home)
    _check(lib().ns_route_plan_create_axis(n, _addr(sh), num_shards, _addr(split), _addr(dims), _addr(homes),
                                           elem_bytes, ctypes.byref(out)))
    return RoutePlan(out.value, n, num_shards, elem_bytes)


def ns_route_plan_query(plan: RoutePlan) -> dict:
    S, n = plan.num_shards, plan.n
    se, he = _arr(_I64, [0] * S), _arr(_I64, [0] * S)
    ho, so = _arr(_I64, [0] * n), _arr(_I64, [0] * (n * S))
    tb, fp = _SZ(0), _U64(0)
    _check(lib().ns_route_plan_query(plan.handle, _addr(se), _addr(he), _addr(ho), _addr(so),
                                     ctypes.addressof(tb), ctypes.addressof(fp)))
    so_l = list(so)[:n * S]
    return {"shard_elems": list(se)[:S], "home_elems": list(he)[:S], "home_offset": list(ho)[:n],
            "shard_offset": [so_l[i * S:(i + 1) * S] for i in range(n)],
            "device_table_bytes": tb.value, "fingerprint": fp.value}


def ns_route_plan_upload(plan: RoutePlan, device_table=None, stream=None):
    """Upload the plan's table. Allocates a torch uint8 device tensor if none is given."""
    if device_table is None:
        nbytes = ns_route_plan_query(plan)["device_table_bytes"]
        device_table = _new_workspace(nbytes, "cuda", stream)
    _check(lib().ns_route_plan_upload(plan.handle, device_table.data_ptr(), _stream(stream)))
    plan.device_table = device_table     # keep the memory alive with the plan
    return device_table


def ns_route_plan_destroy(plan: RoutePlan) -> None:
    if plan.handle:
        lib().ns_route_plan_destroy(plan.handle)
        plan.handle = None


def _ptr_array(bufs, S):
    if len(bufs) != S:
        raise ValueError(f"expected {S} buffers")
    return _arr(_P, [_ptr(b) for b in bufs])


def ns_pack_shards(plan: RoutePlan, shard_bufs, home_bufs, stream=None) -> None:
    src, dst = _ptr_array(shard_bufs, plan.num_shards), _ptr_array(home_bufs, plan.num_shards)
    _check(lib().ns_pack_shards(plan.handle, _addr(src), _addr(dst), _stream(stream)))


def ns_unpack_shards(plan: RoutePlan, home_bufs, shard_bufs, stream=None) -> None:
    src, dst = _ptr_array(home_bufs, plan.num_shards), _ptr_array(shard_bufs, plan.num_shards)
    _check(lib().ns_unpack_shards(plan.handle, _addr(src), _addr(dst), _stream(stream)))


def ns_workspace_bytes(shapes, dtype: int) -> tuple[int, int]:
    sh = _shapes(shapes)
    b, mb = _SZ(0), _SZ(0)
    _check(lib().ns_workspace_bytes(len(shapes), _addr(sh), dtype, ctypes.addressof(b),
                                    ctypes.addressof(mb)))
    return b.value, mb.value


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return NS_BF16
    if t.dtype == torch.float32:
        return NS_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def ns_orthogonalize_batched(inputs, outputs, steps: int = 5, coeffs=(3.4445, -4.7750, 2.0315),
                             eps: float = 1e-7, order=None, workspace=None, stream=None):
    """Newton-Schulz on every tensor of ``inputs`` into ``outputs`` (see ns.h).

    Tensors: contiguous, same dtype (bf16 or f32), on the current GPU. The
    workspace (uint8 device tensor) is allocated with torch if not given.
    Returns the workspace so callers can reuse it.
    """
    n = len(inputs)
    if len(outputs) != n:
        raise ValueError("inputs and outputs differ in length")
    if n == 0:
        return workspace
    dtype = _dtype_code(inputs[0])
    for x, y in zip(inputs, outputs):
        if _dtype_code(x) != dtype or _dtype_code(y) != dtype:
            raise TypeError("all tensors must share one dtype")
        if not (x.is_contiguous() and y.is_contiguous()) or x.shape != y.shape:
            raise ValueError("tensors must be contiguous and outputs shaped like inputs")
    shapes = [tuple(x.shape) for x in inputs]
    if workspace is None:
        need, _ = ns_workspace_bytes(shapes, dtype)
        workspace = _new_workspace(need, inputs[0].device, stream)
    a, b, c = coeffs
    sh = _shapes(shapes)
    ins = _arr(_P, [x.data_ptr() for x in inputs])
    outs = _arr(_P, [y.data_ptr() for y in outputs])
    ord_arr = None if order is None else _arr(_I32, order)   # held alive across the call
    _check(lib().ns_orthogonalize_batched(n, _addr(sh), _addr(ins), _addr(outs), dtype, steps,
                                          float(a), float(b), float(c), float(eps),
                                          None if ord_arr is None else _addr(ord_arr),
                                          workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return workspace


def ns_noalloc_init() -> None:
    """Set up the no-allocation entry point on the current device (see ns.h)."""
    _check(lib().ns_noalloc_init())


def ns_orthogonalize_batched_noalloc(inputs, outputs, steps: int = 5, coeffs=(3.4445, -4.7750, 2.0315),
                                     eps: float = 1e-7, order=None, stream=None) -> None:
    """ns_orthogonalize_batched on the library's own scratch array: no workspace,
    nothing allocated (see ns.h). Tensors: contiguous, one dtype (bf16 or f32)."""
    n = len(inputs)
    if len(outputs) != n:
        raise ValueError("inputs and outputs differ in length")
    if n == 0:
        return
    dtype = _dtype_code(inputs[0])
    for x, y in zip(inputs, outputs):
        if _dtype_code(x) != dtype or _dtype_code(y) != dtype:
            raise TypeError("all tensors must share one dtype")
        if not (x.is_contiguous() and y.is_contiguous()) or x.shape != y.shape:
            raise ValueError("tensors must be contiguous and outputs shaped like inputs")
    a, b, c = coeffs
    sh = _shapes([tuple(x.shape) for x in inputs])
    ins = _arr(_P, [x.data_ptr() for x in inputs])
    outs = _arr(_P, [y.data_ptr() for y in outputs])
    ord_arr = None if order is None else _arr(_I32, order)
    _check(lib().ns_orthogonalize_batched_noalloc(n, _addr(sh), _addr(ins), _addr(outs), dtype, steps, float(a),
                                                  float(b), float(c), float(eps),
                                                  None if ord_arr is None else _addr(ord_arr), _stream(stream)))


def _row_stride(t) -> int:
    """Row stride (elements) of a view whose rows (dims 1..) are contiguous."""
    if t.dim() < 2:
        raise ValueError("views need at least 2 dims")
    inner = 1
    for d in range(t.dim() - 1, 0, -1):
        if t.size(d) > 1 and t.stride(d) != inner:
            raise ValueError("each row of a view (dims 1..) must be contiguous")
        inner *= t.size(d)
    return t.stride(0) if t.size(0) > 1 else inner


def ns_orthogonalize_strided(inputs, outputs, steps: int = 5, coeffs=(3.4445, -4.7750, 2.0315),
                             eps: float = 1e-7, order=None, workspace=None, stream=None):
    """ns_orthogonalize_batched on torch views with contiguous rows and any row
    stride (e.g. column blocks of a fused weight); outputs may be views too."""
    n = len(inputs)
    if len(outputs) != n:
        raise ValueError("inputs and outputs differ in length")
    if n == 0:
        return workspace
    dtype = _dtype_code(inputs[0])
    for x, y in zip(inputs, outputs):
        if _dtype_code(x) != dtype or _dtype_code(y) != dtype or x.shape != y.shape:
            raise ValueError("tensors must share one dtype and outputs be shaped like inputs")
    shapes = [tuple(x.shape) for x in inputs]
    if workspace is None:
        need, _ = ns_workspace_bytes(shapes, dtype)
        workspace = _new_workspace(need, inputs[0].device, stream)
    a, b, c = coeffs
    sh = _shapes(shapes)
    ins = _arr(_P, [x.data_ptr() for x in inputs])
    outs = _arr(_P, [y.data_ptr() for y in outputs])
    lds_in = _arr(_I64, [_row_stride(x) for x in inputs])
    lds_out = _arr(_I64, [_row_stride(y) for y in outputs])
    ord_arr = None if order is None else _arr(_I32, order)
    _check(lib().ns_orthogonalize_strided(n, _addr(sh), _addr(ins), _addr(lds_in), _addr(outs), _addr(lds_out),
                                          dtype, steps, float(a), float(b), float(c), float(eps),
                                          None if ord_arr is None else _addr(ord_arr), workspace.data_ptr(),
                                          workspace.numel(), _stream(stream)))
    return workspace


def ns_routed_workspace_bytes(plan: RoutePlan, dtype: int) -> tuple[int, int]:
    b, mb = _SZ(0), _SZ(0)
    _check(lib().ns_routed_workspace_bytes(plan.handle, dtype, ctypes.addressof(b), ctypes.addressof(mb)))
    return b.value, mb.value


def ns_orthogonalize_routed(plan: RoutePlan, shard_in, shard_out, dtype: int, steps: int = 5,
                            coeffs=(3.4445, -4.7750, 2.0315), eps: float = 1e-7, order=None,
                            workspace=None, stream=None):
    """Newton-Schulz on every tensor of ``plan``, read from and written to its row
    pieces in the shard buffers (see ns.h). ``shard_in`` / ``shard_out``: one
    device tensor (or None for an empty shard) per shard, holding elements of
    ``dtype``'s size. The workspace is allocated with torch if not given and is
    returned."""
    if dtype not in (NS_BF16, NS_F32):
        raise TypeError(f"unsupported dtype code {dtype}")
    src, dst = _ptr_array(shard_in, plan.num_shards), _ptr_array(shard_out, plan.num_shards)
    if workspace is None:
        need, _ = ns_routed_workspace_bytes(plan, dtype)
        dev = next((t.device for t in list(shard_in) + list(shard_out) if t is not None), "cuda")
        workspace = _new_workspace(need, dev, stream)
    a, b, c = coeffs
    ord_arr = None if order is None else _arr(_I32, order)
    _check(lib().ns_orthogonalize_routed(plan.handle, _addr(src), _addr(dst), dtype, steps, float(a),
                                         float(b), float(c), float(eps),
                                         None if ord_arr is None else _addr(ord_arr),
                                         workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return workspace


def ns_gram_workspace_bytes(shapes, dtype: int) -> tuple[int, int]:
    sh = _shapes(shapes)
    b, mb = _SZ(0), _SZ(0)
    _check(lib().ns_gram_workspace_bytes(len(shapes), _addr(sh), dtype, ctypes.addressof(b), ctypes.addressof(mb)))
    return b.value, mb.value


def ns_orthogonalize_gram(inputs, outputs, steps: int = 5, coeffs=(3.4445, -4.7750, 2.0315), eps: float = 1e-7,
                          ridge: float = 0.0, order=None, workspace=None, stream=None):
    """Gram-space Newton-Schulz in fp32 on every tensor of ``inputs`` (see ns.h)."""
    n = len(inputs)
    if len(outputs) != n:
        raise ValueError("inputs and outputs differ in length")
    if n == 0:
        return workspace
    dtype = _dtype_code(inputs[0])
    for x, y in zip(inputs, outputs):
        if _dtype_code(x) != dtype or _dtype_code(y) != dtype:
            raise TypeError("all tensors must share one dtype")
        if not (x.is_contiguous() and y.is_contiguous()) or x.shape != y.shape:
            raise ValueError("tensors must be contiguous and outputs shaped like inputs")
    shapes = [tuple(x.shape) for x in inputs]
    if workspace is None:
        need, _ = ns_gram_workspace_bytes(shapes, dtype)
        workspace = _new_workspace(need, inputs[0].device, stream)
    a, b, c = coeffs
    sh = _shapes(shapes)
    ins = _arr(_P, [x.data_ptr() for x in inputs])
    outs = _arr(_P, [y.data_ptr() for y in outputs])
    ord_arr = None if order is None else _arr(_I32, order)
    _check(lib().ns_orthogonalize_gram(n, _addr(sh), _addr(ins), _addr(outs), dtype, steps, float(a), float(b),
                                       float(c), float(eps), float(ridge),
                                       None if ord_arr is None else _addr(ord_arr), workspace.data_ptr(),
                                       workspace.numel(), _stream(stream)))
    return workspace


def ns_wave_plan(shapes, slots: int, ready_order=None) -> tuple[list[int], int]:
    """(wave_of, num_waves): tensors in gradient-ready order, ``slots`` per wave (see ns.h)."""
    n = len(shapes)
    sh = _shapes(shapes)
    order = None if ready_order is None else _arr(_I32, ready_order)
    wave, num = _arr(_I32, [0] * n), _I32(0)
    _check(lib().ns_wave_plan(n, _addr(sh), None if order is None else _addr(order), slots, _addr(wave),
                              ctypes.addressof(num)))
    return list(wave)[:n], num.value


def ns_orthogonalize_waves(inputs, outputs, wave_of, num_waves: int, ready_events=None, steps: int = 5,
                           coeffs=(3.4445, -4.7750, 2.0315), eps: float = 1e-7, workspace=None, stream=None):
    """ns_orthogonalize_batched wave by wave; wave w waits for ready_events[w]
    (torch.cuda.Event or None). Returns the workspace."""
    n = len(inputs)
    if len(outputs) != n or len(wave_of) != n:
        raise ValueError("inputs, outputs and wave_of differ in length")
    if n == 0:
        return workspace
    dtype = _dtype_code(inputs[0])
    for x, y in zip(inputs, outputs):
        if _dtype_code(x) != dtype or _dtype_code(y) != dtype:
            raise TypeError("all tensors must share one dtype")
        if not (x.is_contiguous() and y.is_contiguous()) or x.shape != y.shape:
            raise ValueError("tensors must be contiguous and outputs shaped like inputs")
    shapes = [tuple(x.shape) for x in inputs]
    if workspace is None:
        need, _ = ns_workspace_bytes(shapes, dtype)
        workspace = _new_workspace(need, inputs[0].device, stream)
    evs = None
    if ready_events is not None:
        if len(ready_events) != num_waves:
            raise ValueError("one event (or None) per wave")
        evs = _arr(_P, [None if e is None else e.cuda_event for e in ready_events])
    a, b, c = coeffs
    sh = _shapes(shapes)
    ins = _arr(_P, [x.data_ptr() for x in inputs])
    outs = _arr(_P, [y.data_ptr() for y in outputs])
    waves = _arr(_I32, wave_of)
    _check(lib().ns_orthogonalize_waves(n, _addr(sh), _addr(ins), _addr(outs), dtype, steps, float(a),
                                        float(b), float(c), float(eps), _addr(waves), num_waves,
                                        None if evs is None else _addr(evs), workspace.data_ptr(),
                                        workspace.numel(), _stream(stream)))
    return workspace


def ns_timing_enable(kinds) -> None:
    """Enable HIP-event timing for the given kinds: True = all, False = none,
    or an iterable of kind numbers (see ns_timing_read)."""
    if kinds is True:
        mask = -1
    elif kinds is False or kinds is None:
        mask = 0
    else:
        mask = 0
        for k in kinds:
            mask |= 1 << int(k)
    _check(lib().ns_timing_enable(mask))


def ns_timing_read(kind: int) -> tuple[float, int, float]:
    """(total_ms, launches, work) for kind 0 = B X product kernel, 1 = pack/unpack,
    2 = norm, 3 = final B X launch, 4 = A = X X^T kernel, 5 = A A kernel,
    6 = small-class kernel."""
    ms, cnt, work = ctypes.c_double(0), _I64(0), ctypes.c_double(0)
    _check(lib().ns_timing_read(kind, ctypes.addressof(ms), ctypes.addressof(cnt),
                                ctypes.addressof(work)))
    return ms.value, cnt.value, work.value
