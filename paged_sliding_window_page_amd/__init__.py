"""Python binding of libpsw.so, the gfx950 paged sliding-window attention library.

Argument marshalling only: every function here checks nothing of its own beyond
what ctypes needs, passes device pointers and sizes to the C ABI declared in
``include/psw.h`` and raises ``PswError`` with the library's message on a
non-zero status.  All computation happens in the library's HIP kernels; there
is no fallback.  Importing this package raises when ``libpsw.so`` has not been
built (``python -m paged_sliding_window_page_amd.build``).

Names follow the C ABI: ``paged_prefill_window_hd256``, ``paged_prefill_hd512``,
``qkv_norm_rope_paged_prefill_hd256``, ``k_v_norm_rope_paged_prefill_hd512``,
``q_norm_rope_prefill_hd512``,
``rope_tables`` (``psw_rope_tables``), and the ``Plan`` object wrapping
``psw_plan_*``.  Tensors are torch tensors on the current HIP device; the stream
is torch's current stream unless one is passed.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpsw.so")

PSW_OK = 0
STATUS = {
    0: "PSW_OK", -1: "PSW_E_NULL", -2: "PSW_E_SHAPE", -3: "PSW_E_RANGE", -4: "PSW_E_OVERFLOW",
    -5: "PSW_E_HEADS", -6: "PSW_E_SCALE", -7: "PSW_E_PLAN", -8: "PSW_E_HIP",
    -9: "PSW_E_UNSUPPORTED",
}


class PswError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code
        self.status = STATUS.get(code, str(code))


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python -m paged_sliding_window_page_amd.build`")

# The library takes torch's device pointers and streams, so it must run on the
# same HIP runtime instance as torch.  torch ships its own libamdhip64 with the
# same soname as the system one; importing torch first makes the dynamic loader
# resolve libpsw.so's dependency to that already-loaded copy.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

c_i64 = ctypes.c_int64
c_i32 = ctypes.c_int32
c_vp = ctypes.c_void_p
c_i32p = ctypes.POINTER(ctypes.c_int32)


class PoolDesc(ctypes.Structure):
    _fields_ = [("base", c_vp), ("numel", c_i64), ("num_layers", c_i64), ("num_pages", c_i64),
                ("page_size", c_i64), ("num_kv_heads", c_i64), ("head_dim", c_i64)]


class PlanDesc(ctypes.Structure):
    _fields_ = [("batch", c_i64), ("qo_indptr", c_i32p), ("kv_page_indptr", c_i32p),
                ("kv_page_indices", c_i32p), ("kv_last_page_len", c_i32p),
                ("num_qo_heads", c_i64), ("num_kv_heads", c_i64), ("head_dim", c_i64),
                ("page_size", c_i64), ("num_pages", c_i64), ("tile_q_override", c_i64),
                ("kv_len", c_i32p)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("batch", c_i64), ("total_qo", c_i64), ("total_pages", c_i64),
                ("max_qo_len", c_i64), ("max_kv_len", c_i64), ("max_page_id", c_i64),
                ("max_last_page_len", c_i64), ("num_qo_heads", c_i64), ("num_kv_heads", c_i64),
                ("head_dim", c_i64), ("page_size", c_i64), ("num_pages", c_i64),
                ("group", c_i64), ("tile_q", c_i64), ("generation", ctypes.c_uint64),
                ("digest", ctypes.c_uint64)]


class KvServerDesc(ctypes.Structure):
    _fields_ = [("local_pages", c_i64), ("global_pages", c_i64), ("local_page_size", c_i64),
                ("global_page_size", c_i64), ("window_left", c_i64), ("rope_positions", c_i64),
                ("local_ring_pages", c_i64)]


class KvRequestState(ctypes.Structure):
    _fields_ = [("frontier", c_i64), ("local_held", c_i64), ("global_held", c_i64),
                ("pending", c_i32), ("pending_tokens", c_i64), ("local_reserved", c_i64),
                ("global_reserved", c_i64)]


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_last_error = _sig("psw_last_error", ctypes.c_char_p)
_version = _sig("psw_version", ctypes.c_char_p)
_mfma_clock = _sig("psw_measure_mfma_clock", ctypes.c_int, c_vp, ctypes.POINTER(ctypes.c_double))
_check_pool = _sig("psw_check_pool", ctypes.c_int, ctypes.POINTER(PoolDesc))
_plan_create = _sig("psw_plan_create", ctypes.c_int, ctypes.POINTER(PlanDesc), c_vp,
                    ctypes.POINTER(c_vp))
_plan_update = _sig("psw_plan_update", ctypes.c_int, c_vp, ctypes.POINTER(PlanDesc))
_plan_destroy = _sig("psw_plan_destroy", None, c_vp)
_plan_info = _sig("psw_plan_get_info", ctypes.c_int, c_vp, ctypes.POINTER(PlanInfo))
_tile_q = _sig("psw_prefill_tile_q", ctypes.c_int, c_i64, c_i64, c_i32p)
_prefill256 = _sig("paged_prefill_window_hd256", ctypes.c_int, c_vp, ctypes.POINTER(PoolDesc),
                   c_i64, c_vp, ctypes.c_float, c_i64, c_vp, c_i32, c_vp)
_prefill512 = _sig("paged_prefill_hd512", ctypes.c_int, c_vp, ctypes.POINTER(PoolDesc), c_i64,
                   c_vp, ctypes.c_float, c_vp, c_i32, c_vp)
_decode256 = _sig("paged_decode_window_hd256", ctypes.c_int, c_vp, ctypes.POINTER(PoolDesc),
                  c_i64, c_vp, ctypes.c_float, c_i64, c_vp, c_i32, c_vp)
_decode512 = _sig("paged_decode_hd512", ctypes.c_int, c_vp, ctypes.POINTER(PoolDesc), c_i64,
                  c_vp, ctypes.c_float, c_vp, c_i32, c_vp)
_decode512_noalloc = _sig("paged_decode_hd512_noalloc", ctypes.c_int, c_vp,
                          ctypes.POINTER(PoolDesc), c_i64, c_vp, ctypes.c_float, c_vp, c_i32,
                          c_vp)
_decode_mode = _sig("psw_plan_set_decode_mode", ctypes.c_int, c_vp, c_i32)
_decode_form = _sig("psw_plan_decode_form", ctypes.c_int, c_vp, c_i64, c_i32p,
                    ctypes.POINTER(c_i64))
_prep256 = _sig("qkv_norm_rope_paged_prefill_hd256", ctypes.c_int, c_vp, ctypes.POINTER(PoolDesc),
                c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64,
                ctypes.c_float, c_vp, c_vp)
_prep512 = _sig("k_v_norm_rope_paged_prefill_hd512", ctypes.c_int, c_vp, ctypes.POINTER(PoolDesc),
                c_i64, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, ctypes.c_float, c_vp)
_prepq512 = _sig("q_norm_rope_prefill_hd512", ctypes.c_int, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64,
                 c_i64, c_i64, ctypes.c_float, c_vp, c_vp)
_kv_create = _sig("psw_kv_server_create", ctypes.c_int, ctypes.POINTER(KvServerDesc),
                  ctypes.POINTER(c_vp))
_kv_destroy = _sig("psw_kv_server_destroy", ctypes.c_int, c_vp)
_kv_free = _sig("psw_kv_server_free_pages", ctypes.c_int, c_vp, ctypes.POINTER(c_i64),
                ctypes.POINTER(c_i64))
_kv_req_create = _sig("psw_kv_request_create", ctypes.c_int, c_vp, ctypes.POINTER(c_vp))
_kv_req_release = _sig("psw_kv_request_release", ctypes.c_int, c_vp, c_vp)
_kv_req_info = _sig("psw_kv_request_info", ctypes.c_int, c_vp, ctypes.POINTER(KvRequestState))
_kv_admit = _sig("psw_kv_admit", ctypes.c_int, c_vp, c_vp, c_i64)
_kv_commit = _sig("psw_kv_commit", ctypes.c_int, c_vp, c_vp)
_kv_abort = _sig("psw_kv_abort", ctypes.c_int, c_vp, c_vp)
_kv_tables = _sig("psw_kv_step_tables", ctypes.c_int, c_vp, ctypes.POINTER(c_vp), c_i64, c_i32,
                  c_i32p, c_i32p, c_i32p, c_i64, c_i32p, c_i32p)
_rope = _sig("psw_rope_tables", ctypes.c_int, c_vp, c_vp, c_i64, c_i64, ctypes.c_double, c_vp)
_dev_err = _sig("psw_plan_device_errors", ctypes.c_int, c_vp)

# every symbol include/psw.h declares
EXPORTS = ["psw_last_error", "psw_version", "psw_check_pool", "psw_plan_create",
           "psw_plan_update", "psw_plan_destroy", "psw_plan_get_info", "psw_prefill_tile_q",
           "paged_prefill_window_hd256", "paged_prefill_hd512", "paged_decode_window_hd256",
           "paged_decode_hd512", "paged_decode_hd512_noalloc", "psw_plan_set_decode_mode",
           "psw_plan_decode_form",
           "qkv_norm_rope_paged_prefill_hd256", "k_v_norm_rope_paged_prefill_hd512",
           "q_norm_rope_prefill_hd512", "psw_rope_tables", "psw_plan_device_errors",
           "psw_kv_server_create", "psw_kv_server_destroy", "psw_kv_server_free_pages",
           "psw_kv_request_create", "psw_kv_request_release", "psw_kv_request_info",
           "psw_kv_admit", "psw_kv_commit", "psw_kv_abort", "psw_kv_step_tables",
           "psw_measure_mfma_clock"]


def _check(rc: int):
    if rc != PSW_OK:
        raise PswError(rc, _last_error().decode(errors="replace"))


def measure_mfma_clock(stream=None) -> float:
    """Shader clock (MHz) with every CU issuing bf16 MFMAs (diagnostic)."""
    mhz = ctypes.c_double()
    _check(_mfma_clock(_stream_handle(stream), ctypes.byref(mhz)))
    return mhz.value


def version() -> str:
    return _version().decode()


def last_error() -> str:
    return _last_error().decode(errors="replace")


def _ptr(t):
    """Device/host address of a tensor (or None / int passthrough)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def pool_desc(pool, *, num_layers, num_pages, page_size, num_kv_heads, head_dim,
              numel=None) -> PoolDesc:
    """Descriptor of a flat bf16 pool tensor (or a raw address with ``numel``)."""
    if numel is None:
        numel = pool.numel()
    return PoolDesc(_ptr(pool), int(numel), int(num_layers), int(num_pages), int(page_size),
                    int(num_kv_heads), int(head_dim))


def check_pool(desc: PoolDesc) -> None:
    _check(_check_pool(ctypes.byref(desc)))


def prefill_tile_q(group: int, head_dim: int) -> int:
    out = ctypes.c_int32(0)
    _check(_tile_q(int(group), int(head_dim), ctypes.byref(out)))
    return out.value


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


class Plan:
    """psw_plan: validated page-table metadata bound to one HIP stream."""

    def __init__(self, qo_indptr, kv_page_indptr, kv_page_indices, kv_last_page_len, *,
                 num_qo_heads, num_kv_heads, head_dim, page_size, num_pages,
                 tile_q_override=0, stream=None, batch=None, kv_len=None):
        self._h = c_vp()
        self.stream = _stream_handle(stream) if stream != "none" else None
        desc, keep = self._desc(qo_indptr, kv_page_indptr, kv_page_indices, kv_last_page_len,
                                num_qo_heads, num_kv_heads, head_dim, page_size, num_pages,
                                tile_q_override, batch, kv_len)
        _check(_plan_create(ctypes.byref(desc), self.stream, ctypes.byref(self._h)))

    @staticmethod
    def _desc(qo_indptr, kv_page_indptr, kv_page_indices, kv_last_page_len, num_qo_heads,
              num_kv_heads, head_dim, page_size, num_pages, tile_q_override, batch, kv_len=None):
        arrs = [_i32(qo_indptr), _i32(kv_page_indptr), _i32(kv_page_indices),
                _i32(kv_last_page_len)]
        if batch is None:
            batch = len(arrs[0]) - 1
        ptrs = [a.ctypes.data_as(c_i32p) if a.size else ctypes.cast(None, c_i32p) for a in arrs]
        kvl = None if kv_len is None else _i32(kv_len)
        if kvl is not None:
            arrs.append(kvl)
        desc = PlanDesc(int(batch), *ptrs, int(num_qo_heads), int(num_kv_heads), int(head_dim),
                        int(page_size), int(num_pages), int(tile_q_override),
                        kvl.ctypes.data_as(c_i32p) if kvl is not None else ctypes.cast(None, c_i32p))
        return desc, arrs

    def update(self, qo_indptr, kv_page_indptr, kv_page_indices, kv_last_page_len, *,
               num_qo_heads, num_kv_heads, head_dim, page_size, num_pages, tile_q_override=0,
               batch=None, kv_len=None):
        desc, keep = self._desc(qo_indptr, kv_page_indptr, kv_page_indices, kv_last_page_len,
                                num_qo_heads, num_kv_heads, head_dim, page_size, num_pages,
                                tile_q_override, batch, kv_len)
        _check(_plan_update(self._h, ctypes.byref(desc)))

    def info(self) -> dict:
        out = PlanInfo()
        _check(_plan_info(self._h, ctypes.byref(out)))
        return {f: getattr(out, f) for f, _ in PlanInfo._fields_}

    def set_decode_mode(self, mode: int) -> None:
        _check(_decode_mode(self.handle, int(mode)))

    def decode_form(self, window_left: int = -1):
        """(direct, work_groups) of the next decode call with this window."""
        d, wg = c_i32(), c_i64()
        _check(_decode_form(self.handle, int(window_left), ctypes.byref(d), ctypes.byref(wg)))
        return bool(d.value), wg.value

    def device_errors(self) -> None:
        _check(_dev_err(self._h))

    @property
    def handle(self):
        return self._h

    def close(self):
        if self._h:
            _plan_destroy(self._h)
            self._h = c_vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def paged_prefill_window_hd256(plan: Plan, pool: PoolDesc, layer: int, q, sm_scale: float,
                               window_left: int, o, stream=None) -> None:
    """o <- windowed paged attention of q over ``layer`` of the pool (o fp32 or bf16)."""
    import torch
    o_dtype = 1 if o.dtype == torch.bfloat16 else 0
    _check(_prefill256(plan.handle, ctypes.byref(pool), int(layer), _ptr(q), float(sm_scale),
                       int(window_left), _ptr(o), o_dtype,
                       plan.stream if stream is None else _stream_handle(stream)))


def paged_prefill_hd512(plan: Plan, pool: PoolDesc, layer: int, q, sm_scale: float, o,
                        stream=None) -> None:
    """o <- full causal paged attention at head_dim 512."""
    import torch
    o_dtype = 1 if o.dtype == torch.bfloat16 else 0
    _check(_prefill512(plan.handle, ctypes.byref(pool), int(layer), _ptr(q), float(sm_scale),
                       _ptr(o), o_dtype,
                       plan.stream if stream is None else _stream_handle(stream)))


DECODE_AUTO, DECODE_SPLIT, DECODE_DIRECT = 0, 1, 2


def paged_decode_window_hd256(plan: "Plan", pool: PoolDesc, layer: int, q, sm_scale: float,
                              window_left: int, o, stream=None) -> None:
    import torch
    o_dtype = 1 if o.dtype == torch.bfloat16 else 0
    _check(_decode256(plan.handle, ctypes.byref(pool), int(layer), _ptr(q), float(sm_scale),
                      int(window_left), _ptr(o), o_dtype,
                      plan.stream if stream is None else _stream_handle(stream)))


def paged_decode_hd512(plan: "Plan", pool: PoolDesc, layer: int, q, sm_scale: float, o,
                       stream=None) -> None:
    import torch
    o_dtype = 1 if o.dtype == torch.bfloat16 else 0
    _check(_decode512(plan.handle, ctypes.byref(pool), int(layer), _ptr(q), float(sm_scale),
                      _ptr(o), o_dtype,
                      plan.stream if stream is None else _stream_handle(stream)))


def paged_decode_hd512_noalloc(plan: "Plan", pool: PoolDesc, layer: int, q, sm_scale: float, o,
                               stream=None) -> None:
    """paged_decode_hd512 with its workspace in the library's static device
    array (no device allocation)."""
    import torch
    o_dtype = 1 if o.dtype == torch.bfloat16 else 0
    _check(_decode512_noalloc(plan.handle, ctypes.byref(pool), int(layer), _ptr(q),
                              float(sm_scale), _ptr(o), o_dtype,
                              plan.stream if stream is None else _stream_handle(stream)))


def qkv_norm_rope_paged_prefill_hd256(plan: Plan, pool: PoolDesc, layer: int, q_in, k_in, v_in,
                                      q_norm_w, k_norm_w, rope_cos, rope_sin, eps: float, q_out,
                                      rope_positions=None, stream=None) -> None:
    if rope_positions is None:
        rope_positions = rope_cos.shape[0]
    _check(_prep256(plan.handle, ctypes.byref(pool), int(layer), _ptr(q_in), _ptr(k_in),
                    _ptr(v_in), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(rope_cos), _ptr(rope_sin),
                    int(rope_positions), int(rope_cos.numel()), int(rope_sin.numel()),
                    float(eps), _ptr(q_out),
                    plan.stream if stream is None else _stream_handle(stream)))


def k_v_norm_rope_paged_prefill_hd512(plan: Plan, pool: PoolDesc, layer: int, k_in, k_norm_w,
                                      rope_cos, rope_sin, eps: float, rope_positions=None,
                                      stream=None) -> None:
    if rope_positions is None:
        rope_positions = rope_cos.shape[0]
    _check(_prep512(plan.handle, ctypes.byref(pool), int(layer), _ptr(k_in), _ptr(k_norm_w),
                    _ptr(rope_cos), _ptr(rope_sin), int(rope_positions), int(rope_cos.numel()),
                    int(rope_sin.numel()), float(eps),
                    plan.stream if stream is None else _stream_handle(stream)))


def q_norm_rope_prefill_hd512(plan: Plan, q_in, q_norm_w, rope_cos, rope_sin, eps: float, q_out,
                              rope_positions=None, stream=None) -> None:
    if rope_positions is None:
        rope_positions = rope_cos.shape[0]
    _check(_prepq512(plan.handle, _ptr(q_in), _ptr(q_norm_w), _ptr(rope_cos), _ptr(rope_sin),
                     int(rope_positions), int(rope_cos.numel()), int(rope_sin.numel()),
                     float(eps), _ptr(q_out),
                     plan.stream if stream is None else _stream_handle(stream)))


def rope_tables(cos_out, sin_out, positions: int, head_dim: int, theta: float,
                stream=None) -> None:
    """Fill fp32 [positions][head_dim/2] cos/sin tables on the device."""
    _check(_rope(_ptr(cos_out), _ptr(sin_out), int(positions), int(head_dim), float(theta),
                 _stream_handle(stream)))


# ------------------------------------------------- two-family page accounting ----

KV_LOCAL, KV_GLOBAL = 0, 1


class KvServer:
    """Page accounting of the two KV families (``psw_kv_*``); host only."""

    def __init__(self, local_pages: int, global_pages: int, local_page_size: int = 16,
                 global_page_size: int = 16, window_left: int = -1, rope_positions: int = 16384,
                 local_ring_pages: int = 0):
        d = KvServerDesc(int(local_pages), int(global_pages), int(local_page_size),
                         int(global_page_size), int(window_left), int(rope_positions),
                         int(local_ring_pages))
        h = c_vp()
        _check(_kv_create(ctypes.byref(d), ctypes.byref(h)))
        self.handle = h.value
        self.page_size = (int(local_page_size), int(global_page_size))

    def free_pages(self):
        lf, gf = c_i64(), c_i64()
        _check(_kv_free(self.handle, ctypes.byref(lf), ctypes.byref(gf)))
        return lf.value, gf.value

    def request(self) -> "KvRequest":
        h = c_vp()
        _check(_kv_req_create(self.handle, ctypes.byref(h)))
        return KvRequest(self, h.value)

    def admit(self, req: "KvRequest", n_new: int) -> None:
        _check(_kv_admit(self.handle, req.handle, int(n_new)))

    def commit(self, req: "KvRequest") -> None:
        _check(_kv_commit(self.handle, req.handle))

    def abort(self, req: "KvRequest") -> None:
        _check(_kv_abort(self.handle, req.handle))

    def release(self, req: "KvRequest") -> None:
        _check(_kv_req_release(self.handle, req.handle))
        req.handle = None

    def step_tables(self, reqs, family: int):
        """(qo_indptr, kv_page_indptr, kv_page_indices, kv_last_page_len, kv_len)
        of one family for a batch of requests with admitted steps, int32 numpy
        arrays (kv_len: the plan's absolute lengths)."""
        n = len(reqs)
        arr = (c_vp * n)(*[r.handle for r in reqs])
        sts = [r.state() for r in reqs]
        if family == KV_LOCAL:
            cap = sum(st.local_held + st.local_reserved for st in sts)
        else:
            cap = sum(st.global_held + st.global_reserved for st in sts)
        cap = max(int(cap), 1)
        qo = np.zeros(n + 1, np.int32)
        kvp = np.zeros(n + 1, np.int32)
        idx = np.zeros(cap, np.int32)
        last = np.zeros(n, np.int32)
        kvl = np.zeros(n, np.int32)
        p = lambda a: a.ctypes.data_as(c_i32p)
        _check(_kv_tables(self.handle, arr, n, int(family), p(qo), p(kvp), p(idx), cap, p(last),
                          p(kvl)))
        return qo, kvp, idx[:kvp[-1]].copy(), last, kvl

    def close(self) -> None:
        if self.handle is not None:
            _check(_kv_destroy(self.handle))
            self.handle = None


class KvRequest:
    def __init__(self, server: KvServer, handle):
        self.server = server
        self.handle = handle

    def state(self) -> KvRequestState:
        st = KvRequestState()
        _check(_kv_req_info(self.handle, ctypes.byref(st)))
        return st
