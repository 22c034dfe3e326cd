"""Python binding of libdita (partitioned video-DiT attention with selective
attention-state reuse on MI355X).

Argument marshalling only: every step of the computation runs in the native library
(`libdita.so`, built in-tree by `python partial_state_reuse_amd/build.py`).  PyTorch is used
for device memory (the cache buffer, outputs) and for the current HIP stream.  If the
library has not been built, importing this package raises ImportError.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdita.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python partial_state_reuse_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

# ----- constants (include/dita.h) -----
OK = 0
STATUS_NAMES = {0: "OK", 1: "INVALID_ARGUMENT", 2: "SHAPE", 3: "UNSUPPORTED", 4: "POLICY",
                5: "CACHE_MISS", 6: "BUFFER_TOO_SMALL", 7: "NO_POLICY", 8: "DEVICE",
                9: "OFFLOADED"}
F32, BF16, FP8_E4M3 = 0, 1, 2
LAYOUT_BHND, LAYOUT_BNHD = 0, 1
_LAYOUTS = {"bhnd": LAYOUT_BHND, "bnhd": LAYOUT_BNHD}
_DTYPES = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3}
SKIP, FRESH, REUSE = 0, 1, 2
POLICY_EXPLICIT, POLICY_FRAME_THRESHOLD, POLICY_FRESH_BUDGET, POLICY_CENTROID_THRESHOLD = 0, 1, 2, 3
POLICY_PLANNER = 4

EXPORTED = ["dita_version", "dita_last_error", "dita_policy_mask", "dita_partition_offsets",
            "dita_cache_required_bytes", "dita_cache_alloc", "dita_cache_reset",
            "dita_cache_free", "dita_set_block_policy", "dita_get_block_plan",
            "dita_attn_step", "dita_cache_read_slot", "dita_set_profiling", "dita_get_stats",
            "dita_planner_mask", "dita_get_planner_state", "dita_cache_merge_groups",
            "dita_cache_offload_bytes", "dita_cache_offload", "dita_cache_restore",
            "dita_attn_step_static", "dita_cache_compact_bytes", "dita_cache_compact",
            "dita_cache_expand"]


class DitaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))


class Geometry(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("tokens", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("frames", ctypes.c_int32), ("grid_h", ctypes.c_int32),
                ("grid_w", ctypes.c_int32), ("num_partitions", ctypes.c_int32),
                ("partition_offsets", ctypes.POINTER(ctypes.c_int32)),
                ("qkv_dtype", ctypes.c_int32), ("cache_o_dtype", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("layout", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32)]


class BlockPolicy(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("explicit_mask", ctypes.POINTER(ctypes.c_uint8)),
                ("max_fresh_frame_dist", ctypes.c_int32), ("reuse_percent", ctypes.c_int32),
                ("max_fresh_centroid2", ctypes.c_int32), ("tile_sparse", ctypes.c_int32),
                ("anchor", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("anchor_period", ctypes.c_int32), ("max_error", ctypes.c_double)]


class StepStats(ctypes.Structure):
    _fields_ = [("steps_done", ctypes.c_int64), ("last_counts", ctypes.c_int32 * 3),
                ("reserved", ctypes.c_int32),
                ("device_fresh_blocks", ctypes.c_uint64), ("device_reuse_blocks", ctypes.c_uint64),
                ("host_fresh_blocks", ctypes.c_uint64), ("host_reuse_blocks", ctypes.c_uint64),
                ("last_fresh_flops", ctypes.c_double), ("last_cache_read_bytes", ctypes.c_double),
                ("last_cache_write_bytes", ctypes.c_double),
                ("device_v_range_errors", ctypes.c_uint64),
                ("profiled_steps", ctypes.c_uint64), ("step_kernel_ms", ctypes.c_double),
                ("prep_kernel_ms", ctypes.c_double), ("device_ref_recomputes", ctypes.c_uint64),
                ("fixed_ref_steps", ctypes.c_uint64), ("fixed_ref_kernel_ms", ctypes.c_double)]


_P = ctypes.c_void_p
_i32p = ctypes.POINTER(ctypes.c_int32)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_sig = {
    "dita_version": (ctypes.c_char_p, []),
    "dita_last_error": (ctypes.c_char_p, []),
    "dita_policy_mask": (ctypes.c_int, [ctypes.POINTER(Geometry), ctypes.POINTER(BlockPolicy),
                                        _u8p, _u8p]),
    "dita_partition_offsets": (ctypes.c_int, [ctypes.POINTER(Geometry), _i32p]),
    "dita_cache_required_bytes": (ctypes.c_int, [ctypes.POINTER(Geometry), _u8p,
                                                 ctypes.POINTER(ctypes.c_size_t)]),
    "dita_cache_alloc": (ctypes.c_int, [ctypes.POINTER(Geometry), _u8p, _P, ctypes.c_size_t,
                                        ctypes.POINTER(_P)]),
    "dita_cache_reset": (ctypes.c_int, [_P]),
    "dita_cache_free": (ctypes.c_int, [_P]),
    "dita_set_block_policy": (ctypes.c_int, [_P, ctypes.POINTER(BlockPolicy)]),
    "dita_get_block_plan": (ctypes.c_int, [_P, _u8p, _i32p, _i32p, _i32p, _i32p, _i32p]),
    "dita_attn_step": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P]),
    "dita_attn_step_static": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P]),
    "dita_cache_read_slot": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, _P, _P, _P]),
    "dita_set_profiling": (ctypes.c_int, [_P, ctypes.c_int32]),
    "dita_get_stats": (ctypes.c_int, [_P, ctypes.POINTER(StepStats)]),
    "dita_planner_mask": (ctypes.c_int, [ctypes.POINTER(Geometry), ctypes.POINTER(BlockPolicy),
                                         _f64p, _u8p, _u8p]),
    "dita_get_planner_state": (ctypes.c_int, [_P, _f32p, _f64p, _i32p, _i32p]),
    "dita_cache_merge_groups": (ctypes.c_int, [_P, ctypes.c_int32, _u8p, _i32p, _P]),
    "dita_cache_offload_bytes": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_size_t)]),
    "dita_cache_offload": (ctypes.c_int, [_P, _P, ctypes.c_size_t, _P]),
    "dita_cache_restore": (ctypes.c_int, [_P, _P, ctypes.c_size_t, _P, ctypes.c_size_t, _P]),
    "dita_cache_compact_bytes": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_size_t)]),
    "dita_cache_compact": (ctypes.c_int, [_P, _P, ctypes.c_size_t, _P]),
    "dita_cache_expand": (ctypes.c_int, [_P, _P, ctypes.c_size_t, _P]),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def _check(status: int):
    if status != OK:
        raise DitaError(status, _lib.dita_last_error().decode())


def version() -> str:
    return _lib.dita_version().decode()


def _u8(arr):
    a = np.ascontiguousarray(arr, dtype=np.uint8)
    return a, a.ctypes.data_as(_u8p)


def make_geometry(batch, heads, tokens, head_dim, frames, grid_h, grid_w, num_partitions,
                  dtype="bf16", offsets=None, softmax_scale=0.0, cache_dtype=None,
                  layout="bhnd", out_dtype="f32"):
    """A Geometry; `offsets` (P+1 ints) or None for the array_split rule; `cache_dtype`
    (cached O) defaults to `dtype` ("fp8" = e4m3, with bf16 Q/K/V); `layout` of Q, K, V and
    out: "bhnd" ([B, H, N, D]) or "bnhd" ([B, N, H, D]); `out_dtype` "f32" or "bf16" (with
    bf16 Q/K/V)."""
    g = Geometry()
    g.batch, g.heads, g.tokens, g.head_dim = batch, heads, tokens, head_dim
    g.frames, g.grid_h, g.grid_w, g.num_partitions = frames, grid_h, grid_w, num_partitions
    dt = _DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    cd = dt if cache_dtype is None else (_DTYPES[cache_dtype] if isinstance(cache_dtype, str)
                                         else int(cache_dtype))
    g.qkv_dtype = dt
    g.cache_o_dtype = cd
    g.softmax_scale = softmax_scale
    g.layout = _LAYOUTS[layout] if isinstance(layout, str) else int(layout)
    g.out_dtype = _DTYPES[out_dtype] if isinstance(out_dtype, str) else int(out_dtype)
    if offsets is not None:
        arr = (ctypes.c_int32 * len(offsets))(*[int(x) for x in offsets])
        g._offsets_keepalive = arr
        g.partition_offsets = ctypes.cast(arr, _i32p)
    return g


def make_policy(kind=POLICY_FRAME_THRESHOLD, max_fresh_frame_dist=0, reuse_percent=0,
                max_fresh_centroid2=0, tile_sparse=False, anchor=False, explicit_mask=None,
                group_size=1, anchor_period=0, max_error=0.0):
    p = BlockPolicy()
    p.kind = int(kind)
    p.max_fresh_frame_dist = int(max_fresh_frame_dist)
    p.reuse_percent = int(reuse_percent)
    p.max_fresh_centroid2 = int(max_fresh_centroid2)
    p.tile_sparse = int(bool(tile_sparse))
    p.anchor = int(bool(anchor))
    p.group_size = int(group_size)
    p.anchor_period = int(anchor_period)
    p.max_error = float(max_error)
    if explicit_mask is not None:
        arr, ptr = _u8(np.asarray(explicit_mask).ravel())
        p._mask_keepalive = arr
        p.explicit_mask = ptr
    return p


def dita_policy_mask(geom: Geometry, policy: BlockPolicy, valid=None) -> np.ndarray:
    P = geom.num_partitions
    out = np.zeros(P * P, dtype=np.uint8)
    vptr = None
    if valid is not None:
        varr, vptr = _u8(np.asarray(valid).ravel())
    _check(_lib.dita_policy_mask(ctypes.byref(geom), ctypes.byref(policy), vptr,
                                 out.ctypes.data_as(_u8p)))
    return out.reshape(P, P)


def dita_planner_mask(geom: Geometry, policy: BlockPolicy, error, valid=None) -> np.ndarray:
    """The planner's decision from predicted errors E (P x P doubles)."""
    P = geom.num_partitions
    out = np.zeros(P * P, dtype=np.uint8)
    e = np.ascontiguousarray(np.asarray(error, dtype=np.float64).ravel())
    vptr = None
    if valid is not None:
        varr, vptr = _u8(np.asarray(valid).ravel())
    _check(_lib.dita_planner_mask(ctypes.byref(geom), ctypes.byref(policy),
                                  e.ctypes.data_as(_f64p), vptr, out.ctypes.data_as(_u8p)))
    return out.reshape(P, P)


def dita_partition_offsets(geom: Geometry) -> np.ndarray:
    out = np.zeros(geom.num_partitions + 1, dtype=np.int32)
    _check(_lib.dita_partition_offsets(ctypes.byref(geom), out.ctypes.data_as(_i32p)))
    return out


def dita_cache_required_bytes(geom: Geometry, active_mask=None) -> int:
    n = ctypes.c_size_t(0)
    aptr = None
    if active_mask is not None:
        arr, aptr = _u8(np.asarray(active_mask).ravel())
    _check(_lib.dita_cache_required_bytes(ctypes.byref(geom), aptr, ctypes.byref(n)))
    return int(n.value)


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


class Cache:
    """A dita cache handle over a device buffer.

    `buffer` may be a torch uint8 device tensor (kept alive here), or None to allocate one
    with torch on `device`.  `buffer_ptr`/`buffer_bytes` bind a raw address instead (no
    device work happens before the first step, so host-only checks can use any address)."""

    def __init__(self, geom: Geometry, active_mask=None, buffer=None, device=None,
                 buffer_ptr=None, buffer_bytes=None):
        self.geom = geom
        self.P = geom.num_partitions
        self._active = None
        aptr = None
        if active_mask is not None:
            self._active, aptr = _u8(np.asarray(active_mask).ravel())
        self.required_bytes = dita_cache_required_bytes(geom, active_mask)
        if buffer_ptr is None:
            if buffer is None:
                import torch
                buffer = torch.empty(self.required_bytes, dtype=torch.uint8,
                                     device=device or "cuda")
            self.buffer = buffer
            buffer_ptr = buffer.data_ptr()
            buffer_bytes = buffer.numel() * buffer.element_size()
        else:
            self.buffer = None
        self._h = _P()
        _check(_lib.dita_cache_alloc(ctypes.byref(geom), aptr, _P(buffer_ptr),
                                     ctypes.c_size_t(buffer_bytes), ctypes.byref(self._h)))

    def __del__(self):
        self.free()

    def free(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            _lib.dita_cache_free(h)
            self._h = _P()

    def reset(self):
        _check(_lib.dita_cache_reset(self._h))

    def set_policy(self, policy: BlockPolicy = None, **kw):
        if policy is None:
            policy = make_policy(**kw)
        _check(_lib.dita_set_block_policy(self._h, ctypes.byref(policy)))

    def plan(self) -> dict:
        P = self.P
        mask = np.zeros(P * P, np.uint8)
        fp = np.zeros(P + 1, np.int32)
        rp = np.zeros(P + 1, np.int32)
        fc = np.zeros(P * P, np.int32)
        rc = np.zeros(P * P, np.int32)
        counts = np.zeros(3, np.int32)
        _check(_lib.dita_get_block_plan(self._h, mask.ctypes.data_as(_u8p),
                                        fp.ctypes.data_as(_i32p), fc.ctypes.data_as(_i32p),
                                        rp.ctypes.data_as(_i32p), rc.ctypes.data_as(_i32p),
                                        counts.ctypes.data_as(_i32p)))
        return {"mask": mask.reshape(P, P), "fresh_ptr": fp, "fresh_cols": fc[:fp[P]],
                "reuse_ptr": rp, "reuse_cols": rc[:rp[P]], "counts": counts}

    def step(self, q, k, v, out=None, lse=None, want_lse=True, stream=None,
             static_scratch=False):
        """Enqueue one step on `stream` (default: torch's current stream).  q/k/v are
        contiguous [B,H,N,D] (or [B,N,H,D]) device tensors; returns (out in the same layout,
        of the geometry's out dtype (f32 or bf16), lse [B,H,N] f32).  Caller-supplied `out` /
        `lse` must be of those dtypes, contiguous, of those shapes and on q's device; anything
        else raises ValueError before a launch.
        `static_scratch` calls dita_attn_step_static (the variant that allocates nothing; the
        outputs must then be passed in, or are allocated here, by torch, before the call)."""
        import torch
        for t in (q, k, v):
            if not t.is_contiguous():
                raise ValueError("q, k, v must be contiguous [B, H, N, D]")
        g = self.geom
        shape = (g.batch, g.heads, g.tokens, g.head_dim)
        if g.layout == LAYOUT_BNHD:
            shape = (g.batch, g.tokens, g.heads, g.head_dim)
        if tuple(q.shape) != shape or tuple(k.shape) != shape or tuple(v.shape) != shape:
            raise ValueError(f"q, k, v must have shape {shape}")
        want = torch.bfloat16 if g.qkv_dtype == BF16 else torch.float32
        if q.dtype != want or k.dtype != want or v.dtype != want:
            raise ValueError(f"q, k, v must be {want}")
        lse_shape = (g.batch, g.heads, g.tokens)
        out_dt = torch.bfloat16 if g.out_dtype == BF16 else torch.float32
        for name, t, shp, dt in (("out", out, shape, out_dt), ("lse", lse, lse_shape,
                                                                torch.float32)):
            if t is None:
                continue
            if t.dtype != dt:
                raise ValueError(f"{name} must be {dt}, not {t.dtype}")
            if tuple(t.shape) != shp:
                raise ValueError(f"{name} must have shape {shp}, not {tuple(t.shape)}")
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
            if t.device != q.device:
                raise ValueError(f"{name} must be on {q.device}, not {t.device}")
        if k.device != q.device or v.device != q.device:
            raise ValueError("q, k and v must be on one device")
        if q.device.type != "cuda":
            raise ValueError(f"q, k, v must be HIP device tensors, not on {q.device}")
        if out is None:
            out = torch.empty(shape, dtype=out_dt, device=q.device)
        if lse is None and want_lse:
            lse = torch.empty(lse_shape, dtype=torch.float32, device=q.device)
        fn = _lib.dita_attn_step_static if static_scratch else _lib.dita_attn_step
        _check(fn(self._h, _P(q.data_ptr()), _P(k.data_ptr()), _P(v.data_ptr()),
                  _P(out.data_ptr()), _P(lse.data_ptr()) if lse is not None else None,
                  _P(_stream_handle(stream))))
        return out, lse

    def step_raw(self, q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr=None, stream_handle=None):
        """The same call with raw device addresses."""
        _check(_lib.dita_attn_step(self._h, _P(q_ptr), _P(k_ptr), _P(v_ptr), _P(out_ptr),
                                   _P(lse_ptr) if lse_ptr else None,
                                   _P(stream_handle) if stream_handle else None))

    def read_slot(self, b, h, i, j, stream=None):
        import torch
        offs = dita_partition_offsets(self.geom)
        n_i = int(offs[i + 1] - offs[i])
        dev = self.buffer.device if self.buffer is not None else "cuda"
        o = torch.empty((n_i, self.geom.head_dim), dtype=torch.float32, device=dev)
        l = torch.empty((n_i,), dtype=torch.float32, device=dev)
        _check(_lib.dita_cache_read_slot(self._h, b, h, i, j, _P(o.data_ptr()),
                                         _P(l.data_ptr()), _P(_stream_handle(stream))))
        return o, l

    def set_profiling(self, enable: bool):
        _check(_lib.dita_set_profiling(self._h, 1 if enable else 0))

    def merge_groups(self, group: int, select=None, stream=None) -> int:
        """Merge cached states of aligned groups of `group` key partitions (per query
        partition); `select` [P, ceil(P/group)] or None for every eligible group.  Returns
        the number of groups merged."""
        sptr = None
        if select is not None:
            sarr, sptr = _u8(np.asarray(select).ravel())
        n = ctypes.c_int32(0)
        _check(_lib.dita_cache_merge_groups(self._h, int(group), sptr, ctypes.byref(n),
                                            _P(_stream_handle(stream))))
        return n.value

    def offload_bytes(self) -> int:
        """Host bytes of the offloaded state (counters, cached lse and O of every slot)."""
        n = ctypes.c_size_t(0)
        _check(_lib.dita_cache_offload_bytes(self._h, ctypes.byref(n)))
        return n.value

    def offload(self, release=True, stream=None):
        """Copy the cache's state into pinned host memory held by this object and mark the
        cache offloaded.  With `release`, wait for the copy and drop the device buffer this
        object holds (its memory goes back to torch's allocator)."""
        import torch
        host = torch.empty(self.offload_bytes(), dtype=torch.uint8, pin_memory=True)
        _check(_lib.dita_cache_offload(self._h, _P(host.data_ptr()),
                                       ctypes.c_size_t(host.numel()),
                                       _P(_stream_handle(stream))))
        self._host_state = host
        if release:
            torch.cuda.synchronize()
            self.buffer = None

    def restore(self, buffer=None, device=None, stream=None):
        """Bind `buffer` (a uint8 device tensor of at least required_bytes; None: a new one)
        and copy the offloaded state back; waits for the copy, then drops the host copy."""
        import torch
        host = getattr(self, "_host_state", None)
        if host is None:
            raise DitaError(1, "the cache is not offloaded by this object")
        if buffer is None:
            buffer = torch.empty(self.required_bytes, dtype=torch.uint8, device=device or "cuda")
        _check(_lib.dita_cache_restore(self._h, _P(buffer.data_ptr()),
                                       ctypes.c_size_t(buffer.numel() * buffer.element_size()),
                                       _P(host.data_ptr()), ctypes.c_size_t(host.numel()),
                                       _P(_stream_handle(stream))))
        self.buffer = buffer
        torch.cuda.synchronize()
        self._host_state = None

    def compact_bytes(self) -> int:
        """Device bytes the cache needs with its merged groups compacted (one slot per stored
        state)."""
        n = ctypes.c_size_t(0)
        _check(_lib.dita_cache_compact_bytes(self._h, ctypes.byref(n)))
        return n.value

    def _rebind(self, fn, nbytes, buffer, device, stream):
        import torch
        if buffer is None:
            dev = device or (self.buffer.device if self.buffer is not None else "cuda")
            buffer = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        _check(fn(self._h, _P(buffer.data_ptr()),
                  ctypes.c_size_t(buffer.numel() * buffer.element_size()),
                  _P(_stream_handle(stream))))
        self._old_buffer = self.buffer        # alive until the stream has passed the copy
        self.buffer = buffer
        return buffer

    def compact(self, buffer=None, device=None, stream=None):
        """Move the cache onto its compacted slot table in `buffer` (a uint8 device tensor of
        at least compact_bytes(); None: a new one).  The old buffer is released after the
        next synchronisation of this object (release_old_buffer)."""
        return self._rebind(_lib.dita_cache_compact, self.compact_bytes(), buffer, device,
                            stream)

    def expand(self, buffer=None, device=None, stream=None):
        """Move a compacted cache back onto the full slot table (required_bytes)."""
        return self._rebind(_lib.dita_cache_expand, self.required_bytes, buffer, device,
                            stream)

    def release_old_buffer(self):
        """Drop the buffer a compact / expand moved away from (synchronises the device)."""
        import torch
        if getattr(self, "_old_buffer", None) is not None:
            torch.cuda.synchronize()
            self._old_buffer = None

    def planner_state(self) -> dict:
        """The planner's measured state (waits for the last step's measurements)."""
        P = self.geom.num_partitions
        steps = ctypes.c_int32(0)
        _check(_lib.dita_get_planner_state(self._h, None, None, None, ctypes.byref(steps)))
        w = np.zeros(P * P, dtype=np.float32)
        delta = np.zeros(max(steps.value, 1) * P, dtype=np.float64)
        fs = np.zeros(P * P, dtype=np.int32)
        _check(_lib.dita_get_planner_state(self._h, w.ctypes.data_as(_f32p),
                                           delta.ctypes.data_as(_f64p),
                                           fs.ctypes.data_as(_i32p), ctypes.byref(steps)))
        return {"w": w.reshape(P, P), "delta": delta[:steps.value * P].reshape(steps.value, P),
                "fresh_step": fs.reshape(P, P), "steps": steps.value}

    def stats(self) -> dict:
        s = StepStats()
        _check(_lib.dita_get_stats(self._h, ctypes.byref(s)))
        return {"steps_done": s.steps_done, "last_counts": list(s.last_counts),
                "device_fresh_blocks": s.device_fresh_blocks,
                "device_reuse_blocks": s.device_reuse_blocks,
                "host_fresh_blocks": s.host_fresh_blocks,
                "host_reuse_blocks": s.host_reuse_blocks,
                "last_fresh_flops": s.last_fresh_flops,
                "last_cache_read_bytes": s.last_cache_read_bytes,
                "last_cache_write_bytes": s.last_cache_write_bytes,
                "device_v_range_errors": s.device_v_range_errors,
                "profiled_steps": s.profiled_steps, "step_kernel_ms": s.step_kernel_ms,
                "prep_kernel_ms": s.prep_kernel_ms,
                "device_ref_recomputes": s.device_ref_recomputes,
                "fixed_ref_steps": s.fixed_ref_steps,
                "fixed_ref_kernel_ms": s.fixed_ref_kernel_ms}


def policy_from(p) -> BlockPolicy:
    """BlockPolicy from any object with the fields of workloads.Policy."""
    return make_policy(kind=p.kind, max_fresh_frame_dist=p.max_fresh_frame_dist,
                       reuse_percent=p.reuse_percent, max_fresh_centroid2=p.max_fresh_centroid2,
                       tile_sparse=p.tile_sparse, anchor=p.anchor,
                       explicit_mask=p.explicit_mask,
                       group_size=getattr(p, "group_size", 1),
                       anchor_period=getattr(p, "anchor_period", 0),
                       max_error=getattr(p, "max_error", 0.0))


def geometry_from(cfg, offsets=None, out_dtype="f32", layout="bhnd") -> Geometry:
    """Geometry from any object with the fields of workloads.Config."""
    return make_geometry(cfg.batch, cfg.heads, cfg.tokens, cfg.head_dim, cfg.frames,
                         cfg.grid_h, cfg.grid_w, cfg.num_partitions, cfg.qkv_dtype,
                         offsets=offsets, cache_dtype=getattr(cfg, "cache_dtype", None),
                         layout=layout, out_dtype=out_dtype)
