"""ctypes binding of the C ABI in include/dec.h (argument marshalling only).

Every function here forwards to libdec.so under the same name. Loading fails loudly when
the library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, List, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdec.so")

DEC_ABI_VERSION = 3
ARCH = {"gqa": 0, "mla": 1, "moe": 2}
STATUS = {0: "DEC_OK", -1: "DEC_E_INVAL", -2: "DEC_E_SHAPE", -3: "DEC_E_CAPACITY", -4: "DEC_E_DEVICE",
          -5: "DEC_E_OCCUPANCY", -6: "DEC_E_HIP", -7: "DEC_E_TIMEOUT", -8: "DEC_E_UNBOUND", -9: "DEC_E_PLAN"}
DTYPE = {0: "bf16", 1: "fp32", 2: "i32", 3: "fp8", 4: "fp4x2", 5: "e8m0"}
WEIGHT_FORMAT = {"bf16": 0, "fp8": 1, "mxfp4": 2}

# task type ids (mirror of the engine's TaskType enum)
TASK_TYPES = {1: "QKV", 2: "ATTN", 3: "OPROJ", 4: "GATEUP", 5: "DOWN", 6: "LMHEAD", 7: "MLA_A", 8: "MLA_B",
              9: "MLA_KVAPP", 10: "MLA_ABSORB", 11: "MLA_ATTN", 12: "MLA_UV", 13: "ROUTER", 14: "SHARED_GU",
              15: "TOPK", 16: "EXPERT_GU", 17: "MOE_DOWN", 18: "OPROJ_G", 19: "HINIT", 20: "ARGMAX",
              21: "IDX_Q", 22: "IDX_SCORE", 23: "IDX_TOPK"}


class DecError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class ModelShape(C.Structure):
    _fields_ = [("abi_version", C.c_int32), ("arch", C.c_int32), ("n_layers", C.c_int32), ("hidden", C.c_int32),
                ("vocab", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("ffn", C.c_int32), ("q_lora_rank", C.c_int32), ("kv_lora_rank", C.c_int32), ("qk_nope", C.c_int32),
                ("qk_rope", C.c_int32), ("v_head", C.c_int32), ("n_routed", C.c_int32), ("n_shared", C.c_int32),
                ("top_k", C.c_int32), ("expert_ffn", C.c_int32), ("rms_eps", C.c_float), ("weight_format", C.c_int32),
                ("rope_theta", C.c_double), ("index_heads", C.c_int32), ("index_dim", C.c_int32),
                ("index_topk", C.c_int32), ("reserved1", C.c_int32)]


class DeviceInfo(C.Structure):
    _fields_ = [("gfx_arch", C.c_int32), ("n_cu", C.c_int32), ("n_xcd", C.c_int32), ("lds_bytes_per_cu", C.c_int32),
                ("max_threads_per_cu", C.c_int32), ("reserved0", C.c_int32)]


class TensorDesc(C.Structure):
    _fields_ = [("name", C.c_char * 64), ("dtype", C.c_int32), ("rank", C.c_int32), ("dims", C.c_int64 * 4),
                ("bytes", C.c_int64)]


class Sizes(C.Structure):
    _fields_ = [("x_bytes", C.c_int64), ("kv_bytes", C.c_int64), ("out_bytes", C.c_int64),
                ("workspace_bytes", C.c_int64), ("weight_bytes", C.c_int64),
                ("algorithmic_bytes_per_step", C.c_int64)]


class TaskDescC(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("id", "type", "layer", "stage", "wg", "xcd", "list_pos", "unit_begin",
                                         "unit_end", "aux0", "aux1", "n_deps", "dep_first", "signal", "signal2",
                                         "aux2", "kv_staged", "aux3")]


class BufferDesc(C.Structure):
    _fields_ = [("name", C.c_char * 64), ("dtype", C.c_int32), ("reserved0", C.c_int32), ("offset", C.c_int64),
                ("count", C.c_int64)]


_lib = None


def lib() -> C.CDLL:
    """Load libdec.so (built by persistent_tile_scheduled_amd.build); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("DEC_LIBRARY", LIB_PATH)  # an alternative build of the same ABI
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: run `python -m persistent_tile_scheduled_amd.build` first")
    L = C.CDLL(path)
    P = C.c_void_p
    sig = {
        "dec_last_error": (C.c_char_p, []),
        "dec_device_query": (C.c_int, [C.POINTER(DeviceInfo)]),
        "dec_plan_create": (C.c_int, [C.POINTER(ModelShape), C.c_int64, C.POINTER(P)]),
        "dec_plan_create_for": (C.c_int, [C.POINTER(ModelShape), C.c_int64, C.POINTER(DeviceInfo), C.POINTER(P)]),
        "dec_plan_destroy": (C.c_int, [P]),
        "dec_plan_n_weights": (C.c_int64, [P]),
        "dec_plan_weight_desc": (C.c_int, [P, C.c_int64, C.POINTER(TensorDesc)]),
        "dec_plan_sizes": (C.c_int, [P, C.POINTER(Sizes)]),
        "dec_plan_n_tasks": (C.c_int64, [P]),
        "dec_plan_tasks": (C.c_int, [P, C.POINTER(TaskDescC), C.c_int64, C.POINTER(C.c_int64)]),
        "dec_plan_n_deps": (C.c_int64, [P]),
        "dec_plan_deps": (C.c_int, [P, C.POINTER(C.c_int32), C.c_int64, C.POINTER(C.c_int64)]),
        "dec_plan_n_counters": (C.c_int64, [P]),
        "dec_plan_n_buffers": (C.c_int64, [P]),
        "dec_plan_buffer_desc": (C.c_int, [P, C.c_int64, C.POINTER(BufferDesc)]),
        "dec_plan_grid": (C.c_int, [P, C.POINTER(C.c_int32), C.POINTER(C.c_int32), C.POINTER(C.c_int32)]),
        "dec_plan_bind": (C.c_int, [P, C.POINTER(P), C.c_int64, P, C.c_int64, P]),
        "dec_plan_bind_scratch": (C.c_int, [P, C.POINTER(P), C.c_int64, P]),
        "dec_step": (C.c_int, [P, P, P, P, P]),
        "dec_plan_n_stages": (C.c_int64, [P]),
        "dec_plan_create_dynamic": (C.c_int, [C.POINTER(ModelShape), C.c_int64, C.POINTER(DeviceInfo), C.POINTER(P)]),
        "dec_step_dynamic": (C.c_int, [P, P, P, P, P, P]),
        "dec_plan_create_verify": (C.c_int, [C.POINTER(ModelShape), C.c_int64, C.c_int32, C.POINTER(DeviceInfo), C.POINTER(P)]),
        "dec_step_stages": (C.c_int, [P, P, P, P, C.c_int32, C.c_int32, P]),
        "dec_plan_status": (C.c_int, [P, P]),
        "dec_plan_reset": (C.c_int, [P, P]),
        "dec_plan_set_watchdog": (C.c_int, [P, C.c_int64]),
        "dec_stream_read": (C.c_int, [P, C.c_int64, P, C.c_int64, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


# the C ABI's exported symbols (every name declared in include/dec.h)
ABI_SYMBOLS = ["dec_last_error", "dec_device_query", "dec_plan_create", "dec_plan_create_for", "dec_plan_destroy",
               "dec_plan_n_weights", "dec_plan_weight_desc", "dec_plan_sizes", "dec_plan_n_tasks", "dec_plan_tasks",
               "dec_plan_n_deps", "dec_plan_deps", "dec_plan_n_counters", "dec_plan_n_buffers",
               "dec_plan_buffer_desc", "dec_plan_grid", "dec_plan_bind", "dec_plan_bind_scratch", "dec_step",
               "dec_plan_n_stages",
               "dec_step_stages", "dec_plan_create_dynamic", "dec_step_dynamic", "dec_plan_status",
               "dec_plan_reset", "dec_plan_set_watchdog", "dec_stream_read", "dec_plan_create_verify"]


def _check(status: int):
    if status != 0:
        raise DecError(status, lib().dec_last_error().decode())


def shape_from_config(cfg: dict) -> ModelShape:
    s = ModelShape()
    s.abi_version = DEC_ABI_VERSION
    s.arch = ARCH[cfg["arch"]]
    for k in ("n_layers", "hidden", "vocab", "n_q_heads", "n_kv_heads", "head_dim", "ffn", "q_lora_rank",
              "kv_lora_rank", "qk_nope", "qk_rope", "v_head", "n_routed", "n_shared", "top_k", "expert_ffn",
              "index_heads", "index_dim", "index_topk"):
        setattr(s, k, int(cfg.get(k, 0) or 0))
    s.rms_eps = float(cfg["rms_eps"])
    s.rope_theta = float(cfg["rope_theta"])
    s.weight_format = WEIGHT_FORMAT[cfg.get("weights", "bf16")]
    return s


def device_info(gfx_arch=950, n_cu=256, n_xcd=8, lds=160 * 1024, max_threads=2048) -> DeviceInfo:
    d = DeviceInfo()
    d.gfx_arch, d.n_cu, d.n_xcd, d.lds_bytes_per_cu, d.max_threads_per_cu = gfx_arch, n_cu, n_xcd, lds, max_threads
    return d


def stream_read(buf_ptr: int, nbytes: int, sink_ptr: int, sink_bytes: int, stream: int = 0):
    """One stream-read launch (dec_stream_read): the device's HBM read ceiling for the engine's loads."""
    _check(lib().dec_stream_read(C.c_void_p(int(buf_ptr)), int(nbytes), C.c_void_p(int(sink_ptr)), int(sink_bytes),
                                 C.c_void_p(int(stream))))


def device_query() -> DeviceInfo:
    d = DeviceInfo()
    _check(lib().dec_device_query(C.byref(d)))
    return d


class Plan:
    """Owner of one dec_plan (host object). All device memory belongs to the caller."""

    def __init__(self, cfg_or_shape, kv_len: Optional[int] = None, device: Optional[DeviceInfo] = None,
                 max_len: Optional[int] = None, n_tokens: Optional[int] = None):
        """A plan for one kv_len, or, with max_len, a plan whose position is read per step
        (dec_plan_create_dynamic), or, with n_tokens (default: a config's "verify" count), a
        verification step of that many tokens (dec_plan_create_verify)."""
        L = lib()
        if isinstance(cfg_or_shape, dict):
            self.shape = shape_from_config(cfg_or_shape)
            if kv_len is None:
                kv_len = cfg_or_shape["kv_len"]
            if n_tokens is None and cfg_or_shape.get("verify"):
                n_tokens = int(cfg_or_shape["verify"])
        else:
            self.shape = cfg_or_shape
        self.dynamic = max_len is not None
        self.kv_len = int(max_len if self.dynamic else kv_len)
        self.n_tokens = 1 if n_tokens is None else int(n_tokens)
        h = C.c_void_p()
        if n_tokens is not None:
            if self.dynamic:
                raise ValueError("a verification plan has a fixed length")
            dev = C.byref(device) if device is not None else None
            _check(L.dec_plan_create_verify(C.byref(self.shape), self.kv_len, self.n_tokens, dev, C.byref(h)))
        elif self.dynamic:
            dev = C.byref(device) if device is not None else None
            _check(L.dec_plan_create_dynamic(C.byref(self.shape), self.kv_len, dev, C.byref(h)))
        elif device is None:
            _check(L.dec_plan_create(C.byref(self.shape), self.kv_len, C.byref(h)))
        else:
            _check(L.dec_plan_create_for(C.byref(self.shape), self.kv_len, C.byref(device), C.byref(h)))
        self.h = h

    def close(self):
        if getattr(self, "h", None):
            lib().dec_plan_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- introspection
    def weight_descs(self) -> List[dict]:
        L = lib()
        out = []
        for i in range(L.dec_plan_n_weights(self.h)):
            d = TensorDesc()
            _check(L.dec_plan_weight_desc(self.h, i, C.byref(d)))
            out.append({"name": d.name.decode(), "dtype": DTYPE[d.dtype], "shape": tuple(d.dims[:d.rank]),
                        "bytes": d.bytes})
        return out

    def sizes(self) -> dict:
        s = Sizes()
        _check(lib().dec_plan_sizes(self.h, C.byref(s)))
        return {k: getattr(s, k) for k, _ in Sizes._fields_}

    def tasks(self) -> List[dict]:
        L = lib()
        n = L.dec_plan_n_tasks(self.h)
        buf = (TaskDescC * max(n, 1))()
        got = C.c_int64()
        _check(L.dec_plan_tasks(self.h, buf, n, C.byref(got)))
        return [{k: getattr(buf[i], k) for k, _ in TaskDescC._fields_} for i in range(got.value)]

    def deps(self) -> List[tuple]:
        L = lib()
        n = L.dec_plan_n_deps(self.h)
        buf = (C.c_int32 * max(2 * n, 2))()
        got = C.c_int64()
        _check(L.dec_plan_deps(self.h, buf, 2 * n, C.byref(got)))
        return [(buf[2 * i], buf[2 * i + 1]) for i in range(got.value)]

    def n_counters(self) -> int:
        return lib().dec_plan_n_counters(self.h)

    def buffers(self) -> Dict[str, dict]:
        L = lib()
        out = {}
        for i in range(L.dec_plan_n_buffers(self.h)):
            d = BufferDesc()
            _check(L.dec_plan_buffer_desc(self.h, i, C.byref(d)))
            out[d.name.decode()] = {"dtype": DTYPE[d.dtype], "offset": d.offset, "count": d.count}
        return out

    def grid(self) -> tuple:
        a, b, c = C.c_int32(), C.c_int32(), C.c_int32()
        _check(lib().dec_plan_grid(self.h, C.byref(a), C.byref(b), C.byref(c)))
        return a.value, b.value, c.value

    # ---- device side
    def bind(self, weight_ptrs: Sequence[int], workspace_ptr: int, workspace_bytes: int, stream: int = 0):
        arr = (C.c_void_p * len(weight_ptrs))(*[C.c_void_p(int(p)) for p in weight_ptrs])
        _check(lib().dec_plan_bind(self.h, arr, len(weight_ptrs), C.c_void_p(int(workspace_ptr)),
                                   int(workspace_bytes), C.c_void_p(int(stream))))

    def bind_scratch(self, weight_ptrs: Sequence[int], stream: int = 0):
        """Bind to the library's static per-device workspace (allocates nothing)."""
        arr = (C.c_void_p * len(weight_ptrs))(*[C.c_void_p(int(p)) for p in weight_ptrs])
        _check(lib().dec_plan_bind_scratch(self.h, arr, len(weight_ptrs), C.c_void_p(int(stream))))

    def step(self, x_ptr: int, kv_ptr: int, out_ptr: int, stream: int = 0):
        _check(lib().dec_step(self.h, C.c_void_p(int(x_ptr)), C.c_void_p(int(kv_ptr)), C.c_void_p(int(out_ptr)),
                              C.c_void_p(int(stream))))

    def n_stages(self) -> int:
        return lib().dec_plan_n_stages(self.h)

    def step_stages(self, x_ptr: int, kv_ptr: int, out_ptr: int, stage_lo: int, stage_hi: int, stream: int = 0):
        _check(lib().dec_step_stages(self.h, C.c_void_p(int(x_ptr)), C.c_void_p(int(kv_ptr)), C.c_void_p(int(out_ptr)),
                                     int(stage_lo), int(stage_hi), C.c_void_p(int(stream))))

    def step_dynamic(self, x_ptr: int, kv_ptr: int, out_ptr: int, state_ptr: int, stream: int = 0):
        """x_ptr 0: start from the embedding row of the state's token."""
        x = C.c_void_p(int(x_ptr)) if x_ptr else None
        _check(lib().dec_step_dynamic(self.h, x, C.c_void_p(int(kv_ptr)), C.c_void_p(int(out_ptr)),
                                      C.c_void_p(int(state_ptr)), C.c_void_p(int(stream))))

    def status(self, stream: int = 0):
        _check(lib().dec_plan_status(self.h, C.c_void_p(int(stream))))

    def reset(self, stream: int = 0):
        _check(lib().dec_plan_reset(self.h, C.c_void_p(int(stream))))

    def set_watchdog(self, microseconds: int):
        _check(lib().dec_plan_set_watchdog(self.h, int(microseconds)))
