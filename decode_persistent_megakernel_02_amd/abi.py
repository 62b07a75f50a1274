"""ctypes binding of libmk.so (include/mk.h, include/mk_debug.h).

Argument marshalling only: every function here forwards to the C entry point
of the same name and raises MkError on a non-zero status.  Device buffers are
torch tensors (their data_ptr()); PyTorch is used only for device memory and
streams.  There is no CPU fallback: importing this module without a built
libmk.so raises.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MK_LIBRARY") or os.path.join(PKG, "libmk.so")  # MK_LIBRARY: another build of the library

MK_ABI_VERSION = 2
MK_OK, MK_ERR_INVALID_ARG, MK_ERR_OUT_OF_MEMORY, MK_ERR_HIP = 0, -1, -2, -3
MK_ERR_CAPACITY, MK_ERR_TIMEOUT, MK_ERR_STATE, MK_ERR_UNSUPPORTED = -4, -5, -6, -7
MK_MODE_MEGAKERNEL, MK_MODE_PER_OP = 0, 1
MK_FLAG_TRACE, MK_FLAG_POISON, MK_FLAG_NO_GRAPH, MK_FLAG_FUSED_MERGE, MK_FLAG_TILED_WEIGHTS = 1, 2, 4, 8, 16
MK_FLAG_SPIN_LIMIT_1 = 32
MK_FLAG_BATCHED_PREFILL = 64
MK_FLAG_SHUFFLE = 128
STATUS_NAMES = {0: "MK_OK", -1: "MK_ERR_INVALID_ARG", -2: "MK_ERR_OUT_OF_MEMORY", -3: "MK_ERR_HIP",
                -4: "MK_ERR_CAPACITY", -5: "MK_ERR_TIMEOUT", -6: "MK_ERR_STATE", -7: "MK_ERR_UNSUPPORTED"}


class MkError(RuntimeError):
    def __init__(self, status, fn, msg):
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class mk_config(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("vocab", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("tie_embeddings", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("max_seq", ctypes.c_int32), ("mode", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("watchdog_ms", ctypes.c_uint32), ("num_cus", ctypes.c_int32), ("attn_split", ctypes.c_int32),
                ("kv_fp32", ctypes.c_int32), ("debug_seed", ctypes.c_uint32)]


_PP = ctypes.POINTER(ctypes.c_void_p)


class mk_weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("attn_norm", _PP), ("wq", _PP), ("wk", _PP), ("wv", _PP), ("wo", _PP), ("ffn_norm", _PP),
                ("w_gate", _PP), ("w_up", _PP), ("w_down", _PP)]


class mk_kv_layout(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("stride_layer", ctypes.c_int64),
                ("stride_batch", ctypes.c_int64), ("stride_head", ctypes.c_int64), ("stride_pos", ctypes.c_int64),
                ("length", ctypes.c_int32), ("batch", ctypes.c_int32), ("elem_bytes", ctypes.c_int32)]


class mk_graph_info(ctypes.Structure):
    _fields_ = [("n_tasks", ctypes.c_int32), ("n_events", ctypes.c_int32), ("n_stages", ctypes.c_int32),
                ("ncu", ctypes.c_int32), ("nsplit", ctypes.c_int32), ("split", ctypes.c_int32),
                ("max_queue", ctypes.c_int32), ("min_queue", ctypes.c_int32), ("max_cu_bytes", ctypes.c_int64),
                ("min_cu_bytes", ctypes.c_int64), ("weight_bytes", ctypes.c_int64)]


class mk_sim_result(ctypes.Structure):
    _fields_ = [("completed", ctypes.c_int32), ("executed", ctypes.c_int32), ("blocked_event", ctypes.c_int32),
                ("race", ctypes.c_int32)]


class mk_debug_view(ctypes.Structure):
    _fields_ = [("xs", ctypes.c_void_p), ("xmid", ctypes.c_void_p), ("q", ctypes.c_void_p),
                ("attn_out", ctypes.c_void_p), ("h", ctypes.c_void_p), ("events", ctypes.c_void_p),
                ("n_events", ctypes.c_int32), ("n_tasks", ctypes.c_int32), ("ncu", ctypes.c_int32),
                ("nsplit", ctypes.c_int32), ("split", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("exact_ops", ctypes.c_uint32), ("op_grid", ctypes.c_int32 * 9)]


class mk_mega_view(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("xmid", ctypes.c_void_p), ("qkv", ctypes.c_void_p),
                ("attn", ctypes.c_void_p), ("h", ctypes.c_void_p), ("epoch", ctypes.c_uint32)]


# Every symbol the headers declare, with its ctypes signature.
_P, _I32, _I64, _U64, _F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float
SIGNATURES = {
    "mk_create": ([ctypes.POINTER(mk_config), ctypes.POINTER(mk_weights), _P, ctypes.POINTER(_P)], _I32),
    "mk_prefill": ([_P, _P, _I32, _I32, _P, _P], _I32),
    "mk_decode_step": ([_P, _P, _P, _P], _I32),
    "mk_synchronize": ([_P], _I32),
    "mk_reset": ([_P], _I32),
    "mk_kv_view": ([_P, ctypes.POINTER(mk_kv_layout)], _I32),
    "mk_last_error": ([], ctypes.c_char_p),
    "mk_destroy": ([_P], None),
    "mk_graph_inspect": ([ctypes.POINTER(mk_config), _I32, ctypes.POINTER(mk_graph_info)], _I32),
    "mk_graph_simulate": ([ctypes.POINTER(mk_config), _I32, _U64, _I32, _I32, ctypes.POINTER(mk_sim_result)], _I32),
    "mk_batched_graph_fault": ([ctypes.POINTER(mk_config), _I32, _I32], _I32),
    "mk_graph_export": ([ctypes.POINTER(mk_config), _I32, _P, _P, _I32, ctypes.POINTER(_I32)], _I32),
    "mk_get_debug_view": ([_P, ctypes.POINTER(mk_debug_view)], _I32),
    "mk_read_status": ([_P, ctypes.POINTER(ctypes.c_uint32)], _I32),
    "mk_read_trace": ([_P, ctypes.POINTER(ctypes.c_uint64), _I32, ctypes.POINTER(_I32),
                       ctypes.POINTER(ctypes.c_double)], _I32),
    "mk_time_ops": ([_P, ctypes.c_uint32, _I32], _I32),
    "mk_read_op_times": ([_P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I32)], _I32),
    "mk_time_op_replay": ([_P, _I32, _I32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I32)], _I32),
    "mk_t_gemv": ([_P, _P, _P, _I32, _I32, _P], _I32),
    "mk_t_rmsnorm": ([_P, _P, _F, _P, _I32, _P], _I32),
    "mk_t_attention": ([_P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P], _I32),
    "mk_t_attention_noalloc": ([_P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P], _I32),
    "mk_t_op_raw": ([_P, _I32, _I32, _P, _P], _I32),
    "mk_t_set_prefill_rows": ([_P, _I32], _I32),
    "mk_generate": ([_P, _P, _I32, _P, _P], _I32),
    "mk_t_bgemm": ([_P, _P, _P, _I32, _I32, _I32, _I32, _P], _I32),
    "mk_tile_weights": ([_P, _P, _I64, _I64, _P], _I32),
    "mk_kv_read": ([_P, _P, _P, _I64], _I32),
    "mk_trace_op": ([_P, _I32, _I32], _I32),
    "mk_t_argmax": ([_P, _I32, _P, _P], _I32),
    "mk_device_info": ([ctypes.POINTER(_I32), ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I32)], _I32),
    "mk_mega_trace": ([_P, _P, _I64, ctypes.POINTER(_I32), ctypes.POINTER(_I32), ctypes.POINTER(_I32),
                       ctypes.POINTER(ctypes.c_double)], _I32),
    "mk_get_mega_view": ([_P, ctypes.POINTER(mk_mega_view)], _I32),
    "mk_t_stream_read": ([_P, _I64, _I32, _I32, _I32, _P, ctypes.POINTER(ctypes.c_float)], _I32),
}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m decode_persistent_megakernel_02_amd.build`")
# PyTorch first: it loads its HIP runtime into the global symbol scope, so the
# library's HIP calls bind to that same runtime (one set of devices, streams
# and queues in the process).  Loaded the other way round, the library would
# bring up a second HIP runtime next to PyTorch's, which then finds no device.
import torch  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)
for _name, (_args, _res) in SIGNATURES.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


def _check(status, fn):
    if status != MK_OK:
        raise MkError(status, fn, lib.mk_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(getattr(stream, "cuda_stream", stream) or 0)


def make_config(shape, max_seq, max_batch=1, mode=MK_MODE_PER_OP, flags=0, watchdog_ms=0, num_cus=0,
                attn_split=0, kv_fp32=True, debug_seed=0) -> mk_config:
    """mk_config from a synth.presets.ModelShape-like object."""
    c = mk_config()
    c.abi_version = MK_ABI_VERSION
    c.n_layers, c.hidden, c.n_q_heads = shape.n_layers, shape.hidden, shape.n_q_heads
    c.n_kv_heads, c.head_dim, c.ffn, c.vocab = shape.n_kv_heads, shape.head_dim, shape.ffn, shape.vocab
    c.rms_eps, c.rope_theta = shape.rms_eps, shape.rope_theta
    c.tie_embeddings = 1 if shape.tie_embeddings else 0
    c.max_batch, c.max_seq, c.mode, c.flags = max_batch, max_seq, mode, flags
    c.watchdog_ms, c.num_cus, c.attn_split = watchdog_ms, num_cus, attn_split
    c.kv_fp32 = 1 if kv_fp32 else 0
    c.debug_seed = debug_seed
    return c


class Handle:
    """An mk_handle plus the Python objects whose memory it borrows."""

    def __init__(self, ptr, keep):
        self.ptr = ptr
        self._keep = keep

    def __del__(self):
        if getattr(self, "ptr", None):
            mk_destroy(self)


LAYER_FIELDS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")


def mk_create(cfg: mk_config, weights: dict, stream=None) -> Handle:
    """weights: name -> device tensor (bf16 or int16/uint16 bits), names as synth.presets.weight_shapes."""
    L = cfg.n_layers
    arrays = {}
    for f in LAYER_FIELDS:
        arr = (ctypes.c_void_p * L)(*[weights[f"layers.{l}.{f}"].data_ptr() for l in range(L)])
        arrays[f] = arr
    w = mk_weights()
    w.embed = weights["embed"].data_ptr()
    w.lm_head = weights["lm_head"].data_ptr() if "lm_head" in weights and not cfg.tie_embeddings else None
    w.final_norm = weights["final_norm"].data_ptr()
    for f in LAYER_FIELDS:
        setattr(w, f, ctypes.cast(arrays[f], _PP))
    out = ctypes.c_void_p()
    _check(lib.mk_create(ctypes.byref(cfg), ctypes.byref(w), _stream(stream), ctypes.byref(out)), "mk_create")
    return Handle(out, (weights, arrays, w, cfg))


def mk_prefill(h: Handle, tokens, next_out, logits=None):
    B, P = tokens.shape
    _check(lib.mk_prefill(h.ptr, _ptr(tokens), B, P, _ptr(next_out), _ptr(logits)), "mk_prefill")


def mk_decode_step(h: Handle, d_in, d_out, logits=None):
    _check(lib.mk_decode_step(h.ptr, _ptr(d_in), _ptr(d_out), _ptr(logits)), "mk_decode_step")


def mk_generate(h: Handle, d_in, n_steps: int, d_out, logits=None):
    """n_steps greedy steps from d_in[0]; ids into d_out[:n_steps] (one launch
    in megakernel mode)."""
    _check(lib.mk_generate(h.ptr, _ptr(d_in), n_steps, _ptr(d_out), _ptr(logits) if logits is not None else None),
           "mk_generate")


def mk_synchronize(h: Handle):
    _check(lib.mk_synchronize(h.ptr), "mk_synchronize")


def mk_reset(h: Handle):
    _check(lib.mk_reset(h.ptr), "mk_reset")


def mk_kv_view(h: Handle) -> mk_kv_layout:
    out = mk_kv_layout()
    _check(lib.mk_kv_view(h.ptr, ctypes.byref(out)), "mk_kv_view")
    return out


def mk_kv_read(h: Handle, k_host, v_host):
    """Copy the K and V caches into two host numpy arrays of the cache's size
    (uint16 for bf16 caches, float32 for fp32)."""
    assert k_host.nbytes == v_host.nbytes and k_host.flags.c_contiguous and v_host.flags.c_contiguous
    _check(lib.mk_kv_read(h.ptr, k_host.ctypes.data, v_host.ctypes.data, k_host.nbytes), "mk_kv_read")


def mk_last_error() -> str:
    return lib.mk_last_error().decode()


def mk_destroy(h: Handle):
    if h.ptr:
        lib.mk_destroy(h.ptr)
        h.ptr = None


def mk_graph_inspect(cfg: mk_config, ncu: int) -> mk_graph_info:
    out = mk_graph_info()
    _check(lib.mk_graph_inspect(ctypes.byref(cfg), ncu, ctypes.byref(out)), "mk_graph_inspect")
    return out


def mk_batched_graph_fault(cfg: mk_config, ncu: int, fault: int) -> None:
    """Raises MkError(MK_ERR_INVALID_ARG) when the validator catches the planted mistake."""
    _check(lib.mk_batched_graph_fault(ctypes.byref(cfg), ncu, fault), "mk_batched_graph_fault")


def mk_graph_simulate(cfg: mk_config, ncu: int, seed: int, workers: int = 7, drop_event: int = -1) -> mk_sim_result:
    out = mk_sim_result()
    _check(lib.mk_graph_simulate(ctypes.byref(cfg), ncu, seed, workers, drop_event, ctypes.byref(out)),
           "mk_graph_simulate")
    return out


TASK_DTYPE = None


def task_dtype():
    import numpy as np
    return np.dtype([("type", "u1"), ("page", "u1"), ("layer", "<u2"), ("in_event", "<u2"), ("out_event", "<u2"),
                     ("in_count", "<u4"), ("stage", "<u2"), ("batch", "<u2"), ("local_slot", "<u2"),
                     ("local_count", "<u2"), ("id", "<u4"), ("a0", "<i4"), ("a1", "<i4"), ("a2", "<i4"),
                     ("a3", "<i4"), ("_pad", "V8")])


def mk_graph_export(cfg: mk_config, ncu: int):
    """(tasks structured array in global order, cu of each task)."""
    import numpy as np
    n = ctypes.c_int32()
    _check(lib.mk_graph_export(ctypes.byref(cfg), ncu, None, None, 0, ctypes.byref(n)), "mk_graph_export")
    tasks = np.zeros(n.value, dtype=task_dtype())
    cu = np.zeros(n.value, dtype=np.int32)
    _check(lib.mk_graph_export(ctypes.byref(cfg), ncu, tasks.ctypes.data, cu.ctypes.data, n.value, ctypes.byref(n)),
           "mk_graph_export")
    return tasks, cu


def mk_get_debug_view(h: Handle) -> mk_debug_view:
    out = mk_debug_view()
    _check(lib.mk_get_debug_view(h.ptr, ctypes.byref(out)), "mk_get_debug_view")
    return out


def mk_read_status(h: Handle):
    out = (ctypes.c_uint32 * 16)()
    _check(lib.mk_read_status(h.ptr, out), "mk_read_status")
    return list(out)


def mk_read_trace(h: Handle):
    import numpy as np
    n = ctypes.c_int32()
    tpu = ctypes.c_double()
    _check(lib.mk_read_trace(h.ptr, None, 0, ctypes.byref(n), ctypes.byref(tpu)), "mk_read_trace")
    buf = np.zeros(2 * n.value, dtype=np.uint64)
    _check(lib.mk_read_trace(h.ptr, buf.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), n.value, ctypes.byref(n),
                             ctypes.byref(tpu)), "mk_read_trace")
    return buf.reshape(-1, 2), tpu.value


TASK_TYPES = {"qkv": 1, "attn": 2, "merge": 3, "o": 4, "gu": 5, "down": 6, "lm": 7, "argmax": 8}
# operator timing also knows the RMSNorm launches of the batched path
OP_TYPES = {"norm": 0, **TASK_TYPES}


def mk_time_ops(h: Handle, types, max_launches: int):
    mask = 0
    for t in types:
        mask |= 1 << OP_TYPES[t]
    _check(lib.mk_time_ops(h.ptr, mask, max_launches), "mk_time_ops")


def mk_read_op_times(h: Handle):
    """{type name: (total ms, launches)} of the timed launches."""
    ms = (ctypes.c_double * 9)()
    n = (ctypes.c_int32 * 9)()
    _check(lib.mk_read_op_times(h.ptr, ms, n), "mk_read_op_times")
    return {name: (ms[i], n[i]) for name, i in OP_TYPES.items() if n[i]}


def mk_time_op_replay(h: Handle, type_name: str, reps: int):
    """(total ms, launches) of `reps` back-to-back replays of one operator's
    launches of a decode step (every layer)."""
    ms = ctypes.c_double()
    n = _I32()
    _check(lib.mk_time_op_replay(h.ptr, OP_TYPES[type_name], reps, ctypes.byref(ms), ctypes.byref(n)),
           "mk_time_op_replay")
    return ms.value, n.value


def mk_trace_op(h: Handle, type_name, layer: int):
    """Log the wave timeline of one GEMV operator launch (None stops logging)."""
    t = -1 if type_name is None else TASK_TYPES[type_name]
    _check(lib.mk_trace_op(h.ptr, t, layer), "mk_trace_op")


def mk_t_gemv(W, x, y, stream=None):
    N, K = W.shape
    _check(lib.mk_t_gemv(_ptr(W), _ptr(x), _ptr(y), N, K, _stream(stream)), "mk_t_gemv")


def mk_t_rmsnorm(x, gamma, eps, y, stream=None):
    _check(lib.mk_t_rmsnorm(_ptr(x), _ptr(gamma), eps, _ptr(y), x.numel(), _stream(stream)), "mk_t_rmsnorm")


def mk_t_attention(q, k, v, T, split, o, stream=None):
    """q [nq, hd] fp32; k, v [nkv, S, hd] bf16 or fp32 (S >= T); o [nq, hd] fp32."""
    nq, hd = q.shape
    nkv, S, _ = k.shape
    f32 = 1 if k.element_size() == 4 else 0
    _check(lib.mk_t_attention(_ptr(q), _ptr(k), _ptr(v), S * hd, nq, nkv, hd, T, split, f32, _ptr(o),
                              _stream(stream)), "mk_t_attention")


def mk_t_set_prefill_rows(h: Handle, rows: int):
    _check(lib.mk_t_set_prefill_rows(h.ptr, rows), "mk_t_set_prefill_rows")


def mk_t_op_raw(h: Handle, op_type: int, layer: int, x, y):
    """The shipped GEMV operator kernel of op_type (1 QKV, 4 O, 5 gate/up, 6
    down, 7 LM head) on the raw input x; y receives its raw dot products."""
    _check(lib.mk_t_op_raw(h.ptr, op_type, layer, _ptr(x), _ptr(y)), "mk_t_op_raw")


def mk_t_attention_noalloc(q, k, v, T, split, o, stream=None):
    """mk_t_attention without any device allocation (static per-device split
    records); asynchronous on `stream`."""
    nq, hd = q.shape
    nkv, S, _ = k.shape
    f32 = 1 if k.element_size() == 4 else 0
    _check(lib.mk_t_attention_noalloc(_ptr(q), _ptr(k), _ptr(v), S * hd, nq, nkv, hd, T, split, f32, _ptr(o),
                                      _stream(stream)), "mk_t_attention_noalloc")


def mk_t_bgemm(W, A, Y, B, tiled=False, stream=None):
    """Y = (A[0, :B] + A[1, :B]) @ W.T on the matrix cores; A [2, Bp, K] bf16 hi/lo
    planes with Bp = 16, 32 or 64 rows, rows >= B zero.  tiled: W [N, K] holds
    the mk_tile_weights layout."""
    N, K = W.shape
    Bp = 16 * (1 if B <= 16 else 2 if B <= 32 else 4)
    assert A.shape == (2, Bp, K) and Y.shape == (B, N)
    _check(lib.mk_t_bgemm(_ptr(W), _ptr(A), _ptr(Y), N, K, B, 1 if tiled else 0, _stream(stream)), "mk_t_bgemm")


def mk_tile_weights(src, dst, stream=None):
    """dst = the tiled layout of the row-major bf16 matrix src [N, K] (device)."""
    N, K = src.shape
    assert dst.numel() == src.numel() and dst.data_ptr() != src.data_ptr()
    _check(lib.mk_tile_weights(_ptr(src), _ptr(dst), N, K, _stream(stream)), "mk_tile_weights")


def mk_t_argmax(x, out, stream=None):
    _check(lib.mk_t_argmax(_ptr(x), x.numel(), _ptr(out), _stream(stream)), "mk_t_argmax")


def mk_device_info():
    n, l = ctypes.c_int32(), ctypes.c_int32()
    t = ctypes.c_double()
    _check(lib.mk_device_info(ctypes.byref(n), ctypes.byref(t), ctypes.byref(l)), "mk_device_info")
    return n.value, t.value, l.value


def mk_mega_trace(h: Handle):
    """(timestamps uint64 [ops, ncu, slots], ticks per us) of the last megakernel step."""
    import numpy as np
    ops, ncu, slots = _I32(), _I32(), _I32()
    tpu = ctypes.c_double()
    _check(lib.mk_mega_trace(h.ptr, None, 0, ctypes.byref(ops), ctypes.byref(ncu), ctypes.byref(slots),
                             ctypes.byref(tpu)), "mk_mega_trace")
    buf = np.zeros(ops.value * ncu.value * slots.value, dtype=np.uint64)
    _check(lib.mk_mega_trace(h.ptr, buf.ctypes.data, buf.size, ctypes.byref(ops), ctypes.byref(ncu),
                             ctypes.byref(slots), ctypes.byref(tpu)), "mk_mega_trace")
    return buf.reshape(ops.value, ncu.value, slots.value), tpu.value


def mk_get_mega_view(h: Handle) -> mk_mega_view:
    out = mk_mega_view()
    _check(lib.mk_get_mega_view(h.ptr, ctypes.byref(out)), "mk_get_mega_view")
    return out


def mk_t_stream_read(src, wgs: int, loads: int, reps: int = 5, stream=None) -> float:
    """Fastest of `reps` streaming reads of the device tensor src (ms)."""
    ms = ctypes.c_float()
    _check(lib.mk_t_stream_read(_ptr(src), src.numel() * src.element_size(), wgs, loads, reps, _stream(stream),
                                ctypes.byref(ms)), "mk_t_stream_read")
    return ms.value
