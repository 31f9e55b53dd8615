"""Python binding of libmikv.so (paged-KV GQA decode for MI355X / gfx950).

Argument marshalling only: every function below forwards to the C entry
point of the same name declared in include/mikv.h. Device buffers are given
as torch tensors (or raw integer addresses); PyTorch supplies device memory
and the current HIP stream. No computation happens here, and there is no
fallback: if the shared library is missing the import of any entry point
raises.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmikv.so")

MI_OK = 0
MI_ERR_INVALID_ARG = -1
MI_ERR_OUT_OF_MEMORY = -2
MI_ERR_NO_FREE_BLOCKS = -3
MI_ERR_HIP = -4
MI_ERR_UNSUPPORTED = -5
MI_ERR_WORKSPACE_TOO_SMALL = -6
MI_ERR_DEVICE_FAULT = -7
MI_ERR_SCRATCH_TOO_SMALL = -8
MI_NOALLOC_SCRATCH_BYTES = 8 << 20

MI_FAULT_BLOCK_ID = 1
MI_FAULT_CONTEXT_LEN = 2
MI_POOL_HOST_ONLY = 1
MI_POOL_KV_FP8 = 2
MI_POOL_SWAP_STAGING = 4
MI_POOL_DECODE_DOT = 8
MI_EVICT_LIFO = 0
MI_EVICT_FIFO = 1
MI_EVICT_LRU = 2

_c = ctypes
_vp = _c.c_void_p
_i32 = _c.c_int32
_u32 = _c.c_uint32
_i64 = _c.c_int64
_sz = _c.c_size_t

# name -> (restype, argtypes); the same list as include/mikv.h
SIGNATURES = {
    "mi_status_string": (_c.c_char_p, [_c.c_int]),
    "mi_kv_pool_init": (_c.c_int, [_c.POINTER(_vp), _i32, _i32, _i32, _i32, _vp, _vp, _u32]),
    "mi_kv_pool_destroy": (_c.c_int, [_vp]),
    "mi_kv_pool_set_scales": (_c.c_int, [_vp, _vp, _vp]),
    "mi_kv_pool_quantize": (_c.c_int, [_vp, _vp, _vp, _vp]),
    "mi_kv_pool_calibrate_scales": (_c.c_int, [_vp, _vp, _vp, _i32, _c.c_float, _vp]),
    "mi_kv_pool_get_scales": (_c.c_int, [_vp, _vp, _vp]),
    "mi_kv_pool_get": (_c.c_int, [_vp, _c.POINTER(_vp), _c.POINTER(_vp)]),
    "mi_kv_pool_shape": (_c.c_int, [_vp, _c.POINTER(_i32), _c.POINTER(_i32), _c.POINTER(_i32),
                                    _c.POINTER(_i32)]),
    "mi_kv_alloc_blocks": (_c.c_int, [_vp, _i32, _c.POINTER(_i32)]),
    "mi_kv_free_blocks": (_c.c_int, [_vp, _i32, _c.POINTER(_i32)]),
    "mi_kv_num_free_blocks": (_i32, [_vp]),
    "mi_kv_blocks_needed": (_i32, [_i32, _i32]),
    "mi_kv_cache_bytes": (_c.c_uint64, [_i64, _i64, _i64, _i64, _i64]),
    "mi_kv_pool_check_errors": (_c.c_int, [_vp, _c.POINTER(_u32)]),
    "mi_write_decode_kv": (_c.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32,
                                      _c.c_double, _vp]),
    "mi_paged_gqa_decode_workspace_bytes": (_sz, [_vp, _i32, _i32, _i32]),
    "mi_paged_gqa_decode": (_c.c_int, [_vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _c.c_float,
                                       _i32, _vp, _sz, _vp]),
    "mi_paged_gqa_decode_split": (_c.c_int, [_vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32,
                                             _c.c_float, _i32, _i32, _vp, _sz, _vp]),
    "mi_paged_gqa_decode_split_workspace_bytes": (_sz, [_vp, _i32, _i32, _i32, _i32]),
    "mi_paged_gqa_decode_noalloc": (_c.c_int, [_vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32,
                                               _c.c_float, _i32, _vp]),
    "mi_hbm_stream_read": (_c.c_int, [_vp, _sz, _vp, _i32, _vp]),
    "mi_paged_gqa_decode_step": (_c.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32,
                                            _i32, _c.c_double, _c.c_float, _i32, _vp, _sz, _vp]),
    "mi_write_prefill_kv": (_c.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32,
                                       _i32, _c.c_double, _vp]),
    "mi_paged_prefill_attention": (_c.c_int, [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32,
                                              _i32, _i32, _c.c_float, _vp]),
    "mi_sched_create": (_c.c_int, [_c.POINTER(_vp), _vp, _i32, _i32, _c.c_double, _c.c_double]),
    "mi_sched_destroy": (_c.c_int, [_vp]),
    "mi_sched_submit": (_c.c_int, [_vp, _c.c_int64, _i32, _i32]),
    "mi_sched_num_waiting": (_i32, [_vp]),
    "mi_sched_num_running": (_i32, [_vp]),
    "mi_sched_step": (_c.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "mi_sched_set_swap_space": (_c.c_int, [_vp, _i32]),
    "mi_sched_set_eviction": (_c.c_int, [_vp, _i32]),
    "mi_sched_num_swapped": (_i32, [_vp]),
    "mi_kv_swap_out": (_c.c_int, [_vp, _vp, _vp, _i32, _vp, _i32, _vp]),
    "mi_kv_swap_in": (_c.c_int, [_vp, _vp, _vp, _i32, _vp, _i32, _vp]),
    "mi_gather_kv": (_c.c_int, [_vp, _vp, _i32, _vp, _i32, _i32, _vp, _vp, _i32, _vp]),
    "mi_decoder_layer_workspace_bytes": (_sz, [_vp, _vp, _i32, _i32]),
    "mi_decoder_layer_decode": (_c.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32,
                                           _vp, _sz, _vp]),
}


class MiLayerConfig(ctypes.Structure):
    _fields_ = [("hidden", _i32), ("num_q_heads", _i32), ("num_kv_heads", _i32),
                ("head_dim", _i32), ("intermediate", _i32), ("rms_eps", _c.c_float),
                ("rope_theta", _c.c_double)]


class MiLayerWeights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("ln1_w", "w_qkv", "w_o", "ln2_w", "w_gate", "w_up", "w_down")]


_LIB = None


def lib():
    """The loaded libmikv.so with argument types set. Raises if it is not built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libmikv.so is not built (%s); run "
                              "`python -m paged_kv_cache_246_amd.build`" % LIB_PATH)
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


class MikvError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__("%s failed: %d (%s)" % (fn, status, status_string(status)))
        self.status = status


def status_string(status):
    return lib().mi_status_string(status).decode()


def _check(fn, rc):
    if rc != MI_OK:
        raise MikvError(fn, rc)
    return rc


def _ptr(x):
    """Device/host address of a torch tensor, or an integer address, or None -> NULL."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ------------------------------------------------------------------ pool
def mi_kv_pool_init(num_blocks, block_size, num_kv_heads, head_dim, k_cache=None,
                    v_cache=None, flags=0):
    h = _vp()
    _check("mi_kv_pool_init", lib().mi_kv_pool_init(
        ctypes.byref(h), num_blocks, block_size, num_kv_heads, head_dim,
        _ptr(k_cache), _ptr(v_cache), flags))
    return h.value


def mi_kv_pool_destroy(pool):
    return _check("mi_kv_pool_destroy", lib().mi_kv_pool_destroy(pool))


def mi_kv_pool_set_scales(pool, k_scales=None, v_scales=None):
    """Per-KV-head scales of an 8-bit pool (host sequences of floats, or None
    for 1.0)."""
    def arr(x):
        if x is None:
            return None
        a = (ctypes.c_float * len(x))(*[float(v) for v in x])
        return a
    ka, va = arr(k_scales), arr(v_scales)
    return _check("mi_kv_pool_set_scales", lib().mi_kv_pool_set_scales(
        pool, ctypes.cast(ka, _vp) if ka is not None else None,
        ctypes.cast(va, _vp) if va is not None else None))


def mi_kv_pool_quantize(pool, k_src, v_src, stream=None):
    return _check("mi_kv_pool_quantize", lib().mi_kv_pool_quantize(
        pool, _ptr(k_src), _ptr(v_src), _stream(stream)))


def mi_kv_pool_calibrate_scales(pool, k, v, rows, margin=1.0, stream=None):
    return _check("mi_kv_pool_calibrate_scales", lib().mi_kv_pool_calibrate_scales(
        pool, _ptr(k), _ptr(v), rows, margin, _stream(stream)))


def mi_kv_pool_get_scales(pool):
    """(k_scales, v_scales) of an 8-bit pool as lists of floats."""
    hkv = mi_kv_pool_shape(pool)[2]
    ks, vs = (ctypes.c_float * hkv)(), (ctypes.c_float * hkv)()
    _check("mi_kv_pool_get_scales", lib().mi_kv_pool_get_scales(pool, ks, vs))
    return list(ks), list(vs)


def mi_kv_pool_get(pool):
    k, v = _vp(), _vp()
    _check("mi_kv_pool_get", lib().mi_kv_pool_get(pool, ctypes.byref(k), ctypes.byref(v)))
    return k.value, v.value


def mi_kv_pool_shape(pool):
    vals = [_i32() for _ in range(4)]
    _check("mi_kv_pool_shape", lib().mi_kv_pool_shape(pool, *[ctypes.byref(x) for x in vals]))
    return tuple(x.value for x in vals)


def mi_kv_alloc_blocks(pool, n):
    ids = (_i32 * max(n, 1))()
    _check("mi_kv_alloc_blocks", lib().mi_kv_alloc_blocks(pool, n, ids))
    return [ids[i] for i in range(n)]


def mi_kv_free_blocks(pool, ids):
    ids = list(ids)
    arr = (_i32 * max(len(ids), 1))(*ids)
    return _check("mi_kv_free_blocks", lib().mi_kv_free_blocks(pool, len(ids), arr))


def mi_kv_num_free_blocks(pool):
    n = lib().mi_kv_num_free_blocks(pool)
    if n < 0:
        raise MikvError("mi_kv_num_free_blocks", n)
    return n


def mi_kv_blocks_needed(num_tokens, block_size):
    n = lib().mi_kv_blocks_needed(num_tokens, block_size)
    if n < 0:
        raise MikvError("mi_kv_blocks_needed", n)
    return n


def mi_kv_cache_bytes(batch, layers, max_seq_len, num_kv_heads, head_dim):
    return lib().mi_kv_cache_bytes(batch, layers, max_seq_len, num_kv_heads, head_dim)


def mi_kv_pool_check_errors(pool):
    """Returns the fault bits (0 if none). Synchronises the device."""
    bits = _u32()
    rc = lib().mi_kv_pool_check_errors(pool, ctypes.byref(bits))
    if rc not in (MI_OK, MI_ERR_DEVICE_FAULT):
        raise MikvError("mi_kv_pool_check_errors", rc)
    return bits.value


# ------------------------------------------------------------- decode step
def mi_write_decode_kv(pool, q, k, v, q_rot, block_table, max_blocks_per_seq, context_lens,
                       batch, num_q_heads, rope_theta, stream=None):
    return _check("mi_write_decode_kv", lib().mi_write_decode_kv(
        pool, _ptr(q), _ptr(k), _ptr(v), _ptr(q_rot), _ptr(block_table), max_blocks_per_seq,
        _ptr(context_lens), batch, num_q_heads, float(rope_theta), _stream(stream)))


def mi_paged_gqa_decode_workspace_bytes(pool, batch, num_q_heads, max_context_len):
    return lib().mi_paged_gqa_decode_workspace_bytes(pool, batch, num_q_heads, max_context_len)


def mi_paged_gqa_decode_split_workspace_bytes(pool, batch, num_q_heads, max_context_len,
                                              split_tokens):
    return lib().mi_paged_gqa_decode_split_workspace_bytes(pool, batch, num_q_heads,
                                                           max_context_len, split_tokens)


def mi_paged_gqa_decode(pool, q_rot, out, block_table, max_blocks_per_seq, context_lens, batch,
                        num_q_heads, softmax_scale, max_context_len, workspace,
                        workspace_bytes, stream=None):
    return _check("mi_paged_gqa_decode", lib().mi_paged_gqa_decode(
        pool, _ptr(q_rot), _ptr(out), _ptr(block_table), max_blocks_per_seq,
        _ptr(context_lens), batch, num_q_heads, float(softmax_scale), max_context_len,
        _ptr(workspace), workspace_bytes, _stream(stream)))


def mi_paged_gqa_decode_noalloc(pool, q_rot, out, block_table, max_blocks_per_seq, context_lens,
                                batch, num_q_heads, softmax_scale, max_context_len, stream=None):
    return _check("mi_paged_gqa_decode_noalloc", lib().mi_paged_gqa_decode_noalloc(
        pool, _ptr(q_rot), _ptr(out), _ptr(block_table), max_blocks_per_seq,
        _ptr(context_lens), batch, num_q_heads, float(softmax_scale), max_context_len,
        _stream(stream)))


def mi_paged_gqa_decode_split(pool, q_rot, out, block_table, max_blocks_per_seq, context_lens,
                              batch, num_q_heads, softmax_scale, max_context_len, split_tokens,
                              workspace, workspace_bytes, stream=None):
    return _check("mi_paged_gqa_decode_split", lib().mi_paged_gqa_decode_split(
        pool, _ptr(q_rot), _ptr(out), _ptr(block_table), max_blocks_per_seq,
        _ptr(context_lens), batch, num_q_heads, float(softmax_scale), max_context_len,
        split_tokens, _ptr(workspace), workspace_bytes, _stream(stream)))


def mi_paged_gqa_decode_step(pool, q, k, v, q_rot, out, block_table, max_blocks_per_seq,
                             context_lens, batch, num_q_heads, rope_theta, softmax_scale,
                             max_context_len, workspace, workspace_bytes, stream=None):
    return _check("mi_paged_gqa_decode_step", lib().mi_paged_gqa_decode_step(
        pool, _ptr(q), _ptr(k), _ptr(v), _ptr(q_rot), _ptr(out), _ptr(block_table),
        max_blocks_per_seq, _ptr(context_lens), batch, num_q_heads, float(rope_theta),
        float(softmax_scale), max_context_len, _ptr(workspace), workspace_bytes, _stream(stream)))


def mi_write_prefill_kv(pool, q, k, v, q_rot, block_table, max_blocks_per_seq, context_lens,
                        cu_seqlens, batch, total_tokens, num_q_heads, rope_theta, stream=None):
    return _check("mi_write_prefill_kv", lib().mi_write_prefill_kv(
        pool, _ptr(q), _ptr(k), _ptr(v), _ptr(q_rot), _ptr(block_table), max_blocks_per_seq,
        _ptr(context_lens), _ptr(cu_seqlens), batch, total_tokens, num_q_heads, rope_theta,
        _stream(stream)))


def mi_paged_prefill_attention(pool, q_rot, out, block_table, max_blocks_per_seq, context_lens,
                               cu_seqlens, batch, total_tokens, max_new_tokens, num_q_heads,
                               softmax_scale=0.0, stream=None):
    return _check("mi_paged_prefill_attention", lib().mi_paged_prefill_attention(
        pool, _ptr(q_rot), _ptr(out), _ptr(block_table), max_blocks_per_seq, _ptr(context_lens),
        _ptr(cu_seqlens), batch, total_tokens, max_new_tokens, num_q_heads, softmax_scale,
        _stream(stream)))


def mi_gather_kv(pool, block_table, max_blocks_per_seq, context_lens, batch, len_extra, k_out,
                 v_out, l_max, stream=None):
    return _check("mi_gather_kv", lib().mi_gather_kv(
        pool, _ptr(block_table), max_blocks_per_seq, _ptr(context_lens), batch, len_extra,
        _ptr(k_out), _ptr(v_out), l_max, _stream(stream)))


# -------------------------------------------------------------- full layer
def layer_config(hidden, num_q_heads, num_kv_heads, head_dim, intermediate, rms_eps, rope_theta):
    return MiLayerConfig(hidden, num_q_heads, num_kv_heads, head_dim, intermediate,
                         rms_eps, rope_theta)


def layer_weights(ln1_w, w_qkv, w_o, ln2_w, w_gate, w_up, w_down):
    return MiLayerWeights(*[_ptr(x) for x in (ln1_w, w_qkv, w_o, ln2_w, w_gate, w_up, w_down)])


def mi_decoder_layer_workspace_bytes(cfg, pool, batch, max_context_len):
    return lib().mi_decoder_layer_workspace_bytes(ctypes.byref(cfg), pool, batch, max_context_len)


def mi_decoder_layer_decode(pool, cfg, weights, x_in, x_out, block_table, max_blocks_per_seq,
                            context_lens, batch, max_context_len, workspace, workspace_bytes,
                            stream=None):
    return _check("mi_decoder_layer_decode", lib().mi_decoder_layer_decode(
        pool, ctypes.byref(cfg), ctypes.byref(weights), _ptr(x_in), _ptr(x_out),
        _ptr(block_table), max_blocks_per_seq, _ptr(context_lens), batch, max_context_len,
        _ptr(workspace), workspace_bytes, _stream(stream)))


# --------------------------------------------------------- step planner
MI_BRAKE_PROCEED, MI_BRAKE_SOFT, MI_BRAKE_HARD = 0, 1, 2


class MiSchedCounts(ctypes.Structure):
    _fields_ = [("num_prefill", ctypes.c_int32), ("num_decode", ctypes.c_int32),
                ("num_preempted", ctypes.c_int32), ("num_finished", ctypes.c_int32),
                ("brake", ctypes.c_int32), ("free_blocks", ctypes.c_int32),
                ("num_swapped_out", ctypes.c_int32), ("num_swap_out", ctypes.c_int32),
                ("num_swap_in", ctypes.c_int32)]


class Scheduler:
    """Host wrapper of mi_sched_*: plans come back as numpy arrays."""

    def __init__(self, pool, max_blocks_per_seq, max_running, hard=0.10, soft=0.30,
                 host_slots=0, evict=MI_EVICT_LIFO):
        import numpy as np
        self._np = np
        h = _vp()
        _check("mi_sched_create", lib().mi_sched_create(ctypes.byref(h), pool, max_blocks_per_seq,
                                                         max_running, hard, soft))
        self.h = h.value
        self.mbps, self.max_running = max_blocks_per_seq, max_running
        R = max_running
        self.ids = np.zeros(R, np.int64)
        self.ctx = np.zeros(R, np.int32)
        self.new = np.zeros(R, np.int32)
        self.table = np.zeros((R, max_blocks_per_seq), np.int32)
        self.pre = np.zeros(R, np.int64)
        self.fin = np.zeros(R, np.int64)
        self.swp = np.zeros(R, np.int64)
        self.so = np.zeros((R * max_blocks_per_seq, 2), np.int32)
        self.si = np.zeros((R * max_blocks_per_seq, 2), np.int32)
        if host_slots:
            _check("mi_sched_set_swap_space", lib().mi_sched_set_swap_space(self.h, host_slots))
        if evict != MI_EVICT_LIFO:
            _check("mi_sched_set_eviction", lib().mi_sched_set_eviction(self.h, evict))

    def submit(self, rid, prompt, max_new):
        return _check("mi_sched_submit", lib().mi_sched_submit(self.h, rid, prompt, max_new))

    def num_waiting(self):
        return lib().mi_sched_num_waiting(self.h)

    def num_running(self):
        return lib().mi_sched_num_running(self.h)

    def num_swapped(self):
        return lib().mi_sched_num_swapped(self.h)

    def step(self):
        c = MiSchedCounts()
        ptr = lambda a: a.ctypes.data
        _check("mi_sched_step", lib().mi_sched_step(self.h, ctypes.byref(c), ptr(self.ids),
                                                     ptr(self.ctx), ptr(self.new), ptr(self.table),
                                                     ptr(self.pre), ptr(self.fin), ptr(self.swp),
                                                     ptr(self.so), ptr(self.si)))
        n = c.num_prefill + c.num_decode
        return {"num_prefill": c.num_prefill, "num_decode": c.num_decode, "brake": c.brake,
                "free_blocks": c.free_blocks, "ids": self.ids[:n].copy(),
                "context_lens": self.ctx[:n].copy(), "new_tokens": self.new[:n].copy(),
                "block_table": self.table[:n].copy(),
                "preempted": self.pre[:c.num_preempted].copy(),
                "finished": self.fin[:c.num_finished].copy(),
                "swapped_out": self.swp[:c.num_swapped_out].copy(),
                "swap_out": self.so[:c.num_swap_out].copy(),
                "swap_in": self.si[:c.num_swap_in].copy()}

    def close(self):
        if self.h:
            lib().mi_sched_destroy(self.h)
            self.h = None


def mi_kv_swap_out(pool, host_k, host_v, host_slots, pairs, stream=None):
    """pairs: numpy int32 [n, 2] (device block, host slot), host memory."""
    import numpy as np
    pr = np.ascontiguousarray(pairs, dtype=np.int32)
    return _check("mi_kv_swap_out", lib().mi_kv_swap_out(
        pool, _ptr(host_k), _ptr(host_v), host_slots, pr.ctypes.data if len(pr) else None,
        len(pr), _stream(stream)))


def mi_kv_swap_in(pool, host_k, host_v, host_slots, pairs, stream=None):
    """pairs: numpy int32 [n, 2] (host slot, device block), host memory."""
    import numpy as np
    pr = np.ascontiguousarray(pairs, dtype=np.int32)
    return _check("mi_kv_swap_in", lib().mi_kv_swap_in(
        pool, _ptr(host_k), _ptr(host_v), host_slots, pr.ctypes.data if len(pr) else None,
        len(pr), _stream(stream)))


# ------------------------------------------------------------ measurement
def mi_hbm_stream_read(src, nbytes, sink, workgroups, stream=None):
    return _check("mi_hbm_stream_read", lib().mi_hbm_stream_read(
        _ptr(src), nbytes, _ptr(sink), workgroups, _stream(stream)))
