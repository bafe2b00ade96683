"""Python binding of the mixed-batch quantized-KV attention library (libmab.so).

Argument marshalling only: every step of the attention path runs in the HIP
kernels behind the C ABI declared in ``include/mab.h``.  PyTorch provides
device memory and the current stream; nothing here computes on tensors.  The
functions carry the names of the C entry points.

If the shared library has not been built, every call raises ``RuntimeError``
(build it with ``python -m mixed_attention_block_amd.build``); there is no
fallback path.
"""

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmab.so")

MAB_KV_Q8 = 1
MAB_KV_Q4 = 2
MAB_KV_F16 = 3
FORMATS = {"q8": MAB_KV_Q8, "q4": MAB_KV_Q4, "f16": MAB_KV_F16}
MAB_BATCH_INVARIANT = 1  # batch flag: decode and verify rows bit-identical whatever shares the batch
INVARIANT_PIECE_KEYS = 512  # MAB_INVARIANT_PIECE_KEYS


class MabError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: status {status}: {mab_status_string(status)}")


class KVLayout(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("k_format", ctypes.c_int32),
                ("v_format", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class Batch(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_rows", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("q_start", ctypes.c_void_p), ("prefix_len", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("q_start_host", ctypes.c_void_p),
                ("prefix_len_host", ctypes.c_void_p)]


class SchedConfig(ctypes.Structure):
    _fields_ = [("sessions", ctypes.c_int32), ("prefill_chunk", ctypes.c_int32),
                ("max_pending_per_client", ctypes.c_int32), ("near_done_gate", ctypes.c_int32),
                ("max_decode_rows", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32)]


class StepInfo(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("num_seqs", ctypes.c_int32), ("num_rows", ctypes.c_int32),
                ("pending", ctypes.c_int32)]


_lib_handle = None


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mixed_attention_block_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        lay, bat = ctypes.POINTER(KVLayout), ctypes.POINTER(Batch)
        lib.kv_block_bytes.argtypes, lib.kv_block_bytes.restype = [i32], i32
        lib.kv_pool_bytes.argtypes, lib.kv_pool_bytes.restype = [lay, i32], i64
        lib.attention_workspace_bytes.argtypes = [lay, bat]
        lib.attention_workspace_bytes.restype = i64
        lib.kv_append_quant.argtypes = [lay, bat, P, P, P, P, P]
        lib.kv_append_quant.restype = i32
        lib.mixed_attention_fwd.argtypes = [lay, bat, P, P, P, f32, P, P, i64, P]
        lib.mixed_attention_fwd.restype = i32
        lib.mixed_attention_fwd_timed.argtypes = [lay, bat, P, P, P, f32, P, P, i64, P, P, P]
        lib.mixed_attention_fwd_timed.restype = i32
        lib.mixed_attention_fwd_noalloc.argtypes = [lay, bat, P, P, P, f32, P, P]
        lib.mixed_attention_fwd_noalloc.restype = i32
        lib.mab_status_string.argtypes, lib.mab_status_string.restype = [i32], ctypes.c_char_p
        lib.mab_debug_status.argtypes, lib.mab_debug_status.restype = [i32], i32
        lib.mab_probe_stream_read.argtypes = [P, i64, P, P]
        lib.mab_probe_stream_read.restype = i32
        lib.mab_probe_mfma_f16.argtypes, lib.mab_probe_mfma_f16.restype = [i32, P, P], i64
        lib.mab_sched_create.argtypes = [ctypes.POINTER(SchedConfig), ctypes.POINTER(P)]
        lib.mab_sched_create.restype = i32
        lib.mab_sched_destroy.argtypes, lib.mab_sched_destroy.restype = [P], None
        lib.mab_sched_submit.argtypes = [P, i32, i32, i32, ctypes.POINTER(i64)]
        lib.mab_sched_submit.restype = i32
        lib.mab_sched_step.argtypes = [P, ctypes.POINTER(StepInfo), P, P, P, P, P, P, i32]
        lib.mab_sched_step.restype = i32
        _lib_handle = lib
    return _lib_handle


def make_layout(num_q_heads, num_kv_heads, head_dim, page_size, num_pages, k_format="q8",
                v_format="q8"):
    """A ``KVLayout``; formats are "q8"/"q4"/"f16" or the MAB_KV_* integers."""
    kf = FORMATS.get(k_format, k_format)
    vf = FORMATS.get(v_format, v_format)
    return KVLayout(num_q_heads, num_kv_heads, head_dim, page_size, num_pages, kf, vf, 0)


class BatchDesc:
    """A ``Batch`` plus the objects whose memory it points to (kept alive here).

    ``q_start``, ``prefix_len``, ``block_table``: int32 device tensors;
    ``q_start_host``, ``prefix_len_host``: int32 host arrays with the same values.
    """

    def __init__(self, q_start, prefix_len, block_table, q_start_host, prefix_len_host, flags=0):
        self._keep = [q_start, prefix_len, block_table,
                      np.ascontiguousarray(q_start_host, dtype=np.int32),
                      np.ascontiguousarray(prefix_len_host, dtype=np.int32)]
        for t in (q_start, prefix_len, block_table):
            _check_tensor(t, "int32", "descriptor")
        qh, ph = self._keep[3], self._keep[4]
        num_seqs = len(ph)
        if len(qh) != num_seqs + 1:
            raise ValueError("q_start_host must have num_seqs + 1 entries")
        max_pages = block_table.shape[-1] if block_table.dim() == 2 else max(1, block_table.numel())
        self.struct = Batch(num_seqs, int(qh[-1]) if num_seqs else 0, int(max_pages), int(flags),
                            q_start.data_ptr(), prefix_len.data_ptr(), block_table.data_ptr(),
                            qh.ctypes.data, ph.ctypes.data)


def _check_tensor(t, dtype, name):
    if not t.is_contiguous():
        raise ValueError(f"{name}: tensor must be contiguous")
    if str(t.dtype).split(".")[-1] != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: expected a device tensor")


def _stream_handle(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def kv_block_bytes(fmt):
    return _lib().kv_block_bytes(FORMATS.get(fmt, fmt))


def kv_pool_bytes(layout, fmt):
    return _lib().kv_pool_bytes(ctypes.byref(layout), FORMATS.get(fmt, fmt))


def attention_workspace_bytes(layout, batch):
    n = _lib().attention_workspace_bytes(ctypes.byref(layout), ctypes.byref(batch.struct))
    if n < 0:
        raise MabError(-n, "attention_workspace_bytes")
    return n


def kv_append_quant(layout, batch, k_new, v_new, k_pool, v_pool, stream=None):
    """Quantize the rows' new K/V into the pools (device tensors, in place)."""
    _check_tensor(k_new, "float16", "k_new")
    _check_tensor(v_new, "float16", "v_new")
    _check_tensor(k_pool, "uint8", "k_pool")
    _check_tensor(v_pool, "uint8", "v_pool")
    st = _lib().kv_append_quant(ctypes.byref(layout), ctypes.byref(batch.struct),
                                k_new.data_ptr(), v_new.data_ptr(), k_pool.data_ptr(),
                                v_pool.data_ptr(), _stream_handle(stream))
    if st:
        raise MabError(st, "kv_append_quant")


def mixed_attention_fwd(layout, batch, q, k_pool, v_pool, sm_scale, out, workspace, stream=None):
    """One attention step of the mixed batch; writes ``out`` (fp32)."""
    _check_tensor(q, "float16", "q")
    _check_tensor(k_pool, "uint8", "k_pool")
    _check_tensor(v_pool, "uint8", "v_pool")
    _check_tensor(out, "float32", "out")
    _check_tensor(workspace, "uint8", "workspace")
    st = _lib().mixed_attention_fwd(ctypes.byref(layout), ctypes.byref(batch.struct),
                                    q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                    float(sm_scale), out.data_ptr(), workspace.data_ptr(),
                                    workspace.numel(), _stream_handle(stream))
    if st:
        raise MabError(st, "mixed_attention_fwd")


def mixed_attention_fwd_timed(layout, batch, q, k_pool, v_pool, sm_scale, out, workspace, kernel_start,
                              kernel_stop, stream=None):
    """mixed_attention_fwd that also records the torch.cuda.Event pair
    ``kernel_start``/``kernel_stop`` right before and after its attention
    kernel (before the merge kernels): their elapsed time is that kernel's."""
    _check_tensor(q, "float16", "q")
    _check_tensor(k_pool, "uint8", "k_pool")
    _check_tensor(v_pool, "uint8", "v_pool")
    _check_tensor(out, "float32", "out")
    _check_tensor(workspace, "uint8", "workspace")
    handles = []
    for ev in (kernel_start, kernel_stop):
        if ev.cuda_event == 0:  # torch creates the event lazily, at its first record
            ev.record(stream)
        handles.append(ctypes.c_void_p(ev.cuda_event))
    st = _lib().mixed_attention_fwd_timed(ctypes.byref(layout), ctypes.byref(batch.struct),
                                          q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                          float(sm_scale), out.data_ptr(), workspace.data_ptr(),
                                          workspace.numel(), _stream_handle(stream), *handles)
    if st:
        raise MabError(st, "mixed_attention_fwd_timed")


NOALLOC_SCRATCH_BYTES = 128 << 20  # MAB_NOALLOC_SCRATCH_BYTES


def mixed_attention_fwd_noalloc(layout, batch, q, k_pool, v_pool, sm_scale, out, stream=None):
    """mixed_attention_fwd with the library's fixed per-device scratch array
    as workspace (no allocation; overlapping calls on one device race)."""
    _check_tensor(q, "float16", "q")
    _check_tensor(k_pool, "uint8", "k_pool")
    _check_tensor(v_pool, "uint8", "v_pool")
    _check_tensor(out, "float32", "out")
    st = _lib().mixed_attention_fwd_noalloc(ctypes.byref(layout), ctypes.byref(batch.struct),
                                            q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                            float(sm_scale), out.data_ptr(), _stream_handle(stream))
    if st:
        raise MabError(st, "mixed_attention_fwd_noalloc")


def mab_status_string(status):
    return _lib().mab_status_string(int(status)).decode()


def mab_debug_status(reset=True):
    """1 if a kernel met an out-of-range page id since the last reset (checked
    only while MAB_DEBUG=1 is set in the environment), else 0."""
    st = _lib().mab_debug_status(1 if reset else 0)
    if st < 0:
        raise MabError(-st, "mab_debug_status")
    return st


def mab_probe_stream_read(buf, sink, stream=None):
    """Enqueue one stream read of the device tensor ``buf`` (its whole storage)."""
    nbytes = buf.numel() * buf.element_size()
    st = _lib().mab_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), _stream_handle(stream))
    if st:
        raise MabError(st, "mab_probe_stream_read")
    return nbytes


def mab_probe_mfma_f16(iters, sink, stream=None):
    """Enqueue the dense fp16 matrix-core probe; returns the flops enqueued."""
    n = _lib().mab_probe_mfma_f16(int(iters), sink.data_ptr(), _stream_handle(stream))
    if n < 0:
        raise MabError(-n, "mab_probe_mfma_f16")
    return n


MAB_ERR_QUOTA = 7
STEP_KINDS = {0: None, 1: "decode", 2: "merged"}


class Step:
    """One tick of ``Scheduler.step``: host int32 arrays of the step's batch
    (``q_start``, ``prefix_len``, ``block_table``) plus ``request_id``, ``emit``
    and ``finished`` per sequence."""

    def __init__(self, kind, request_id, q_start, prefix_len, block_table, emit, finished, pending):
        self.kind = kind
        self.request_id = request_id
        self.q_start = q_start
        self.prefix_len = prefix_len
        self.block_table = block_table
        self.emit = emit
        self.finished = finished
        self.pending = pending

    @property
    def num_seqs(self):
        return len(self.prefix_len)

    @property
    def q_len(self):
        return np.diff(self.q_start)

    def batch(self, device="cuda"):
        """The step's ``BatchDesc`` with device copies of the descriptor."""
        import torch
        dev = [torch.from_numpy(np.ascontiguousarray(a)).to(device)
               for a in (self.q_start, self.prefix_len, self.block_table)]
        return BatchDesc(dev[0], dev[1], dev[2], self.q_start, self.prefix_len)


class Scheduler:
    """The library's step scheduler (``mab_sched_*``): submit requests, then
    call ``step()`` once per engine tick."""

    def __init__(self, sessions, prefill_chunk, max_pending_per_client, near_done_gate, page_size,
                 num_pages, max_pages_per_seq, max_decode_rows=0):
        self.config = SchedConfig(sessions, prefill_chunk, max_pending_per_client, near_done_gate,
                                  max_decode_rows, page_size, num_pages, max_pages_per_seq)
        lib = _lib()
        handle = ctypes.c_void_p()
        st = lib.mab_sched_create(ctypes.byref(self.config), ctypes.byref(handle))
        if st:
            raise MabError(st, "mab_sched_create")
        self._h = handle
        self._lib = lib
        self.capacity = (max_decode_rows or sessions) + 1
        cap, width = self.capacity, max_pages_per_seq
        self._ids = np.zeros(cap, np.int64)
        self._qs = np.zeros(cap + 1, np.int32)
        self._pl = np.zeros(cap, np.int32)
        self._bt = np.zeros(cap * width, np.int32)
        self._emit = np.zeros(cap, np.int32)
        self._fin = np.zeros(cap, np.int32)
        self._info = StepInfo()

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.mab_sched_destroy(h)
            self._h = None

    def submit(self, client, prompt_len, token_limit):
        """Returns (status, request id): status 0, or MAB_ERR_QUOTA (7) / 2
        with id -1.  Other failures raise."""
        rid = ctypes.c_int64(-1)
        st = self._lib.mab_sched_submit(self._h, client, prompt_len, token_limit, ctypes.byref(rid))
        if st not in (0, 2, MAB_ERR_QUOTA):
            raise MabError(st, "mab_sched_submit")
        return st, rid.value

    def step(self):
        """One tick; None when there is nothing to run, else a ``Step``."""
        st = self._lib.mab_sched_step(self._h, ctypes.byref(self._info), self._ids.ctypes.data,
                                      self._qs.ctypes.data, self._pl.ctypes.data, self._bt.ctypes.data,
                                      self._emit.ctypes.data, self._fin.ctypes.data, self.capacity)
        if st:
            raise MabError(st, "mab_sched_step")
        info = self._info
        if info.kind == 0:
            return None
        n, width = info.num_seqs, self.config.max_pages_per_seq
        return Step(STEP_KINDS[info.kind], self._ids[:n].copy(), self._qs[:n + 1].copy(),
                    self._pl[:n].copy(), self._bt[:n * width].reshape(n, width).copy(),
                    self._emit[:n].copy(), self._fin[:n].copy(), info.pending)
