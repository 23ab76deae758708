"""Thin ctypes binding of libtk (include/tk.h).

Argument marshalling only: every step of a training step runs in the HIP
library.  PyTorch supplies device memory and the current stream.  The names
follow the C ABI: ``compile`` (tk_compile), ``Program.query``, ``allocate``,
``validate_into``, ``run_into``, ``__call__`` -- the execution boundary of the
trainkernel pages (runtime.py: ``compile_program``, ``CompiledProgram``,
``ExecutionBuffers``).
"""
from __future__ import annotations

import ctypes
import os
import sys
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtk.so")

TK_F32, TK_F16, TK_BF16, TK_I8 = 0, 1, 2, 3
TK_E_ABORTED = 12
DTYPE_CODES = {"f32": TK_F32, "f16": TK_F16, "bf16": TK_BF16, "i8": TK_I8}
STATUS = {0: "TK_OK", 1: "TK_E_ARG", 2: "TK_E_PARSE", 3: "TK_E_UNSUPPORTED", 4: "TK_E_SHAPE", 5: "TK_E_STRIDE",
          6: "TK_E_DTYPE", 7: "TK_E_DEVICE", 8: "TK_E_ALIAS", 9: "TK_E_WORKSPACE", 10: "TK_E_COUNT",
          11: "TK_E_HIP", 12: "TK_E_ABORTED"}


class TkTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 8), ("strides", ctypes.c_int64 * 8),
                ("storage_base", ctypes.c_void_p), ("storage_bytes", ctypes.c_uint64),
                ("device", ctypes.c_int32), ("requires_grad", ctypes.c_int32)]


class TkOptions(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "blocks_per_cu", "max_blocks", "fuse_pointwise", "fuse_epilogues", "inline_input_casts",
        "split_k_gemv", "threads_per_block", "fuse_updates", "barrier_every_op", "num_cus",
        "gemm_split_k", "force_grid", "launch_mode", "gemm_tile", "batch_epilogues", "colsum_fusion")]


STATS_FIELDS = ["n_stages", "grid_barriers", "materialized_ops", "inlined_ops", "fused_epilogues",
                "side_epilogues", "fused_updates", "matrix_core_ops", "direct_outputs", "direct_state_commits",
                "staged_commits", "grid_size", "max_work_items", "num_cus", "blocks_per_cu", "occupancy",
                "vgprs", "sgprs", "lds_bytes", "scratch_bytes", "n_tasks"]


class TkStats(ctypes.Structure):
    _fields_ = [("workspace_bytes", ctypes.c_uint64)] + [(n, ctypes.c_int32) for n in STATS_FIELDS] + \
               [("reserved", ctypes.c_int32 * 5)]


ALLOC_FN = ctypes.CFUNCTYPE(ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32)

_lib = None


class TkError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status
        self.status_name = STATUS.get(status, str(status))


def lib():
    """Load libtk.so; fails loudly when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libtk.so is not built ({LIB_PATH}); run persistent_whole_step_amd.build")
        # PyTorch ships its own HIP runtime library.  Import it first, so that
        # libtk binds to that same runtime: loading libtk first would bring in
        # a second copy of the runtime, which then finds no device.
        import torch  # noqa: F401
        l = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        l.tk_default_options.argtypes = [P(TkOptions)]
        l.tk_compile.argtypes = [ctypes.c_char_p, ctypes.c_size_t, P(TkOptions), ctypes.c_int32, P(ctypes.c_void_p)]
        l.tk_query.argtypes = [ctypes.c_void_p, P(TkStats)]
        l.tk_dump_plan.argtypes = [ctypes.c_void_p, ctypes.c_char_p, ctypes.c_size_t, P(ctypes.c_size_t)]
        l.tk_plan_bytes.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, P(ctypes.c_size_t)]
        l.tk_allocate.argtypes = [ctypes.c_void_p, P(TkTensor), ctypes.c_size_t, ALLOC_FN, ctypes.c_void_p,
                                  P(TkTensor), ctypes.c_size_t, P(TkTensor), ctypes.c_void_p]
        l.tk_validate_into.argtypes = [ctypes.c_void_p, P(TkTensor), ctypes.c_size_t, P(TkTensor), ctypes.c_size_t,
                                       P(TkTensor)]
        l.tk_run_into.argtypes = [ctypes.c_void_p, P(TkTensor), ctypes.c_size_t, P(TkTensor), ctypes.c_size_t,
                                  P(TkTensor), ctypes.c_void_p]
        l.tk_run_into_noalloc.argtypes = [ctypes.c_void_p, P(TkTensor), ctypes.c_size_t, P(TkTensor),
                                          ctypes.c_size_t, ctypes.c_void_p]
        l.tk_workspace_init.argtypes = [ctypes.c_void_p, P(TkTensor), ctypes.c_void_p]
        l.tk_workspace_status.argtypes = [P(TkTensor), ctypes.c_void_p, P(ctypes.c_int32), P(ctypes.c_int32)]
        l.tk_set_debug.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64]
        l.tk_read_timestamps.argtypes = [ctypes.c_void_p, P(TkTensor), ctypes.c_void_p, P(ctypes.c_uint64),
                                         ctypes.c_size_t]
        l.tk_destroy.argtypes = [ctypes.c_void_p]
        l.tk_destroy.restype = None
        l.tk_last_error.restype = ctypes.c_char_p
        for f in ("tk_compile", "tk_query", "tk_dump_plan", "tk_plan_bytes", "tk_allocate", "tk_validate_into",
                  "tk_run_into", "tk_run_into_noalloc",
                  "tk_workspace_init", "tk_workspace_status", "tk_set_debug", "tk_read_timestamps"):
            getattr(l, f).restype = ctypes.c_int
        _lib = l
    return _lib


def _check(status: int):
    if status != 0:
        raise TkError(status, lib().tk_last_error().decode())


def options(**kw) -> TkOptions:
    o = TkOptions()
    lib().tk_default_options(ctypes.byref(o))
    for k, v in kw.items():
        setattr(o, k, int(v))
    return o


# ---------------------------------------------------------------- tensors --

def _torch_dtype_code(t) -> int:
    import torch
    m = {torch.float32: TK_F32, torch.float16: TK_F16, torch.bfloat16: TK_BF16, torch.int8: TK_I8}
    if t.dtype not in m:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return m[t.dtype]


def tensor_from_storage(a, dt: str, device="cuda:0"):
    """Device tensor holding numpy storage `a` of program dtype `dt` (bf16 is
    carried as uint16 bit patterns).  Argument marshalling only."""
    import numpy as np
    import torch
    if dt == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def storage_from_tensor(t, dt: str):
    """Host numpy storage of a tensor of program dtype `dt` (bf16 as uint16)."""
    import numpy as np
    import torch
    t = t.detach().cpu()
    if dt == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def describe(t, raw_bytes: bool = False) -> TkTensor:
    """A tk_tensor for a torch tensor (storage extent used for aliasing).
    raw_bytes: a uint8 workspace, described as bytes (TK_I8); otherwise uint8
    is rejected, since no program value is unsigned."""
    import torch
    d = TkTensor()
    d.data = t.data_ptr() if t.numel() else 0
    if raw_bytes:
        if t.dtype != torch.uint8:
            raise TypeError(f"workspace must be a uint8 byte tensor, got {t.dtype}")
        d.dtype = TK_I8
    else:
        d.dtype = _torch_dtype_code(t)
    d.ndim = t.dim()
    for i, (s, st) in enumerate(zip(t.shape, t.stride())):
        d.shape[i] = s
        d.strides[i] = st
    st = t.untyped_storage()
    d.storage_base = st.data_ptr() if st.nbytes() else 0
    d.storage_bytes = st.nbytes()
    d.device = t.device.index if t.device.type == "cuda" else -2
    d.requires_grad = int(bool(t.requires_grad))
    return d


def describe_fake(shape, dtype: str, data: int, device: int = 0, strides=None, storage=None) -> TkTensor:
    """A tk_tensor for an arbitrary (never dereferenced) address: CPU tests of
    the validation rules."""
    d = TkTensor()
    d.data = data
    d.dtype = DTYPE_CODES[dtype]
    d.ndim = len(shape)
    if strides is None:
        strides, acc = [], 1
        for s in reversed(shape):
            strides.insert(0, acc)
            acc *= max(1, s)
    for i, (s, st) in enumerate(zip(shape, strides)):
        d.shape[i] = s
        d.strides[i] = st
    if storage is not None:
        d.storage_base, d.storage_bytes = storage
    d.device = device
    return d


def _array(descs):
    arr = (TkTensor * max(1, len(descs)))()
    for i, x in enumerate(descs):
        arr[i] = x
    return arr


def _stream_handle(stream=None):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


@dataclass
class ExecutionBuffers:
    """Caller-owned outputs and workspace.  Reuse only when previous work on
    them is ordered (same stream or synchronised)."""
    outputs: tuple
    workspace: object


class Program:
    """One compiled whole-step program (tk_program)."""

    def __init__(self, handle, text: str, device: int):
        self._h = handle
        self.text = text
        self.device = device
        self._outputs = None

    def __del__(self, _finalizing=sys.is_finalizing):
        # At interpreter shutdown the HIP runtime (and a profiler's tool
        # library) may already be torn down: device calls from a finaliser
        # then crash the process.  Programs still alive then are left to the
        # process exit; close() releases one deterministically.
        if _finalizing():
            return
        self.close()

    def close(self):
        """tk_destroy: free the program's plan (no launch may be running)."""
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.tk_destroy(h)
        self._h = None

    # ---------------------------------------------------------- queries --
    def query(self) -> dict:
        s = TkStats()
        _check(lib().tk_query(self._h, ctypes.byref(s)))
        d = {"workspace_bytes": s.workspace_bytes}
        for n in STATS_FIELDS:
            d[n] = getattr(s, n)
        return d

    def dump(self) -> str:
        need = ctypes.c_size_t(0)
        _check(lib().tk_dump_plan(self._h, None, 0, ctypes.byref(need)))
        buf = ctypes.create_string_buffer(need.value)
        _check(lib().tk_dump_plan(self._h, buf, need.value, None))
        return buf.value.decode()

    def plan_bytes(self) -> bytes:
        """tk_plan_bytes: the device plan as uploaded (csrc/plan.h layout)."""
        need = ctypes.c_size_t(0)
        _check(lib().tk_plan_bytes(self._h, None, 0, ctypes.byref(need)))
        buf = ctypes.create_string_buffer(max(1, need.value))
        _check(lib().tk_plan_bytes(self._h, buf, need.value, None))
        return buf.raw[:need.value]

    def resource_usage(self) -> dict:
        q = self.query()
        return {"vgprs_per_thread": q["vgprs"], "scratch_bytes_per_thread": q["scratch_bytes"],
                "lds_bytes_per_block": q["lds_bytes"], "resident_blocks_per_cu": q["occupancy"]}

    def set_debug(self, timestamps: bool = False, stagger_seed: int = 0, deadline_ticks: int = 0):
        _check(lib().tk_set_debug(self._h, int(timestamps), int(stagger_seed), int(deadline_ticks)))

    # ------------------------------------------------------- execution --
    def _output_specs(self):
        if self._outputs is None:
            import torch
            tmap = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "i8": torch.int8}
            outs = []
            for line in self.text.splitlines():
                tok = line.split(";")[0].split()
                if tok and tok[0] == "out":
                    _, dt, shape, _, _ = tok[1].split(":")
                    shp = () if shape == "-" else tuple(int(v) for v in shape.split("x"))
                    outs.append((shp, tmap[dt]))
            self._outputs = outs
        return self._outputs

    def allocate(self, *inputs) -> ExecutionBuffers:
        """Outputs (in-place slots bind their input) and an initialised workspace."""
        import torch
        keep = []

        @ALLOC_FN
        def _alloc(ctx, nbytes, device):
            t = torch.empty(max(1, int(nbytes)), dtype=torch.uint8, device=f"cuda:{device}")
            keep.append(t)
            return t.data_ptr()

        n_out = len(self._output_specs())
        ins = _array([describe(t) for t in inputs])
        outs = _array([TkTensor() for _ in range(n_out)])
        ws = TkTensor()
        _check(lib().tk_allocate(self._h, ins, len(inputs), _alloc, None, outs, n_out, ctypes.byref(ws),
                                 _stream_handle()))
        # Re-wrap the raw allocations as typed tensors (same storage).
        result = []
        inplace = self._inplace_map()
        k = 0
        for slot, (shape, dt) in enumerate(self._output_specs()):
            if slot in inplace:
                result.append(inputs[inplace[slot]])
                continue
            raw = keep[k]
            k += 1
            n = 1
            for s in shape:
                n *= s
            result.append(raw.view(dt)[:n].view(shape) if n else raw.view(dt)[:0].view(shape))
        wst = keep[k]
        return ExecutionBuffers(tuple(result), wst)

    def _inplace_map(self):
        m = {}
        for line in self.text.splitlines():
            tok = line.split(";")[0].split()
            if tok and tok[0] == "inplace":
                m[int(tok[1])] = int(tok[2])
        return m

    def _descs(self, inputs, buffers):
        ins = _array([describe(t) for t in inputs])
        outs = _array([describe(t) for t in buffers.outputs])
        ws = describe(buffers.workspace, raw_bytes=True)
        return ins, outs, ws

    def validate_into(self, *inputs, buffers: ExecutionBuffers):
        ins, outs, ws = self._descs(inputs, buffers)
        _check(lib().tk_validate_into(self._h, ins, len(inputs), outs, len(buffers.outputs), ctypes.byref(ws)))

    def init_workspace(self, workspace, stream=None):
        ws = describe(workspace, raw_bytes=True)
        _check(lib().tk_workspace_init(self._h, ctypes.byref(ws), _stream_handle(stream)))

    def run_into(self, *inputs, buffers: ExecutionBuffers, stream=None):
        for t in inputs:
            if t.is_neg() or t.is_conj():
                raise ValueError("tk: resolve lazy negative or conjugate input views before execution")
        ins, outs, ws = self._descs(inputs, buffers)
        _check(lib().tk_run_into(self._h, ins, len(inputs), outs, len(buffers.outputs), ctypes.byref(ws),
                                 _stream_handle(stream)))
        inplace = self._inplace_map()
        if inplace:
            import torch
            torch.autograd.graph.increment_version([inputs[i] for i in inplace.values()])
        return buffers.outputs

    def run_into_noalloc(self, *inputs, outputs, stream=None):
        """tk_run_into_noalloc: run in the library's static per-device
        workspace; `outputs` are caller tensors as for run_into (in-place
        slots are their input tensors).  Nothing is allocated."""
        for t in inputs:
            if t.is_neg() or t.is_conj():
                raise ValueError("tk: resolve lazy negative or conjugate input views before execution")
        ins = _array([describe(t) for t in inputs])
        outs = _array([describe(t) for t in outputs])
        _check(lib().tk_run_into_noalloc(self._h, ins, len(inputs), outs, len(outputs), _stream_handle(stream)))
        inplace = self._inplace_map()
        if inplace:
            import torch
            torch.autograd.graph.increment_version([inputs[i] for i in inplace.values()])
        return tuple(outputs)

    def __call__(self, *inputs):
        """Allocate fresh buffers, run, wait for the step and check that it
        completed: a launch that stopped at a timed-out grid barrier raises
        TkError (TK_E_ABORTED) instead of returning partial outputs."""
        bufs = self.allocate(*inputs)
        outs = self.run_into(*inputs, buffers=bufs)
        self.check_workspace(bufs.workspace)
        return outs

    def check_workspace(self, workspace, stream=None):
        """Synchronise `stream` and raise TkError (TK_E_ABORTED) when a launch
        on `workspace` stopped at a timed-out grid barrier."""
        aborted, stage = self.workspace_status(workspace, stream)
        if aborted:
            raise TkError(TK_E_ABORTED, f"tk: a launch stopped at a grid barrier that timed out (stage {stage}); "
                                        "its outputs are incomplete")

    def workspace_status(self, workspace, stream=None):
        ws = describe(workspace, raw_bytes=True)
        a, s = ctypes.c_int32(0), ctypes.c_int32(0)
        _check(lib().tk_workspace_status(ctypes.byref(ws), _stream_handle(stream), ctypes.byref(a), ctypes.byref(s)))
        return bool(a.value), s.value

    def read_timestamps(self, workspace, stream=None):
        n = 4 * self.query()["n_stages"]
        ws = describe(workspace, raw_bytes=True)
        arr = (ctypes.c_uint64 * max(1, n))()
        _check(lib().tk_read_timestamps(self._h, ctypes.byref(ws), _stream_handle(stream), arr, n))
        return list(arr)[:n]


def compile(text: str, device: int = 0, opts: TkOptions | None = None, **kw) -> Program:
    """tk_compile.  device=-1 compiles a plan only (no GPU needed)."""
    if opts is None:
        opts = options(**kw)
    h = ctypes.c_void_p()
    raw = text.encode()
    _check(lib().tk_compile(raw, len(raw), ctypes.byref(opts), int(device), ctypes.byref(h)))
    prog = Program(h, text, device)
    prog.launch_mode = int(opts.launch_mode)
    return prog


class StepGraph:
    """A captured sequence of whole-step launches, replayed as one unit.

    The steady-state loop of the runtime page's graph-replayed benchmark (README,
    Benchmark section: state feedback over resident batches): one launch per
    (inputs, buffers) variant, captured once on a private stream, then replayed
    any number of times.  Parameters updated in place feed the next replay.
    Every variant's tensors must stay alive and unmoved while the graph exists.
    The program must use launch_mode=1 (ordinary launches are capturable;
    cooperative ones are not), and its workspace must be initialised before
    capture (tk_allocate does it).  Nothing in a step clears memory with a
    memset node."""

    def __init__(self, program: "Program", variants):
        import torch
        if getattr(program, "launch_mode", 0) != 1:
            raise ValueError("tk: graph capture needs a program compiled with launch_mode=1")
        self.program = program
        self.variants = list(variants)
        self._graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(self._graph):
            for ins, bufs in self.variants:
                program.run_into(*ins, buffers=bufs)

    def replay(self):
        """Enqueue every captured step on the current stream."""
        self._graph.replay()

    @property
    def steps(self) -> int:
        return len(self.variants)


def validate_fake(prog: Program, inputs, outputs, workspace):
    """tk_validate_into on hand-made descriptors (no memory touched)."""
    ins = _array(inputs)
    outs = _array(outputs)
    _check(lib().tk_validate_into(prog._h, ins, len(inputs), outs, len(outputs), ctypes.byref(workspace)))
