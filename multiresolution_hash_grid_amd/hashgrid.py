"""Thin Python binding of libhashgrid (include/hashgrid.h).

Argument marshalling only: every step of the encoding runs in the HIP kernels
of the library.  PyTorch provides device memory and the current stream.  The
functions carry the C names and raise ``HashGridError`` with the library's
message when a call returns a negative code.  There is no fallback: if the
library is not built, loading it fails loudly.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import threading
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_PKG, "libhashgrid.so")

HG_OK, HG_EINVAL, HG_EUNSUPPORTED, HG_EHIP = 0, -1, -2, -3
HG_F32, HG_F16 = 0, 1
(HG_TUNE_FWD_LANES, HG_TUNE_BWD_LANES, HG_TUNE_CHUNK_POINTS, HG_TUNE_XCD_MAP, HG_TUNE_BWD_BINNED,
 HG_TUNE_FWD_UNROLL, HG_TUNE_FWD_NT, HG_TUNE_FWD_STAGED, HG_TUNE_BWD_PART_LOG2,
 HG_TUNE_BWD_GROUP_MIB, HG_TUNE_BWD_DENSE, HG_TUNE_FWD_SPLIT_KIB, HG_TUNE_FWD_DENSE,
 HG_TUNE_FWD_ORDER) = range(14)
_DTYPES = {"f32": HG_F32, "f16": HG_F16}
_TORCH_DTYPES = {HG_F32: torch.float32, HG_F16: torch.float16}


HG_ADAM_ZERO_GRAD = 1


class HashGridError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"hashgrid error {code}: {message}")
        self.code = code


class _Config(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "n_dims", "n_levels", "n_features", "log2_table_size", "base_resolution",
        "finest_resolution", "table_dtype", "grad_dtype")]


class _Adam(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("step", ctypes.c_int32)]


class _MlpParams(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in ("w1", "b1", "w2", "b2", "w3", "b3")] + [("coord_inputs", ctypes.c_int32)]


class _MlpGrads(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in ("dw1", "db1", "dw2", "db2", "dw3", "db3")]


MLP_SHAPES = {"w1": (64, 32), "b1": (64,), "w2": (64, 64), "b2": (64,), "w3": (4, 64), "b3": (4,)}
MLP_COORDS = 3  # raw coordinates the TinyNeRF head puts before the encoding


def mlp_shapes(coord_inputs: int = 0) -> dict:
    """Parameter shapes of the MLP head: the NeRFace head (coord_inputs = 0,
    W1 [64, 32]) or the TinyNeRF head (coord_inputs = 3, input [x, e], W1
    [64, 35])."""
    if coord_inputs not in (0, MLP_COORDS):
        raise ValueError(f"coord_inputs must be 0 or {MLP_COORDS}")
    return dict(MLP_SHAPES, w1=(64, 32 + coord_inputs))


@dataclass(frozen=True)
class HashGridConfig:
    """Grid description; defaults are the pages' standard grid (L=16, F=2,
    T=2^19, N_min=16, N_max=512)."""
    n_levels: int = 16
    n_features: int = 2
    log2_table_size: int = 19
    base_resolution: int = 16
    finest_resolution: int = 512
    table_dtype: str = "f32"
    grad_dtype: str = "f32"
    n_dims: int = 3

    @property
    def table_size(self) -> int:
        return 1 << self.log2_table_size

    @property
    def out_features(self) -> int:
        return self.n_levels * self.n_features

    @property
    def table_shape(self) -> tuple:
        return (self.n_levels, self.table_size, self.n_features)

    @property
    def torch_table_dtype(self) -> torch.dtype:
        return _TORCH_DTYPES[_DTYPES[self.table_dtype]]

    @property
    def torch_grad_dtype(self) -> torch.dtype:
        """Element type of the table gradient buffer (binary16 only on the
        binned backward, which then rounds each entry once)."""
        return _TORCH_DTYPES[_DTYPES[self.grad_dtype]]

    def c(self) -> _Config:
        return _Config(self.n_dims, self.n_levels, self.n_features, self.log2_table_size,
                       self.base_resolution, self.finest_resolution,
                       _DTYPES.get(self.table_dtype, -1), _DTYPES.get(self.grad_dtype, -1))

    @staticmethod
    def of(w) -> "HashGridConfig":
        """Config of a workload from ``multiresolution_hash_grid_amd.inputs``."""
        return HashGridConfig(w.n_levels, w.n_features, w.log2_table_size, w.base_resolution,
                              w.finest_resolution, w.table_dtype, n_dims=getattr(w, "n_dims", 3))


_lock = threading.Lock()
_lib = None


def load_library(path: str = LIBRARY_PATH) -> ctypes.CDLL:
    """Load the built library; raises if it is missing (build it with
    ``python -m multiresolution_hash_grid_amd.build``)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError(f"{path} is not built; run python -m multiresolution_hash_grid_amd.build")
            lib = ctypes.CDLL(path)
            P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
            C = ctypes.POINTER(_Config)
            sigs = {
                "hashgrid_abi_version": ([], ctypes.c_int),
                "hashgrid_last_error": ([], ctypes.c_char_p),
                "hashgrid_resolutions": ([C, P], ctypes.c_int),
                "hashgrid_forward": ([C, P, I64, P, P, I64, P, ctypes.c_size_t, P], ctypes.c_int),
                "hashgrid_forward_workspace_size": ([C, I64, P], ctypes.c_int),
                "hashgrid_backward": ([C, P, I64, P, I64, P, P, ctypes.c_size_t, P], ctypes.c_int),
                "hashgrid_backward_workspace_size": ([C, I64, P, P], ctypes.c_int),
                "hashgrid_backward_noalloc": ([C, P, I64, P, I64, P, P], ctypes.c_int),
                "hashgrid_debug_corners": ([C, P, I64, P, P, P], ctypes.c_int),
                "hashgrid_input_grad": ([C, P, I64, P, P, I64, P, P, ctypes.c_size_t, P], ctypes.c_int),
                "hashgrid_input_grad_workspace_size": ([C, I64, P], ctypes.c_int),
                "hashgrid_mlp_workspace_size": ([C, I64, P, P], ctypes.c_int),
                "hashgrid_mlp_forward": ([C, P, I64, P, ctypes.POINTER(_MlpParams), P, P, ctypes.c_size_t, P],
                                         ctypes.c_int),
                "hashgrid_mlp_backward": ([C, P, I64, P, ctypes.POINTER(_MlpParams), P, ctypes.POINTER(_MlpGrads),
                                           P, P, ctypes.c_size_t, P], ctypes.c_int),
                "hashgrid_adam_step": ([ctypes.POINTER(_Adam), I64, P, P, P, P, P, I32, P], ctypes.c_int),
                "hashgrid_tune": ([ctypes.c_int, ctypes.c_int], ctypes.c_int),
                "hashgrid_tune_get": ([ctypes.c_int], ctypes.c_int),
            }
            for name, (args, res) in sigs.items():
                fn = getattr(lib, name)
                fn.argtypes = args
                fn.restype = res
            del I32
            _lib = lib
    return _lib


def _check(rc: int) -> None:
    if rc != HG_OK:
        raise HashGridError(rc, load_library().hashgrid_last_error().decode())


def _stream(t: torch.Tensor, stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _keep_for_stream(t: torch.Tensor, stream, *bufs) -> None:
    """Buffers a wrapper allocated come from torch's caching allocator on the
    current stream.  When the kernels run on another stream, mark them used
    there so that the allocator does not hand them to a later allocation
    before that stream's work is done."""
    if stream is None:
        return
    cur = torch.cuda.current_stream(t.device)
    if not isinstance(stream, torch.cuda.Stream):
        if int(stream) == cur.cuda_stream:
            return
        stream = torch.cuda.ExternalStream(int(stream), device=t.device)
    if stream.cuda_stream == cur.cuda_stream:
        return
    for b in bufs:
        if isinstance(b, torch.Tensor):
            b.record_stream(stream)


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _points(cfg: HashGridConfig, x: torch.Tensor) -> torch.Tensor:
    _dev(x, "x", torch.float32)
    if x.dim() != 2 or x.shape[1] != cfg.n_dims or not x.is_contiguous():
        raise ValueError(f"x must be a contiguous [n, {cfg.n_dims}] tensor")
    return x


def abi_version() -> int:
    return load_library().hashgrid_abi_version()


def hashgrid_resolutions(cfg: HashGridConfig) -> list:
    out = (ctypes.c_int32 * max(cfg.n_levels, 1))()
    c = cfg.c()
    _check(load_library().hashgrid_resolutions(ctypes.byref(c), out))
    return list(out)


def _workspace(workspace, sizer, name):
    """(pointer, bytes) of a workspace argument: a uint8 GPU tensor, "auto"
    (allocated here through torch's caching allocator) or None."""
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError(f"{name} must be a tensor, 'auto' or None")
        workspace = sizer()
    if workspace is None:
        return None, 0, None
    _dev(workspace, name, torch.uint8)
    return workspace.data_ptr(), workspace.numel(), workspace


def hashgrid_forward_workspace_size(cfg: HashGridConfig, n: int) -> int:
    """Bytes of the level-major staging buffer of a forward over n points."""
    out = ctypes.c_size_t(0)
    c = cfg.c()
    _check(load_library().hashgrid_forward_workspace_size(ctypes.byref(c), n, ctypes.byref(out)))
    return out.value


def forward_workspace(cfg: HashGridConfig, n: int, device) -> torch.Tensor:
    return torch.empty(max(1, hashgrid_forward_workspace_size(cfg, n)), dtype=torch.uint8, device=device)


def hashgrid_forward(cfg: HashGridConfig, x: torch.Tensor, table: torch.Tensor,
                     out: torch.Tensor | None = None, workspace="auto", stream=None) -> torch.Tensor:
    """Encode points ``x`` [n, D] into ``out`` [n, >= L*F] (allocated when None;
    only the first L*F columns of each row are written).  ``workspace``: a
    uint8 GPU tensor, "auto" or None (write the rows directly)."""
    _points(cfg, x)
    _dev(table, "table", cfg.torch_table_dtype)
    if tuple(table.shape) != cfg.table_shape or not table.is_contiguous():
        raise ValueError(f"table must be a contiguous {cfg.table_shape} tensor")
    n = x.shape[0]
    made = out is None
    if out is None:
        out = torch.empty((n, cfg.out_features), device=x.device, dtype=torch.float32)
    _dev(out, "out", torch.float32)
    if out.dim() != 2 or out.shape[0] != n or out.stride(1) != 1 or out.shape[1] < cfg.out_features:
        raise ValueError("out must be [n, >= L*F] with unit column stride")
    auto = isinstance(workspace, str)
    ws_ptr, ws_bytes, _keep = _workspace(workspace, lambda: forward_workspace(cfg, n, x.device) if n else None,
                                         "workspace")
    c = cfg.c()
    _check(load_library().hashgrid_forward(ctypes.byref(c), x.data_ptr(), n, table.data_ptr(),
                                           out.data_ptr(), out.stride(0), ws_ptr, ws_bytes,
                                           _stream(x, stream)))
    _keep_for_stream(x, stream, out if made else None, _keep if auto else None)
    return out


def hashgrid_backward_workspace_size(cfg: HashGridConfig, n: int) -> tuple:
    """(bytes for a one-pass binned backward of n points, minimum bytes)."""
    full, least = ctypes.c_size_t(0), ctypes.c_size_t(0)
    c = cfg.c()
    _check(load_library().hashgrid_backward_workspace_size(ctypes.byref(c), n, ctypes.byref(full),
                                                           ctypes.byref(least)))
    return full.value, least.value


def backward_workspace(cfg: HashGridConfig, n: int, device) -> torch.Tensor | None:
    """A device buffer sized for the one-pass binned backward (None if the
    configuration has no binned path)."""
    full, _ = hashgrid_backward_workspace_size(cfg, n)
    if full == 0:
        return None
    return torch.empty(full, dtype=torch.uint8, device=device)


def hashgrid_backward(cfg: HashGridConfig, x: torch.Tensor, dout: torch.Tensor,
                      dtable: torch.Tensor, workspace="auto", stream=None) -> torch.Tensor:
    """Accumulate the table gradient of ``dout`` [n, >= L*F] into ``dtable``
    (table shape, ``cfg.torch_grad_dtype``: float32, or float16 with
    grad_dtype "f16", which needs the binned path's workspace).
    ``workspace``: a uint8 GPU tensor, "auto" (sized by
    hashgrid_backward_workspace_size and allocated here) or None (the atomic
    scatter)."""
    _points(cfg, x)
    n = x.shape[0]
    _dev(dout, "dout", torch.float32)
    if dout.dim() != 2 or dout.shape[0] != n or dout.stride(1) != 1 or dout.shape[1] < cfg.out_features:
        raise ValueError("dout must be [n, >= L*F] with unit column stride")
    _dev(dtable, "dtable", cfg.torch_grad_dtype)
    if tuple(dtable.shape) != cfg.table_shape or not dtable.is_contiguous():
        raise ValueError(f"dtable must be a contiguous {cfg.table_shape} tensor")
    auto = isinstance(workspace, str)
    ws_ptr, ws_bytes, _keep = _workspace(workspace, lambda: backward_workspace(cfg, n, x.device) if n else None,
                                         "workspace")
    c = cfg.c()
    _check(load_library().hashgrid_backward(ctypes.byref(c), x.data_ptr(), n, dout.data_ptr(),
                                            dout.stride(0), dtable.data_ptr(), ws_ptr, ws_bytes,
                                            _stream(x, stream)))
    _keep_for_stream(x, stream, _keep if auto else None)
    return dtable


def hashgrid_backward_noalloc(cfg: HashGridConfig, x: torch.Tensor, dout: torch.Tensor,
                              dtable: torch.Tensor, stream=None) -> torch.Tensor:
    """hashgrid_backward without any workspace allocation: the library's own
    fixed device scratch holds the binned records (calls that overlap on one
    device race on it).  Accumulates into ``dtable``."""
    _points(cfg, x)
    n = x.shape[0]
    _dev(dout, "dout", torch.float32)
    if dout.dim() != 2 or dout.shape[0] != n or dout.stride(1) != 1 or dout.shape[1] < cfg.out_features:
        raise ValueError("dout must be [n, >= L*F] with unit column stride")
    _dev(dtable, "dtable", cfg.torch_grad_dtype)
    if tuple(dtable.shape) != cfg.table_shape or not dtable.is_contiguous():
        raise ValueError(f"dtable must be a contiguous {cfg.table_shape} tensor")
    c = cfg.c()
    _check(load_library().hashgrid_backward_noalloc(ctypes.byref(c), x.data_ptr(), n, dout.data_ptr(),
                                                    dout.stride(0), dtable.data_ptr(), _stream(x, stream)))
    return dtable


def hashgrid_debug_corners(cfg: HashGridConfig, x: torch.Tensor, stream=None):
    """(idx int32 [n, L, 2^D] holding the uint32 indices, w float32 [n, L, 2^D])."""
    _points(cfg, x)
    n = x.shape[0]
    K = 1 << cfg.n_dims
    idx = torch.empty((n, cfg.n_levels, K), device=x.device, dtype=torch.int32)
    w = torch.empty((n, cfg.n_levels, K), device=x.device, dtype=torch.float32)
    c = cfg.c()
    _check(load_library().hashgrid_debug_corners(ctypes.byref(c), x.data_ptr(), n, idx.data_ptr(),
                                                 w.data_ptr(), _stream(x, stream)))
    _keep_for_stream(x, stream, idx, w)
    return idx, w


def hashgrid_input_grad_workspace_size(cfg: HashGridConfig, n: int) -> int:
    """Bytes of the level-major stage of an input-gradient call over n points."""
    out = ctypes.c_size_t(0)
    c = cfg.c()
    _check(load_library().hashgrid_input_grad_workspace_size(ctypes.byref(c), n, ctypes.byref(out)))
    return out.value


def hashgrid_input_grad(cfg: HashGridConfig, x: torch.Tensor, table: torch.Tensor, dout: torch.Tensor,
                        dx: torch.Tensor | None = None, workspace="auto", stream=None) -> torch.Tensor:
    """dL/dx [n, D] (fp32, written) of upstream ``dout`` [n, >= L*F].
    ``workspace``: a uint8 GPU tensor, "auto" or None (point-major path)."""
    _points(cfg, x)
    n = x.shape[0]
    _dev(table, "table", cfg.torch_table_dtype)
    if tuple(table.shape) != cfg.table_shape or not table.is_contiguous():
        raise ValueError(f"table must be a contiguous {cfg.table_shape} tensor")
    _dev(dout, "dout", torch.float32)
    if dout.dim() != 2 or dout.shape[0] != n or dout.stride(1) != 1 or dout.shape[1] < cfg.out_features:
        raise ValueError("dout must be [n, >= L*F] with unit column stride")
    made = dx is None
    if dx is None:
        dx = torch.empty((n, cfg.n_dims), device=x.device, dtype=torch.float32)
    _dev(dx, "dx", torch.float32)
    if tuple(dx.shape) != (n, cfg.n_dims) or not dx.is_contiguous():
        raise ValueError(f"dx must be a contiguous [n, {cfg.n_dims}] tensor")

    def alloc():
        size = hashgrid_input_grad_workspace_size(cfg, n) if n else 0
        return torch.empty(size, dtype=torch.uint8, device=x.device) if size else None

    auto = isinstance(workspace, str)
    ws_ptr, ws_bytes, _keep = _workspace(workspace, alloc, "workspace")
    c = cfg.c()
    _check(load_library().hashgrid_input_grad(ctypes.byref(c), x.data_ptr(), n, table.data_ptr(), dout.data_ptr(),
                                              dout.stride(0), dx.data_ptr(), ws_ptr, ws_bytes,
                                              _stream(x, stream)))
    _keep_for_stream(x, stream, dx if made else None, _keep if auto else None)
    return dx


def hashgrid_mlp_workspace_size(cfg: HashGridConfig, n: int) -> tuple:
    """(binary16 encoding stage bytes, backward workspace bytes) of the MLP head."""
    st, bw = ctypes.c_size_t(0), ctypes.c_size_t(0)
    c = cfg.c()
    _check(load_library().hashgrid_mlp_workspace_size(ctypes.byref(c), n, ctypes.byref(st), ctypes.byref(bw)))
    return st.value, bw.value


def _mlp_coords(params) -> int:
    """The head's coordinate inputs, read from W1's width (32: 0, 35: 3)."""
    if len(params) != 6:
        raise ValueError("params must be [w1, b1, w2, b2, w3, b3]")
    w1 = params[0]
    if w1.dim() != 2 or w1.shape[1] not in (32, 32 + MLP_COORDS):
        raise ValueError(f"w1 must be [64, 32] (NeRFace head) or [64, {32 + MLP_COORDS}] (TinyNeRF head)")
    return int(w1.shape[1]) - 32


def _mlp_params(params) -> _MlpParams:
    """[w1, b1, w2, b2, w3, b3]: binary16 weights [out][in], fp32 biases,
    contiguous GPU tensors; W1 [64, 32], or [64, 35] for the TinyNeRF head."""
    names = ("w1", "b1", "w2", "b2", "w3", "b3")
    coords = _mlp_coords(params)
    shapes = mlp_shapes(coords)
    ptrs = []
    for name, t in zip(names, params):
        _dev(t, name, torch.float16 if name[0] == "w" else torch.float32)
        if tuple(t.shape) != shapes[name] or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {shapes[name]} tensor")
        ptrs.append(t.data_ptr())
    return _MlpParams(*ptrs, coords)


def hashgrid_mlp_forward(cfg: HashGridConfig, x: torch.Tensor, table: torch.Tensor, params,
                         y: torch.Tensor | None = None, stage: torch.Tensor | None = None, stream=None):
    """Encoder + MLP head forward.  Returns (y [n, 4] fp32, stage), the stage
    (uint8, the binary16 encoding) being what hashgrid_mlp_backward needs."""
    _points(cfg, x)
    n = x.shape[0]
    _dev(table, "table", cfg.torch_table_dtype)
    if tuple(table.shape) != cfg.table_shape or not table.is_contiguous():
        raise ValueError(f"table must be a contiguous {cfg.table_shape} tensor")
    mp = _mlp_params(params)
    st_bytes, _ = hashgrid_mlp_workspace_size(cfg, n)
    made = (stage is None, y is None)
    if stage is None:
        stage = torch.empty(max(st_bytes, 1), dtype=torch.uint8, device=x.device)
    _dev(stage, "stage", torch.uint8)
    if y is None:
        y = torch.empty((n, 4), device=x.device, dtype=torch.float32)
    _dev(y, "y", torch.float32)
    if tuple(y.shape) != (n, 4) or not y.is_contiguous():
        raise ValueError("y must be a contiguous [n, 4] tensor")
    c = cfg.c()
    _check(load_library().hashgrid_mlp_forward(ctypes.byref(c), x.data_ptr(), n, table.data_ptr(), ctypes.byref(mp),
                                               y.data_ptr(), stage.data_ptr(), stage.numel(), _stream(x, stream)))
    _keep_for_stream(x, stream, stage if made[0] else None, y if made[1] else None)
    return y, stage


def hashgrid_mlp_backward(cfg: HashGridConfig, x: torch.Tensor, stage: torch.Tensor, params, dy: torch.Tensor,
                          grads, dtable: torch.Tensor, workspace="auto", stream=None) -> None:
    """Accumulate the MLP's weight and bias gradients into ``grads`` ([dw1, db1,
    dw2, db2, dw3, db3], fp32) and the table gradient into ``dtable``."""
    _points(cfg, x)
    n = x.shape[0]
    mp = _mlp_params(params)
    _dev(stage, "stage", torch.uint8)
    _dev(dy, "dy", torch.float32)
    if tuple(dy.shape) != (n, 4) or not dy.is_contiguous():
        raise ValueError("dy must be a contiguous [n, 4] tensor")
    names = ("dw1", "db1", "dw2", "db2", "dw3", "db3")
    if len(grads) != 6:
        raise ValueError("grads must be [dw1, db1, dw2, db2, dw3, db3]")
    shapes = mlp_shapes(mp.coord_inputs)
    for name, t in zip(names, grads):
        _dev(t, name, torch.float32)
        if tuple(t.shape) != shapes[name[1:]] or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {shapes[name[1:]]} tensor")
    g = _MlpGrads(*[t.data_ptr() for t in grads])
    _dev(dtable, "dtable", cfg.torch_grad_dtype)
    if tuple(dtable.shape) != cfg.table_shape or not dtable.is_contiguous():
        raise ValueError(f"dtable must be a contiguous {cfg.table_shape} tensor")
    auto = isinstance(workspace, str)
    ws_ptr, ws_bytes, _keep = _workspace(
        workspace, lambda: torch.empty(max(1, hashgrid_mlp_workspace_size(cfg, n)[1]), dtype=torch.uint8,
                                       device=x.device), "workspace")
    c = cfg.c()
    _check(load_library().hashgrid_mlp_backward(ctypes.byref(c), x.data_ptr(), n, stage.data_ptr(), ctypes.byref(mp),
                                                dy.data_ptr(), ctypes.byref(g), dtable.data_ptr(), ws_ptr, ws_bytes,
                                                _stream(x, stream)))
    _keep_for_stream(x, stream, _keep if auto else None)


def hashgrid_adam_step(param: torch.Tensor, m: torch.Tensor, v: torch.Tensor, grad: torch.Tensor, *,
                       lr: float, step: int, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
                       param_f16: torch.Tensor | None = None, zero_grad: bool = False, stream=None) -> None:
    """One Adam update of ``param`` in place (fp32, any shape, contiguous),
    with its moments ``m`` and ``v`` and gradient ``grad`` of the same shape;
    ``step`` is the 1-based update index.  ``param_f16`` (fp16, same shape)
    receives the updated values rounded to half; ``zero_grad`` clears ``grad``."""
    for name, t in (("param", param), ("m", m), ("v", v), ("grad", grad)):
        _dev(t, name, torch.float32)
        if t.shape != param.shape or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous with the shape of param")
    half_ptr = None
    if param_f16 is not None:
        _dev(param_f16, "param_f16", torch.float16)
        if param_f16.shape != param.shape or not param_f16.is_contiguous():
            raise ValueError("param_f16 must be contiguous with the shape of param")
        half_ptr = param_f16.data_ptr()
    opt = _Adam(lr, beta1, beta2, eps, step)
    _check(load_library().hashgrid_adam_step(ctypes.byref(opt), param.numel(), param.data_ptr(), m.data_ptr(),
                                             v.data_ptr(), grad.data_ptr(), half_ptr,
                                             HG_ADAM_ZERO_GRAD if zero_grad else 0, _stream(param, stream)))


class HashGridAdam(torch.optim.Optimizer):
    """Adam over fp32 hash tables through hashgrid_adam_step (no weight decay:
    the pages switch it off for the tables).  A drop-in for torch.optim.Adam on
    such parameters; ``zero_grad_in_step`` clears each gradient inside the
    update, so the next backward can accumulate into it directly."""

    def __init__(self, params, lr=1e-2, betas=(0.9, 0.999), eps=1e-8, zero_grad_in_step=False):
        super().__init__(params, dict(lr=lr, betas=betas, eps=eps))
        self.zero_grad_in_step = zero_grad_in_step

    @torch.no_grad()
    def step(self, closure=None):
        loss = closure() if closure is not None else None
        for group in self.param_groups:
            b1, b2 = group["betas"]
            for p in group["params"]:
                if p.grad is None:
                    continue
                st = self.state[p]
                if not st:
                    st["step"] = 0
                    st["exp_avg"] = torch.zeros_like(p, memory_format=torch.contiguous_format)
                    st["exp_avg_sq"] = torch.zeros_like(p, memory_format=torch.contiguous_format)
                st["step"] += 1
                hashgrid_adam_step(p, st["exp_avg"], st["exp_avg_sq"], p.grad, lr=group["lr"], step=st["step"],
                                   beta1=b1, beta2=b2, eps=group["eps"], zero_grad=self.zero_grad_in_step)
        return loss


def hashgrid_tune(key: int, value: int) -> None:
    _check(load_library().hashgrid_tune(key, value))


def hashgrid_tune_get(key: int) -> int:
    v = load_library().hashgrid_tune_get(key)
    if v < 0:
        _check(v)
    return v


def _grad_config(cfg: HashGridConfig, param_dtype, n: int) -> HashGridConfig:
    """Config for the autograd table gradient: a binary16 parameter gets a
    binary16 gradient buffer where the binned path exists (each entry rounded
    once, the same bits as rounding the fp32 gradient, half the memory), fp32
    otherwise."""
    if param_dtype == torch.float16 and n > 0 and hashgrid_backward_workspace_size(cfg, n)[0] > 0:
        return dataclasses.replace(cfg, grad_dtype="f16")
    return dataclasses.replace(cfg, grad_dtype="f32")


class HashGridFunction(torch.autograd.Function):
    """Autograd wrapper: forward through hashgrid_forward; the table gradient
    through hashgrid_backward into a zeroed fp32 buffer and, when x requires
    grad, dL/dx through hashgrid_input_grad.  ``kernel_table`` (optional) is
    the table the kernels read -- e.g. a binary16 copy of an fp32 ``table``,
    which then receives the fp32 gradient unrounded."""

    @staticmethod
    def forward(ctx, x, table, cfg, kernel_table=None):
        ctx.cfg = cfg
        kt = (table if kernel_table is None else kernel_table).contiguous()
        x = x.contiguous()
        ctx.save_for_backward(x, kt)
        ctx.table_dtype = table.dtype
        return hashgrid_forward(cfg, x, kt)

    @staticmethod
    def backward(ctx, dout):
        x, kt = ctx.saved_tensors
        cfg = ctx.cfg
        dout = dout.contiguous()
        dx = grad = None
        if ctx.needs_input_grad[0]:
            dx = hashgrid_input_grad(cfg, x, kt, dout)
        if ctx.needs_input_grad[1]:
            gcfg = _grad_config(cfg, ctx.table_dtype, x.shape[0])
            grad = torch.zeros(cfg.table_shape, device=x.device, dtype=gcfg.torch_grad_dtype)
            hashgrid_backward(gcfg, x, dout, grad)
            if grad.dtype != ctx.table_dtype:
                grad = grad.to(ctx.table_dtype)
        return dx, grad, None, None


class HashGridEncoder(torch.nn.Module):
    """Multiresolution hash-grid encoder with the pages' constructor arguments
    (ipipp.com HashGridEncoder): ``forward(x [N, D]) -> [N, L*F]`` (D = 3 by default).  The L
    tables live in one [L, T, F] parameter initialised uniform(-1e-4, 1e-4).

    With ``table_dtype="f16"`` the kernels read binary16 tables (jsqmd.com's
    half-precision storage tip).  By default (``fp32_master=True``) the
    parameter itself stays fp32 and each forward reads a binary16 copy of it,
    so the fp32 gradient reaches the parameter unrounded (gradients of ~1e-8,
    common for tables, would underflow in binary16).  ``fp32_master=False``
    keeps the parameter in binary16, and its gradient is rounded to binary16."""

    def __init__(self, n_levels=16, n_features_per_level=2, log2_hashmap_size=19,
                 base_resolution=16, finest_resolution=512, table_dtype="f32", device="cuda", n_dims=3,
                 fp32_master=True):
        super().__init__()
        self.cfg = HashGridConfig(n_levels, n_features_per_level, log2_hashmap_size,
                                  base_resolution, finest_resolution, table_dtype, n_dims=n_dims)
        self.resolutions = hashgrid_resolutions(self.cfg)
        t = torch.empty(self.cfg.table_shape, dtype=torch.float32, device=device).uniform_(-1e-4, 1e-4)
        self.fp32_master = bool(fp32_master) and table_dtype == "f16"
        if self.fp32_master:
            t = t.to(torch.float16).to(torch.float32)  # the values the kernels read, exactly
        self.embeddings = torch.nn.Parameter(t if self.fp32_master else t.to(self.cfg.torch_table_dtype))

    def kernel_table(self) -> torch.Tensor:
        """The table in the dtype the kernels read."""
        if self.fp32_master:
            return self.embeddings.detach().to(torch.float16)
        return self.embeddings

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if self.fp32_master:
            return HashGridFunction.apply(x, self.embeddings, self.cfg, self.kernel_table())
        return HashGridFunction.apply(x, self.embeddings, self.cfg)


class HashGridMLPFunction(torch.autograd.Function):
    """Autograd of encoder + MLP head: the forward keeps the binary16 encoding
    stage, the backward gives the table gradient and the fp32 gradients of the
    (fp32 master) weights and biases; no gradient flows to x."""

    @staticmethod
    def forward(ctx, x, table, w1, b1, w2, b2, w3, b3, cfg, kernel_table=None):
        x = x.contiguous()
        kt = (table if kernel_table is None else kernel_table).contiguous()
        params = [w1.to(torch.float16).contiguous(), b1.float().contiguous(), w2.to(torch.float16).contiguous(),
                  b2.float().contiguous(), w3.to(torch.float16).contiguous(), b3.float().contiguous()]
        y, stage = hashgrid_mlp_forward(cfg, x, kt, params)
        ctx.cfg = cfg
        ctx.save_for_backward(x, stage, *params)
        ctx.dtypes = [t.dtype for t in (w1, b1, w2, b2, w3, b3)]
        ctx.table_dtype = table.dtype
        return y

    @staticmethod
    def backward(ctx, dy):
        x, stage, *params = ctx.saved_tensors
        cfg = ctx.cfg
        grads = [torch.zeros(p.shape, device=x.device) for p in params]
        gcfg = _grad_config(cfg, ctx.table_dtype, x.shape[0])
        dtable = torch.zeros(cfg.table_shape, device=x.device, dtype=gcfg.torch_grad_dtype)
        hashgrid_mlp_backward(gcfg, x, stage, params, dy.contiguous().float(), grads, dtable)
        if dtable.dtype != ctx.table_dtype:
            dtable = dtable.to(ctx.table_dtype)
        return (None, dtable, *[g.to(dt) for g, dt in zip(grads, ctx.dtypes)], None, None)


class HashGridMLP(torch.nn.Module):
    """The encoder followed by the NeRFace head of ipipp.com section 3:
    Linear(32, 64), ReLU, Linear(64, 64), ReLU, Linear(64, 4) with biases;
    ``forward(x [N, 3]) -> [N, 4]`` (density and colour channels).  With
    ``coord_inputs=3`` the head is jsqmd.com's TinyNeRF (section 4): the point
    is concatenated before its encoding, Linear(35, 64) then the same layers.
    Weights are fp32 masters initialised Xavier-uniform; biases are
    initialised as torch.nn.Linear does, U(-1/sqrt(fan_in), 1/sqrt(fan_in)).
    The matrix cores read the weights (and the head's inputs) as binary16."""

    def __init__(self, table_dtype="f16", device="cuda", coord_inputs: int = 0, **encoder_kw):
        super().__init__()
        self.encoder = HashGridEncoder(table_dtype=table_dtype, device=device, **encoder_kw)
        if self.encoder.cfg.out_features != 32:
            raise ValueError("the MLP head takes 32 encoded features (L * F = 32)")
        fin1 = mlp_shapes(coord_inputs)["w1"][1]
        layers = []
        for fin, fout in ((fin1, 64), (64, 64), (64, 4)):
            w = torch.empty((fout, fin), device=device)
            torch.nn.init.xavier_uniform_(w)
            b = torch.empty(fout, device=device).uniform_(-1.0 / fin ** 0.5, 1.0 / fin ** 0.5)
            layers += [torch.nn.Parameter(w), torch.nn.Parameter(b)]
        self.w1, self.b1, self.w2, self.b2, self.w3, self.b3 = layers

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        enc = self.encoder
        kt = enc.kernel_table() if enc.fp32_master else None
        return HashGridMLPFunction.apply(x, enc.embeddings, self.w1, self.b1, self.w2, self.b2, self.w3,
                                         self.b3, enc.cfg, kt)
