"""Thin Python binding of libmoeq.so (include/moeq.h): argument marshalling only.

Every step of the path runs in the HIP library.  torch supplies device memory and
the current stream; this module turns tensors into pointers, allocates outputs
with torch, and raises :class:`MoeqError` on a negative status.  If the library
is not built the first call raises; there is no other path.
"""
from __future__ import annotations

import ctypes as C
import dataclasses
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOEQ_LIB names another build of the same library (the host-sanitized one)
LIB_PATH = os.environ.get("MOEQ_LIB") or os.path.join(_HERE, "csrc", "libmoeq.so")

OK, EINVAL, ESHAPE, EDTYPE, ERANGE, EWORKSPACE, EUNSUPPORTED, EDEVICE = 0, -1, -2, -3, -4, -5, -6, -7
F32, F16, BF16 = 0, 1, 2
FMT_AWQ, FMT_MXFP4_BANK = 0, 1

_TORCH_DT = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
_DT_TORCH = {v: k for k, v in _TORCH_DT.items()}

# every symbol include/moeq.h declares
EXPORTS = ("moeq_route_workspace_bytes", "moeq_route_bind", "moe_dispatch",
           "moe_dispatch_static", "moe_dispatch_counts", "awq_grouped_swiglu", "awq_grouped_down", "moe_combine",
           "awq_input_backward", "moe_combine_backward", "moe_dispatch_backward",
           "moe_dispatch_weights_backward", "awq_swiglu_input_backward_workspace_bytes",
           "awq_swiglu_input_backward", "awq_expert_workspace_bytes", "awq_expert_forward",
           "awq_expert_input_backward", "frozen_awq_workspace_bytes", "frozen_awq_forward",
           "mx8_workspace_bytes", "mx8_quantize", "mx8_grouped_swiglu", "mx8_grouped_down",
           "moeq_status_string", "moeq_last_error")


class MoeqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"moeq status {status}: {message}")
        self.status = status


class Route(C.Structure):
    """moeq_route: host struct of device pointers into one caller-owned workspace."""
    _fields_ = [("T", C.c_int32), ("E", C.c_int32), ("top_k", C.c_int32),
                ("token_blocks", C.c_int32), ("workspace", C.c_void_p),
                ("workspace_bytes", C.c_size_t), ("expert_offsets", C.c_void_p),
                ("row_src", C.c_void_p), ("slot_pos", C.c_void_p), ("block_base", C.c_void_p),
                ("tile_offsets", C.c_void_p), ("tile_expert", C.c_void_p),
                ("magic", C.c_uint32)]


class Experts(C.Structure):
    """moeq_experts: one packed expert cube (AWQ or MXFP4 bank)."""
    _fields_ = [("format", C.c_int), ("experts", C.c_int32), ("expert_start", C.c_int32),
                ("in_features", C.c_int32), ("out_features", C.c_int32),
                ("group_size", C.c_int32), ("qweight", C.c_void_p), ("qzeros", C.c_void_p),
                ("scales", C.c_void_p), ("scale_dtype", C.c_int), ("bias", C.c_void_p),
                ("interleaved_gate_up", C.c_int32)]


class SwiGLU(C.Structure):
    _fields_ = [("clamp", C.c_float), ("alpha", C.c_float), ("up_offset", C.c_float),
                ("gate_one_sided", C.c_int32)]


_lib = None


def lib():
    """Load libmoeq.so once; raise if it is missing (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                           "(there is no CPU or PyTorch fallback)")
    L = C.CDLL(LIB_PATH)
    vp, i32 = C.c_void_p, C.c_int32
    L.moeq_route_workspace_bytes.restype = C.c_size_t
    L.moeq_route_workspace_bytes.argtypes = [i32, i32, i32]
    L.moeq_route_bind.restype = C.c_int
    L.moeq_route_bind.argtypes = [C.POINTER(Route), vp, C.c_size_t, i32, i32, i32]
    L.moe_dispatch.restype = C.c_int
    L.moe_dispatch.argtypes = [vp, C.c_int, i32, i32, vp, C.c_int, i32, vp, i32, vp, vp, vp, vp,
                               C.POINTER(Route), vp]
    L.moe_dispatch_static.restype = C.c_int
    L.moe_dispatch_static.argtypes = L.moe_dispatch.argtypes
    L.moe_dispatch_counts.restype = C.c_int
    L.moe_dispatch_counts.argtypes = [C.POINTER(Route), vp, i32, vp, vp]
    L.awq_grouped_swiglu.restype = C.c_int
    L.awq_grouped_swiglu.argtypes = [C.POINTER(Route), vp, C.c_int, C.POINTER(Experts),
                                     C.POINTER(Experts), SwiGLU, vp, vp]
    L.awq_grouped_down.restype = C.c_int
    L.awq_grouped_down.argtypes = [C.POINTER(Route), vp, C.c_int, C.POINTER(Experts), vp, vp]
    L.moe_combine.restype = C.c_int
    L.moe_combine.argtypes = [C.POINTER(Route), vp, C.c_int, i32, vp, vp, vp]
    L.awq_input_backward.restype = C.c_int
    L.awq_input_backward.argtypes = [C.POINTER(Route), vp, C.c_int, i32, C.POINTER(Experts),
                                     vp, vp]
    L.moe_combine_backward.restype = C.c_int
    L.moe_combine_backward.argtypes = [C.POINTER(Route), vp, C.c_int, i32, vp, vp, vp, vp, vp]
    L.moe_dispatch_backward.restype = C.c_int
    L.moe_dispatch_backward.argtypes = [C.POINTER(Route), vp, C.c_int, i32, vp, vp]
    L.moe_dispatch_weights_backward.restype = C.c_int
    L.moe_dispatch_weights_backward.argtypes = [C.POINTER(Route), vp, vp, vp, vp, vp]
    L.awq_swiglu_input_backward_workspace_bytes.restype = C.c_size_t
    L.awq_swiglu_input_backward_workspace_bytes.argtypes = [i32, i32, C.c_int]
    L.awq_swiglu_input_backward.restype = C.c_int
    L.awq_swiglu_input_backward.argtypes = [C.POINTER(Route), vp, C.c_int, C.POINTER(Experts),
                                            C.POINTER(Experts), C.POINTER(Experts), SwiGLU, vp,
                                            vp, vp, C.c_size_t, vp]
    L.awq_expert_workspace_bytes.restype = C.c_size_t
    L.awq_expert_workspace_bytes.argtypes = [i32, i32, i32, i32, C.c_int]
    L.awq_expert_forward.restype = C.c_int
    L.awq_expert_forward.argtypes = [vp, C.c_int, i32, vp, C.POINTER(Experts), vp, vp,
                                     C.c_size_t, vp]
    L.awq_expert_input_backward.restype = C.c_int
    L.awq_expert_input_backward.argtypes = [vp, C.c_int, i32, vp, C.POINTER(Experts), vp, vp,
                                            C.c_size_t, vp]
    L.frozen_awq_workspace_bytes.restype = C.c_size_t
    L.frozen_awq_workspace_bytes.argtypes = [i32]
    L.frozen_awq_forward.restype = C.c_int
    L.frozen_awq_forward.argtypes = [vp, C.c_int, i32, C.POINTER(Experts), vp, vp, C.c_size_t,
                                     vp]
    L.mx8_workspace_bytes.restype = C.c_size_t
    L.mx8_workspace_bytes.argtypes = [i32, i32]
    L.mx8_quantize.restype = C.c_int
    L.mx8_quantize.argtypes = [vp, C.c_int, i32, i32, vp, vp, vp]
    L.mx8_grouped_swiglu.restype = C.c_int
    L.mx8_grouped_swiglu.argtypes = [C.POINTER(Route), vp, C.c_int, C.POINTER(Experts), SwiGLU,
                                     vp, vp, C.c_size_t, vp]
    L.mx8_grouped_down.restype = C.c_int
    L.mx8_grouped_down.argtypes = [C.POINTER(Route), vp, C.c_int, C.POINTER(Experts), vp, vp,
                                   C.c_size_t, vp]
    L.moeq_status_string.restype = C.c_char_p
    L.moeq_status_string.argtypes = [C.c_int]
    L.moeq_last_error.restype = C.c_char_p
    L.moeq_last_error.argtypes = []
    _lib = L
    return L


def _check(status: int):
    if status != OK:
        L = lib()
        raise MoeqError(status, f"{L.moeq_status_string(status).decode()}: "
                                f"{L.moeq_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise MoeqError(EINVAL, "tensors must be contiguous")
    return C.c_void_p(t.data_ptr())


def _stream(device) -> C.c_void_p:
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dt(t: torch.Tensor) -> int:
    return _TORCH_DT.get(t.dtype, 99)


# ------------------------------------------------------------------ payloads
@dataclasses.dataclass
class AwqExperts:
    """AWQ expert cube: qweight int32 [E,K,N/8], qzeros int32 [E,K/g,N/8],
    scales [E,K/g,N] (fp32/fp16/bf16), bias [E,N] in the scale dtype or None."""
    qweight: torch.Tensor
    qzeros: torch.Tensor
    scales: torch.Tensor
    group_size: int
    bias: Optional[torch.Tensor] = None
    expert_start: int = 0

    def c(self) -> Experts:
        self.validate()
        E, K, W8 = self.qweight.shape
        return Experts(FMT_AWQ, E, self.expert_start, K, W8 * 8, self.group_size,
                       _ptr(self.qweight), _ptr(self.qzeros), _ptr(self.scales),
                       _dt(self.scales), _ptr(self.bias), 0)

    def validate(self) -> None:
        """Shapes, dtypes and device of the payload tensors.  The C descriptor has
        no dtype field for the bias (it is read in the scale dtype), so a bias of
        another dtype or shape is rejected here rather than misread."""
        qw, qz, sc, b = self.qweight, self.qzeros, self.scales, self.bias
        if qw.dim() != 3 or qz.dim() != 3 or sc.dim() != 3:
            raise MoeqError(ESHAPE, "AWQ qweight, qzeros and scales are rank-3 [E, ., .]")
        if qw.dtype != torch.int32 or qz.dtype != torch.int32:
            raise MoeqError(EDTYPE, "AWQ qweight and qzeros are int32 words")
        if sc.dtype not in _TORCH_DT:
            raise MoeqError(EDTYPE, f"AWQ scales must be fp32, fp16 or bf16, not {sc.dtype}")
        E, K, W8 = qw.shape
        g = int(self.group_size)
        if g <= 0 or K % g:
            raise MoeqError(ESHAPE, f"group size {g} does not divide in_features {K}")
        N = W8 * 8
        if tuple(qz.shape) != (E, K // g, W8):
            raise MoeqError(ESHAPE, f"qzeros shape {tuple(qz.shape)} != {(E, K // g, W8)}")
        if tuple(sc.shape) != (E, K // g, N):
            raise MoeqError(ESHAPE, f"scales shape {tuple(sc.shape)} != {(E, K // g, N)}")
        if b is not None:
            if b.dtype != sc.dtype:
                raise MoeqError(EDTYPE, f"AWQ bias dtype {b.dtype} differs from the scale "
                                        f"dtype {sc.dtype} (the bias is held in the scale dtype)")
            if tuple(b.shape) != (E, N):
                raise MoeqError(ESHAPE, f"bias shape {tuple(b.shape)} != {(E, N)}")
        devs = {t.device for t in (qw, qz, sc, b) if t is not None}
        if len(devs) != 1:
            raise MoeqError(EINVAL, "AWQ payload tensors live on different devices")


@dataclasses.dataclass
class Mxfp4Bank:
    """MXFP4 bank: blocks uint8 [E,R,C/32,16], scales uint8 [E,R,C/32], bias bf16 [E,R]."""
    blocks: torch.Tensor
    scales: torch.Tensor
    bias: torch.Tensor
    interleaved_gate_up: bool
    expert_start: int = 0

    def c(self) -> Experts:
        self.validate()
        E, R, NB, _ = self.blocks.shape
        return Experts(FMT_MXFP4_BANK, E, self.expert_start, NB * 32, R, 32, _ptr(self.blocks),
                       None, _ptr(self.scales), BF16, _ptr(self.bias),
                       1 if self.interleaved_gate_up else 0)

    def validate(self) -> None:
        """Bank shapes and dtypes (native.rs validate): blocks u8 [E, R, C/32, 16],
        E8M0 scales u8 [E, R, C/32], bias bf16 [E, R]."""
        bl, sc, b = self.blocks, self.scales, self.bias
        if bl.dim() != 4 or bl.shape[3] != 16:
            raise MoeqError(ESHAPE, "MXFP4 blocks are [E, rows, cols/32, 16]")
        if bl.dtype != torch.uint8 or sc.dtype != torch.uint8:
            raise MoeqError(EDTYPE, "MXFP4 blocks and E8M0 scales are uint8")
        E, R, NB, _ = bl.shape
        if tuple(sc.shape) != (E, R, NB):
            raise MoeqError(ESHAPE, f"MXFP4 scales shape {tuple(sc.shape)} != {(E, R, NB)}")
        if b is None or b.dtype != torch.bfloat16:
            raise MoeqError(EDTYPE, "MXFP4 banks carry a bf16 bias")
        if tuple(b.shape) != (E, R):
            raise MoeqError(ESHAPE, f"MXFP4 bias shape {tuple(b.shape)} != {(E, R)}")
        if len({bl.device, sc.device, b.device}) != 1:
            raise MoeqError(EINVAL, "MXFP4 bank tensors live on different devices")


# ------------------------------------------------------------------ route
class RouteState:
    """A moeq_route plus the torch-owned workspace it points into."""

    def __init__(self, T: int, E: int, top_k: int, device="cuda"):
        nbytes = lib().moeq_route_workspace_bytes(T, E, top_k)
        if nbytes == 0:
            raise MoeqError(EINVAL, f"invalid route shape T={T} E={E} top_k={top_k}")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.c = Route()
        _check(lib().moeq_route_bind(C.byref(self.c), _ptr(self.workspace), nbytes, T, E, top_k))
        self.T, self.E, self.top_k = T, E, top_k
        self.device = self.workspace.device

    @property
    def A(self) -> int:
        return self.T * self.top_k

    def _view(self, ptr_attr: str, n: int) -> torch.Tensor:
        off = getattr(self.c, ptr_attr) - self.workspace.data_ptr()
        return self.workspace[off:off + 4 * n].view(torch.int32)

    @property
    def expert_offsets(self) -> torch.Tensor:
        return self._view("expert_offsets", self.E + 1)

    @property
    def row_src(self) -> torch.Tensor:
        return self._view("row_src", self.A)

    @property
    def slot_pos(self) -> torch.Tensor:
        return self._view("slot_pos", self.A).view(self.T, self.top_k)

    def tile_lists(self):
        """Internal m-tile lists of the tiled kernels: (tile_offsets [E+1], tile_expert,
        tile_order), the last two of length ceil(A/128) + E (entries past the
        m-tile count are unused)."""
        cap = (self.A + 127) // 128 + self.E
        te = self._view("tile_expert", 2 * cap)
        return self._view("tile_offsets", self.E + 1), te[:cap], te[cap:]


# ------------------------------------------------------------------ calls
def moe_dispatch(x: torch.Tensor, logits: torch.Tensor, expert_bias: Optional[torch.Tensor],
                 top_k: int, route: Optional[RouteState] = None, out: Optional[dict] = None):
    """Router top-k + FP32 softmax + COPY dispatch.  Returns a dict with values,
    weights, selected, row_experts and route (moe_exchange.rs MoeDispatched)."""
    T, K = x.shape
    E = logits.shape[1]
    if route is None:
        route = RouteState(T, E, top_k, x.device)
    A = T * top_k
    if out is None:
        out = dict(values=torch.empty(A, K, dtype=x.dtype, device=x.device),
                   weights=torch.empty(T, top_k, dtype=torch.float32, device=x.device),
                   selected=torch.empty(T, top_k, dtype=torch.int32, device=x.device),
                   row_experts=torch.empty(A, dtype=torch.int32, device=x.device))
    if logits.dtype not in (torch.float32, torch.bfloat16) or (
            expert_bias is not None and expert_bias.dtype != torch.float32):
        raise MoeqError(EDTYPE, "logits are fp32 or bf16, the expert bias fp32")
    _check(lib().moe_dispatch(_ptr(x), _dt(x), T, K, _ptr(logits), _dt(logits), E,
                              _ptr(expert_bias), top_k,
                              _ptr(out["values"]), _ptr(out["weights"]), _ptr(out["selected"]),
                              _ptr(out["row_experts"]), C.byref(route.c), _stream(x.device)))
    out["route"] = route
    return out


class StaticRoute:
    """A moeq_route bound by moe_dispatch_static to the library's fixed device
    array: valid until the next moe_dispatch_static on the same GPU."""

    def __init__(self, device):
        self.c = Route()
        self.device = torch.device(device)
        self.T = self.E = self.top_k = 0

    @property
    def A(self) -> int:
        return self.T * self.top_k


def moe_dispatch_static(x: torch.Tensor, logits: torch.Tensor,
                        expert_bias: Optional[torch.Tensor], top_k: int,
                        out: Optional[dict] = None, route: Optional[StaticRoute] = None):
    """moe_dispatch with the route in the library's fixed per-GPU array (no route
    workspace).  Returns the same dict as moe_dispatch, with a StaticRoute."""
    T, K = x.shape
    E = logits.shape[1]
    A = T * top_k
    if out is None:
        out = dict(values=torch.empty(A, K, dtype=x.dtype, device=x.device),
                   weights=torch.empty(T, top_k, dtype=torch.float32, device=x.device),
                   selected=torch.empty(T, top_k, dtype=torch.int32, device=x.device),
                   row_experts=torch.empty(A, dtype=torch.int32, device=x.device))
    if logits.dtype not in (torch.float32, torch.bfloat16) or (
            expert_bias is not None and expert_bias.dtype != torch.float32):
        raise MoeqError(EDTYPE, "logits are fp32 or bf16, the expert bias fp32")
    if route is None:
        route = StaticRoute(x.device)
    _check(lib().moe_dispatch_static(_ptr(x), _dt(x), T, K, _ptr(logits), _dt(logits), E,
                                     _ptr(expert_bias),
                                     top_k, _ptr(out["values"]), _ptr(out["weights"]),
                                     _ptr(out["selected"]), _ptr(out["row_experts"]),
                                     C.byref(route.c), _stream(x.device)))
    route.T, route.E, route.top_k = T, E, top_k
    out["route"] = route
    return out


def moe_dispatch_counts(route: RouteState, expert_prefix: Sequence[int]) -> list:
    """Rows per contiguous global expert range [prefix[r], prefix[r+1]) (synchronises)."""
    pre = (C.c_int64 * len(expert_prefix))(*[int(v) for v in expert_prefix])
    R = len(expert_prefix) - 1
    cnt = (C.c_int64 * max(R, 1))()
    _check(lib().moe_dispatch_counts(C.byref(route.c), C.cast(pre, C.c_void_p), R,
                                     C.cast(cnt, C.c_void_p), _stream(route.device)))
    return [int(cnt[i]) for i in range(max(R, 0))]


def awq_grouped_swiglu(route: RouteState, values: torch.Tensor, gate, up=None,
                       clamp: float = 0.0, alpha: float = 1.0, up_offset: float = 0.0,
                       h: Optional[torch.Tensor] = None,
                       gate_one_sided: bool = False) -> torch.Tensor:
    gc = gate.c()
    uc = None if up is None else up.c()
    I = gc.out_features // 2 if isinstance(gate, Mxfp4Bank) else gc.out_features
    if h is None:
        h = torch.empty(values.shape[0], I, dtype=values.dtype, device=values.device)
    _check(lib().awq_grouped_swiglu(C.byref(route.c), _ptr(values), _dt(values), C.byref(gc),
                                    None if uc is None else C.byref(uc),
                                    SwiGLU(clamp, alpha, up_offset, int(gate_one_sided)),
                                    _ptr(h),
                                    _stream(values.device)))
    return h


def awq_grouped_down(route: RouteState, h: torch.Tensor, down,
                     y: Optional[torch.Tensor] = None) -> torch.Tensor:
    dc = down.c()
    if y is None:
        y = torch.empty(h.shape[0], dc.out_features, dtype=h.dtype, device=h.device)
    _check(lib().awq_grouped_down(C.byref(route.c), _ptr(h), _dt(h), C.byref(dc), _ptr(y),
                                  _stream(h.device)))
    return y


def moe_combine(route: RouteState, y: torch.Tensor, weights: torch.Tensor,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    K = y.shape[1]
    if out is None:
        out = torch.empty(route.T, K, dtype=y.dtype, device=y.device)
    _check(lib().moe_combine(C.byref(route.c), _ptr(y), _dt(y), K, _ptr(weights), _ptr(out),
                             _stream(y.device)))
    return out


def awq_input_backward(route: Optional[RouteState], grad: torch.Tensor, w: AwqExperts,
                       grad_in: Optional[torch.Tensor] = None) -> torch.Tensor:
    wc = w.c()
    rows = grad.shape[0]
    if grad_in is None:
        grad_in = torch.empty(rows, wc.in_features, dtype=grad.dtype, device=grad.device)
    _check(lib().awq_input_backward(None if route is None else C.byref(route.c), _ptr(grad),
                                    _dt(grad), rows, C.byref(wc), _ptr(grad_in),
                                    _stream(grad.device)))
    return grad_in


# ------------------------------------------------------------------ backward path
def moe_combine_backward(route: RouteState, y: torch.Tensor, weights: torch.Tensor,
                         grad: torch.Tensor, experts: bool = True, want_weights: bool = True,
                         grad_y: Optional[torch.Tensor] = None,
                         grad_weights: Optional[torch.Tensor] = None):
    """Combine VJP with a MoeCombineSelection: (grad_y [A,K] or None,
    grad_weights [T,top_k] fp32 or None); only the requested ones are formed."""
    K = y.shape[1]
    gy = gw = None
    if experts:
        gy = torch.empty_like(y) if grad_y is None else grad_y
    if want_weights:
        gw = (torch.empty(route.T, route.top_k, dtype=torch.float32, device=y.device)
              if grad_weights is None else grad_weights)
    _check(lib().moe_combine_backward(C.byref(route.c), _ptr(y), _dt(y), K, _ptr(weights),
                                      _ptr(grad), _ptr(gy), _ptr(gw), _stream(y.device)))
    return gy, gw


def moe_dispatch_backward(route: RouteState, grad: torch.Tensor,
                          grad_x: Optional[torch.Tensor] = None) -> torch.Tensor:
    """COPY VJP: sums each token's expert-sorted row derivatives (no weights)."""
    K = grad.shape[1]
    if grad_x is None:
        grad_x = torch.empty(route.T, K, dtype=grad.dtype, device=grad.device)
    _check(lib().moe_dispatch_backward(C.byref(route.c), _ptr(grad), _dt(grad), K, _ptr(grad_x),
                                       _stream(grad.device)))
    return grad_x


def moe_dispatch_weights_backward(route: RouteState, selected: torch.Tensor,
                                  weights: torch.Tensor, grad_weights: torch.Tensor,
                                  grad_logits: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Fixed-selection logit VJP of the FP32 routing weights: [T, E] fp32."""
    for t in (weights, grad_weights):
        if t.dtype != torch.float32:
            raise MoeqError(EDTYPE, "weights and their gradient are fp32")
    if grad_logits is None:
        grad_logits = torch.empty(route.T, route.E, dtype=torch.float32,
                                  device=weights.device)
    _check(lib().moe_dispatch_weights_backward(C.byref(route.c), _ptr(selected), _ptr(weights),
                                               _ptr(grad_weights), _ptr(grad_logits),
                                               _stream(weights.device)))
    return grad_logits


def awq_swiglu_input_backward_workspace_bytes(rows: int, I: int, dtype: torch.dtype) -> int:
    return int(lib().awq_swiglu_input_backward_workspace_bytes(rows, I,
                                                               _TORCH_DT.get(dtype, 99)))


def awq_swiglu_input_backward(route: RouteState, values: torch.Tensor, gate: AwqExperts,
                              up: AwqExperts, down: AwqExperts, grad: torch.Tensor,
                              clamp: float = 0.0, alpha: float = 1.0, up_offset: float = 0.0,
                              workspace: Optional[torch.Tensor] = None,
                              grad_values: Optional[torch.Tensor] = None,
                              gate_one_sided: bool = False) -> torch.Tensor:
    """Input VJP through down, SwiGLU and gate/up (first order): [A, K] act."""
    gc, uc, dc = gate.c(), up.c(), down.c()
    A = values.shape[0]
    nbytes = awq_swiglu_input_backward_workspace_bytes(A, gc.out_features, values.dtype)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=values.device)
    if grad_values is None:
        grad_values = torch.empty_like(values)
    _check(lib().awq_swiglu_input_backward(C.byref(route.c), _ptr(values), _dt(values),
                                           C.byref(gc), C.byref(uc), C.byref(dc),
                                           SwiGLU(clamp, alpha, up_offset,
                                                  int(gate_one_sided)), _ptr(grad),
                                           _ptr(grad_values), _ptr(workspace),
                                           workspace.numel(), _stream(values.device)))
    return grad_values


# ------------------------------------------------------------------ rows in any order
def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    return workspace


def awq_expert_workspace_bytes(rows: int, experts: int, in_features: int, out_features: int,
                               dtype: torch.dtype) -> int:
    return int(lib().awq_expert_workspace_bytes(rows, experts, in_features, out_features,
                                                _TORCH_DT.get(dtype, 99)))


def awq_expert_forward(x: torch.Tensor, global_ids: torch.Tensor, w,
                       y: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Rows in any order, each with its global expert ID; output in the incoming
    order (packed_experts.rs packed_expert_forward).  Synchronises (ID check)."""
    wc = w.c()
    rows = x.shape[0]
    if y is None:
        y = torch.empty(rows, wc.out_features, dtype=x.dtype, device=x.device)
    nbytes = lib().awq_expert_workspace_bytes(rows, wc.experts, wc.in_features,
                                              wc.out_features, _dt(x))
    workspace = _workspace(nbytes, x.device, workspace)
    _check(lib().awq_expert_forward(_ptr(x), _dt(x), rows, _ptr(global_ids), C.byref(wc),
                                    _ptr(y), _ptr(workspace), workspace.numel(),
                                    _stream(x.device)))
    return y


def awq_expert_input_backward(grad: torch.Tensor, global_ids: torch.Tensor, w: AwqExperts,
                              grad_in: Optional[torch.Tensor] = None,
                              workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Input VJP of awq_expert_forward, rows in the incoming order."""
    wc = w.c()
    rows = grad.shape[0]
    if grad_in is None:
        grad_in = torch.empty(rows, wc.in_features, dtype=grad.dtype, device=grad.device)
    nbytes = lib().awq_expert_workspace_bytes(rows, wc.experts, wc.in_features,
                                              wc.out_features, _dt(grad))
    workspace = _workspace(nbytes, grad.device, workspace)
    _check(lib().awq_expert_input_backward(_ptr(grad), _dt(grad), rows, _ptr(global_ids),
                                           C.byref(wc), _ptr(grad_in), _ptr(workspace),
                                           workspace.numel(), _stream(grad.device)))
    return grad_in


def frozen_awq_forward(x: torch.Tensor, w, y: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One packed projection (a one-expert cube) over all rows (frozen_awq.rs)."""
    wc = w.c()
    rows = x.shape[0]
    if y is None:
        y = torch.empty(rows, wc.out_features, dtype=x.dtype, device=x.device)
    workspace = _workspace(lib().frozen_awq_workspace_bytes(rows), x.device, workspace)
    _check(lib().frozen_awq_forward(_ptr(x), _dt(x), rows, C.byref(wc), _ptr(y),
                                    _ptr(workspace), workspace.numel(), _stream(x.device)))
    return y


# ------------------------------------------------------------------ MXFP8 activations
def mx8_quantize(x: torch.Tensor):
    """OCP MXFP8 quantization of bf16 rows: (codes uint8 [rows, K], scales uint8 [rows, K/32])."""
    rows, K = x.shape
    q = torch.empty(rows, K, dtype=torch.uint8, device=x.device)
    s = torch.empty(rows, K // 32, dtype=torch.uint8, device=x.device)
    _check(lib().mx8_quantize(_ptr(x), _dt(x), rows, K, _ptr(q), _ptr(s), _stream(x.device)))
    return q, s


def _mx8_workspace(rows: int, K: int, device, workspace):
    return _workspace(int(lib().mx8_workspace_bytes(rows, K)), device, workspace)


def mx8_grouped_swiglu(route: RouteState, values: torch.Tensor, gate_up: Mxfp4Bank,
                       clamp: float = 0.0, alpha: float = 1.0, up_offset: float = 0.0,
                       gate_one_sided: bool = False, h: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Interleaved gate/up bank on the block-scaled MFMA with MXFP8 values -> h [A, I] bf16."""
    gc = gate_up.c()
    if h is None:
        h = torch.empty(values.shape[0], gc.out_features // 2, dtype=values.dtype,
                        device=values.device)
    workspace = _mx8_workspace(values.shape[0], gc.in_features, values.device, workspace)
    _check(lib().mx8_grouped_swiglu(C.byref(route.c), _ptr(values), _dt(values), C.byref(gc),
                                    SwiGLU(clamp, alpha, up_offset, int(gate_one_sided)),
                                    _ptr(h), _ptr(workspace), workspace.numel(),
                                    _stream(values.device)))
    return h


def mx8_grouped_down(route: RouteState, h: torch.Tensor, down: Mxfp4Bank,
                     y: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Plain bank on the block-scaled MFMA with MXFP8 h -> y [A, K] bf16."""
    dc = down.c()
    if y is None:
        y = torch.empty(h.shape[0], dc.out_features, dtype=h.dtype, device=h.device)
    workspace = _mx8_workspace(h.shape[0], dc.in_features, h.device, workspace)
    _check(lib().mx8_grouped_down(C.byref(route.c), _ptr(h), _dt(h), C.byref(dc), _ptr(y),
                                  _ptr(workspace), workspace.numel(), _stream(h.device)))
    return y


def moe_ffn(x, logits, expert_bias, top_k, gate, up, down, clamp=0.0, alpha=1.0, up_offset=0.0,
            gate_one_sided=False):
    """The whole forward path: dispatch -> gate/up + SwiGLU -> down -> combine."""
    d = moe_dispatch(x, logits, expert_bias, top_k)
    h = awq_grouped_swiglu(d["route"], d["values"], gate, up, clamp, alpha, up_offset,
                           gate_one_sided=gate_one_sided)
    y = awq_grouped_down(d["route"], h, down)
    return moe_combine(d["route"], y, d["weights"]), d
