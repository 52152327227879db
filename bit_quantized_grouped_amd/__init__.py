"""Python binding of the 4-bit grouped MoE layer's C ABI (include/moe_q4.h).

Argument marshalling only: every step of the layer runs in the HIP kernels
of libmoe_q4.so.  PyTorch is used for device memory and streams.  If the
library has not been built this module raises on first use; there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_Q4_LIB may name another build of the same library (e.g. other tile sizes)
LIB_PATH = os.environ.get("MOE_Q4_LIB") or os.path.join(HERE, "libmoe_q4.so")

MOE_OK = 0
MOE_ERR_NULL = -1
MOE_ERR_SHAPE = -2
MOE_ERR_ALIGN = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_HIP = -5
MOE_ERR_UNIMPLEMENTED = -6


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_str(status)})")


LAYOUT_ROWS = 0      # row-major code words
LAYOUT_TILES = 1     # tile-packed code words (moe_q4_prepack)


class MoeQ4Mat(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p),
                ("layout", ctypes.c_int32)]


class MoeRouting(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "topk_idx", "topk_w", "counts", "offsets", "sorted_assign", "assign_row",
        "block_expert", "block_row", "n_blocks")]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_S = ctypes.c_size_t

_SIGNATURES = {
    "moe_abi_version": (_I, []),
    "moe_status_str": (ctypes.c_char_p, [_I]),
    "moe_route_max_blocks": (_I, [_I, _I, _I, _I]),
    "moe_route_workspace_bytes": (_S, [_I, _I, _I, _I]),
    "moe_route": (_I, [_P, _I, _I, _I, _I, ctypes.POINTER(MoeRouting), _P, _S, _P]),
    "moe_gemm_workspace_bytes": (_S, [_I, _I, _I, _I, _I, _I, _I]),
    "moe_grouped_gemm_q4": (_I, [_P, _I, _I, _I, _I, _I, _I, _I, ctypes.POINTER(MoeRouting)]
                            + [ctypes.POINTER(MoeQ4Mat)] * 6 + [_P, _P, _P, _S, _P]),
    "moe_expert_gateup_q4": (_I, [_P, _I, _I, _I, _I, _I, _I, _I, ctypes.POINTER(MoeRouting)]
                             + [ctypes.POINTER(MoeQ4Mat)] * 4 + [_P, _S, _P]),
    "moe_expert_down_q4": (_I, [_I, _I, _I, _I, _I, _I, _I, ctypes.POINTER(MoeRouting)]
                           + [ctypes.POINTER(MoeQ4Mat)] * 2 + [_P, _P, _P, _S, _P]),
    "moe_layer_q4": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _I] + [ctypes.POINTER(MoeQ4Mat)] * 6
                     + [ctypes.POINTER(MoeRouting), _P, _S, _P, _P, _P, _S, _P, _P]),
    "moe_combine": (_I, [_P, _P, ctypes.POINTER(MoeRouting), _I, _I, _I, _P, _P]),
    "moe_dequant_q4_bf16": (_I, [ctypes.POINTER(MoeQ4Mat), _I, _I, _I, _P, _P, _P]),
    "moe_q4_prepack": (_I, [_P, _I, _I, _I, _P, _P]),
    "moe_combine_gated": (_I, [_P, _P, _P, ctypes.POINTER(MoeRouting), _I, _I, _I, _P, _P]),
    "moe_router": (_I, [_P, _I, _I, _P, _I, _P, _P, _P, _P]),
    "moe_expert_gateup_bf16": (_I, [_P, _I, _I, _I, _I, _I, _I, _I, ctypes.POINTER(MoeRouting)]
                               + [_P] * 4 + [_P, _S, _P]),
    "moe_expert_down_bf16": (_I, [_I, _I, _I, _I, _I, _I, _I, ctypes.POINTER(MoeRouting)]
                             + [_P] * 2 + [_P, _P, _P, _S, _P]),
    "moe_read_probe_sink_words": (_S, [_S]),
    "moe_read_probe": (_I, [_P, _S, _P, _S, _P]),
    "moe_decode_workspace_bytes": (_S, [_I, _I, _I, _I, _I]),
    "moe_decode_q4": (_I, [_P, _P, _I, _I, _I, _I, _I, _I] + [ctypes.POINTER(MoeQ4Mat)] * 6
                      + [ctypes.POINTER(MoeRouting), _P, _P, _S, _P]),
    "moe_decode_q4_sequential": (_I, [_P, _P, _I, _I, _I, _I, _I, _I]
                                 + [ctypes.POINTER(MoeQ4Mat)] * 6 + [_P, _P, _S, _P]),
    "moe_layer_workspace_bytes": (_S, [_I, _I, _I, _I, _I, _I, _I]),
    "moe_layer_chunked": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _I, _I]
                          + [ctypes.POINTER(MoeQ4Mat)] * 6 + [_P, _P, _S, _P]),
}

EXPORTED = tuple(_SIGNATURES)


def lib():
    """The loaded C-ABI library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(python bit_quantized_grouped_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


# ---------------------------------------------------------------------------
# Device containers (plumbing: torch allocations + the C structs over them)
# ---------------------------------------------------------------------------

class DeviceQMat:
    """One 4-bit matrix set [n_exp, N, K] resident on the device."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor,
                 layout: int = LAYOUT_ROWS):
        self.codes, self.scales, self.biases, self.layout = codes, scales, biases, layout
        self.struct = MoeQ4Mat(codes.data_ptr(), scales.data_ptr(), biases.data_ptr(), layout)

    def prepacked(self, stream=None) -> "DeviceQMat":
        """The same matrices with the code words in the tile-packed order (scales and biases
        are shared with this object)."""
        assert self.layout == LAYOUT_ROWS
        n_exp, N, G = self.scales.shape
        dst = torch.empty_like(self.codes)
        _check(lib().moe_q4_prepack(_ptr(self.codes), n_exp, N, G * 64, _ptr(dst),
                                    _stream(stream, dst.device)), "moe_q4_prepack")
        return DeviceQMat(dst, self.scales, self.biases, LAYOUT_TILES)

    @classmethod
    def from_host(cls, m, device) -> "DeviceQMat":
        """m: object with numpy .codes uint32, .scales/.biases uint16."""
        codes = torch.from_numpy(m.codes.view("int32")).to(device)
        scales = torch.from_numpy(m.scales.view("int16")).to(device)
        biases = torch.from_numpy(m.biases.view("int16")).to(device)
        return cls(codes, scales, biases)

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.codes, self.scales, self.biases))


class DeviceRouting:
    """Caller-owned routing output arrays for one layer call of T tokens."""

    def __init__(self, T: int, E: int, k: int, block_rows: int, device):
        self.T, self.E, self.k, self.block_rows = T, E, k, block_rows
        self.max_blocks = route_max_blocks(T, E, k, block_rows)
        i32 = dict(dtype=torch.int32, device=device)
        self.topk_idx = torch.empty((T, k), **i32)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=device)
        self.counts = torch.empty(E, **i32)
        self.offsets = torch.empty(E + 1, **i32)
        self.sorted_assign = torch.empty(T * k, **i32)
        self.assign_row = torch.empty(T * k, **i32)
        self.block_expert = torch.empty(self.max_blocks, **i32)
        self.block_row = torch.empty(self.max_blocks, **i32)
        self.n_blocks = torch.empty(1, **i32)
        self.struct = MoeRouting(*[getattr(self, n).data_ptr() for n, _ in MoeRouting._fields_])

    def to_host(self) -> dict:
        return {n: getattr(self, n).cpu().numpy() for n, _ in MoeRouting._fields_}


# ---------------------------------------------------------------------------
# The C ABI, one Python function per entry point (same names)
# ---------------------------------------------------------------------------

def abi_version() -> int:
    return lib().moe_abi_version()


def route_max_blocks(T, E, k, block_rows) -> int:
    v = lib().moe_route_max_blocks(T, E, k, block_rows)
    _check(min(v, 0), "moe_route_max_blocks")
    return v


def route_workspace_bytes(T, E, k, block_rows) -> int:
    return lib().moe_route_workspace_bytes(T, E, k, block_rows)


def gemm_workspace_bytes(T, H, I, I_sh, E, k, block_rows) -> int:
    return lib().moe_gemm_workspace_bytes(T, H, I, I_sh, E, k, block_rows)


def layer_workspace_bytes(chunk_tokens, H, I, I_sh, E, k, block_rows) -> int:
    return lib().moe_layer_workspace_bytes(chunk_tokens, H, I, I_sh, E, k, block_rows)


def moe_route(logits: torch.Tensor, k: int, block_rows: int, routing: DeviceRouting,
              ws: torch.Tensor, stream=None):
    T, E = logits.shape
    _check(lib().moe_route(_ptr(logits), T, E, k, block_rows, ctypes.byref(routing.struct),
                           _ptr(ws), ws.numel() * ws.element_size(),
                           _stream(stream, logits.device)), "moe_route")


def _mat(m):
    return None if m is None else ctypes.byref(m.struct)


def moe_grouped_gemm_q4(x: torch.Tensor, I: int, I_sh: int, E: int, k: int, block_rows: int,
                        routing: DeviceRouting, gate, up, down, sh_gate, sh_up, sh_down,
                        expert_out: torch.Tensor, shared_out, ws: torch.Tensor, stream=None):
    T, H = x.shape
    _check(lib().moe_grouped_gemm_q4(
        _ptr(x), T, H, I, I_sh, E, k, block_rows, ctypes.byref(routing.struct),
        _mat(gate), _mat(up), _mat(down), _mat(sh_gate), _mat(sh_up), _mat(sh_down),
        _ptr(expert_out), _ptr(shared_out), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream, x.device)), "moe_grouped_gemm_q4")


def moe_expert_gateup_q4(x: torch.Tensor, I: int, I_sh: int, E: int, k: int, block_rows: int,
                         routing: DeviceRouting, gate, up, sh_gate, sh_up, ws: torch.Tensor,
                         stream=None):
    T, H = x.shape
    _check(lib().moe_expert_gateup_q4(
        _ptr(x), T, H, I, I_sh, E, k, block_rows, ctypes.byref(routing.struct),
        _mat(gate), _mat(up), _mat(sh_gate), _mat(sh_up), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream, x.device)), "moe_expert_gateup_q4")


def moe_expert_down_q4(T: int, H: int, I: int, I_sh: int, E: int, k: int, block_rows: int,
                       routing: DeviceRouting, down, sh_down, expert_out: torch.Tensor, shared_out,
                       ws: torch.Tensor, stream=None):
    _check(lib().moe_expert_down_q4(
        T, H, I, I_sh, E, k, block_rows, ctypes.byref(routing.struct), _mat(down), _mat(sh_down),
        _ptr(expert_out), _ptr(shared_out), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream, expert_out.device)), "moe_expert_down_q4")


def moe_layer_q4(x: torch.Tensor, logits: torch.Tensor, I: int, I_sh: int, E: int, k: int,
                 block_rows: int, routing: DeviceRouting, route_ws: torch.Tensor, gate, up, down,
                 sh_gate, sh_up, sh_down, expert_out: torch.Tensor, shared_out,
                 gemm_ws: torch.Tensor, y: torch.Tensor, stream=None):
    T, H = x.shape
    _check(lib().moe_layer_q4(
        _ptr(x), _ptr(logits), T, H, I, I_sh, E, k, block_rows,
        _mat(gate), _mat(up), _mat(down), _mat(sh_gate), _mat(sh_up), _mat(sh_down),
        ctypes.byref(routing.struct), _ptr(route_ws), route_ws.numel() * route_ws.element_size(),
        _ptr(expert_out), _ptr(shared_out), _ptr(gemm_ws),
        gemm_ws.numel() * gemm_ws.element_size(), _ptr(y), _stream(stream, x.device)),
        "moe_layer_q4")


def moe_combine(expert_out: torch.Tensor, shared_out, routing: DeviceRouting, k: int,
                y: torch.Tensor, stream=None):
    T, H = y.shape
    _check(lib().moe_combine(_ptr(expert_out), _ptr(shared_out), ctypes.byref(routing.struct),
                             T, H, k, _ptr(y), _stream(stream, y.device)), "moe_combine")


def moe_dequant_q4_bf16(m: DeviceQMat, n_exp: int, N: int, K: int, out: torch.Tensor, counts=None,
                        stream=None):
    """Expand a 4-bit matrix set [n_exp, N, K] into bf16 `out` [n_exp, N, K]; experts with
    counts[e] == 0 are skipped when counts (device int32 [n_exp]) is given."""
    _check(lib().moe_dequant_q4_bf16(ctypes.byref(m.struct), n_exp, N, K, _ptr(counts), _ptr(out),
                                     _stream(stream, out.device)), "moe_dequant_q4_bf16")


def moe_expert_gateup_bf16(x: torch.Tensor, I: int, I_sh: int, E: int, k: int, block_rows: int,
                           routing: DeviceRouting, gate, up, sh_gate, sh_up, ws: torch.Tensor,
                           stream=None):
    """moe_expert_gateup_q4 over bf16 weight tensors (gate/up [E, I, H], shared [1, I_sh, H])."""
    T, H = x.shape
    _check(lib().moe_expert_gateup_bf16(
        _ptr(x), T, H, I, I_sh, E, k, block_rows, ctypes.byref(routing.struct),
        _ptr(gate), _ptr(up), _ptr(sh_gate), _ptr(sh_up), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream, x.device)), "moe_expert_gateup_bf16")


def moe_expert_down_bf16(T: int, H: int, I: int, I_sh: int, E: int, k: int, block_rows: int,
                         routing: DeviceRouting, down, sh_down, expert_out: torch.Tensor, shared_out,
                         ws: torch.Tensor, stream=None):
    """moe_expert_down_q4 over bf16 weight tensors (down [E, H, I], shared [1, H, I_sh])."""
    _check(lib().moe_expert_down_bf16(
        T, H, I, I_sh, E, k, block_rows, ctypes.byref(routing.struct), _ptr(down), _ptr(sh_down),
        _ptr(expert_out), _ptr(shared_out), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream, expert_out.device)), "moe_expert_down_bf16")


def moe_combine_gated(expert_out: torch.Tensor, shared_out: torch.Tensor, shared_gate: torch.Tensor,
                      routing: DeviceRouting, k: int, y: torch.Tensor, stream=None):
    """moe_combine with the shared expert weighted per token by shared_gate (fp32 [T])."""
    T, H = y.shape
    _check(lib().moe_combine_gated(_ptr(expert_out), _ptr(shared_out), _ptr(shared_gate),
                                   ctypes.byref(routing.struct), T, H, k, _ptr(y),
                                   _stream(stream, y.device)), "moe_combine_gated")


def moe_router(x: torch.Tensor, w_router: torch.Tensor, logits: torch.Tensor, w_gate=None,
               gate=None, stream=None):
    """logits [T, E] (fp32) = x [T, H] (bf16) @ w_router [E, H]^T; optionally
    gate [T] = sigmoid(x @ w_gate)."""
    T, H = x.shape
    E = w_router.shape[0]
    _check(lib().moe_router(_ptr(x), T, H, _ptr(w_router), E, _ptr(w_gate), _ptr(logits),
                            _ptr(gate), _stream(stream, x.device)), "moe_router")


def read_probe_sink_words(nbytes: int) -> int:
    return lib().moe_read_probe_sink_words(nbytes)


def moe_read_probe(buf: torch.Tensor, sink: torch.Tensor, stream=None):
    """Stream every byte of buf once; sink[i] = XOR of the uint32 words of 32 KB range i."""
    _check(lib().moe_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                sink.numel() * sink.element_size() // 4,
                                _stream(stream, buf.device)), "moe_read_probe")


def decode_workspace_bytes(H, I, I_sh, E, k) -> int:
    return lib().moe_decode_workspace_bytes(H, I, I_sh, E, k)


def moe_decode_q4(x: torch.Tensor, logits: torch.Tensor, I: int, I_sh: int, k: int,
                  block_rows: int, gate, up, down, sh_gate, sh_up, sh_down, routing, y: torch.Tensor,
                  ws: torch.Tensor, stream=None):
    """One token (x [1, H], logits [1, E]) through the whole layer in one launch."""
    H = x.shape[1]
    E = logits.shape[1]
    _check(lib().moe_decode_q4(
        _ptr(x), _ptr(logits), H, I, I_sh, E, k, block_rows, _mat(gate), _mat(up), _mat(down),
        _mat(sh_gate), _mat(sh_up), _mat(sh_down),
        None if routing is None else ctypes.byref(routing.struct), _ptr(y), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream, x.device)), "moe_decode_q4")


def moe_decode_q4_sequential(x: torch.Tensor, logits: torch.Tensor, I: int, I_sh: int, k: int,
                             gate, up, down, sh_gate, sh_up, sh_down, y: torch.Tensor,
                             ws: torch.Tensor, stream=None):
    """x [n, H], logits [n, E]: n single-token decode launches back to back."""
    n, H = x.shape
    E = logits.shape[1]
    _check(lib().moe_decode_q4_sequential(
        _ptr(x), _ptr(logits), n, H, I, I_sh, E, k, _mat(gate), _mat(up), _mat(down),
        _mat(sh_gate), _mat(sh_up), _mat(sh_down), _ptr(y), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream, x.device)), "moe_decode_q4_sequential")


def moe_layer_chunked(x: torch.Tensor, logits: torch.Tensor, I: int, I_sh: int, k: int,
                      block_rows: int, chunk_tokens: int, gate, up, down, sh_gate, sh_up,
                      sh_down, y: torch.Tensor, ws: torch.Tensor, stream=None):
    T, H = x.shape
    E = logits.shape[1]
    _check(lib().moe_layer_chunked(
        _ptr(x), _ptr(logits), T, H, I, I_sh, E, k, block_rows, chunk_tokens,
        _mat(gate), _mat(up), _mat(down), _mat(sh_gate), _mat(sh_up), _mat(sh_down),
        _ptr(y), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream, x.device)),
        "moe_layer_chunked")


# ---------------------------------------------------------------------------
# Convenience: one layer's device weights and buffers, running the three calls
# ---------------------------------------------------------------------------

def _bytes_tensor(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


class MoeLayer:
    """Device-resident weights of one layer plus per-call buffers for T tokens."""

    def __init__(self, weights, H: int, I: int, I_sh: int, E: int, k: int, device,
                 block_rows: int = 32, prepack: bool = False):
        self.H, self.I, self.I_sh, self.E, self.k = H, I, I_sh, E, k
        self.block_rows = block_rows
        self.device = torch.device(device)
        up = lambda m: None if m is None else DeviceQMat.from_host(m, self.device)  # noqa: E731
        self.gate, self.up, self.down = up(weights.gate), up(weights.up), up(weights.down)
        self.sh_gate, self.sh_up, self.sh_down = (up(weights.sh_gate), up(weights.sh_up),
                                                  up(weights.sh_down))
        if prepack:   # load time: code words into the tile-packed order, row-major copies freed
            for name in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down"):
                m = getattr(self, name)
                if m is not None:
                    setattr(self, name, m.prepacked())
            torch.cuda.synchronize(self.device)
        self._bufs = {}

    @classmethod
    def from_device(cls, mats, H: int, I: int, I_sh: int, E: int, k: int, device,
                    block_rows: int = 32) -> "MoeLayer":
        """A layer over device-resident DeviceQMat objects (gate, up, down, sh_gate, sh_up,
        sh_down; the shared three may be None)."""
        layer = cls.__new__(cls)
        layer.H, layer.I, layer.I_sh, layer.E, layer.k = H, I, I_sh, E, k
        layer.block_rows = block_rows
        layer.device = torch.device(device)
        (layer.gate, layer.up, layer.down, layer.sh_gate, layer.sh_up, layer.sh_down) = mats
        layer._bufs = {}
        return layer

    def weight_mats(self):
        return (self.gate, self.up, self.down, self.sh_gate, self.sh_up, self.sh_down)

    def buffers(self, T: int) -> dict:
        if T not in self._bufs:
            d = self.device
            b = dict(
                routing=DeviceRouting(T, self.E, self.k, self.block_rows, d),
                route_ws=_bytes_tensor(route_workspace_bytes(T, self.E, self.k, self.block_rows), d),
                gemm_ws=_bytes_tensor(gemm_workspace_bytes(T, self.H, self.I, self.I_sh, self.E,
                                                           self.k, self.block_rows), d),
                expert_out=torch.empty((T * self.k, self.H), dtype=torch.bfloat16, device=d),
                shared_out=(torch.empty((T, self.H), dtype=torch.bfloat16, device=d)
                            if self.I_sh else None),
                y=torch.empty((T, self.H), dtype=torch.bfloat16, device=d),
            )
            self._bufs[T] = b
        return self._bufs[T]

    def forward(self, x: torch.Tensor, logits: torch.Tensor, out: torch.Tensor | None = None,
                stream=None) -> dict:
        """One moe_layer_q4 call (route -> grouped GEMM -> combine on one stream);
        returns the buffers used."""
        T = x.shape[0]
        b = self.buffers(T)
        y = b["y"] if out is None else out
        moe_layer_q4(x, logits, self.I, self.I_sh, self.E, self.k, self.block_rows, b["routing"],
                     b["route_ws"], *self.weight_mats(), b["expert_out"], b["shared_out"],
                     b["gemm_ws"], y, stream)
        return dict(b, y=y)

    def forward_three_calls(self, x: torch.Tensor, logits: torch.Tensor,
                            out: torch.Tensor | None = None, stream=None) -> dict:
        """moe_route, moe_grouped_gemm_q4 and moe_combine in order on one stream."""
        T = x.shape[0]
        b = self.buffers(T)
        y = b["y"] if out is None else out
        moe_route(logits, self.k, self.block_rows, b["routing"], b["route_ws"], stream)
        moe_grouped_gemm_q4(x, self.I, self.I_sh, self.E, self.k, self.block_rows, b["routing"],
                            *self.weight_mats(), b["expert_out"], b["shared_out"], b["gemm_ws"],
                            stream)
        moe_combine(b["expert_out"], b["shared_out"], b["routing"], self.k, y, stream)
        return dict(b, y=y)

    def decode(self, x: torch.Tensor, logits: torch.Tensor, y: torch.Tensor, routing=None,
               ws=None, stream=None):
        """One token through the batch-1 decode path (two launches); returns the workspace."""
        if ws is None:
            ws = _bytes_tensor(decode_workspace_bytes(self.H, self.I, self.I_sh, self.E, self.k),
                               self.device)
        moe_decode_q4(x, logits, self.I, self.I_sh, self.k, self.block_rows, *self.weight_mats(),
                      routing, y, ws, stream)
        return ws

    def bf16_weights(self) -> dict:
        """Device buffers for the weights expanded to bf16 (allocated once, reused)."""
        if not hasattr(self, "_bf16"):
            d, E, H, I, Is = self.device, self.E, self.H, self.I, self.I_sh
            bf = lambda *shape: torch.empty(shape, dtype=torch.bfloat16, device=d)  # noqa: E731
            self._bf16 = dict(gate=bf(E, I, H), up=bf(E, I, H), down=bf(E, H, I),
                              sh_gate=bf(1, Is, H) if Is else None,
                              sh_up=bf(1, Is, H) if Is else None,
                              sh_down=bf(1, H, Is) if Is else None)
        return self._bf16

    def forward_unfused(self, x: torch.Tensor, logits: torch.Tensor, stream=None) -> dict:
        """The unfused baseline: route, expand the routed experts' and the shared expert's
        4-bit weights to bf16 in memory, then the two GEMM phases over the bf16 weights,
        then combine; returns the buffers used."""
        T = x.shape[0]
        b = self.buffers(T)
        r = b["routing"]
        E, H, I, Is = self.E, self.H, self.I, self.I_sh
        moe_route(logits, self.k, self.block_rows, r, b["route_ws"], stream)
        w = self.bf16_weights()
        for name, m, shape, counts in (("gate", self.gate, (E, I, H), r.counts),
                                       ("up", self.up, (E, I, H), r.counts),
                                       ("down", self.down, (E, H, I), r.counts),
                                       ("sh_gate", self.sh_gate, (1, Is, H), None),
                                       ("sh_up", self.sh_up, (1, Is, H), None),
                                       ("sh_down", self.sh_down, (1, H, Is), None)):
            if m is not None:
                moe_dequant_q4_bf16(m, *shape, w[name], counts, stream)
        moe_expert_gateup_bf16(x, I, Is, E, self.k, self.block_rows, r, w["gate"], w["up"],
                               w["sh_gate"], w["sh_up"], b["gemm_ws"], stream)
        moe_expert_down_bf16(T, H, I, Is, E, self.k, self.block_rows, r, w["down"], w["sh_down"],
                             b["expert_out"], b["shared_out"], b["gemm_ws"], stream)
        moe_combine(b["expert_out"], b["shared_out"], r, self.k, b["y"], stream)
        return b

    def forward_chunked(self, x, logits, chunk_tokens: int, y: torch.Tensor, ws=None, stream=None):
        T = x.shape[0]
        if ws is None:
            ws = _bytes_tensor(layer_workspace_bytes(min(chunk_tokens, T), self.H, self.I,
                                                     self.I_sh, self.E, self.k, self.block_rows),
                               self.device)
        moe_layer_chunked(x, logits, self.I, self.I_sh, self.k, self.block_rows, chunk_tokens,
                          *self.weight_mats(), y, ws, stream)
        return ws


def bf16_from_bits(bits_np, device) -> torch.Tensor:
    """uint16 bf16 bit patterns (numpy) -> bf16 device tensor (a reinterpreting copy)."""
    return torch.from_numpy(bits_np.view("int16")).to(device).view(torch.bfloat16)


def bf16_to_bits(t: torch.Tensor):
    """bf16 tensor -> uint16 numpy bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view("uint16")
