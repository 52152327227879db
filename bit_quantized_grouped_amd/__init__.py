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
# the in-tree build of build.py; no other library can be substituted
LIB_PATH = os.path.join(HERE, "libmoe_q4.so")

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
LAYOUT_TILES_SB = 2  # tile-packed code words + packed scale|bias words (moe_q4_pack_scales)


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
    "moe_q4_pack_scales": (_I, [_P, _P, _I, _I, _I, _P, _P]),
    "moe_combine_gated": (_I, [_P, _P, _P, ctypes.POINTER(MoeRouting), _I, _I, _I, _P, _P]),
    "moe_router": (_I, [_P, _I, _I, _P, _I, _P, _P, _P, _P]),
    "moe_expert_gateup_bf16": (_I, [_P, _I, _I, _I, _I, _I, _I, _I, ctypes.POINTER(MoeRouting)]
                               + [_P] * 4 + [_P, _S, _P]),
    "moe_expert_down_bf16": (_I, [_I, _I, _I, _I, _I, _I, _I, ctypes.POINTER(MoeRouting)]
                             + [_P] * 2 + [_P, _P, _P, _S, _P]),
    "moe_read_probe_sink_words": (_S, [_S]),
    "moe_read_probe": (_I, [_P, _S, _P, _S, _P]),
    "moe_launch_probe": (_I, [_P, _I, _I, _I, _I, _I, _I, _P]),
    "moe_decode_workspace_bytes": (_S, [_I, _I, _I, _I, _I]),
    "moe_decode_q4": (_I, [_P, _P, _I, _I, _I, _I, _I, _I] + [ctypes.POINTER(MoeQ4Mat)] * 6
                      + [ctypes.POINTER(MoeRouting), _P, _P, _S, _P]),
    "moe_decode_noalloc_max_bytes": (_S, []),
    "moe_decode_q4_noalloc": (_I, [_P, _P, _I, _I, _I, _I, _I, _I] + [ctypes.POINTER(MoeQ4Mat)] * 6
                              + [ctypes.POINTER(MoeRouting), _P, _P]),
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


def lib_fingerprint() -> dict:
    """Path and SHA-256 (first 16 hex digits) of the library this process loads."""
    import hashlib
    with open(LIB_PATH, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()[:16]
    return {"path": LIB_PATH, "sha256_16": digest}


def status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def _ptr(t):
    """Device address of t for the C call (None for None)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"arguments must be device tensors (got a tensor on {t.device})")
    return ctypes.c_void_p(t.data_ptr())


# ---------------------------------------------------------------------------
# Argument checks.  The C ABI sees only pointers and sizes, so a tensor of the
# wrong dtype, shape or layout, or routing arrays built for another call,
# would reach the kernels as out-of-range addresses.  These checks run before
# any C call; they raise TypeError (dtype) or ValueError (everything else).
# ---------------------------------------------------------------------------

def _tensor(t, name, dtype=None, shape=None):
    """t must be a contiguous device tensor, of `dtype` and `shape` when given."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t     # the device is checked when the address is taken (_ptr, _mat, _rt)


def _opt_tensor(t, name, present: bool, dtype=None, shape=None):
    """t is required when `present`, and must be None otherwise."""
    if not present:
        if t is not None:
            raise ValueError(f"{name}: must be None here")
        return None
    if t is None:
        raise ValueError(f"{name}: required")
    return _tensor(t, name, dtype, shape)


def _ws(t, name="ws"):
    """A workspace: any contiguous device tensor (its byte size is checked by the library)."""
    return _tensor(t, name)


def _routing_for(r, name, T, E, k, block_rows):
    if not isinstance(r, DeviceRouting):
        raise TypeError(f"{name}: expected a DeviceRouting")
    if (r.T, r.E, r.k, r.block_rows) != (T, E, k, block_rows):
        raise ValueError(f"{name}: built for T={r.T} E={r.E} k={r.k} block_rows={r.block_rows}, "
                         f"the call has T={T} E={E} k={k} block_rows={block_rows}")
    return r


def _qmat_for(m, name, n_exp, N, K, present=True):
    if not present:
        if m is not None:
            raise ValueError(f"{name}: must be None here")
        return None
    if not isinstance(m, DeviceQMat):
        raise TypeError(f"{name}: expected a DeviceQMat")
    packed = m.layout == LAYOUT_TILES_SB
    b_shape = None if m.biases is None else tuple(m.biases.shape)
    if K % 64 or (tuple(m.codes.shape), tuple(m.scales.shape), b_shape) != (
            (n_exp, N, K // 8), (n_exp, N, K // 64), None if packed else (n_exp, N, K // 64)):
        raise ValueError(f"{name}: codes {tuple(m.codes.shape)}, scales {tuple(m.scales.shape)}, "
                         f"biases {b_shape} do not hold a [{n_exp}, {N}, {K}] set"
                         + (" with packed scale|bias words" if packed else ""))
    for part in ("codes", "scales", "biases"):
        if getattr(m, part) is not None:
            _tensor(getattr(m, part), f"{name}.{part}")
    return m


def _expert_mats(gate, up, down, sh_gate, sh_up, sh_down, E, H, I, I_sh):
    """Check the six matrix sets of a layer (down or the gate/up pair may be skipped by
    passing False for them)."""
    if gate is not False:
        _qmat_for(gate, "gate", E, I, H)
        _qmat_for(up, "up", E, I, H)
        _qmat_for(sh_gate, "sh_gate", 1, I_sh, H, present=I_sh > 0)
        _qmat_for(sh_up, "sh_up", 1, I_sh, H, present=I_sh > 0)
    if down is not False:
        _qmat_for(down, "down", E, H, I)
        _qmat_for(sh_down, "sh_down", 1, H, I_sh, present=I_sh > 0)


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


# ---------------------------------------------------------------------------
# Device containers (plumbing: torch allocations + the C structs over them)
# ---------------------------------------------------------------------------

class DeviceQMat:
    """One 4-bit matrix set [n_exp, N, K] resident on the device."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor, biases,
                 layout: int = LAYOUT_ROWS, plain=None):
        """layout LAYOUT_TILES_SB: scales holds the packed scale|bias words (int32, same
        shape as the bf16 scales) and biases is None; plain optionally keeps the bf16
        (scales, biases) they were packed from, for the row-wise readers (decode)."""
        self.codes, self.scales, self.biases, self.layout = codes, scales, biases, layout
        self.plain = plain
        self.struct = MoeQ4Mat(codes.data_ptr(), scales.data_ptr(),
                               None if biases is None else biases.data_ptr(), layout)

    def row_view(self) -> "DeviceQMat":
        """The matrices for calls that read scales row by row (batch-1 decode): a
        LAYOUT_TILES view over the same code words and the plain scales, when this
        object has packed scale|bias words and kept the plain ones; else itself."""
        if self.layout == LAYOUT_TILES_SB and self.plain is not None:
            return DeviceQMat(self.codes, self.plain[0], self.plain[1], LAYOUT_TILES)
        return self

    def prepacked(self, pack_scales: bool = False, stream=None) -> "DeviceQMat":
        """The same matrices with the code words in the tile-packed order (load time); with
        pack_scales also the scales and biases packed into scale|bias words
        (LAYOUT_TILES_SB), else shared with this object (LAYOUT_TILES)."""
        assert self.layout == LAYOUT_ROWS
        n_exp, N, G = self.scales.shape
        dst = torch.empty_like(self.codes)
        st = _stream(stream, dst.device)
        _check(lib().moe_q4_prepack(_ptr(self.codes), n_exp, N, G * 64, _ptr(dst), st),
               "moe_q4_prepack")
        if not pack_scales:
            return DeviceQMat(dst, self.scales, self.biases, LAYOUT_TILES)
        sb = torch.empty((n_exp, N, G), dtype=torch.int32, device=dst.device)
        _check(lib().moe_q4_pack_scales(_ptr(self.scales), _ptr(self.biases), n_exp, N, G * 64,
                                        _ptr(sb), st), "moe_q4_pack_scales")
        return DeviceQMat(dst, sb, None, LAYOUT_TILES_SB, plain=(self.scales, self.biases))

    @classmethod
    def from_host(cls, m, device) -> "DeviceQMat":
        """m: object with numpy .codes uint32, .scales/.biases uint16."""
        codes = torch.from_numpy(m.codes.view("int32")).to(device)
        scales = torch.from_numpy(m.scales.view("int16")).to(device)
        biases = torch.from_numpy(m.biases.view("int16")).to(device)
        return cls(codes, scales, biases)

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.codes, self.scales, self.biases)
                   if t is not None)


def prepacked_mats(mats, pack_scales: bool = True, stream=None):
    """Load time: a layer's six row-major matrix sets (gate, up, down, sh_gate, sh_up,
    sh_down; None skipped) with tile-packed code words, and with pack_scales the gate and
    up sets' scales and biases packed too (LAYOUT_TILES_SB; the down sets stay
    LAYOUT_TILES)."""
    return tuple(None if m is None else m.prepacked(pack_scales and i in (0, 1, 3, 4), stream)
                 for i, m in enumerate(mats))


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


BF16, F32, I32 = torch.bfloat16, torch.float32, torch.int32


def moe_route(logits: torch.Tensor, k: int, block_rows: int, routing: DeviceRouting,
              ws: torch.Tensor, stream=None):
    _tensor(logits, "logits", F32)
    if logits.dim() != 2:
        raise ValueError("logits: expected [T, E]")
    T, E = logits.shape
    _routing_for(routing, "routing", T, E, k, block_rows)
    _ws(ws, "route_ws")
    _check(lib().moe_route(_ptr(logits), T, E, k, block_rows, _rt(routing),
                           _ptr(ws), ws.numel() * ws.element_size(),
                           _stream(stream, logits.device)), "moe_route")


def _mat(m):
    if m is None:
        return None
    for part in (m.codes, m.scales, m.biases):
        _ptr(part)
    return ctypes.byref(m.struct)


def _rt(r):
    _ptr(r.topk_idx)
    return ctypes.byref(r.struct)


def _x_of(x):
    _tensor(x, "x", BF16)
    if x.dim() != 2:
        raise ValueError("x: expected [T, H]")
    return x.shape


def moe_grouped_gemm_q4(x: torch.Tensor, I: int, I_sh: int, E: int, k: int, block_rows: int,
                        routing: DeviceRouting, gate, up, down, sh_gate, sh_up, sh_down,
                        expert_out: torch.Tensor, shared_out, ws: torch.Tensor, stream=None):
    T, H = _x_of(x)
    _routing_for(routing, "routing", T, E, k, block_rows)
    _expert_mats(gate, up, down, sh_gate, sh_up, sh_down, E, H, I, I_sh)
    _tensor(expert_out, "expert_out", BF16, (T * k, H))
    _opt_tensor(shared_out, "shared_out", I_sh > 0, BF16, (T, H))
    _ws(ws)
    _check(lib().moe_grouped_gemm_q4(
        _ptr(x), T, H, I, I_sh, E, k, block_rows, _rt(routing),
        _mat(gate), _mat(up), _mat(down), _mat(sh_gate), _mat(sh_up), _mat(sh_down),
        _ptr(expert_out), _ptr(shared_out), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream, x.device)), "moe_grouped_gemm_q4")


def moe_expert_gateup_q4(x: torch.Tensor, I: int, I_sh: int, E: int, k: int, block_rows: int,
                         routing: DeviceRouting, gate, up, sh_gate, sh_up, ws: torch.Tensor,
                         stream=None):
    T, H = _x_of(x)
    _routing_for(routing, "routing", T, E, k, block_rows)
    _expert_mats(gate, up, False, sh_gate, sh_up, None, E, H, I, I_sh)
    _ws(ws)
    _check(lib().moe_expert_gateup_q4(
        _ptr(x), T, H, I, I_sh, E, k, block_rows, _rt(routing),
        _mat(gate), _mat(up), _mat(sh_gate), _mat(sh_up), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream, x.device)), "moe_expert_gateup_q4")


def moe_expert_down_q4(T: int, H: int, I: int, I_sh: int, E: int, k: int, block_rows: int,
                       routing: DeviceRouting, down, sh_down, expert_out: torch.Tensor, shared_out,
                       ws: torch.Tensor, stream=None):
    _routing_for(routing, "routing", T, E, k, block_rows)
    _expert_mats(False, None, down, None, None, sh_down, E, H, I, I_sh)
    _tensor(expert_out, "expert_out", BF16, (T * k, H))
    _opt_tensor(shared_out, "shared_out", I_sh > 0, BF16, (T, H))
    _ws(ws)
    _check(lib().moe_expert_down_q4(
        T, H, I, I_sh, E, k, block_rows, _rt(routing), _mat(down), _mat(sh_down),
        _ptr(expert_out), _ptr(shared_out), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream, expert_out.device)), "moe_expert_down_q4")


def moe_layer_q4(x: torch.Tensor, logits: torch.Tensor, I: int, I_sh: int, E: int, k: int,
                 block_rows: int, routing: DeviceRouting, route_ws: torch.Tensor, gate, up, down,
                 sh_gate, sh_up, sh_down, expert_out: torch.Tensor, shared_out,
                 gemm_ws: torch.Tensor, y: torch.Tensor, stream=None):
    T, H = _x_of(x)
    _tensor(logits, "logits", F32, (T, E))
    _routing_for(routing, "routing", T, E, k, block_rows)
    _expert_mats(gate, up, down, sh_gate, sh_up, sh_down, E, H, I, I_sh)
    _tensor(expert_out, "expert_out", BF16, (T * k, H))
    _opt_tensor(shared_out, "shared_out", I_sh > 0, BF16, (T, H))
    _tensor(y, "y", BF16, (T, H))
    _ws(route_ws, "route_ws")
    _ws(gemm_ws, "gemm_ws")
    _check(lib().moe_layer_q4(
        _ptr(x), _ptr(logits), T, H, I, I_sh, E, k, block_rows,
        _mat(gate), _mat(up), _mat(down), _mat(sh_gate), _mat(sh_up), _mat(sh_down),
        _rt(routing), _ptr(route_ws), route_ws.numel() * route_ws.element_size(),
        _ptr(expert_out), _ptr(shared_out), _ptr(gemm_ws),
        gemm_ws.numel() * gemm_ws.element_size(), _ptr(y), _stream(stream, x.device)),
        "moe_layer_q4")


def moe_combine(expert_out: torch.Tensor, shared_out, routing: DeviceRouting, k: int,
                y: torch.Tensor, stream=None):
    _tensor(y, "y", BF16)
    if y.dim() != 2:
        raise ValueError("y: expected [T, H]")
    T, H = y.shape
    if not isinstance(routing, DeviceRouting) or (routing.T, routing.k) != (T, k):
        raise ValueError("routing: not built for this call's T and k")
    _tensor(expert_out, "expert_out", BF16, (T * k, H))
    if shared_out is not None:
        _tensor(shared_out, "shared_out", BF16, (T, H))
    _check(lib().moe_combine(_ptr(expert_out), _ptr(shared_out), _rt(routing),
                             T, H, k, _ptr(y), _stream(stream, y.device)), "moe_combine")


def moe_dequant_q4_bf16(m: DeviceQMat, n_exp: int, N: int, K: int, out: torch.Tensor, counts=None,
                        stream=None):
    """Expand a 4-bit matrix set [n_exp, N, K] into bf16 `out` [n_exp, N, K]; experts with
    counts[e] == 0 are skipped when counts (device int32 [n_exp]) is given."""
    _qmat_for(m, "m", n_exp, N, K)
    _tensor(out, "out", BF16, (n_exp, N, K))
    if counts is not None:
        _tensor(counts, "counts", I32, (n_exp,))
    _check(lib().moe_dequant_q4_bf16(ctypes.byref(m.struct), n_exp, N, K, _ptr(counts), _ptr(out),
                                     _stream(stream, out.device)), "moe_dequant_q4_bf16")


def moe_expert_gateup_bf16(x: torch.Tensor, I: int, I_sh: int, E: int, k: int, block_rows: int,
                           routing: DeviceRouting, gate, up, sh_gate, sh_up, ws: torch.Tensor,
                           stream=None):
    """moe_expert_gateup_q4 over bf16 weight tensors (gate/up [E, I, H], shared [1, I_sh, H])."""
    T, H = _x_of(x)
    _routing_for(routing, "routing", T, E, k, block_rows)
    _tensor(gate, "gate", BF16, (E, I, H))
    _tensor(up, "up", BF16, (E, I, H))
    _opt_tensor(sh_gate, "sh_gate", I_sh > 0, BF16, (1, I_sh, H))
    _opt_tensor(sh_up, "sh_up", I_sh > 0, BF16, (1, I_sh, H))
    _ws(ws)
    _check(lib().moe_expert_gateup_bf16(
        _ptr(x), T, H, I, I_sh, E, k, block_rows, _rt(routing),
        _ptr(gate), _ptr(up), _ptr(sh_gate), _ptr(sh_up), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream, x.device)), "moe_expert_gateup_bf16")


def moe_expert_down_bf16(T: int, H: int, I: int, I_sh: int, E: int, k: int, block_rows: int,
                         routing: DeviceRouting, down, sh_down, expert_out: torch.Tensor, shared_out,
                         ws: torch.Tensor, stream=None):
    """moe_expert_down_q4 over bf16 weight tensors (down [E, H, I], shared [1, H, I_sh])."""
    _routing_for(routing, "routing", T, E, k, block_rows)
    _tensor(down, "down", BF16, (E, H, I))
    _opt_tensor(sh_down, "sh_down", I_sh > 0, BF16, (1, H, I_sh))
    _tensor(expert_out, "expert_out", BF16, (T * k, H))
    _opt_tensor(shared_out, "shared_out", I_sh > 0, BF16, (T, H))
    _ws(ws)
    _check(lib().moe_expert_down_bf16(
        T, H, I, I_sh, E, k, block_rows, _rt(routing), _ptr(down), _ptr(sh_down),
        _ptr(expert_out), _ptr(shared_out), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream, expert_out.device)), "moe_expert_down_bf16")


def moe_combine_gated(expert_out: torch.Tensor, shared_out: torch.Tensor, shared_gate: torch.Tensor,
                      routing: DeviceRouting, k: int, y: torch.Tensor, stream=None):
    """moe_combine with the shared expert weighted per token by shared_gate (fp32 [T])."""
    _tensor(y, "y", BF16)
    if y.dim() != 2:
        raise ValueError("y: expected [T, H]")
    T, H = y.shape
    if not isinstance(routing, DeviceRouting) or (routing.T, routing.k) != (T, k):
        raise ValueError("routing: not built for this call's T and k")
    _tensor(expert_out, "expert_out", BF16, (T * k, H))
    _tensor(shared_out, "shared_out", BF16, (T, H))
    _tensor(shared_gate, "shared_gate", F32, (T,))
    _check(lib().moe_combine_gated(_ptr(expert_out), _ptr(shared_out), _ptr(shared_gate),
                                   _rt(routing), T, H, k, _ptr(y),
                                   _stream(stream, y.device)), "moe_combine_gated")


def moe_router(x: torch.Tensor, w_router: torch.Tensor, logits: torch.Tensor, w_gate=None,
               gate=None, stream=None):
    """logits [T, E] (fp32) = x [T, H] (bf16) @ w_router [E, H]^T; optionally
    gate [T] = sigmoid(x @ w_gate)."""
    T, H = _x_of(x)
    _tensor(w_router, "w_router", BF16)
    if w_router.dim() != 2 or w_router.shape[1] != H:
        raise ValueError("w_router: expected [E, H]")
    E = w_router.shape[0]
    _tensor(logits, "logits", F32, (T, E))
    if (w_gate is None) != (gate is None):
        raise ValueError("w_gate and gate: both given or both None")
    if w_gate is not None:
        _tensor(w_gate, "w_gate", BF16, (H,))
        _tensor(gate, "gate", F32, (T,))
    _check(lib().moe_router(_ptr(x), T, H, _ptr(w_router), E, _ptr(w_gate), _ptr(logits),
                            _ptr(gate), _stream(stream, x.device)), "moe_router")


def read_probe_sink_words(nbytes: int) -> int:
    return lib().moe_read_probe_sink_words(nbytes)


def moe_read_probe(buf: torch.Tensor, sink: torch.Tensor, stream=None):
    """Stream every byte of buf once; sink[i] = XOR of the uint32 words of 32 KB range i."""
    _tensor(buf, "buf")
    _tensor(sink, "sink")
    _check(lib().moe_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                sink.numel() * sink.element_size() // 4,
                                _stream(stream, buf.device)), "moe_read_probe")


def moe_launch_probe(buf: torch.Tensor, n_launches: int, shape_a, shape_b, dep: bool,
                     stream=None):
    """n_launches kernels alternating (grid, threads) shape_a and shape_b; dep: each reads the
    word the previous one wrote (buf: int32 [3] on the device)."""
    _tensor(buf, "buf", I32, (3,))
    _check(lib().moe_launch_probe(_ptr(buf), n_launches, shape_a[0], shape_a[1], shape_b[0],
                                  shape_b[1], int(dep), _stream(stream, buf.device)),
           "moe_launch_probe")


def decode_workspace_bytes(H, I, I_sh, E, k) -> int:
    return lib().moe_decode_workspace_bytes(H, I, I_sh, E, k)


def moe_decode_q4(x: torch.Tensor, logits: torch.Tensor, I: int, I_sh: int, k: int,
                  block_rows: int, gate, up, down, sh_gate, sh_up, sh_down, routing, y: torch.Tensor,
                  ws: torch.Tensor, stream=None):
    """One token (x [1, H], logits [1, E]) through the whole layer (two launches)."""
    _, H = _x_of(x)
    _tensor(x, "x", BF16, (1, H))
    _tensor(logits, "logits", F32)
    if logits.dim() != 2 or logits.shape[0] != 1:
        raise ValueError("logits: expected [1, E]")
    E = logits.shape[1]
    _expert_mats(gate, up, down, sh_gate, sh_up, sh_down, E, H, I, I_sh)
    if routing is not None:
        _routing_for(routing, "routing", 1, E, k, block_rows)
    _tensor(y, "y", BF16, (1, H))
    _ws(ws)
    _check(lib().moe_decode_q4(
        _ptr(x), _ptr(logits), H, I, I_sh, E, k, block_rows, _mat(gate), _mat(up), _mat(down),
        _mat(sh_gate), _mat(sh_up), _mat(sh_down),
        None if routing is None else _rt(routing), _ptr(y), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream, x.device)), "moe_decode_q4")


def decode_noalloc_max_bytes() -> int:
    return lib().moe_decode_noalloc_max_bytes()


def moe_decode_q4_noalloc(x: torch.Tensor, logits: torch.Tensor, I: int, I_sh: int, k: int,
                          block_rows: int, gate, up, down, sh_gate, sh_up, sh_down, routing,
                          y: torch.Tensor, stream=None):
    """moe_decode_q4 with the library's device-resident scratch as its workspace (no
    allocation; calls that overlap on one GPU race)."""
    _, H = _x_of(x)
    _tensor(x, "x", BF16, (1, H))
    _tensor(logits, "logits", F32)
    if logits.dim() != 2 or logits.shape[0] != 1:
        raise ValueError("logits: expected [1, E]")
    E = logits.shape[1]
    _expert_mats(gate, up, down, sh_gate, sh_up, sh_down, E, H, I, I_sh)
    if routing is not None:
        _routing_for(routing, "routing", 1, E, k, block_rows)
    _tensor(y, "y", BF16, (1, H))
    _check(lib().moe_decode_q4_noalloc(
        _ptr(x), _ptr(logits), H, I, I_sh, E, k, block_rows, _mat(gate), _mat(up), _mat(down),
        _mat(sh_gate), _mat(sh_up), _mat(sh_down),
        None if routing is None else _rt(routing), _ptr(y), _stream(stream, x.device)),
        "moe_decode_q4_noalloc")


def moe_decode_q4_sequential(x: torch.Tensor, logits: torch.Tensor, I: int, I_sh: int, k: int,
                             gate, up, down, sh_gate, sh_up, sh_down, y: torch.Tensor,
                             ws: torch.Tensor, stream=None):
    """x [n, H], logits [n, E]: n single-token decode calls back to back."""
    n, H = _x_of(x)
    _tensor(logits, "logits", F32)
    if logits.dim() != 2 or logits.shape[0] != n:
        raise ValueError("logits: expected [n, E]")
    E = logits.shape[1]
    _expert_mats(gate, up, down, sh_gate, sh_up, sh_down, E, H, I, I_sh)
    _tensor(y, "y", BF16, (n, H))
    _ws(ws)
    _check(lib().moe_decode_q4_sequential(
        _ptr(x), _ptr(logits), n, H, I, I_sh, E, k, _mat(gate), _mat(up), _mat(down),
        _mat(sh_gate), _mat(sh_up), _mat(sh_down), _ptr(y), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream, x.device)), "moe_decode_q4_sequential")


def moe_layer_chunked(x: torch.Tensor, logits: torch.Tensor, I: int, I_sh: int, k: int,
                      block_rows: int, chunk_tokens: int, gate, up, down, sh_gate, sh_up,
                      sh_down, y: torch.Tensor, ws: torch.Tensor, stream=None):
    T, H = _x_of(x)
    _tensor(logits, "logits", F32)
    if logits.dim() != 2 or logits.shape[0] != T:
        raise ValueError("logits: expected [T, E]")
    E = logits.shape[1]
    _expert_mats(gate, up, down, sh_gate, sh_up, sh_down, E, H, I, I_sh)
    _tensor(y, "y", BF16, (T, H))
    _ws(ws)
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
                 block_rows: int = 32, prepack=False):
        """prepack: False (row-major code words), True (tile-packed code words, packed
        gate/up scale|bias words) or "codes" (tile-packed code words only)."""
        self.H, self.I, self.I_sh, self.E, self.k = H, I, I_sh, E, k
        self.block_rows = block_rows
        self.device = torch.device(device)
        up = lambda m: None if m is None else DeviceQMat.from_host(m, self.device)  # noqa: E731
        self.gate, self.up, self.down = up(weights.gate), up(weights.up), up(weights.down)
        self.sh_gate, self.sh_up, self.sh_down = (up(weights.sh_gate), up(weights.sh_up),
                                                  up(weights.sh_down))
        if prepack:   # load time: tile-packed code words and, unless prepack == "codes", packed
            # gate/up scale|bias words; the row-major copies are freed
            (self.gate, self.up, self.down, self.sh_gate, self.sh_up,
             self.sh_down) = prepacked_mats(self.weight_mats(), pack_scales=prepack != "codes")
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

    def decode_mats(self):
        """The six matrix sets for batch-1 decode, which reads scales row by row: packed
        scale|bias sets are given as their plain-scale views (same code words)."""
        return tuple(None if m is None else m.row_view() for m in self.weight_mats())

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
        moe_decode_q4(x, logits, self.I, self.I_sh, self.k, self.block_rows, *self.decode_mats(),
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
