"""The Python binding rejects tensors that do not match the call before any C
call is made (no GPU needed: CPU tensors fail the device check last, so
dtype, shape and contiguity mistakes are reported first).  Without these
checks a wrong buffer would reach the kernels as an out-of-range address."""
import pytest
import torch

import bit_quantized_grouped_amd as bq

T, H, I, E, k = 8, 256, 128, 16, 2


def _routing(T_=T, E_=E, k_=k, br=32):
    return bq.DeviceRouting(T_, E_, k_, br, "cpu")


def _qmat(n_exp, N, K):
    return bq.DeviceQMat(torch.zeros((n_exp, N, K // 8), dtype=torch.int32),
                         torch.zeros((n_exp, N, K // 64), dtype=torch.int16),
                         torch.zeros((n_exp, N, K // 64), dtype=torch.int16))


def _mats(I_sh=I):
    sh = I_sh > 0
    return (_qmat(E, I, H), _qmat(E, I, H), _qmat(E, H, I),
            _qmat(1, I_sh, H) if sh else None, _qmat(1, I_sh, H) if sh else None,
            _qmat(1, H, I_sh) if sh else None)


def _bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def _layer_call(x=None, logits=None, routing=None, mats=None, eo=None, so="default", y=None,
                I_sh=I):
    x = _bf16(T, H) if x is None else x
    logits = torch.zeros((T, E), dtype=torch.float32) if logits is None else logits
    routing = _routing() if routing is None else routing
    mats = _mats(I_sh) if mats is None else mats
    eo = _bf16(T * k, H) if eo is None else eo
    so = (_bf16(T, H) if I_sh else None) if isinstance(so, str) else so
    y = _bf16(T, H) if y is None else y
    ws = torch.zeros(256, dtype=torch.uint8)
    bq.moe_layer_q4(x, logits, I, I_sh, E, k, 32, routing, ws, *mats, eo, so, ws, y)


def test_well_formed_cpu_call_fails_only_on_the_device_check():
    with pytest.raises(ValueError, match="device tensors"):
        _layer_call()


@pytest.mark.parametrize("kw,exc,msg", [
    (dict(x=torch.zeros((T, H), dtype=torch.float16)), TypeError, "x: dtype"),
    (dict(x=_bf16(H, T).t()), ValueError, "x: must be contiguous"),
    (dict(logits=torch.zeros((T, E), dtype=torch.float64)), TypeError, "logits: dtype"),
    (dict(logits=torch.zeros((T, E + 1), dtype=torch.float32)), ValueError, "logits: shape"),
    (dict(routing=_routing(T_=T + 1)), ValueError, "routing: built for"),
    (dict(routing=_routing(k_=k + 1)), ValueError, "routing: built for"),
    (dict(routing=_routing(br=16)), ValueError, "routing: built for"),
    (dict(eo=_bf16(T * k - 1, H)), ValueError, "expert_out: shape"),
    (dict(y=_bf16(T, H + 64)), ValueError, "y: shape"),
    (dict(so=None), ValueError, "shared_out: required"),
    (dict(I_sh=0, so=_bf16(T, H)), ValueError, "sh_gate: must be None|shared_out: must be None"),
])
def test_layer_call_rejects_mismatched_buffers(kw, exc, msg):
    with pytest.raises(exc, match=msg):
        _layer_call(**kw)


def test_weight_sets_must_hold_the_layer_shape():
    g, u, d, sg, su, sd = _mats()
    with pytest.raises(ValueError, match="gate: codes"):
        _layer_call(mats=(_qmat(E, I, H + 64), u, d, sg, su, sd))
    with pytest.raises(ValueError, match="down: codes"):
        _layer_call(mats=(g, u, _qmat(E, I, H), sg, su, sd))
    with pytest.raises(TypeError, match="up: expected a DeviceQMat"):
        _layer_call(mats=(g, "up", d, sg, su, sd))


def test_route_and_combine_check_their_routing():
    logits = torch.zeros((T, E), dtype=torch.float32)
    ws = torch.zeros(256, dtype=torch.uint8)
    with pytest.raises(ValueError, match="routing: built for"):
        bq.moe_route(logits, k, 32, _routing(E_=E + 1), ws)
    with pytest.raises(ValueError, match="routing: not built"):
        bq.moe_combine(_bf16(T * k, H), None, _routing(T_=T - 1), k, _bf16(T, H))
    with pytest.raises(ValueError, match="expert_out: shape"):
        bq.moe_combine(_bf16(T * k, H - 64), None, _routing(), k, _bf16(T, H))


def test_decode_checks_one_token_shapes():
    mats = _mats()
    ws = torch.zeros(256, dtype=torch.uint8)
    lg = torch.zeros((1, E), dtype=torch.float32)
    with pytest.raises(ValueError, match="x: shape"):
        bq.moe_decode_q4(_bf16(2, H), lg, I, I, k, 32, *mats, None, _bf16(1, H), ws)
    with pytest.raises(ValueError, match="y: shape"):
        bq.moe_decode_q4(_bf16(1, H), lg, I, I, k, 32, *mats, None, _bf16(2, H), ws)
    with pytest.raises(ValueError, match="routing: built for"):
        bq.moe_decode_q4(_bf16(1, H), lg, I, I, k, 32, *mats, _routing(T_=2), _bf16(1, H), ws)
