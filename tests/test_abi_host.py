"""The C-ABI library loads, exports every function include/moe_q4.h declares,
and rejects bad arguments on the host with the documented status codes
(no GPU needed: these paths return before any HIP call)."""
import ctypes
import os
import re

import pytest

import bit_quantized_grouped_amd as bq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "moe_q4.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert len(names) >= 10
    L = bq.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(bq.EXPORTED)


def test_version_and_status_strings():
    assert bq.abi_version() == 5
    for st, txt in [(0, "ok"), (-1, "null pointer"), (-2, "bad shape"), (-3, "misaligned pointer"),
                    (-4, "workspace too small"), (-5, "HIP launch error"), (-6, "unimplemented"),
                    (-99, "unknown status")]:
        assert bq.status_str(st) == txt


def test_max_blocks_and_workspace_sizes():
    assert bq.route_max_blocks(512, 256, 8, 32) == 128 + 256
    assert bq.route_max_blocks(2048, 256, 8, 32) == 512 + 256
    assert bq.route_max_blocks(1, 256, 8, 32) == 1 + 8
    assert bq.route_max_blocks(64, 16, 2, 32) == 4 + 16
    assert bq.lib().moe_route_max_blocks(1, 256, 8, 48) == bq.MOE_ERR_SHAPE
    # k = 4, 8, 16 above the one-launch size: T*k words of per-chunk match information
    assert bq.route_workspace_bytes(512, 256, 8, 32) == 512 * 8 * 4
    assert bq.route_workspace_bytes(512, 256, 4, 32) == 512 * 4 * 4
    assert bq.route_workspace_bytes(512, 256, 16, 32) == 512 * 16 * 4
    assert bq.route_workspace_bytes(65, 256, 8, 32) == 9 * 256   # 65 * 8 words, rounded up to 256 bytes
    assert bq.route_workspace_bytes(64, 256, 8, 32) == 0     # one launch, no workspace
    assert bq.route_workspace_bytes(512, 256, 2, 32) == 0    # other k: no workspace
    assert bq.route_workspace_bytes(512, 256, 6, 32) == 0
    assert bq.route_workspace_bytes(0, 256, 8, 32) == 0
    # h (T*k x I) + shared h (T x I_sh), bf16
    assert bq.gemm_workspace_bytes(512, 2048, 512, 512, 256, 8, 32) >= 512 * 8 * 512 * 2 + 512 * 512 * 2
    assert bq.gemm_workspace_bytes(512, 2000, 512, 512, 256, 8, 32) == 0
    assert bq.layer_workspace_bytes(2048, 2048, 512, 512, 256, 8, 32) > 2048 * 8 * 2048 * 2


def test_shape_limits_keep_byte_offsets_in_31_bits():
    """The kernels form 32-bit byte offsets inside one buffer: T*k*max(H, I) and
    T*max(H, I_sh) bf16 elements stay below 2^30, one expert's H*max(I, I_sh) / 2
    bytes of code words below 2^31."""
    ws = bq.gemm_workspace_bytes
    # T*k*H = 2^30 - 2^21 (accepted) and 2^30 (rejected), H = 2048, k = 8
    assert ws(65536 - 128, 2048, 512, 512, 256, 8, 32) > 0
    assert ws(65536, 2048, 512, 512, 256, 8, 32) == 0
    # T*I_sh = 2^30 with k = 1, H = 64 (T*k*max(H, I) stays below the bound)
    assert ws(1 << 14, 64, 64, 1 << 16, 256, 1, 32) == 0
    assert ws((1 << 14) - 1, 64, 64, 1 << 16, 256, 1, 32) > 0
    # H*I = 2^32 (one expert's codes would be 2^31 bytes) with T = 1
    assert ws(1, 65536, 65536, 0, 4, 1, 32) == 0
    assert ws(1, 65536, 65536 - 64, 0, 4, 1, 32) > 0
    L = bq.lib()
    r = _routing()
    assert L.moe_combine(FAKE, None, ctypes.byref(r), 65536, 2048, 8, FAKE, None) == bq.MOE_ERR_SHAPE
    # the bf16-weight GEMMs: one expert's bf16 matrix below 2^31 bytes (H*I < 2^30)
    args = lambda H, I: [1, H, I, 0, 4, 1, 32, ctypes.byref(r), FAKE, None, FAKE, None, FAKE, 1 << 40, None]  # noqa: E731
    assert L.moe_expert_down_bf16(*args(32768, 32768)) == bq.MOE_ERR_SHAPE


P = ctypes.c_void_p
FAKE = P(0x10000)          # never dereferenced: validation fails first
MISALIGNED = P(0x10008)


def _routing(ptr=FAKE):
    return bq.MoeRouting(*([ptr.value] * 9))


def _mat(codes=FAKE):
    return bq.MoeQ4Mat(codes.value, FAKE.value, FAKE.value)


def test_route_rejects_bad_arguments():
    L = bq.lib()
    r = _routing()
    ok_ws = 256
    assert L.moe_route(None, 64, 16, 2, 32, ctypes.byref(r), FAKE, ok_ws, None) == bq.MOE_ERR_NULL
    assert L.moe_route(FAKE, 64, 16, 2, 32, None, FAKE, ok_ws, None) == bq.MOE_ERR_NULL
    bad = bq.MoeRouting(*([FAKE.value] * 8 + [None]))
    assert L.moe_route(FAKE, 64, 16, 2, 32, ctypes.byref(bad), FAKE, ok_ws, None) == bq.MOE_ERR_NULL
    for T, E, k, br in [(0, 16, 2, 32), (64, 16, 17, 32), (64, 16, 0, 32), (64, 1001, 2, 32),
                        (64, 16, 2, 8), (64, 16, 2, 128)]:
        assert L.moe_route(FAKE, T, E, k, br, ctypes.byref(r), FAKE, 1 << 30, None) == bq.MOE_ERR_SHAPE
    assert L.moe_route(P(0x10002), 64, 16, 2, 32, ctypes.byref(r), FAKE, ok_ws, None) == bq.MOE_ERR_ALIGN
    assert L.moe_route(FAKE, 64, 16, 2, 32, ctypes.byref(r), P(0x10010), ok_ws, None) == bq.MOE_ERR_ALIGN


def test_gemm_rejects_bad_arguments():
    L = bq.lib()
    r = _routing()
    m = _mat()
    ws = bq.gemm_workspace_bytes(64, 256, 128, 128, 16, 2, 32)

    def call(x=FAKE, T=64, H=256, I=128, I_sh=128, E=16, k=2, br=32, mats=None, eo=FAKE, so=FAKE,
             wsb=ws):
        mats = mats or [m] * 6
        args = [x, T, H, I, I_sh, E, k, br, ctypes.byref(r)]
        args += [ctypes.byref(q) if q is not None else None for q in mats]
        args += [eo, so, FAKE, wsb, None]
        return L.moe_grouped_gemm_q4(*args)

    assert call(x=None) == bq.MOE_ERR_NULL
    assert call(eo=None) == bq.MOE_ERR_NULL
    assert call(so=None) == bq.MOE_ERR_NULL
    assert call(H=200) == bq.MOE_ERR_SHAPE
    assert call(I=96) == bq.MOE_ERR_SHAPE
    assert call(I_sh=32) == bq.MOE_ERR_SHAPE
    assert call(I_sh=0, so=None) == bq.MOE_ERR_SHAPE    # shared matrices passed without I_sh
    assert call(mats=[_mat(MISALIGNED)] + [m] * 5) == bq.MOE_ERR_ALIGN
    assert call(x=P(0x10004)) == bq.MOE_ERR_ALIGN
    assert call(wsb=ws - 1) == bq.MOE_ERR_WORKSPACE
    nul = bq.MoeQ4Mat(FAKE.value, None, FAKE.value)
    assert call(mats=[m, nul, m, m, m, m]) == bq.MOE_ERR_NULL


def test_layer_call_rejects_bad_arguments():
    L = bq.lib()
    r = _routing()
    m = _mat()
    ws = bq.gemm_workspace_bytes(64, 256, 128, 128, 16, 2, 32)

    def call(x=FAKE, lg=FAKE, T=64, H=256, I=128, I_sh=128, E=16, k=2, br=32, mats=None,
             rws=FAKE, rwsb=256, eo=FAKE, so=FAKE, gws=FAKE, wsb=ws, y=FAKE):
        mats = mats or [m] * 6
        args = [x, lg, T, H, I, I_sh, E, k, br]
        args += [ctypes.byref(q) if q is not None else None for q in mats]
        args += [ctypes.byref(r), rws, rwsb, eo, so, gws, wsb, y, None]
        return L.moe_layer_q4(*args)

    assert call(x=None) == bq.MOE_ERR_NULL
    assert call(lg=None) == bq.MOE_ERR_NULL
    assert call(y=None) == bq.MOE_ERR_NULL
    assert call(gws=None) == bq.MOE_ERR_NULL
    assert call(so=None) == bq.MOE_ERR_NULL
    assert call(H=200) == bq.MOE_ERR_SHAPE
    assert call(k=17) == bq.MOE_ERR_SHAPE
    assert call(br=48) == bq.MOE_ERR_SHAPE
    assert call(I_sh=0, so=None) == bq.MOE_ERR_SHAPE
    assert call(lg=P(0x10002)) == bq.MOE_ERR_ALIGN
    assert call(y=P(0x10008)) == bq.MOE_ERR_ALIGN
    assert call(gws=P(0x10010)) == bq.MOE_ERR_ALIGN
    assert call(wsb=ws - 1) == bq.MOE_ERR_WORKSPACE


def test_read_probe_sizes_and_bad_arguments():
    L = bq.lib()
    assert bq.read_probe_sink_words(16) == 1
    assert bq.read_probe_sink_words(32768) == 1
    assert bq.read_probe_sink_words(32768 + 16) == 2
    assert bq.read_probe_sink_words(1 << 30) == (1 << 30) // 32768
    sink_ok = 1 << 20
    assert L.moe_read_probe(None, 1 << 20, FAKE, sink_ok, None) == bq.MOE_ERR_NULL
    assert L.moe_read_probe(FAKE, 1 << 20, None, sink_ok, None) == bq.MOE_ERR_NULL
    for nbytes in (0, 8, 24, 1000):
        assert L.moe_read_probe(FAKE, nbytes, FAKE, sink_ok, None) == bq.MOE_ERR_SHAPE
    assert L.moe_read_probe(P(0x10008), 1 << 20, FAKE, sink_ok, None) == bq.MOE_ERR_ALIGN
    assert L.moe_read_probe(FAKE, 1 << 20, P(0x10002), sink_ok, None) == bq.MOE_ERR_ALIGN
    assert L.moe_read_probe(FAKE, 1 << 20, FAKE, 31, None) == bq.MOE_ERR_WORKSPACE


def test_combine_and_chunked_reject_bad_arguments():
    L = bq.lib()
    r = _routing()
    assert L.moe_combine(None, None, ctypes.byref(r), 4, 256, 2, FAKE, None) == bq.MOE_ERR_NULL
    assert L.moe_combine(FAKE, None, ctypes.byref(r), 4, 100, 2, FAKE, None) == bq.MOE_ERR_SHAPE
    assert L.moe_combine(FAKE, None, ctypes.byref(r), 4, 256, 2, MISALIGNED, None) == bq.MOE_ERR_ALIGN
    m = _mat()
    mats = [ctypes.byref(m)] * 6
    ws = bq.layer_workspace_bytes(32, 256, 128, 128, 16, 2, 32)
    args = lambda chunk, wsb: [FAKE, FAKE, 64, 256, 128, 128, 16, 2, 32, chunk] + mats + [FAKE, FAKE, wsb, None]  # noqa: E731
    assert L.moe_layer_chunked(*args(0, ws)) == bq.MOE_ERR_SHAPE
    assert L.moe_layer_chunked(*args(32, ws - 1)) == bq.MOE_ERR_WORKSPACE


def test_split_phases_reject_bad_arguments():
    L = bq.lib()
    r = _routing()
    m = _mat()
    ws = bq.gemm_workspace_bytes(64, 256, 128, 128, 16, 2, 32)
    gu = lambda x=FAKE, I_sh=128, mats=None, wsb=ws, wsp=FAKE: L.moe_expert_gateup_q4(  # noqa: E731
        x, 64, 256, 128, I_sh, 16, 2, 32, ctypes.byref(r),
        *[ctypes.byref(q) if q is not None else None for q in (mats or [m] * 4)], wsp, wsb, None)
    assert gu(x=None) == bq.MOE_ERR_NULL
    assert gu(x=P(0x10002)) == bq.MOE_ERR_ALIGN
    assert gu(I_sh=0) == bq.MOE_ERR_SHAPE                     # shared matrices without I_sh
    assert gu(wsb=ws - 1) == bq.MOE_ERR_WORKSPACE
    assert gu(wsp=None) == bq.MOE_ERR_NULL
    assert gu(wsp=P(0x10010)) == bq.MOE_ERR_ALIGN
    dn = lambda eo=FAKE, so=FAKE, I_sh=128, mats=None, wsb=ws: L.moe_expert_down_q4(  # noqa: E731
        64, 256, 128, I_sh, 16, 2, 32, ctypes.byref(r),
        *[ctypes.byref(q) if q is not None else None for q in (mats or [m] * 2)], eo, so, FAKE, wsb, None)
    assert dn(eo=None) == bq.MOE_ERR_NULL
    assert dn(so=None) == bq.MOE_ERR_NULL
    assert dn(eo=MISALIGNED) == bq.MOE_ERR_ALIGN
    assert dn(mats=[_mat(MISALIGNED), m]) == bq.MOE_ERR_ALIGN
    assert dn(wsb=ws - 1) == bq.MOE_ERR_WORKSPACE


def test_decode_rejects_bad_arguments():
    L = bq.lib()
    m = _mat()
    mats = [ctypes.byref(m)] * 6
    ws = bq.decode_workspace_bytes(2048, 512, 512, 256, 8)
    assert ws >= 9 * 512 * 2
    assert bq.decode_workspace_bytes(2048, 512, 512, 256, 65) == 0     # k > 64
    call = lambda x=FAKE, k=8, H=2048, y=FAKE, wsb=ws, r=None: L.moe_decode_q4(  # noqa: E731
        x, FAKE, H, 512, 512, 256, k, 32, *mats, r, y, FAKE, wsb, None)
    assert call(x=None) == bq.MOE_ERR_NULL
    assert call(y=None) == bq.MOE_ERR_NULL
    assert call(k=65) == bq.MOE_ERR_SHAPE
    assert call(H=2000) == bq.MOE_ERR_SHAPE
    assert call(y=MISALIGNED) == bq.MOE_ERR_ALIGN
    assert call(wsb=ws - 1) == bq.MOE_ERR_WORKSPACE
    bad = bq.MoeRouting(*([FAKE.value] * 8 + [None]))
    assert call(r=ctypes.byref(bad)) == bq.MOE_ERR_NULL
    assert L.moe_decode_q4_sequential(FAKE, FAKE, 0, 2048, 512, 512, 256, 8, *mats, FAKE, FAKE,
                                      ws, None) == bq.MOE_ERR_SHAPE


def test_unfused_baseline_rejects_bad_arguments():
    L = bq.lib()
    m = _mat()
    dq = lambda mat=m, n=4, N=64, K=128, out=FAKE: L.moe_dequant_q4_bf16(  # noqa: E731
        ctypes.byref(mat) if mat is not None else None, n, N, K, None, out, None)
    assert dq(mat=None) == bq.MOE_ERR_NULL
    assert dq(out=None) == bq.MOE_ERR_NULL
    assert dq(K=100) == bq.MOE_ERR_SHAPE
    assert dq(n=0) == bq.MOE_ERR_SHAPE
    assert dq(n=1 << 12, N=1 << 12, K=1 << 12) == bq.MOE_ERR_SHAPE    # 2^33 words
    assert dq(out=MISALIGNED) == bq.MOE_ERR_ALIGN
    assert dq(mat=_mat(MISALIGNED)) == bq.MOE_ERR_ALIGN
    r = _routing()
    ws = bq.gemm_workspace_bytes(64, 256, 128, 128, 16, 2, 32)
    gu = lambda x=FAKE, w=FAKE, sh=FAKE, I_sh=128, wsb=ws: L.moe_expert_gateup_bf16(  # noqa: E731
        x, 64, 256, 128, I_sh, 16, 2, 32, ctypes.byref(r), w, FAKE, sh, sh, FAKE, wsb, None)
    assert gu(x=None) == bq.MOE_ERR_NULL
    assert gu(w=None) == bq.MOE_ERR_NULL
    assert gu(w=MISALIGNED) == bq.MOE_ERR_ALIGN
    assert gu(sh=None) == bq.MOE_ERR_NULL                      # I_sh > 0 needs shared weights
    assert gu(I_sh=0) == bq.MOE_ERR_SHAPE                      # shared weights without I_sh
    assert gu(wsb=ws - 1) == bq.MOE_ERR_WORKSPACE
    dn = lambda eo=FAKE, so=FAKE, w=FAKE, I_sh=128: L.moe_expert_down_bf16(  # noqa: E731
        64, 256, 128, I_sh, 16, 2, 32, ctypes.byref(r), w, FAKE if I_sh else None, eo, so, FAKE, ws,
        None)
    assert dn(eo=None) == bq.MOE_ERR_NULL
    assert dn(so=None) == bq.MOE_ERR_NULL
    assert dn(w=MISALIGNED) == bq.MOE_ERR_ALIGN
    assert dn(I_sh=0) == bq.MOE_ERR_SHAPE                      # shared_out without I_sh


def test_router_and_gated_combine_reject_bad_arguments():
    L = bq.lib()
    rt = lambda x=FAKE, T=16, H=256, wr=FAKE, E=64, wg=None, lg=FAKE, g=None: L.moe_router(  # noqa: E731
        x, T, H, wr, E, wg, lg, g, None)
    assert rt(x=None) == bq.MOE_ERR_NULL
    assert rt(lg=None) == bq.MOE_ERR_NULL
    assert rt(wg=FAKE) == bq.MOE_ERR_NULL          # gate row without a gate output
    assert rt(g=FAKE) == bq.MOE_ERR_NULL           # gate output without a gate row
    assert rt(H=100) == bq.MOE_ERR_SHAPE
    assert rt(E=0) == bq.MOE_ERR_SHAPE
    assert rt(E=1001) == bq.MOE_ERR_SHAPE
    assert rt(T=0) == bq.MOE_ERR_SHAPE
    assert rt(x=MISALIGNED) == bq.MOE_ERR_ALIGN
    assert rt(wg=MISALIGNED, g=FAKE) == bq.MOE_ERR_ALIGN
    r = _routing()
    cg = lambda so=FAKE, g=FAKE, y=FAKE: L.moe_combine_gated(  # noqa: E731
        FAKE, so, g, ctypes.byref(r), 8, 256, 2, y, None)
    assert cg(so=None) == bq.MOE_ERR_NULL
    assert cg(g=None) == bq.MOE_ERR_NULL
    assert cg(g=P(0x10002)) == bq.MOE_ERR_ALIGN
    assert cg(y=MISALIGNED) == bq.MOE_ERR_ALIGN


def test_layout_validation():
    L = bq.lib()
    r = _routing()
    ws = bq.gemm_workspace_bytes(64, 256, 128, 128, 16, 2, 32)
    rows, tiles, bad = _mat(), _mat(), _mat()
    tiles.layout, bad.layout = bq.LAYOUT_TILES, 7
    gu = lambda mats: L.moe_expert_gateup_q4(  # noqa: E731
        FAKE, 64, 256, 128, 128, 16, 2, 32, ctypes.byref(r), *[ctypes.byref(q) for q in mats],
        FAKE, ws, None)
    assert gu([bad, bad, bad, bad]) == bq.MOE_ERR_SHAPE                 # unknown layout
    assert gu([rows, tiles, rows, rows]) == bq.MOE_ERR_SHAPE            # mixed layouts
    assert L.moe_dequant_q4_bf16(ctypes.byref(tiles), 4, 64, 128, None, FAKE, None) \
        == bq.MOE_ERR_UNIMPLEMENTED                                     # expands row-major only
    pp = lambda src=FAKE, N=64, K=128, dst=P(0x20000): L.moe_q4_prepack(  # noqa: E731
        src, 2, N, K, dst, None)
    assert pp(src=None) == bq.MOE_ERR_NULL
    assert pp(N=96) == bq.MOE_ERR_SHAPE
    assert pp(K=100) == bq.MOE_ERR_SHAPE
    assert pp(dst=FAKE) == bq.MOE_ERR_SHAPE                             # in place
    assert pp(dst=MISALIGNED) == bq.MOE_ERR_ALIGN


def test_chunked_driver_checks_the_chunk_shape_not_the_prompt():
    """A 131072-token prompt in chunks of 2048 (H 2048, k 8): T*k*H is 2^31, past the
    one-call limit, but every kernel works inside one chunk, so validation passes and
    the call stops only at the undersized workspace."""
    L = bq.lib()
    m = _mat()
    mats = [ctypes.byref(m)] * 6
    T, H, I, E, k = 131072, 2048, 512, 256, 8
    assert bq.gemm_workspace_bytes(T, H, I, I, E, k, 32) == 0          # one call: too large
    ws = bq.layer_workspace_bytes(2048, H, I, I, E, k, 32)
    assert ws > 0
    args = lambda T_, chunk, wsb: [FAKE, FAKE, T_, H, I, I, E, k, 32, chunk] + mats + [FAKE, FAKE, wsb, None]  # noqa: E731
    assert L.moe_layer_chunked(*args(T, 2048, ws - 1)) == bq.MOE_ERR_WORKSPACE
    # a chunk past the per-call limit is still rejected
    assert L.moe_layer_chunked(*args(T, 65536, 1 << 40)) == bq.MOE_ERR_SHAPE
    # the routing bound T*k < 2^30 holds for the whole prompt
    assert L.moe_layer_chunked(*args(1 << 27, 2048, 1 << 40)) == bq.MOE_ERR_SHAPE


def test_packed_scale_layout_rules():
    """MOE_Q4_LAYOUT_TILES_SB: biases may be NULL and the packed words need 4-byte alignment;
    gate-side matrices share one layout, down matrices are never packed-scale, and all share
    one code-word order.  moe_q4_pack_scales' argument checks.  Host only: every call stops
    at a check (valid combinations at the workspace size)."""
    L = bq.lib()
    T, H, I, I_sh, E, k, br = 64, 256, 128, 128, 16, 2, 32
    sb = bq.MoeQ4Mat(256, 256, None, bq.LAYOUT_TILES_SB)
    tiles = bq.MoeQ4Mat(256, 256, 256, bq.LAYOUT_TILES)
    rows = bq.MoeQ4Mat(256, 256, 256, bq.LAYOUT_ROWS)
    r = bq.MoeRouting(*([16] * 9))
    by = ctypes.byref

    def gemm(g, d, sg, sd):
        return L.moe_grouped_gemm_q4(256, T, H, I, I_sh, E, k, br, by(r), by(g), by(g), by(d),
                                     by(sg), by(sg), by(sd), 256, 256, 256, 0, None)
    assert gemm(sb, tiles, sb, tiles) == bq.MOE_ERR_WORKSPACE
    assert gemm(tiles, tiles, tiles, tiles) == bq.MOE_ERR_WORKSPACE
    assert gemm(sb, sb, sb, sb) == bq.MOE_ERR_SHAPE          # down matrices are not packed
    assert gemm(sb, rows, sb, rows) == bq.MOE_ERR_SHAPE      # code-word orders differ
    assert gemm(sb, tiles, tiles, tiles) == bq.MOE_ERR_SHAPE  # gate/up and shared gate/up differ
    assert gemm(bq.MoeQ4Mat(256, 258, None, bq.LAYOUT_TILES_SB), tiles, sb, tiles) == bq.MOE_ERR_ALIGN
    assert gemm(bq.MoeQ4Mat(256, 256, None, bq.LAYOUT_TILES), tiles, sb, tiles) == bq.MOE_ERR_NULL
    assert gemm(bq.MoeQ4Mat(256, 256, 256, 3), tiles, sb, tiles) == bq.MOE_ERR_SHAPE

    P = L.moe_q4_pack_scales
    assert P(256, 512, 1, 60, 64, 1024, None) == bq.MOE_ERR_SHAPE      # N not a multiple of 64
    assert P(256, 512, 1, 64, 96, 1024, None) == bq.MOE_ERR_SHAPE      # K not a multiple of 64
    assert P(None, 512, 1, 64, 64, 1024, None) == bq.MOE_ERR_NULL
    assert P(256, 512, 1, 64, 64, None, None) == bq.MOE_ERR_NULL
    assert P(256, 512, 1, 64, 64, 256, None) == bq.MOE_ERR_SHAPE       # in place over the scales
    assert P(256, 512, 1, 64, 64, 1026, None) == bq.MOE_ERR_ALIGN
    assert P(256, 512, 1 << 16, 1 << 12, 1 << 12, 1024, None) == bq.MOE_ERR_SHAPE   # >= 2^31 words
