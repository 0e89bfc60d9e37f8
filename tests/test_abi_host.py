"""The C ABI library loads, exports every entry point include/biloco.h
declares, and rejects bad arguments on the host (no GPU, no HIP call)."""
import os
import re

import pytest

from bit_weight_gemm_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "biloco.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(biloco_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = B.lib()
    names = _declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    assert sorted(names) == sorted(B.EXPORTED)


def test_status_strings():
    assert B.biloco_status_string(0) == "BILOCO_OK"
    assert B.biloco_status_string(4) == "BILOCO_ERR_WORKSPACE_TOO_SMALL"
    assert B.biloco_status_string(99) == "BILOCO_ERR_UNKNOWN"


A = 1 << 36  # fake, 16-byte aligned, far-apart "device" addresses: never dereferenced


def _args(M=1, N=256, K=256, r=16, ws_bytes=None, **over):
    base = dict(a_codes=A * 1, a_scales=A * 2, x_bf16=A * 3, w_codes=A * 4, w_scales=A * 5,
                v_packed=A * 6, u_packed=A * 7, alpha_bf16=A * 8, y=A * 10, workspace=A * 20)
    base.update(over)
    if ws_bytes is None:
        ws_bytes = B.biloco_gemm_workspace_bytes(M, N, K, r)
    return (base["a_codes"], base["a_scales"], base["x_bf16"], base["w_codes"], base["w_scales"],
            base["v_packed"], base["u_packed"], base["alpha_bf16"], M, N, K, r, base["y"],
            base["workspace"], ws_bytes)


def test_check_accepts_valid():
    assert B.biloco_gemm_check(*_args()) == B.BILOCO_OK
    assert B.biloco_gemm_check(*_args(M=32, N=5120, K=13824, r=512)) == B.BILOCO_OK


@pytest.mark.parametrize("kw,status", [
    (dict(M=0), B.BILOCO_ERR_INVALID_VALUE),
    (dict(M=33), B.BILOCO_ERR_UNSUPPORTED),
    (dict(N=0), B.BILOCO_ERR_INVALID_VALUE),
    (dict(K=0), B.BILOCO_ERR_INVALID_VALUE),
    (dict(K=48), B.BILOCO_ERR_UNSUPPORTED),
    (dict(K=40), B.BILOCO_ERR_INVALID_VALUE),
    (dict(r=-1), B.BILOCO_ERR_INVALID_VALUE),
    (dict(N=65536, K=65536), B.BILOCO_ERR_UNSUPPORTED),     # R's codes: 2^31 bytes
    (dict(N=1 << 24, K=32, r=1024), B.BILOCO_ERR_UNSUPPORTED),  # U's words: 2^31 bytes
])
def test_check_rejects_shapes(kw, status):
    args = list(_args(ws_bytes=1 << 20))
    M, N, K, r = kw.get("M", 1), kw.get("N", 256), kw.get("K", 256), kw.get("r", 16)
    args[8:12] = [M, N, K, r]
    assert B.biloco_gemm_check(*args) == status


@pytest.mark.parametrize("name", ["a_codes", "a_scales", "x_bf16", "w_codes", "w_scales",
                                  "v_packed", "u_packed", "alpha_bf16", "y", "workspace"])
def test_check_rejects_null(name):
    assert B.biloco_gemm_check(*_args(**{name: None})) == B.BILOCO_ERR_INVALID_VALUE


@pytest.mark.parametrize("name", ["a_codes", "w_scales", "y", "workspace", "v_packed"])
def test_check_rejects_misaligned(name):
    good = dict(a_codes=A * 1, w_scales=A * 5, y=A * 10, workspace=A * 20, v_packed=A * 6)
    assert B.biloco_gemm_check(*_args(**{name: good[name] + 8})) == B.BILOCO_ERR_INVALID_VALUE


def test_r0_allows_null_lowrank_operands():
    args = _args(r=0, x_bf16=None, v_packed=None, u_packed=None, alpha_bf16=None, workspace=None)
    assert B.biloco_gemm_check(*args) == B.BILOCO_OK


def test_workspace_too_small():
    need = B.biloco_gemm_workspace_bytes(8, 13824, 5120, 512)
    assert need > 0
    args = _args(M=8, N=13824, K=5120, r=512, ws_bytes=need - 1)
    assert B.biloco_gemm_check(*args) == B.BILOCO_ERR_WORKSPACE_TOO_SMALL


def test_output_aliasing_rejected():
    # y overlapping w_codes
    assert B.biloco_gemm_check(*_args(y=A * 4 + 16)) == B.BILOCO_ERR_INVALID_VALUE


def test_schedule_queries():
    for M, N, K, r in [(1, 256, 256, 16), (1, 5120, 5120, 512), (8, 13824, 5120, 512),
                       (32, 5120, 13824, 512), (32, 8192, 8192, 1024)]:
        s = B.biloco_default_schedule(M, N, K, r)
        avail = B.biloco_schedules_for(M, N, K, r)
        assert s in avail, (M, s, avail)
        assert B.BILOCO_SCHED_UNFUSED in avail
        for sch in avail:
            assert B.biloco_gemm_check(*_args(M, N, K, r), schedule=sch) == B.BILOCO_OK
    assert B.biloco_default_schedule(0, 1, 32, 0) == 0
    assert B.biloco_gemm_check(*_args(), schedule=B.BILOCO_SCHED_MFMA_ZEPI + 1) == B.BILOCO_ERR_INVALID_VALUE


def test_prep_entry_points_reject_before_hip():
    L = B.lib()
    A = 0x10000
    assert L.biloco_pack_signs(None, 16, 16, A, None) == B.BILOCO_ERR_INVALID_VALUE
    assert L.biloco_pack_signs(A, 0, 16, A * 2, None) == B.BILOCO_ERR_INVALID_VALUE
    assert L.biloco_pack_signs(A + 1, 16, 16, A * 2, None) == B.BILOCO_ERR_INVALID_VALUE
    assert L.biloco_quant_act_fp4(A, 1, 48, A * 2, A * 3, None) == B.BILOCO_ERR_UNSUPPORTED
    assert L.biloco_quant_act_fp4(A, 0, 64, A * 2, A * 3, None) == B.BILOCO_ERR_INVALID_VALUE
    assert L.biloco_quant_act_fp4(None, 1, 64, A * 2, A * 3, None) == B.BILOCO_ERR_INVALID_VALUE
    # codes overlapping x
    assert L.biloco_quant_act_fp4(A, 1, 64, A + 64, A * 3, None) == B.BILOCO_ERR_INVALID_VALUE


def test_quant_weight_rejects_before_hip():
    L = B.lib()
    A = 1 << 36
    ws = B.biloco_quant_weight_workspace_bytes(64, 64)
    assert 0 < ws <= 64 * 1024
    ok = (A, 64, 64, A * 2, A * 3, A * 4, A * 5, ws, None)

    def call(**kw):
        names = ["w", "N", "K", "codes", "scales", "g", "ws", "wsb", "stream"]
        args = dict(zip(names, ok))
        args.update(kw)
        return L.biloco_quant_weight_nvfp4(*[args[n] for n in names])

    assert call(N=0) == B.BILOCO_ERR_INVALID_VALUE
    assert call(K=8) == B.BILOCO_ERR_INVALID_VALUE
    assert call(K=40) == B.BILOCO_ERR_INVALID_VALUE
    assert call(N=1 << 30, K=1 << 10) == B.BILOCO_ERR_UNSUPPORTED
    for name in ["w", "codes", "scales", "g", "ws"]:
        assert call(**{name: None}) == B.BILOCO_ERR_INVALID_VALUE, name
        assert call(**{name: ok[["w", "N", "K", "codes", "scales", "g", "ws"].index(name)] + 4}) \
            == B.BILOCO_ERR_INVALID_VALUE, name
    assert call(wsb=ws - 1) == B.BILOCO_ERR_WORKSPACE_TOO_SMALL
    assert call(codes=A + 256) == B.BILOCO_ERR_INVALID_VALUE          # codes inside w
    assert call(g=A * 3 + 16) == B.BILOCO_ERR_INVALID_VALUE           # g inside scales
    with pytest.raises(B.BilocoError):
        B.biloco_quant_weight_workspace_bytes(3, 24)


def test_peel_rejects_before_hip():
    L = B.lib()
    A = 1 << 36
    ws = B.biloco_peel_workspace_bytes(64, 64, 8)
    assert ws > 0
    names = ["W", "m", "n", "r", "T", "vi", "up", "vp", "alpha", "ag", "R", "ws", "wsb", "stream"]
    ok = dict(W=A, m=64, n=64, r=8, T=2, vi=A * 2, up=A * 3, vp=A * 4, alpha=A * 5, ag=A * 6,
              R=A * 7, ws=A * 8, wsb=ws, stream=None)

    def call(**kw):
        args = dict(ok)
        args.update(kw)
        return L.biloco_peel_decompose(*[args[k] for k in names])

    assert call(m=0) == B.BILOCO_ERR_INVALID_VALUE
    assert call(n=6) == B.BILOCO_ERR_INVALID_VALUE
    assert call(r=0) == B.BILOCO_ERR_INVALID_VALUE
    assert call(T=0) == B.BILOCO_ERR_INVALID_VALUE
    assert call(r=1025) == B.BILOCO_ERR_UNSUPPORTED
    assert call(m=1 << 19) == B.BILOCO_ERR_UNSUPPORTED
    for k in ["W", "vi", "up", "vp", "alpha", "ws"]:
        assert call(**{k: None}) == B.BILOCO_ERR_INVALID_VALUE, k
        assert call(**{k: ok[k] + 8}) == B.BILOCO_ERR_INVALID_VALUE, k
    assert call(wsb=ws - 1) == B.BILOCO_ERR_WORKSPACE_TOO_SMALL
    assert call(R=A + 64) == B.BILOCO_ERR_INVALID_VALUE               # R inside W


def test_gemm_quant_rejects_before_hip():
    L = B.lib()
    M, N, K, r = 2, 256, 256, 16
    ws = B.biloco_gemm_workspace_bytes(M, N, K, r)
    names = ["x", "ac", "as_", "wc", "wsc", "g", "vp", "up", "al", "M", "N", "K", "r", "y", "ws",
             "wsb", "sched", "stream"]
    ok = dict(x=A * 3, ac=A * 1, as_=A * 2, wc=A * 4, wsc=A * 5, g=1.0, vp=A * 6, up=A * 7,
              al=A * 8, M=M, N=N, K=K, r=r, y=A * 10, ws=A * 20, wsb=ws, sched=0, stream=None)

    def call(**kw):
        args = dict(ok)
        args.update(kw)
        return L.biloco_gemm_lowrank_quant(*[args[k] for k in names])

    assert call(x=None) == B.BILOCO_ERR_INVALID_VALUE
    assert call(x=None, r=0, vp=None, up=None, al=None) == B.BILOCO_ERR_INVALID_VALUE
    assert call(ac=None) == B.BILOCO_ERR_INVALID_VALUE
    assert call(M=33) == B.BILOCO_ERR_UNSUPPORTED
    assert call(wsb=ws - 1) == B.BILOCO_ERR_WORKSPACE_TOO_SMALL
    assert call(ac=A * 3 + 64) == B.BILOCO_ERR_INVALID_VALUE       # codes inside x
    assert call(as_=A * 4 + 16) == B.BILOCO_ERR_INVALID_VALUE      # scales inside w_codes
    assert call(ac=A * 2) == B.BILOCO_ERR_INVALID_VALUE            # codes over scales
    assert call(sched=9) == B.BILOCO_ERR_INVALID_VALUE


def test_timeline_stamps_only_in_the_measurement_build():
    """The per-wave timeline stamps are compiled only into libbiloco_tl.so
    (BILOCO_TIMELINE); the product library holds neither the stamp arrays'
    readers nor any other timeline symbol."""
    import subprocess
    from bit_weight_gemm_amd import build as hb

    def dynamic_symbols(path):
        out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True,
                             text=True, check=True).stdout
        return {line.split()[-1] for line in out.splitlines() if line.strip()}

    product = dynamic_symbols(B.LIB_PATH)
    assert not any(s.startswith("biloco_tl_") for s in product)
    if not os.path.exists(hb.TL_LIB):
        pytest.skip("timeline build not present (built by __graft_entry__.build())")
    tl = dynamic_symbols(hb.TL_LIB)
    for name in ("biloco_tl_gemv_zero", "biloco_tl_gemv_read", "biloco_tl_mfma_zero",
                 "biloco_tl_mfma_read"):
        assert name in tl, name
    # the measurement build exports the same C ABI as the product
    for name in B.EXPORTED:
        assert name in tl, name
