"""The C ABI without a GPU: the library loads, exports every entry point the
headers declare, and rejects bad arguments on the host (before any HIP call)
with the documented status codes."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "gpt_transformer_step_amd", "libgptstep.so")


@pytest.fixture(scope="module")
def B():
    if not os.path.exists(LIB):
        from gpt_transformer_step_amd import build
        build.build()
    from gpt_transformer_step_amd import binding
    return binding


def _declared():
    names = set()
    for h in ("gptstep.h", "gptstep_ops.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[\w]+\*?\s+\*?((?:gpt|muon|normuon|adamw)_\w+)\s*\(", src, flags=re.M):
            names.add(m.group(1))
    return names


def test_every_declared_symbol_is_exported(B):
    names = _declared()
    assert {"gpt_step_fwd", "gpt_step_bwd", "muon_update", "normuon_update", "adamw_update", "gpt_workspace_size",
            "gpt_op_gemm", "gpt_step_bwd_scaled", "muon_update_noalloc"} <= names
    lib = B.lib()
    missing = [n for n in sorted(names) if not hasattr(lib, n)]
    assert not missing, missing
    # the binding marshals exactly the declared entry points
    assert set(B.EXPORTED) == names


def test_abi_version_and_status_strings(B):
    lib = B.lib()
    assert lib.gpt_abi_version() == 3
    for code, text in [(0, b"ok"), (-1, b"invalid argument"), (-2, b"invalid shape"),
                       (-3, b"workspace too small"), (-4, b"HIP runtime error"), (-5, b"unsupported")]:
        assert lib.gpt_status_string(code) == text


def test_shape_validation(B):
    for depth, vocab, T, Bn, prec, code in [
        (3, 32768, 2048, 32, 0, -2),    # odd depth: heads are 128 wide
        (0, 32768, 2048, 32, 0, -2),
        (20, 0, 2048, 32, 0, -2),
        (20, 32768, 0, 32, 0, -2),
        (20, 32768, 2048, 0, 0, -2),
        (20, 32768, 2048, 32, 7, -5),   # unknown precision
    ]:
        with pytest.raises(B.GptError) as e:
            B.param_count(B.shape(depth, vocab, T, Bn, prec))
        assert e.value.code == code


def test_param_count_and_layout(B):
    from gpt_transformer_step_amd import inputs
    for depth in (2, 12, 20, 26):
        sh = B.shape(depth, 32768, 2048, 16)
        dims = inputs.Dims.from_depth(depth)
        assert B.param_count(sh) == inputs.n_params(dims)
        offs = B.param_layout(sh)
        expect, o = [], 0
        for _, shp in inputs.packed_tensors(dims):
            expect.append(o)
            o += shp[0] * shp[1]
        assert offs == expect
    # depth 20: 477.10 M parameters (block matrices 393.22 M + two 41.94 M tables)
    assert B.param_count(B.shape(20, 32768, 2048, 32)) == 477_102_080


@pytest.mark.parametrize("depth,kv,features", [(4, 0, "vsrb"), (6, 1, "v"), (20, 5, "sr"), (2, 0, "b")])
def test_param_layout_with_features(B, depth, kv, features):
    """The library's packed order with the record-model tensors equals the
    input generator's (value-embedding tables, gates, then the scalar block)."""
    import numpy as np
    from gpt_transformer_step_amd import inputs
    sh = B.shape(depth, 1000, 64, 2, n_kv_head=kv, features=features)
    dims = inputs.Dims.from_depth(depth, 1000, kv, features=features)
    assert B.param_count(sh) == inputs.n_params(dims)
    offs = B.param_layout(sh)
    expect, o = [], 0
    for _, shp in inputs.packed_tensors(dims):
        expect.append(o)
        o += int(np.prod(shp))
    assert offs == expect
    assert len(offs) == 2 + 7 * depth + 6


def test_unknown_feature_bits_rejected(B):
    sh = B.shape(2, 100, 8, 1)
    sh.features = 16
    with pytest.raises(B.GptError) as e:
        B.param_count(sh)
    assert e.value.code == -2


def test_workspace_queries(B):
    ws20 = B.workspace_size(B.shape(20, 32768, 2048, 32))
    ws12 = B.workspace_size(B.shape(12, 32768, 2048, 16))
    assert ws20 > ws12 > 0
    assert ws20 < 64 * 2 ** 30   # fits comfortably in 288 GB of HBM
    assert B.muon_workspace_size(80, 1280, 1280) > 0
    for args in [(0, 64, 64), (1, 63, 64), (1, 64, 0)]:
        with pytest.raises(B.GptError) as e:
            B.muon_workspace_size(*args)
        assert e.value.code == -1


def test_step_rejects_null_and_small_workspace_on_host(B):
    lib = B.lib()
    sh = B.shape(2, 1024, 64, 2)
    params = B.Params(None, None, None)
    loss = ctypes.c_void_p(0)
    rc = lib.gpt_step_fwd(ctypes.byref(sh), ctypes.byref(params), None, loss, None, None, None, 0, None)
    assert rc == -1
    # non-null but unaligned / too-small workspace: rejected before any device access
    fake = ctypes.c_void_p(4096)
    params = B.Params(fake, fake, fake)
    rc = lib.gpt_step_fwd(ctypes.byref(sh), ctypes.byref(params), fake, fake, None, None, fake, 16, None)
    assert rc == -3
    rc = lib.gpt_step_bwd(ctypes.byref(sh), ctypes.byref(params), fake, 2, fake, 1 << 40, None)
    assert rc == -1   # accumulate must be 0 or 1
    assert b"accumulate" in lib.gpt_last_error()


def test_muon_rejects_on_host(B):
    lib = B.lib()
    c = (ctypes.c_float * 3)(1.0, 0.0, 0.0)
    fake = ctypes.c_void_p(4096)
    rc = lib.muon_update(None, None, fake, None, None, 1, 64, 64, c, 0, 0.1, 0.9, 0.0, fake, 1 << 30, None)
    assert rc == -1   # ns_steps < 1
    rc = lib.muon_update(None, None, fake, None, None, 1, 64, 64, c, 1, 0.1, 0.9, 0.0, fake, 10, None)
    assert rc == -3   # workspace too small
    rc = lib.muon_update(None, None, None, None, None, 1, 64, 64, c, 1, 0.1, 0.9, 0.0, fake, 1 << 30, None)
    assert rc == -1   # G is NULL


def test_normuon_rejects_on_host(B):
    lib = B.lib()
    c = (ctypes.c_float * 3)(1.0, 0.0, 0.0)
    fake = ctypes.c_void_p(4096)

    def call(V=fake, per_row=1, beta2=0.95, eps=1e-8, ws_bytes=1 << 30, steps=1):
        return lib.normuon_update(None, None, fake, None, V, None, 1, 64, 64, per_row, c, steps, 0.1, 0.9, 0.0,
                                  beta2, eps, fake, ws_bytes, None)

    assert call(V=None) == -1
    assert b"V" in lib.gpt_last_error()
    assert call(per_row=2) == -1
    assert call(beta2=1.0) == -1
    assert call(eps=-1.0) == -1
    assert call(steps=0) == -1
    assert call(ws_bytes=10) == -3


def test_gemm_rejects_on_host(B):
    lib = B.lib()
    fake = ctypes.c_void_p(4096)
    rc = lib.gpt_op_gemm(64, 64, 64, 1, fake, 0, 60, 0, fake, 0, 64, 0, fake, 0, 64, 0, 1.0, 0.0, None)
    assert rc == -1   # lda not a multiple of 8
    rc = lib.gpt_op_gemm(64, 64, 64, 1, fake, 3, 64, 0, fake, 0, 64, 0, fake, 0, 64, 0, 1.0, 0.0, None)
    assert rc == -5   # unknown layout
    assert lib.gpt_op_gemm(0, 64, 64, 1, None, 0, 64, 0, None, 0, 64, 0, None, 0, 64, 0, 1.0, 0.0, None) == 0


def test_profile_categories(B):
    cats = B.profile_categories()
    assert "attn_fwd" in cats and "gemm_fc_relu2_fwd" in cats and len(set(cats)) == len(cats)


def test_fp8_ops_reject_on_host(B):
    lib = B.lib()
    fake = ctypes.c_void_p(4096)
    # rows not a multiple of 16
    rc = lib.gpt_op_quantize_fp8(fake, 1, 64, 8, 64, 0, fake, fake, 64, None, 0, fake, None)
    assert rc == -1
    rc = lib.gpt_op_quantize_fp8(fake, 1, 64, 16, 64, 2, fake, fake, 64, None, 0, fake, None)
    assert rc == -5   # unknown format
    rc = lib.gpt_op_quantize_fp8(fake, 1, 64, 16, 64, 0, None, fake, 64, None, 0, fake, None)
    assert rc == -1   # scale is NULL
    K, MN = 0, 1
    rc = lib.gpt_op_gemm_fp8(64, 64, 24, fake, 0, K, 32, fake, 0, K, 32, fake, 64, fake, fake, 0.0, None)
    assert rc == -1   # K not a multiple of 16
    rc = lib.gpt_op_gemm_fp8(64, 64, 32, fake, 0, K, 32, fake, 0, K, 32, fake, 64, None, fake, 0.0, None)
    assert rc == -1   # scale_a NULL
    assert lib.gpt_op_gemm_fp8(0, 64, 32, None, 0, K, 32, None, 0, K, 32, None, 64, None, None, 0.0, None) == 0
    # m/n-contiguous operands: E5M2 x E4M3 with B m/n-contiguous only
    rc = lib.gpt_op_gemm_fp8(64, 64, 32, fake, 0, K, 32, fake, 0, MN, 64, fake, 64, fake, fake, 0.0, None)
    assert rc == -5
    rc = lib.gpt_op_gemm_fp8(64, 64, 32, fake, 1, MN, 64, fake, 0, K, 32, fake, 64, fake, fake, 0.0, None)
    assert rc == -5
    rc = lib.gpt_op_gemm_fp8(64, 64, 32, fake, 1, K, 32, fake, 0, 2, 64, fake, 64, fake, fake, 0.0, None)
    assert rc == -1   # unknown layout
    rc = lib.gpt_op_gemm_fp8(64, 40, 32, fake, 1, K, 32, fake, 0, MN, 48, fake, 64, fake, fake, 0.0, None)
    assert rc == -1   # m/n-contiguous B with N not a multiple of 16
    rc = lib.gpt_op_gemm_fp8(64, 64, 32, fake, 1, MN, 32, fake, 0, MN, 64, fake, 64, fake, fake, 0.0, None)
    assert rc == -1   # lda below M for an m-contiguous A
    assert B.fp8_partials(65536, 1280) == 1024 and B.fp8_partials(16, 16) == 1


def test_fp8_workspace_is_larger(B):
    bf = B.workspace_size(B.shape(4, 4096, 256, 2, B.PREC_BF16))
    f8 = B.workspace_size(B.shape(4, 4096, 256, 2, B.PREC_FP8))
    assert f8 > bf


def test_adamw_and_scaled_bwd_reject_on_host(B):
    lib = B.lib()
    fake = ctypes.c_void_p(4096)
    assert lib.adamw_update(None, None, None, None, None, 0, 1, 1e-3, 0.9, 0.95, 1e-8, 0.0, 1.0, None) == 0
    rc = lib.adamw_update(fake, None, fake, fake, fake, 6, 1, 1e-3, 0.9, 0.95, 1e-8, 0.0, 1.0, None)
    assert rc == -1   # n not a multiple of 4
    rc = lib.adamw_update(fake, None, fake, fake, fake, 8, 0, 1e-3, 0.9, 0.95, 1e-8, 0.0, 1.0, None)
    assert rc == -1   # step is 1-based
    rc = lib.adamw_update(fake, None, None, fake, fake, 8, 1, 1e-3, 0.9, 0.95, 1e-8, 0.0, 1.0, None)
    assert rc == -1   # G NULL
    sh = B.shape(2, 1024, 64, 2)
    params = B.Params(fake, fake, fake)
    rc = lib.gpt_step_bwd_scaled(ctypes.byref(sh), ctypes.byref(params), fake, 0, -1.0, fake, 1 << 40, None)
    assert rc == -1   # loss_scale must be positive
