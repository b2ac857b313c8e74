"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol include/vw4.h declares, validates arguments before enqueuing
anything, and its host quantiser matches the oracle bit for bit."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from verify_step_w4_amd import binding as B
from verify_step_w4_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "vw4.h")).read()
    return set(re.findall(r"^VW4_API\s+[\w\s\*]+?\b(\w+)\(", src, flags=re.M))


def test_exports_every_declared_symbol():
    names = _declared()
    assert {"w4_skinny_gemm", "verify_logits", "spec_accept"} <= names
    L = B.lib()
    for n in names:
        assert hasattr(L, n), n
    assert names == set(B.SIGNATURES), "binding signatures out of sync with vw4.h"


def test_version_and_error_strings():
    assert B.version().startswith("vw4")
    assert isinstance(B.last_error(), str)


def test_rowstat_layout():
    assert B.ROWSTAT_DTYPE.itemsize == 32
    assert B.ROWSTAT_DTYPE.fields["log_z"][1] == 8
    assert B.ROWSTAT_DTYPE.fields["argmax"][1] == 16


def test_host_quantizer_matches_oracle():
    g = np.random.default_rng(4)
    w = (g.standard_normal((33, 640)) * 0.02).astype(np.float32)
    w[0, :64] = 0.0
    w[1, 64:128] *= 1e-7          # fp16-subnormal scale
    w[2, 128:192] = 1.5e-8         # scale underflows to zero
    w[3, 192:256] = np.float32(7.5) * np.float32(2.0 ** -10)  # exact halves
    c1, s1 = B.w4_quantize_host(w)
    c2, s2 = oracle.w4_quantize(w)
    assert np.array_equal(s1, s2)
    assert np.array_equal(c1, c2)


def test_host_quantizer_on_a_layer_shape():
    w = synth.linear_weights(7, 64, 5120)
    c1, s1 = B.w4_quantize_host(w)
    c2, s2 = oracle.w4_quantize(w)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_packed_sizes():
    cb, sb = B.packed_sizes(100, 320)
    assert cb == 128 * 160 and sb == 128 * 5 * 2
    assert B.lib().vw4_w4_packed_bytes(10, 100, None) == 0


def test_workspace_queries():
    assert B.gemm_workspace_bytes(4, 151936, 5120) == 0          # enough tiles: no K split across workgroups
    assert B.gemm_workspace_bytes(4, 5120, 5120) > 0
    assert B.verify_workspace_bytes(4, 151936) > 0
    assert B.accept_workspace_bytes(1, 151936) > 0
    assert B.lib().vw4_workspace_bytes(0, 10) == 0
    assert B.lib().vw4_accept_workspace_bytes(1, 0) == 0


def _call(name, *args):
    return getattr(B.lib(), name)(*args)


@pytest.mark.parametrize("M,N,K,ldx,ldy,ydt", [
    (0, 64, 64, 64, 64, 0), (9, 64, 64, 64, 64, 0), (1, 0, 64, 64, 64, 0), (1, 64, 100, 128, 64, 0),
    (1, 64, 64, 60, 64, 0), (1, 64, 64, 64, 10, 0), (1, 64, 64, 64, 64, 7),
])
def test_gemm_rejects_bad_arguments(M, N, K, ldx, ldy, ydt):
    fake = ctypes.c_void_p(0x100000)  # never dereferenced: validation fails first
    rc = _call("w4_skinny_gemm", fake, ldx, fake, fake, fake, ldy, ydt, M, N, K, None, 0, None)
    assert rc == B.VW4_EINVAL
    assert "w4_skinny_gemm" in B.last_error()


def test_gemm_requires_workspace_when_split():
    fake = ctypes.c_void_p(0x100000)
    rc = _call("w4_skinny_gemm", fake, 5120, fake, fake, fake, 5120, 0, 4, 5120, 5120, None, 0, None)
    assert rc == B.VW4_EWORKSPACE


def test_verify_logits_rejects_bad_arguments():
    fake = ctypes.c_void_p(0x100000)
    assert _call("verify_logits", None, 0, None, None, 0, 100, 64, 0.6, 0.95, fake, fake, fake, 1 << 20,
                 None) == B.VW4_EINVAL
    assert _call("verify_logits", None, 0, None, None, 4, 100, 64, -1.0, 0.95, fake, fake, fake, 1 << 20,
                 None) == B.VW4_EINVAL
    assert _call("verify_logits", None, 0, None, None, 4, 100, 64, 0.6, 0.0, fake, fake, fake, 1 << 20,
                 None) == B.VW4_EINVAL
    assert _call("verify_logits", None, 0, None, None, 4, 100, 64, 0.6, 0.95, fake, fake, fake, 16,
                 None) == B.VW4_EWORKSPACE


def test_spec_accept_rejects_bad_arguments():
    fake = ctypes.c_void_p(0x100000)
    args = lambda B_, D, V: (fake, 0, fake, 0, fake, 0, fake, B_, D, V, 0.6, 1, 0, fake, fake, fake, fake,
                             1 << 20, None)
    assert _call("spec_accept", *args(1, 8, 100)) == B.VW4_EINVAL
    assert _call("spec_accept", *args(0, 3, 100)) == B.VW4_EINVAL
    assert _call("spec_accept", *args(1, 3, 0)) == B.VW4_EINVAL
    a = list(args(1, 3, 100))
    a[4] = None  # q missing with D > 0
    assert _call("spec_accept", *a) == B.VW4_EINVAL


def test_draft_side_rejects_bad_arguments():
    fake = ctypes.c_void_p(0x100000)   # 256-byte aligned, never dereferenced: validation fails first
    assert B.lib().vw4_draft_workspace_bytes(0) == 0
    assert B.draft_workspace_bytes(151936) > B.accept_workspace_bytes(1, 151936)
    ws = B.draft_workspace_bytes(1000)
    ds = lambda V, T, depth, ws_bytes, tok=fake: _call("draft_sample", fake, fake, V, T, 1, None, 0, depth, fake, tok,
                                                       fake, fake, ws_bytes, None)
    assert ds(0, 0.6, 0, ws) == B.VW4_EINVAL
    assert ds(1000, -0.5, 0, ws) == B.VW4_EINVAL
    assert ds(1000, 0.6, 1024, ws) == B.VW4_EINVAL
    assert ds(1000, 0.6, 0, ws, tok=None) == B.VW4_EINVAL
    assert ds(1000, 0.6, 0, 64) == B.VW4_EWORKSPACE
    mi = lambda d, ldh, eps=1e-6: _call("vw4_mtp_input", fake, ldh, 2, None, fake, d, 100, fake, fake, fake, eps, d,
                                        fake, None)
    assert mi(12, 16) == B.VW4_EINVAL          # d % 8
    assert mi(8200, 8200) == B.VW4_EINVAL      # d > 8192
    assert mi(256, 128) == B.VW4_EINVAL        # ldh < d
    assert mi(256, 256, eps=-1.0) == B.VW4_EINVAL
    assert "vw4_mtp_input" in B.last_error()
    er = lambda d, n: _call("vw4_embed_rows", fake, d, 100, d, fake, n, fake, d, None)
    assert er(256, 0) == B.VW4_EINVAL
    assert er(12, 1) == B.VW4_EINVAL
    assert "vw4_embed_rows" in B.last_error()


def test_w8_host_quantizer_matches_oracle():
    rng = np.random.default_rng(12)
    w = rng.normal(0.0, 0.02, (45, 384)).astype(np.float32)
    w[2, :64] = 0.0
    w[4, 64:128] = 1e-9
    w[6, 200] = -5.0
    c1, s1 = B.w8_quantize_host(w)
    c2, s2 = oracle.w8_quantize(w)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_w8_gemm_rejects_bad_arguments():
    fake = ctypes.c_void_p(0x100000)
    g = lambda M, N, K, ldx, ydt: _call("w8_skinny_gemm", fake, ldx, fake, fake, fake, fake, N, ydt, M, N, K, None, 0,
                                        None)
    assert g(0, 64, 64, 64, 0) == B.VW4_EINVAL
    assert g(9, 64, 64, 64, 0) == B.VW4_EINVAL
    assert g(1, 64, 100, 128, 0) == B.VW4_EINVAL
    assert g(1, 64, 64, 60, 0) == B.VW4_EINVAL
    assert g(1, 64, 64, 64, 5) == B.VW4_EINVAL
    assert g(4, 5120, 5120, 5120, 0) == B.VW4_EWORKSPACE      # split-K plan, no workspace
    assert B.w8_workspace_bytes(4, 5120, 5120) > 0 and B.lib().vw4_w8_workspace_bytes(0, 64, 64) == 0


def test_w8_partials_layout_and_validation():
    # the layout does not depend on M (so verify rows equal one-row steps), and
    # never exceeds the 8 slices the decoder's consumers read
    for N, K in ((7168, 5120), (5120, 5120), (34816, 5120), (5120, 17408), (151936, 5120)):
        lay = {M: B.w8_partials_layout(M, N, K) for M in (1, 4, 8)}
        assert len(set(lay.values())) == 1
        S, ldp = lay[1]
        assert 1 <= S <= 8 and ldp % 64 == 0 and ldp >= N
    fake = ctypes.c_void_p(0x100000)
    assert _call("w8_skinny_gemm_partials", fake, 60, fake, fake, fake, fake, 1, 64, 64, None) == B.VW4_EINVAL
    assert _call("w8_skinny_gemm_partials", fake, 64, fake, fake, fake, fake, 9, 64, 64, None) == B.VW4_EINVAL
    assert _call("w8_skinny_gemm_partials", fake, 64, fake, fake, fake, None, 1, 64, 64, None) == B.VW4_EINVAL


def test_k_beyond_the_largest_is_rejected():
    """K = 65536 is the largest accepted; the next multiple of 64 is refused
    by every format's workspace query and partial-slice layout."""
    for name in ("vw4_w8_workspace_bytes", "vw4_w6_workspace_bytes", "vw4_w5_workspace_bytes",
                 "vw4_w3_workspace_bytes", "vw4_w2_workspace_bytes", "vw4_f16_workspace_bytes",
                 "vw4_bf16_workspace_bytes"):
        assert getattr(B.lib(), name)(4, 64, 65600) == 0, name
    for fn in (B.w8_partials_layout, B.w6_partials_layout, B.w5_partials_layout, B.w3_partials_layout,
               B.w2_partials_layout):
        with pytest.raises(B.VW4Error):
            fn(4, 64, 65600)
        assert fn(4, 64, 65536)[0] >= 1
    with pytest.raises(B.VW4Error):
        B.gemm_partials_layout(4, 64, 65600)


def test_swiglu_entry_points_validate():
    fake = ctypes.c_void_p(0x100000)
    for fmt in ("w8", "w6", "w5", "w3"):
        f = f"{fmt}_skinny_gemm_swiglu"
        assert _call(f, fake, 64, fake, fake, fake, fake, 32, 4, 48, 64, None) == B.VW4_EINVAL     # F % 32
        assert _call(f, fake, 64, fake, fake, fake, fake, 16, 4, 32, 64, None) == B.VW4_EINVAL     # lda < F
        assert _call(f, fake, 64, fake, fake, fake, None, 32, 4, 32, 64, None) == B.VW4_EINVAL     # null a
    assert _call("w2_skinny_gemm_swiglu", fake, 64, fake, fake, fake, 32, 9, 32, 64, None) == B.VW4_EINVAL
    for kind in ("f16", "bf16"):
        assert _call(f"{kind}_skinny_gemm_swiglu", fake, 60, fake, fake, 32, 1, 32, 64, None) == B.VW4_EINVAL


def test_w16_sizes_and_validation():
    assert B.lib().vw4_w16_packed_bytes(100, 320) == 128 * 320 * 2
    assert B.lib().vw4_w16_packed_bytes(10, 100) == 0
    for kind in ("f16", "bf16"):
        assert B.w16_workspace_bytes(9, 64, 64, kind) == 0
        assert B.w16_workspace_bytes(4, 5120, 5120, kind) == B.gemm_workspace_bytes(4, 5120, 5120)
        assert B.w16_partials_layout(4, 5120, 5120, kind) == B.w16_partials_layout(1, 5120, 5120, kind)
        fake = ctypes.c_void_p(0x100000)
        assert _call(f"{kind}_skinny_gemm", fake, 64, fake, fake, 64, 0, 9, 64, 64, None, 0, None) == B.VW4_EINVAL
        assert _call(f"{kind}_skinny_gemm", fake, 64, None, fake, 64, 0, 1, 64, 64, None, 0, None) == B.VW4_EINVAL
        assert _call(f"{kind}_skinny_gemm", fake, 64, fake, fake, 64, 0, 1, 64, 100, None, 0, None) == B.VW4_EINVAL
        assert _call(f"{kind}_skinny_gemm_partials", fake, 64, fake, None, 1, 64, 64, None) == B.VW4_EINVAL
    assert _call("vw4_w16_pack", None, 64, 64, ctypes.c_void_p(0x100000), None) == B.VW4_EINVAL


@pytest.mark.parametrize("b", [3, 2])
def test_w3_w2_host_quantizers_match_oracle_and_sizes(b):
    rng = np.random.default_rng(20 + b)
    w = rng.normal(0.0, 0.02, (45, 384)).astype(np.float32)
    w[3, 64:128] = 0.0
    w[7, 100] = 4.0
    c1, s1 = getattr(B, f"w{b}_quantize_host")(w)
    c2, s2 = getattr(oracle, f"w{b}_quantize")(w)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    assert c1.min() >= (1 if b == 3 else 0) and c1.max() <= (7 if b == 3 else 2)
    if b == 3:
        assert B.lib().vw4_w3_hi_plane_bytes(100, 320) == 128 * 320 // 8
        assert B.lib().vw4_w3_lo_plane_bytes(100, 320) == 128 * 320 // 4
        assert B.lib().vw4_w3_lo_plane_bytes(10, 100) == 0
        assert B.w3_workspace_bytes(9, 64, 64) == 0
    else:
        assert B.lib().vw4_w2_packed_bytes(100, 320) == 128 * 320 // 4
        assert B.lib().vw4_w2_packed_bytes(10, 100) == 0
        assert B.w2_workspace_bytes(9, 64, 64) == 0
    fake = ctypes.c_void_p(0x100000)
    if b == 3:
        assert _call("w3_skinny_gemm", fake, 64, fake, fake, fake, fake, 64, 0, 9, 64, 64, None, 0, None) == B.VW4_EINVAL
        assert _call("w3_skinny_gemm_partials", fake, 64, fake, fake, fake, None, 1, 64, 64, None) == B.VW4_EINVAL
    else:
        assert _call("w2_skinny_gemm", fake, 64, fake, fake, fake, 64, 0, 9, 64, 64, None, 0, None) == B.VW4_EINVAL
        assert _call("w2_skinny_gemm", fake, 60, fake, fake, fake, 64, 0, 1, 64, 64, None, 0, None) == B.VW4_EINVAL
        assert _call("w2_skinny_gemm_partials", fake, 64, fake, fake, None, 1, 64, 64, None) == B.VW4_EINVAL


def test_w5_host_quantizer_matches_oracle_and_sizes():
    rng = np.random.default_rng(11)
    w = rng.normal(0.0, 0.02, (45, 384)).astype(np.float32)
    w[3, 64:128] = 0.0
    w[7, 100] = 4.0
    c1, s1 = B.w5_quantize_host(w)
    c2, s2 = oracle.w5_quantize(w)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    assert c1.min() >= 1 and c1.max() <= 31
    assert B.lib().vw4_w5_hi_plane_bytes(100, 320) == 128 * 320 // 8
    assert B.lib().vw4_w5_hi_plane_bytes(10, 100) == 0
    assert B.w5_workspace_bytes(9, 64, 64) == 0
    fake = ctypes.c_void_p(0x100000)
    assert _call("w5_skinny_gemm", fake, 64, fake, fake, fake, fake, 64, 0, 9, 64, 64, None, 0, None) == B.VW4_EINVAL
    assert _call("w5_skinny_gemm_partials", fake, 64, fake, fake, fake, None, 1, 64, 64, None) == B.VW4_EINVAL


def test_w6_host_quantizer_matches_oracle_and_sizes():
    rng = np.random.default_rng(13)
    w = rng.normal(0.0, 0.02, (45, 384)).astype(np.float32)
    w[2, :64] = 0.0
    w[6, 200] = -5.0
    c1, s1 = B.w6_quantize_host(w)
    c2, s2 = oracle.w6_quantize(w)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    assert B.lib().vw4_w6_hi_plane_bytes(100, 320) == 128 * 320 // 4
    assert B.lib().vw4_w6_hi_plane_bytes(10, 100) == 0
    fake = ctypes.c_void_p(0x100000)
    assert _call("w6_skinny_gemm", fake, 64, fake, fake, fake, fake, 64, 0, 9, 64, 64, None, 0, None) == B.VW4_EINVAL
