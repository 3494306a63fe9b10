"""The C ABI on the host side (no GPU): the library loads, exports every entry point that
include/w8inv.h declares, and rejects invalid arguments before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w8inv.h")

w8 = pytest.importorskip("invariant_quantized_decode_amd")
L = w8.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w8[a-z0-9_]*|vocab_[a-z0-9_]*)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 33
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(w8.EXPORTS)


def test_kernel_query_is_host_only_and_rejects_bad_shapes():
    """The kernel-name query is host-only; it names one kernel per (N, K, T_pad, scales alignment)."""
    q = L.w8_linear_invariant_kernel
    assert q(6144, 5120, 32, fake(4096)) == b"gemm_w8g32_split_lds<2, 3, true, 0, false>"
    assert q(6144, 5120, 32, fake(4098)) == b"gemm_w8g32_split_lds<2, 3, false, 0, false>"  # scales not 16-byte aligned
    assert q(248320, 5120, 32, fake(4096)) == b"gemm_w8g32_tiles<2, true, false>"
    assert q(248320, 5120, 32, fake(4098)) == b"gemm_w8g32_tiles<2, false, false>"   # scales not 16-byte aligned
    assert q(248320, 5088, 16, fake(4096)) == b"gemm_w8g32_tiles<1, false, false>"   # K/32 = 159
    assert q(34816, 5120, 64, fake(4096)) == b"gemm_w8g32_split_lds<4, 2, true, 0, false>"
    assert q(5120, 17408, 64, fake(4096)) == b"gemm_w8g32_split_lds<4, 2, false, 0, false>"  # scales too large for LDS
    for bad in ((6144, 5100, 32), (0, 5120, 32), (6144, 5120, 24), (6144, 5120, 80)):
        assert q(*bad, fake(4096)) == b""


def test_status_strings_and_version():
    assert L.w8i_status_string(0) == b"W8I_OK"
    for code in range(-8, 0):
        assert L.w8i_status_string(code).decode().startswith(w8.STATUS[code])
    assert b"gfx950" in L.w8i_version()


def fake(addr):
    """A non-NULL pointer value the validation layer can inspect; never dereferenced on failure paths."""
    return ctypes.c_void_p(addr)


A = 0x10000  # 16-byte aligned dummy address


def linear(W=A, S=A, X=A, t=4, T=32, Y=A, N=64, K=256, ldx=256, ldy=64):
    return L.w8_linear_invariant(fake(W) if W else None, fake(S) if S else None, fake(X) if X else None, t, T,
                                 fake(Y) if Y else None, N, K, ldx, ldy, None, 0, None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=24), -4), (dict(T=128), -4), (dict(t=33), -4), (dict(t=-1), -4),
    (dict(W=0), -1), (dict(Y=0), -1), (dict(X=0), -1), (dict(S=0), -1),
    (dict(K=100, ldx=100), -2), (dict(K=0, ldx=0), -2), (dict(N=0), -2), (dict(ldx=128), -2), (dict(ldy=32), -2),
    (dict(W=A + 8), -3), (dict(X=A + 4), -3), (dict(ldx=260), -3), (dict(S=A + 1), -3), (dict(Y=A + 1), -3),
])
def test_linear_rejects_invalid_arguments(kw, code):
    assert linear(**kw) == code


def test_linear_t_zero_is_a_no_op():
    assert linear(t=0, W=0, S=0, X=0, Y=0) == 0


def test_workspace_queries():
    """The K-slice workspace: 8 fp64 sums per output at the width the kernels run at (min(T_pad, 32)),
    for at most 64 strips of 32 rows; 0 elsewhere and for arguments a call would reject."""
    for q in (L.w8_linear_invariant_workspace_bytes, L.w8_linear_invariant_packed_workspace_bytes):
        q.restype = ctypes.c_size_t
        assert q(6144, 5120, 32) == 0                      # 192 strips: the one-launch kernels
        assert q(1024, 5120, 16) == 8 * 16 * 1024 * 8
        assert q(1024, 5120, 32) == 8 * 32 * 1024 * 8
        assert q(1000, 5120, 64) == 8 * 32 * 1000 * 8       # run at 32 when t <= 32
        assert q(2048, 1024, 48) == 8 * 32 * 2048 * 8
        assert q(2049, 1024, 32) == 0                       # 65 strips
        assert q(1024, 5100, 32) == 0 and q(1024, 5120, 24) == 0 and q(0, 5120, 32) == 0


def test_misaligned_workspace_is_rejected():
    args = (fake(A), fake(A), fake(A), 4, 32, fake(A), 64, 256, 256, 64)
    assert L.w8_linear_invariant(*args, fake(A + 4), 1 << 20, None) == -3
    assert L.w8_linear_invariant_packed(*args, fake(A + 4), 1 << 20, None) == -3


def linear_add(W=A, S=A, X=A, R=A + 0x100000, t=4, T=32, Y=A + 0x200000, N=64, K=256, ldx=256, ldr=64, ldy=64):
    return L.w8_linear_add_invariant(fake(W) if W else None, fake(S) if S else None, fake(X) if X else None,
                                     fake(R) if R else None, t, T, fake(Y) if Y else None, N, K, ldx, ldr, ldy, None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=24), -4), (dict(t=33), -4), (dict(R=0), -1), (dict(W=0), -1), (dict(ldr=32), -2),
    (dict(R=A + 0x100001), -3), (dict(X=A + 4), -3), (dict(K=100, ldx=100), -2),
    (dict(R=A + 0x200000 + 2), -2),                    # residual overlaps y without being y
    (dict(R=A + 0x200000, ldr=128, ldy=64), -2),       # same pointer, different strides
])
def test_linear_add_rejects_invalid_arguments(kw, code):
    assert linear_add(**kw) == code


def test_linear_add_accepts_y_equal_to_residual_and_t_zero():
    assert linear_add(t=0, W=0, S=0, X=0, R=0, Y=0) == 0
    # validation passes for exact aliasing (launch not reached: t = 0 short-circuits before any device work)
    assert linear_add(t=0, R=A + 0x200000) == 0


def linear_swiglu(W=A, S=A, X=A, t=4, T=32, Y=A, F=64, K=256, ldx=256, ldy=64):
    return L.w8_linear_swiglu_invariant(fake(W) if W else None, fake(S) if S else None, fake(X) if X else None,
                                        t, T, fake(Y) if Y else None, F, K, ldx, ldy, None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=80), -4), (dict(t=-1), -4), (dict(F=0), -2), (dict(ldy=63), -2), (dict(Y=0), -1), (dict(S=0), -1),
    (dict(W=A + 4), -3), (dict(K=96, ldx=96, F=1 << 31), -2),   # 2F * K >= 2^32
])
def test_linear_swiglu_rejects_invalid_arguments(kw, code):
    assert linear_swiglu(**kw) == code


def test_pack_sizes_and_validation():
    wb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert L.w8_pack_bytes(6144, 5120, ctypes.byref(wb), ctypes.byref(sb)) == 0
    assert (wb.value, sb.value) == (192 * 80 * 2048, 192 * 80 * 128)     # whole strips x pairs of groups
    assert L.w8_pack_bytes(33, 160, ctypes.byref(wb), ctypes.byref(sb)) == 0
    assert (wb.value, sb.value) == (2 * 3 * 2048, 2 * 3 * 128)          # ragged rows, odd K/32 padded
    assert L.w8_pack_bytes(33, 100, ctypes.byref(wb), ctypes.byref(sb)) == -2
    assert L.w8_pack_bytes(1 << 20, 8192, ctypes.byref(wb), ctypes.byref(sb)) == -2   # 8 GiB of codes
    assert L.w8_pack_bytes(64, 256, None, ctypes.byref(sb)) == -1
    assert L.w8_pack(fake(A), fake(A), 64, 256, fake(A + 8), fake(A), None) == -3
    assert L.w8_pack(fake(A), None, 64, 256, fake(A), fake(A), None) == -1
    assert L.w8_pack(fake(A), fake(A), 64, 250, fake(A), fake(A), None) == -2


def test_packed_kernel_query():
    q = L.w8_linear_invariant_packed_kernel
    assert q(6144, 5120, 32) == b"gemm_w8g32_split_lds<2, 3, false, 0, true>"
    assert q(1024, 5120, 64) == b"gemm_w8g32_split_lds<4, 2, false, 0, true>"  # t > 32 at T_pad 64
    assert q(34816, 5120, 64) == b"gemm_w8g32_split_lds<4, 2, false, 0, true>"
    assert q(248320, 5120, 32) == b"gemm_w8g32_tiles<2, false, true>"
    assert q(248320, 5120, 64) == b"gemm_w8g32_split_lds<4, 2, false, 0, true>"
    assert q(6144, 5100, 32) == b"" and q(6144, 5120, 24) == b""


def test_packed_linear_validation():
    f = L.w8_linear_invariant_packed
    assert f(fake(A), fake(A), fake(A), 0, 32, fake(A), 64, 256, 256, 64, None, 0, None) == 0
    assert f(fake(A), fake(A), fake(A), 4, 24, fake(A), 64, 256, 256, 64, None, 0, None) == -4
    assert f(fake(A), fake(A + 4), fake(A), 4, 32, fake(A), 64, 256, 256, 64, None, 0, None) == -3
    assert f(None, fake(A), fake(A), 4, 32, fake(A), 64, 256, 256, 64, None, 0, None) == -1
    assert f(fake(A), fake(A), fake(A), 4, 32, fake(A), 64, 256, 256, 32, None, 0, None) == -2


def logprob(Lg=A, T=A, block=4096, out=A, t=4, V=248320, ldl=248320, ws=A, wsb=1 << 20):
    return L.vocab_block_logprob(fake(Lg) if Lg else None, fake(T) if T else None, block, fake(out) if out else None,
                                 t, V, ldl, fake(ws) if ws else None, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(block=1000), -5), (dict(block=128), -5), (dict(block=65536), -5),
    (dict(t=-1), -4), (dict(Lg=0), -1), (dict(T=0), -1), (dict(out=0), -1),
    (dict(V=0, ldl=0), -2), (dict(ldl=1000), -2),
    (dict(Lg=A + 1), -3), (dict(T=A + 4), -3), (dict(out=A + 2), -3),
    (dict(ws=0), -6), (dict(wsb=100), -6), (dict(ws=A + 4), -3),
])
def test_logprob_rejects_invalid_arguments(kw, code):
    assert logprob(**kw) == code


def test_direct_and_argmax_validation():
    assert L.vocab_block_logprob_direct(fake(A), fake(A), 1000, fake(A), 4, 248320, 248320, fake(A), 1 << 20,
                                        None) == -5
    assert L.vocab_block_logprob_direct(fake(A), fake(A), 4096, fake(A), 4, 248320, 248320, fake(A), 100, None) == -6
    f = L.vocab_argmax
    need = L.vocab_argmax_workspace_bytes(32, 248320)
    assert need == 32 * 61 * 8
    assert f(fake(A), fake(A), 0, 248320, 248320, None, 0, None) == 0
    assert f(None, fake(A), 4, 248320, 248320, fake(A), need, None) == -1
    assert f(fake(A), fake(A + 4), 4, 248320, 248320, fake(A), need, None) == -3
    assert f(fake(A), fake(A), 4, 248320, 1000, fake(A), need, None) == -2
    assert f(fake(A), fake(A), 4, (1 << 31) + 1, (1 << 31) + 1, fake(A), 1 << 30, None) == -2
    assert f(fake(A), fake(A), 4, 248320, 248320, fake(A), 10, None) == -6
    assert f(fake(A), fake(A), 4, 248320, 248320, fake(A + 4), need, None) == -3


def test_logprob_workspace_size():
    nb = (248320 + 4095) // 4096
    need = L.vocab_block_logprob_workspace_bytes(32, 248320, 4096)
    assert need >= 2 * 32 * nb * 4 and need % 256 == 0
    assert L.vocab_block_logprob_workspace_bytes(32, 248320, 1000) == 0
    assert logprob(t=0, Lg=0, T=0, out=0, ws=0) == 0


def test_noalloc_logprob_validation():
    """The entry point that allocates nothing validates like vocab_block_logprob and refuses, before any
    device access, a call whose maxima and partials would not fit the fixed 1 MiB scratch."""
    f = L.vocab_block_logprob_noalloc
    assert w8.NOALLOC_SCRATCH_BYTES == 1 << 20
    assert f(fake(A), fake(A), 1000, fake(A), 4, 248320, 248320, None) == -5
    assert f(fake(A), fake(A), 4096, fake(A), -1, 248320, 248320, None) == -4
    assert f(None, None, 4096, None, 0, 248320, 248320, None) == 0
    assert f(None, fake(A), 4096, fake(A), 4, 248320, 248320, None) == -1
    assert f(fake(A), fake(A), 4096, fake(A), 4, 248320, 1000, None) == -2
    assert f(fake(A), fake(A + 4), 4096, fake(A), 4, 248320, 248320, None) == -3
    # 64 columns x 2^22 entries in blocks of 4096: 2 x 256 KiB fits; blocks of 256: 2 x 4 MiB does not
    assert L.vocab_block_logprob_workspace_bytes(64, 1 << 22, 4096) <= 1 << 20
    assert L.vocab_block_logprob_workspace_bytes(64, 1 << 22, 256) > 1 << 20
    assert f(fake(A), fake(A), 256, fake(A), 64, 1 << 22, 1 << 22, None) == -8
    assert L.w8i_status_string(-8).decode().startswith("W8I_ESCRATCH")


def test_pair_and_attn_input_proj_validation():
    """linear_pair checks both projections' operands; attn_input_proj checks the norm's input, the
    workspace and the projection, all before any device access."""
    f = L.w8_linear_pair_invariant
    ok = (fake(A), fake(A), fake(A), fake(A), fake(A), 4, 32, fake(A), fake(A), 64, 32, 256, 256, 64, 32, None)
    assert f(*ok[:5], 0, 32, None, None, 64, 32, 256, 256, 64, 32, None) == 0          # t == 0
    assert f(*ok[:5], 4, 24, *ok[7:]) == -4                                             # T_pad
    assert f(fake(A), fake(A), None, fake(A), *ok[4:]) == -1                            # Wb NULL
    assert f(*ok[:9], 64, 32, 256, 256, 64, 16, None) == -2                             # ldyb < Nb
    assert f(*ok[:2], fake(A + 8), *ok[3:]) == -3                                       # Wb misaligned
    assert L.w8_linear_pair_invariant_packed(fake(A), fake(A), fake(A), fake(A + 2), *ok[4:]) == -3  # Spb
    g = L.w8_attn_input_proj_invariant
    need = L.w8_attn_input_proj_workspace_bytes(32, 5120)
    assert need == 32 * 5120 * 2
    assert L.w8_attn_input_proj_workspace_bytes(3, 100) == 768 and L.w8_attn_input_proj_workspace_bytes(3, 70000) == 0
    args = lambda **kw: [kw.get(k, v) for k, v in dict(  # noqa: E731
        h=fake(A), w=None, eps=ctypes.c_float(1e-6), W=fake(A), S=fake(A), t=4, T=32, y=fake(A), N=7168, H=5120,
        ldh=5120, ldy=7168, ws=fake(A), wsb=L.w8_attn_input_proj_workspace_bytes(4, 5120), st=None).items()]
    need = L.w8_attn_input_proj_workspace_bytes(4, 5120)
    assert g(*args()) != -6 and g(*args(t=0, h=None, W=None)) == 0
    assert g(*args(ws=None)) == -6 and g(*args(wsb=need - 2)) == -6 and g(*args(ws=fake(A + 8))) == -3
    assert g(*args(h=None)) == -1 and g(*args(H=70000, ldh=70000)) == -2 and g(*args(ldh=100)) == -2
    assert g(*args(H=5100, ldh=5100)) == -2           # the projection's K = H must be a multiple of 32
    assert g(*args(T=40)) == -4 and g(*args(W=None)) == -1


def test_fused_head_logprob_validation():
    f = L.w8_head_logprob_invariant
    need = L.w8_head_logprob_workspace_bytes(32, 248320, 4096)
    assert need == 32 * 970 * 4 + 32 * 61 * 4 + (256 - 32 * 61 * 4 % 256)  # maxima and partials, each 256-aligned
    assert L.w8_head_logprob_workspace_bytes(32, 248320, 1000) == 0
    args = lambda **kw: [kw.get(k, v) for k, v in dict(  # noqa: E731
        W=fake(A), S=fake(A), x=fake(A), tg=fake(A), t=4, T=32, block=4096, lg=fake(A), out=fake(A), V=248320,
        K=5120, ldx=5120, ldl=248320, ws=fake(A), wsb=L.w8_head_logprob_workspace_bytes(4, 248320, 4096),
        st=None).items()]
    need = L.w8_head_logprob_workspace_bytes(4, 248320, 4096)
    assert f(*args(t=0, W=None)) == 0
    assert f(*args(T=64, t=40)) == -4 and f(*args(T=24)) == -4
    assert f(*args(block=1000)) == -5 and f(*args(tg=None)) == -1 and f(*args(out=None)) == -1
    assert f(*args(ldl=1000)) == -2 and f(*args(ws=None)) == -6 and f(*args(wsb=need - 4)) == -6
    assert f(*args(ws=fake(A + 8))) == -3 and f(*args(out=fake(A + 2))) == -3
    assert L.w8_head_logprob_invariant_packed(*args(S=fake(A + 2))) == -3


def test_glue_and_hooks_reject_invalid_arguments():
    assert L.w8i_rmsnorm(None, None, ctypes.c_float(1e-6), fake(A), 2, 64, 64, 64, None) == -1
    assert L.w8i_rmsnorm(fake(A), None, ctypes.c_float(1e-6), fake(A), 2, 70000, 70000, 70000, None) == -2
    assert L.w8i_swiglu(fake(A), fake(A), 2, 64, 100, 64, None) == -2
    assert L.w8i_residual_add(fake(A), fake(A + 1), fake(A), 2, 64, 64, 64, 64, None) == -3
    assert L.w8i_exp32(fake(A), fake(A + 2), 10, None) == -3
    assert L.w8i_log32(None, fake(A), 10, None) == -1
    assert L.w8i_exp32(None, None, 0, None) == 0


def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros((64, 256), dtype=torch.int8)
    s = torch.zeros((64, 8), dtype=torch.float16)
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        w8.w8_linear_invariant(q, s, x, 4, 32, y=torch.zeros((4, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        w8.w8i_exp32(torch.zeros(8), y=torch.zeros(8))


def test_calibration_library_exports_its_header_and_validates():
    """libw8calib.so (the measurement helpers of include/w8calib.h, outside the decode path) exports
    what its header declares and rejects bad arguments on the host."""
    from invariant_quantized_decode_amd import calib
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "w8calib.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(w8c_[a-z0-9_]*)\s*\(", text)))
    assert names == ["w8c_mfma_bf16", "w8c_stream_read", "w8c_strip_read"]
    C = calib._lib()
    for n in names:
        assert hasattr(C, n), n
    fake = ctypes.c_void_p(256)  # never dereferenced: every call below fails validation first
    assert C.w8c_stream_read(None, 1024, 1, fake, 2048, None) == -1
    assert C.w8c_stream_read(fake, 1000, 1, fake, 2048, None) == -2       # not a multiple of 16
    assert C.w8c_stream_read(fake, 1024, 0, fake, 2048, None) == -2       # no workgroups
    assert C.w8c_stream_read(ctypes.c_void_p(264), 1024, 1, fake, 2048, None) == -3
    assert C.w8c_stream_read(fake, 1024, 2, fake, 2048, None) == -6       # sink for one workgroup only
    assert C.w8c_mfma_bf16(1, 1, None, 1024, None) == -1
    assert C.w8c_mfma_bf16(1, 0, fake, 1024, None) == -2
    assert C.w8c_mfma_bf16(0, 1, fake, 1024, None) == -2
    assert C.w8c_mfma_bf16(2, 1, fake, 1024, None) == -6
    assert C.w8c_strip_read(fake, None, 8, 80, 1, fake, 2048, None) == -1
    assert C.w8c_strip_read(fake, fake, 0, 80, 1, fake, 2048, None) == -2      # no strips
    assert C.w8c_strip_read(fake, fake, 8, 1 << 20, 1, fake, 2048, None) == -2  # 2^32 bytes of codes or more
    assert C.w8c_strip_read(fake, fake, 8, 80, 0, fake, 2048, None) == -2      # no workgroups
    assert C.w8c_strip_read(ctypes.c_void_p(264), fake, 8, 80, 1, fake, 2048, None) == -3
    assert C.w8c_strip_read(fake, fake, 8, 80, 2, fake, 2048, None) == -6      # sink for one workgroup only


def test_kernel_digest_follows_code_not_comments():
    """The digest that ties a stored counter profile to the kernel it measured ignores comments and
    layout but not code (string and character literals included)."""
    import invariant_quantized_decode_amd as w8
    a = 'int f(int x) { return x + 1; } // one\n'
    assert w8._code_only(a) == w8._code_only('/* doc */ int f(int x)\n{\n    return x + 1;  // two\n}\n')
    assert w8._code_only(a) != w8._code_only('int f(int x) { return x + 2; }')
    assert w8._code_only('s = "a // b";') == 's = "a // b";'
    assert w8._code_only("c = '/'; /* x */ d = '\\''; // y") == "c = '/'; d = '\\'';"
    assert re.fullmatch(r"[0-9a-f]{16}", w8.kernel_source_digest())
