"""Host-side tests of the C ABI (no GPU, no compute call).

The library must load, export every function include/linattn.h declares, and
reject invalid arguments on the host with the documented status before any
HIP call; zero sizes are a no-op.
"""
import ctypes
import os
import re

import pytest

import kernelized_attention_scan_amd as K
from kernelized_attention_scan_amd import _binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(
    __file__))), "include", "linattn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(K.LIB_PATH):
        pytest.fail("liblinattn.so not built: run python -m "
                    "kernelized_attention_scan_amd.build")
    return K.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert header_functions() == sorted(B.SYMBOLS)


def test_library_exports_every_header_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_status_strings(lib):
    names = [lib.la_status_str(i).decode() for i in range(6)]
    assert names == ["LA_OK", "LA_ERR_INVALID_ARG", "LA_ERR_UNSUPPORTED",
                     "LA_ERR_WORKSPACE", "LA_ERR_HIP", "LA_ERR_EXCHANGE"]
    assert lib.la_status_str(99).decode() == "LA_ERR_UNKNOWN"


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def fwd(lib, B=1, H=1, n=64, d=64, df=64, mapk=1, omega=None, decay=None,
        causal=1, dtype=1, ws=None, ptr=FAKE):
    return lib.la_forward(ptr, ptr, ptr, ptr, B, H, n, d, df, mapk, omega,
                          decay, causal, dtype, ws, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), B.LA_ERR_INVALID_ARG),
    (dict(H=-2), B.LA_ERR_INVALID_ARG),
    (dict(n=-5), B.LA_ERR_INVALID_ARG),
    (dict(mapk=7), B.LA_ERR_INVALID_ARG),
    (dict(dtype=5), B.LA_ERR_INVALID_ARG),
    (dict(causal=2), B.LA_ERR_INVALID_ARG),
    (dict(d=0), B.LA_ERR_INVALID_ARG),
    (dict(df=-1), B.LA_ERR_INVALID_ARG),
    (dict(df=32), B.LA_ERR_INVALID_ARG),             # ELU1 needs d_feat == d
    (dict(d=48, df=48), B.LA_ERR_UNSUPPORTED),
    (dict(d=256, df=256), B.LA_ERR_UNSUPPORTED),
    (dict(mapk=0, df=512), B.LA_ERR_UNSUPPORTED),
    (dict(mapk=2, df=256, omega=None), B.LA_ERR_INVALID_ARG),  # no omega
    (dict(ptr=None), B.LA_ERR_INVALID_ARG),
    (dict(B=8, n=4096, ws=None), B.LA_ERR_WORKSPACE),          # segments
    (dict(causal=0, n=4096, ws=None), B.LA_ERR_WORKSPACE),     # segments
])
def test_forward_rejects(lib, kw, status):
    assert fwd(lib, **kw) == status
    assert lib.la_last_error().decode() != ""


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(n=0),
                                dict(B=0, ptr=None)])
def test_forward_zero_sizes_are_noops(lib, kw):
    assert fwd(lib, **kw) == B.LA_OK


def test_workspace_bytes(lib):
    # single segment, causal, elu1: no workspace
    assert K.forward_workspace_bytes(1, 1, 64, 64, 64) == 0
    # rejected arguments report 0
    assert K.forward_workspace_bytes(-1, 1, 64, 64, 64) == 0
    assert K.forward_workspace_bytes(1, 1, 64, 48, 48) == 0
    # segmented: a fixed synchronisation area (256 bytes + 512 lines of 128
    # bytes, one per unit a split can have) + units * nseg fp32 aggregates of
    # d' x (d + 16) (mu and, in the extra 16-column block, nu) + units * nseg
    # floats (each segment's sum of log decay, for per-position decay)
    sync = 256 + 512 * 128
    ws = K.forward_workspace_bytes(4, 8, 4096, 64, 64)
    units = 32
    nseg = 8                     # 256 target groups (one per CU) / 32 units
    slot = 64 * (64 + 16)
    a256 = lambda x: (x + 255) // 256 * 256
    assert ws == sync + a256(units * nseg * slot * 4) + a256(units * nseg * 4)
    # at most 16 segments per unit
    one = K.forward_workspace_bytes(1, 1, 1 << 16, 64, 64)
    assert one == sync + a256(16 * slot * 4) + a256(16 * 4)
    # 512 units or more: one segment each, no workspace
    assert K.forward_workspace_bytes(8, 64, 1 << 16, 64, 64) == 0
    # bf16 Performer: the map is fused into the forward, so no q', k' in the
    # workspace; one workgroup per CU -> 256 target groups / 32 units = 8
    # segments, aggregates of d' x (d + 16) = 256 x 80
    wp = K.forward_workspace_bytes(4, 8, 8192, 64, 256, "performer")
    assert wp == sync + a256(32 * 8 * 256 * 80 * 4) + a256(32 * 8 * 4)
    # fp32 storage keeps the unfused map: Q', K' (fp32, m wide) in it
    wf = K.forward_workspace_bytes(4, 8, 8192, 64, 256, "performer",
                                   dtype=__import__("torch").float32)
    assert wf >= 2 * 4 * 8 * 8192 * 256 * 4
    # non-causal over one segment keeps its total on chip; several need one
    assert K.forward_workspace_bytes(1, 1, 64, 64, 64, causal=False) == 0
    assert K.forward_workspace_bytes(1, 1, 4096, 64, 64, causal=False) > 0
    # unfused Performer without segments: Q', K' still start after the
    # synchronisation area, which a shared workspace keeps zero for
    # segmented calls
    f32 = __import__("torch").float32
    assert K.forward_workspace_bytes(1, 2, 17, 32, 128, "performer",
                                     dtype=f32) == sync + 2 * a256(2 * 17 * 128 * 4)
    # fp32 storage with d_feat 256 and d 128 splits the value columns in two
    # halves of 64, each its own computation with its own segments: 64 rows
    # = 2 chunks of 32 -> 2 segments per half, aggregates of 256 x (64 + 16)
    wv = K.forward_workspace_bytes(1, 1, 64, 128, 256, "identity",
                                   dtype=__import__("torch").float32)
    assert wv == sync + a256(2 * 2 * 256 * 80 * 4) + a256(2 * 2 * 4)


@pytest.mark.parametrize("B,H,n", [(1, 1, 1), (1, 2, 17), (2, 3, 64),
                                   (4, 8, 999), (16, 40, 64), (1, 1, 5000)])
@pytest.mark.parametrize("d,m", [(32, 64), (64, 256), (128, 128)])
def test_unfused_performer_features_never_overlap_sync_area(B, H, n, d, m):
    # fp32 storage takes the unfused Performer path: q', k' go through the
    # workspace, and they always start after the synchronisation area
    # (which a workspace shared with segmented calls keeps zero), whether
    # or not this call has segments
    import torch
    need = K.forward_workspace_bytes(B, H, n, d, m, "performer",
                                     dtype=torch.float32)
    sync = 256 + 512 * 128
    feat = (B * H * n * m * 4 + 255) // 256 * 256
    assert need >= sync + 2 * feat


def test_featmap_rejects(lib):
    f = lib.la_featmap
    assert f(FAKE, FAKE, None, -1, 64, 0, 1, 1, 1, None) == B.LA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, None, 10, 64, 0, 9, 1, 1, None) == B.LA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, None, 10, 64, 0, 1, 3, 1, None) == B.LA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, None, 10, 48, 0, 1, 1, 1, None) == B.LA_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, None, 10, 64, 256, 2, 1, 1, None) == B.LA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, 10, 64, 250, 2, 1, 1, None) == B.LA_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, 10, 64, 512, 2, 1, 1, None) == B.LA_ERR_UNSUPPORTED
    assert f(None, FAKE, None, 10, 64, 0, 1, 1, 1, None) == B.LA_ERR_INVALID_ARG
    assert f(None, None, None, 0, 64, 0, 1, 1, 1, None) == B.LA_OK


def test_decode_rejects(lib):
    f = lib.la_decode_step
    P = FAKE
    assert f(P, P, P, P, P, P, -1, 1, 64, 64, 1, None, None, 1, None) == \
        B.LA_ERR_INVALID_ARG
    assert f(P, P, P, P, P, P, 1, 1, 64, 32, 1, None, None, 1, None) == \
        B.LA_ERR_INVALID_ARG
    assert f(P, P, P, P, P, P, 1, 1, 64, 64, 4, None, None, 1, None) == \
        B.LA_ERR_INVALID_ARG
    assert f(P, P, P, P, P, P, 1, 1, 48, 48, 1, None, None, 1, None) == \
        B.LA_ERR_UNSUPPORTED
    assert f(P, P, P, P, P, P, 1, 1, 64, 256, 2, None, None, 1, None) == \
        B.LA_ERR_INVALID_ARG
    assert f(None, P, P, P, P, P, 1, 1, 64, 64, 1, None, None, 1, None) == \
        B.LA_ERR_INVALID_ARG
    assert f(None, None, None, None, None, None, 0, 5, 64, 64, 1, None, None,
             1, None) == B.LA_OK


def test_forward_state_rejects(lib):
    f = lib.la_forward_state
    P = FAKE
    # the state outputs are required
    assert f(P, P, P, P, 1, 1, 64, 64, 64, 1, None, None, 1, 1, None, None, P,
             None) == B.LA_ERR_INVALID_ARG
    assert f(P, P, P, P, 1, 1, 64, 64, 64, 1, None, None, 1, 1, None, P, None,
             None) == B.LA_ERR_INVALID_ARG
    # the same validation as la_forward
    assert f(P, P, P, P, -1, 1, 64, 64, 64, 1, None, None, 1, 1, None, P, P,
             None) == B.LA_ERR_INVALID_ARG
    assert f(P, P, P, P, 1, 1, 64, 48, 48, 1, None, None, 1, 1, None, P, P,
             None) == B.LA_ERR_UNSUPPORTED
    # no units: nothing to do
    assert f(None, None, None, None, 0, 4, 64, 64, 64, 1, None, None, 1, 1,
             None, P, P, None) == B.LA_OK


def test_workspace_check_rejects_null(lib):
    assert lib.la_workspace_check(None, None) == B.LA_ERR_INVALID_ARG
    assert lib.la_last_error().decode() != ""


def test_last_error_is_cleared_on_success(lib):
    assert fwd(lib, B=-1) == B.LA_ERR_INVALID_ARG
    assert lib.la_last_error().decode() != ""
    assert fwd(lib, B=0) == B.LA_OK
    assert lib.la_last_error().decode() == ""


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 16)
    with pytest.raises(ValueError):
        K.forward(x, x, x)


# --------------------------------------------------------------------------
# Binding: shapes and dtypes are checked on the host before any pointer is
# taken (a mismatch would otherwise become an out-of-bounds device access)
# --------------------------------------------------------------------------

def _t(*shape, dtype=None):
    import torch
    return torch.zeros(*shape, dtype=dtype or torch.bfloat16)


@pytest.mark.parametrize("kw,exc", [
    (dict(out=_t(1, 2, 16, 32)), ValueError),                 # out too small
    (dict(out=_t(1, 2, 16, 64, dtype=__import__("torch").float32)), TypeError),
    (dict(decay=_t(3, dtype=__import__("torch").float32)), ValueError),  # != H
    (dict(decay=_t(2)), TypeError),                           # not fp32
    (dict(feature_map="performer"), ValueError),              # no omega
    (dict(feature_map="performer",
          omega=_t(32, 128, dtype=__import__("torch").float32)), ValueError),
    (dict(feature_map="performer", omega=_t(64, 128)), TypeError),
    (dict(mu_out=_t(1, 2, 64, 64, dtype=__import__("torch").float32)),
     ValueError),                                             # nu_out missing
    (dict(mu_out=_t(1, 2, 64, 32, dtype=__import__("torch").float32),
          nu_out=_t(1, 2, 64, dtype=__import__("torch").float32)), ValueError),
    (dict(workspace=_t(100, dtype=__import__("torch").float32)), TypeError),
])
def test_binding_forward_rejects_bad_shapes(kw, exc):
    q = _t(1, 2, 16, 64)
    with pytest.raises(exc):
        K.forward(q, q, q, **kw)


def test_binding_forward_rejects_mismatched_qkv():
    with pytest.raises(ValueError):
        K.forward(_t(1, 2, 16, 64), _t(1, 2, 16, 32), _t(1, 2, 16, 64))
    with pytest.raises(ValueError):      # elu1 keeps the width
        K.forward(_t(1, 2, 16, 32), _t(1, 2, 16, 32), _t(1, 2, 16, 64))
    with pytest.raises(TypeError):
        import torch
        K.forward(_t(1, 2, 16, 64), _t(1, 2, 16, 64),
                  _t(1, 2, 16, 64, dtype=torch.float32))


@pytest.mark.parametrize("kw,exc", [
    (dict(q=_t(2, 3, 32)), ValueError),                      # q width != d
    (dict(k=_t(2, 4, 64)), ValueError),                      # k heads
    (dict(out=_t(2, 3, 16)), ValueError),
    (dict(decay=_t(4, dtype=__import__("torch").float32)), ValueError),
    (dict(feature_map="performer",
          omega=_t(64, 32, dtype=__import__("torch").float32)), ValueError),
    (dict(feature_map="identity"), ValueError),              # q must be d_feat
    (dict(nu=_t(2, 3, 32, dtype=__import__("torch").float32)), ValueError),
])
def test_binding_decode_rejects_bad_shapes(kw, exc):
    import torch
    args = dict(mu=_t(2, 3, 64, 64, dtype=torch.float32),
                nu=_t(2, 3, 64, dtype=torch.float32), q=_t(2, 3, 64),
                k=_t(2, 3, 64), v=_t(2, 3, 64))
    if kw.get("feature_map") == "identity":
        args["mu"] = _t(2, 3, 16, 64, dtype=torch.float32)
        args["nu"] = _t(2, 3, 16, dtype=torch.float32)
    extra = {k: v for k, v in kw.items() if k not in args}
    args.update({k: v for k, v in kw.items() if k in args})
    with pytest.raises(exc):
        K.decode_step(args["mu"], args["nu"], args["q"], args["k"],
                      args["v"], **extra)


def test_binding_featmap_rejects_bad_shapes():
    import torch
    x = _t(10, 64)
    with pytest.raises(ValueError):
        K.featmap(x, "performer", omega=_t(32, 64, dtype=torch.float32))
    with pytest.raises(ValueError):
        K.featmap(x, "elu1", out=_t(10, 32))


def test_backward_workspace_bytes(lib):
    import torch
    a256 = lambda x: (x + 255) // 256 * 256
    # G~ rows of d + 2 values padded to a multiple of 32; elu + 1 adds the
    # features phi(k) and phi(q), identity uses k and q themselves
    rows = 2 * 3 * 100
    # bf16 at d = 128 runs the segmented roles, which map k, q themselves
    # (no K', Q' rows) and keep segment aggregates: 6 units, 100 rows = 2
    # chunks -> 2 segments, 2 roles (dq; dk, whose state dv shares) x 8
    # waves x 10 feature tiles x 256 floats each, then one float per segment
    assert K.backward_workspace_bytes(2, 3, 100, 128) == (
        a256(rows * 160 * 2) + a256(2 * 6 * 2 * (8 * 10 * 256 + 1) * 4))
    # one chunk: one segment, no aggregates
    assert K.backward_workspace_bytes(2, 3, 64, 128) == a256(384 * 160 * 2)
    assert K.backward_workspace_bytes(2, 3, 100, 128, dtype=torch.float32) == (
        a256(rows * 160 * 4) + 2 * a256(rows * 128 * 4))
    assert K.backward_workspace_bytes(2, 3, 100, 16, "identity") == a256(rows * 32 * 2)
    assert K.backward_workspace_bytes(2, 3, 100, 64, dtype=torch.float32) == (
        a256(rows * 96 * 4) + 2 * a256(rows * 64 * 4))
    # rejected or empty: 0
    assert K.backward_workspace_bytes(2, 3, 100, 48) == 0
    assert K.backward_workspace_bytes(2, 3, 0, 64) == 0
    # the Performer map: G~ rows, then K', Q' (bf16) and dq', dk' (fp32),
    # d_feat values each
    assert K.backward_workspace_bytes(2, 3, 100, 64, "performer",
                                      d_feat=256) == (
        a256(rows * 96 * 2) + 2 * a256(rows * 256 * 2) +
        2 * a256(rows * 256 * 4))
    assert K.backward_workspace_bytes(2, 3, 100, 64, "performer") == (
        a256(rows * 96 * 2) + 2 * a256(rows * 64 * 2) +
        2 * a256(rows * 64 * 4))
    # Performer sizes not built: d = 16, d * d_feat > 16384
    assert K.backward_workspace_bytes(2, 3, 100, 16, "performer") == 0
    assert K.backward_workspace_bytes(2, 3, 100, 128, "performer",
                                      d_feat=256) == 0


def test_backward_rejects_null_workspace(lib):
    # host-side validation: nothing is enqueued, no device memory is touched
    vp = ctypes.c_void_p(16)
    st = lib.la_backward(vp, vp, vp, vp, vp, vp, vp, vp, vp, 1, 1, 64, 64, 64,
                         B.MAP_ELU1, None, None, B.LA_BF16, None, None)
    assert st == B.LA_ERR_WORKSPACE
    assert "workspace" in lib.la_last_error().decode()


def test_backward_gated_workspace_bytes(lib):
    import torch
    a256 = lambda x: (x + 255) // 256 * 256
    rows = 2 * 3 * 100
    # a decay per position runs the same kernels as la_backward: bf16 at
    # d = 128 takes the segmented roles, whose aggregates are followed by
    # each segment's sum of log2 gamma (one float per role, unit, segment)
    assert K.backward_workspace_bytes(2, 3, 100, 128, gated=True) == (
        a256(rows * 160 * 2) + a256(2 * 6 * 2 * (8 * 10 * 256 + 1) * 4))
    assert K.backward_workspace_bytes(2, 3, 100, 128, gated=True) == (
        K.backward_workspace_bytes(2, 3, 100, 128))
    assert K.backward_workspace_bytes(2, 3, 100, 64, "identity",
                                      gated=True) == a256(rows * 96 * 2)
    assert K.backward_workspace_bytes(2, 3, 100, 32, dtype=torch.float32,
                                      gated=True) == (
        a256(rows * 64 * 4) + 2 * a256(rows * 32 * 4))
    # the Performer map: as la_backward's; not built: d != d_feat, other
    # d; empty sizes
    assert K.backward_workspace_bytes(2, 3, 100, 64, "performer",
                                      d_feat=256, gated=True) == (
        K.backward_workspace_bytes(2, 3, 100, 64, "performer", d_feat=256))
    assert K.backward_workspace_bytes(2, 3, 100, 16, "performer",
                                      gated=True) == 0
    assert K.backward_workspace_bytes(2, 3, 100, 48, gated=True) == 0
    assert K.backward_workspace_bytes(2, 3, 0, 64, gated=True) == 0


def test_gated_train_and_backward_reject(lib):
    # host-side validation only: nothing is enqueued
    vp = ctypes.c_void_p(16)
    bwd = lambda lay, mapk, lam, ws: lib.la_backward_gated(
        vp, vp, vp, vp, vp, vp, vp, vp, vp, 1, 1, 64, 64, 64, mapk, None,
        lam, lay, B.LA_BF16, ws, None)
    assert bwd(B.LD_CHANNEL, B.MAP_ELU1, vp, vp) == B.LA_ERR_UNSUPPORTED
    assert bwd(B.LD_BOTH, B.MAP_ELU1, vp, vp) == B.LA_ERR_UNSUPPORTED
    assert bwd(7, B.MAP_ELU1, vp, vp) == B.LA_ERR_INVALID_ARG
    # the Performer map needs omega
    assert bwd(B.LD_POSITION, B.MAP_PERFORMER, vp, vp) == B.LA_ERR_INVALID_ARG
    assert bwd(B.LD_POSITION, B.MAP_ELU1, None, vp) == B.LA_ERR_INVALID_ARG
    assert bwd(B.LD_POSITION, B.MAP_ELU1, vp, None) == B.LA_ERR_WORKSPACE
    fwd = lambda lay, den, lam: lib.la_forward_gated_train(
        vp, vp, vp, vp, den, 1, 1, 64, 64, 64, B.MAP_ELU1, None, lam, lay,
        B.LA_BF16, vp, None)
    assert fwd(B.LD_CHANNEL, vp, vp) == B.LA_ERR_UNSUPPORTED
    assert fwd(B.LD_POSITION, None, vp) == B.LA_ERR_INVALID_ARG
    assert fwd(B.LD_POSITION, vp, None) == B.LA_ERR_INVALID_ARG


def test_binding_rejects_decay_with_log_decay():
    import torch
    x = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    den = torch.ones(1, 1, 64)
    lam = torch.zeros(1, 1, 64)
    with pytest.raises(ValueError):
        K.backward(x, x, x, x, den, x, decay=torch.ones(1), log_decay=lam)
    with pytest.raises(ValueError):
        K.backward(x, x, x, x, den, x, log_decay=torch.zeros(1, 1, 63))
    with pytest.raises(TypeError):
        K.forward_train(x, x, x, log_decay=lam.double())


def test_binding_backward_rejects_small_workspace():
    import torch
    x = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    den = torch.ones(1, 1, 64)
    ws = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError):
        K.backward(x, x, x, x, den, x, workspace=ws)


def test_gated_workspace_bytes(lib):
    import torch
    a256 = lambda x: (x + 255) // 256 * 256
    sync = 256 + 512 * 128
    # the per-position layout shares la_forward's workspace
    assert K.gated_workspace_bytes(4, 8, 4096, 64, 64, layout="position") == \
        K.forward_workspace_bytes(4, 8, 4096, 64, 64)
    # a decay per row: 16-row chunks, about 512 workgroups in all and at
    # most 16 segments per unit; units * (nseg + 1) aggregate slots of
    # d' x d state floats + d' (nu) + d' (summed log2 decay), after the
    # synchronisation area of la_forward (never written by this path)
    for layout in ("channel", "both"):
        ws = K.gated_workspace_bytes(4, 8, 4096, 64, 64, layout=layout)
        nseg = 16                # 512 / 32 units, 256 chunks
        assert ws == sync + a256(32 * (nseg + 1) * (64 * 64 + 2 * 64) * 4)
    # d' below 32 is padded to 32 in the slot (its state rows 16..31 stay 0)
    ws = K.gated_workspace_bytes(1, 2, 100, 128, 16, "identity", "channel")
    nseg = 7                     # 7 chunks of 16 rows, 256 target per unit
    assert ws == sync + a256(2 * (nseg + 1) * (128 * 32 + 2 * 32) * 4)
    # causal over one segment: no aggregates, no workspace
    assert K.gated_workspace_bytes(1, 1, 16, 64, 64, layout="channel") == 0
    assert K.gated_workspace_bytes(600, 1, 4096, 64, 64, layout="channel") == 0
    # non-causal always takes the aggregate and carry launches
    assert K.gated_workspace_bytes(1, 1, 16, 64, 64, layout="channel",
                                   causal=False) == \
        sync + a256(2 * (64 * 64 + 2 * 64) * 4)
    # Performer: Q', K' (d' wide, storage type) after the aggregates
    wp = K.gated_workspace_bytes(1, 1, 16, 64, 256, "performer", "both")
    assert wp == sync + 2 * a256(16 * 256 * 2)
    wf = K.gated_workspace_bytes(1, 1, 16, 64, 256, "performer", "both",
                                 dtype=torch.float32)
    assert wf == sync + 2 * a256(16 * 256 * 4)
    # rejected arguments report 0
    assert K.gated_workspace_bytes(1, 1, 64, 48, 48, layout="channel") == 0
    assert K.gated_workspace_bytes(1, 1, 64, 64, 32, "elu1", "both") == 0
    assert lib.la_forward_gated_workspace_bytes(1, 1, 64, 64, 64, 1, 7, 1,
                                                1) == 0


def test_gated_rows_rejects(lib):
    f = lib.la_forward_gated
    lam = FAKE
    # ELU1 needs d_feat == d; unsupported sizes; bad causal; null pointers
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 32, 1, None, lam, 0, 1, 1,
             FAKE, None, None, None) == B.LA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 48, 48, 1, None, lam, 2, 1, 1,
             FAKE, None, None, None) == B.LA_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 64, 1, None, lam, 0, 2, 1,
             FAKE, None, None, None) == B.LA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 64, 1, None, None, 0, 1, 1,
             FAKE, None, None, None) == B.LA_ERR_INVALID_ARG
    assert f(None, FAKE, FAKE, FAKE, 1, 1, 64, 64, 64, 1, None, lam, 2, 1, 1,
             FAKE, None, None, None) == B.LA_ERR_INVALID_ARG
    # Performer without omega; missing workspace where one is needed
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 128, 2, None, lam, 0, 1, 1,
             FAKE, None, None, None) == B.LA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 64, 1, None, lam, 0, 0, 1,
             None, None, None, None) == B.LA_ERR_WORKSPACE
    # empty sizes are no-ops
    assert f(FAKE, FAKE, FAKE, FAKE, 0, 1, 64, 64, 64, 1, None, lam, 0, 1, 1,
             None, None, None, None) == B.LA_OK
