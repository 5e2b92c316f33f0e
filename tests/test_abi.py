"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host with the documented
status before anything is enqueued.  Only invalid calls are made here (fake,
never-dereferenced addresses), so no kernel is launched."""
import ctypes
import os
import subprocess

import pytest

from mxfp4_expert_weight_amd import binding as B


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from mxfp4_expert_weight_amd import build
        build.build(verbose=False)
    return B.lib()


def test_exports_every_declared_function(lib):
    names = B.header_functions()
    assert set(names) >= {"moe_route", "moe_sort_by_expert", "moe_mxfp4_forward",
                          "moe_mxfp4_dequantize", "moe_topk_softmax", "moe_workspace_bytes",
                          "moe_status_string"}
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_status_strings(lib):
    for st in range(6):
        assert B.status_string(st)
    assert B.status_string(0) == "ok"


def test_workspace_bytes(lib):
    ws = B.moe_workspace_bytes(1, 8, 512, 2560, 768)
    assert ws >= 256 + (8 + 1) * 768 * 2 and ws % 256 == 0
    assert B.moe_workspace_bytes(512, 8, 512, 2560, 768) > ws
    assert B.moe_workspace_bytes(1, 8, 512, 2561, 768) == 0        # H % 32
    assert B.moe_workspace_bytes(1, 9, 8, 256, 128) == 0           # k > E
    assert B.moe_workspace_bytes(0, 8, 512, 2560, 768) == 0        # M < 1
    assert B.moe_workspace_bytes(1, 8, 2048, 2560, 768) == 0       # E > limit


A = 0x100000        # 16-byte-aligned fake addresses: only reached on invalid calls
MIS = 0x100008      # 8-byte aligned, not 16


def _status(fn, *args):
    with pytest.raises(B.MoeError) as ei:
        fn(*args)
    return ei.value.status


def test_route_host_checks(lib):
    r = B.moe_route
    assert _status(r, None, A, None, 0, 1, 2560, 512, 8, A, A, A, 0) == B.MOE_ERR_NULL
    assert _status(r, A, A, None, 0, 0, 2560, 512, 8, A, A, A, 0) == B.MOE_ERR_SHAPE
    assert _status(r, A, A, None, 0, 1, 2559, 512, 8, A, A, A, 0) == B.MOE_ERR_SHAPE
    assert _status(r, A, A, None, 0, 1, 2560, 512, 0, A, A, A, 0) == B.MOE_ERR_SHAPE
    assert _status(r, A, A, None, 0, 1, 2560, 4, 8, A, A, A, 0) == B.MOE_ERR_SHAPE
    assert _status(r, A, A, None, 0, 1, 2560, 512, 33, A, A, A, 0) == B.MOE_ERR_SHAPE
    assert _status(r, A, A, A, 7, 1, 2560, 512, 8, A, A, A, 0) == B.MOE_ERR_SHAPE   # bias stride
    assert _status(r, MIS, A, None, 0, 1, 2560, 512, 8, A, A, A, 0) == B.MOE_ERR_ALIGN
    assert _status(r, A, MIS, None, 0, 1, 2560, 512, 8, A, A, A, 0) == B.MOE_ERR_ALIGN


def test_topk_and_sort_host_checks(lib):
    assert _status(B.moe_topk_softmax, None, 1, 512, 8, A, A, 0) == B.MOE_ERR_NULL
    assert _status(B.moe_topk_softmax, A, 1, 1025, 8, A, A, 0) == B.MOE_ERR_SHAPE
    assert _status(B.moe_topk_softmax, A, 70000, 512, 8, A, A, 0) == B.MOE_ERR_SHAPE
    assert _status(B.moe_sort_by_expert, A, 1, 8, 512, A, A, A, None, 0) == B.MOE_ERR_NULL
    assert _status(B.moe_sort_by_expert, A, 1, 0, 512, A, A, A, A, 0) == B.MOE_ERR_SHAPE


def test_forward_host_checks(lib):
    w = B.make_weights(A, A, A, A, 512, 2560, 768, 1)
    ws = B.moe_workspace_bytes(4, 8, 512, 2560, 768)
    f = B.moe_mxfp4_forward
    args = [A, w, 4, 8, A, A, A, A, A, A, A, ws, 0]
    assert _status(f, *([None] + args[1:])) == B.MOE_ERR_NULL
    assert _status(f, *(args[:1] + [None] + args[2:])) == B.MOE_ERR_NULL
    bad = B.make_weights(A, None, A, A, 512, 2560, 768, 1)
    assert _status(f, *(args[:1] + [bad] + args[2:])) == B.MOE_ERR_NULL
    for shape in [(512, 2560, 700, 1), (512, 2560, 768, 2), (512, 0, 768, 1), (0, 2560, 768, 1)]:
        bw = B.make_weights(A, A, A, A, *shape)
        assert _status(f, *(args[:1] + [bw] + args[2:])) == B.MOE_ERR_SHAPE, shape
    mis = B.make_weights(A, A, MIS, A, 512, 2560, 768, 1)
    assert _status(f, *(args[:1] + [mis] + args[2:])) == B.MOE_ERR_ALIGN
    assert _status(f, *(args[:10] + [A + 16, ws, 0])) == B.MOE_ERR_ALIGN      # workspace 256-aligned
    assert _status(f, *(args[:11] + [ws - 1, 0])) == B.MOE_ERR_WORKSPACE


@pytest.mark.parametrize("name", ["moe_layer", "moe_layer_w4a8", "moe_layer_ex"])
def test_layer_host_checks(lib, name):
    w = B.make_weights(A, A, A, A, 512, 2560, 768, 1)
    ws = B.moe_workspace_bytes(1, 8, 512, 2560, 768)
    f = getattr(B, name)
    if name == "moe_layer_ex":
        ex = f
        f = lambda *a: ex(*a[:-1], None, a[-1])      # noqa: E731  (NULL options)
    args = [A, A, None, 0, w, 1, 8, A, A, A, A, A, A, A, A, A, ws, 0]
    assert _status(f, *([None] + args[1:])) == B.MOE_ERR_NULL
    assert _status(f, *(args[:4] + [None] + args[5:])) == B.MOE_ERR_NULL
    assert _status(f, *(args[:5] + [0] + args[6:])) == B.MOE_ERR_SHAPE
    assert _status(f, *(args[:2] + [A, 3] + args[4:])) == B.MOE_ERR_SHAPE         # bias stride
    assert _status(f, *(args[:1] + [MIS] + args[2:])) == B.MOE_ERR_ALIGN
    assert _status(f, *(args[:16] + [ws - 1, 0])) == B.MOE_ERR_WORKSPACE


def test_noalloc_layer_host_checks(lib):
    """moe_layer_noalloc: the moe_layer checks, then the layer's workspace must
    fit the library's static array (8 MiB: the Ling layer up to M = 57), else
    MOE_ERR_WORKSPACE -- all before the device is touched."""
    assert B.NOALLOC_WORKSPACE_BYTES == 8 << 20
    w = B.make_weights(A, A, A, A, 512, 2560, 768, 1)
    f = B.moe_layer_noalloc
    args = [A, A, None, 0, w, 1, 8, A, A, A, A, A, A, A, A, 0]
    assert _status(f, *([None] + args[1:])) == B.MOE_ERR_NULL
    assert _status(f, *(args[:4] + [None] + args[5:])) == B.MOE_ERR_NULL
    assert _status(f, *(args[:14] + [None, 0])) == B.MOE_ERR_NULL                 # y
    assert _status(f, *(args[:5] + [0] + args[6:])) == B.MOE_ERR_SHAPE
    assert _status(f, *(args[:2] + [A, 3] + args[4:])) == B.MOE_ERR_SHAPE         # bias stride
    assert _status(f, *(args[:1] + [MIS] + args[2:])) == B.MOE_ERR_ALIGN
    bad = B.make_weights(A, A, A, A, 512, 2560, 700, 1)
    assert _status(f, *(args[:4] + [bad] + args[5:])) == B.MOE_ERR_SHAPE
    assert B.moe_workspace_bytes(57, 8, 512, 2560, 768) <= B.NOALLOC_WORKSPACE_BYTES
    assert B.moe_workspace_bytes(58, 8, 512, 2560, 768) > B.NOALLOC_WORKSPACE_BYTES
    assert _status(f, *(args[:5] + [58] + args[6:])) == B.MOE_ERR_WORKSPACE
    assert _status(f, *(args[:5] + [512] + args[6:])) == B.MOE_ERR_WORKSPACE


def test_read_probe_host_checks(lib):
    """moe_read_probe: pointers, sizes and alignment checked on the host."""
    f = B.moe_read_probe
    n, mb = 3, 2088960
    words = B.read_probe_words(n, mb)
    assert words == 3 * 128
    assert _status(f, None, A, n, mb, A, words) == B.MOE_ERR_NULL
    assert _status(f, A, A, n, mb, None, words) == B.MOE_ERR_NULL
    assert _status(f, A, A, n, mb, A, words, A, None) == B.MOE_ERR_NULL        # one event of two
    assert _status(f, A, A, 0, mb, A, words) == B.MOE_ERR_SHAPE
    assert _status(f, A, A, n, 8, A, words) == B.MOE_ERR_SHAPE
    assert _status(f, A, A, n, mb + 4, A, words) == B.MOE_ERR_SHAPE            # not a multiple of 16
    assert _status(f, A, A, n, mb, A, words - 1) == B.MOE_ERR_SHAPE
    assert _status(f, A + 4, A, n, mb, A, words) == B.MOE_ERR_ALIGN


def test_exec_opts_host_checks(lib):
    """moe_exec_opts: act8 in {0, 1}; helper streams come as a pair, with all
    four events (checked before anything is enqueued)."""
    w = B.make_weights(A, A, A, A, 512, 2560, 768, 1)
    ws = B.moe_workspace_bytes(24, 8, 512, 2560, 768)
    args = [A, A, None, 0, w, 24, 8, A, A, A, A, A, A, A, A, A, ws]
    fwd = [A, w, 24, 8, A, A, A, A, A, A, A, ws]
    cases = [(B.make_opts(act8=2), B.MOE_ERR_SHAPE),
             (B.make_opts(helper_streams=[A, None], helper_events=[A, A, A, A]), B.MOE_ERR_NULL),
             (B.make_opts(helper_streams=[None, A], helper_events=[A, A, A, A]), B.MOE_ERR_NULL),
             (B.make_opts(helper_streams=[A, A]), B.MOE_ERR_NULL),
             (B.make_opts(helper_streams=[A, A], helper_events=[A, A, None, A]), B.MOE_ERR_NULL)]
    for o, st in cases:
        assert _status(B.moe_layer_ex, *args, o, 0) == st
        assert _status(B.moe_mxfp4_forward_ex, *fwd, o, 0) == st
    # a valid options struct still meets the other checks first
    assert _status(B.moe_layer_ex, *args[:5], 0, *args[6:], B.make_opts(act8=1), 0) == B.MOE_ERR_SHAPE
    with pytest.raises(ValueError):
        B.make_opts(helper_events=[A])


def test_dequant_host_checks(lib):
    d = B.moe_mxfp4_dequantize
    assert _status(d, None, A, 4, 64, A, 0) == B.MOE_ERR_NULL
    assert _status(d, A, A, 4, 48, A, 0) == B.MOE_ERR_SHAPE
    assert _status(d, A, A, 0, 64, A, 0) == B.MOE_ERR_SHAPE
    assert _status(d, MIS, A, 4, 64, A, 0) == B.MOE_ERR_ALIGN


def test_library_has_no_oracle_or_fallback():
    """The product path never routes through the oracle or a CPU fallback."""
    pkg = os.path.dirname(B.__file__)
    for root, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(root, fn)).read()
                assert "import oracle" not in src and "from oracle" not in src, fn


def test_lmhead_host_checks(lib):
    q, p = B.moe_lmhead_fp8_quantize, B.moe_lmhead_fp8_logits
    assert _status(q, None, 10, 2560, A, A, 0) == B.MOE_ERR_NULL
    assert _status(q, A, 0, 2560, A, A, 0) == B.MOE_ERR_SHAPE
    assert _status(q, A, 10, 2550, A, A, 0) == B.MOE_ERR_SHAPE          # H % 32
    assert _status(q, A, 10, 16384, A, A, 0) == B.MOE_ERR_SHAPE         # H > limit
    assert _status(q, MIS, 10, 2560, A, A, 0) == B.MOE_ERR_ALIGN
    assert _status(p, A, A, None, 1, 10, 2560, A, 0) == B.MOE_ERR_NULL
    assert _status(p, A, A, A, 9, 10, 2560, A, 0) == B.MOE_ERR_SHAPE     # M > 8
    assert _status(p, A, A, A, 5, 10, 8192, A, 0) == B.MOE_ERR_SHAPE     # M * H > 32768
    assert _status(p, A, A, A, 1, 0, 2560, A, 0) == B.MOE_ERR_SHAPE
    assert _status(p, A, MIS, A, 1, 10, 2560, A, 0) == B.MOE_ERR_ALIGN


def test_mxfp8_quantize_host_checks(lib):
    f = B.moe_mxfp8_quantize
    assert _status(f, None, 4, 64, A, A, A, 0) == B.MOE_ERR_NULL
    assert _status(f, A, 4, 64, None, None, None, 0) == B.MOE_ERR_NULL        # no output at all
    assert _status(f, A, 0, 64, A, A, A, 0) == B.MOE_ERR_SHAPE
    assert _status(f, A, 4, 48, A, A, A, 0) == B.MOE_ERR_SHAPE                # K % 32
    assert _status(f, A, 4, 0, A, A, A, 0) == B.MOE_ERR_SHAPE
    assert _status(f, MIS, 4, 64, A, A, A, 0) == B.MOE_ERR_ALIGN
    assert _status(f, A, 4, 64, MIS, A, A, 0) == B.MOE_ERR_ALIGN


def test_prefetch_host_checks(lib):
    s = B.moe_prefetch_select
    assert _status(s, None, 4, 512, 1, 9, A, A, 0) == B.MOE_ERR_NULL           # ids with n_ids > 0
    assert _status(s, A, 4, 512, 1, 9, None, A, 0) == B.MOE_ERR_NULL
    assert _status(s, A, 4, 512, 1, 9, A, None, 0) == B.MOE_ERR_NULL
    assert _status(s, A, 1 << 20, 512, 1, 9, A, A, 0) == B.MOE_ERR_SHAPE      # n_ids > limit
    assert _status(s, A, 4, 1025, 1, 9, A, A, 0) == B.MOE_ERR_SHAPE
    assert _status(s, A, 4, 512, 2, 9, A, A, 0) == B.MOE_ERR_SHAPE
    assert _status(s, A, 4, 512, 1, 65536, A, A, 0) == B.MOE_ERR_SHAPE        # list > limit
    assert _status(s, A, 4, 512, 1, -1, A, A, 0) == B.MOE_ERR_SHAPE
    assert _status(s, A + 2, 4, 512, 1, 9, A, A, 0) == B.MOE_ERR_ALIGN
    p = B.moe_prefetch_experts
    w = B.make_weights(A, A, A, A, 512, 2560, 768, 1)
    assert _status(p, None, A, A, 9, 3, A, 0) == B.MOE_ERR_NULL
    assert _status(p, B.make_weights(A, A, None, A, 512, 2560, 768, 1), A, A, 9, 3, A, 0) == B.MOE_ERR_NULL
    assert _status(p, w, None, A, 9, 3, A, 0) == B.MOE_ERR_NULL
    assert _status(p, w, A, A, 9, 3, None, 0) == B.MOE_ERR_NULL
    assert _status(p, w, A, A, 9, 0, A, 0) == B.MOE_ERR_SHAPE                # parts
    assert _status(p, w, A, A, 9, 4, A, 0) == B.MOE_ERR_SHAPE
    assert _status(p, w, A, A, 65536, 3, A, 0) == B.MOE_ERR_SHAPE            # list > limit
    assert _status(p, w, A, A, -1, 3, A, 0) == B.MOE_ERR_SHAPE
    assert _status(p, B.make_weights(A, A, A, A, 512, 2560, 770, 1), A, A, 9, 3, A, 0) == B.MOE_ERR_SHAPE
    assert _status(p, B.make_weights(A, A, A, A, 512, 2560, 768, 3), A, A, 9, 3, A, 0) == B.MOE_ERR_SHAPE
    assert _status(p, B.make_weights(A, MIS, A, A, 512, 2560, 768, 1), A, A, 9, 3, A, 0) == B.MOE_ERR_ALIGN
    assert _status(p, w, A + 2, A, 9, 3, A, 0) == B.MOE_ERR_ALIGN


def test_hinted_layer_host_checks(lib):
    w = B.make_weights(A, A, A, A, 512, 2560, 768, 1)
    ws = B.moe_workspace_bytes(1, 8, 512, 2560, 768)
    f = B.moe_layer_hinted
    args = [A, A, None, 0, w, 1, 8, A, A, A, A, A, A, A, A, A, ws]
    assert _status(f, *(args + [A, None])) == B.MOE_ERR_NULL          # hint without its count
    assert _status(f, *(args + [None, A])) == B.MOE_ERR_NULL
    assert _status(f, *(args + [A + 2, A])) == B.MOE_ERR_ALIGN
    assert _status(f, *([None] + args[1:] + [A, A])) == B.MOE_ERR_NULL
    assert _status(f, *(args[:5] + [0] + args[6:] + [A, A])) == B.MOE_ERR_SHAPE
