"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and rejects invalid arguments before any device work.

No call here reaches a kernel launch: each one fails host-side validation
first (bad problem, null or misaligned pointer, short workspace).  Device
pointers are never dereferenced on the host, so fake addresses are safe.
"""
import ctypes
import os
import re

import pytest

from lm_head_cross_amd import _lib
from lm_head_cross_amd.flce import make_problem

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for h in sorted(os.listdir(inc)):
        if not h.endswith(".h"):
            continue
        src = re.sub(r"/\*.*?\*/", "", open(os.path.join(inc, h)).read(), flags=re.S)
        names |= set(re.findall(r"\b((?:flce|chunked_ce)_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_abi():
    assert _declared_functions() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.flce_version() >= 100


def test_status_strings():
    lib = _lib.load()
    for code in range(5):
        s = lib.flce_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.flce_status_string(99).decode() == "unknown status"


def _ws(problem):
    lib = _lib.load()
    out = ctypes.c_size_t(0)
    code = lib.flce_workspace_size(ctypes.byref(problem), ctypes.byref(out))
    return code, out.value


def test_workspace_size_bounds():
    # Llama-3-8B head at 4096 tokens: no scratch buffer of logits shape may
    # exceed a quarter of a bf16 [T, Vu] array.
    p = make_problem(4096, 4096, 128256)
    code, ws = _ws(p)
    assert code == _lib.FLCE_OK
    full_logits = 4096 * 128256 * 2
    assert ws < full_logits  # whole workspace below one bf16 [T, V] buffer
    # padded vocabulary, softcap
    code, ws3 = _ws(make_problem(8192, 3072, 262144, 256000, softcap=30.0))
    assert code == _lib.FLCE_OK and ws3 < 8192 * 256000 * 2
    code, ws0 = _ws(make_problem(0, 128, 1000))
    assert code == _lib.FLCE_OK and ws0 == 0
    # sparse-label packed batch and long peaked head
    for T, H, V in ((16384, 5120, 152064), (65536, 8192, 128256)):
        code, w = _ws(make_problem(T, H, V, softcap=30.0))
        assert code == _lib.FLCE_OK and w < T * V * 2


def test_fp32_head_workspace():
    """An fp32 head is staged by default (the workspace holds a bf16 copy of
    the usable rows); rounded on load it needs no staged copy, only one
    backward chunk's rounded rows.  With H not a multiple of 128 the head is
    staged either way."""
    import torch
    a = _ws(make_problem(8192, 3072, 262144, 256000, softcap=30.0))
    b = _ws(make_problem(8192, 3072, 262144, 256000, softcap=30.0, weight_dtype=torch.float32))
    c = _ws(make_problem(8192, 3072, 262144, 256000, softcap=30.0, weight_dtype=torch.float32,
                         round_head_on_load=True))
    assert a[0] == b[0] == c[0] == _lib.FLCE_OK
    assert b[1] - a[1] == 256000 * 3072 * 2  # bf16 copy of the usable rows only
    assert a[1] < c[1] <= a[1] + 256000 * 3072 * 2 // 4  # at most a quarter of the usable rows
    d = _ws(make_problem(4096, 2880, 201088, 200000, weight_dtype=torch.float32))
    e = _ws(make_problem(4096, 2880, 201088, 200000, weight_dtype=torch.float32, round_head_on_load=True))
    assert d[0] == e[0] == _lib.FLCE_OK and d[1] == e[1]


def test_dw_tile_flags_leave_the_workspace_alone():
    """Fixing the dW tile changes the launch plan, not the workspace (sized
    for the widest chunk the planner may take); so does reusing the
    forward's staged head."""
    for shape in ((4096, 4096, 128256, 128256), (8192, 3072, 262144, 256000), (700, 400, 2000, 1900)):
        sizes = {_ws(make_problem(*shape, dw_tile=t, head_staged=h)) for t in (None, 256, 384) for h in (False, True)}
        assert len(sizes) == 1 and next(iter(sizes))[0] == _lib.FLCE_OK
    with pytest.raises(ValueError):
        make_problem(64, 512, 1000, dw_tile=128)


def test_unaligned_hidden_stages_a_padded_head():
    """H a multiple of 8 but not of 128: the head's usable rows are staged
    with rows of Hp = ceil(H/128)*128 elements; the fp32 accumulator of dH
    keeps rows of H.  Against the same problem at H = Hp (nothing staged):"""
    T, V, H, Hp = 4096, 201088, 2880, 2944
    a = _ws(make_problem(T, H, V))
    b = _ws(make_problem(T, Hp, V))
    assert a[0] == b[0] == _lib.FLCE_OK
    assert a[1] - b[1] == V * Hp * 2 - T * (Hp - H) * 4
    for h in (8, 136, 200, 1600):
        assert _ws(make_problem(64, h, 1000))[0] == _lib.FLCE_OK


def test_largest_accepted_sizes():
    for T, H, V in ((1 << 21, 4096, 128256), (4096, 4096, 1 << 23), (256, 1 << 20, 1024)):
        assert _ws(make_problem(T, H, V))[0] == _lib.FLCE_OK, (T, H, V)


def test_library_source_allocates_no_device_memory():
    """The caller owns every buffer: no allocation or free call in the HIP
    sources (the workspace comes in as an argument)."""
    csrc = os.path.join(ROOT, "lm_head_cross_amd", "csrc")
    banned = re.compile(r"\b(hipMalloc\w*|hipFree\w*|hipHostMalloc|hipExtMallocWithFlags|hipMemAlloc\w*|malloc|new\s+\w)")
    for name in sorted(os.listdir(csrc)):
        text = open(os.path.join(csrc, name)).read()
        code = re.sub(r"//[^\n]*|/\*.*?\*/", "", text, flags=re.S)
        assert not banned.search(code), (name, banned.search(code).group(0))


@pytest.mark.parametrize("kw,expect", [
    (dict(num_tokens=-1), _lib.FLCE_ERR_INVALID_ARG),
    (dict(hidden=0), _lib.FLCE_ERR_INVALID_ARG),
    (dict(vocab=0), _lib.FLCE_ERR_INVALID_ARG),
    (dict(unpadded_vocab=0), _lib.FLCE_ERR_INVALID_ARG),
    (dict(unpadded_vocab=1001), _lib.FLCE_ERR_INVALID_ARG),
    (dict(softcap=-1.0), _lib.FLCE_ERR_INVALID_ARG),
    (dict(softcap=float("nan")), _lib.FLCE_ERR_INVALID_ARG),
    (dict(softcap=float("inf")), _lib.FLCE_ERR_INVALID_ARG),
    (dict(reduction=2), _lib.FLCE_ERR_INVALID_ARG),
    (dict(num_label_tokens=0), _lib.FLCE_ERR_INVALID_ARG),
    (dict(hidden=100), _lib.FLCE_ERR_UNSUPPORTED),
    (dict(hidden=12), _lib.FLCE_ERR_UNSUPPORTED),
    (dict(hidden=4100), _lib.FLCE_ERR_UNSUPPORTED),
    (dict(weight_dtype=7), _lib.FLCE_ERR_UNSUPPORTED),
    (dict(flags=16), _lib.FLCE_ERR_INVALID_ARG),
    (dict(flags=1), _lib.FLCE_ERR_INVALID_ARG),  # rounding on load needs an fp32 head
    (dict(flags=6), _lib.FLCE_ERR_INVALID_ARG),  # both dW tiles
    (dict(flags=4), _lib.FLCE_ERR_INVALID_ARG),  # 384-row dW tiles need H >= 384
    # 32-bit tile offsets: beyond these sizes the call is refused
    (dict(num_tokens=(1 << 21) + 1), _lib.FLCE_ERR_UNSUPPORTED),
    (dict(vocab=(1 << 23) + 8, unpadded_vocab=1000), _lib.FLCE_ERR_UNSUPPORTED),
    (dict(hidden=(1 << 20) + 8), _lib.FLCE_ERR_UNSUPPORTED),
])
def test_invalid_problem_rejected(kw, expect):
    p = make_problem(64, 128, 1000)
    for k, v in kw.items():
        setattr(p, k, v)
    code, _ = _ws(p)
    assert code == expect
    lib = _lib.load()
    fake = ctypes.c_void_p(1 << 20)
    assert lib.flce_forward(ctypes.byref(p), fake, fake, fake, fake, fake, None, None, fake, 1 << 30,
                            None) == expect
    assert lib.flce_backward(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, None, fake,
                             1 << 30, None) == expect


def test_null_problem():
    lib = _lib.load()
    assert lib.flce_workspace_size(None, None) == _lib.FLCE_ERR_INVALID_ARG
    assert lib.flce_forward(None, None, None, None, None, None, None, None, None, 0, None) == \
        _lib.FLCE_ERR_INVALID_ARG


def test_pointer_and_workspace_checks():
    lib = _lib.load()
    p = make_problem(64, 128, 1000)
    code, need = _ws(p)
    assert code == 0 and need > 0
    a = 1 << 24  # fake, aligned device addresses
    P = ctypes.byref(p)
    V = ctypes.c_void_p
    # missing required pointers
    assert lib.flce_forward(P, V(a), None, V(a), V(a), V(a), None, None, V(a), need, None) == 1
    assert lib.flce_forward(P, V(a), V(a), V(a), None, V(a), None, None, V(a), need, None) == 1
    assert lib.flce_forward(P, V(a), V(a), V(a), V(a), None, None, None, V(a), need, None) == 1
    assert lib.flce_backward(P, V(a), V(a), V(a), V(a), None, V(a), V(a), None, V(a), need, None) == 1
    # misaligned operands
    assert lib.flce_forward(P, V(a + 2), V(a), V(a), V(a), V(a), None, None, V(a), need, None) == 2
    assert lib.flce_forward(P, V(a), V(a + 8), V(a), V(a), V(a), None, None, V(a), need, None) == 2
    # workspace: missing, misaligned, short
    assert lib.flce_forward(P, V(a), V(a), V(a), V(a), V(a), None, None, None, need, None) == 3
    assert lib.flce_forward(P, V(a), V(a), V(a), V(a), V(a), None, None, V(a + 64), need, None) == 3
    assert lib.flce_forward(P, V(a), V(a), V(a), V(a), V(a), None, None, V(a), need - 1, None) == 3
    assert lib.flce_backward(P, V(a), V(a), V(a), V(a), V(a), V(a), V(a), None, V(a), need - 1, None) == 3


def test_python_binding_argument_errors():
    with pytest.raises(ValueError):
        make_problem(4, 128, 10, reduction="none")
    with pytest.raises(ValueError):
        make_problem(4, 128, 10, num_label_tokens=-3)


# ---------------------------------------------------------------------------
# Cross-entropy over given logits (include/chunked_ce.h)
# ---------------------------------------------------------------------------


def _ce_ws(problem):
    out = ctypes.c_size_t(0)
    return _lib.load().chunked_ce_workspace_size(ctypes.byref(problem), ctypes.byref(out)), out.value


def test_chunked_ce_workspace_is_per_position():
    from lm_head_cross_amd.chunked_ce import make_ce_problem
    code, ws = _ce_ws(make_ce_problem(4096, 128256))
    assert code == _lib.FLCE_OK and 4096 * 4 <= ws < 4096 * 16
    code, ws = _ce_ws(make_ce_problem(0, 10))
    assert code == _lib.FLCE_OK and ws == 0


@pytest.mark.parametrize("kw,expect", [
    (dict(vocab=0), _lib.FLCE_ERR_INVALID_ARG),
    (dict(num_tokens=-1), _lib.FLCE_ERR_INVALID_ARG),
    (dict(chunk_len=0), _lib.FLCE_ERR_INVALID_ARG),
    (dict(reduction=7), _lib.FLCE_ERR_INVALID_ARG),
    (dict(num_label_tokens=0), _lib.FLCE_ERR_INVALID_ARG),
    (dict(logits_dtype=5), _lib.FLCE_ERR_UNSUPPORTED),
])
def test_chunked_ce_invalid_problem_rejected(kw, expect):
    from lm_head_cross_amd.chunked_ce import make_ce_problem
    p = make_ce_problem(8, 100)
    for k, v in kw.items():
        setattr(p, k, v)
    assert _ce_ws(p)[0] == expect
    lib = _lib.load()
    f = ctypes.c_void_p(1 << 20)
    assert lib.chunked_ce_forward(ctypes.byref(p), f, f, None, 0, f, f, None, None, f, 1 << 20, None) == expect
    assert lib.chunked_ce_backward(ctypes.byref(p), f, f, None, 0, f, f, f, None, f, 1 << 20, None) == expect


def test_chunked_ce_pointer_checks():
    from lm_head_cross_amd.chunked_ce import make_ce_problem
    lib = _lib.load()
    p = make_ce_problem(64, 1000)
    code, need = _ce_ws(p)
    P = ctypes.byref(p)
    V = ctypes.c_void_p
    a = 1 << 24
    # required pointers
    assert lib.chunked_ce_forward(P, None, V(a), None, 0, V(a), V(a), None, None, V(a), need, None) == 1
    assert lib.chunked_ce_forward(P, V(a), V(a), None, 0, None, V(a), None, None, V(a), need, None) == 1
    assert lib.chunked_ce_backward(P, V(a), V(a), None, 0, V(a), None, V(a), None, V(a), need, None) == 1
    # mask element size
    assert lib.chunked_ce_forward(P, V(a), V(a), V(a), 3, V(a), V(a), None, None, V(a), need, None) == 1
    # alignment: logits, labels, mask elements
    assert lib.chunked_ce_forward(P, V(a + 2), V(a), None, 0, V(a), V(a), None, None, V(a), need, None) == 2
    assert lib.chunked_ce_forward(P, V(a), V(a + 4), None, 0, V(a), V(a), None, None, V(a), need, None) == 2
    assert lib.chunked_ce_forward(P, V(a), V(a), V(a + 2), 4, V(a), V(a), None, None, V(a), need, None) == 2
    # workspace
    assert lib.chunked_ce_forward(P, V(a), V(a), None, 0, V(a), V(a), None, None, None, need, None) == 3
    assert lib.chunked_ce_forward(P, V(a), V(a), None, 0, V(a), V(a), None, None, V(a), need - 1, None) == 3
    # gradient may not overlap the logits
    assert lib.chunked_ce_backward(P, V(a), V(a), None, 0, V(a), V(a), V(a + 1024), None, V(a), need, None) == 1
    # in-place label rewrite
    assert lib.chunked_ce_mask_labels(V(a), None, 1, 8, -100, None) == 1
    assert lib.chunked_ce_mask_labels(V(a), V(a), 1, -1, -100, None) == 1
    assert lib.chunked_ce_mask_labels(V(a + 4), V(a), 1, 8, -100, None) == 2
    assert lib.chunked_ce_mask_labels(None, None, 1, 0, -100, None) == 0


def test_chunked_ce_module_arguments():
    import lm_head_cross_amd as L
    with pytest.raises(ValueError):
        L.ChunkedCrossEntropy(chunk_len=0)
    with pytest.raises(ValueError):
        L.ChunkedCrossEntropy(reduction="none")
    with pytest.raises(NotImplementedError):
        L.make_ce_problem(4, 10, dtype=__import__("torch").float16)


def test_backward_plan_of_the_head_workloads():
    """The backward's chunk width and dW tile as the planner picks them for 256
    compute units, as measured best on MI355X (chunk widths in 256-row tiles:
    96, 250, 144, 114; 384-row dW tiles wherever they measured faster)."""
    from lm_head_cross_amd import flce_backward_plan
    cases = {
        (4096, 4096, 128256, 128256): (96 * 256, 6, 256),
        (8192, 3072, 262144, 256000): (250 * 256, 4, 384),
        (16384, 5120, 152064, 152064): (144 * 256, 5, 384),
        (65536, 8192, 128256, 128256): (114 * 256, 5, 384),
    }
    for shape, want in cases.items():
        assert flce_backward_plan(make_problem(*shape), 256) == want, shape


def test_backward_plan_bounds_and_flags():
    """Every chunk is whole 256-row tiles, at most a quarter of the usable rows
    (or one tile), the chunks cover Vu, and the dW tile follows the flags."""
    from lm_head_cross_amd import flce_backward_plan
    for T, H, V, Vu in ((64, 128, 1000, 1000), (700, 400, 2000, 1900), (4096, 2880, 201088, 200000),
                        (1000, 512, 3000, 3000), (300, 128, 383, 300), (5, 8, 7, 1)):
        for cu in (64, 256, 304):
            rows, n, tile = flce_backward_plan(make_problem(T, H, V, Vu), cu)
            assert rows % 256 == 0 and rows <= max(256, Vu // 1024 * 256)
            assert n == -(-Vu // rows) and tile in (256, 384)
            assert flce_backward_plan(make_problem(T, H, V, Vu, dw_tile=256), cu)[2] == 256
            if H >= 384:
                assert flce_backward_plan(make_problem(T, H, V, Vu, dw_tile=384), cu)[2] == 384
    assert flce_backward_plan(make_problem(0, 128, 1000), 256)[1] == 0
    with pytest.raises(ValueError):
        flce_backward_plan(make_problem(64, 128, 1000, 1001), 256)
