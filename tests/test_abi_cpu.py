"""C ABI contract checks that need no GPU.

The library must load without a device, export every function declared in
include/sg.h, and reject bad arguments before touching HIP.  No compute call is
made here: every call below fails validation first.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sg.h")
LIB = os.path.join(ROOT, "post_pruning_amd", "libsg.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libsg.so not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sg_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def sg():
    import post_pruning_amd as sg
    sg.load_library()
    return sg


def test_header_declares_the_four_calls():
    names = _declared()
    for f in ("sg_hessian_accumulate", "sg_prepare_hinv", "sg_prune_layer",
              "sg_reconstruction_error"):
        assert f in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    for name in _declared():
        assert hasattr(lib, name), name


def test_version_and_status_strings(sg):
    assert sg.sg_abi_version() == 2
    assert sg.sg_status_string(0) == "SG_OK"
    assert sg.sg_status_string(3) == "SG_ERR_WORKSPACE"
    assert sg.sg_status_string(99) == "SG_ERR_UNKNOWN"


def test_workspace_sizes_pure_host(sg):
    # Factorisation: two padded n_pad^2 fp32 matrices (+ a small tail).
    assert sg.sg_workspace_bytes(sg.SG_OP_PREPARE_HINV, 0, 4096) >= 2 * 4096 * 4096 * 4
    assert sg.sg_workspace_bytes(sg.SG_OP_PREPARE_HINV, 0, 1000) >= 2 * 1024 * 1024 * 4
    # Prune: select state + an m x 128 fp32 error block.
    assert sg.sg_workspace_bytes(sg.SG_OP_PRUNE, 4096, 4096, 0, 128) >= 4096 * 128 * 4
    # Hessian: the small-n, many-token case splits the tokens: 96 tiles of
    # 256 x 384 cover the lower triangle (row panel I takes the column panels
    # up to its last row: 1, 2, 2, 3, 4, 4, ... for 16 row panels), in 8
    # equal splits (768 workgroups, three full rounds of 256 CUs); one fp32
    # partial tile per split and tile after a 256-byte aligned counter array.
    tiles = sum(min(4095, 256 * i + 255) // 384 + 1 for i in range(16))
    assert tiles == 96
    assert sg.sg_workspace_bytes(sg.SG_OP_HESSIAN, 0, 4096, 262144, 0) == 512 + tiles * 8 * 256 * 384 * 4
    # ... and the large-n case needs no split: only the lockstep counters,
    # 8 XCDs x ceil(ceil(4256 / 8) / 32) = 17 rounds of 32 workgroups.
    assert sg.sg_workspace_bytes(sg.SG_OP_HESSIAN, 0, 28672, 32768, 0) == 768
    assert sg.sg_workspace_bytes(sg.SG_OP_RECON, 64, 128, 512, 0) >= 8
    # invalid arguments give 0
    assert sg.sg_workspace_bytes(sg.SG_OP_PRUNE, 10, 10, 0, 0) == 0
    assert sg.sg_workspace_bytes(sg.SG_OP_PRUNE, 10, 10, 0, 129) == 0
    assert sg.sg_workspace_bytes(77, 1, 1, 1, 1) == 0


def _lib(sg):
    return sg.load_library()


def test_null_pointers_rejected_before_device(sg):
    lib = _lib(sg)
    st = lib.sg_hessian_accumulate(None, 16, None, sg.SG_BF16, 8, 16, None, 0, None)
    assert st == sg.SG_ERR_INVALID_ARGUMENT
    assert "NULL" in sg.sg_last_error_message()
    st = lib.sg_prepare_hinv(None, None, 16, 0.01, None, None, 0, None, None, None, None)
    assert st == sg.SG_ERR_INVALID_ARGUMENT
    st = lib.sg_prune_layer(None, None, None, 0, 4, 4, 4, None, 0, 0.5, 0, 1, 4, None, None, 0, None)
    assert st == sg.SG_ERR_INVALID_ARGUMENT
    st = lib.sg_reconstruction_error(None, 0, None, 0, 4, None, 4, 4, None, 0, 4, 4, None, 0, None)
    assert st == sg.SG_ERR_INVALID_ARGUMENT
    st = lib.sg_pack_two_four(None, 0, None, None, None, None, 4, 8, None)
    assert st == sg.SG_ERR_INVALID_ARGUMENT
    st = lib.sg_prune_quantize_layer(None, None, None, None, None, 4, None, 0, 4, 4, 4, None, 0, 0.5,
                                     0, 1, 4, None, None, 0, None)
    assert st == sg.SG_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("bits,code", [(1, 1), (9, 1), (4, 3)])
def test_prune_quantize_validation(sg, bits, code):
    # bits out of range, then (valid bits) a workspace that is too small
    st = _lib(sg).sg_prune_quantize_layer(ctypes.c_void_p(0x3000), None, None, FAKE, FAKE, bits, FAKE,
                                          0, 64, 128, 128, FAKE, 0, 0.5, 0, 1, 128, None,
                                          ctypes.c_void_p(0x10000), 0, None)
    assert st == code, sg.sg_last_error_message()


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case fails validation first


@pytest.mark.parametrize("args,code", [
    # n out of range, T < 1, ldx < n, unknown dtype, misaligned bf16 pointer
    (dict(n=0), 1), (dict(T=0), 1), (dict(ldx=8), 1), (dict(dt=7), 2),
    (dict(X=ctypes.c_void_p(0x1002)), 2), (dict(ldx=20), 2),
    # bf16 rows 2^28 elements apart or more
    (dict(ldx=1 << 28), 2),
])
def test_hessian_validation(sg, args, code):
    a = dict(H=FAKE, n=16, X=FAKE, dt=sg.SG_BF16, T=8, ldx=16)
    a.update(args)
    st = _lib(sg).sg_hessian_accumulate(a["H"], a["n"], a["X"], a["dt"], a["T"], a["ldx"], None, 0,
                                        None)
    assert st == code, sg.sg_last_error_message()


S1, S2, E1, E2 = (ctypes.c_void_p(a) for a in (0x5000, 0x6000, 0x7000, 0x8000))


@pytest.mark.parametrize("args,code", [
    (dict(damp=-0.1), 1), (dict(damp=float("nan")), 1), (dict(alias=True), 1),
    (dict(ws=0), 3),
    # the update stream and its two events go together, all distinct
    (dict(side=(S2, None, None)), 1), (dict(side=(S2, E1, None)), 1),
    (dict(side=(None, E1, E2)), 1), (dict(side=(S1, E1, E2)), 1), (dict(side=(S2, E1, E1)), 1),
])
def test_prepare_validation(sg, args, code):
    a = dict(damp=0.01, alias=False, ws=10 ** 9, side=(None, None, None))
    a.update(args)
    Hinv = FAKE if a["alias"] else ctypes.c_void_p(0x2000)
    st = _lib(sg).sg_prepare_hinv(Hinv, FAKE, 64, a["damp"], FAKE, ctypes.c_void_p(0x10000),
                                  a["ws"], S1, *a["side"])
    assert st == code, sg.sg_last_error_message()


def test_library_creates_no_stream_or_event():
    # Every stream and event the library enqueues on is the caller's.
    csrc = os.path.join(ROOT, "post_pruning_amd", "csrc")
    for f in os.listdir(csrc):
        text = open(os.path.join(csrc, f)).read()
        for call in ("hipStreamCreate", "hipEventCreate", "hipExtStreamCreate"):
            assert call not in text, (f, call)


@pytest.mark.parametrize("args,code", [
    (dict(kind=0, sp=1.5), 1),            # sparsity out of [0, 1]
    (dict(kind=2, sp=-0.1), 1),           # per-row sparsity out of [0, 1]
    (dict(kind=1, nk=3, mg=2), 1),        # N > M
    (dict(kind=1, nk=2, mg=3, n=96, bs=96), 2),  # M neither divides nor is a multiple of 16
    (dict(kind=1, nk=2, mg=4, n=130), 1),  # M does not divide n
    (dict(kind=1, nk=2, mg=8, bs=12), 1),  # M does not divide blocksize
    (dict(bs=0), 2), (dict(bs=129), 2),   # blocksize range
    (dict(kind=5), 1),                    # unknown kind
    (dict(ldw=10), 1),                    # ldw < n
    (dict(m=70000, n=70000), 2),          # m*n >= 2^32
    (dict(ws=0), 3),                      # workspace too small
    (dict(alias=True, dt=1), 1),          # aliasing a bf16 W
])
def test_prune_validation(sg, args, code):
    a = dict(kind=0, sp=0.5, nk=0, mg=1, bs=128, m=64, n=128, ldw=None, ws=10 ** 9, alias=False,
             dt=0)
    a.update(args)
    ldw = a["ldw"] if a["ldw"] is not None else a["n"]
    Wout = FAKE if a["alias"] else ctypes.c_void_p(0x3000)
    st = _lib(sg).sg_prune_layer(Wout, None, FAKE, a["dt"], a["m"], a["n"], ldw, FAKE, a["kind"],
                                 a["sp"], a["nk"], a["mg"], a["bs"], None, ctypes.c_void_p(0x10000),
                                 a["ws"], None)
    assert st == code, sg.sg_last_error_message()


def test_recon_validation(sg):
    lib = _lib(sg)
    st = lib.sg_reconstruction_error(FAKE, 0, FAKE, 0, 4, FAKE, 4, 8, FAKE, 0, 4, 8, None, 0, None)
    assert st == sg.SG_ERR_INVALID_ARGUMENT  # ldw < n
    st = lib.sg_reconstruction_error(FAKE, 0, FAKE, 0, 8, FAKE, 4, 8, FAKE, 0, 4, 8, None, 0, None)
    assert st == sg.SG_ERR_WORKSPACE


@pytest.mark.parametrize("m,n,dt,code", [
    (4, 10, 0, 1),   # n not a multiple of 4
    (0, 8, 0, 1),    # m < 1
    (4, 0, 0, 1),    # n < 4
    (4, 8, 7, 2),    # value dtype
])
def test_pack_validation(sg, m, n, dt, code):
    st = _lib(sg).sg_pack_two_four(FAKE, dt, FAKE, FAKE, FAKE, FAKE, m, n, None)
    assert st == code, sg.sg_last_error_message()


@pytest.mark.parametrize("splits,nseg", [
    (None, 2),            # no splits
    ([0, 64, 128], 0),    # nseg < 1
    ([0, 64, 128], 17),   # nseg > SG_MAX_SEGMENTS
    ([0, 64, 100], 2),    # does not end at m_total
    ([0, 80, 64, 128], 3),  # not increasing
    ([4, 64, 128], 2),    # does not start at 0
])
def test_shared_validation(sg, splits, nseg):
    arr = None
    if splits is not None:
        arr = ctypes.cast((ctypes.c_int64 * 18)(*(splits + [128] * (18 - len(splits)))), ctypes.c_void_p)
    st = _lib(sg).sg_prune_layers_shared(ctypes.c_void_p(0x3000), None, None, None, None, 0, FAKE, 0,
                                         128, 128, 128, arr, nseg, FAKE, 0, 0.5, 0, 1, 128, None,
                                         ctypes.c_void_p(0x10000), 10 ** 9, None)
    assert st == sg.SG_ERR_INVALID_ARGUMENT, sg.sg_last_error_message()


@pytest.mark.parametrize("vec,bs,kind,nk,mg,code", [
    (8, 128, 0, 0, 1, 2),     # vec not 1 or 16
    (16, 120, 0, 0, 1, 1),    # block size not a multiple of 16
    (16, 96, 1, 2, 3, 1),     # M neither divides 16 nor is a multiple of it (caught first here)
])
def test_vector_validation(sg, vec, bs, kind, nk, mg, code):
    st = _lib(sg).sg_prune_layer_vector(ctypes.c_void_p(0x3000), None, FAKE, 0, 64, 96, 96, FAKE, kind, 0.5,
                                        nk, mg, bs, vec, None, ctypes.c_void_p(0x10000), 10 ** 9, None)
    assert st == code, sg.sg_last_error_message()


def test_product_path_imports_no_oracle():
    # The library binding must not import, call or read the oracle.
    src_dir = os.path.join(ROOT, "post_pruning_amd")
    for dirpath, _, files in os.walk(src_dir):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f


def test_pattern_parsing(sg):
    assert sg.parse_pattern(0.5) == (sg.SG_UNSTRUCTURED, 0.5, 0, 1)
    assert sg.parse_pattern("2:4") == (sg.SG_NM, 0.0, 2, 4)
    assert sg.parse_pattern("16:64") == (sg.SG_NM, 0.0, 16, 64)
    assert sg.parse_pattern("16:128") == (sg.SG_NM, 0.0, 16, 128)
    assert sg.parse_pattern("0.5/row") == (sg.SG_UNSTRUCTURED_ROW, 0.5, 0, 1)


def test_noalloc_validation(sg):
    lib = _lib(sg)
    # null pointers and sizes are rejected first
    st = lib.sg_prune_layer_noalloc(None, None, None, 0, 4, 4, 4, None, 0, 0.5, 0, 1, 4, None, None)
    assert st == sg.SG_ERR_INVALID_ARGUMENT
    # a layer whose workspace exceeds the scratch array: rejected before the device is touched
    need = sg.sg_workspace_bytes(sg.SG_OP_PRUNE, 30000, 256, 0, 128)
    assert need > sg.SG_NOALLOC_SCRATCH_BYTES
    st = lib.sg_prune_layer_noalloc(ctypes.c_void_p(0x3000), None, FAKE, 0, 30000, 256, 256, FAKE, 0, 0.5,
                                    0, 1, 128, None, None)
    assert st == sg.SG_ERR_UNSUPPORTED and "scratch" in sg.sg_last_error_message()
    # the largest m the array serves at blocksize 128
    assert sg.sg_workspace_bytes(sg.SG_OP_PRUNE, 21600, 28672, 0, 128) <= sg.SG_NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("splits,nseg,hinv", [
    (None, 2, True),            # no splits
    ([0, 64, 128], 2, False),   # no factor array
    ([0, 64, 128], 0, True),    # nseg < 1
    ([0, 64, 100], 2, True),    # does not end at m_total
    ([0, 80, 64, 128], 3, True),  # not increasing
])
def test_batched_validation(sg, splits, nseg, hinv):
    arr = None
    if splits is not None:
        arr = ctypes.cast((ctypes.c_int64 * 18)(*(splits + [128] * (18 - len(splits)))), ctypes.c_void_p)
    hv = ctypes.cast((ctypes.c_void_p * 16)(*([0x1000] * 16)), ctypes.c_void_p) if hinv else None
    st = _lib(sg).sg_prune_layers_batched(ctypes.c_void_p(0x3000), None, None, None, None, 0, FAKE, 0,
                                          128, 128, 128, arr, nseg, hv, 0, 0.5, 0, 1, 128, None,
                                          ctypes.c_void_p(0x10000), 10 ** 9, None)
    assert st == sg.SG_ERR_INVALID_ARGUMENT, sg.sg_last_error_message()


def test_batched_null_factor_rejected(sg):
    arr = ctypes.cast((ctypes.c_int64 * 3)(0, 64, 128), ctypes.c_void_p)
    hv = ctypes.cast((ctypes.c_void_p * 2)(0x1000, None), ctypes.c_void_p)
    st = _lib(sg).sg_prune_layers_batched(ctypes.c_void_p(0x3000), None, None, None, None, 0, FAKE, 0,
                                          128, 128, 128, arr, 2, hv, 0, 0.5, 0, 1, 128, None,
                                          ctypes.c_void_p(0x10000), 10 ** 9, None)
    assert st == sg.SG_ERR_INVALID_ARGUMENT and "Hinv[1]" in sg.sg_last_error_message()


def _ptr_array(vals):
    return ctypes.cast((ctypes.c_void_p * len(vals))(*vals), ctypes.c_void_p)


@pytest.mark.parametrize("case", ["nl0", "nl17", "null_entry", "alias_h", "same_out", "small_ws", "events"])
def test_prepare_hinv_batched_validation(sg, case):
    """sg_prepare_hinv_batched rejects bad arguments before anything is enqueued."""
    n = 256
    per = sg.sg_workspace_bytes(sg.SG_OP_PREPARE_HINV, 0, n)
    nl = 2
    hin = [0x10000, 0x20000]
    out = [0x30000, 0x40000]
    ws_bytes = nl * per
    upd = ev = None
    expect = sg.SG_ERR_INVALID_ARGUMENT
    if case == "nl0":
        nl = 0
    elif case == "nl17":
        nl = 17
        hin, out = [0x10000 + i for i in range(17)], [0x90000 + i for i in range(17)]
    elif case == "null_entry":
        hin = [0x10000, None]
    elif case == "alias_h":
        out = [0x30000, 0x10000]
    elif case == "same_out":
        out = [0x30000, 0x30000]
    elif case == "small_ws":
        ws_bytes = nl * per - 1
        expect = sg.SG_ERR_WORKSPACE
    elif case == "events":
        upd = ctypes.c_void_p(0x5000)  # a stream without the two events
    st = _lib(sg).sg_prepare_hinv_batched(_ptr_array(out), _ptr_array(hin), nl, n, 0.01,
                                          ctypes.c_void_p(0x6000), ctypes.c_void_p(0x100000), ws_bytes,
                                          None, upd, ev, ev)
    assert st == expect, (case, sg.sg_last_error_message())
