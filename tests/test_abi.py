"""CPU checks of the C ABI: the library loads, exports every symbol that
include/gla.h declares, and rejects bad arguments before touching a GPU.
No compute call is made here (these tests run without a GPU)."""
import ctypes
import math
import os
import re
import sys

import pytest

import gated_bidirectional_linear_amd as gla
from gated_bidirectional_linear_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_HIP, E_ALLOC, E_D, E_ALIAS, E_TOO_LARGE = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9


def declared_functions():
    names = set()
    for path in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names.update(re.findall(r"\b(gla_\w+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_and_binding_agree():
    assert declared_functions() == sorted(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_strings(lib):
    assert lib.gla_version() >> 16 == 1
    assert lib.gla_version() & 0xFFFF >= 6   # 1.1: gla_block_causal_forward_at; 1.2: fp8 e4m3 I/O; 1.3: token-causal;
    #                                          1.4: batches; 1.5: gla_forward_noalloc; 1.6: fp8 e5m2 I/O
    for st in (OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_HIP, E_ALLOC, E_D, E_ALIAS, E_TOO_LARGE):
        s = lib.gla_status_string(st).decode()
        assert s and s != "unknown status"
    assert lib.gla_status_string(-99).decode() == "unknown status"
    names = [lib.gla_kernel_name(i).decode() for i in range(4)]
    assert names == ["rope_table_kernel", "state_partial_kernel", "state_reduce_kernel", "output_kernel"]


# fake, never-dereferenced device addresses, 16-byte aligned and far apart
A = 1 << 40
P = [ctypes.c_void_p(A + i * (1 << 36)) for i in range(10)]


def fwd(lib, T=2, H=4, W=4, heads=2, d=32, eps=1e-6, dtype=1, ptrs=None):
    p = list(P if ptrs is None else ptrs)
    return lib.gla_forward(p[0], p[1], p[2], p[3], p[4], p[5], T, H, W, heads, d, eps, p[6], None, dtype)


def bc(lib, F=1, T=2, H=4, W=4, heads=2, d=32, eps=1e-6, dtype=1, ptrs=None):
    p = list(P if ptrs is None else ptrs)
    return lib.gla_block_causal_forward(p[0], p[1], p[2], p[3], p[4], p[5], T, H, W, heads, d, eps, p[6], None,
                                        p[7], p[8], F, dtype)


def bc_at(lib, F=1, t_offset=0, T=2, H=4, W=4, heads=2, d=32, eps=1e-6, dtype=1, ptrs=None):
    p = list(P if ptrs is None else ptrs)
    return lib.gla_block_causal_forward_at(p[0], p[1], p[2], p[3], p[4], p[5], T, H, W, heads, d, eps, p[6], None,
                                           p[7], p[8], F, t_offset, dtype)


def tc(lib, include_self=1, t_offset=0, T=2, H=4, W=4, heads=2, d=32, eps=1e-6, dtype=1, ptrs=None):
    p = list(P if ptrs is None else ptrs)
    return lib.gla_token_causal_forward(p[0], p[1], p[2], p[3], p[4], p[5], T, H, W, heads, d, eps, p[6], None,
                                        p[7], p[8], include_self, t_offset, dtype)


def test_token_causal_argument_errors(lib):
    assert tc(lib, include_self=2) == E_SHAPE
    assert tc(lib, include_self=-1) == E_SHAPE
    assert tc(lib, t_offset=-1) == E_SHAPE
    assert tc(lib, t_offset=2**31 - 2, T=5) == E_SHAPE
    assert tc(lib, include_self=2, dtype=7) == E_DTYPE     # dtype keeps its precedence
    assert tc(lib, d=48) == E_D
    assert tc(lib, heads=0) == E_SHAPE
    for i in (0, 6, 7, 8):
        p = list(P)
        p[i] = None
        assert tc(lib, ptrs=p) == E_NULL, i
    p = list(P)
    p[7] = p[6]          # state_S over out
    assert tc(lib, ptrs=p) == E_ALIAS
    nulls = [None] * 10
    assert tc(lib, T=0, ptrs=nulls) == OK                   # empty grid
    assert tc(lib, include_self=0, t_offset=7, T=0, ptrs=nulls) == OK


def test_frame_offset_errors(lib):
    assert bc_at(lib, F=2, t_offset=-2) == E_SHAPE
    assert bc_at(lib, F=3, t_offset=4) == E_SHAPE              # not a whole number of blocks
    assert bc_at(lib, F=1, t_offset=2**31 - 2, T=5) == E_SHAPE  # t_offset + T past INT32_MAX
    assert bc_at(lib, F=0, t_offset=0) == E_SHAPE
    assert bc_at(lib, F=2, t_offset=-2, dtype=7) == E_DTYPE    # dtype keeps its precedence
    nulls = [None] * 10
    assert bc_at(lib, F=3, t_offset=6, T=0, ptrs=nulls) == OK   # empty grid, valid offset
    assert bc_at(lib, F=3, t_offset=6, ptrs=[None] + P[1:]) == E_NULL


def test_dtype_and_head_dim_errors(lib):
    assert fwd(lib, dtype=4) == E_DTYPE          # 0 fp32, 1 bf16, 2 fp8 e4m3, 3 fp8 e5m2 are the known codes
    assert fwd(lib, dtype=-1) == E_DTYPE
    for dt in (0, 1, 2, 3):                       # known dtypes reach the later checks
        assert fwd(lib, dtype=dt, d=48) == E_D
        assert fwd(lib, dtype=dt, heads=0) == E_SHAPE
    for d in (0, 16, 48, 96, 256):
        assert fwd(lib, d=d) == E_D
        assert bc(lib, d=d) == E_D


def test_shape_errors(lib):
    assert fwd(lib, T=-1) == E_SHAPE
    assert fwd(lib, W=-3) == E_SHAPE
    assert fwd(lib, heads=0) == E_SHAPE
    for eps in (0.0, -1e-6, math.nan, math.inf, 1e-40):   # 1e-40 is subnormal
        assert fwd(lib, eps=eps) == E_SHAPE
    assert fwd(lib, T=2000, H=2000, W=2000) == E_SHAPE       # N >= 2^31
    assert fwd(lib, T=1000, H=1000, W=1000, heads=64, d=128) == E_SHAPE  # N*heads*d >= 2^40
    # token rows of 2^26 bytes or more (heads * d * element size): the 32-bit tile ranges would overflow
    assert fwd(lib, T=1, H=1, W=1, heads=1 << 17, d=128, dtype=0) == E_SHAPE
    assert fwd(lib, T=1, H=1, W=1, heads=1 << 18, d=128, dtype=1) == E_SHAPE
    assert fwd(lib, T=1, H=1, W=1, heads=(1 << 17) - 1, d=128, dtype=1, ptrs=[None] * 10) == E_NULL  # just below
    assert bc(lib, F=0) == E_SHAPE
    assert bc(lib, F=-2) == E_SHAPE


def test_null_errors(lib):
    for i in range(7):
        p = list(P)
        p[i] = None
        assert fwd(lib, ptrs=p) == E_NULL, i
    for i in (7, 8):
        p = list(P)
        p[i] = None
        assert bc(lib, ptrs=p) == E_NULL, i


def test_alignment_errors(lib):
    for i in range(7):
        p = list(P)
        p[i] = ctypes.c_void_p(A + i * (1 << 36) + 8)
        assert fwd(lib, ptrs=p) == E_ALIGN, i


def test_alias_errors(lib):
    for i in range(6):
        p = list(P)
        p[6] = p[i]
        assert fwd(lib, ptrs=p) == E_ALIAS, i
    p = list(P)
    p[7] = p[6]          # state_S over out
    assert bc(lib, ptrs=p) == E_ALIAS
    p = list(P)
    p[8] = ctypes.c_void_p(P[7].value + 16)  # state_z inside state_S
    assert bc(lib, ptrs=p) == E_ALIAS


def test_empty_grid_returns_ok_without_device_work(lib):
    nulls = [None] * 10
    assert fwd(lib, T=0, ptrs=nulls) == OK
    assert fwd(lib, T=3, H=0, ptrs=nulls) == OK
    assert bc(lib, F=2, T=0, ptrs=nulls) == OK


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(32, 2, 32)
    with pytest.raises(ValueError):
        gla.forward(q, q, q, torch.zeros(32, 2), q, torch.ones(32), (2, 4, 4))


def test_binding_checks_shapes_before_the_device():
    torch = pytest.importorskip("torch")
    q = torch.zeros(31, 2, 32)
    with pytest.raises(ValueError):
        gla.forward(q, q, q, torch.zeros(31, 2), q, torch.ones(32), (2, 4, 4))


def fb(lib, batch=2, T=2, H=4, W=4, heads=2, d=32, eps=1e-6, dtype=1, ptrs=None):
    p = list(P if ptrs is None else ptrs)
    return lib.gla_forward_batch(p[0], p[1], p[2], p[3], p[4], p[5], batch, T, H, W, heads, d, eps, p[6], None, dtype)


def bcb(lib, batch=2, F=1, t_offset=0, T=2, H=4, W=4, heads=2, d=32, eps=1e-6, dtype=1, ptrs=None):
    p = list(P if ptrs is None else ptrs)
    return lib.gla_block_causal_forward_batch(p[0], p[1], p[2], p[3], p[4], p[5], batch, T, H, W, heads, d, eps,
                                              p[6], None, p[7], p[8], F, t_offset, dtype)


def tcb(lib, batch=2, include_self=1, t_offset=0, T=2, H=4, W=4, heads=2, d=32, eps=1e-6, dtype=1, ptrs=None):
    p = list(P if ptrs is None else ptrs)
    return lib.gla_token_causal_forward_batch(p[0], p[1], p[2], p[3], p[4], p[5], batch, T, H, W, heads, d, eps,
                                              p[6], None, p[7], p[8], include_self, t_offset, dtype)


def test_batch_argument_errors(lib):
    for call in (fb, bcb, tcb):
        assert call(lib, batch=0) == E_SHAPE
        assert call(lib, batch=-3) == E_SHAPE
        assert call(lib, batch=0, dtype=7) == E_DTYPE                  # dtype keeps its precedence
        assert call(lib, batch=1 << 20, T=1 << 11, H=1, W=1) == E_SHAPE  # batch * T frames past 2^31
        assert call(lib, batch=1 << 10, T=1 << 10, H=32, W=32, heads=8, d=128) == E_SHAPE   # past 2^40 elements
        assert call(lib, batch=3, T=0, ptrs=[None] * 10) == OK           # empty grid
    assert bcb(lib, F=3, t_offset=4) == E_SHAPE
    assert tcb(lib, include_self=2) == E_SHAPE


def test_batch_extents_in_alias_checks(lib):
    """The tensors of all items count: a second item's rows or state overlap."""
    item_rows = 2 * 4 * 4 * 2 * 32 * 2           # one item's q bytes (bf16)
    p = list(P)
    p[6] = ctypes.c_void_p(A + item_rows)        # out right after item 0 of q
    assert fb(lib, batch=2, ptrs=p) == E_ALIAS
    item_state = 2 * 32 * 32 * 4                  # one item's state_S bytes
    p = list(P)
    p[8] = ctypes.c_void_p(A + 7 * (1 << 36) + item_state)   # state_z right after item 0 of state_S
    assert bcb(lib, batch=2, ptrs=p) == E_ALIAS
    assert tcb(lib, batch=2, ptrs=p) == E_ALIAS


def test_plan_override_argument_errors(lib):
    assert lib.gla_plan_override(-1, 1) == E_SHAPE
    assert lib.gla_plan_override(7, 1) == E_SHAPE        # past GLA_PLAN_NUM_KNOBS
    assert lib.gla_plan_override(0, -1) == E_SHAPE
    assert lib.gla_plan_override(0, (1 << 24) + 1) == E_SHAPE
    for knob in range(7):
        assert lib.gla_plan_override(knob, 0) == OK


def test_plan_knobs_match_the_header():
    text = open(os.path.join(ROOT, "include", "gla_internal.h")).read()
    knobs = dict((name.lower(), int(v)) for name, v in re.findall(r"GLA_PLAN_(\w+)\s*=\s*(\d+)", text))
    knobs.pop("num_knobs")
    assert knobs == gla.PLAN_KNOBS


def test_library_reads_no_environment():
    """The launch plan is not taken from the environment: no getenv in the
    library's sources."""
    csrc = os.path.join(ROOT, "gated_bidirectional_linear_amd", "csrc")
    for name in os.listdir(csrc):
        assert "getenv" not in open(os.path.join(csrc, name)).read(), name


_NO_DEVICE_SCRIPT = r"""
import ctypes, sys
sys.path.insert(0, {root!r})
from gated_bidirectional_linear_amd import _lib
lib = _lib.load()
hip = ctypes.CDLL("libamdhip64.so.7")
n = ctypes.c_int(0)
if hip.hipGetDeviceCount(ctypes.byref(n)) == 0 and n.value > 0:
    sys.exit(77)        # a device is visible: these fake pointers must not reach it
A = 1 << 40
p = [ctypes.c_void_p(A + i * (1 << 36)) for i in range(10)]
r = [lib.gla_forward(p[0], p[1], p[2], p[3], p[4], p[5], 2, 4, 4, 2, 32, 1e-6, p[6], None, 1),
     lib.gla_block_causal_forward(p[0], p[1], p[2], p[3], p[4], p[5], 2, 4, 4, 2, 32, 1e-6, p[6], None,
                                  p[7], p[8], 1, 1),
     lib.gla_token_causal_forward(p[0], p[1], p[2], p[3], p[4], p[5], 2, 4, 4, 2, 32, 1e-6, p[6], None,
                                  p[7], p[8], 1, 0, 1)]
print(r)
sys.exit(0 if r == [-5, -5, -5] else 1)
"""


def test_compute_call_without_a_device_returns_hip_error():
    """A valid call in a process that sees no GPU returns GLA_ERR_HIP (no
    crash, nothing enqueued).  Run in a child process, which exits early if a
    device is visible there."""
    import subprocess
    import sys
    res = subprocess.run([sys.executable, "-c", _NO_DEVICE_SCRIPT.format(root=ROOT)], capture_output=True,
                         text=True, timeout=120)
    if res.returncode == 77:
        pytest.skip("a GPU is visible: the no-device path cannot be exercised here")
    assert res.returncode == 0, res.stdout + res.stderr


def fna(lib, T=2, H=4, W=4, heads=2, d=32, eps=1e-6, dtype=1, ptrs=None):
    p = list(P if ptrs is None else ptrs)
    return lib.gla_forward_noalloc(p[0], p[1], p[2], p[3], p[4], p[5], T, H, W, heads, d, eps, p[6], None, dtype)


def test_noalloc_validation_and_size_limit(lib):
    """gla_forward_noalloc validates like gla_forward and rejects, before any
    device work, calls whose scratch exceeds its 64 MiB static buffer."""
    assert fna(lib, dtype=4) == E_DTYPE
    assert fna(lib, d=48) == E_D
    assert fna(lib, heads=0) == E_SHAPE
    assert fna(lib, ptrs=[None] + P[1:]) == E_NULL
    p = list(P)
    p[6] = p[0]
    assert fna(lib, ptrs=p) == E_ALIAS
    assert fna(lib, T=0, ptrs=[None] * 10) == OK
    # RoPE rows of 600,000 frames: 600,000 * 16 pairs * 8 bytes = 77 MB
    assert fna(lib, T=600_000, H=1, W=1, heads=1, d=128) == E_TOO_LARGE
    # 1,024 heads at d = 128: at least 2 * 1,024 states of 66 KB
    assert fna(lib, T=2, H=4, W=4, heads=1024, d=128) == E_TOO_LARGE


def _run(code):
    import subprocess
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)


def test_library_shares_torchs_hip_runtime():
    """Loaded before anything imports torch (as a first knob call does), the
    library still binds to PyTorch's HIP runtime: one runtime in the process."""
    r = _run("import gated_bidirectional_linear_amd as gla, gated_bidirectional_linear_amd._lib as L\n"
             "gla.plan_override('pass2_heads', 0)\n"
             "import torch\n"
             "print(len(L.hip_runtimes()))")
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().splitlines()[-1] == "1"


def test_second_hip_runtime_is_refused():
    """A process that already mapped another copy of the HIP runtime is
    refused with an error rather than left to mix two runtimes."""
    import glob
    import torch
    others = [p for p in glob.glob("/opt/rocm*/lib/libamdhip64.so*") if os.path.isfile(p)]
    if not others or os.path.dirname(torch.__file__) in others[0]:
        pytest.skip("no second HIP runtime on this machine")
    r = _run(f"import ctypes; ctypes.CDLL({others[0]!r})\n"
             "import gated_bidirectional_linear_amd._lib as L\n"
             "try:\n    L.load()\nexcept RuntimeError as e:\n    print('refused', e)\n")
    assert r.returncode == 0, r.stderr
    assert "refused" in r.stdout and "more than one HIP runtime" in r.stdout
