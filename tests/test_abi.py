"""The C-ABI library without a GPU: it loads, exports what the header
declares, and rejects bad arguments on the host before touching a device."""
import ctypes
import math
import os
import re

import pytest

from mla_tree_verify_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_verify.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_verify\w*)\s*\(", text)))


def test_library_exports_every_declared_function(lib):
    declared = header_functions()
    assert set(declared) == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), f"{name} not exported"


def test_strerror(lib):
    assert _lib.strerror(0) == "ok"
    for code in range(1, 10):
        assert _lib.strerror(code) != "unknown status"
    assert _lib.strerror(99) == "unknown status"


def test_check_tree(lib):
    assert _lib.check_tree([-1, 0, 0, 1, -1]) == _lib.MLAV_OK
    assert _lib.check_tree([-1, 0, 2]) == _lib.MLAV_ERR_TREE
    assert _lib.check_tree([0]) == _lib.MLAV_ERR_TREE
    assert _lib.check_tree([-2]) == _lib.MLAV_ERR_TREE
    arr = (ctypes.c_int32 * 1)(-1)
    assert lib.mla_verify_check_tree(None, 1) == _lib.MLAV_ERR_NULL
    assert lib.mla_verify_check_tree(arr, 0) == _lib.MLAV_ERR_SHAPE
    assert lib.mla_verify_check_tree(arr, 65) == _lib.MLAV_ERR_SHAPE


@pytest.mark.parametrize("q,p,cus", [(9, 256, 256), (9, 4096, 256), (9, 16384, 256), (33, 16384, 256),
                                     (9, 65536, 256), (1, 0, 256), (64, 1, 304), (2, 31, 8), (9, 16384, 1)])
def test_plan_properties(lib, q, p, cus):
    n = p + q
    pl = _lib.plan(q, 64, 1, n, n, cus)
    assert pl.tile == 32
    assert pl.chunk % pl.tile == 0 and pl.chunk >= pl.tile
    assert pl.nsplit == math.ceil(n / pl.chunk)  # chunks cover [0, n) without overlap
    assert (pl.nsplit - 1) * pl.chunk < n
    assert pl.combine == (1 if pl.nsplit > 1 else 0)
    nwork = q * pl.nsplit
    assert pl.grid >= nwork and pl.grid % 8 == 0 and pl.grid - nwork < 8
    if q >= cus:
        assert pl.nsplit == 1
    # about one workgroup per CU once the KV is long enough
    if n >= 64 * cus and q <= cus:
        assert nwork <= cus


def test_plan_forced_split(lib):
    pl = _lib.plan(9, 64, 1, 16393, 16393, 256, nsplit=7)
    assert pl.nsplit <= 7 and pl.nsplit >= 6
    pl1 = _lib.plan(9, 64, 1, 16393, 16393, 256, nsplit=1)
    assert pl1.nsplit == 1 and pl1.combine == 0


def test_plan_batched(lib):
    pl = _lib.plan(33, 64, 8, 80000, 32801, 256)
    assert pl.nsplit == math.ceil(32801 / pl.chunk)


def test_workspace_size(lib):
    n = 16393
    pl = _lib.plan(9, 64, 1, n, n, 256)
    # default: int16 partials (1024 B per row) plus an fp32 lse and an fp32 scale per row
    ws = _lib.workspace_size(9, 64, 1, n, n, num_cus=256)
    assert ws == pl.nsplit * 9 * 64 * (512 * 2 + 4 + 4)
    # fp32 partials: 512 values and an lse per row
    assert _lib.workspace_size(9, 64, 1, n, n, num_cus=256, partials=1) == pl.nsplit * 9 * 64 * 513 * 4
    # the VALU cross-check kernel always uses fp32 partials
    assert _lib.workspace_size(9, 64, 1, n, n, num_cus=256, kernel=1) == pl.nsplit * 9 * 64 * 513 * 4
    assert _lib.workspace_size(9, 64, 1, 265, 265, num_cus=256, nsplit=1) == 0
    # any head count: 9 x 8 = 72 rows -> 2 row blocks of 64
    pl8 = _lib.plan(9, 8, 1, n, n, 256)
    assert _lib.workspace_size(9, 8, 1, n, n, num_cus=256) == pl8.nsplit * 2 * 64 * (512 * 2 + 8)
    assert _lib.workspace_size(9, 1025, 1, n, n, num_cus=256) == 0  # beyond MLAV_MAX_HEADS -> 0
    assert _lib.workspace_size(0, 64, 1, n, n, num_cus=256) == 0


def test_plan_merged_in_split_kernel(lib):
    """With merge = 1, plans of 2..4 splits with int16 partials merge in the
    split kernel (combine = 2) and add one 8-byte ticket per row block to the
    workspace; merge = 0 (the default), fp32 partials or the VALU kernel keep
    the combine kernel."""
    for n, ns in [(100, 2), (150, 3), (250, 4)]:
        pl = _lib.plan(9, 64, 1, n, n, 256, merge=1)
        assert pl.nsplit == ns and pl.combine == 2
        ws = _lib.workspace_size(9, 64, 1, n, n, num_cus=256, merge=1)
        assert ws == ns * 9 * 64 * (512 * 2 + 8) + 9 * 8
        pl0 = _lib.plan(9, 64, 1, n, n, 256)
        assert pl0.nsplit == ns and pl0.combine == 1
        assert _lib.workspace_size(9, 64, 1, n, n, num_cus=256) == ns * 9 * 64 * (512 * 2 + 8)
        assert _lib.plan(9, 64, 1, n, n, 256, partials=1, merge=1).combine == 1
        assert _lib.plan(9, 64, 1, n, n, 256, kernel=1, merge=1).combine == 1
    # 5 or more splits: the combine kernel
    pl5 = _lib.plan(9, 64, 1, 300, 300, 256, merge=1)
    assert pl5.nsplit == 5 and pl5.combine == 1
    # batched, any head count: tickets for every (sequence, row block)
    pl = _lib.plan(9, 8, 3, 3 * 150, 150, 256, merge=1)
    assert pl.combine == 2
    assert (_lib.workspace_size(9, 8, 3, 450, 150, num_cus=256, merge=1)
            == 3 * pl.nsplit * 2 * 64 * (512 * 2 + 8) + 3 * 2 * 8)
    # one split: no workspace, no combine
    assert _lib.plan(9, 64, 1, 60, 60, 256, merge=1).combine == 0


def test_plan_errors(lib):
    with pytest.raises(_lib.MLAVError) as e:
        _lib.plan(9, 1025, 1, 100, 100, 256)
    assert e.value.status == _lib.MLAV_ERR_SHAPE
    for args in [(0, 64, 1, 100, 100, 256), (65, 64, 1, 100, 100, 256), (9, 64, 1, 5, 5, 256),
                 (9, 64, 2, 100, 200, 256)]:
        with pytest.raises(_lib.MLAVError) as e:
            _lib.plan(*args)
        assert e.value.status == _lib.MLAV_ERR_SHAPE
    with pytest.raises(_lib.MLAVError) as e:
        _lib.plan(9, 64, 1, 100, 100, 0)
    assert e.value.status == _lib.MLAV_ERR_ARG
    with pytest.raises(_lib.MLAVError) as e:
        _lib.plan(9, 64, 1, 100, 100, 256, pv_mode=5)
    assert e.value.status == _lib.MLAV_ERR_ARG


def test_plan_refuses_launches_beyond_32_bits(lib):
    # 1024 row blocks x 16384 splits: 2^24 workgroups of 256 threads
    n = 16384 * 32
    with pytest.raises(_lib.MLAVError) as e:
        _lib.plan(64, 1024, 1, n, n, 256, nsplit=16384)
    assert e.value.status == _lib.MLAV_ERR_SHAPE
    assert _lib.plan(64, 1024, 1, n, n, 256, nsplit=8192).nsplit == 8192
    # 600 sequences of 64 x 1024 rows in two splits: the fp32-partial combine
    # (128 threads per row) would pass 2^32 threads, the int16 one (64) does not
    assert _lib.plan(64, 1024, 600, 600 * 128, 128, 256, nsplit=2).combine == 1
    with pytest.raises(_lib.MLAVError) as e:
        _lib.plan(64, 1024, 600, 600 * 128, 128, 256, nsplit=2, partials=1)
    assert e.value.status == _lib.MLAV_ERR_SHAPE
    # the VALU kernel takes 16 workgroups per item: 1024 row blocks x 2048 splits
    assert _lib.plan(64, 1024, 1, 65536, 65536, 256, nsplit=2048).nsplit == 2048
    with pytest.raises(_lib.MLAVError) as e:
        _lib.plan(64, 1024, 1, 65536, 65536, 256, nsplit=2048, kernel=1)
    assert e.value.status == _lib.MLAV_ERR_SHAPE


# fake, aligned addresses: validation must reject the call before any use
A = 0x10000


def call(lib, **kw):
    args = dict(qn=A, qr=A, lat=A, rope=A, parent=A, prefix=100, scale=0.07, out=A, lse=A, q=9, h=64,
                ws=None, wsb=0, stream=None)
    args.update(kw)
    return lib.mla_verify(args["qn"], args["qr"], args["lat"], args["rope"], args["parent"], args["prefix"],
                          args["scale"], args["out"], args["lse"], args["q"], args["h"], args["ws"],
                          args["wsb"], args["stream"])


def test_host_validation_errors(lib):
    for k in ("qn", "qr", "lat", "rope", "parent", "out", "lse"):
        assert call(lib, **{k: None}) == _lib.MLAV_ERR_NULL
    assert call(lib, q=0) == _lib.MLAV_ERR_SHAPE
    assert call(lib, q=65) == _lib.MLAV_ERR_SHAPE
    assert call(lib, h=0) == _lib.MLAV_ERR_SHAPE
    assert call(lib, h=1025) == _lib.MLAV_ERR_SHAPE
    assert call(lib, prefix=-1) == _lib.MLAV_ERR_SHAPE
    for k in ("qn", "qr", "lat", "rope", "out"):
        assert call(lib, **{k: A + 8}) == _lib.MLAV_ERR_ALIGN
    for k in ("lse", "parent"):
        assert call(lib, **{k: A + 2}) == _lib.MLAV_ERR_ALIGN
    assert call(lib, scale=float("nan")) == _lib.MLAV_ERR_ARG
    assert call(lib, scale=float("inf")) == _lib.MLAV_ERR_ARG
    assert call(lib, scale=0.0) == _lib.MLAV_ERR_ARG
    assert call(lib, scale=-0.5) == _lib.MLAV_ERR_ARG
    for bad in (_lib.Options(0, 0, 0, 2, 0), _lib.Options(0, 0, 0, -1, 0), _lib.Options(0, 0, 0, 0, 3),
                _lib.Options(0, 0, 2, 0, 0), _lib.Options(0, 2, 0, 0, 0), _lib.Options(-1, 0, 0, 0, 0),
                _lib.Options(0, 0, 0, 0, 0, 2), _lib.Options(0, 0, 0, 0, 0, -1)):
        assert lib.mla_verify_ex(A, A, A, A, A, 100, 0.07, A, A, 9, 64, None, 0, None,
                                 ctypes.byref(bad)) == _lib.MLAV_ERR_ARG


def test_batched_validation_errors(lib):
    opt = _lib.options()
    f = lib.mla_verify_batched
    ok = dict(offs=A, batch=2, total=200, maxkv=100)

    def c(**kw):
        d = dict(ok)
        d.update(kw)
        return f(A, A, A, A, A, d["offs"], d["batch"], d["total"], d["maxkv"], 0.07, A, A, 9, 64, None, 0,
                 None, ctypes.byref(opt))

    assert c(offs=None) == _lib.MLAV_ERR_NULL
    assert c(offs=A + 4) == _lib.MLAV_ERR_ALIGN
    assert c(batch=0) == _lib.MLAV_ERR_SHAPE
    assert c(maxkv=5) == _lib.MLAV_ERR_SHAPE
    assert c(total=10) == _lib.MLAV_ERR_SHAPE
    assert c(maxkv=300) == _lib.MLAV_ERR_SHAPE


def test_combine_validation(lib):
    f = lib.mla_verify_combine
    assert f(None, A, 2, 64, A, A, None) == _lib.MLAV_ERR_NULL
    assert f(A, A, 0, 64, A, A, None) == _lib.MLAV_ERR_SHAPE
    assert f(A, A, 2, 63, A, A, None) == _lib.MLAV_ERR_SHAPE
    assert f(A + 4, A, 2, 64, A, A, None) == _lib.MLAV_ERR_ALIGN


def test_paged_validation_errors(lib):
    opt = _lib.options()
    f = lib.mla_verify_paged
    ok = dict(idx=A, pool=1000, offs=None, batch=1, total=300, maxkv=300)

    def c(**kw):
        d = dict(ok)
        d.update(kw)
        return f(A, A, A, A, d["idx"], d["pool"], A, d["offs"], d["batch"], d["total"], d["maxkv"], 0.07, A, A,
                 9, 64, None, 0, None, ctypes.byref(opt))

    assert c(idx=None) == _lib.MLAV_ERR_NULL
    assert c(idx=A + 2) == _lib.MLAV_ERR_ALIGN
    assert c(pool=0) == _lib.MLAV_ERR_SHAPE
    assert c(pool=4000001) == _lib.MLAV_ERR_SHAPE
    assert c(batch=0) == _lib.MLAV_ERR_SHAPE
    assert c(total=5, maxkv=5) == _lib.MLAV_ERR_SHAPE
    # without offsets there is exactly one sequence of total_kv rows
    assert c(batch=2, total=600, maxkv=300) == _lib.MLAV_ERR_ARG
    assert c(maxkv=200) == _lib.MLAV_ERR_ARG
    assert c(offs=A + 4, batch=2, total=600, maxkv=300) == _lib.MLAV_ERR_ALIGN


def test_plan_counts_row_blocks(lib):
    """The planner fills the CUs with (row block, split) work items: a row
    block is 64 consecutive (token, head) rows, so H = 8 at q = 9 has 2 blocks
    and H = 128 has 18."""
    n = 16393
    for heads, blocks in ((64, 9), (8, 2), (16, 3), (128, 18), (1, 1)):
        pl = _lib.plan(9, heads, 1, n, n, 256)
        assert pl.grid >= blocks * pl.nsplit and pl.grid % 8 == 0
        assert blocks * pl.nsplit <= 256 or pl.chunk == 64


def test_partials_plan_chunk_bounds(lib):
    """A caller-made plan whose chunk exceeds MLAV_MAX_KV (the kernels take the
    chunk as a 32-bit key count) is refused, whatever its split count."""
    opt = _lib.options()
    f = lib.mla_verify_partials

    def c(nsplit, chunk, prefix=100):
        plan = _lib.Plan(nsplit, 32, chunk, 0, 0)
        return f(A, A, A, A, A, prefix, 0.07, A, A, 9, 64, ctypes.byref(plan), None, ctypes.byref(opt))

    assert c(1, 1 << 40) == _lib.MLAV_ERR_ARG
    assert c(1, 4000032) == _lib.MLAV_ERR_ARG
    assert c(1, 48) == _lib.MLAV_ERR_ARG  # not a multiple of the tile
    assert c(0, 64) == _lib.MLAV_ERR_ARG
    assert c(3, 32, prefix=100) == _lib.MLAV_ERR_ARG  # 109 rows in chunks of 32 need 4 splits
    # 1024 row blocks x 16384 chunks of 32 keys: 2^32 threads in the split launch
    plan = _lib.Plan(16384, 32, 32, 0, 0)
    assert f(A, A, A, A, A, 16384 * 32 - 64, 0.07, A, A, 64, 1024, ctypes.byref(plan), None,
             ctypes.byref(opt)) == _lib.MLAV_ERR_SHAPE


def test_combine_row_bound(lib):
    f = lib.mla_verify_combine
    assert f(A, A, 2, (1 << 24) + 64, A, A, None) == _lib.MLAV_ERR_SHAPE
    assert f(A, A, 2, 1 << 34, A, A, None) == _lib.MLAV_ERR_SHAPE


def test_probe_library_exports_its_header():
    """The benchmark's probes: a separate library with its own header."""
    path = os.path.join(ROOT, "mla_tree_verify_amd", "libmla_verify_probe.so")
    if not os.path.exists(path):
        pytest.skip("probe library not built")
    text = open(os.path.join(ROOT, "include", "mla_verify_probe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    declared = sorted(set(re.findall(r"\b(mlav_probe\w*)\s*\(", text)))
    assert declared == ["mlav_probe_mfma", "mlav_probe_mfma_per_wave", "mlav_probe_step_mix",
                        "mlav_probe_steps_per_iteration"]
    probe = ctypes.CDLL(path)
    for name in declared:
        assert hasattr(probe, name)
    probe.mlav_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p]
    probe.mlav_probe_mfma.restype = ctypes.c_int32
    buf = ctypes.create_string_buffer(64)
    # argument errors are caught on the host, before any launch
    assert probe.mlav_probe_mfma(0, 10, buf, buf, None) == 2
    assert probe.mlav_probe_mfma(1, 0, buf, buf, None) == 2
    assert probe.mlav_probe_mfma(1, 10, None, buf, None) == 2
    assert probe.mlav_probe_mfma(1, 10, buf, None, None) == 2
    assert probe.mlav_probe_mfma_per_wave() == 16
    probe.mlav_probe_step_mix.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    probe.mlav_probe_step_mix.restype = ctypes.c_int32
    assert probe.mlav_probe_step_mix(1, 10, 8, buf, buf, buf, None) == 2  # parts beyond the three bits
    assert probe.mlav_probe_step_mix(1, 10, -1, buf, buf, buf, None) == 2
    assert probe.mlav_probe_step_mix(0, 10, 7, buf, buf, buf, None) == 2
    assert probe.mlav_probe_step_mix(1, 10, 7, None, buf, buf, None) == 2
    assert probe.mlav_probe_steps_per_iteration() == 4


@pytest.mark.parametrize("lens,q,heads,cus", [
    ([3766, 1817, 19196, 18627, 2261, 3227, 10553, 1319], 33, 64, 256),  # a ragged batch of 8
    ([265] * 4, 9, 64, 256), ([4105] * 32, 9, 64, 256), ([16393] * 4, 9, 64, 256),  # equal lengths
    ([10, 100000], 9, 64, 256), ([70] * 63 + [5000], 2, 8, 256), ([64, 65, 127, 128, 129], 1, 1, 8),
])
def test_batched_plan_covers_the_chunk_list(lib, lens, q, heads, cus):
    """Batched plans: the chunks of every sequence fit the grid (each chunk's
    row blocks are one work item each), whatever the lengths behind the host's
    total and maximum; equal lengths fill the CUs in no more tile steps than
    one chunk per sequence would, and unequal ones spread over the CUs."""
    total, mx, b = sum(lens), max(lens), len(lens)
    pl = _lib.plan(q, heads, b, total, mx, cus)
    assert pl.tile == 32 and pl.chunk % 32 == 0 and pl.chunk >= 64
    assert pl.nsplit == math.ceil(mx / pl.chunk)
    nrb = math.ceil(q * heads / 64)
    chunks = sum(math.ceil(n / pl.chunk) for n in lens)
    assert chunks <= math.ceil(total / pl.chunk) + b - 1  # the bound the grid is sized for
    assert pl.grid >= chunks * nrb and pl.grid % 8 == 0
    assert pl.grid <= (math.ceil(total / pl.chunk) + b - 1) * nrb + 64  # rounded up to whole rounds of runs
    if len(set(lens)) == 1:
        # equal lengths: no more rounds of workgroups over the CUs than one chunk per sequence would take
        rounds = math.ceil(math.ceil(chunks * nrb / 8) / (cus // 8))
        one = math.ceil(math.ceil(b * nrb / 8) / (cus // 8))
        assert rounds * pl.chunk <= one * math.ceil(mx / 32) * 32
    else:
        # unequal lengths: the long sequences are cut so that at least half the CUs get work
        assert chunks * nrb >= min(cus // 2, nrb * b)


def test_plain_c_caller(tmp_path):
    """tests/c_abi_check.c: the headers compile as strict C99, the library
    links from C, and its host-only entry points behave as documented."""
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    libdir = os.path.join(ROOT, "mla_tree_verify_amd")
    if gcc is None:
        pytest.skip("gcc not found")
    for name in ("libmla_verify.so", "libmla_verify_probe.so"):
        if not os.path.exists(os.path.join(libdir, name)):
            pytest.skip(f"{name} not built")
    exe = str(tmp_path / "c_abi_check")
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi_check.c"), "-L", libdir, "-lmla_verify", "-lmla_verify_probe",
           f"-Wl,-rpath,{libdir}", "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr
    assert "c abi ok" in run.stdout
