"""The C ABI library on the CPU: it loads, exports every symbol the header
declares, sizes workspaces, and rejects bad arguments on the host before any
launch (every call below fails validation, so no HIP work is attempted)."""
import ctypes
import glob
import math
import os
import re
import shutil
import subprocess

import pytest

from conftest import ROOT

tlb = pytest.importorskip("token_level_block_amd")

HEADER = os.path.join(ROOT, "include", "uniprefill.h")
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))
FAKE = 1 << 20            # a nonzero, 256-aligned address that is never dereferenced
FAKE_MIS = FAKE + 2       # misaligned


def declared_functions():
    """Every up_* function declared in any include/*.h header."""
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(up_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 8
    lib = ctypes.CDLL(tlb.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(tlb.EXPORTED)


def test_status_strings():
    for code in range(0, -7, -1):
        assert tlb.status_string(code) and tlb.status_string(code) != "unknown status"
    assert tlb.status_string(-99) == "unknown status"


def p(**kw):
    base = dict(num_heads_q=32, num_heads_kv=8, head_dim=128, block_size=64, num_sink=128, window=128,
                top_p=0.99)
    base.update(kw)
    scores_in = base.pop("scores_in", False)
    return tlb.make_params(**base, scores_in=scores_in)


def test_max_blocks_bound():
    assert tlb.max_blocks(64, 1, 131072) == 2048 + 1
    assert tlb.max_blocks(64, 4, 30720) == 480 + 4
    assert tlb.max_blocks(0, 1, 10) == -1
    # the bound covers any split of max_tokens into num_reqs requests
    for lens in ([1] * 7, [64, 64, 1], [63, 1, 127], [4096, 8192, 16384, 2048]):
        T, R = sum(lens), len(lens)
        assert sum(math.ceil(L / 64) for L in lens) <= tlb.max_blocks(64, R, T)


def test_workspace_sizes():
    prm = p()
    ws = tlb.select_workspace_bytes(prm, 1, 131072)
    rows = 32 * 128
    # block partials + chunk partials dominate
    assert ws >= 4 * rows * (2048 + 1)
    assert ws % 256 == 0
    assert tlb.select_workspace_bytes(p(scores_in=True), 1, 131072) < 64 * 1024
    assert tlb.select_workspace_bytes(p(head_dim=96), 1, 100) == 0
    assert tlb.compact_workspace_bytes(4, 30720) > 0
    assert tlb.compact_workspace_bytes(-1, 10) == 0


def call_select(prm, q=FAKE, qs=32 * 128, k=FAKE, ks=8 * 128, cu=FAKE, R=1, T=4096, scores=None,
                mask=FAKE, kept=FAKE, ws=FAKE, wsb=None):
    if wsb is None:
        wsb = tlb.select_workspace_bytes(prm, R, T) if tlb.select_workspace_bytes(prm, R, T) else 1 << 40
    return tlb.select_blocks(prm, q, qs, k, ks, cu, R, T, scores, None, None, None, mask, kept, ws,
                             workspace_bytes=wsb, stream=0, raise_on_error=False)


@pytest.mark.parametrize("kw,code", [
    (dict(num_heads_kv=5), tlb.UP_ERR_SHAPE),
    (dict(num_heads_q=0), tlb.UP_ERR_SHAPE),
    (dict(head_dim=96), tlb.UP_ERR_PARAM),
    (dict(block_size=48), tlb.UP_ERR_PARAM),
    (dict(block_size=0), tlb.UP_ERR_PARAM),
    (dict(window=0), tlb.UP_ERR_PARAM),
    (dict(num_sink=-1), tlb.UP_ERR_PARAM),
    (dict(top_p=0.0), tlb.UP_ERR_PARAM),
    (dict(top_p=1.5), tlb.UP_ERR_PARAM),
    (dict(top_p=float("nan")), tlb.UP_ERR_PARAM),
    (dict(softmax_scale=float("inf")), tlb.UP_ERR_PARAM),
])
def test_select_rejects_params(kw, code):
    assert call_select(p(**kw)) == code


def test_select_rejects_nulls_shapes_alignment_workspace():
    prm = p()
    assert tlb.select_blocks(None, FAKE, 1, FAKE, 1, FAKE, 1, 1, None, None, None, None, FAKE, FAKE,
                             FAKE, workspace_bytes=1 << 30, stream=0, raise_on_error=False) == tlb.UP_ERR_NULL
    assert call_select(prm, q=None) == tlb.UP_ERR_NULL
    assert call_select(prm, cu=None) == tlb.UP_ERR_NULL
    assert call_select(prm, mask=None) == tlb.UP_ERR_NULL
    assert call_select(prm, kept=None) == tlb.UP_ERR_NULL
    assert call_select(prm, ws=None) == tlb.UP_ERR_NULL
    assert call_select(p(scores_in=True), q=None, k=None, scores=None) == tlb.UP_ERR_NULL
    assert call_select(prm, R=-1) == tlb.UP_ERR_SHAPE
    assert call_select(prm, T=-5) == tlb.UP_ERR_SHAPE
    assert call_select(prm, T=2 ** 31) == tlb.UP_ERR_SHAPE
    assert call_select(prm, qs=100) == tlb.UP_ERR_SHAPE          # smaller than Hq*d
    assert call_select(prm, q=FAKE_MIS) == tlb.UP_ERR_ALIGN
    assert call_select(prm, ks=8 * 128 + 4) == tlb.UP_ERR_ALIGN
    assert call_select(prm, ws=FAKE + 16) == tlb.UP_ERR_ALIGN
    need = tlb.select_workspace_bytes(prm, 1, 4096)
    assert call_select(prm, wsb=need - 1) == tlb.UP_ERR_WORKSPACE


def test_scores_in_mode_accepts_any_block_size_in_planning():
    prm = p(scores_in=True, block_size=7, head_dim=1)
    assert tlb.select_workspace_bytes(prm, 3, 1000) > 0
    # still rejects a too-small workspace before launching
    assert call_select(prm, q=None, k=None, scores=FAKE, wsb=16) == tlb.UP_ERR_WORKSPACE


def call_compact(mask=FAKE, cu=FAKE, R=2, T=1000, src=(FAKE,), dst=(FAKE,), rb=(8192,), iout=FAKE,
                 cuo=FAKE, ws=FAKE, wsb=1 << 30):
    return tlb.compact(mask, cu, R, T, list(src), list(dst), list(rb), None, iout, cuo, ws,
                       workspace_bytes=wsb, stream=0, raise_on_error=False)


def test_compact_rejects():
    assert call_compact(mask=None) == tlb.UP_ERR_NULL
    assert call_compact(iout=None) == tlb.UP_ERR_NULL
    assert call_compact(src=(None,)) == tlb.UP_ERR_NULL
    assert call_compact(R=-1) == tlb.UP_ERR_SHAPE
    assert call_compact(rb=(6,)) == tlb.UP_ERR_PARAM
    assert call_compact(rb=(0,)) == tlb.UP_ERR_PARAM
    assert call_compact(src=(FAKE,) * 9, dst=(FAKE,) * 9, rb=(16,) * 9) == tlb.UP_ERR_PARAM
    assert call_compact(mask=FAKE + 1) == tlb.UP_ERR_ALIGN
    assert call_compact(src=(FAKE + 2,)) == tlb.UP_ERR_ALIGN
    assert call_compact(wsb=tlb.compact_workspace_bytes(2, 1000) - 1) == tlb.UP_ERR_WORKSPACE


def test_compact_noalloc_rejects_before_any_hip_work():
    """Same validation as up_compact, and streams past the scratch's maximum
    rejected up front (the scratch is never located for a rejected call)."""
    lib = tlb._lib
    vp = ctypes.c_void_p
    src = (vp * 1)(FAKE)
    dst = (vp * 1)(FAKE + 4096)
    rb = (ctypes.c_int64 * 1)(16)
    call = lambda mask, cu, R, T, n=1, rbx=rb: lib.up_compact_noalloc(mask, cu, R, T, n, src, dst, rbx, None, FAKE,
                                                                     FAKE, None)
    assert tlb.COMPACT_NOALLOC_MAX_TOKENS == 4000000
    assert call(FAKE, FAKE, 1, tlb.COMPACT_NOALLOC_MAX_TOKENS + 1) == tlb.UP_ERR_WORKSPACE
    assert call(FAKE, FAKE, -1, 100) == tlb.UP_ERR_SHAPE
    assert call(None, FAKE, 1, 100) == tlb.UP_ERR_NULL
    assert call(FAKE_MIS, FAKE, 1, 100) == tlb.UP_ERR_ALIGN
    assert call(FAKE, FAKE, 1, 100, n=9) == tlb.UP_ERR_PARAM
    assert call(FAKE, FAKE, 1, 100, rbx=(ctypes.c_int64 * 1)(6)) == tlb.UP_ERR_PARAM


def test_scatter_and_metadata_reject():
    sb = lambda **kw: tlb.scatter_back(kw.get("c", FAKE), kw.get("rb", 16), kw.get("im", FAKE), FAKE,
                                       kw.get("R", 1), 10, kw.get("full", FAKE), kw.get("fr", 10),
                                       stream=0, raise_on_error=False)
    assert sb(c=None) == tlb.UP_ERR_NULL
    assert sb(full=None) == tlb.UP_ERR_NULL
    assert sb(rb=3) == tlb.UP_ERR_PARAM
    assert sb(R=-1) == tlb.UP_ERR_SHAPE
    assert sb(fr=-1) == tlb.UP_ERR_SHAPE
    assert sb(c=FAKE + 1) == tlb.UP_ERR_ALIGN
    md = lambda **kw: tlb.update_metadata(kw.get("layer", 0), 4, kw.get("R", 1), FAKE, FAKE,
                                          kw.get("sl", FAKE), FAKE, FAKE, kw.get("dl", FAKE), FAKE,
                                          kw.get("md", 4), FAKE, stream=0, raise_on_error=False)
    assert md(layer=-1) == tlb.UP_ERR_SHAPE
    assert md(R=-1) == tlb.UP_ERR_SHAPE
    assert md(sl=None) == tlb.UP_ERR_NULL
    assert md(dl=None) == tlb.UP_ERR_NULL
    assert md(md=-1) == tlb.UP_ERR_SHAPE


def test_python_binding_raises():
    with pytest.raises(tlb.UniPrefillError):
        call = tlb.select_blocks(p(head_dim=96), FAKE, 1, FAKE, 1, FAKE, 1, 1, None, None, None, None,
                                 FAKE, FAKE, FAKE, workspace_bytes=1, stream=0)
        del call


def test_single_hip_runtime_in_process():
    """The binding loads torch before libuniprefill, so the process holds one
    HIP runtime and one HSA runtime (torch bundles its own copies under the
    same sonames as the ROCm install)."""
    maps = open("/proc/self/maps").read()
    hip = set(re.findall(r"(/\S*libamdhip64\S*)", maps))
    hsa = set(re.findall(r"(/\S*libhsa-runtime64\S*)", maps))
    assert len(hip) == 1, hip
    assert len(hsa) <= 1, hsa


def test_peaks_library_exports_and_rejects():
    """libuppeaks (the benchmark's reference-rate probes) loads, exports its
    five calls, and rejects bad arguments before launching anything."""
    path = os.path.join(os.path.dirname(tlb.LIB_PATH), "libuppeaks.so")
    lib = ctypes.CDLL(path)
    for name in ("upk_mfma_out_floats", "upk_mfma_flops", "upk_mfma_launch", "upk_mfma16_launch",
                 "upk_copy_launch"):
        assert hasattr(lib, name), name
    lib.upk_mfma_flops.restype = ctypes.c_double
    lib.upk_mfma_flops.argtypes = [ctypes.c_int32]
    lib.upk_mfma_out_floats.restype = ctypes.c_int64
    lib.upk_mfma_out_floats.argtypes = [ctypes.c_int32]
    # 8 waves x 256 trips x 16 MFMAs x (2 * 32 * 32 * 16) flops per workgroup
    assert lib.upk_mfma_flops(1) == 8 * 256 * 16 * 2 * 32 * 32 * 16
    assert lib.upk_mfma_out_floats(3) == 3 * 512
    lib.upk_mfma_launch.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    lib.upk_copy_launch.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                    ctypes.c_void_p]
    assert lib.upk_mfma_launch(None, 4, None) == -1
    assert lib.upk_mfma_launch(FAKE, 0, None) == -1
    lib.upk_mfma16_launch.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    assert lib.upk_mfma16_launch(None, 4, None) == -1
    assert lib.upk_mfma16_launch(FAKE, 0, None) == -1
    assert lib.upk_copy_launch(FAKE, FAKE, 100, 4, None) == -1      # not a multiple of 16
    assert lib.upk_copy_launch(FAKE_MIS, FAKE, 64, 4, None) == -1
    assert lib.upk_copy_launch(None, FAKE, 64, 4, None) == -1


def test_slot_mapping_and_kv_write_reject():
    sm = lambda **kw: tlb.slot_mapping(kw.get("bt", FAKE), kw.get("bts", 8), kw.get("w", 8), kw.get("B", 16),
                                       kw.get("cu", FAKE), kw.get("sl", FAKE), kw.get("R", 2),
                                       kw.get("T", 100), kw.get("out", FAKE), stream=0, raise_on_error=False)
    assert sm(cu=None) == tlb.UP_ERR_NULL
    assert sm(sl=None) == tlb.UP_ERR_NULL
    assert sm(out=None) == tlb.UP_ERR_NULL
    assert sm(bt=None) == tlb.UP_ERR_NULL
    assert sm(R=-1) == tlb.UP_ERR_SHAPE
    assert sm(T=-1) == tlb.UP_ERR_SHAPE
    assert sm(T=2 ** 31) == tlb.UP_ERR_SHAPE
    assert sm(w=9) == tlb.UP_ERR_SHAPE            # wider than the row stride
    assert sm(w=-1) == tlb.UP_ERR_SHAPE
    assert sm(B=0) == tlb.UP_ERR_PARAM
    assert sm(out=FAKE + 4) == tlb.UP_ERR_ALIGN   # int64 output
    assert sm(cu=FAKE + 2) == tlb.UP_ERR_ALIGN
    kv = lambda **kw: tlb.write_kv_cache(kw.get("k", FAKE), kw.get("ks", 2048), kw.get("v", FAKE),
                                         kw.get("vs", 2048), kw.get("rb", 2048), kw.get("sl", FAKE),
                                         kw.get("cu", FAKE), kw.get("R", 1), kw.get("T", 10),
                                         kw.get("kc", FAKE), kw.get("vc", FAKE), kw.get("cs", 64),
                                         stream=0, raise_on_error=False)
    assert kv(k=None) == tlb.UP_ERR_NULL
    assert kv(kc=None) == tlb.UP_ERR_NULL
    assert kv(sl=None) == tlb.UP_ERR_NULL
    assert kv(v=None) == tlb.UP_ERR_NULL          # value without value_cache (or the reverse)
    assert kv(vc=None) == tlb.UP_ERR_NULL
    assert kv(rb=6) == tlb.UP_ERR_PARAM
    assert kv(rb=0) == tlb.UP_ERR_PARAM
    assert kv(ks=1024) == tlb.UP_ERR_SHAPE        # stride below the row size
    assert kv(cs=-1) == tlb.UP_ERR_SHAPE
    assert kv(R=-1) == tlb.UP_ERR_SHAPE
    assert kv(ks=2050) == tlb.UP_ERR_ALIGN
    assert kv(k=FAKE + 2) == tlb.UP_ERR_ALIGN
    assert kv(sl=FAKE + 4) == tlb.UP_ERR_ALIGN


def test_ffn_rejects_before_any_hip_work():
    lib = tlb._lib
    assert lib.up_ffn_workspace_bytes(0, 64, 4) == 0
    assert lib.up_ffn_workspace_bytes(4096, 14330, 4) == 0      # not a multiple of 8
    assert lib.up_ffn_workspace_bytes(64, 64, -1) == 0
    assert lib.up_ffn_workspace_bytes(64, 64, 10) >= 10 * 64 * 2
    with pytest.raises(tlb.UniPrefillError):
        tlb.FFN(-8, 64)
    ws = 1 << 30
    fwd = lambda *a: lib.up_ffn_forward(*a)
    assert fwd(4096, 14330, FAKE, 4, FAKE, FAKE, FAKE, FAKE, ws, None) == tlb.UP_ERR_PARAM
    assert fwd(64, 64, FAKE, -1, FAKE, FAKE, FAKE, FAKE, ws, None) == tlb.UP_ERR_SHAPE
    assert fwd(64, 64, None, 4, FAKE, FAKE, FAKE, FAKE, ws, None) == tlb.UP_ERR_NULL
    assert fwd(64, 64, FAKE, 4, FAKE, FAKE, None, FAKE, ws, None) == tlb.UP_ERR_NULL
    assert fwd(64, 64, FAKE_MIS, 4, FAKE, FAKE, FAKE, FAKE, ws, None) == tlb.UP_ERR_ALIGN
    assert fwd(64, 64, FAKE, 4, FAKE, FAKE, FAKE, FAKE, 16, None) == tlb.UP_ERR_WORKSPACE
    # zero rows: nothing to do, nothing read
    assert fwd(64, 64, None, 0, None, None, None, None, 0, None) == tlb.UP_OK


def test_header_is_plain_c(tmp_path):
    """include/uniprefill.h compiles as C99 with -pedantic -Werror, and a C
    program linked against the library sizes workspaces and gets the
    documented status codes (tests/abi_check.c; host-side paths only)."""
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path / "abi_check")
    libdir = os.path.dirname(tlb.LIB_PATH)
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_check.c"),
                    "-L", libdir, "-luniprefill", f"-Wl,-rpath,{libdir}", "-o", exe],
                   check=True, capture_output=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    got = dict(line.split(" ", 1) for line in out.splitlines())
    assert got == {
        "max_blocks": str(tlb.max_blocks(64, 1, 131072)),
        "select_ws_positive": "1",
        "compact_ws_positive": "1",
        "status_ok": "set",
        "select_null_params": str(tlb.UP_ERR_NULL),
        "select_bad_p": str(tlb.UP_ERR_PARAM),
        "select_profiled_bad_p": str(tlb.UP_ERR_PARAM),
        "select_small_workspace": str(tlb.UP_ERR_WORKSPACE),
        "scatter_odd_rows": str(tlb.UP_ERR_PARAM),
        "metadata_negative_layer": str(tlb.UP_ERR_SHAPE),
    }


def build_host_check(gxx, name, tmp_path):
    """Build a host-side planner check with g++, under AddressSanitizer and
    UndefinedBehaviorSanitizer (any finding aborts the run) where the toolchain
    has their runtimes, else plainly."""
    exe = str(tmp_path / name.replace(".cc", ""))
    base = [gxx, "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-Werror", os.path.join(ROOT, "tests", name), "-o", exe]
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    if subprocess.run(base[:1] + san + base[1:], capture_output=True).returncode != 0:
        subprocess.run(base, check=True, capture_output=True)
    return exe


def test_score_planner_invariants(tmp_path):
    """score_plan.h (host C++): every window query covered by exactly the
    planned slices, shapes within the kernel's register and wave budget,
    chunk lengths multiples of G within their bounds, and the launch shapes
    of the measured workloads (tests/plan_check.cc)."""
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no C++ compiler")
    exe = build_host_check(gxx, "plan_check.cc", tmp_path)
    p = subprocess.run([exe], capture_output=True, text=True)
    assert p.returncode == 0, p.stderr
    assert p.stdout.startswith("ok ") and int(p.stdout.split()[1]) > 1000


def test_copy_planner_invariants(tmp_path):
    """copy_plan.h (host C++): the multiply-high division that maps a flat
    copy's 16-byte units to rows equals integer division, every buffer of a
    launch owns a non-empty workgroup range, and flat buffers fit 32-bit unit
    indices and are covered by their workgroups (tests/copy_plan_check.cc)."""
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no C++ compiler")
    exe = build_host_check(gxx, "copy_plan_check.cc", tmp_path)
    p = subprocess.run([exe], capture_output=True, text=True)
    assert p.returncode == 0, p.stderr
    assert p.stdout.startswith("ok ") and int(p.stdout.split()[1]) > 1000000


def test_ffn_tile_walk_covers_every_tile_once(tmp_path):
    """ffn_walk.h (host C++, the same functions the FFN GEMM kernel calls):
    for every panel count up to 72 x 70 and the model shapes, the launch's
    workgroups compute each 256 x 256 tile exactly once, and the first 32
    workgroups of an XCD share at least 4 weight panels and one group of
    token panels (tests/ffn_walk_check.cc)."""
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no C++ compiler")
    exe = build_host_check(gxx, "ffn_walk_check.cc", tmp_path)
    p = subprocess.run([exe], capture_output=True, text=True)
    assert p.returncode == 0, p.stderr
    assert p.stdout.startswith("ok ") and int(p.stdout.split()[1]) > 1000000


def test_select_rejects_a_score_grid_beyond_32_bits():
    """A window so long that (key chunks x query slices) would not fit the
    grid's 32-bit x dimension is rejected at planning, not launched short."""
    prm = p(num_heads_kv=1, window=1 << 19)          # Hq * n = 2^24, 32768 query slices
    assert tlb.select_workspace_bytes(prm, 1, 2 ** 31 - 1) == 0
    assert call_select(prm, T=2 ** 31 - 1) == tlb.UP_ERR_SHAPE
    assert tlb.select_workspace_bytes(prm, 1, 4096) > 0   # the same parameters on a short batch plan fine
