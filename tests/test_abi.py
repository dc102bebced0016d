"""The C ABI without a GPU: the library loads, exports what include/fa.h
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

fa = pytest.importorskip("exact_io_aware_12_amd")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(fa_\w+)\s*\(", text,
                                 flags=re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == ["fa_bwd", "fa_bwd_dropout", "fa_bwd_dropout_stage",
                                    "fa_bwd_ex",
                                    "fa_bwd_kvlen", "fa_bwd_kvlen_stage",
                                    "fa_bwd_noalloc", "fa_bwd_num_stages", "fa_bwd_softcap",
                                    "fa_bwd_softcap_stage", "fa_bwd_stage",
                                    "fa_bwd_window", "fa_bwd_window_softcap",
                                    "fa_bwd_window_softcap_stage", "fa_bwd_window_stage",
                                    "fa_bwd_workspace_size", "fa_check_cu_seqlens", "fa_fwd",
                                    "fa_fwd_dropout", "fa_fwd_ex",
                                    "fa_fwd_fp8",
                                    "fa_fwd_kvcache", "fa_fwd_kvcache_fp8",
                                    "fa_fwd_kvcache_fp8_stage", "fa_fwd_kvcache_local",
                                    "fa_fwd_kvcache_num_stages", "fa_fwd_kvcache_stage",
                                    "fa_fwd_kvcache_workspace_size", "fa_fwd_kvlen",
                                    "fa_fwd_softcap", "fa_fwd_window", "fa_fwd_window_softcap",
                                    "fa_kvcache_fp8_num_splits", "fa_kvcache_num_splits",
                                    "fa_status_string"]


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(fa.lib_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def declared_prototypes():
    """{name: (return type, [parameter types])} from include/fa.h."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    protos = {}
    for m in re.finditer(r"^\s*((?:const\s+)?\w+\s*\**)\s*(fa_\w+)\s*\(([^)]*)\)\s*;", text,
                         flags=re.M):
        params = [p.strip() for p in m.group(3).split(",")]
        types = [] if params == ["void"] else [re.sub(r"\s*\b\w+$", "", p).strip() for p in params]
        protos[m.group(2)] = (m.group(1).strip(), types)
    return protos


def test_binding_prototypes_match_the_header():
    """Every ctypes signature the binding sets equals the C prototype in
    include/fa.h, parameter by parameter; the dtype arguments are fa_dtype."""
    C = {"int": ctypes.c_int, "fa_dtype": ctypes.c_int, "float": ctypes.c_float,
         "size_t": ctypes.c_size_t, "uint64_t": ctypes.c_uint64, "hipStream_t": ctypes.c_void_p,
         "const char*": ctypes.c_char_p}
    protos = declared_prototypes()
    assert sorted(protos) == declared_functions()
    for name, (ret, params) in protos.items():
        fn = getattr(fa.lib, name)
        assert fn.restype is C[ret], (name, ret)
        want = [ctypes.c_void_p if p.endswith("*") else C[p] for p in params]
        assert list(fn.argtypes) == want, (name, params)
        for p, orig in zip(params, re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
                           .split(name + "(", 1)[1].split(")", 1)[0].split(",")):
            if re.search(r"\b(dtype|out_dtype)\s*$", orig.strip()):
                assert p == "fa_dtype", (name, orig)


def test_binding_loads_torch_hip_runtime_first():
    """The binding imports torch before it loads libfa.so, so the library binds to
    torch's HIP runtime (a second runtime could not see torch's memory). In a fresh
    interpreter, importing the binding leaves exactly one libamdhip64 mapped, and
    it is torch's."""
    import subprocess
    import sys
    code = ("import exact_io_aware_12_amd, torch, os\n"
            "maps = open('/proc/self/maps').read().split('\\n')\n"
            "libs = sorted({l.split()[-1] for l in maps if 'libamdhip64' in l})\n"
            "print(len(libs), int(os.path.dirname(torch.__file__) in libs[0]))\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                         timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split() == ["1", "1"], out.stdout


def test_binding_source_imports_torch_before_loading():
    src = open(os.path.join(ROOT, "exact_io_aware_12_amd", "__init__.py")).read()
    body = src[src.index("def _load():"):]
    assert body.index("import torch") < body.index("ctypes.CDLL(")


def test_status_strings():
    for code in (0, -1, -2, -3, -4):
        assert fa.fa_status_string(code).startswith(
            {0: "FA_OK", -1: "FA_ERR_INVALID_ARG", -2: "FA_ERR_UNSUPPORTED", -3: "FA_ERR_HIP",
             -4: "FA_ERR_WORKSPACE"}[code])
    assert fa.fa_status_string(7) == "unknown fa status"


# Fake, never-dereferenced device addresses: every call below must be refused
# by the host-side checks before anything is enqueued.
P = 0x1000


def fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=2, N=16, d=64, scale=0.125, causal=0,
             cu=None, dtype=fa.FA_FP16, stream=None)
    a.update(kw)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["N"],
                     a["d"], a["scale"], a["causal"], a["cu"], a["dtype"], a["stream"])


def bwd(**kw):
    a = dict(B=1, Hq=2, Hkv=2, N=16, d=64, scale=0.125, causal=0, dtype=fa.FA_BF16, ws=P,
             wsb=1 << 20)
    a.update(kw)
    ptrs = [kw.get(n, P) for n in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv")]
    return fa.fa_bwd(*ptrs, a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["scale"], a["causal"],
                     None, a["dtype"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=-1), fa.FA_ERR_INVALID_ARG),
    (dict(B=-1), fa.FA_ERR_INVALID_ARG),
    (dict(N=-5), fa.FA_ERR_INVALID_ARG),
    (dict(Hq=0), fa.FA_ERR_INVALID_ARG),
    (dict(Hq=3, Hkv=2), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-0.1), fa.FA_ERR_INVALID_ARG),
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(k=P + 8), fa.FA_ERR_INVALID_ARG),      # not 16-byte aligned
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=512), fa.FA_ERR_UNSUPPORTED),
    (dict(B=1 << 16, N=1 << 16), fa.FA_ERR_UNSUPPORTED),
    (dict(B=0), fa.FA_OK),                       # empty batch: no-op
    (dict(N=0, q=None, k=None), fa.FA_OK),       # empty sequence: no-op, pointers unused
])
def test_fwd_host_checks(kw, status):
    assert fwd(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=5), fa.FA_ERR_INVALID_ARG),
    (dict(Hq=4, Hkv=3), fa.FA_ERR_INVALID_ARG),
    (dict(dv=None), fa.FA_ERR_INVALID_ARG),
    (dict(do=P + 2), fa.FA_ERR_INVALID_ARG),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(d=512), fa.FA_ERR_UNSUPPORTED),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(wsb=64), fa.FA_ERR_WORKSPACE),
    (dict(B=0), fa.FA_OK),
])
def test_bwd_host_checks(kw, status):
    assert bwd(**kw) == status


def test_bwd_stage_index_checked():
    assert fa.fa_bwd_num_stages() == 3
    ptrs = [P] * 9
    for bad in (-1, 3, 100):
        assert fa.fa_bwd_stage(bad, *ptrs, 1, 2, 2, 16, 64, 0.125, 0, None, 0, P, 1 << 20,
                               None) == fa.FA_ERR_INVALID_ARG
    # a valid stage goes through fa_bwd's own checks
    assert fa.fa_bwd_stage(1, *ptrs, 1, 2, 2, 16, 64, 0.125, 0, None, 0, None, 0,
                           None) == fa.FA_ERR_WORKSPACE


def test_workspace_size():
    assert fa.fa_bwd_workspace_size(2, 16, 16, 16384, 128) == 2 * 16 * (2 * 16384 + 64) * 4
    assert fa.fa_bwd_workspace_size(1, 2, 2, 3, 64) == 1280         # 2·2·67·4 = 1072 -> 256 granule
    assert fa.fa_bwd_workspace_size(1, 3, 2, 16, 64) == 0            # Hq % Hkv != 0
    assert fa.fa_bwd_workspace_size(1, 2, 2, 16, 80) == 0            # unsupported d


def test_no_device_reports_hip_error():
    """A valid request with no GPU present fails at the launch, not in the checks."""
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert fwd() == fa.FA_ERR_HIP
    assert fwd(d=256) == fa.FA_ERR_HIP          # the forward accepts d = 256
    assert kvc(d=256) == fa.FA_ERR_HIP


def kvc(**kw):
    a = dict(q=P, k=P, v=P, lens=P, o=P, lse=P, B=2, Hq=4, Hkv=2, Nq=1, Nk=64, d=128,
             scale=0.125, causal=1, splits=2, dtype=fa.FA_BF16, ws=P, wsb=1 << 20)
    a.update(kw)
    return fa.fa_fwd_kvcache(a["q"], a["k"], a["v"], a["lens"], a["o"], a["lse"], a["B"], a["Hq"],
                             a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"],
                             a["splits"], a["dtype"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=5), fa.FA_ERR_INVALID_ARG),
    (dict(Hq=3), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=-1), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=-1), fa.FA_ERR_INVALID_ARG),
    (dict(splits=-1), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=512), fa.FA_ERR_UNSUPPORTED),
    (dict(lens=None), fa.FA_ERR_INVALID_ARG),
    (dict(q=P + 8), fa.FA_ERR_INVALID_ARG),
    (dict(lens=P + 2), fa.FA_ERR_INVALID_ARG),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(wsb=16), fa.FA_ERR_WORKSPACE),
    (dict(B=0), fa.FA_OK),
    (dict(Nq=0), fa.FA_OK),
])
def test_kvcache_host_checks(kw, status):
    assert kvc(**kw) == status


def test_kvcache_splits_and_workspace():
    # rows per (entry, KV head) = (Hq/Hkv)·Nq = 4 -> one 32-row block; with no device the
    # residency bound is 3 workgroups per CU (48 KiB of LDS each) on 256 CUs: 768 / (16·8) = 6
    assert fa.fa_kvcache_num_splits(16, 32, 8, 1, 8192, 128) == 6
    # at most one range per 256 keys (eight 32-key tiles)
    assert fa.fa_kvcache_num_splits(1, 2, 2, 1, 100, 64) == 1
    assert fa.fa_kvcache_num_splits(1, 2, 2, 1, 4096, 64) == 16
    assert fa.fa_kvcache_num_splits(1, 2, 2, 1, 4097, 64) == 17
    assert fa.fa_kvcache_num_splits(1, 2, 2, 1, 0, 64) == 1
    assert fa.fa_kvcache_num_splits(1, 3, 2, 1, 64, 64) == 0
    assert fa.fa_fwd_kvcache_workspace_size(2, 4, 2, 3, 64, 128, 5) == (5 * 2 * 4 * 3 * 129 * 4 + 255) // 256 * 256
    # num_splits = 0: the larger automatic count (6 for both caches here)
    assert fa.fa_fwd_kvcache_workspace_size(16, 32, 8, 1, 8192, 128, 0) == 6 * 16 * 32 * 129 * 4
    assert fa.fa_fwd_kvcache_workspace_size(1, 2, 2, 1, 64, 80, 1) == 0


def test_kvcache_stage_index_checked():
    assert fa.fa_fwd_kvcache_num_stages() == 2
    for stage in (-1, 2):
        assert fa.fa_fwd_kvcache_stage(stage, P, P, P, P, P, P, 2, 4, 2, 1, 64, 128, 0.125, 1, 2,
                                       fa.FA_BF16, P, 1 << 20, None) == fa.FA_ERR_INVALID_ARG
    # a valid stage still runs the host checks first
    assert fa.fa_fwd_kvcache_stage(0, P, P, P, P, P, P, 2, 4, 2, 1, 64, 96, 0.125, 1, 2,
                                   fa.FA_BF16, P, 1 << 20, None) == fa.FA_ERR_UNSUPPORTED


def fkv(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, Hq=4, Hkv=2, Nq=100, Nk=300, d=128, scale=0.125,
             causal=1, cq=None, ck=None, dtype=fa.FA_BF16)
    a.update(kw)
    return fa.fa_fwd_kvlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                           a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"], a["cq"], a["ck"],
                           a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(cq=P), fa.FA_ERR_INVALID_ARG),             # one cu_seqlens without the other
    (dict(ck=P), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=-1), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=-1), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=7), fa.FA_ERR_INVALID_ARG),
    (dict(Hq=3), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(k=None), fa.FA_ERR_INVALID_ARG),           # keys to read but no pointer
    (dict(v=P + 8), fa.FA_ERR_INVALID_ARG),
    (dict(B=1 << 20, Nk=1 << 12), fa.FA_ERR_UNSUPPORTED),
    (dict(B=0), fa.FA_OK),
    (dict(Nq=0), fa.FA_OK),
])
def test_fwd_kvlen_host_checks(kw, status):
    assert fkv(**kw) == status


def test_fwd_kvlen_no_device_reports_hip_error():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert fkv() == fa.FA_ERR_HIP
    assert fkv(Nk=0, k=None, v=None) == fa.FA_ERR_HIP   # no key: k, v may be NULL
    assert fkv(d=256, causal=0, cq=P, ck=P) == fa.FA_ERR_HIP


def kvcl(**kw):
    a = dict(q=P, k=P, v=P, lens=P, o=P, lse=P, B=2, Hq=4, Hkv=2, Nq=1, Nk=64, d=128,
             scale=0.125, causal=1, wl=16, cap=30.0, splits=2, dtype=fa.FA_BF16, ws=P,
             wsb=1 << 20)
    a.update(kw)
    return fa.fa_fwd_kvcache_local(a["q"], a["k"], a["v"], a["lens"], a["o"], a["lse"], a["B"],
                                   a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"],
                                   a["causal"], a["wl"], a["cap"], a["splits"], a["dtype"],
                                   a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(wl=-2), fa.FA_ERR_INVALID_ARG),
    (dict(cap=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(cap=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(cap=1e-45, scale=1.0), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=4), fa.FA_ERR_INVALID_ARG),
    (dict(lens=None), fa.FA_ERR_INVALID_ARG),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(B=0), fa.FA_OK),
])
def test_kvcache_local_host_checks(kw, status):
    assert kvcl(**kw) == status


def test_kvcache_local_no_device_reports_hip_error():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert kvcl() == fa.FA_ERR_HIP
    assert kvcl(wl=-1, cap=0.0, d=256, causal=0) == fa.FA_ERR_HIP


def kvc8(stage=None, **kw):
    a = dict(q=P, k=P, v=P, lens=P, o=P, lse=P, B=2, Hq=4, Hkv=2, Nq=1, Nk=64, d=128,
             scale=0.125, causal=1, dk=0.01, dv=0.02, splits=2, dtype=fa.FA_BF16, ws=P,
             wsb=1 << 20)
    a.update(kw)
    args = (a["q"], a["k"], a["v"], a["lens"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
            a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"], a["dk"], a["dv"], a["splits"],
            a["dtype"], a["ws"], a["wsb"], None)
    if stage is None:
        return fa.fa_fwd_kvcache_fp8(*args)
    return fa.fa_fwd_kvcache_fp8_stage(stage, *args)


@pytest.mark.parametrize("kw,status", [
    (dict(dk=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(dv=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(dk=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(dv=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(dk=1e38, scale=100.0), fa.FA_ERR_INVALID_ARG),   # scale·descale_k overflows
    (dict(dtype=5), fa.FA_ERR_INVALID_ARG),
    (dict(Hq=3), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(lens=None), fa.FA_ERR_INVALID_ARG),
    (dict(k=P + 8), fa.FA_ERR_INVALID_ARG),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(B=0), fa.FA_OK),
    (dict(B=0, dk=0.0), fa.FA_ERR_INVALID_ARG),
])
def test_kvcache_fp8_host_checks(kw, status):
    assert kvc8(**kw) == status


def test_kvcache_fp8_splits():
    # half the LDS per workgroup: 6 resident per CU; the e4m3 count takes half of
    # them, rounded up: 768 / (16·8) = 6 ranges (and ceil(768 / 512) = 2 for 64 entries)
    assert fa.fa_kvcache_fp8_num_splits(16, 32, 8, 1, 8192, 128) == 6
    assert fa.fa_kvcache_fp8_num_splits(64, 32, 8, 1, 2048, 128) == 2
    # d = 256 keeps the full round: 2 resident per CU (registers), 512 / (16·8) = 4 ranges
    assert fa.fa_kvcache_fp8_num_splits(16, 32, 8, 1, 8192, 256) == 4
    for shape in [(16, 32, 8, 1, 8192, 128), (1, 2, 2, 1, 100, 64), (1, 8, 1, 1, 40000, 256),
                  (3, 12, 4, 5, 777, 64), (64, 8, 8, 1, 1 << 20, 128), (4, 32, 8, 4, 4096, 128)]:
        n8, n16 = fa.fa_kvcache_fp8_num_splits(*shape), fa.fa_kvcache_num_splits(*shape)
        assert n8 >= n16 >= 1, shape
        ws = fa.fa_fwd_kvcache_workspace_size(*shape, 0)
        assert ws == fa.fa_fwd_kvcache_workspace_size(*shape, n8), shape
    assert fa.fa_kvcache_fp8_num_splits(1, 3, 2, 1, 64, 64) == 0


def test_kvcache_fp8_stage_index_checked():
    for stage in (-1, 2):
        assert kvc8(stage=stage) == fa.FA_ERR_INVALID_ARG
    assert kvc8(stage=0, d=96) == fa.FA_ERR_UNSUPPORTED


def test_kvcache_fp8_no_device_reports_hip_error():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert kvc8() == fa.FA_ERR_HIP
    assert kvc8(d=64, dtype=fa.FA_FP16, causal=0) == fa.FA_ERR_HIP
    assert kvc8(stage=1, d=256) == fa.FA_ERR_HIP


def fwdw(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=2, N=16, d=64, scale=0.125, wl=3, wr=0,
             cu=None, dtype=fa.FA_FP16, stream=None)
    a.update(kw)
    return fa.fa_fwd_window(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                            a["N"], a["d"], a["scale"], a["wl"], a["wr"], a["cu"], a["dtype"],
                            a["stream"])


def bwdw(stage=None, **kw):
    a = dict(B=1, Hq=2, Hkv=2, N=16, d=64, scale=0.125, wl=3, wr=2, dtype=fa.FA_BF16, ws=P,
             wsb=1 << 20)
    a.update(kw)
    ptrs = [kw.get(n, P) for n in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv")]
    args = (*ptrs, a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["scale"], a["wl"], a["wr"], None,
            a["dtype"], a["ws"], a["wsb"], None)
    if stage is None:
        return fa.fa_bwd_window(*args)
    return fa.fa_bwd_window_stage(stage, *args)


@pytest.mark.parametrize("kw,status", [
    (dict(wl=-2), fa.FA_ERR_INVALID_ARG),
    (dict(wr=-7), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=3), fa.FA_ERR_INVALID_ARG),
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(v=P + 4), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(B=1, Hq=1, Hkv=1, N=1 << 30), fa.FA_ERR_UNSUPPORTED),   # window arithmetic bound
    # the causal band runs the causal kernels, no window arithmetic: it reaches the launch
    (dict(B=1, Hq=1, Hkv=1, N=1 << 30, wl=-1, wr=0), None),
    (dict(B=0), fa.FA_OK),
])
def test_fwd_window_host_checks(kw, status):
    if status is None:
        torch = pytest.importorskip("torch")
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
        assert fwdw(**kw) == fa.FA_ERR_HIP
        return
    assert fwdw(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(wl=-3), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(dk=P + 8), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_OK),
])
def test_bwd_window_host_checks(kw, status):
    assert bwdw(**kw) == status


def test_bwd_window_stage_index_checked():
    for bad in (-2, 3, 9):
        assert bwdw(stage=bad) == fa.FA_ERR_INVALID_ARG
    assert bwdw(stage=1, ws=None) == fa.FA_ERR_WORKSPACE   # a valid stage runs the checks


def test_window_no_device_reports_hip_error():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert fwdw() == fa.FA_ERR_HIP
    assert fwdw(d=256, wl=5, wr=5) == fa.FA_ERR_HIP
    assert bwdw() == fa.FA_ERR_HIP


def fwd8(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=2, N=16, d=128, scale=0.125, causal=0,
             cu=None, dq=0.01, dk=0.02, dv=0.5, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.fa_fwd_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                         a["N"], a["d"], a["scale"], a["causal"], a["cu"], a["dq"], a["dk"],
                         a["dv"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dq=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(dk=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(dv=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(dv=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(dq=1e30, dk=1e30), fa.FA_ERR_INVALID_ARG),     # scale·dq·dk overflows
    (dict(dtype=2), fa.FA_ERR_INVALID_ARG),
    (dict(causal=3), fa.FA_ERR_INVALID_ARG),
    (dict(Hq=3, Hkv=2), fa.FA_ERR_INVALID_ARG),
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(k=P + 8), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=512), fa.FA_ERR_UNSUPPORTED),
    (dict(B=0), fa.FA_OK),
    (dict(N=0, q=None), fa.FA_OK),
])
def test_fwd_fp8_host_checks(kw, status):
    assert fwd8(**kw) == status


def test_fwd_fp8_no_device_reports_hip_error():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert fwd8() == fa.FA_ERR_HIP
    assert fwd8(causal=1, dtype=fa.FA_FP16) == fa.FA_ERR_HIP
    assert fwd8(d=64) == fa.FA_ERR_HIP and fwd8(d=256) == fa.FA_ERR_HIP


def fwdc(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=2, N=16, d=64, scale=0.125, causal=1,
             cap=30.0, cu=None, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.fa_fwd_softcap(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                             a["N"], a["d"], a["scale"], a["causal"], a["cap"], a["cu"],
                             a["dtype"], a["stream"])


def bwdc(stage=None, **kw):
    a = dict(B=1, Hq=2, Hkv=2, N=16, d=64, scale=0.125, causal=0, cap=30.0, dtype=fa.FA_FP16,
             ws=P, wsb=1 << 20)
    a.update(kw)
    ptrs = [kw.get(n, P) for n in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv")]
    args = (*ptrs, a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["scale"], a["causal"], a["cap"],
            None, a["dtype"], a["ws"], a["wsb"], None)
    if stage is None:
        return fa.fa_bwd_softcap(*args)
    return fa.fa_bwd_softcap_stage(stage, *args)


@pytest.mark.parametrize("kw,status", [
    (dict(cap=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(cap=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(cap=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(cap=1e-45, scale=1.0), fa.FA_ERR_INVALID_ARG),    # scale / cap overflows
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=7), fa.FA_ERR_INVALID_ARG),
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=P + 2), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(B=0), fa.FA_OK),
    (dict(N=0, cap=5.0), fa.FA_OK),
])
def test_fwd_softcap_host_checks(kw, status):
    assert fwdc(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(cap=-2.0), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(dq=P + 8), fa.FA_ERR_INVALID_ARG),
    (dict(causal=5), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_OK),
])
def test_bwd_softcap_host_checks(kw, status):
    assert bwdc(**kw) == status


def test_bwd_softcap_stage_index_checked():
    for bad in (-2, 3):
        assert bwdc(stage=bad) == fa.FA_ERR_INVALID_ARG
    assert bwdc(stage=2, ws=None) == fa.FA_ERR_WORKSPACE


def test_softcap_no_device_reports_hip_error():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert fwdc() == fa.FA_ERR_HIP
    assert fwdc(cap=0.0) == fa.FA_ERR_HIP      # no cap: the plain kernels
    assert bwdc() == fa.FA_ERR_HIP
    assert fwdc(d=256) == fa.FA_ERR_HIP        # soft cap at d = 256 (fwd and bwd)
    assert bwdc(d=256) == fa.FA_ERR_HIP


def fwdwc(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=2, N=16, d=64, scale=0.125, wl=3, wr=0,
             cap=20.0, cu=None, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.lib.fa_fwd_window_softcap(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"],
                                        a["Hkv"], a["N"], a["d"], a["scale"], a["wl"], a["wr"],
                                        a["cap"], a["cu"], a["dtype"], a["stream"])


def bwdwc(stage=None, **kw):
    a = dict(B=1, Hq=2, Hkv=2, N=16, d=64, scale=0.125, wl=3, wr=2, cap=20.0, dtype=fa.FA_BF16,
             ws=P, wsb=1 << 20)
    a.update(kw)
    ptrs = [kw.get(n, P) for n in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv")]
    args = (*ptrs, a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["scale"], a["wl"], a["wr"],
            a["cap"], None, a["dtype"], a["ws"], a["wsb"], None)
    if stage is None:
        return fa.lib.fa_bwd_window_softcap(*args)
    return fa.lib.fa_bwd_window_softcap_stage(stage, *args)


@pytest.mark.parametrize("kw,status", [
    (dict(cap=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(cap=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(wl=-2), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_OK),
])
def test_fwd_window_softcap_host_checks(kw, status):
    assert fwdwc(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(cap=0.0, wr=-5), fa.FA_ERR_INVALID_ARG),
    (dict(cap=-3.0), fa.FA_ERR_INVALID_ARG),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(B=0), fa.FA_OK),
])
def test_bwd_window_softcap_host_checks(kw, status):
    assert bwdwc(**kw) == status


def test_window_softcap_stage_and_no_device():
    for bad in (-2, 3):
        assert bwdwc(stage=bad) == fa.FA_ERR_INVALID_ARG
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert fwdwc() == fa.FA_ERR_HIP
    assert fwdwc(d=256) == fa.FA_ERR_HIP
    assert bwdwc() == fa.FA_ERR_HIP
    assert bwdwc(d=256, stage=1) == fa.FA_ERR_HIP


def fwdd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=2, N=16, d=64, scale=0.125, causal=0,
             p=0.1, seed=1234, cu=None, dtype=fa.FA_FP16, stream=None)
    a.update(kw)
    return fa.fa_fwd_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                             a["N"], a["d"], a["scale"], a["causal"], a["p"], a["seed"], a["cu"],
                             a["dtype"], a["stream"])


def bwdd(stage=None, **kw):
    a = dict(B=1, Hq=2, Hkv=2, N=16, d=128, scale=0.125, causal=1, p=0.2, seed=2 ** 63 + 5,
             dtype=fa.FA_BF16, ws=P, wsb=1 << 20)
    a.update(kw)
    ptrs = [kw.get(n, P) for n in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv")]
    args = (*ptrs, a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["scale"], a["causal"], a["p"],
            a["seed"], None, a["dtype"], a["ws"], a["wsb"], None)
    if stage is None:
        return fa.fa_bwd_dropout(*args)
    return fa.fa_bwd_dropout_stage(stage, *args)


@pytest.mark.parametrize("kw,status", [
    (dict(p=-0.1), fa.FA_ERR_INVALID_ARG),
    (dict(p=1.0), fa.FA_ERR_INVALID_ARG),
    (dict(p=0.999), fa.FA_ERR_INVALID_ARG),    # no weight kept: t = 0
    (dict(p=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(v=None), fa.FA_ERR_INVALID_ARG),
    (dict(lse=P + 4), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(B=0), fa.FA_OK),
    (dict(N=0, p=0.5), fa.FA_OK),
])
def test_fwd_dropout_host_checks(kw, status):
    assert fwdd(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(p=1.5), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(dv=P + 8), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_OK),
])
def test_bwd_dropout_host_checks(kw, status):
    assert bwdd(**kw) == status


def test_bwd_dropout_stage_index_checked():
    for bad in (-2, 3):
        assert bwdd(stage=bad) == fa.FA_ERR_INVALID_ARG
    assert bwdd(stage=0, ws=None) == fa.FA_ERR_WORKSPACE


def test_dropout_no_device_reports_hip_error():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert fwdd() == fa.FA_ERR_HIP
    assert fwdd(p=0.0) == fa.FA_ERR_HIP       # no dropout: the plain kernels
    assert bwdd() == fa.FA_ERR_HIP


def test_binding_dropout_needs_a_seed():
    torch = pytest.importorskip("torch")
    q = torch.zeros((1, 4, 2, 64), dtype=torch.float16)
    with pytest.raises(ValueError):
        fa._dropout_args(0.1, None, None, 0.0)
    with pytest.raises(NotImplementedError):
        fa._dropout_args(0.1, 3, (5, 0), 0.0)
    assert fa._dropout_args(0.0, None, None, 0.0) is None
    assert fa._dropout_args(0.25, 7, None, 0.0) == (0.25, 7)
    del q


def test_bwd_d256_reaches_the_launch():
    """The plain, windowed, soft-capped and dropout backward accept d = 256."""
    torch = pytest.importorskip("torch")
    assert fa.fa_bwd_workspace_size(1, 2, 2, 16, 256) == fa.fa_bwd_workspace_size(1, 2, 2, 16, 64)
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert bwd(d=256) == fa.FA_ERR_HIP
    assert bwd(d=256, causal=1) == fa.FA_ERR_HIP
    assert bwdw(d=256) == fa.FA_ERR_HIP


def _bwd_tensors(dtype="bf16", T=8, Hq=2, Hkv=1, d=64):
    import torch
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    q = torch.zeros(1, T, Hq, d, dtype=dt)
    k = torch.zeros(1, T, Hkv, d, dtype=dt)
    return dict(dout=q.clone(), q=q, k=k, v=k.clone(), o=q.clone(),
                lse=torch.zeros(Hq, T, dtype=torch.float32))


@pytest.mark.parametrize("bad", ["dout_dtype", "o_dtype", "dout_shape", "lse_dtype", "lse_shape",
                                 "v_shape", "k_dtype"])
def test_binding_backward_rejects_bad_tensors(bad):
    """flash_attn_backward checks every tensor's dtype and shape before it looks
    at devices or launches anything (these are CPU tensors: a launch would fail)."""
    import torch
    t = _bwd_tensors()
    if bad == "dout_dtype":
        t["dout"] = t["dout"].float()
    elif bad == "o_dtype":
        t["o"] = t["o"].half()
    elif bad == "dout_shape":
        t["dout"] = t["dout"][:, :4]
    elif bad == "lse_dtype":
        t["lse"] = t["lse"].double()
    elif bad == "lse_shape":
        t["lse"] = t["lse"][:, :4]
    elif bad == "v_shape":
        t["v"] = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    elif bad == "k_dtype":
        t["k"] = t["k"].half()
    with pytest.raises((TypeError, ValueError)):
        fa.flash_attn_backward(t["dout"], t["q"], t["k"], t["v"], t["o"], t["lse"], causal=True)


def test_binding_forward_rejects_mixed_dtypes_and_shapes():
    import torch
    q = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        fa.flash_attn_func(q, q.half(), q)
    with pytest.raises(ValueError):
        fa.flash_attn_func(q, q, q[:, :4])


def test_bwd_noalloc_host_checks():
    """fa_bwd_noalloc refuses sizes its fixed scratch cannot hold (FA_ERR_WORKSPACE)
    and bad arguments before it touches a device; without a device a valid call
    reports FA_ERR_HIP (the scratch address cannot be looked up)."""
    lim = 32 << 20
    args = lambda B, Hq, N, **kw: [P] * 9 + [B, Hq, kw.get("Hkv", 1), N, kw.get("d", 64),
                                             kw.get("scale", 0.125), kw.get("causal", 1),
                                             None, kw.get("dtype", fa.FA_BF16), None]
    assert fa.fa_bwd_workspace_size(1, 1, 1, lim // 8 - 64, 64) <= lim
    assert fa.fa_bwd_noalloc(*args(1, 1, lim // 8 - 64)) == fa.FA_ERR_HIP
    assert fa.fa_bwd_noalloc(*args(1, 1, lim // 8)) == fa.FA_ERR_WORKSPACE
    assert fa.fa_bwd_noalloc(*args(2, 32, 65536)) == fa.FA_ERR_WORKSPACE
    assert fa.fa_bwd_noalloc(*args(1, 2, 16, causal=2)) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_noalloc(*args(1, 2, 16, dtype=5)) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_noalloc(*args(1, 3, 16, Hkv=2)) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_noalloc(*args(1, 2, 16, d=96)) == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_bwd_noalloc(*args(0, 2, 16)) == fa.FA_OK


def bkv(stage=None, **kw):
    a = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, B=2, Hq=4, Hkv=2, Nq=16, Nk=40,
             d=128, scale=0.088, causal=1, cq=None, ck=None, dtype=fa.FA_BF16, ws=P,
             wsb=1 << 20, stream=None)
    a.update(kw)
    args = [a[n] for n in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "B", "Hq", "Hkv",
                           "Nq", "Nk", "d", "scale", "causal", "cq", "ck", "dtype", "ws", "wsb",
                           "stream")]
    return fa.fa_bwd_kvlen(*args) if stage is None else fa.fa_bwd_kvlen_stage(stage, *args)


@pytest.mark.parametrize("kw,status", [
    (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=-1), fa.FA_ERR_INVALID_ARG),
    (dict(Hq=3), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=7), fa.FA_ERR_INVALID_ARG),
    (dict(cq=P), fa.FA_ERR_INVALID_ARG),
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(dk=None), fa.FA_ERR_INVALID_ARG),
    (dict(dv=P + 8), fa.FA_ERR_INVALID_ARG),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(wsb=64), fa.FA_ERR_WORKSPACE),
    (dict(B=0), fa.FA_OK),
    (dict(Nq=0, Nk=0), fa.FA_OK),
    (dict(Nq=0, q=None, o=None, do=None, lse=None, dq=None), fa.FA_ERR_HIP),
    (dict(Nk=0, k=None, v=None, dk=None, dv=None), fa.FA_ERR_HIP),
    (dict(), fa.FA_ERR_HIP),
])
def test_bwd_kvlen_host_checks(kw, status):
    """Bad arguments are refused on the host; valid ones (here with no device)
    reach the launch and report FA_ERR_HIP. With no query or no key the
    pointers of the empty side may be NULL."""
    assert bkv(**kw) == status


def test_bwd_kvlen_stage_index_checked():
    assert bkv(stage=3) == fa.FA_ERR_INVALID_ARG
    assert bkv(stage=-1) == fa.FA_ERR_INVALID_ARG
    assert bkv(stage=1) == fa.FA_ERR_HIP


def _cu_check(values, B, N):
    import numpy as np
    a = np.ascontiguousarray(np.asarray(values, dtype=np.int32))
    return fa.fa_check_cu_seqlens(a.ctypes.data if a.size else None, B, N)


@pytest.mark.parametrize("values,B,N,ok", [
    ([0], 0, 0, True),
    ([0, 5], 1, 5, True),
    ([0, 5], 1, 4, False),            # a sequence longer than N
    ([1, 5], 1, 8, False),            # first entry not 0
    ([0, 5, 3], 2, 8, False),         # decreasing
    ([0, 0, 0, 7], 3, 7, True),       # empty sequences
    ([0, 2**31 - 1], 1, 2**31 - 1, True),
    ([0, 2**31 - 1, -2**31], 2, 2**31 - 1, False),   # no wrap-around
])
def test_check_cu_seqlens_cases(values, B, N, ok):
    assert _cu_check(values, B, N) == (fa.FA_OK if ok else fa.FA_ERR_INVALID_ARG)


def test_check_cu_seqlens_bad_arguments():
    assert fa.fa_check_cu_seqlens(None, 1, 4) == fa.FA_ERR_INVALID_ARG
    assert _cu_check([0, 1], -1, 4) == fa.FA_ERR_INVALID_ARG
    assert _cu_check([0, 1], 1, -1) == fa.FA_ERR_INVALID_ARG


def test_check_cu_seqlens_random_against_brute_force():
    """Random arrays, half with one entry nudged: the library agrees with the
    packing convention checked length by length in Python."""
    import numpy as np
    rng = np.random.default_rng(7)
    for _ in range(500):
        B, N = int(rng.integers(0, 30)), int(rng.integers(0, 200))
        v = np.zeros(B + 1, dtype=np.int64)
        v[1:] = np.cumsum(rng.integers(0, N + 1, size=B))
        if B and rng.random() < 0.5:
            v[rng.integers(0, B + 1)] += int(rng.integers(-3, 4))
        ok = v[0] == 0 and all(0 <= v[s + 1] - v[s] <= N for s in range(B))
        assert _cu_check(v, B, N) == (fa.FA_OK if ok else fa.FA_ERR_INVALID_ARG), (v, N)


def test_library_exports_exactly_the_header():
    """The library's exported functions are the header's declarations and
    nothing else (host symbols are hidden; the C ABI is the whole interface)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm (binutils) is not installed")
    out = subprocess.run([nm, "-D", "--defined-only", fa.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    funcs = sorted(line.split()[-1] for line in out.splitlines()
                   if len(line.split()) == 3 and line.split()[1] == "T")
    assert funcs == declared_functions()


# ---- fa_fwd_ex / fa_bwd_ex: the options struct ----------------------------------

def test_attn_options_layout():
    """The ctypes mirror has the C layout the library asserts at compile time."""
    import ctypes
    O = fa.FaAttnOptions
    assert ctypes.sizeof(O) == 40
    assert (O.mask.offset, O.window_left.offset, O.softcap.offset, O.dropout_p.offset,
            O.dropout_seed.offset) == (8, 12, 20, 24, 32)


def fwd_ex(opts, **kw):
    import ctypes
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=2, N=16, d=64, scale=0.125,
             dtype=fa.FA_FP16)
    a.update(kw)
    ptr = None if opts is None else ctypes.addressof(opts)
    return fa.fa_fwd_ex(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                        a["N"], a["d"], a["scale"], ptr, None, a["dtype"], None)


def bwd_ex(opts, **kw):
    import ctypes
    a = dict(B=1, Hq=2, Hkv=2, N=16, d=64, scale=0.125, dtype=fa.FA_BF16, ws=P, wsb=1 << 20)
    a.update(kw)
    ptrs = [kw.get(n, P) for n in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv")]
    ptr = None if opts is None else ctypes.addressof(opts)
    return fa.fa_bwd_ex(*ptrs, a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["scale"], ptr, None,
                        a["dtype"], a["ws"], a["wsb"], None)


def _short_struct():
    o = fa.attn_options()
    o.struct_size = 32
    return o


@pytest.mark.parametrize("opts,kw,status", [
    (None, {}, fa.FA_ERR_INVALID_ARG),                                            # NULL options
    ("short", {}, fa.FA_ERR_INVALID_ARG),                                         # struct too small
    (dict(mask=3), {}, fa.FA_ERR_INVALID_ARG),                                    # no such mask
    (dict(mask=-1), {}, fa.FA_ERR_INVALID_ARG),
    (dict(mask=fa.FA_MASK_WINDOW, dropout_p=0.1), {}, fa.FA_ERR_UNSUPPORTED),    # no kernel has both
    (dict(softcap=5.0, dropout_p=0.1), {}, fa.FA_ERR_UNSUPPORTED),
    (dict(mask=fa.FA_MASK_WINDOW, window=(-2, 0)), {}, fa.FA_ERR_INVALID_ARG),   # fa_fwd_window's check
    (dict(softcap=-1.0), {}, fa.FA_ERR_INVALID_ARG),                              # fa_fwd_softcap's check
    (dict(softcap=float("nan")), {}, fa.FA_ERR_INVALID_ARG),
    (dict(dropout_p=1.5), {}, fa.FA_ERR_INVALID_ARG),                             # fa_fwd_dropout's check
    (dict(mask=fa.FA_MASK_CAUSAL), dict(dtype=7), fa.FA_ERR_INVALID_ARG),         # fa_fwd's check
    (dict(mask=fa.FA_MASK_CAUSAL), dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(mask=fa.FA_MASK_CAUSAL, softcap=5.0), dict(B=0), fa.FA_OK),             # empty batch
])
def test_ex_host_checks(opts, kw, status):
    o = None if opts is None else _short_struct() if opts == "short" else fa.attn_options(**opts)
    assert fwd_ex(o, **kw) == status
    bkw = {k: v for k, v in kw.items() if k != "dtype"}
    if "dtype" in kw:
        bkw["dtype"] = kw["dtype"]
    assert bwd_ex(o, **bkw) == status


def test_ex_backward_workspace_checked():
    assert bwd_ex(fa.attn_options(mask=fa.FA_MASK_CAUSAL), ws=None) == fa.FA_ERR_WORKSPACE
    assert bwd_ex(fa.attn_options(dropout_p=0.2, dropout_seed=3), wsb=64) == fa.FA_ERR_WORKSPACE


def test_ex_no_device_reports_hip_error():
    """Each route passes its checks and fails only at the launch without a GPU."""
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    for opts in (dict(), dict(mask=fa.FA_MASK_CAUSAL), dict(mask=fa.FA_MASK_WINDOW, window=(8, 0)),
                 dict(softcap=5.0), dict(mask=fa.FA_MASK_WINDOW, window=(8, 8), softcap=5.0),
                 dict(mask=fa.FA_MASK_CAUSAL, dropout_p=0.2, dropout_seed=9)):
        assert fwd_ex(fa.attn_options(**opts)) == fa.FA_ERR_HIP, opts
        assert bwd_ex(fa.attn_options(**opts)) == fa.FA_ERR_HIP, opts
