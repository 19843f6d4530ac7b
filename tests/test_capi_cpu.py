"""The C ABI seen from plain C: include/xfer.h compiles as C11 with gcc, a C
program links libxfer.so and calls host-only entry points, every struct size
and field offset the C compiler lays out equals the Python binding's ctypes
(and numpy) layout, and every exported call's parameter list in the header
matches the binding's argtypes and restype in count, width and signedness,
so no call reads an argument or a field at the wrong place or width."""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

import bf16_wire_all_amd as x

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "bf16_wire_all_amd")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")

CTYPES = {"xfer_shard": x.Shard, "xfer_run_table": x.RunTableC, "xfer_region": x.Region,
          "xfer_runs_plan": x.RunsPlan, "xfer_descs_plan": x.DescsPlan, "xfer_pages": x.PagesC,
          "xfer_pages_plan": x.PagesPlan, "xfer_op": x.Op, "xfer_allreduce2_desc": x.AllReduce2Desc}
DTYPES = {"xfer_max_idx": x.MAX_IDX, "xfer_top2": x.TOP2_REC, "xfer_desc": x.DESC}


@pytest.fixture(scope="module")
def layout(tmp_path_factory):
    x.lib()                                   # libxfer.so is built
    exe = str(tmp_path_factory.mktemp("capi") / "abi_layout")
    inc = os.environ.get("ROCM_PATH", "/opt/rocm") + "/include"
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", inc, "-I",
           os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "capi", "abi_layout.c"), "-o", exe,
           "-L", LIBDIR, "-lxfer", "-Wl,-rpath," + LIBDIR]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr[-3000:]
    sizes, fields, calls = {}, {}, {}
    for line in r.stdout.splitlines():
        a = line.split()
        if a[0] == "call":
            calls[a[1]] = a[2:]
        elif a[1] == ".":
            sizes[a[0]] = int(a[2])
        else:
            fields.setdefault(a[0], {})[a[1]] = int(a[2])
    return sizes, fields, calls


@pytest.mark.parametrize("name", sorted(CTYPES))
def test_ctypes_layout_matches_c(layout, name):
    sizes, fields, _ = layout
    S = CTYPES[name]
    assert ctypes.sizeof(S) == sizes[name]
    assert [f[0] for f in S._fields_] == list(fields[name])          # same fields, same order
    for f, off in fields[name].items():
        assert getattr(S, f).offset == off, f


@pytest.mark.parametrize("name", sorted(DTYPES))
def test_numpy_record_layout_matches_c(layout, name):
    sizes, fields, _ = layout
    dt = np.dtype(DTYPES[name])
    assert dt.itemsize == sizes[name]
    assert list(dt.names) == list(fields[name])
    for f, off in fields[name].items():
        assert dt.fields[f][1] == off, f


def test_host_calls_from_c_match_python(layout):
    _, _, calls = layout
    st, nr, r0, r1, s0, s1 = calls["runs_encode"]
    t = x.runs_encode(np.array([[0x1000, 0x2000, 0x3000], [0x9000, 0x8000, 0x7000]], np.uint64), 16)
    assert (int(st), int(nr)) == (x.OK, t.n_runs)
    assert (int(r0), int(r1)) == tuple(int(v) for v in t.runs_per_lane)
    assert (int(s0), int(s1)) == (0x1000, -0x1000)                 # one ascending, one descending run
    st, n_ops, kind2, stream2 = (int(v) for v in calls["schedule"])
    ops = x.allreduce2_schedule(3, 2)
    assert (st, n_ops, kind2, stream2) == (x.OK, len(ops), ops[2]["kind"], ops[2]["stream"])
    st, n_deps = (int(v) for v in calls["graph_deps"])
    assert (st, n_deps) == (x.E_RANGE, len(x.allreduce2_graph_deps(3, 2)))
    assert calls["status"] == ["named"]


def _decls():
    """(name, return type, [parameter types]) of every XFER_API declaration."""
    import re
    src = open(os.path.join(ROOT, "include", "xfer.h")).read()
    out = []
    for ret, args in re.findall(r"XFER_API\s+([^;]*?)\s*\(([^)]*)\)\s*;", src, re.S):
        ret = " ".join(ret.split())
        m = re.match(r"(.*?)(\w+)$", ret)
        params = []
        for a in " ".join(args.split()).split(","):
            a = a.strip()
            if a and a != "void":
                params.append(re.match(r"(.*?)\w+$", a).group(1).replace("const ", "").replace(" ", ""))
        out.append((m.group(2), m.group(1).replace("const ", "").replace(" ", ""), params))
    return out


SCALARS = {"int": ctypes.c_int, "uint32_t": ctypes.c_uint32, "uint64_t": ctypes.c_uint64,
           "size_t": ctypes.c_size_t, "int64_t": ctypes.c_int64}
STRUCTS = {"xfer_shard*": x.Shard, "xfer_run_table*": x.RunTableC, "xfer_region*": x.Region,
           "xfer_runs_plan*": x.RunsPlan, "xfer_descs_plan*": x.DescsPlan, "xfer_pages*": x.PagesC,
           "xfer_pages_plan*": x.PagesPlan, "xfer_op*": x.Op, "xfer_allreduce2_desc*": x.AllReduce2Desc}
HANDLES = {"hipStream_t", "hipGraphExec_t"}          # opaque pointers passed by value


def _compatible(c_type, py):
    if c_type in SCALARS:
        return py is SCALARS[c_type]
    if c_type in STRUCTS:
        return py is ctypes.c_void_p or py is ctypes.POINTER(STRUCTS[c_type])
    if c_type == "hipGraphExec_t*":
        return py is ctypes.POINTER(ctypes.c_void_p)
    if c_type.endswith("*") or c_type in HANDLES:
        return py is ctypes.c_void_p or (isinstance(py, type) and issubclass(py, ctypes._Pointer))
    return False


def test_every_exported_signature_matches_the_binding():
    """Argument count, width and signedness of every exported call as the
    binding declares it (ctypes argtypes / restype) equal the header's."""
    L = x.lib()
    decls = _decls()
    assert sorted(d[0] for d in decls) == sorted(x.EXPORTED)
    for name, ret, params in decls:
        fn = getattr(L, name)
        assert len(fn.argtypes) == len(params), name
        for i, (c_type, py) in enumerate(zip(params, fn.argtypes)):
            assert _compatible(c_type, py), (name, i, c_type, py)
        want_ret = {"int": ctypes.c_int, "size_t": ctypes.c_size_t, "uint32_t": ctypes.c_uint32,
                    "char*": ctypes.c_char_p}[ret]
        assert fn.restype is want_ret, (name, ret, fn.restype)
