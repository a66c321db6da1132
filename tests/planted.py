"""Planting mistakes in the oracle and checking that its pins catch each one (CPU only).

A code mistake replaces one piece of text inside one function of a copy of the oracle's C
source; the copy is built with gcc and the oracle loads it through MPGEMM_ORACLE_LIB.  A
parameter mistake is a Python statement run before the pins.  Each mistake runs the pin files
named for it in a child pytest process; the children run side by side, OpenMP held to one
thread each."""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mpgemm_oracle.c")


def plant(src: str, fn: str, old: str, new: str) -> str:
    """src with the first `old` inside function `fn` (from its header to its closing brace)
    replaced by `new`."""
    start = src.index(fn)
    end = src.index("\n}\n", start)
    pos = src.index(old, start)
    assert pos + len(old) <= end, f"the planted text must lie inside {fn}"
    return src[:pos] + new + src[pos + len(old):]


def pins_fail(files, lib=None, prelude="", lib_var="MPGEMM_ORACLE_LIB", args=()) -> bool:
    """True when at least one pin of `files` fails (and none errors) with the library `lib`
    (None: the built one) named by `lib_var`, after `prelude` has run."""
    env = dict(os.environ, OMP_NUM_THREADS="1")
    if lib is not None:
        env[lib_var] = lib
    code = (prelude + "import sys, pytest\n"
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu'] + "
            f"{list(files) + list(args)!r}))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    return r.returncode == 1 and " failed" in r.stdout


def _build(src: str, path: str) -> str:
    with open(path + ".c", "w") as f:
        f.write(src)
    subprocess.run(["gcc", "-O1", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                    "-fPIC", "-shared", "-o", path + ".so", path + ".c", "-lm"], check=True)
    return path + ".so"


def survivors(code: dict, params: dict, param_prelude) -> list:
    """Names of the mistakes no pin catches.  code: name -> (function, old, new, pin files);
    params: name -> (keyword arguments, pin files); param_prelude(kwargs) -> Python source."""
    src = open(SRC).read()
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with tempfile.TemporaryDirectory() as tmp, ThreadPoolExecutor(workers) as pool:
        def one_code(item):
            t, (name, (fn, old, new, files)) = item
            lib = _build(plant(src, fn, old, new), os.path.join(tmp, f"m{t}"))
            return name, pins_fail(files, lib=lib)

        def one_param(item):
            name, (kw, files) = item
            return name, pins_fail(files, prelude=param_prelude(kw))

        results = list(pool.map(one_code, enumerate(sorted(code.items()))))
        results += list(pool.map(one_param, sorted(params.items())))
    return [name for name, caught in results if not caught]


HOST_SRC = os.path.join(ROOT, "mixed_precision_dense_amd", "csrc", "mpgemm_host.cpp")


def host_survivors(code: dict, files, args=()) -> list:
    """Names of the mistakes in the library's host-only argument checks (mpgemm_host.cpp,
    built alone with g++ and loaded through MPGEMM_HOST_CHECK_LIB) that no test of `files`
    catches.  code: name -> (function, old, new)."""
    src = open(HOST_SRC).read()
    csrc = os.path.dirname(HOST_SRC)
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with tempfile.TemporaryDirectory() as tmp, ThreadPoolExecutor(workers) as pool:
        def one(item):
            t, (name, (fn, old, new)) = item
            path = os.path.join(tmp, f"h{t}")
            with open(path + ".cpp", "w") as f:
                f.write(plant(src, fn, old, new))
            subprocess.run(["g++", "-std=c++17", "-fPIC", "-shared", "-O1",
                            "-I" + os.path.join(ROOT, "include"), "-I" + csrc, "-o",
                            path + ".so", path + ".cpp"], check=True)
            return name, pins_fail(files, lib=path + ".so", lib_var="MPGEMM_HOST_CHECK_LIB",
                                   args=args)

        results = list(pool.map(one, enumerate(sorted(code.items()))))
    return [name for name, caught in results if not caught]
