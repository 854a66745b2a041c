"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle (oracle/oracle.c) and the library's host packers and quantizers
(csrc/pack.cpp with csrc/abi.cpp) are rebuilt with gcc/g++ and
-fsanitize=address,undefined (every UB check fatal), then exercised in a
child process with the sanitizer runtime preloaded:

  * the oracle: the whole CPU pin suite (tests/test_oracle_*.py) runs
    against the sanitized build (TT_ORACLE_LIB), so every oracle function is
    driven through its pinned cases;
  * the host library code: every packer and quantizer on ragged shapes, into
    destination buffers of exactly the queried size (a write past the end
    hits the sanitizer's red zone), plus the error paths that must write
    nothing; the bytes are then compared with the regular build.

Only host code is built here (no GPU code, no hipcc).
"""
import os
import subprocess
import sys
import textwrap

import numpy as np
import pytest

import bit_weight_only_mxfp4_amd as tt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_weight_only_mxfp4_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1", "-fPIC", "-shared"]


def _runtime():
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def san(tmp_path_factory):
    if _runtime() is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    d = tmp_path_factory.mktemp("san")
    lib_oracle = str(d / "liboracle_san.so")
    lib_pack = str(d / "libttpack_san.so")
    subprocess.run(["gcc", "-std=c99", "-ffp-contract=off", *SAN,
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", lib_oracle, "-lm"],
                   check=True)
    subprocess.run(["g++", "-std=c++17", *SAN, os.path.join(CSRC, "pack.cpp"),
                    os.path.join(CSRC, "abi.cpp"), "-o", lib_pack], check=True)
    env = dict(os.environ, LD_PRELOAD=_runtime(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", TT_ORACLE_LIB=lib_oracle)
    return dict(dir=d, oracle=lib_oracle, pack=lib_pack, env=env)


def _clean(proc):
    text = proc.stdout + proc.stderr
    assert "AddressSanitizer" not in text, text[-4000:]
    assert "runtime error:" not in text, text[-4000:]
    assert proc.returncode == 0, text[-4000:]


def test_oracle_pins_under_sanitizers(san):
    tests = sorted(f for f in os.listdir(os.path.join(ROOT, "tests"))
                   if f.startswith("test_oracle_") and f.endswith(".py"))
    proc = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                           *[os.path.join(ROOT, "tests", f) for f in tests]],
                          cwd=ROOT, env=san["env"], capture_output=True, text=True, timeout=900)
    _clean(proc)
    assert " passed" in proc.stdout


_PACK_SCRIPT = textwrap.dedent("""
    import ctypes, sys
    import numpy as np
    L = ctypes.CDLL(sys.argv[1])
    out_dir = sys.argv[2]
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    for name, res, args in (
        ("tt_mxfp4_matrix_pack_bytes", I64, [I64, I64]),
        ("tt_mxfp4_gateup_pack_bytes", I64, [I64, I64]),
        ("tt_pack_mxfp4_matrix", I32, [P, P, P, I64, I64, P, I64]),
        ("tt_pack_mxfp4_gateup", I32, [P, P, P, P, P, P, I64, I64, P, I64]),
        ("tt_quantize_mxfp4", I32, [P, I64, I64, P, P, P]),
        ("tt_quantize_int4_affine", I32, [P, I64, I64, I64, P, P, P]),
        ("tt_int4_pack_bytes", I64, [I64, I64, I64]),
        ("tt_pack_int4", I32, [P, P, P, I64, I64, I64, P, I64]),
        ("tt_fp8_pack_bytes", I64, [I64, I64]),
        ("tt_pack_fp8_matrix", I32, [P, P, I64, I64, P, I64])):
        f = getattr(L, name); f.restype = res; f.argtypes = args
    p = lambda a: None if a is None else a.ctypes.data_as(P)
    gen = np.random.default_rng(0)
    saved = {}

    def exact(nbytes):
        # a fresh heap block of exactly nbytes: one byte past it is a red zone
        return np.empty(nbytes, np.uint8)

    for n, k in ((1, 32), (17, 96), (33, 2880), (16, 256), (5, 4096)):
        c = gen.integers(0, 256, (n, k // 2), dtype=np.uint8)
        s = gen.integers(0, 256, (n, k // 32), dtype=np.uint8)
        ps = gen.uniform(0.5, 1.5, n).astype(np.float32)
        dst = exact(L.tt_mxfp4_matrix_pack_bytes(n, k))
        assert L.tt_pack_mxfp4_matrix(p(c), p(s), p(ps), n, k, p(dst), dst.size) == 0
        saved[f"mx_{n}_{k}"] = dst.copy()
        small = np.full(dst.size - 1, 7, np.uint8)
        assert L.tt_pack_mxfp4_matrix(p(c), p(s), None, n, k, p(small), small.size) == -5
        assert np.all(small == 7)
    for inter, hidden in ((1, 32), (9, 160), (37, 2880)):
        g = [gen.integers(0, 256, (inter, hidden // 2), dtype=np.uint8),
             gen.integers(0, 256, (inter, hidden // 32), dtype=np.uint8),
             gen.uniform(0.5, 1.5, inter).astype(np.float32)]
        u = [a.copy() for a in g]
        dst = exact(L.tt_mxfp4_gateup_pack_bytes(inter, hidden))
        assert L.tt_pack_mxfp4_gateup(*(p(a) for a in g), *(p(a) for a in u), inter, hidden,
                                      p(dst), dst.size) == 0
        saved[f"gu_{inter}_{hidden}"] = dst.copy()
    for n, k in ((1, 32), (3, 96), (7, 2048)):
        w = (gen.standard_normal((n, k)) * 0.02).astype(np.float32)
        w[0, :32] = 0
        codes, scales, ps = exact(n * k // 2), exact(n * k // 32), np.empty(n, np.float32)
        assert L.tt_quantize_mxfp4(p(w), n, k, p(codes), p(scales), p(ps)) == 0
        saved[f"q_{n}_{k}"] = np.concatenate([codes, scales, ps.view(np.uint8)])
        w[n - 1, k - 1] = np.nan
        codes2 = np.full(n * k // 2, 3, np.uint8)
        assert L.tt_quantize_mxfp4(p(w), n, k, p(codes2), p(scales), None) == -6
        assert np.all(codes2 == 3)
    for n, k in ((1, 2), (3, 130), (5, 200), (2, 1000), (16, 5120)):
        w = (gen.standard_normal((n, k)) * 0.02).astype(np.float32)
        w[0, :min(k, 128)] = 0
        G = -(-k // 128)
        q, s, z = exact(n * k // 2), np.empty(n * G, np.uint16), np.empty(n * G, np.uint16)
        assert L.tt_quantize_int4_affine(p(w), n, k, 128, p(q), p(s), p(z)) == 0
        dst = exact(L.tt_int4_pack_bytes(n, k, 128))
        assert L.tt_pack_int4(p(q), p(s), p(z), n, k, 128, p(dst), dst.size) == 0
        saved[f"i4_{n}_{k}"] = dst.copy()
    for n, k in ((1, 8), (9, 200), (17, 1000)):
        c = gen.integers(0, 256, (n, k), dtype=np.uint8)
        sc = gen.uniform(0.5, 1.5, n).astype(np.float32)
        dst = exact(L.tt_fp8_pack_bytes(n, k))
        assert L.tt_pack_fp8_matrix(p(c), p(sc), n, k, p(dst), dst.size) == 0
        saved[f"f8_{n}_{k}"] = dst.copy()
    np.savez(out_dir + "/packed.npz", **saved)
    print("host packers ok")
""")


def test_host_packers_under_sanitizers(san):
    script = san["dir"] / "pack_san.py"
    script.write_text(_PACK_SCRIPT)
    proc = subprocess.run([sys.executable, str(script), san["pack"], str(san["dir"])],
                          env=san["env"], capture_output=True, text=True, timeout=600)
    _clean(proc)
    # the sanitized build wrote the same bytes as the library's own build
    got = np.load(san["dir"] / "packed.npz")
    gen = np.random.default_rng(0)
    for n, k in ((1, 32), (17, 96), (33, 2880), (16, 256), (5, 4096)):
        c = gen.integers(0, 256, (n, k // 2), dtype=np.uint8)
        s = gen.integers(0, 256, (n, k // 32), dtype=np.uint8)
        ps = gen.uniform(0.5, 1.5, n).astype(np.float32)
        assert np.array_equal(got[f"mx_{n}_{k}"], tt.pack_mxfp4_matrix(c, s, ps, n, k))
