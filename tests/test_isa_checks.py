"""Checks on the gfx950 assembly the kernels compile to (test code; CPU only,
hipcc cross-compiles).

* The asynchronous global->LDS copies are inline assembly that set M0 (the
  LDS base of the copy) and issue the copy at once. The compiler treats M0 as
  reserved and does not honour it as a clobber of inline assembly, so the
  copies are safe only while no compiler-generated instruction keeps a value
  in M0. Every reference to M0 in the assembly must therefore be one of the
  copies' own writes, and each write must be followed by its copy before any
  other instruction but a wait state.
* The build disables the packed fp32 VALU forms; none may appear.
"""
import concurrent.futures
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "adaptive_softmax_attention_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ("mala_fwd.hip", "mala_bwd.hip", "mala_bwd_kv.hip", "mala_decode.hip", "mala_api.hip")

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc not available")


def _device_asm(name, tmp):
    from adaptive_softmax_attention_amd import build
    out = os.path.join(tmp, name + ".s")
    flags = [f for f in build.FLAGS if f not in ("-fPIC",)]
    extra = getattr(build, "EXTRA", {}).get(name, [])
    r = subprocess.run([HIPCC, *flags, *extra, "--cuda-device-only", "-S",
                        os.path.join(CSRC, name), "-o", out],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = []
    for line in open(out):
        code = line.split(";")[0].strip()
        if code and not code.startswith(".") and not code.endswith(":"):
            lines.append(code)
    return lines


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("isa"))
    with concurrent.futures.ThreadPoolExecutor(len(SOURCES)) as ex:
        return dict(zip(SOURCES, ex.map(lambda n: _device_asm(n, tmp), SOURCES)))


def test_m0_is_used_only_by_the_async_copies(asm):
    m0 = re.compile(r"\bm0\b")
    copies = 0
    for name, lines in asm.items():
        for k, code in enumerate(lines):
            if not m0.search(code):
                continue
            assert code.startswith("s_mov_b32 m0,"), f"{name}: {code}"
            nxt = [c for c in lines[k + 1:k + 4] if not c.startswith("s_nop")]
            assert nxt and nxt[0].startswith("global_load_lds_"), f"{name}: {code} -> {nxt[:1]}"
            copies += 1
        # and every copy is preceded by its own M0 write
        for k, code in enumerate(lines):
            if code.startswith("global_load_lds_"):
                prev = [c for c in lines[max(0, k - 3):k] if not c.startswith("s_nop")]
                assert prev and prev[-1].startswith("s_mov_b32 m0,"), f"{name}: {code}"
    assert copies > 0


def test_no_packed_fp32_valu(asm):
    packed = re.compile(r"^v_pk_(add|mul|fma)_f32\b")
    for name, lines in asm.items():
        bad = [c for c in lines if packed.match(c)]
        assert not bad, f"{name}: {bad[:3]}"
