"""Device code built with the library's own flags (CPU only, hipcc cross-compiles
for gfx950): no packed-fp32 VALU forms anywhere, and every kernel within the
register budget without scratch spills."""
import glob
import importlib.util
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_22_amd", "csrc")


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "_pa_build_isa", os.path.join(ROOT, "paged_kv_cache_22_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    B = _build_module()
    try:
        hipcc = B._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa")
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def one(src):
        dst = os.path.join(out, os.path.basename(src) + ".s")
        p = subprocess.run([hipcc, *B.flags_for(os.path.basename(src)), "--cuda-device-only", "-S",
                            src, "-o", dst],
                           capture_output=True, text=True)
        assert p.returncode == 0, p.stderr[-2000:]
        return os.path.basename(src), open(dst).read()

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        return dict(ex.map(one, srcs))


def test_no_packed_fp32_valu(device_asm):
    pat = re.compile(r"^\s*v_pk_(add|mul|fma)_f32\b", re.M)
    for name, text in device_asm.items():
        hits = pat.findall(text)
        assert not hits, f"{name}: {len(hits)} packed-fp32 instructions"


def test_no_scratch_spills(device_asm):
    for name, text in device_asm.items():
        sizes = re.findall(r"\.amdhsa_private_segment_fixed_size\s+(\d+)", text)
        with open(os.path.join(CSRC, name)) as f:
            has_kernels = "__global__" in f.read()   # (or from the headers it includes)
        assert sizes or not has_kernels, f"{name}: no kernel descriptors"
        assert all(int(x) == 0 for x in sizes), f"{name}: a kernel uses scratch ({sizes})"


def test_copy_bases_not_sign_extended(device_asm):
    """The prefill kernel's global-to-LDS copies take a 64-bit scalar base
    assembled from two uniform 32-bit halves; widening the low half as a
    signed value (s_bfe_i64 of the low word) would put 0xffffffff in the high
    word of every address whose low word has bit 31 set."""
    text = device_asm["prefill.hip"]
    assert "global_load_lds_dwordx4" in text
    assert not re.search(r"^\s*s_bfe_i64\b", text, re.M), "sign-extended 64-bit value in prefill"
