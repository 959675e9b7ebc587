"""Checks on the gfx950 code the compiler makes of every kernel (CPU only).

Each HIP source is compiled to device assembly with the library's own flags,
and every kernel in it must have:

* no vector-register spills and no scratch memory (spills to memory would cost
  more than the kernels' whole memory budget);
* no double-precision arithmetic (the path computes in fp32; a stray fp64
  operation, e.g. an integer min/max resolved through a floating overload,
  runs on the vector unit and makes what it feeds non-uniform);
* no waterfall loop around a buffer access, and few v_readfirstlane: a
  buffer resource that the compiler cannot prove uniform is read lane by lane
  and every load or store through it becomes a loop (this once cost the state
  pass 10 % on long segments).
"""
import concurrent.futures as cf
import glob
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "linear_attention_rnn_finch_amd"))

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# a waterfall loop over one resource needs 4 per access; a uniform integer
# division (item / H and the like) takes one
MAX_READFIRSTLANE = 12

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")


def _device_asm(src, out_dir):
    import build_lib
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    flags = [f for f in build_lib.FLAGS if f != "-fPIC"]
    cmd = [HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return open(out).read()


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    out_dir = str(tmp_path_factory.mktemp("asm"))
    sources = sorted(glob.glob(os.path.join(ROOT, "linear_attention_rnn_finch_amd", "csrc", "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        texts = list(ex.map(lambda s: _device_asm(s, out_dir), sources))
    yield dict(zip(map(os.path.basename, sources), texts))
    shutil.rmtree(out_dir, ignore_errors=True)


def _kernels(text):
    """{kernel symbol: (body, metadata dict)} of one device assembly file."""
    bodies = {}
    for m in re.finditer(r"^(_Z\w+):\s*;\s*@", text, re.M):
        end = text.find(".Lfunc_end", m.end())          # the whole kernel, every exit included
        bodies[m.group(1)] = text[m.end():end]
    meta = {}
    for block in re.split(r"\n\s+- \.", text):
        name = re.search(r"\.name:\s+(\S+)", block)
        if name and name.group(1) in bodies:
            meta[name.group(1)] = {k: int(v) for k, v in re.findall(
                r"\.(vgpr_spill_count|sgpr_spill_count|private_segment_fixed_size|vgpr_count):\s+(\d+)", block)}
    return {k: (bodies[k], meta.get(k, {})) for k in bodies}


def test_every_source_has_kernels(assembly):
    with_kernels = [f for f, t in assembly.items() if _kernels(t)]
    for f in ("wkv_chunk.hip", "wkv_decode.hip", "wkv_serial.hip", "wkv_epilogue.hip"):
        assert f in with_kernels


def test_no_spills_no_scratch(assembly):
    bad = []
    for f, text in assembly.items():
        for k, (_, meta) in _kernels(text).items():
            assert "vgpr_spill_count" in meta and "private_segment_fixed_size" in meta, (f, k)
            if meta["vgpr_spill_count"] or meta["private_segment_fixed_size"]:
                bad.append((f, k, meta))
    assert not bad, bad


def test_no_double_precision_arithmetic(assembly):
    bad = [(f, k, sorted(set(re.findall(r"\bv_\w+_f64\w*", body))))
           for f, text in assembly.items() for k, (body, _) in _kernels(text).items()
           if re.search(r"\bv_\w+_f64", body)]
    assert not bad, bad


def test_no_waterfall_loops(assembly):
    bad = []
    for f, text in assembly.items():
        for k, (body, _) in _kernels(text).items():
            rfl = len(re.findall(r"\bv_readfirstlane_b32\b", body))
            loops = len(re.findall(r"s_and_saveexec_b64[^\n]*\n\s*(?:buffer|global)_(?:load|store)", body))
            if rfl > MAX_READFIRSTLANE or loops:
                bad.append((f, k, rfl, loops))
    assert not bad, bad


def test_the_checks_see_a_waterfall_loop(tmp_path):
    """The waterfall check itself: a buffer load through a resource built from
    a per-lane value must be flagged."""
    src = tmp_path / "probe.hip"
    src.write_text(r'''
#include <hip/hip_runtime.h>
__global__ void probe(const float *p, float *out, int n) {
    const int rows = (int)fmaxf((float)(n - (int)threadIdx.x), 0.f);   // per-lane record count
    auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(p), (short)0, rows * 4, 0x00020000);
    out[threadIdx.x] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, 0, 0, 0));
}
''')
    text = _device_asm(str(src), str(tmp_path))
    body, _ = _kernels(text)[next(iter(_kernels(text)))]
    assert len(re.findall(r"s_and_saveexec_b64[^\n]*\n\s*(?:buffer|global)_(?:load|store)", body)) >= 1
