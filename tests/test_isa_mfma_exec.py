"""Every MFMA of the library runs with the whole wave enabled (CPU; compiles the kernels to gfx950
assembly with hipcc).

An MFMA mixes its operands across the wave's 64 lanes, so an MFMA issued while EXEC is narrowed by a
lane-dependent branch (a store of the rows below M) computes the enabled lanes' outputs from disabled
lanes' operands.  The kernels pin their accumulators before such branches; this test checks the
generated code: for every v_mfma, the nearest preceding instruction in the kernel's code that writes
EXEC must be one that restores it (or there is none)."""
import concurrent.futures as cf
import glob
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_scaled_fp8_r9k_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _device_asm(src, out_dir):
    from block_scaled_fp8_r9k_amd.build import CFLAGS
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    flags = [f for f in CFLAGS if f not in ("-fPIC",)]
    subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", out], check=True, capture_output=True)
    return out


def mfma_under_narrowed_exec(asm_text):
    bad = {}
    kern, last = None, None
    for ln in asm_text.splitlines():
        m = re.match(r"^(_Z\S+):", ln)
        if m:
            kern, last = m.group(1), None
            continue
        t = ln.strip()
        if re.match(r"s_(and|andn2|or|xor)_saveexec", t) or re.match(r"s_(and|andn2|or|xor|mov|cselect)_b64 exec", t):
            last = t
        elif t.startswith("v_mfma") and kern and last and not (
                last.startswith("s_or_b64 exec, exec") or last.startswith("s_mov_b64 exec, -1")):
            bad.setdefault(kern, last)
    return bad


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_no_mfma_under_narrowed_exec(tmp_path):
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        outs = list(ex.map(lambda s: _device_asm(s, str(tmp_path)), srcs))
    found = {}
    n_mfma = 0
    for o in outs:
        text = open(o).read()
        n_mfma += text.count("v_mfma")
        found.update(mfma_under_narrowed_exec(text))
    assert n_mfma > 100
    assert not found, f"MFMAs after an exec-narrowing instruction in: {sorted(found)[:5]}"


def test_check_flags_a_sunk_mfma():
    # the pattern the check exists for: an MFMA inside a lane-dependent branch
    asm = "\n".join(["_ZN3r9k1kEv:", "v_cmp_gt_i64_e32 vcc, s[14:15], v[4:5]", "s_and_saveexec_b64 s[2:3], vcc",
                     "v_mfma_scale_f32_16x16x128_f8f6f4 v[6:9], v[16:23], v[24:31], 0, v6, v6",
                     "s_or_b64 exec, exec, s[2:3]", "s_endpgm"])
    assert mfma_under_narrowed_exec(asm) == {"_ZN3r9k1kEv": "s_and_saveexec_b64 s[2:3], vcc"}
    ok = "\n".join(["_ZN3r9k1kEv:", "s_and_saveexec_b64 s[2:3], vcc", "s_or_b64 exec, exec, s[2:3]",
                    "v_mfma_scale_f32_16x16x128_f8f6f4 v[6:9], v[16:23], v[24:31], 0, v6, v6", "s_endpgm"])
    assert mfma_under_narrowed_exec(ok) == {}
