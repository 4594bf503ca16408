"""Properties of the gfx950 code that the decode kernels' speed rests on and
that no numerical test can see (CPU only: hipcc cross-compiles the device
code to assembly; skipped where hipcc is missing).

The streaming loads of a decode chunk carry the nontemporal hint, and the
chunks that start inside a sequence's shared prefix (shared_lens) load with
the default, cache-retaining policy instead. The two load paths sit in the
two arms of one branch; a compiler that takes them for the same loads hoists
them out of the branch and drops the hint from both, which leaves the results
unchanged and costs the shared-prefix workload about 8% of its speed.
"""

import os
import re
import shutil
import subprocess

import pytest

from paged_kv_cache_439_amd import build as pbuild

CSRC = pbuild.CSRC


@pytest.fixture(scope="module")
def decode_asm(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    out = tmp_path_factory.mktemp("isa") / "decode.s"
    cmd = [hipcc] + pbuild.COMMON + ["-x", "hip", "--cuda-device-only", "-S",
                                     os.path.join(CSRC, "decode.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def kernel_body(asm, pattern):
    names = re.findall(r"^(\S*" + pattern + r"\S*):", asm, re.M)
    assert names, pattern
    start = asm.index(names[0] + ":")
    return asm[start:asm.index(".Lfunc_end", start)]


# balanced and fixed-split kernels over bf16 pools, D 128, 1/2/4 heads per
# wave, 8 loads per lane per tensor, and the paired E4M3 kernel (mangled
# template arguments)
STREAMING = [
    "paged_decode_balanced_kernelIttLi128ELi1ELi8ELb1E",
    "paged_decode_balanced_kernelIttLi128ELi2ELi8ELb1E",
    "paged_decode_balanced_kernelIttLi128ELi4ELi8ELb1E",
    "paged_decode_balanced_kernelIttLi64ELi1ELi8ELb1E",
    "paged_decode_kernelIttLi128ELi2ELi8ELb1E",
    # E4M3 pools, head_dim 64, one head per wave: KV head pairs (whole lines)
    "paged_decode_balanced_kernelIthLi64ELi1ELi8ELb1ELb1E",
]


@pytest.mark.parametrize("kernel", STREAMING)
def test_streaming_and_shared_loads_both_present(decode_asm, kernel):
    body = kernel_body(decode_asm, kernel)
    loads = re.findall(r"global_load_dwordx4[^\n]*", body)
    nt = [l for l in loads if l.rstrip().endswith(" nt")]
    # 8 K + 8 V nontemporal loads per chunk on the streaming path, and the
    # same 16 plain loads on the shared-prefix path (plus the query and
    # new-row loads, which are plain)
    assert len(nt) == 16, (kernel, len(nt))
    assert len(loads) - len(nt) >= 16, (kernel, len(loads) - len(nt))


# The prefill tile loop holds the output accumulators, the query operands and
# a tile's logits in registers at two workgroups per CU. Register allocation
# of that loop has been seen to flip between two outcomes on small changes
# elsewhere in the kernel: accumulators kept in place, or copied between two
# register sets every tile (about 130 extra 64-bit moves per loop iteration,
# plus spills). The second costs time, not correctness, so only this test
# sees it.
@pytest.fixture(scope="module")
def prefill_asm(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    text = ""
    for src in ("prefill.hip", "mixed.hip"):
        out = tmp_path_factory.mktemp("isa") / (src + ".s")
        cmd = [hipcc] + pbuild.COMMON + ["-x", "hip", "--cuda-device-only", "-S",
                                         os.path.join(CSRC, src), "-o", str(out)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        text += out.read_text()
    return text


def kernel_meta(asm, name):
    start = asm.index(name + ":")
    end = asm.index(".end_amdhsa_kernel", start)
    meta = asm[end:end + 4000]
    scratch = int(re.search(r"ScratchSize:\s*(\d+)", meta).group(1))
    return asm[start:asm.index(".Lfunc_end", start)], scratch


# head_dim 128, four query heads per workgroup: bf16 and E4M3 pools, and the
# mixed batch's kernel (prefill body beside the decode workers)
PREFILL_KERNELS = [
    "_ZN2pa20prefill_chunk_kernelILi128ELi4EtEEvNS_13PrefillParamsE",
    "_ZN2pa20prefill_chunk_kernelILi128ELi4EhEEvNS_13PrefillParamsE",
    "_ZN2pa20prefill_chunk_kernelILi64ELi4EtEEvNS_13PrefillParamsE",
    "_ZN2pa18mixed_batch_kernelILi128ELi4ELb1EtEEvNS_11MixedParamsE",
]


@pytest.mark.parametrize("kernel", PREFILL_KERNELS)
def test_prefill_accumulators_stay_in_place(prefill_asm, kernel):
    body, scratch = kernel_meta(prefill_asm, kernel)
    moves = len(re.findall(r"\bv_mov_b64", body))
    assert scratch == 0, (kernel, "scratch bytes", scratch)
    assert moves <= 64, (kernel, "v_mov_b64", moves)


# The balanced decode waves set their issue priority from the share of their
# own range still to do (the four levels of s_setprio); the mixed batch's
# decode waves share their SIMDs with prefill waves and keep the default.
BALANCED = [k for k in STREAMING if k.startswith("paged_decode_balanced_kernel")]


@pytest.mark.parametrize("kernel", BALANCED)
def test_balanced_decode_sets_progress_priority(decode_asm, kernel):
    body = kernel_body(decode_asm, kernel)
    levels = set(re.findall(r"s_setprio (\d)", body))
    assert levels == {"0", "1", "2", "3"}, (kernel, levels)


def test_mixed_batch_keeps_default_priority(prefill_asm):
    body, _ = kernel_meta(prefill_asm, "_ZN2pa18mixed_batch_kernelILi128ELi4ELb1EtEEvNS_11MixedParamsE")
    assert "s_setprio" not in body


def test_decode_kernels_use_no_scratch(decode_asm):
    names = re.findall(r"^(_ZN2pa\w*paged_decode\w*kernel\w*):", decode_asm, re.M)
    assert len(names) >= 20, len(names)
    spilled = [n for n in names if kernel_meta(decode_asm, n)[1] != 0]
    assert not spilled, spilled
