"""The streaming kernels' generated gfx950 code (no GPU needed: hipcc
cross-compiles).

Every 8- and 16-byte global load and store of the AdamW, accumulation,
reduction and norm kernels must carry the non-temporal hint.  This is the layout the
kernels were measured in: a loop transformation in the compiler once
promoted the AdamW stores out of a one-iteration loop and dropped the hint,
costing about 10 points of HBM bandwidth without changing any result.  No
kernel may use scratch memory (register spills).  The AdamW kernels round
the 16-bit parameter from the stored float32 master: no fused fp16 mix
instruction (which would round the unrounded fma result instead).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
STREAMING = ("adam_update", "adam_update_devcoef", "grad_accumulate", "grad_reduce", "grad_sum_norm",
             "sqnorm_partials")


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which("hipcc")):
        pytest.skip("hipcc not available")
    from zero_sharded_mixed_partition_amd import build as B
    out = str(tmp_path_factory.mktemp("asm") / "shard_step.s")
    cmd = [HIPCC, f"--offload-arch={B.ARCH}", "-O3", "-std=c++17", f"-I{B.INCLUDE}", f"-I{B.CSRC}",
           *B.DEVICE_FLAGS, "--cuda-device-only", "-S", os.path.join(B.CSRC, "shard_step.hip"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    text = open(out).read()
    found = {}
    for m in re.finditer(r"^(_Z\S+):\s*; @", text, re.M):
        end = text.find("s_endpgm", m.end())
        meta = re.search(r"\.amdhsa_kernel " + re.escape(m.group(1)) + r"\n(.*?)\.end_amdhsa_kernel", text, re.S)
        found[m.group(1)] = (text[m.end():end], meta.group(1) if meta else "")
    return found


def _kind(name):
    for k in sorted(STREAMING, key=len, reverse=True):
        if re.search(r"\d" + k + r"I", name):
            return k
    return None


def test_every_streaming_kernel_is_present(kernels):
    kinds = {_kind(n) for n in kernels}
    assert set(STREAMING) <= kinds, kinds


def test_vector_accesses_are_non_temporal(kernels):
    checked = 0
    for name, (body, _) in kernels.items():
        if _kind(name) is None:
            continue
        ops = re.findall(r"^\s*(global_(?:load|store)_dwordx[24])\b([^\n]*)", body, re.M)
        if _kind(name) == "sqnorm_partials":          # its one vector store is the per-block partial
            ops = [o for o in ops if o[0].startswith("global_load")]
        if _kind(name) == "grad_sum_norm":            # the per-task partial: one plain 8-byte store
            partial = [o for o in ops if o[0] == "global_store_dwordx2" and not o[1].rstrip().endswith(" nt")]
            assert len(partial) == 1, f"{name}: {len(partial)} plain 8-byte stores"
            ops = [o for o in ops if o not in partial]
        assert ops, name
        plain = [o for o in ops if not o[1].rstrip().endswith(" nt")]
        assert not plain, f"{name}: {len(plain)} of {len(ops)} vector accesses without the hint"
        checked += 1
    assert checked >= 20


def test_no_kernel_spills(kernels):
    for name, (_, meta) in kernels.items():
        m = re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", meta)
        assert m and int(m.group(1)) == 0, f"{name} uses scratch memory"


def test_adamw_writeback_rounds_the_stored_master(kernels):
    """v_fma_mixlo/mixhi_f16 (or v_mad_mix*) writing fp16 would round the
    update's exact fma result to the parameter copy, skipping the float32
    rounding of the stored master (one ulp apart in about 6 of 100,000
    parameters).  Only the plain conversions may form the copy."""
    checked = 0
    for name, (body, _) in kernels.items():
        if _kind(name) not in ("adam_update", "adam_update_devcoef"):
            continue
        fused = re.findall(r"^\s*(v_(?:fma|mad)_mix(?:lo|hi)_f16)\b", body, re.M)
        assert not fused, f"{name}: {len(fused)} fused fp16 conversions"
        checked += 1
    assert checked >= 8
