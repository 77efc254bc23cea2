"""The MFMA-mix microbenchmark's generator (no GPU): every loop block issues
four matrix products with the stated vector and LDS instructions after each,
waits for its LDS reads inside the same block, and the source builds for
gfx950."""
import re
import shutil

import pytest

from block_masked_attention_amd.microbench import mfma_mix


@pytest.mark.parametrize("op,v,l", mfma_mix.mixes())
def test_block_contents(op, v, l):
    lines = mfma_mix.block(op, v, l).split("\\n\\t")
    assert sum(x.startswith("v_mfma_f32_32x32x16_bf16") for x in lines) == 4
    assert sum(x.startswith(f"v_{op}_f32") for x in lines) == 4 * v
    reads = [i for i, x in enumerate(lines) if x.startswith("ds_read_b128")]
    assert len(reads) == 4 * l
    if l:
        # the reads complete before the block ends (no load left in flight
        # across asm statements)
        assert lines[-1] == "s_waitcnt lgkmcnt(0)" and max(reads) < len(lines) - 1
    # read destinations and vector registers stay clear of the operands and
    # accumulators (v0..v71) and of the constants (v96..v99)
    for x in lines[1:]:
        for r in re.findall(r"v\[?(\d+)", x.split(",")[0].split()[1]) if not x.startswith(("v_mfma", "s_")) else []:
            assert 72 <= int(r) < 96 or 100 <= int(r) < 116


@pytest.mark.skipif(shutil.which("hipcc") is None and not __import__("os").path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not installed")
def test_builds(tmp_path):
    exe = mfma_mix.build(str(tmp_path))
    assert (tmp_path / "mfma_mix").exists() and exe.endswith("mfma_mix")


def test_power_block_contents():
    """The power microbenchmark's loop block: four products over the two A and
    two B operand sets (every pairing once), v vector instructions and l LDS
    reads after each, the reads waited for inside the block; the vector
    instructions write only v80..v95 and the reads only v100..v115."""
    from block_masked_attention_amd.microbench import mfma_power
    for v, l in mfma_power.MIXES:
        lines = mfma_power.block(v, l).split("\\n\\t")
        mf = [x for x in lines if x.startswith("v_mfma_f32_32x32x16_bf16")]
        assert len(mf) == 4 and len(lines) == 4 + 4 * v + 4 * l + (1 if l else 0)
        pairs = {tuple(x.replace(",", "").split()[2:4]) for x in mf}
        assert pairs == {("v[64:67]", "v[68:71]"), ("v[72:75]", "v[76:79]"),
                         ("v[64:67]", "v[76:79]"), ("v[72:75]", "v[68:71]")}
        accs = [x.replace(",", "").split()[1] for x in mf]
        assert accs == [f"v[{16 * m}:{16 * m + 15}]" for m in range(4)]
        reads = [i for i, x in enumerate(lines) if x.startswith("ds_read_b128")]
        assert len(reads) == 4 * l
        if l:
            assert lines[-1] == "s_waitcnt lgkmcnt(0)" and max(reads) < len(lines) - 1
        for x in lines:
            if x.startswith("v_fma_f32"):
                assert 80 <= int(x.split()[1].rstrip(",")[1:]) < 96
            if x.startswith("ds_read_b128"):
                lo, hi = x.split()[1].strip("v[],").split(":")
                assert 100 <= int(lo) and int(hi) < 116


@pytest.mark.skipif(shutil.which("hipcc") is None and not __import__("os").path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not installed")
def test_power_builds(tmp_path):
    from block_masked_attention_amd.microbench import mfma_power
    exe = mfma_power.build(str(tmp_path))
    assert (tmp_path / "mfma_power").exists() and exe.endswith("mfma_power")
