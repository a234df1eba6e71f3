"""Every kernel of libopq runs without scratch memory: the gfx950 assembly of
each HIP source, compiled with the library's flags (no GPU needed), reports no
private segment and no spilled vector register for any kernel."""
import re
from concurrent.futures import ThreadPoolExecutor

import pytest

from w4a16_linear_amd import build

HIP_SOURCES = [s for s in build.SOURCES if s.endswith(".hip")]


def _kernels(asm: str):
    """(name, {field: value}) for every kernel in the assembly's metadata."""
    meta = asm[asm.index("amdhsa.kernels:"):]
    for blk in re.split(r"\n  - \.", meta)[1:]:
        name = re.search(r"\.name:\s+(\S+)", blk)
        fields = {k: int(v) for k, v in re.findall(
            r"\.(private_segment_fixed_size|vgpr_spill_count|sgpr_spill_count|vgpr_count):\s+(\d+)", blk)}
        yield (name.group(1) if name else "?"), fields


@pytest.fixture(scope="module")
def assembly():
    with ThreadPoolExecutor(max_workers=len(HIP_SOURCES)) as ex:
        return dict(zip(HIP_SOURCES, ex.map(build.device_asm, HIP_SOURCES)))


@pytest.mark.slow
@pytest.mark.parametrize("src", HIP_SOURCES)
def test_no_scratch(assembly, src):
    kernels = list(_kernels(assembly[src]))
    assert kernels, f"no kernel metadata in {src}"
    bad = [(n, f) for n, f in kernels
           if f.get("private_segment_fixed_size", 0) or f.get("vgpr_spill_count", 0)]
    assert not bad, f"{src}: kernels using scratch: {bad[:3]}"
