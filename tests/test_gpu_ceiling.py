"""The ceiling probes (tests/native/ceiling_probe.hip) run and give plausible figures:
every matrix-instruction rate is positive and at most the published peak for its
type (a rate above it would mean the probe counts work it does not do), the
L2-resident loads outrun HBM, and the HBM streams stay below 8 TB/s.  The full
measurement is `python bench.py --ceiling`."""
import pytest

import bench

pytestmark = pytest.mark.gpu


def test_ceiling_probes_are_plausible():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rows = bench.ceiling_probes(quick=True)
    by = {}
    for r in rows:
        print(f"[ceiling] {r}", flush=True)
        by.setdefault(r["probe"], []).append(r)
    for _, name, dt in bench.CEIL_MFMA:
        for r in by[name]:
            assert 0 < r["rate"] <= 1.001 * bench.CEIL_PEAK[dt], r
    l2 = max(r["rate"] for r in by["l2_read_to_registers"])
    hbm = by["hbm_read_nt"][0]["rate"]
    assert 0 < hbm < 8.0 and l2 > hbm, (l2, hbm)
    assert 0 < by["hbm_write_nt"][0]["rate"] < 8.0
    assert by["lds_read_b128"][0]["rate"] > l2
