"""Cross-XCD visibility within one launch, the hardware fact behind keeping the scoring
and the selection in two launches.

A selection in the scoring launch would have to read, from one workgroup, scores and
candidate blocks that workgroups on the other XCDs wrote moments before.  Each XCD has
its own L2, so that only works when the stores are written through (sc1) and the loads
are served coherently (sc1); then every word of every epoch is fresh.  With plain stores
or plain loads, the probe reads stale words (printed; run with -s).  The one-launch
version built on sc1 stores, sc1 loads and an arrival counter was slower than the launch
boundary it replaced."""
import ctypes

import pytest

pytestmark = pytest.mark.gpu


def _run(lib, st, ld, nwg=2048, epochs=500):
    checks, stale = ctypes.c_uint32(0), ctypes.c_uint32(0)
    rc = lib.xcd_coherence_probe(st, ld, nwg, epochs, ctypes.byref(checks), ctypes.byref(stale))
    assert rc == 0, rc
    return checks.value, stale.value


def test_sc1_stores_and_loads_see_every_word():
    from tests import probes
    lib = probes.load("xcd_coherence")
    print("\n2,048 workgroups x 256 words, 500 epochs: the last arriver's stale words")
    for st, ld in [(1, 1), (0, 1), (1, 0), (0, 0)]:
        checks, stale = _run(lib, st, ld)
        print(f"  stores {'sc1' if st else 'plain':5s} loads {'sc1' if ld else 'plain':5s}: "
              f"{checks} checks, {stale} stale words")
        assert checks == 500
        if st and ld:
            assert stale == 0
