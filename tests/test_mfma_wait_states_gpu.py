"""The wait states the hazard check assumes, measured on this GPU.

tests/mfma_wait_probe.hip issues one MFMA per kernel, waits a fixed number
of wait states, and reads the last result register; a lane that reads the
finished value counts as fresh.  The check in tests/mfma_hazards.py needs
every lane fresh at its stated count (fp8 scaled product 20, bf16 product
12).  One state fewer is reported too: on the MI355X it reads the old
value, which is why the compiler's 19 after the fp8 product is not enough.
"""
import json
import os
import subprocess

import pytest

import mfma_hazards as H
import probe_build

from gpu_util import note, torch_or_skip

pytestmark = pytest.mark.gpu


def test_mfma_results_are_ready_after_the_checked_wait_states():
    torch_or_skip()
    exe = probe_build.PROBE_BIN if os.path.exists(probe_build.PROBE_BIN) else probe_build.build()
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    rows = [json.loads(l) for l in r.stdout.splitlines() if l.startswith("{")]
    got = {(x["mfma"], x["wait_states"]): x["fresh_lanes"] for x in rows}
    for (mfma, waits), fresh in sorted(got.items()):
        note("%s after %d wait states: %d of 64 lanes read the result" % (mfma, waits, fresh))
    for mfma, need in H.WAIT_STATES.items():
        assert got[(mfma, need)] == 64, (mfma, need)
        assert got[(mfma, need + 4)] == 64, (mfma, need + 4)
        assert (mfma, need - 1) in got
