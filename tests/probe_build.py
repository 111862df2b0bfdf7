"""Build of the test probes: tests/mfma_wait_probe.hip -> tests/_build/mfma_wait_probe
(gfx950), run by tests/test_mfma_wait_states_gpu.py."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_SRC = os.path.join(HERE, "mfma_wait_probe.hip")
PROBE_BIN = os.path.join(HERE, "_build", "mfma_wait_probe")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build() -> str:
    os.makedirs(os.path.dirname(PROBE_BIN), exist_ok=True)
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", PROBE_SRC, "-o", PROBE_BIN + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("probe build failed:\n%s" % r.stderr)
    os.replace(PROBE_BIN + ".tmp", PROBE_BIN)
    return PROBE_BIN


if __name__ == "__main__":
    print(build())
