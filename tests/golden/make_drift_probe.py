"""Write drift_probe_small.txt: the oracle's perturbation probe on the small
bf16 configuration (d = 512, 8 heads, 12 layers, G = 12, W = 128), 4
sequences over 150 steps.  It calls only the oracle (through the probe in
tests/test_oracle_bf16.py) and the seeded input generators.

    python tests/golden/make_drift_probe.py
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
sys.path.insert(0, os.path.dirname(HERE))

from test_oracle_bf16 import probe, PROBE_REPORT, PROBE_ROWS, PROBE_STEPS  # noqa: E402

d, p = probe()
with open(os.path.join(HERE, "drift_probe_small.txt"), "w") as f:
    f.write("# Perturbation probe of the oracle, small bf16 configuration (d 512, H 8, L 12,\n"
            f"# F 2048, W 128, G 12, V 4096), {PROBE_ROWS} sequences from H_0, {PROBE_STEPS} steps.\n"
            "# Columns: step t, rel-L2 over the sequences of (bf16 emulation - float64)\n"
            "# logits, rel-L2 of (float64 with e and memory scaled by 1 +- 2^-9 - float64).\n"
            "# Written by tests/golden/make_drift_probe.py from the oracle alone.\n")
    for t in PROBE_REPORT:
        f.write(f"{t} {d[t - 1]:.4e} {p[t - 1]:.4e}\n")
print(open(os.path.join(HERE, "drift_probe_small.txt")).read())
