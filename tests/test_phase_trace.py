"""Host side of the phase-trace tool (quantized_kv_attention_amd/phase_trace.py):
the summary of a synthetic stamp array, with 32-bit wrap-around."""
import numpy as np

from quantized_kv_attention_amd import phase_trace as pt


def test_summary_of_synthetic_stamps():
    t = np.zeros((pt.WGS, 8, pt.SLOTS), np.int64)
    n = 4
    base = 2**32 - 150  # the 100 MHz counter wraps inside the kernel
    for g in range(n):
        for w in range(8):
            s = base + 10 * w
            stamps = {0: s, 1: s + 200, 2: s + 300, 3: s + 320, 4: s + 400, 5: s + 450, 15: s + 900, 18: s + 1200,
                      19: s + 1230}
            for k, v in stamps.items():
                t[g, w, k] = v % 2**32
            t[g, w, 20] = 1 if g == 0 else 0
            t[g, w, 22] = 1000
            t[g, w, 23] = 1000 + 18000  # 18,000 shader cycles over the 6 us loop: 3 GHz
    text = pt.summarise(t, "synthetic")
    assert "synthetic: 4 work-groups" in text
    assert "storing new tokens (1)" in text and "other (3)" in text
    # wavefront 0 starts the work-group: query landed 2 us, loop end 9 us, end 12.3 us
    line = [x for x in text.splitlines() if x.strip().startswith("wavefront 0")][1]
    assert "query landed 2.00" in line and "key loop end 9.00" in line and "outputs start 12.30" in line
    assert "(3.00 GHz in the loop)" in line
    # wavefront 7 starts 0.7 us after the work-group
    line7 = [x for x in text.splitlines() if x.strip().startswith("wavefront 7")][1]
    assert "start 0.70" in line7


def test_summary_without_wide_work_groups():
    # a call that ran no 64-row work-group leaves the stamps at zero
    t = np.zeros((pt.WGS, 8, pt.SLOTS), np.int64)
    assert "no work-group of verify_wide_kernel ran" in pt.summarise(t, "plain")
