"""Parity margins of the GPU tests, kept for the end-of-run summary.

Each comparison of a layer output records max |gpu - oracle| / RMS(oracle)
and which bar it passed: "strict" (<= 2e-2 RMS over every compared element)
or "strict+bf16" (the strict bar plus half a bf16 ulp of each reference
element, 2^-8 |ref_i|). tests/conftest.py prints the list after the run, so
the margins appear in the output even when pytest captures the tests' own
prints.
"""
RECORDS = []


def record(name, err, rms, bar, extra=""):
    RECORDS.append((name, err / rms if rms > 0 else 0.0, bar, extra))
