"""HBM traffic of the decode kernels as the profiler's counters measured it.

The counters come from two rocprofv3 ``--pmc`` passes (FETCH_SIZE, then
WRITE_SIZE) over a short run of the benchmark; the summary under ``profiles/``
records them per dispatch, already scaled by the factor that a plain
device-to-device copy of known size gives for the same counter.  A summary is
valid only for the kernel source it was taken on: it stores a digest of the
decode sources, and :func:`traffic_bytes` returns None once they differ.
"""
from __future__ import annotations

import hashlib
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(_HERE)
DECODE_SOURCES = ("csrc/decode.hip", "csrc/pop_device.h", "csrc/pop_internal.h")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "decode_kernels_llama2_7b_b1_hbm_traffic.md")
_LINE = re.compile(r"^kernel=(?P<k>.+?) fetch_bytes=(?P<f>\d+) write_bytes=(?P<w>\d+) digest=(?P<d>[0-9a-f]+)$")


def source_digest(files=DECODE_SOURCES) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(_HERE, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_bytes(kernel: str, path: str = TRAFFIC_SUMMARY):
    """(fetch, write) HBM bytes per launch of ``kernel`` from the summary, or
    None if there is none or the decode sources changed since it was taken."""
    if not os.path.exists(path):
        return None
    digest = source_digest()
    with open(path) as fh:
        for line in fh:
            m = _LINE.match(line.strip())
            if m and m["k"] == kernel and m["d"] == digest:
                return int(m["f"]), int(m["w"])
    return None
