"""The trace decoder and per-(layer, instruction) summary behind the step
trace summaries (persistent_interpreter_amd.trace), on a hand-built record
buffer: the header, eight words per record (the opcode/layer/unit word and
seven 100 MHz timestamps), records never written skipped."""
import math

import numpy as np

from persistent_interpreter_amd import trace


def _buf(records, ncu=2, stride=3):
    raw = np.zeros(4 + ncu * stride * 8, dtype=np.uint64)
    raw[:3] = (ncu, stride, 8)
    for (cu, i), (op, layer, unit, wait, start, done, begin, xready, epi, xlast) in records.items():
        w = 4 + (cu * stride + i) * 8
        raw[w:w + 8] = (op | (layer << 8) | (unit << 24), wait, start, done, begin, xready, epi, xlast)
    return raw


def test_decode_and_summary():
    t0 = 1_000_000
    recs = {
        # QKV of layer 0 on two workgroups, then one attention unit
        (0, 0): (1, 0, 5, t0 + 100, t0 + 150, t0 + 400, t0, t0 + 120, t0 + 380, t0 + 130),
        (1, 0): (1, 0, 6, t0 + 200, t0 + 260, t0 + 600, t0 + 10, t0 + 220, t0 + 590, t0 + 240),
        (1, 1): (2, 0, 7, t0 + 650, t0 + 660, t0 + 700, t0 + 640, 0, t0 + 690, 0),
    }
    a = trace.decode(_buf(recs))
    assert len(a) == 3                       # the unwritten records are skipped
    r = a[(a["cu"] == 1) & (a["idx"] == 0)][0]
    assert (r["op"], r["layer"], r["unit"]) == (1, 0, 6)
    # microseconds from the earliest event (t_begin of workgroup 0)
    assert math.isclose(r["t_wait"], 2.0) and math.isclose(r["t_done"], 6.0)
    assert math.isclose(r["t_begin"], 0.1) and math.isclose(r["t_epi"], 5.9)
    att = a[a["op"] == 2][0]
    assert math.isnan(att["t_xready"])      # a timestamp never taken is NaN
    rows = {x["op"]: x for x in trace.summary(a)}
    q = rows["qkv"]
    assert q["units"] == 2
    assert math.isclose(q["first_ready"], 1.0) and math.isclose(q["last_ready"], 2.0)
    assert math.isclose(q["median_done"], 5.0) and math.isclose(q["last_done"], 6.0)
    assert math.isclose(q["busy_med"], (2.5 + 3.4) / 2)      # done - start
    assert math.isclose(q["xprod_med"], (0.2 + 0.2) / 2)     # first piece - waits done
    assert math.isclose(q["epi_med"], (0.2 + 0.1) / 2)       # done - epilogue start
    assert math.isnan(rows["attn"]["xprod_med"])
