"""CPU check that the attention cases of the GPU parity tests reach every
instance of the packed-bit attention kernel (tests/att_variants.py restates
the launcher's choice from the states' widths and the group)."""
import numpy as np

import att_variants as av
import synth
from oracle import codec


def test_cases_reach_every_instance():
    seen = set()
    for cfg, avg, g, n, spec in av.CASES:
        w = synth.WORKLOADS[cfg]
        bits = None if spec is None else av.widths(spec)
        sts = [codec.calibrate_head(synth.stream(w, 0, 0, 1, kind, n=n), min(w.n_calib, n), avg, bits=bits)
               for kind in (0, 1)]
        seen.add(av.instance([int(np.sum(s["bits"], dtype=np.int64)) for s in sts], [s["bits"] for s in sts], g))
    assert seen == av.ALL_INSTANCES, av.ALL_INSTANCES ^ seen


def test_value_columns_of_simple_widths():
    # 8-bit codes from bit 0: one column each; a 3-bit code at bit 6 crosses one boundary
    assert av.value_columns([8, 8, 8]) == 3
    assert av.value_columns([6, 3, 7]) == 1 + 2 + 1
    assert av.value_columns([0, 0, 5]) == 1
