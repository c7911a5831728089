"""The oracle against its pins (CPU only; see tests/oracle_pins.py for what each pins)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("name", sorted(ALL_PINS))
def test_pin(name):
    ALL_PINS[name](oracle.get())


def test_rejects_bad_metadata():
    import numpy as np
    import pa_inputs as pi
    case = pi.config1()
    orc = oracle.get()
    f = oracle.case_fields(case)
    bad = dict(f, past_lens=np.array([600], np.int32))               # L + T > max_context_len
    assert orc.run(**bad)[0] == oracle.ERR_META
    bt = case.block_tables.copy()
    bt[0, 3] = case.num_blocks                                        # block id out of range
    assert orc.run(**dict(f, block_tables=bt))[0] == oracle.ERR_META
    assert orc.run(**dict(f, subsequence_begins=np.array([0, 2], np.int32)))[0] == oracle.ERR_META
    assert orc.run(**dict(f, num_kv_heads=3))[0] == oracle.ERR_ARG     # Hq % Hkv != 0
