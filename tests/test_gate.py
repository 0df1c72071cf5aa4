"""The runnable gate (tests/gate.py): the pages' four parts and their summary
line, on the CPU oracle and on the GPU library; and that the gate's checks
catch a planted mistake (planted in a wrapper around the oracle, on the CPU)."""
import os
import subprocess
import sys

import numpy as np
import pytest

from conftest import ROOT

sys.path.insert(0, os.path.join(ROOT, "tests"))
import gate  # noqa: E402

LINES = [
    "PKV KAT pool alloc/exhaust/recycle OK",
    "PKV EQUIV paged==contiguous BIT-EXACT (5+1+3 rows, 2 layers, GQA) OK",
    "PKV FORK+COW both forks BIT-EXACT vs contiguous replays OK",
    "PKV REWIND truncate-then-append BIT-EXACT (spec-decode contract) OK",
    "LIAR-KILL pool-mechanics=1 equiv-bitexact=1 fork-cow=1 rewind=1",
    "PAGED_KV_GATE DONE",
]


def _run(*args):
    p = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "gate.py"), *args],
                       capture_output=True, text=True, timeout=600)
    return p.returncode, [l for l in p.stdout.splitlines() if l.strip()]


def test_gate_on_the_oracle_prints_the_summary_and_exits_0():
    rc, lines = _run()
    assert rc == 0, lines
    assert lines == LINES


class _Flip(gate.OracleBackend):
    """The oracle with one output bit flipped in the paged path's layer-1
    output of the `nth` paged attention call."""

    def __init__(self, nth):
        super().__init__()
        self.calls = 0
        self.nth = nth

    def attn_paged(self, pool, seq, layer, Q, K, V, n):
        rc, out = super().attn_paged(pool, seq, layer, Q, K, V, n)
        self.calls += 1
        if self.calls == self.nth:
            out = out.copy()
            out.view(np.uint32)[0, 0] ^= 1
        return rc, out


@pytest.mark.parametrize("nth,code", [(1, 24), (3, 34), (5, 44), (9, 92), (11, 93),
                                      (13, 96)])
def test_gate_catches_a_flipped_bit(nth, code):
    """Calls 1-6 are the three EQUIV rounds (2 layers each), 7-8 fork A's
    prefill round, 9-10 fork A's divergent round, 11-12 fork B's, 13-14 the
    rewind."""
    with pytest.raises(gate.Fail) as e:
        gate.run(_Flip(nth))
    assert e.value.code == code


@pytest.mark.gpu
def test_gate_on_the_gpu_library():
    rc, lines = _run("--gpu")
    assert rc == 0, lines
    assert lines[-len(LINES):] == LINES
