"""The entry point's smoke check (one small quantize, GEMV, LM-head epilogue
and top-p draw on cuda:0, each against the oracle) runs as part of the GPU
suite, so a change to the binding that breaks it shows up here."""

import pytest

pytestmark = pytest.mark.gpu


def test_smoke_runs_against_the_oracle():
    import __graft_entry__ as g

    g.smoke()
