"""The excused rate over every parity comparison of the session.

A draw whose uniform lies within 1e-6 of its threshold or running sum (in the
normalised units of the distribution drawn from) may differ from the oracle;
the rate of such excusals over all draws compared must stay at or below 1e-4.
The parity tests add their counts to gpu_harness.TOTALS as they check; this
test runs after them (file order) and asserts the session's rate.
"""
import pytest

pytestmark = pytest.mark.gpu

H = pytest.importorskip("gpu_harness")


def test_session_excused_rate():
    tot = H.TOTALS
    H.say(f"[excused] session: {tot.excused} excused of {tot.n_draws} draws "
          f"({tot.excused / max(tot.n_draws, 1):.3g}); boundary draws {tot.boundary_draws}; "
          f"max|a err|={tot.max_a_err:.3g} max|C err|={tot.max_cdf_err:.3g} "
          f"max prob rel={tot.max_prob_rel:.3g}")
    if tot.n_draws == 0:
        pytest.skip("no parity comparison ran in this session")
    assert tot.excused <= 1e-4 * tot.n_draws, (tot.excused, tot.n_draws)
