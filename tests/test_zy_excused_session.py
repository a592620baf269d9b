"""Session total of excused near-tie disagreements (runs after the parity tests).

Every sampling comparison of the session adds its decisions taken and its
excused disagreements to ``parity_util.SESSION``; in total the excused ones
must stay below 1e-4 of the decisions."""
import pytest

from tests import parity_util

pytestmark = pytest.mark.gpu


def test_session_excused_rate():
    s = parity_util.SESSION
    if s.decisions == 0:
        pytest.skip("no sampling comparison ran in this session")
    print(f"session: {s.excused} excused of {s.decisions} decisions taken ({s.excused_rate:.2e})", flush=True)
    assert s.excused_rate < parity_util.MAX_EXCUSED_RATE
