"""The package's smoke entry (one tiny layer call on the first GPU, checked
against the oracle) runs as it is shipped, together with ``MixQLinear``,
the module wrapper it drives."""
import pytest

pytestmark = pytest.mark.gpu


def test_smoke_entry():
    import __graft_entry__

    __graft_entry__.smoke()
