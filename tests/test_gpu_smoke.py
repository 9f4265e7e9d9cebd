"""The round-end smoke check (__graft_entry__.smoke) runs as part of the GPU
suite, so a broken check or a broken path shows up with the other tests."""
import pytest

pytestmark = pytest.mark.gpu


def test_smoke():
    import __graft_entry__
    __graft_entry__.smoke()
