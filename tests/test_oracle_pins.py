"""The oracle against facts outside itself (CPU only)."""

import pytest

import pins


@pytest.mark.parametrize("name,fn", pins.ALL_CHECKS, ids=[n for n, _ in pins.ALL_CHECKS])
def test_pin(name, fn):
    fn()


def test_check_ids_unique():
    names = [n for n, _ in pins.ALL_CHECKS]
    assert len(names) == len(set(names))
