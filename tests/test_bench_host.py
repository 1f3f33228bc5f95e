"""Host logic of bench.py that runs before any GPU work."""
import sys
from types import SimpleNamespace

import pytest

import bench


def test_variant_selection():
    assert bench.selected_variants(",".join(bench.VARIANTS)) == list(bench.VARIANTS)
    assert bench.selected_variants("ffd_peaked") == ["ffd_peaked"]
    assert bench.selected_variants("paged,,ffd") == ["paged", "ffd"]
    with pytest.raises(SystemExit):
        bench.selected_variants("paged,nope")


def test_ffd_deltas_override():
    assert bench._ffd_override(SimpleNamespace(ffd_deltas=None)) == {}
    assert bench._ffd_override(SimpleNamespace(ffd_deltas="5")) == {"deltas": (5.0,)}
    assert bench._ffd_override(SimpleNamespace(ffd_deltas="5,7.5")) == {"deltas": (5.0, 7.5)}
    with pytest.raises(ValueError):
        bench._ffd_override(SimpleNamespace(ffd_deltas="five"))


def test_more_than_one_gpu_is_refused(monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2


def test_unknown_variant_is_refused_before_gpu_work(monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--variants", "nope"])
    with pytest.raises(SystemExit):
        bench.main()
