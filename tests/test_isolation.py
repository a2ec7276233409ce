"""The product path and the oracle stay apart, and the product path fails
loudly when its HIP library is missing (there is no fallback)."""
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sources(pattern):
    return [f for f in glob.glob(os.path.join(ROOT, pattern), recursive=True) if os.path.isfile(f)]


def test_package_never_mentions_the_oracle():
    files = _sources("gated_delta_rule_48_amd/**/*.py") + _sources("gated_delta_rule_48_amd/csrc/*") + \
        _sources("include/*.h")
    assert files
    for f in files:
        text = open(f, errors="ignore").read()
        assert not re.search(r"\boracle\b", text), f"{f} refers to the oracle"


def test_oracle_never_imports_the_package():
    for f in _sources("oracle/*.py") + _sources("oracle/*.c"):
        text = open(f, errors="ignore").read()
        assert "gated_delta_rule_48_amd" not in text and "kda.h" not in text, f


def test_missing_library_fails_loudly(monkeypatch):
    import gated_delta_rule_48_amd as kda
    monkeypatch.setattr(kda, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libkda.so"))
    monkeypatch.setattr(kda, "_lib", None)
    with pytest.raises(ImportError):
        kda.load_library()
