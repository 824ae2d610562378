"""The usage example in README.md runs as written."""
from __future__ import annotations

import os
import re

import pytest

from tests._gpu import needs_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]


def test_readme_example_runs(capsys):
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    text = open(os.path.join(root, "README.md"), encoding="utf-8").read()
    blocks = re.findall(r"```python\n(.*?)```", text, re.S)
    assert len(blocks) == 1, "README.md holds one python example"
    exec(compile(blocks[0], "README.md example", "exec"), {})
    out = capsys.readouterr().out
    assert "example ok (3, 16, 512) True [[150, 150, 21], [149, 150, 20]]" in out
