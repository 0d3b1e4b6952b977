"""The README's Python example runs as written: a rule turn and a Mean-K step through the binding."""

import os
import re

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_python_example_runs(capsys):
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", text, re.S)
    assert blocks, "README.md has no Python example"
    exec(compile(blocks[0], "README.md", "exec"), {})
    out = capsys.readouterr().out.split()
    assert out[-2:] == ["4096", "512"]          # kept positions (the budget C) and selected blocks
