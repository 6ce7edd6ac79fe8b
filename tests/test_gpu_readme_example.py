"""The Python example in README.md runs as written (against the built library, on the GPU)."""
import os
import re

import pytest

pytestmark = pytest.mark.gpu

README = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")


def test_readme_python_example_runs(capsys):
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    blocks = re.findall(r"```python\n(.*?)```", open(README).read(), flags=re.S)
    assert blocks, "README.md has no python example"
    exec(compile(blocks[0], "README.md example", "exec"), {"__name__": "readme_example"})
    out = capsys.readouterr().out.split()
    assert int(out[0]) == 201   # 200 prefilled tokens + 1 decoded and committed
