"""The product path has no CPU implementation and never touches the oracle:
importing the package loads no oracle module, no package source imports the
oracle or the input generators, and every entry point rejects CPU tensors
(there is nothing to fall back to)."""
import os
import re
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "fp4_block_quantization_nvfp4_amd")


def test_import_loads_no_oracle():
    code = ("import sys; import fp4_block_quantization_nvfp4_amd, fp4_block_quantization_nvfp4_amd.api; "
            "bad = [m for m in sys.modules if m == 'oracle' or m.startswith('oracle.') or m == 'workloads']; "
            "print(bad); sys.exit(1 if bad else 0)")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr


def test_no_package_source_imports_the_oracle():
    pat = re.compile(r"^\s*(import|from)\s+(oracle|workloads)\b", re.M)
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert not pat.search(src), f


@pytest.mark.parametrize("call", ["quantize", "qdq", "quantize_4over6", "quantize_2d", "quantize_rowcol",
                                  "quantize_4over6_2d", "amax"])
def test_cpu_tensors_are_rejected(call):
    import fp4_block_quantization_nvfp4_amd as nv
    x = torch.zeros((16, 32), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        getattr(nv, call)(x)
