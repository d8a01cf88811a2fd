"""Build and run the four-over-six replica (tests/c/fos_check.c) and read
the adversarial blocks it writes (records of n fp32 values, then A, bound,
err and bf16 flag as fp32, then the exact pick as int32)."""
from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "c", "fos_check.c")


def build(tmpdir) -> str:
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = os.path.join(str(tmpdir), "fos_check")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-o", exe, SRC, "-lm"], check=True)
    return exe


def run(exe, mode, n, seed, out=None, A=None, timeout=600):
    args = [exe, mode, str(n), str(seed)]
    if out is not None:
        args.append(str(out))
        if A is not None:
            args.append(repr(float(A)))
    res = subprocess.run(args, capture_output=True, text=True, timeout=timeout)
    return res.returncode, res.stdout + res.stderr


def summary(text) -> dict:
    line = [l for l in text.splitlines() if "evals=" in l][-1]
    kv = dict(t.split("=") for t in line.split()[1:])
    return {k: float(v) for k, v in kv.items()}


def read(path, n):
    """-> (x [R, n] float32, A [R] float32, bound [R], mse [R] bool,
    bf16 [R] bool, pick4 [R] bool)"""
    rec = np.dtype([("x", "<f4", (n,)), ("hdr", "<f4", (4,)), ("pick", "<i4")])
    r = np.fromfile(path, dtype=rec)
    h = r["hdr"]
    return (r["x"].astype(np.float32), h[:, 0].astype(np.float32), h[:, 1], h[:, 2] != 0,
            h[:, 3] != 0, r["pick"] != 0)
