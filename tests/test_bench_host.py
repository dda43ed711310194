"""Host-side parts of bench.py, without a GPU: the CPU baseline on small CPU
tensors, the refusal of several GPUs, and a static check that every call of
one of bench.py's own functions binds to that function's signature (the
GPU-only paths are otherwise exercised only on the GPU)."""
import ast
import inspect
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _small_case(random_emb):
    B, S, NL, Hq, Hkv, d, V = 2, 16, 2, 4, 1, 32, 64
    W = Hq * d
    lens = [64, 32]
    w = dict(B=B, S=S, layers=NL, lens=lens, gamma=0.8, tau=1.0, name="host")
    if random_emb:
        w["random_emb"] = True
    g = torch.Generator().manual_seed(7)
    T = sum(lens)
    bf = torch.bfloat16
    kc = [torch.randn(T, Hkv, d, generator=g).to(bf) for _ in range(NL)]
    vc = [torch.randn(T, Hkv, d, generator=g).to(bf) for _ in range(NL)]
    qb = [torch.randn(B, S, Hq, d, generator=g).to(bf) for _ in range(NL)]
    kb = [torch.randn(B, S, Hkv, d, generator=g).to(bf) for _ in range(NL)]
    vb = [torch.randn(B, S, Hkv, d, generator=g).to(bf) for _ in range(NL)]
    ada = torch.randn(NL, 3, B, W, generator=g) * 0.1
    logits = torch.randn(B, S, V, generator=g).to(bf)
    start = torch.tensor([0, lens[0]])
    adaln = (torch.ones(B), torch.randn(B, 256, generator=g),
             (torch.randn(256, 3 * W, generator=g) * 0.05).to(bf),
             torch.randn(3 * W, generator=g) * 0.1, torch.randn(NL, 3, W, generator=g) * 0.1)
    return w, (kc, vc, qb, kb, vb, ada, logits, start) + adaln


@pytest.mark.parametrize("random_emb", [False, True])
def test_cpu_baseline_fields(random_emb):
    w, args = _small_case(random_emb)
    r = bench.cpu_baseline(w, 2, *args)
    assert r["kind"] == "oracle" and r["unit"] == "query-tokens/s"
    assert r["value"] > 0 and r["cores"] >= 1 and r["host_cpu_count"] >= 1
    assert "adaLN" in r["sample"] and "attention" in r["sample"] and "unmasking" in r["sample"]


def test_several_gpus_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stdout


def test_calls_bind_to_signatures():
    """Every call in bench.py of a function bench.py defines at module level
    passes arguments its signature accepts (counted positionally and by
    keyword; calls that unpack * or ** are skipped)."""
    src = open(os.path.join(ROOT, "bench.py")).read()
    tree = ast.parse(src)
    funcs = {n.name: getattr(bench, n.name) for n in tree.body if isinstance(n, ast.FunctionDef)}
    checked = 0
    for node in ast.walk(tree):
        if not (isinstance(node, ast.Call) and isinstance(node.func, ast.Name)
                and node.func.id in funcs):
            continue
        if any(isinstance(a, ast.Starred) for a in node.args) or any(k.arg is None for k in node.keywords):
            continue
        sig = inspect.signature(funcs[node.func.id])
        try:
            sig.bind(*range(len(node.args)), **{k.arg: None for k in node.keywords})
        except TypeError as e:
            pytest.fail(f"bench.py line {node.lineno}: {node.func.id}(...) does not bind: {e}")
        checked += 1
    assert checked >= 5
