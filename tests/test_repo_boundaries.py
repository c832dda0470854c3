"""The separations the parity claims rest on, checked from the sources (CPU only).

* The product package never imports the oracle, so no result it returns can come from the CPU
  implementation it is checked against.
* The oracle imports nothing of the package and no GPU or binding module, so the two share no
  code.
* The profile summaries are short text files whose commands run files that are in the
  repository.
"""
import ast
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PACKAGE = os.path.join(ROOT, "kv_cache_decode_split_amd")
ORACLE = os.path.join(ROOT, "oracle")
PROFILES = os.path.join(ROOT, "profiles")


def _python_files(folder):
    out = []
    for dirpath, _, files in os.walk(folder):
        if "__pycache__" in dirpath:
            continue
        out += [os.path.join(dirpath, f) for f in files if f.endswith(".py")]
    return sorted(out)


def _imported_modules(path):
    """Top-level names of every module `path` imports (absolute imports), and whether it has
    relative ones."""
    tree = ast.parse(open(path, encoding="utf-8").read(), filename=path)
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.level == 0 and node.module:
            names.add(node.module.split(".")[0])
    return names


@pytest.mark.parametrize("path", _python_files(PACKAGE), ids=os.path.basename)
def test_package_never_imports_the_oracle(path):
    assert "oracle" not in _imported_modules(path)


@pytest.mark.parametrize("path", _python_files(ORACLE), ids=os.path.basename)
def test_oracle_imports_no_product_or_gpu_code(path):
    allowed = {"__future__", "math", "struct", "itertools", "typing", "numpy"}
    assert _imported_modules(path) <= allowed


def test_bench_uses_the_oracle_only_for_its_cpu_baselines():
    """bench.py may run the oracle for the reported CPU baseline only: every import of it sits
    in a function body, under a test of the --no-cpu-baseline switch or in the function that
    times the CPU."""
    src = open(os.path.join(ROOT, "bench.py"), encoding="utf-8").read()
    tree = ast.parse(src)
    parents = {}
    for node in ast.walk(tree):
        for child in ast.iter_child_nodes(node):
            parents[child] = node
    found = 0
    for node in ast.walk(tree):
        if isinstance(node, ast.ImportFrom) and node.module and node.module.split(".")[0] == "oracle":
            found += 1
            chain, p = [], parents.get(node)
            while p is not None:
                chain.append(p)
                p = parents.get(p)
            funcs = [c.name for c in chain if isinstance(c, ast.FunctionDef)]
            guards = [ast.unparse(c.test) for c in chain if isinstance(c, ast.If)]
            assert funcs, "an oracle import at module level"
            assert any("cpu" in f for f in funcs) or any("no_cpu_baseline" in g for g in guards), (
                funcs, guards)
    assert found >= 1


def test_profile_summaries_are_short_text_with_runnable_commands():
    names = sorted(os.listdir(PROFILES))
    assert names, "no profile summaries"
    for name in names:
        path = os.path.join(PROFILES, name)
        assert os.path.splitext(name)[1] in (".md", ".txt", ".json"), name
        assert os.path.getsize(path) < 64 * 1024, name
        text = open(path, encoding="utf-8").read()
        assert "_work" not in text and "/root/reference" not in text, name
        if name.endswith(".md"):
            commands = [line for line in text.splitlines() if "rocprofv3" in line]
            assert commands, f"{name}: no command"
            for line in commands:
                for rel in re.findall(r"\$REPO/([\w./-]+\.(?:py|sh))", line):
                    assert os.path.isfile(os.path.join(ROOT, rel)), (name, rel)
