"""The oracle and the product share no code: neither imports the other, and
the seeded generators import neither."""
import ast
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _imports(path):
    mods = set()
    for dirpath, _, files in os.walk(path):
        for f in files:
            if not f.endswith(".py"):
                continue
            tree = ast.parse(open(os.path.join(dirpath, f)).read())
            for node in ast.walk(tree):
                if isinstance(node, ast.Import):
                    mods.update(a.name.split(".")[0] for a in node.names)
                elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
                    mods.add(node.module.split(".")[0])
    return mods


def test_oracle_does_not_import_product():
    assert "query_aware_prefill_amd" not in _imports(os.path.join(ROOT, "oracle"))


def test_product_does_not_import_oracle_or_tests():
    mods = _imports(os.path.join(ROOT, "query_aware_prefill_amd"))
    assert "oracle" not in mods and "tests" not in mods and "workloads" not in mods


def test_generators_import_neither():
    mods = _imports(os.path.join(ROOT, "workloads"))
    assert "oracle" not in mods and "query_aware_prefill_amd" not in mods


def test_product_sources_name_no_oracle_path():
    for dirpath, _, files in os.walk(os.path.join(ROOT, "query_aware_prefill_amd")):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert "oracle/" not in src and "import oracle" not in src, f
