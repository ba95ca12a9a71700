"""The oracle and the HIP path share no code, and workloads holds no arithmetic of the method.

The imports of every Python file under oracle/, workloads/ and
exact_attention_20_amd/ are read with ast (so an import inside a function
counts too) and checked against what each package may use:
  * oracle/ imports neither the library package nor workloads;
  * the library package imports neither oracle nor workloads;
  * workloads/ imports neither the oracle nor the library package.
The product path (bench.py's timed legs, the library) reaches the oracle only
through bench.py's cpu_baseline functions, checked last.
"""
import ast
import glob
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = "exact_attention_20_amd"
FORBIDDEN = {"oracle": {PKG, "workloads"}, PKG: {"oracle", "workloads"}, "workloads": {"oracle", PKG}}


def imported_modules(path):
    tree = ast.parse(open(path).read(), filename=path)
    mods = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            mods.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.level == 0 and node.module:
            mods.add(node.module.split(".")[0])
        elif isinstance(node, ast.Call) and getattr(node.func, "attr", getattr(node.func, "id", "")) in (
                "import_module", "__import__") and node.args and isinstance(node.args[0], ast.Constant):
            mods.add(str(node.args[0].value).split(".")[0])
    return mods


def test_packages_do_not_import_each_other():
    bad = []
    for pkg, forbidden in FORBIDDEN.items():
        files = glob.glob(os.path.join(ROOT, pkg, "**", "*.py"), recursive=True)
        assert files, f"no Python files under {pkg}/"
        for f in files:
            hit = imported_modules(f) & forbidden
            if hit:
                bad.append(f"{os.path.relpath(f, ROOT)} imports {sorted(hit)}")
    assert not bad, "\n".join(bad)


def test_native_sources_share_nothing_with_the_oracle():
    # the oracle is pure Python; no native source or build file names it
    for f in glob.glob(os.path.join(ROOT, PKG, "csrc", "*")) + glob.glob(os.path.join(ROOT, "include", "*")):
        assert "oracle" not in open(f, errors="replace").read(), f"{os.path.relpath(f, ROOT)} names the oracle"


def test_bench_uses_the_oracle_only_in_its_cpu_baseline():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    users = set()
    for fn in [n for n in ast.walk(tree) if isinstance(n, ast.FunctionDef)]:
        for node in ast.walk(fn):
            if isinstance(node, (ast.Import, ast.ImportFrom)):
                names = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module or ""]
                if any(n.split(".")[0] == "oracle" for n in names):
                    users.add(fn.name)
    top = [n for n in tree.body if isinstance(n, (ast.Import, ast.ImportFrom))]
    assert not any("oracle" in ast.dump(n) for n in top), "bench.py imports the oracle at module level"
    assert users and all(u.startswith("cpu_baseline") for u in users), sorted(users)
