"""Structural guards (CPU): the product path never reaches the oracle, the
oracle never reaches the product path, the input generators hold neither,
and the binding fails loudly, with no fallback, when libvl.so is missing."""
import ast
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "vocab_softmax_loss_amd")


def imported_modules(path):
    tree = ast.parse(open(path).read(), filename=path)
    mods = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            mods.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module:
            mods.add(node.module.split(".")[0])
    return mods


def py_files(d):
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(".py"):
                yield os.path.join(root, f)


def test_package_never_imports_the_oracle():
    for f in py_files(PKG):
        assert "oracle" not in imported_modules(f), f
    for f in os.listdir(os.path.join(PKG, "csrc")):
        text = open(os.path.join(PKG, "csrc", f)).read()
        assert "oracle" not in text.lower(), f


def test_oracle_never_imports_the_package():
    for f in py_files(os.path.join(ROOT, "oracle")):
        mods = imported_modules(f)
        assert "vocab_softmax_loss_amd" not in mods and "torch" not in mods, f
    text = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert "vl.h" not in text and "vl_device" not in text and "vl_launch" not in text


def test_input_generators_hold_neither_side():
    for f in py_files(os.path.join(ROOT, "gen")):
        mods = imported_modules(f)
        assert "oracle" not in mods and "vocab_softmax_loss_amd" not in mods, f


def test_binding_fails_loudly_without_the_library(tmp_path):
    # a copy of the package without libvl.so: importing it must raise
    dst = tmp_path / "vocab_softmax_loss_amd"
    dst.mkdir()
    shutil.copy(os.path.join(PKG, "__init__.py"), dst / "__init__.py")
    code = ("import sys; sys.path.insert(0, sys.argv[1])\n"
            "try:\n"
            "    import vocab_softmax_loss_amd\n"
            "except ImportError as e:\n"
            "    print('ImportError:', e); sys.exit(3)\n"
            "sys.exit(0)\n")
    r = subprocess.run([sys.executable, "-c", code, str(tmp_path)], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 3, r.stdout + r.stderr
    assert "libvl.so" in r.stdout
