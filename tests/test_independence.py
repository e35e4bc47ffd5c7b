"""The oracle and the HIP path share no code: neither imports the other."""
import ast
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _imports(path):
    names = set()
    for dirpath, _, files in os.walk(path):
        for f in files:
            if f.endswith(".py"):
                tree = ast.parse(open(os.path.join(dirpath, f)).read())
                for node in ast.walk(tree):
                    if isinstance(node, ast.Import):
                        names.update(a.name.split(".")[0] for a in node.names)
                    elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
                        names.add(node.module.split(".")[0])
    return names


def test_oracle_does_not_import_product():
    assert "block_ar_canvas_amd" not in _imports(os.path.join(ROOT, "oracle"))


def test_product_does_not_import_oracle():
    assert "oracle" not in _imports(os.path.join(ROOT, "block_ar_canvas_amd"))


def test_input_module_is_standalone():
    imp = _imports(os.path.join(ROOT, "dg_inputs"))
    assert "oracle" not in imp and "block_ar_canvas_amd" not in imp


def test_product_sources_do_not_mention_oracle_paths():
    csrc = os.path.join(ROOT, "block_ar_canvas_amd")
    for dirpath, _, files in os.walk(csrc):
        for f in files:
            if f.endswith((".hip", ".h", ".cpp", ".py")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle/" not in text and "import oracle" not in text, f
