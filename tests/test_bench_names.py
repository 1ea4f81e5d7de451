"""Static check of bench.py, which only runs on a GPU: every name a function
reads is bound somewhere it can see (its own parameters and assignments, an
enclosing function, the module, or the builtins). A leg that reads a name
bound only in another leg would otherwise surface as a NameError at the end
of a GPU run."""
import ast
import builtins
import pathlib

import pytest

BENCH = pathlib.Path(__file__).resolve().parent.parent / "bench.py"


def _bound(node):
    """Names bound directly in a function body (not in nested functions)."""
    out = set()
    a = node.args
    for arg in a.posonlyargs + a.args + a.kwonlyargs + [x for x in (a.vararg, a.kwarg) if x]:
        out.add(arg.arg)
    stack = list(node.body)
    while stack:
        n = stack.pop()
        if isinstance(n, (ast.FunctionDef, ast.AsyncFunctionDef, ast.ClassDef)):
            out.add(n.name)
            continue
        if isinstance(n, ast.Lambda):
            continue
        if isinstance(n, ast.Name) and isinstance(n.ctx, (ast.Store, ast.Del)):
            out.add(n.id)
        elif isinstance(n, (ast.Import, ast.ImportFrom)):
            for al in n.names:
                out.add((al.asname or al.name).split(".")[0])
        elif isinstance(n, ast.ExceptHandler) and n.name:
            out.add(n.name)
        elif isinstance(n, (ast.Global, ast.Nonlocal)):
            out.update(n.names)
        stack.extend(ast.iter_child_nodes(n))
    return out


def _comp_bound(node):
    out = set()
    for n in ast.walk(node):
        if isinstance(n, ast.comprehension):
            for t in ast.walk(n.target):
                if isinstance(t, ast.Name):
                    out.add(t.id)
    return out


def _unbound(tree):
    module = _bound(ast.FunctionDef(name="<module>", args=ast.arguments(
        posonlyargs=[], args=[], vararg=None, kwonlyargs=[], kw_defaults=[], kwarg=None, defaults=[]),
        body=tree.body, decorator_list=[]))
    missing = []

    def visit(fn, scopes):
        here = _bound(fn) if not isinstance(fn, ast.Lambda) else {a.arg for a in fn.args.args}
        here |= _comp_bound(fn)
        env = scopes + [here]
        stack = list(fn.body) if not isinstance(fn, ast.Lambda) else [fn.body]
        while stack:
            n = stack.pop()
            if isinstance(n, (ast.FunctionDef, ast.AsyncFunctionDef, ast.Lambda)):
                visit(n, env)
                continue
            if isinstance(n, ast.Name) and isinstance(n.ctx, ast.Load):
                if not any(n.id in s for s in env) and n.id not in module and not hasattr(builtins, n.id):
                    missing.append((getattr(fn, "name", "<lambda>"), n.id, n.lineno))
            stack.extend(ast.iter_child_nodes(n))

    for top in tree.body:
        if isinstance(top, (ast.FunctionDef, ast.AsyncFunctionDef)):
            visit(top, [])
    return missing


def test_every_name_read_in_bench_is_bound():
    missing = _unbound(ast.parse(BENCH.read_text()))
    assert not missing, missing


def test_the_check_sees_a_name_bound_only_in_another_function():
    src = "def a():\n    x = 1\n    return x\n\ndef b():\n    return x\n"
    assert [m[:2] for m in _unbound(ast.parse(src))] == [("b", "x")]
