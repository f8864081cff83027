"""Host check of bench.py's line assembly: every key the per-workload
summaries read from a leg's result exists in the result dict that leg
builds (read from the source, so no GPU run is needed to catch a summary
that would fail at the end of a long bench run)."""
import ast
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _functions():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    return {n.name: n for n in ast.walk(tree) if isinstance(n, ast.FunctionDef)}


def _result_keys(fn):
    """Top-level string keys of the dict literal assigned to `result`, plus
    keys added later as result["..."] = ... or by a conditional key
    expression (both alternatives)."""
    keys = set()
    for node in ast.walk(fn):
        if isinstance(node, ast.Assign) and any(isinstance(t, ast.Name) and t.id == "result" for t in node.targets) \
                and isinstance(node.value, ast.Dict):
            for k in node.value.keys:
                if isinstance(k, ast.Constant):
                    keys.add(k.value)
                elif isinstance(k, ast.IfExp):
                    keys.update(x.value for x in (k.body, k.orelse) if isinstance(x, ast.Constant))
        if isinstance(node, ast.Assign):
            for t in node.targets:
                if isinstance(t, ast.Subscript) and isinstance(t.value, ast.Name) and t.value.id == "result" \
                        and isinstance(t.slice, ast.Constant):
                    keys.add(t.slice.value)
    return keys


def _read_keys(fn):
    """Keys read unconditionally as r["..."] (reads guarded by `if k in r`
    are comprehension variables, not constants, and are skipped)."""
    return {n.slice.value for n in ast.walk(fn)
            if isinstance(n, ast.Subscript) and isinstance(n.value, ast.Name) and n.value.id == "r"
            and isinstance(n.slice, ast.Constant)}


def test_summaries_read_only_keys_their_legs_write():
    f = _functions()
    for summary, leg in (("summarise_decode", "decode_leg"), ("summarise_select", "bench_select")):
        missing = _read_keys(f[summary]) - _result_keys(f[leg])
        assert not missing, f"{summary} reads {sorted(missing)}, which {leg} does not write"
