"""Runs the oracle's pins (tests/test_oracle_pins.py, tests/test_lmhead_cpu.py) against another build of
the oracle library, given as a path: the planted-mutation check of
tests/test_oracle_mutants.py starts one process per mutant with this script.

Exit status 0: every pin passed. 1: some pin failed (its name is printed).
"""
import ctypes
import inspect
import os
import sys
import traceback

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)

import oracle  # noqa: E402


def main(lib_path):
    oracle._lib = oracle._configure(ctypes.CDLL(lib_path))
    import test_lmhead_cpu
    import test_oracle_pins
    from beam_search_top_amd import synth
    fns = []
    for mod in (test_oracle_pins, test_lmhead_cpu):
        fns += sorted(inspect.getmembers(mod, inspect.isfunction), key=lambda kv: kv[1].__code__.co_firstlineno)
    for name, fn in fns:
        if fn.__module__ not in ("test_oracle_pins", "test_lmhead_cpu"):
            continue
        if not name.startswith("test_"):
            continue
        args = inspect.signature(fn).parameters
        calls = [dict(dtype=d) for d in (synth.F32, synth.F16, synth.BF16)] if "dtype" in args else [{}]
        for kw in calls:
            try:
                fn(**kw)
            except Exception:  # an assertion of a pin (or an error it raised) catches the mutant
                print(f"caught by {name}{kw or ''}:", traceback.format_exc(limit=1).strip().splitlines()[-1],
                      flush=True)
                return 1
    print("every pin passed", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
