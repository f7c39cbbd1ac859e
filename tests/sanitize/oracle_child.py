"""Child process of tests/test_sanitizers.py: the oracle recurrence from a
sanitizer build (its path in argv[1]) on small problems, compared bit for bit
with the results of the normal build stored in argv[2] (.npz)."""
import importlib
import sys

import numpy as np

# the module itself (the package exports a function of the same name)
rec = importlib.import_module("oracle.recurrence")

rec._LIB = sys.argv[1]
ref = np.load(sys.argv[2])
n = 0
for key in sorted(k for k in ref.files if k.endswith("_q")):
    name = key[:-2]
    get = lambda f: ref[f"{name}_{f}"]
    s0 = get("s0") if f"{name}_s0" in ref.files else None
    o, s = rec.recurrence(get("q"), get("k"), get("v"), get("g"), get("beta"),
                          float(get("scale")), s0, rule=str(get("rule")))
    assert np.array_equal(o, get("o")) and np.array_equal(s, get("s")), name
    n += 1
print(f"sanitized oracle: {n} problems equal the normal build bit for bit")
