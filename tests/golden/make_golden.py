"""Write tests/golden/oracle_small.json: oracle results for small seeded cases.

Calls only the CPU oracle (``oracle/``) on inputs from the seeded generator
(``datagen``); nothing here comes from the HIP library.  The fixture guards
the oracle and the generator against silent drift: a change to either that
alters these values must be deliberate and re-run this script.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import datagen  # noqa: E402
import oracle  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small.json")


def cases():
    """(name, inputs) for the fixture: a plain RMSNorm with a ragged hidden,
    an outlier row set, and an RMSNorm+RoPE case with rows > seq_len."""
    yield "rms_3x40", dict(x=datagen.make_x(3, 40, seed=77, stream=1),
                           w=datagen.make_w(40, seed=77, stream=2), eps=1e-6)
    yield "rms_2x64_outliers", dict(x=datagen.make_x(2, 64, seed=78, stream=1, sigma=2.0,
                                                     outlier_p=0.05, outlier_scale=50.0),
                                    w=None, eps=1e-6)
    c, s = datagen.rope_tables(3, 16, 10000.0)
    yield "rope_5x32_h2d16_seq3", dict(x=datagen.make_x(5, 32, seed=79, stream=1),
                                       w=datagen.make_w(32, seed=79, stream=2), eps=1e-6,
                                       cos=c, sin=s, heads=2, head_dim=16)
    yield "ropei_5x32_h2d16_seq3", dict(x=datagen.make_x(5, 32, seed=80, stream=1),
                                        w=datagen.make_w(32, seed=80, stream=2), eps=1e-6,
                                        cos=c, sin=s, heads=2, head_dim=16, interleaved=True)


def compute(o, inp):
    if "cos" in inp:
        y = o.rmsnorm_rope(inp["x"], inp["w"], inp["cos"], inp["sin"], inp["heads"],
                           inp["head_dim"], inp["eps"], interleaved=inp.get("interleaved", False))
    else:
        y = o.rmsnorm(inp["x"], inp["w"], inp["eps"])
    ref32, ref16 = o.round(y)
    return ref32, ref16


def main():
    o = oracle.Oracle()
    doc = {"generated_by": "tests/golden/make_golden.py (CPU oracle only)", "cases": {}}
    for name, inp in cases():
        ref32, ref16 = compute(o, inp)
        doc["cases"][name] = {
            "x_fnv": datagen.fnv1a64(inp["x"]),
            "ref32_hex": [format(int(v), "08x") for v in ref32.view("uint32").reshape(-1)],
            "ref16_hex": [format(int(v), "04x") for v in ref16.reshape(-1)],
        }
    with open(OUT, "w") as f:
        json.dump(doc, f, indent=0)
        f.write("\n")
    print("wrote", OUT)


if __name__ == "__main__":
    main()
