"""Write tests/golden/oracle_sha256.json: SHA-256 of the oracle's outputs on seeded inputs.

Calls only `oracle` and `synth`.  A later change to the oracle's arithmetic that moves
any of these hashes has to say, in its commit message, which passage justifies it.
Run:  python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_sha256.json")


def sha(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def compute() -> dict:
    res = {}
    w = synth.config1().data
    r = oracle.quantize_rows(w, 31)
    res["input.config1"] = sha(w)
    res["config1.codes"] = sha(r["codes"])
    res["config1.scales"] = sha(r["scales"])
    res["config1.dq"] = sha(r["dq"])

    ts = synth.config2()
    res["input.config2"] = sha(*[t.data for t in ts])
    out = oracle.export([(t.name, t.data) for t in ts], oracle.Policy())
    res["config2.codes"] = sha(*[o["codes"] for o in out if "codes" in o])
    res["config2.scales"] = sha(*[o["scales"] for o in out if "scales" in o])
    res["config2.f16"] = sha(*[o["f16"] for o in out if "f16" in o])
    res["config2.dq"] = sha(*[o["dq"] for o in out])

    ws = synth.config3_weights(layers=1)
    gs = synth.config3_grads(0, layers=1)
    res["input.config3.layer0"] = sha(*[t.data for t in ws], *[g.data for g in gs])
    fq = [oracle.fakequant_rows(t.data, 31, 1, 1, g_bf16=g.data) for t, g in zip(ws, gs)]
    res["config3.layer0.dq"] = sha(*[f["dq"] for f in fq])
    res["config3.layer0.scales"] = sha(*[f["scales"] for f in fq])
    res["config3.layer0.mask"] = sha(*[f["mask"] for f in fq])
    res["config3.layer0.g_out"] = sha(*[f["g_out"] for f in fq])

    ts4 = synth.config4()
    out4 = oracle.export([(t.name, t.data) for t in ts4], oracle.Policy(q6=(6, 1, 1)),
                         awq={t.name: t.awq_s for t in ts4 if t.awq_s is not None})
    res["input.config4"] = sha(*[t.data for t in ts4], *[t.awq_s for t in ts4 if t.awq_s is not None])
    res["config4.codes"] = sha(*[o["codes"] for o in out4])
    res["config4.scales"] = sha(*[o["scales"] for o in out4])
    res["config4.awq"] = sha(*[o["awq"] for o in out4 if "awq" in o])
    res["config4.dq"] = sha(*[o["dq"] for o in out4])
    return res


if __name__ == "__main__":
    res = compute()
    with open(OUT, "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
        f.write("\n")
    print(f"wrote {len(res)} hashes to {OUT}")
