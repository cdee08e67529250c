"""Write tests/golden/tiny_bruteforce.json and tiny_bruteforce_tau.json (run
from the repository root).

The pages print no worked example, so the stored values are computed here by
the 50-digit brute-force implementation in ``oracle/bruteforce.py`` (plain
loops over the definition: per unmasked position, KL of the renormalised top-K
teacher distribution from the full-vocabulary student distribution at the K
cached ids, summed; gradients by central differences).  The definition
follows the agentlenshq.com page "LLMのための効率的な知識蒸留…", sections
"1. Top-K Logit Cachingによるオフライン蒸留" and "2. Fused Chunked KL Loss".
This script calls only ``oracle/`` and the seeded tiny cases.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

import mpmath  # noqa: E402

from oracle import bruteforce  # noqa: E402
from oracle_cases import TINY, case_problem  # noqa: E402


def s(x):
    return mpmath.nstr(x, 30)


def main():
    out = {"source": "oracle/bruteforce.py at 50 digits; definition per the agentlenshq.com page, "
                     "sections '1. Top-K Logit Cachingによるオフライン蒸留' and '2. Fused Chunked KL Loss'",
           "cases": []}
    for spec in TINY:
        name, n, d, v, k, seed, masked = spec
        H, W, ids, a, mask = case_problem(spec)
        L, lses, rls = bruteforce.loss(H.tolist(), W.tolist(), ids.tolist(), a.tolist(),
                                       None if mask is None else mask.tolist())
        dH, dW = bruteforce.grad_fd(H.tolist(), W.tolist(), ids.tolist(), a.tolist(),
                                    None if mask is None else mask.tolist(), g=0.37)
        out["cases"].append({
            "name": name, "n": n, "d": d, "v": v, "k": k, "seed": seed, "masked": list(masked),
            "H": H.tolist(), "W": W.tolist(), "t_ids": ids.tolist(), "t_logits": a.tolist(),
            "g": 0.37,
            "loss": s(L), "lse": [s(x) for x in lses], "row_loss": [s(x) for x in rls],
            "dH": [[s(x) for x in r] for r in dH], "dW": [[s(x) for x in r] for r in dW],
        })
    path = os.path.join(ROOT, "tests", "golden", "tiny_bruteforce.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)

    # temperature: the same brute force with the teacher and student logits
    # divided by tau and the sum multiplied by tau^2 (the usual
    # temperature-scaled distillation loss; the aihot.vn page, section
    # "Mô hình học sinh thu được", reports loss-choice ablations without
    # defining any)
    out = {"source": "oracle/bruteforce.py at 50 digits with a temperature tau: teacher softmax(a / tau), "
                     "student softmax(z / tau), tau^2 times the KL at the K ids",
           "cases": []}
    for spec, tau in [(TINY[0], 2.5), (TINY[2], 0.6), (TINY[3], 1.7)]:
        name, n, d, v, k, seed, masked = spec
        H, W, ids, a, mask = case_problem(spec)
        mk = None if mask is None else mask.tolist()
        L, lses, rls = bruteforce.loss(H.tolist(), W.tolist(), ids.tolist(), a.tolist(), mk, tau=tau)
        dH, dW = bruteforce.grad_fd(H.tolist(), W.tolist(), ids.tolist(), a.tolist(), mk, g=0.37, tau=tau)
        out["cases"].append({
            "name": f"{name}-tau{tau}", "n": n, "d": d, "v": v, "k": k, "seed": seed, "masked": list(masked),
            "H": H.tolist(), "W": W.tolist(), "t_ids": ids.tolist(), "t_logits": a.tolist(),
            "g": 0.37, "tau": tau,
            "loss": s(L), "lse": [s(x) for x in lses], "row_loss": [s(x) for x in rls],
            "dH": [[s(x) for x in r] for r in dH], "dW": [[s(x) for x in r] for r in dW],
        })
    path = os.path.join(ROOT, "tests", "golden", "tiny_bruteforce_tau.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
