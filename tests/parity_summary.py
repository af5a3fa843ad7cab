"""Condense a parity log (the file RQ_PARITY_LOG names while the GPU tests run)
into a short text summary: per test, the packed-code comparisons (elements,
boundary exemptions, mismatches) and the worst attention error against the
oracle; then the records kept verbatim (full-size runs, query precision).

    python3 tests/parity_summary.py LOG [GENERATING_COMMAND]
"""
import re
import sys
from collections import OrderedDict

CODES = re.compile(r"elements=(\d+) exempt=(\d+) \(frac [^)]*\) meta_exempt=(\d+) alpha_exempt=(\d+) bad=(\d+)")
ERR = re.compile(r"max rel err ([0-9.eE+-]+)")
VERBATIM = ("sharp logits", "attention max rel err", "precise", "saturat", "fp16 range")


def summarize(path: str, command: str = "") -> str:
    tests = OrderedDict()
    keep = []
    for line in open(path):
        test, _, msg = line.rstrip("\n").partition("\t")
        t = tests.setdefault(test, {"elements": 0, "exempt": 0, "meta": 0, "alpha": 0, "bad": 0, "cmp": 0,
                                    "err": 0.0, "nerr": 0})
        m = CODES.search(msg)
        if m:
            e, x, me, ae, b = map(int, m.groups())
            t["elements"] += e
            t["exempt"] += x
            t["meta"] += me
            t["alpha"] += ae
            t["bad"] += b
            t["cmp"] += 1
        m = ERR.search(msg)
        if m:
            t["err"] = max(t["err"], float(m.group(1)))
            t["nerr"] += 1
        if any(k in msg for k in VERBATIM):
            keep.append(f"{test.split('::')[-1]}\t{msg}")
    out = [f"# parity summary of {sum(1 for _ in open(path))} records from {len(tests)} tests"]
    if command:
        out.append(f"# log made by: {command}")
    out.append(f"# summary made by: python3 tests/parity_summary.py {path}")
    out.append("test\tcode_comparisons\telements\texempt\tmeta_exempt\talpha_exempt\tbad\tattention_checks\tworst_rel_err")
    tot = {"elements": 0, "exempt": 0, "bad": 0, "err": 0.0}
    for test, t in tests.items():
        out.append(f"{test}\t{t['cmp']}\t{t['elements']}\t{t['exempt']}\t{t['meta']}\t{t['alpha']}\t{t['bad']}\t"
                   f"{t['nerr']}\t{t['err']:.3e}")
        for k in ("elements", "exempt", "bad"):
            tot[k] += t[k]
        tot["err"] = max(tot["err"], t["err"])
    out.append(f"# total: {tot['elements']} code elements compared, {tot['exempt']} exempted, {tot['bad']} mismatched; "
               f"worst attention max rel err {tot['err']:.3e}")
    out.append("# records kept verbatim")
    out.extend(keep)
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    print(summarize(sys.argv[1], sys.argv[2] if len(sys.argv) > 2 else ""), end="")
