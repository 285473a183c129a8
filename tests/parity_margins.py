"""Summarise a GPU run's parity log into a markdown table.

    KDA_PARITY_LOG=margins.jsonl python -m pytest tests -m gpu ...
    python tests/parity_margins.py margins.jsonl "<command that made the log>" > profiles/parity_margins.md

Each line of the log is one case of a GPU parity test (written by
kda_testutil.report): its measured max|gpu - ref| / max|ref| per tensor.
The bar of a value is 1e-4 for cases on fp32 inputs and 1e-2 otherwise;
"y_err_over_bar" (the layer's gated output) is already a ratio to its
row-wise bar (1.0); "carried" (how much of a final state came from before the
checked span) and "o_own_max" (a packed sequence divided by its own maximum,
stricter than the metric) are reported without a bar.
"""
import json
import sys

INFO = {"carried", "o_own_max", "ok", "G_abs"}
NAMED = ("tiny_fp32", "prefill_4k", "varlen_8", "long_1m", "decode_256")


def bar_of(case: str, key: str):
    if key in INFO:
        return None
    if key == "y_err_over_bar":
        return 1.0
    return 1e-4 if "fp32" in case else 1e-2


def main(path: str, command: str) -> None:
    rows = [json.loads(line) for line in open(path) if line.strip()]
    worst = {}
    for r in rows:
        for key, val in r["errors"].items():
            bar = bar_of(r["case"], key)
            if bar is None:
                continue
            k = (r["suite"], key, bar)
            if k not in worst or val / bar > worst[k][0] / bar:
                worst[k] = (val, r["case"], r["test"])
    print("# Parity margins of the GPU tests\n")
    print("Every GPU parity case's measured max|gpu - ref| / max|ref| per tensor against")
    print("the fp64 oracle (bars: 1e-2 for bf16 inputs on the MFMA path, 1e-4 for the")
    print("fp32 path; the layer's gated output is held row by row, its value is the")
    print("largest ratio of a row's error to that row's bound).  Command:\n")
    print(f"    {command}\n")
    print(f"{len(rows)} cases logged.\n")
    print("## Worst case of each kind\n")
    print("| suite | value | bar | worst | of bar | case |")
    print("|---|---|---|---|---|---|")
    for (suite, key, bar), (val, case, _) in sorted(worst.items()):
        print(f"| {suite} | {key} | {bar:g} | {val:.3e} | {val / bar:.0%} | {case} |")
    print("\n## The named workloads and the composition pins\n")
    print("| test | case | values |")
    print("|---|---|---|")
    for r in rows:
        if r["suite"] != "composition" and not r["case"].startswith(NAMED):
            continue
        vals = ", ".join(f"{k} {v:.2e}" for k, v in r["errors"].items())
        test = r["test"].split("::", 1)[-1]
        print(f"| {test} | {r['case']} | {vals} |")


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2] if len(sys.argv) > 2 else "(command not given)")
