"""Format the parity figures the GPU tests append to $FA_PARITY_LOG as a markdown table.

Usage: FA_PARITY_LOG=out.jsonl python -m pytest tests -m gpu ...; then
       python tests/parity_table.py out.jsonl [test-name filter ...]
One line per (test, workload): rows compared, max / mean |dO|, max |dL| and the counts
of elements above 1e-2 split by |O_ref| (< 2, [2, 4), >= 4) with the faithful-rounding
exceptions taken at >= 4.
"""
import json
import sys


def main(path, filters):
    rows = [json.loads(line) for line in open(path)]
    if filters:
        rows = [r for r in rows if any(f in r.get("test", "") for f in filters)]
    print("| test | workload | shape B,H,Nq,Nk,d | dtype | causal | sigma_qk | rows | max abs dO | "
          "mean abs dO | max abs dL | >1e-2 at abs O_ref <2 / [2,4) / >=4 | faithful at >=4 |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        test = r.get("test", "").split("::")[-1]
        over = (f"{r['over_lt2']} / {r['over_2_4']} / {r['over_ge4']}" if "over_lt2" in r else "n/a (fp32)")
        print(f"| {test} | {r['workload']} | {r['B']},{r['H']},{r['Nq']},{r['Nk']},{r['d']} | "
              f"{r['dtype']} | {int(r['causal'])} | {r['sigma_qk']:g} | {r['rows']} | "
              f"{r['max_do']:.3e} | {r['mean_do']:.3e} | {r['max_dl']:.3e} | {over} | "
              f"{r.get('faithful_ge4', 0)} |")


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2:])
