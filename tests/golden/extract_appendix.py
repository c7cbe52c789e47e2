"""Writes tests/golden/appendix_acceptance_all.json from the text of the vLLM
blog post "speculative-decoding-amd-gpus", Appendix (per target model, drafting
method and dataset: one table row per proposal length N with the speed-up, the
throughput, MAL, AR and the per-position acceptance p1..pN in percent, as
printed).  Run once by hand where a text copy of the page is available:

    python tests/golden/extract_appendix.py PAGE_TEXT [--exclude-model NAME ...]

--exclude-model leaves out every table whose target model is NAME (the part
of the table title before the first " / ").  The committed JSON is what the
tests read; nothing reads the page at test time.
"""
import argparse
import json
import os
import re

ROW = re.compile(r"^N=(\d+)\s+([0-9.]+)x\s*\|\s*([0-9,]+)\s*tok/sMAL\s+([0-9.]+)\s*\|\s*AR\s+([0-9.]+)%\s*(.*)$")


def main(path, exclude=()):
    lines = open(path, encoding="utf-8").read().splitlines()
    start = next(i for i, l in enumerate(lines) if l.strip() == "Appendix")
    rows, table = [], None
    for l in lines[start:]:
        s = l.strip()
        if " / " in s and not s.startswith("N") and "tok/s" not in s and len(s) < 120:
            table = s
            continue
        m = ROW.match(s)
        if m and table and table.split(" / ")[0] not in exclude:
            N = int(m.group(1))
            p = [int(x) for x in re.findall(r"(\d+)%", m.group(6))]
            if len(p) != N:
                continue
            rows.append(dict(table=table, N=N, MAL=float(m.group(4)), AR=float(m.group(5)), p=p))
    out = dict(source="vLLM blog 'speculative-decoding-amd-gpus', Appendix tables: every row whose "
                      "per-position cells parse (N cells for proposal length N); MAL and AR as printed "
                      "(2 decimals, 1 decimal percent), p1..pN in whole percent.",
               rows=rows)
    dst = os.path.join(os.path.dirname(os.path.abspath(__file__)), "appendix_acceptance_all.json")
    with open(dst, "w") as f:
        json.dump(out, f, indent=0)
    print(f"{len(rows)} rows from {len({r['table'] for r in rows})} tables -> {dst}")


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("page_text")
    ap.add_argument("--exclude-model", action="append", default=[])
    args = ap.parse_args()
    main(args.page_text, tuple(args.exclude_model))
