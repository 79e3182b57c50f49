"""Summarize the GPU-vs-oracle parity records in this folder into SUMMARY.md.

The GPU tests (tests/test_gpu_parity.py) write parity_<workload>.jsonl: one
"quantize summary" line per compared vector set, one line per mismatch (each
must be a near-tie: an index within 1e-4 sigma of a threshold, a sign within
1e-4 ||r|| of zero, an fp16 scale within 1e-5 relative of a rounding midpoint),
and one line per decode comparison.  Copies of those files are kept here;
this script only counts what they hold.

    python tests/parity_records/summarize.py
"""
import glob
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def main():
    out = ["# GPU parity records", "",
           "Counts from the `parity_<workload>.jsonl` files beside this summary (written by "
           "`tests/test_gpu_parity.py` on an MI355X). Every mismatch is listed in those files with its "
           "tensor, sequence, head, token, coordinate, oracle and GPU value and its distance to the "
           "decision boundary. Index entries: near-tie band 1e-4/sqrt(d) in u units; sign entries: "
           "1e-4 rho = 1e-4 times the residual norm; at most 0.01 % of entries may differ, every one of them a near-tie.", ""]
    for path in sorted(glob.glob(os.path.join(HERE, "parity_*.jsonl"))):
        rows = [json.loads(l) for l in open(path)]
        run = next((r for r in rows if r.get("kind") == "run"), {})
        wl = os.path.basename(path)[len("parity_"):-len(".jsonl")]
        out += [f"## {wl}", "", f"Kernel sources: `{run.get('source_hash', '?')}`.", "",
                "| vectors compared | label | index entries | in band | mismatches | sign entries | in band "
                "| mismatches | fp16 scale near-ties | max rel err of nu | max rel err of rho |",
                "|---|---|---|---|---|---|---|---|---|---|---|"]
        for r in rows:
            if r.get("kind") != "quantize summary":
                continue
            f = lambda k: "-" if r.get(k) is None else r[k]
            g = lambda k: "-" if r.get(k) is None else f"{r[k]:.2e}"
            out.append(f"| {r['n_vectors']} | {r['label']} | {f('index_entries')} | {f('index_near_ties')} | "
                       f"{r['n_index_mismatch']} | {f('sign_entries')} | {f('sign_near_ties')} | "
                       f"{r['n_sign_mismatch']} | {r['n_scale_near_ties']} | {g('nu_max_rel')} | {g('rho_max_rel')} |")
        dec = [r for r in rows if r.get("kind") == "decode"]
        if dec:
            worst = max(dec, key=lambda r: r["err_over_maxV"])
            out += ["", f"Decode: {len(dec)} (sequence, kv head) outputs compared, worst "
                        f"{worst['err_over_maxV']:.2e} x max|V| ({worst['label']}, sequence {worst['sequence']}, "
                        f"kv head {worst['kv_head']}, {worst['length']} tokens); tolerance 1e-4 x max|V|."]
        mism = [r for r in rows if r.get("kind") in ("index", "sign")]
        if mism:
            far = max(r.get("distance_sigma", r.get("distance_rho", 0)) for r in mism)
            out += ["", f"Listed mismatches: {len(mism)}; the farthest from its boundary is {far:.2e} "
                        "(sigma units for indices, residual-norm units for signs), inside the 1e-4 band."]
        out.append("")
    with open(os.path.join(HERE, "SUMMARY.md"), "w") as fh:
        fh.write("\n".join(out))


if __name__ == "__main__":
    main()
