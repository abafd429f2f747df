"""Turn the parity records of a GPU test session into a markdown table.

The GPU tests record every comparison with the fp64 oracle when the session
runs with ATTN_PARITY_RECORD=<file> (tests/conftest.py writes one JSON object
a line). This prints, for each full-size workload test, the plain max-abs
error of the output and of the LSE, and a summary of the edge-case tests.

    python tests/parity_report.py parity_records.jsonl
"""

import json
import sys

# full-size workload tests (every output element compared), in workload order
FULL_SIZE = [
    ("1 tiny varlen", "test_gpu_varlen.py::test_config1_tiny_full_parity"),
    ("2 dense DiT", "test_gpu_varlen.py::test_full_size_config_every_row[config2]"),
    ("3 causal GQA varlen", "test_gpu_varlen.py::test_full_size_config_every_row[config3]"),
    ("4 paged decode", "test_gpu_paged.py::test_config4_full_size_every_sequence"),
    ("5 video block-sparse", "test_gpu_sparse.py::test_config5_full_size_with_oracle_map_every_tile"),
    ("6 chunked paged prefill", "test_gpu_paged_prefill.py::test_chunked_prefill_full_size_every_row"),
    ("7 speculative decode", "test_gpu_paged_prefill.py::test_spec_decode_full_size_every_row"),
    ("8 sliding-window decode", "test_gpu_variants.py::test_sliding_window_decode_full_size_every_sequence"),
    ("9 masked cross-attention", "test_gpu_variants.py::test_masked_cross_full_size"),
    ("10 padded batch", "test_gpu_variants.py::test_padded_full_size"),
    ("head_dim 64 dense 2 x 4096, 24 heads", "test_gpu_varlen.py::test_head_dim_full_size_every_row[64-False]"),
    ("head_dim 96 dense 2 x 4096, 24 heads", "test_gpu_varlen.py::test_head_dim_full_size_every_row[96-False]"),
    ("head_dim 192 dense 2 x 4096, 24 heads", "test_gpu_varlen.py::test_head_dim_full_size_every_row[192-False]"),
    ("head_dim 256 dense 2 x 4096, 24 heads", "test_gpu_varlen.py::test_head_dim_full_size_every_row[256-False]"),
    ("head_dim 256 causal 2 x 4096, 24 heads", "test_gpu_varlen.py::test_head_dim_full_size_every_row[256-True]"),
]


def main(path):
    recs = [json.loads(line) for line in open(path) if line.strip()]
    by_test = {}
    for r in recs:
        by_test.setdefault(r["test"].split("tests/")[-1], []).append(r)
    print("| Workload | Elements | Output max-abs | Output max |ref| | LSE max-abs | Bound |")
    print("|---|---|---|---|---|---|")
    for label, test in FULL_SIZE:
        rs = by_test.get(test, [])
        out = [r for r in rs if r["name"] == "out"]
        lse = [r for r in rs if r["name"] == "lse"]
        if not out:
            print(f"| {label} | — | not recorded | | | |")
            continue
        o = max(out, key=lambda r: r["max_abs"])
        lmax = max((r["max_abs"] for r in lse), default=float("nan"))
        bound = "1e-2 flat (half-ulp above |O| 4)" if not o.get("few_keys") else "1e-2 + half-ulp"
        print(f"| {label} | {o['elements']} | {o['max_abs']:.2e} | {o['max_abs_ref']:.2f} | {lmax:.2e} | {bound} |")
    named = {t for _, t in FULL_SIZE}
    edge = [r for t, rs in by_test.items() if t not in named for r in rs]
    eo = [r for r in edge if r["name"] != "lse"]
    el = [r for r in edge if r["name"] == "lse"]
    fk = [r for r in eo if r.get("few_keys")]
    st = [r for r in eo if not r.get("few_keys")]
    print()
    print(f"Other comparisons: {len(eo)} output and {len(el)} LSE records over "
          f"{len({r['test'] for r in edge})} tests.")
    if st:
        print(f"- flat bound: {len(st)} records, worst max-abs {max(r['max_abs_below_flat_limit'] for r in st):.2e} "
              f"below |O| 4")
    if fk:
        print(f"- few-keys bound: {len(fk)} records, worst max-abs {max(r['max_abs'] for r in fk):.2e}, "
              f"worst below |O| 4 {max(r['max_abs_below_flat_limit'] for r in fk):.2e}")
    if el:
        print(f"- LSE: worst max-abs {max(r['max_abs'] for r in el):.2e}")
    print(f"- over their bound: {sum(r['over_tol'] for r in recs)} elements")


if __name__ == "__main__":
    main(sys.argv[1])
