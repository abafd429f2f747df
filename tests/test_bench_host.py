"""Host-side checks of bench.py's bookkeeping (no GPU): the traffic records
are tied to the code of the kernel sources they were measured on."""

import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_code_only_strips_comments_but_not_strings():
    b = _bench()
    src = 'int a = 1;  // note\n/* block\n   comment */\nconst char* s = "x // y \\" /* z */";\n\n   \nint b;\n'
    assert b.code_only(src) == 'int a = 1;\nconst char* s = "x // y \\" /* z */";\nint b;'


def test_comment_edits_keep_the_hash_and_code_edits_change_it():
    b = _bench()
    base = "__global__ void k(int* p) {\n  p[0] = 1;  // store\n}\n"
    assert b.code_only(base) == b.code_only("// a kernel\n" + base.replace("// store", "// the store"))
    assert b.code_only(base) != b.code_only(base.replace("p[0] = 1", "p[0] = 2"))


def test_traffic_records_are_well_formed():
    # a record whose sources changed since it was measured reports null (the
    # bench line then carries "traffic": null until the counters are taken again)
    b = _bench()
    for name, rec in b.TRAFFIC.items():
        assert rec["kernel"], name
        if "fetch_kib" not in rec:  # no counters taken for this workload: traffic is null
            assert b.traffic_bytes(name) is None
            continue
        assert rec["fetch_kib"] > 0 and rec["write_kib"] > 0, name
        assert len(rec["sha256"]) == 16 and int(rec["sha256"], 16) >= 0, name
        for f in rec["sources"]:
            assert os.path.exists(os.path.join(b.CSRC, f)), (name, f)
        t = b.traffic_bytes(name)
        assert t is None or t == int(round((rec["fetch_kib"] * b.FETCH_SCALE + rec["write_kib"] * b.WRITE_SCALE) * 1024))
