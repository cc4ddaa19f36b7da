"""Host-side checks of the profile tooling: the decode-source hash that ties a
committed traffic summary to the kernel code it was measured on follows the
code and ignores comments and layout, and traffic summaries scale the
counters by the copy of known size and count only the call they are for."""
from paged_kv_cache_260_amd import profiling


def test_code_text_drops_comments_and_layout():
    src = ('int a = 1; // trailing\n/* block\n   comment */ const char *s = "a // b /* c */";\n'
           "char q = '\"';\n  int   b;\n")
    assert profiling.code_text(src) == 'int a = 1; const char *s = "a // b /* c */"; char q = \'"\'; int b;'


def test_code_text_follows_code_changes():
    base = "x = y + 1; // note\n"
    assert profiling.code_text(base) == profiling.code_text("x = y + 1;   // other note\n\n")
    assert profiling.code_text(base) != profiling.code_text("x = y + 2; // note\n")
    assert profiling.code_text('s = "//";') == 's = "//";'


def test_source_hash_is_stable():
    assert profiling.source_hash() == profiling.source_hash()
    assert len(profiling.source_hash()) == 16


# --- traffic summaries from counter CSVs (rocprofv3's column names) ---------

_SHARED = "_ZN3pkv12_GLOBAL__N_119paged_decode_kernelIDF16_Li128ELi16ELb0ELi4EEEvNS_10DecodeArgsE"
_PLAIN = "_ZN3pkv12_GLOBAL__N_119paged_decode_kernelIDF16_Li128ELi4ELb0ELi0EEEvNS_10DecodeArgsE"


def _write_csv(path, header, rows):
    with open(path, "w") as f:
        f.write(",".join(header) + "\n")
        for r in rows:
            f.write(",".join(str(x) for x in r) + "\n")


def _counter_rows(counter, per_kernel):
    rows, d = [], 0
    for name, values in per_kernel:
        for v in values:
            rows.append((d, name, counter, v))
            d += 1
    return rows


def _inputs(tmp_path):
    stats = tmp_path / "stats.csv"
    _write_csv(stats, ["Name", "Calls", "AverageNs", "Percentage", "MinNs", "MaxNs"],
               [(_SHARED, 3, 36000, 40.0, 35000, 37000), (_PLAIN, 3, 41000, 60.0, 40000, 42000)])
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    # a 2 GiB copy reads half its KiB on FETCH_SIZE and all of them on WRITE_SIZE
    copy_kib = 2 * 2 ** 30 / 1024
    fetch = tmp_path / "fetch.csv"
    _write_csv(fetch, hdr, _counter_rows("FETCH_SIZE", [("copyBuffer", [copy_kib / 2]),
                                                        (_SHARED, [999.0, 1000.0, 1000.0]),
                                                        (_PLAIN, [5000.0, 4000.0, 4000.0])]))
    write = tmp_path / "write.csv"
    _write_csv(write, hdr, _counter_rows("WRITE_SIZE", [("copyBuffer", [copy_kib]),
                                                        (_SHARED, [10.0, 10.0, 10.0]),
                                                        (_PLAIN, [20.0, 20.0, 20.0])]))
    return stats, fetch, write


def test_traffic_counts_only_the_named_call(tmp_path):
    """A run that times two kinds of call: --only keeps the other out of the
    per-call total; FETCH_SIZE is scaled by what the copy of known size read
    (x2 here), WRITE_SIZE likewise (x1), and the first (cold) dispatch of a
    kernel is left out of its average."""
    stats, fetch, write = _inputs(tmp_path)
    out = tmp_path / "out"
    r = profiling.summarize("t", "cmd", str(stats), str(fetch), str(write), 1000 * 2048, 2 * 2 ** 30, str(out),
                            only=["paged_decode_kernel (shared prefix, one launch)"])
    assert list(r["per_kernel"]) == ["paged_decode_kernel (shared prefix, one launch)"]
    assert abs(r["fetch_scale"] - 2.0) < 1e-12 and abs(r["write_scale"] - 1.0) < 1e-12
    assert r["traffic_bytes_per_call"] == (1000.0 * 2 + 10.0) * 1024
    assert (out / "t_traffic.json").exists() and (out / "t_traffic.md").exists()
    both = profiling.summarize("u", "cmd", str(stats), str(fetch), str(write), 1, 2 * 2 ** 30, str(out))
    assert both["traffic_bytes_per_call"] == (1000.0 * 2 + 10.0 + 4000.0 * 2 + 20.0) * 1024


def test_no_traffic_file_without_counters(tmp_path):
    stats, _, _ = _inputs(tmp_path)
    out = tmp_path / "out"
    profiling.summarize("s", "cmd", str(stats), None, None, 0, 2 * 2 ** 30, str(out))
    assert (out / "s_kernel_stats.md").exists()
    assert not (out / "s_traffic.json").exists()


def test_decode_kernel_labels_carry_mode_and_host_order():
    base = "_ZN3pkv12_GLOBAL__N_119paged_decode_kernelIDF16bLi128ELi4ELb0ELi5"
    assert profiling.short_name(base + "EEEvNS_10DecodeArgsE") == "paged_decode_kernel (append)"
    assert profiling.short_name(base + "ELb0EEEvNS_10DecodeArgsE") == "paged_decode_kernel (append)"
    assert profiling.short_name(base + "ELb1EEEvNS_10DecodeArgsE") == "paged_decode_kernel (append, host order)"
    assert profiling.short_name(_PLAIN) == "paged_decode_kernel"
