"""Host checks of the counter-summary gate: roofline.traffic is reported only
for the kernel code the counters were taken on, and comments do not count."""
from partial_context_patch_amd import profiling as P


def _sources():
    out = {}
    for rel in P.KERNEL_SOURCES:
        with open(P.os.path.join(P.HERE, rel), encoding="utf-8") as f:
            out[rel] = f.read()
    return out


def test_hash_ignores_comments_and_blank_lines():
    src = _sources()
    base = P.kernel_source_hash(src)
    assert base == P.kernel_source_hash()
    rel = P.KERNEL_SOURCES[0]
    edited = dict(src)
    edited[rel] = "// a new comment line\n\n" + src[rel].replace("\n", "  // trailing note\n", 3)
    assert P.kernel_source_hash(edited) == base


def test_hash_sees_code_changes():
    src = _sources()
    base = P.kernel_source_hash(src)
    for rel in P.KERNEL_SOURCES:
        edited = dict(src)
        edited[rel] = src[rel] + "\nstatic const int npa_probe_constant = 1;\n"
        assert P.kernel_source_hash(edited) != base
    rel = P.KERNEL_SOURCES[0]
    edited = dict(src)
    edited[rel] = src[rel].replace("kBN = 64", "kBN = 128", 1)
    assert edited[rel] != src[rel]
    assert P.kernel_source_hash(edited) != base


def _write_pass(d, rows):
    d.mkdir(parents=True, exist_ok=True)
    with open(d / "run_counter_collection.csv", "w") as f:
        f.write('"Kernel_Name","Counter_Name","Counter_Value"\n')
        for kernel, counter, value in rows:
            f.write(f'"{kernel}","{counter}",{value}\n')


def test_counter_summary_scales_bytes_by_the_calibration_copy(tmp_path):
    """The plain 512 MiB copy fixes the KiB-to-byte scale of each counter: here
    FETCH_SIZE reads half of its bytes (scale 2) and WRITE_SIZE all of them
    (scale 1), so 1000 / 500 KiB on the attention kernel are 2 048 000 read and
    512 000 written bytes."""
    import json

    copy = "void at::native::copyBuffer<float>(...)"
    attn = "void npa::(anonymous namespace)::attn_bf16_kernel<64, 1, false, false>(npa::AttnArgs)"
    _write_pass(tmp_path / "p1", [(copy, "FETCH_SIZE", 262144), (attn, "FETCH_SIZE", 1000),
                                  (attn, "FETCH_SIZE", 1000)])
    _write_pass(tmp_path / "p2", [(copy, "WRITE_SIZE", 524288), (attn, "WRITE_SIZE", 400),
                                  (attn, "WRITE_SIZE", 600)])
    text = P.counters([str(tmp_path / "p1"), str(tmp_path / "p2")], "unit_case", "cmd")
    summary = json.loads(text.strip().splitlines()[-1][len("summary-json: "):])
    assert abs(summary["fetch_scale"] - 2.0) < 1e-12 and abs(summary["write_scale"] - 1.0) < 1e-12
    assert abs(summary["attention_hbm_bytes"] - (1000 * 1024 * 2 + 500 * 1024)) < 1e-6
    assert summary["kernel_source_hash"] == P.kernel_source_hash()
