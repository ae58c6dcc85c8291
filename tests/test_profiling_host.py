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
