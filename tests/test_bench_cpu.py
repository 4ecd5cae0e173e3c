"""Host-side pieces of bench.py: the source hash that ties a counter record to a kernel's code."""
import os
import shutil

import pytest

import bench


def test_code_only_drops_comments_and_keeps_literals():
    src = 'int a; // tail\nconst char* s = "// kept /* too */";\n/* block\n   comment */ int b;\nchar q = \'"\';  // "\n'
    assert bench.code_only(src) == 'int a; const char* s = "// kept /* too */"; int b; char q = \'"\';'
    assert bench.code_only('asm volatile("s_waitcnt vmcnt(0)" ::: "memory");') == \
        'asm volatile("s_waitcnt vmcnt(0)" ::: "memory");'
    assert bench.code_only('x = "a\\"b"; // c') == 'x = "a\\"b";'


@pytest.fixture
def csrc_copy(tmp_path, monkeypatch):
    src = os.path.join(bench.ROOT, "gqa_attention_sinks_sink_amd", "csrc")
    dst = tmp_path / "gqa_attention_sinks_sink_amd" / "csrc"
    shutil.copytree(src, dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return dst


@pytest.mark.parametrize("kind", sorted(bench.KERNEL_SOURCES))
def test_source_hash_follows_code_not_comments(csrc_copy, kind):
    before = bench.source_hash(kind)
    path = csrc_copy / bench.KERNEL_SOURCES[kind][0]
    text = path.read_text()
    path.write_text("// a new header line\n" + text.replace("\n", "\n\n", 3) + "/* trailing note */\n")
    assert bench.source_hash(kind) == before
    path.write_text(text + "\nnamespace { int unused_marker; }\n")
    assert bench.source_hash(kind) != before
