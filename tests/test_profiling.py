"""Host-side checks of the profile tooling: the decode-source hash that ties a
committed traffic summary to the kernel code it was measured on follows the
code and ignores comments and layout."""
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
