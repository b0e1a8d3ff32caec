"""The source digest that counter records carry: comment and layout edits keep
it, code edits change it (host logic, no GPU)."""
from sparse_expert_ffn_amd import buildlib


def test_code_only_drops_comments_keeps_strings():
    a = 'int a; // note "x"\n/* block\n comment */ asm("v_mov  // kept"); x   =  1;'
    b = 'int a;\n asm("v_mov  // kept");\tx = 1;  // other note'
    assert buildlib._code_only(a) == buildlib._code_only(b)
    assert '"v_mov  // kept"' in buildlib._code_only(a)


def test_code_edit_changes_code_only():
    a = "int k = 32; // stage K"
    assert buildlib._code_only(a) != buildlib._code_only("int k = 64; // stage K")
    assert buildlib._code_only(a) != buildlib._code_only('int k = 32; const char* s = "//";')


def test_digest_is_stable():
    assert buildlib.source_digest() == buildlib.source_digest()
    assert len(buildlib.source_digest()) == 64
