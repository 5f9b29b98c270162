"""The library's source digest (the stamp the loader checks) follows the code
and nothing else: comments and layout do not change it, any code does."""
from precision_quantization_amd.build import code_tokens


def test_comments_and_layout_do_not_count():
    a = 'int x = 1; // one\n/* block\n comment */ float y;\n'
    b = 'int x = 1;\n\n\n   float y;   // other words\n'
    assert code_tokens(a) == code_tokens(b)


def test_code_and_literals_count():
    assert code_tokens("int x = 1;") != code_tokens("int x = 2;")
    # comment markers inside literals are code
    s = 'const char* p = "a // b /* c */";'
    assert code_tokens(s) == s
    assert code_tokens("char c = '\\'';") == "char c = '\\'';"


def test_preprocessor_lines_stay_lines():
    t = code_tokens('#define A 1 // note\n#define B 2\nint z;\n')
    assert t.splitlines()[:2] == ["#define A 1", "#define B 2"]
