"""The traffic record's digest follows the kernel code, not its comments."""
from sigmoid_top_routing_amd import profiling


def test_comments_and_spacing_do_not_change_the_code_text():
    a = "int f(int x) {  // add one\n    return x + 1; /* done */\n}\n"
    b = "// a new header comment\nint f(int x) {\n  return x + 1;\n}\n"
    assert profiling.code_text(a) == profiling.code_text(b)


def test_a_code_change_changes_the_code_text():
    a = "int f(int x) { return x + 1; }"
    b = "int f(int x) { return x + 2; }"
    assert profiling.code_text(a) != profiling.code_text(b)
