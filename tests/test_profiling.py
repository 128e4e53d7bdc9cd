"""CPU tests of the profile bookkeeping: a traffic summary stays valid while
its kernel's code is unchanged (comments and layout do not count) and is
ignored once the code changes."""
from chunked_gated_delta_08_amd import profiling


def test_code_digest_ignores_comments_and_layout():
    a = "int f(int x) {\n    return x + 1;   // one more\n}\n/* trailing\n   block */\n"
    b = "// header\nint f(int x) { return x + 1; }\n"
    c = "int f(int x) {\n    return x + 2;   // one more\n}\n"
    assert profiling._code_of(a) == profiling._code_of(b)
    assert profiling._code_of(a) != profiling._code_of(c)
    # a line broken inside a call is the same code; a space between two names is not dropped
    assert profiling._code_of("x = f(g(y));") == profiling._code_of("x = f(\n    g(y));")
    assert profiling._code_of("int x;") != profiling._code_of("intx;")


def test_code_digest_follows_the_files(tmp_path, monkeypatch):
    monkeypatch.setattr(profiling, "ROOT", str(tmp_path))
    f = tmp_path / "k.hip"
    f.write_text("__global__ void k() { }  // v1\n")
    d1 = profiling.source_digest(["k.hip"])
    f.write_text("// a note\n__global__ void k()\n{\n}\n")
    assert profiling.source_digest(["k.hip"]) == d1
    f.write_text("__global__ void k() { int x = 0; }\n")
    assert profiling.source_digest(["k.hip"]) != d1
