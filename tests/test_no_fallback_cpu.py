"""The product path has no fallback: without the HIP library every call raises, and the
package never loads the CPU oracle (which is test infrastructure only)."""
import os
import subprocess
import sys
import textwrap

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(code):
    r = subprocess.run([sys.executable, "-c", textwrap.dedent(code)], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout


def test_missing_library_raises():
    out = _run("""
        import exact_attention_35_amd.capi as c
        c.library_path = lambda: "/nonexistent/libfa.so"
        c._lib = None
        try:
            c.lib()
        except RuntimeError as e:
            print("raised", "not built" in str(e))
        else:
            print("no error")
    """)
    assert out.strip() == "raised True"


def test_package_does_not_load_the_oracle():
    out = _run("""
        import sys
        import exact_attention_35_amd, exact_attention_35_amd.capi, exact_attention_35_amd.roofline
        import exact_attention_35_amd.workloads, exact_attention_35_amd.build
        print(sorted(m for m in sys.modules if m == "oracle" or m.startswith("oracle.")))
    """)
    assert out.strip() == "[]"


def test_package_sources_do_not_name_the_oracle_module():
    pkg = os.path.join(ROOT, "exact_attention_35_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "import oracle" not in text and "from oracle" not in text, f
