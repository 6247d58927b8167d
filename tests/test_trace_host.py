"""LCA_TRACE (no GPU): with the variable set, every C-ABI call logs one "[lca]" line to stderr with its
shapes and first position, and a rejected call also logs its error code and message; unset (or "0"), the
library prints nothing.  Each case runs in a fresh interpreter, since the flag is read once per process.
Only calls that fail host validation are made (a valid call would launch a kernel)."""
import os
import subprocess
import sys
import textwrap

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = textwrap.dedent("""
    import ctypes as C
    import long_context_attention_22_amd as lca
    L = lca.lib()
    FAKE = 0x7F0000000000
    pos = (C.c_int64 * 1)(1 << 20)
    # top-k with k = 0: rejected before any launch
    rc = L.lca_topk_select(C.c_void_p(FAKE), lca.BF16, 262144, 1, 1, pos, 4, 0, C.c_void_p(FAKE), None, 0, None)
    assert rc == lca.EINVAL, rc
    # HCA attention with an unsupported output dtype
    kv = lca._KV(FAKE, FAKE + 65536, FAKE + 4096, lca.FP8, 512, 64, 8192)
    rc = L.lca_hca_attn(C.c_void_p(FAKE), lca.BF16, 64, 1, 1, pos, kv, 128, kv, 128, None, C.c_float(0.04),
                        C.c_double(1e4), C.c_void_p(FAKE), 7, None, None, 0, None)
    assert rc == lca.EDTYPE, rc
    print("done")
""")


def _run(env_value):
    env = dict(os.environ)
    env.pop("LCA_TRACE", None)
    if env_value is not None:
        env["LCA_TRACE"] = env_value
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    r = subprocess.run([sys.executable, "-c", SCRIPT], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "done" in r.stdout
    return [ln for ln in r.stderr.splitlines() if ln.startswith("[lca]")]


def test_trace_logs_calls_and_errors():
    lines = _run("1")
    assert any(ln.startswith("[lca] lca_topk_select B=1 T=1") and "k=0" in ln and "q_pos[0]=1048576" in ln
               for ln in lines), lines
    assert any("-> error" in ln and "k must be >= 1" in ln for ln in lines), lines
    assert any(ln.startswith("[lca] lca_hca_attn B=1 T=1 H=64") and "cap=8192" in ln for ln in lines), lines
    assert any("-> error" in ln and "out_dtype" in ln for ln in lines), lines


def test_trace_off_prints_nothing():
    assert _run(None) == []
    assert _run("0") == []
