"""The host code of libwf (the C ABI glue, the round planner and the launch
wrappers) under AddressSanitizer, LeakSanitizer and UndefinedBehaviorSanitizer.

tests/hostsan.py compiles the library with the sanitizers on its host code
only, and this test runs the host-side CPU tests (tests/test_abi_cpu.py,
tests/test_rollout_cpu.py: every argument check, the table operations, the
planner and the round runner's refusals) against it in a child process. The
run must pass with no memory error, no undefined behaviour and no leak whose
allocation stack passes through the library. (The uninstrumented interpreter
and runtime libraries keep allocations of their own until exit; those are not
the library's and are not counted.)
"""
import re

import pytest

import hostsan

pytestmark = pytest.mark.slow

# a symbolized frame of the library's own sources (file:line); frames that the fast
# unwinder misattributes land on unsymbolized offsets and do not match
LIB_FRAMES = re.compile(r"(wf_api|rollout)\.cpp:\d+|(kv_cache|rope3d|attn_fwd|attn_i8qk|w8a8)\.hip:\d+")


def _leak_reports(text: str):
    """Allocation stacks of the leak report, one string per leaked allocation site."""
    blocks = re.split(r"\n(?=(?:Direct|Indirect) leak of)", text)
    return [b for b in blocks if b.startswith(("Direct leak of", "Indirect leak of"))]


def test_host_code_clean_under_sanitizers():
    lib = hostsan.build_sanitized()
    res = hostsan.run_host_tests(lib, leaks=True)
    out = res.stdout.decode(errors="replace")
    summary = [l for l in out.splitlines() if re.search(r"\d+ (passed|failed)", l)]
    print(summary[-1] if summary else out[-2000:])
    assert summary and "failed" not in summary[-1] and "passed" in summary[-1], out[-4000:]
    assert "ERROR: AddressSanitizer" not in out, out[out.find("ERROR: AddressSanitizer"):][:4000]
    assert "runtime error:" not in out, out[out.find("runtime error:") - 200:][:4000]
    ours = [b for b in _leak_reports(out) if LIB_FRAMES.search(b)]
    assert not ours, "\n\n".join(ours[:5])
    # the sanitizers were live: the library carries their checks
    assert hostsan.instrumented(lib)
