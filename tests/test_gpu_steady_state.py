"""Steady-state forwards load no code and allocate nothing.

One plan serves forwards at token counts in every block-size bucket
(tests/steady_state_child.py, run under rocprofv3 with HIP and HSA API,
memory-allocation and kernel traces).  Between the child's two marker calls
-- after the plan's first forward -- the trace must hold no code-object
load, no allocation and no HIP call but kernel launches and their
bookkeeping.  The pages trace a tenfold time-to-first-token regression to
code loaded for each new context length (AWS ML blog "Efficiently serve
dozens of fine-tuned models with vLLM on Amazon SageMaker AI and Amazon
Bedrock", section "Execution optimizations").
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from lora_expert_gemm_amd import profiling  # noqa: E402

pytestmark = pytest.mark.gpu

# what a forward may call on the host once its kernels are resolved
LAUNCH_ONLY = {"hipLaunchKernel", "__hipPushCallConfiguration", "__hipPopCallConfiguration",
               "hipGetLastError", "hipFuncSetAttribute", "hipGetDevice"}


@pytest.mark.skipif(shutil.which("rocprofv3") is None, reason="rocprofv3 not installed")
def test_steady_state_forwards_load_and_allocate_nothing(tmp_path):
    out = tmp_path / "trace"
    cmd = ["rocprofv3", "--hip-trace", "--hsa-trace", "--memory-allocation-trace",
           "--kernel-trace", "-f", "csv", "-d", str(out), "-o", "steady", "--",
           sys.executable, os.path.join(ROOT, "tests", "steady_state_child.py")]
    print("[steady] " + " ".join(cmd), flush=True)
    p = subprocess.run(cmd, cwd="/tmp", env=dict(os.environ, TMPDIR="/tmp"),
                       capture_output=True, text=True, timeout=240)
    # (the profiler may exit non-zero after a complete run; the child's own
    # last line and the trace files decide)
    assert "[child] done" in p.stdout, (p.stdout[-3000:], p.stderr[-3000:])
    buckets = {kv.split(":")[1] for kv in p.stdout.split("[child] buckets ")[1].split("\n")[0].split()}
    assert len(buckets) >= 4, buckets
    w = profiling.steady_window(str(out))
    assert w["forbidden_inside"] == {}, w["forbidden_inside"]
    assert w["alloc_inside"] == {}, w["alloc_inside"]
    extra = set(w["hip_inside"]) - LAUNCH_ONLY
    assert not extra, {k: w["hip_inside"][k] for k in extra}
    assert w["hip_inside"].get("hipLaunchKernel", 0) >= 3 * 21
    # the code was loaded before: at start-up and by the plan's first forward
    assert w["hsa_before"].get("hsa_executable_load_agent_code_object", 0) >= 1
