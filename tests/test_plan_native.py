"""The planner's CPU checks (tests/native/plan_check.cpp): the chunk grid the kernels
derive on the device equals the host enumeration, the call tables are laid out
consistently, and 64-bit addresses are rebuilt from unsigned halves.  Built with the
host compiler against csrc/plan.cpp; no GPU."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_planner_native_checks(tmp_path):
    exe = str(tmp_path / "plan_check")
    src = os.path.join(ROOT, "tests", "native", "plan_check.cpp")
    plan = os.path.join(ROOT, "gated_deltanet_recurrent_chunk_amd", "csrc", "plan.cpp")
    # plain host C++: the planner holds no device code (gdn.h only needs the HIP types)
    subprocess.run(["g++", "-O1", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I",
                    os.path.join(ROOT, "include"), src, plan, "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
