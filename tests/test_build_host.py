"""Build script host logic: compiler diagnostics are filtered, not dropped."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location("_moe_build_for_test",
                                                  os.path.join(ROOT, "expert_routed_ffn_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_only_the_host_feature_note_is_filtered():
    b = _build_module()
    note = "warning: '-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
    real = "ffn_gemv.hip:10:5: warning: unused variable 'x' [-Wunused-variable]"
    out = b._diagnostics("\n".join([note, real, "", note]))
    assert out == real
    assert b._diagnostics(note + "\n\n") == ""


def test_device_code_keeps_the_packed_fp32_flag():
    b = _build_module()
    flags = " ".join(b.CFLAGS)
    assert "-Xclang -target-feature -Xclang -packed-fp32-ops" in flags
    assert "--offload-arch=gfx950" in flags and "-ffp-contract=off" in flags
