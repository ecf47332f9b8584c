"""Host-side checks of the build script: the stamp that decides whether the
library on disk is current covers every source and every compiler flag,
including the per-source device flags (a library built with another
scheduler for the decode GEMV must be rebuilt, not loaded)."""
import importlib.util
import os

from tests.conftest import ROOT


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "_tl_build_test", os.path.join(ROOT, "looped_weight_shared_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_device_flags_name_existing_sources_and_enter_the_stamp():
    b = _build_module()
    srcs = set(os.listdir(os.path.join(ROOT, "looped_weight_shared_amd", "csrc")))
    assert b.DEVICE_FLAGS, "the decode GEMV takes its own scheduler"
    for name, flags in b.DEVICE_FLAGS.items():
        assert name in srcs, name
        # device-only: an -mllvm option on the host pass names an x86 scheduler
        assert flags[0] == "-Xarch_device" and all(not f.startswith("-mllvm ") for f in flags)
    h0 = b.source_hash()
    saved = dict(b.DEVICE_FLAGS)
    try:
        b.DEVICE_FLAGS["w4gemv.hip"] = ["-Xarch_device", "-mllvm=-amdgpu-sched-strategy=max-ilp"]
        assert b.source_hash() != h0
        del b.DEVICE_FLAGS["w4gemv.hip"]
        assert b.source_hash() != h0
    finally:
        b.DEVICE_FLAGS.clear()
        b.DEVICE_FLAGS.update(saved)
    assert b.source_hash() == h0


def test_the_stamp_covers_every_kernel_source(tmp_path, monkeypatch):
    """Changing any byte of a HIP source or kernel header changes the stamp."""
    b = _build_module()
    h0 = b.source_hash()
    csrc = os.path.join(ROOT, "looped_weight_shared_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if not name.endswith((".hip", ".h")):
            continue
        real_open = open

        def fake_open(path, mode="r", *a, _name=name, **k):
            f = real_open(path, mode, *a, **k)
            if os.path.basename(str(path)) == _name and "b" in mode:
                data = f.read() + b"\n"
                f.close()
                import io
                return io.BytesIO(data)
            return f
        monkeypatch.setattr("builtins.open", fake_open)
        assert b.source_hash() != h0, name
        monkeypatch.undo()
    assert b.source_hash() == h0
