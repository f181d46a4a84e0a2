"""The in-tree build notices when the library is older than its sources."""
import os
import shutil

from selective_state_space_72_amd import build as hip_build


def _sandbox(tmp_path, monkeypatch):
    root = tmp_path / "repo"
    csrc = root / "pkg" / "csrc"
    inc = root / "include"
    shutil.copytree(hip_build.CSRC, csrc)
    shutil.copytree(hip_build.INCLUDE, inc)
    lib = root / "pkg" / "libmambascan.so"
    monkeypatch.setattr(hip_build, "ROOT", str(root))
    monkeypatch.setattr(hip_build, "CSRC", str(csrc))
    monkeypatch.setattr(hip_build, "INCLUDE", str(inc))
    monkeypatch.setattr(hip_build, "LIBRARY", str(lib))
    monkeypatch.setattr(hip_build, "DIGEST_FILE", str(lib) + ".digest")
    lib.write_bytes(b"stand-in")
    (root / "pkg" / "libmambascan.so.digest").write_text(hip_build.source_digest() + "\n")
    return csrc, inc


def test_library_current_when_digest_matches(tmp_path, monkeypatch):
    _sandbox(tmp_path, monkeypatch)
    assert hip_build.is_built()


def test_editing_any_source_marks_library_stale(tmp_path, monkeypatch):
    csrc, inc = _sandbox(tmp_path, monkeypatch)
    for path in [sorted(csrc.glob("*.hip"))[0], sorted(csrc.glob("*.h"))[0],
                 sorted(inc.glob("*.h"))[0]]:
        before = path.read_text()
        path.write_text(before + "\n// edited\n")
        assert not hip_build.is_built(), f"editing {path.name} went unnoticed"
        path.write_text(before)
        assert hip_build.is_built()


def test_missing_digest_means_not_built(tmp_path, monkeypatch):
    _sandbox(tmp_path, monkeypatch)
    os.remove(hip_build.DIGEST_FILE)
    assert not hip_build.is_built()
