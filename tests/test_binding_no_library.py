"""The binding fails loudly when the HIP library is missing: there is no
CPU fallback, so a call without libtplinear.so raises before anything runs."""
import pytest

import tensor_linear_amd as tl


def test_missing_library_raises(monkeypatch, tmp_path):
    monkeypatch.setattr(tl, "LIB_PATH", str(tmp_path / "libtplinear.so"))
    monkeypatch.setattr(tl, "_lib", None)
    with pytest.raises(ImportError, match="libtplinear.so is missing"):
        tl.lib
    with pytest.raises(ImportError):
        tl.tp_row_workspace_bytes(tl.TP_ROW_SUM, 4, 4, 2)
