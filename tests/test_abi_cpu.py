"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and validates configurations on the host."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssb.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ssb_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    from self_speculative_block_amd import _lib
    if not os.path.exists(_lib.LIB):
        from self_speculative_block_amd.build import build_library
        build_library()
    return _lib.load()


def test_library_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) >= 18
    for n in names:
        assert hasattr(lib, n), n
    from self_speculative_block_amd._lib import SIGNATURES
    assert sorted(SIGNATURES) == names


def _cfg(**kw):
    from self_speculative_block_amd._lib import SsbConfig, SSB_BF16
    c = SsbConfig(n_layers=24, hidden=1024, n_heads=16, n_kv_heads=4, head_dim=64, ffn=4096, vocab=60000,
                  mask_id=59999, eos_id=59998, block_B=32, page_tokens=16, max_rows=2048,
                  max_positions=8192, rms_eps=1e-6, rope_theta=10000.0, dtype=SSB_BF16)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_config_validation(lib):
    from self_speculative_block_amd._lib import SSB_EINVAL, SSB_OK
    assert lib.ssb_check_config(ctypes.byref(_cfg())) == SSB_OK
    bad = [dict(head_dim=48), dict(hidden=1000), dict(hidden=384), dict(n_kv_heads=3), dict(n_kv_heads=8),
           dict(ffn=3000), dict(mask_id=60000), dict(eos_id=59999), dict(block_B=65), dict(page_tokens=32),
           dict(max_rows=0), dict(max_rows=4000), dict(max_rows=16, block_B=32), dict(dtype=7),
           dict(max_positions=1), dict(n_layers=0), dict(ffn=16384), dict(n_heads=128, n_kv_heads=32),
           dict(max_batch=65), dict(max_batch=-1), dict(features=2)]
    for kw in bad:
        assert lib.ssb_check_config(ctypes.byref(_cfg(**kw))) == SSB_EINVAL, kw
        assert lib.ssb_last_error()
    assert lib.ssb_check_config(None) == SSB_EINVAL
    assert lib.ssb_check_config(ctypes.byref(_cfg(ffn=8192))) == SSB_OK     # split down projection
    tiny = _cfg(n_layers=2, hidden=128, n_heads=4, n_kv_heads=4, head_dim=32, ffn=512, vocab=512, mask_id=511,
                eos_id=510, block_B=8, dtype=0)
    assert lib.ssb_check_config(ctypes.byref(tiny)) == SSB_OK


def test_null_arguments_are_rejected_without_a_gpu(lib):
    from self_speculative_block_amd._lib import SSB_EINVAL
    size = ctypes.c_size_t()
    assert lib.ssb_pool_bytes(None, 4, ctypes.byref(size)) == SSB_EINVAL
    assert lib.ssb_kv_state(None, None, None, None) == SSB_EINVAL
    assert lib.ssb_kv_reset(None) == SSB_EINVAL
    assert lib.ssb_pool_init(None, None, 0, 1, None) == SSB_EINVAL
    assert lib.ssb_kv_create(None, 16, None) == SSB_EINVAL
    assert lib.ssb_init_model(ctypes.byref(_cfg()), None, None, None) == SSB_EINVAL
    assert lib.ssb_model_memory(None, ctypes.byref(size), None) == SSB_EINVAL
    lib.ssb_free_model(None)
    lib.ssb_kv_free(None)
    lib.ssb_pool_free(None)


def test_struct_layouts_match_the_header(tmp_path):
    """The ctypes mirrors of the header's structs have the C compiler's sizes and offsets."""
    import subprocess
    from self_speculative_block_amd import _lib
    structs = {"ssb_config": _lib.SsbConfig, "ssb_stats": _lib.SsbStats, "ssb_request": _lib.SsbRequest,
               "ssb_serve_stats": _lib.SsbServeStats, "ssb_weights": _lib.SsbWeights}
    lines = ["#include <stdio.h>", "#include <stddef.h>", f'#include "{HEADER}"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-o", str(exe), str(src)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l.strip()}
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)


def test_serve_rejects_bad_arguments_without_a_gpu(lib):
    from self_speculative_block_amd._lib import SSB_EINVAL
    assert lib.ssb_serve(None, None, None, 0, 1, 0, 0, 16, None, None) == SSB_EINVAL
    assert lib.ssb_ar_step_batch(None, None, 1, None, None) == SSB_EINVAL
