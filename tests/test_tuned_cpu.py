"""Tuned-configuration files without a device: the signature of the compiled
configuration list and the validation of the file format (include/swiglu.h)."""
import pytest

import gemm_epilogues_mlp_amd as sw


def _write(tmp_path, text, name="t.txt"):
    p = tmp_path / name
    p.write_text(text)
    return str(p)


def _header():
    return f"swiglu-tuned {sw.swiglu_config_signature():016x} gfx950\n"


def _first(variant):
    return next(i for i in range(sw.swiglu_config_count())
                if sw.swiglu_config_info(i)["variant"] == variant)


def test_signature_is_stable_and_nonzero():
    s = sw.swiglu_config_signature()
    assert s != 0 and s == sw.swiglu_config_signature()


def test_valid_file_with_comments_and_provenance(tmp_path):
    i, s, g = _first(sw.VARIANT_INTERLEAVE), _first(sw.VARIANT_SYNC), _first(sw.VARIANT_GEMM)
    text = ("# comment\n\n" + _header() +
            f"2 300 264 200 {i} 12.5us builtin 3 14.0us\n"
            f"   1 300 264 200 {s}\n# another comment\n3 128 4864 896 {g}\n")
    assert sw.swiglu_tuned_check(_write(tmp_path, text)) == 3


def test_header_only_is_valid_and_empty(tmp_path):
    assert sw.swiglu_tuned_check(_write(tmp_path, _header())) == 0


@pytest.mark.parametrize("text,status", [
    ("", sw.ERR_INVALID_ARG),                                          # no header
    ("# only a comment\n", sw.ERR_INVALID_ARG),
    ("swiglu-tuned zz gfx950\n", sw.ERR_INVALID_ARG),                  # bad signature field
    ("swiglu-tuned 0123456789abcdef gfx950\n", sw.ERR_UNSUPPORTED),    # another build
    ("HEADER2 300 264\n", sw.ERR_INVALID_ARG),                         # short entry
    ("HEADER2 -1 264 200 0\n", sw.ERR_INVALID_ARG),                    # negative size
    ("HEADER2 300 264 200 999999\n", sw.ERR_INVALID_ARG),              # no such config
    ("HEADERWRONGVARIANT", sw.ERR_INVALID_ARG),                        # id of another variant
])
def test_invalid_files_are_refused(tmp_path, text, status):
    if text.startswith("HEADERWRONGVARIANT"):
        text = _header() + f"2 300 264 200 {_first(sw.VARIANT_SYNC)}\n"
    elif text.startswith("HEADER"):
        text = _header() + text[len("HEADER"):]
    with pytest.raises(sw.SwiGLUError) as e:
        sw.swiglu_tuned_check(_write(tmp_path, text))
    assert e.value.status == status


def test_overlong_line_and_missing_file_are_refused(tmp_path):
    with pytest.raises(sw.SwiGLUError) as e:
        sw.swiglu_tuned_check(_write(tmp_path, _header() + "2 " + "1" * 600 + "\n"))
    assert e.value.status == sw.ERR_INVALID_ARG
    with pytest.raises(sw.SwiGLUError) as e:
        sw.swiglu_tuned_check(str(tmp_path / "missing.txt"))
    assert e.value.status == sw.ERR_INVALID_ARG


def test_create_tuned_checks_the_file_before_the_device(tmp_path):
    # without a GPU the file error is reported first; with one, creation works
    import torch
    bad = _write(tmp_path, "swiglu-tuned 0123456789abcdef gfx950\n")
    with pytest.raises(sw.SwiGLUError) as e:
        sw.swiglu_create_tuned(0, bad)
    assert e.value.status == sw.ERR_UNSUPPORTED
    if not torch.cuda.is_available():
        with pytest.raises(sw.SwiGLUError) as e:
            sw.swiglu_create_tuned(0, _write(tmp_path, _header(), "ok.txt"))
        assert e.value.status == sw.ERR_DEVICE


def test_shipped_tuned_file_matches_this_build():
    """The package's tuned file for MI355X is signed for the compiled
    configuration list, every entry names a configuration of its own variant,
    and it adds only shapes beyond the five built-in workload entries."""
    n = sw.swiglu_tuned_check(sw.TUNED_MI355X)
    assert n > 0
    five = {(128, 4864, 896), (2048, 8960, 1536), (16, 18944, 3584), (8192, 18944, 3584),
            (4096, 29568, 8192)}
    lines = [ln.split() for ln in open(sw.TUNED_MI355X)
             if ln.strip() and not ln.startswith("#") and not ln.startswith("swiglu-tuned")]
    assert len(lines) == n
    for t in lines:
        v, M, N, K, cid = (int(x) for x in t[:5])
        assert (M, N, K) not in five
        assert sw.swiglu_config_info(cid)["variant"] == v
