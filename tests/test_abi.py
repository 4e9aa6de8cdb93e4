"""The C-ABI library without a GPU: it loads, exports every function that
include/echo.h declares, and rejects invalid arguments with the documented
codes before making any HIP call."""
import ctypes
import os
import re

import pytest

from error_compensated_bit_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "echo.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(echo_[a-z_]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("echo_state_reset", "echo_quantize_feedback", "echo_owner_reduce_requant",
              "echo_dequant_gather"):
        assert n in names


def test_library_exports_every_declared_function():
    lib = B.load_library()
    names = declared_functions()
    assert set(names) == set(B.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_segment_len_agrees_with_the_oracle():
    """Two independent implementations of the segment layout agree."""
    import oracle as O
    for n in (1, 7, 100, 127, 128, 129, 1000, 1024, 4095, 65537, 536870912, 536870913):
        for P in (1, 2, 3, 4, 7, 8, 16):
            for g in (32, 64, 128):
                assert B.echo_segment_len(n, P, g) == O.segment_len(n, P, g), (n, P, g)
    assert B.echo_segment_len(0, 2, 128) == 0
    assert B.echo_segment_len(100, 17, 128) == 0
    assert B.echo_segment_len(100, 2, 48) == 0
    assert B.echo_segment_len((1 << 63) - 1, 2, 128) == 0      # no overflow in the rounding
    assert B.echo_segment_len(1 << 42, 16, 128) == 1 << 38


def test_state_sizes():
    assert B.echo_state_bytes(1000, B.ECHO_STATE_F32) == 8000
    assert B.echo_state_bytes(1000, B.ECHO_STATE_BF16) == 4000
    assert B.echo_state_bytes(0, B.ECHO_STATE_F32) == 0
    assert B.echo_state_bytes(10, 7) == 0


def test_payload_sizes():
    assert B.echo_codes_bytes(1024, 4) == 512
    assert B.echo_codes_bytes(1024, 8) == 1024
    assert B.echo_codes_bytes(1023, 4) == 0
    assert B.echo_codes_bytes(1024, 5) == 0
    assert B.echo_params_bytes(1024, 128) == 32
    assert B.echo_params_bytes(1000, 128) == 0


def test_constants_match_the_header():
    text = open(HEADER).read()
    for name in ("ECHO_OK", "ECHO_ERR_ARG", "ECHO_ERR_SHAPE", "ECHO_ERR_ALIGN", "ECHO_ERR_HIP",
                 "ECHO_IN_BF16", "ECHO_IN_F16", "ECHO_OUT_BF16", "ECHO_OUT_F32",
                 "ECHO_STATE_F32", "ECHO_STATE_BF16", "ECHO_MAX_RANKS", "ECHO_GROUP"):
        m = re.search(rf"#define\s+{name}\s+(-?\d+)", text)
        assert m and int(m.group(1)) == getattr(B, name), name
    assert ctypes.sizeof(B.echo_config) == 36 and ctypes.sizeof(B.echo_seg) == 16


# Invalid arguments: every call below must return before any HIP call (there
# is no GPU here).  Fake, 16-byte aligned device addresses are never touched.
A = 0x10000
SEGS = (B.echo_seg * 16)(*[B.echo_seg(A, A) for _ in range(16)])


def cfg(**kw):
    return ctypes.byref(B.make_config(**kw))


@pytest.mark.parametrize("call,code", [
    (lambda L: L.echo_quantize_feedback(None, 2, 0, 256, A, A, SEGS, None), B.ECHO_ERR_ARG),
    (lambda L: L.echo_quantize_feedback(cfg(bits=3), 2, 0, 256, A, A, SEGS, None), B.ECHO_ERR_ARG),
    (lambda L: L.echo_quantize_feedback(cfg(group=48), 2, 0, 256, A, A, SEGS, None), B.ECHO_ERR_ARG),
    (lambda L: L.echo_quantize_feedback(cfg(group=256), 2, 0, 512, A, A, SEGS, None), B.ECHO_ERR_ARG),
    (lambda L: L.echo_quantize_feedback(cfg(in_dtype=7), 2, 0, 256, A, A, SEGS, None), B.ECHO_ERR_ARG),
    (lambda L: L.echo_quantize_feedback(cfg(eta=float("nan")), 2, 0, 256, A, A, SEGS, None), B.ECHO_ERR_ARG),
    (lambda L: L.echo_quantize_feedback(cfg(beta_short=1.0), 2, 0, 256, A, A, SEGS, None), B.ECHO_ERR_ARG),
    (lambda L: L.echo_quantize_feedback(cfg(beta_long=-0.1), 2, 0, 256, A, A, SEGS, None), B.ECHO_ERR_ARG),
    (lambda L: L.echo_quantize_feedback(cfg(mix_long=1.5), 2, 0, 256, A, A, SEGS, None), B.ECHO_ERR_ARG),
    (lambda L: L.echo_quantize_feedback(cfg(), 0, 0, 256, A, A, SEGS, None), B.ECHO_ERR_ARG),
    (lambda L: L.echo_quantize_feedback(cfg(), 17, 0, 17 * 128, A, A, SEGS, None), B.ECHO_ERR_ARG),
    (lambda L: L.echo_quantize_feedback(cfg(), 2, 2, 256, A, A, SEGS, None), B.ECHO_ERR_ARG),
    (lambda L: L.echo_quantize_feedback(cfg(), 2, -1, 256, A, A, SEGS, None), B.ECHO_ERR_ARG),
    (lambda L: L.echo_quantize_feedback(cfg(), 2, 0, 0, A, A, SEGS, None), B.ECHO_ERR_SHAPE),
    (lambda L: L.echo_quantize_feedback(cfg(), 2, 0, -5, A, A, SEGS, None), B.ECHO_ERR_SHAPE),
    (lambda L: L.echo_dequant_gather(cfg(), 2, 0, SEGS, A, None), B.ECHO_ERR_SHAPE),
    (lambda L: L.echo_quantize_feedback(cfg(), 2, 0, 2 * 128 * ((1 << 31) + 1), A, A, SEGS, None),
     B.ECHO_ERR_SHAPE),
    (lambda L: L.echo_quantize_feedback(cfg(), 2, 0, (1 << 63) - 1, A, A, SEGS, None),
     B.ECHO_ERR_SHAPE),
    (lambda L: L.echo_dequant_gather(cfg(), 16, (1 << 62) + 7, SEGS, A, None), B.ECHO_ERR_SHAPE),
    (lambda L: L.echo_state_reset(cfg(), A, (1 << 62), None), B.ECHO_ERR_ARG),
    (lambda L: L.echo_quantize_feedback(cfg(), 2, 0, 256, None, A, SEGS, None), B.ECHO_ERR_ARG),
    (lambda L: L.echo_quantize_feedback(cfg(), 2, 0, 256, A + 8, A, SEGS, None), B.ECHO_ERR_ALIGN),
    (lambda L: L.echo_quantize_feedback(cfg(), 2, 0, 256, A, A + 4, SEGS, None), B.ECHO_ERR_ALIGN),
    (lambda L: L.echo_quantize_feedback(cfg(), 2, 0, 256, A, A, None, None), B.ECHO_ERR_ARG),
    (lambda L: L.echo_quantize_feedback(
        cfg(), 2, 0, 256, A, A, (B.echo_seg * 2)(B.echo_seg(A, A), B.echo_seg(None, A)), None),
     B.ECHO_ERR_ARG),
    (lambda L: L.echo_quantize_feedback(
        cfg(), 2, 0, 256, A, A, (B.echo_seg * 2)(B.echo_seg(A, A), B.echo_seg(A, A + 2)), None),
     B.ECHO_ERR_ALIGN),
    (lambda L: L.echo_owner_reduce_requant(cfg(), 2, 0, 256, A, A, SEGS, None, None), B.ECHO_ERR_ARG),
    (lambda L: L.echo_owner_reduce_requant(cfg(), 2, 0, 256, A, A, None, SEGS, None), B.ECHO_ERR_ARG),
    (lambda L: L.echo_owner_reduce_requant(cfg(bits=8, out_dtype=2), 2, 0, 256, A, A, SEGS, SEGS, None),
     B.ECHO_ERR_ARG),
    (lambda L: L.echo_dequant_gather(cfg(), 2, 256, None, A, None), B.ECHO_ERR_ARG),
    (lambda L: L.echo_dequant_gather(cfg(), 2, 256, SEGS, A + 1, None), B.ECHO_ERR_ALIGN),
    (lambda L: L.echo_state_reset(None, A, 10, None), B.ECHO_ERR_ARG),
    (lambda L: L.echo_state_reset(cfg(state_dtype=5), A, 10, None), B.ECHO_ERR_ARG),
    (lambda L: L.echo_state_reset(cfg(), A, 0, None), B.ECHO_ERR_ARG),
    (lambda L: L.echo_state_reset(cfg(), A + 8, 10, None), B.ECHO_ERR_ALIGN),
    (lambda L: L.echo_state_reset(cfg(), None, 10, None), B.ECHO_ERR_ARG),
])
def test_invalid_arguments_return_codes(call, code):
    assert call(B.load_library()) == code


def test_error_strings():
    for c in (0, -1, -2, -3, -4, 99):
        assert isinstance(B.error_string(c), str) and B.error_string(c)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback: without the built library the binding raises, naming the
    file and how to build it."""
    from error_compensated_bit_amd import binding
    monkeypatch.setattr(binding, "_LIB", None)
    monkeypatch.setattr(binding, "library_path", lambda: str(tmp_path / "libecho_amd.so"))
    with pytest.raises(RuntimeError, match="build"):
        binding.load_library()


def test_prepared_call_reports_the_code_of_its_call():
    """A prepared (pre-marshalled) call runs the same validation on every
    call: an invalid configuration raises with ECHO_ERR_ARG before any HIP
    call, each time it is called."""
    import torch
    x = torch.zeros(256, dtype=torch.int16)
    st = torch.zeros(512, dtype=torch.float32)
    pay = B.Payload(torch.zeros(64, dtype=torch.uint8), torch.zeros(1, dtype=torch.int32))
    bad = B.make_config(bits=5)
    for prep in (B.prepare_quantize_feedback(bad, 2, 0, 256, x, st, [None, pay], stream=0),
                 B.prepare_owner_reduce_requant(bad, 2, 0, 256, x, st, [None, pay], pay, stream=0),
                 B.prepare_dequant_gather(bad, 2, 256, [pay, pay], x, stream=0)):
        for _ in range(2):
            with pytest.raises(B.EchoError) as e:
                prep()
            assert e.value.code == B.ECHO_ERR_ARG
