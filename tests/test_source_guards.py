"""Host-side guards over the HIP sources (no GPU, no compiler run).

The ROCm 7.2 clang front end lowers ``__builtin_bit_cast(T, v[i])``, with ``v``
an ext_vector_type value and ``v[i]`` one of its elements, to a cast of element
0 whatever ``i`` is (the emitted IR holds a single ``extractelement ..., i64 0``
reused for every index).  A row-sum variant of the extend kernel that summed
packed bf16 weights this way counted the first pair four times.  The kernels
here bit-cast whole vectors only; this test keeps it that way: copy an element
into a scalar before casting it.
"""
import pathlib
import re

CSRC = pathlib.Path(__file__).resolve().parents[1] / "cross_model_shared_amd" / "csrc"


def _bit_cast_operands(text):
    """Yield (line, operand) for every __builtin_bit_cast(type, operand) in text."""
    for m in re.finditer(r"__builtin_bit_cast\s*\(", text):
        i, paren, angle, comma = m.end(), 1, 0, None
        while i < len(text) and paren:
            c = text[i]
            if c == "(":
                paren += 1
            elif c == ")":
                paren -= 1
            elif c == "<":
                angle += 1
            elif c == ">" and angle:
                angle -= 1
            elif c == "," and paren == 1 and angle == 0 and comma is None:
                comma = i
            i += 1
        line = text.count("\n", 0, m.start()) + 1
        yield line, text[comma + 1:i - 1].strip() if comma is not None else ""


def test_bit_cast_operands_are_whole_values():
    sources = sorted(CSRC.glob("*.hip")) + sorted(CSRC.glob("*.h")) + sorted(CSRC.glob("*.cpp"))
    assert sources
    seen = 0
    for path in sources:
        for line, operand in _bit_cast_operands(path.read_text()):
            seen += 1
            assert "[" not in operand, f"{path.name}:{line}: __builtin_bit_cast of a subscript ({operand})"
    assert seen >= 1


def test_guard_catches_a_subscript():
    text = "x = __builtin_bit_cast(bf16x2_t, pb[cb][w]);\ny = __builtin_bit_cast(u32x2, v);\n"
    ops = list(_bit_cast_operands(text))
    assert ops == [(1, "pb[cb][w]"), (2, "v")]
