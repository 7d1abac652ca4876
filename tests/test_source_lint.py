"""Source checks on the HIP kernels that need no GPU."""
import os
import re

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "bit_quantized_lora_02_amd", "csrc")


def _sources():
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, name)) as f:
                yield name, f.read()


def test_no_bit_cast_of_vector_element():
    """hipcc lowers __builtin_bit_cast of a vector-element lvalue (v[i]) as a read of element 0, so
    every such cast takes a scalar copy instead; this pins that no subscripted operand slips back in."""
    pat = re.compile(r"__builtin_bit_cast\(\s*[\w:<> ]+,\s*[^(),]*\]\s*\)")
    bad = [(name, m.group(0)) for name, text in _sources() for m in pat.finditer(text)]
    assert not bad, f"bit_cast of a subscripted operand: {bad}"


def test_no_hand_written_packed_fp32():
    """The packed binary32 instructions stay out of the sources (they are disabled at build time too)."""
    pat = re.compile(r"v_pk_(add|mul|fma)_f32")
    bad = [name for name, text in _sources() if pat.search(text)]
    assert not bad, f"packed binary32 instructions written by hand in {bad}"
