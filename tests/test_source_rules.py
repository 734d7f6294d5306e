"""Rules the HIP sources keep (host only, read from the source text).

Inline asm may hold only scalar instructions that leave the scalar condition code alone: the
compiler keeps values in it across an asm statement (the carry between the two halves of a 64-bit
address add), and an asm block that changed it would corrupt such an address."""
import pathlib
import re

CSRC = pathlib.Path(__file__).resolve().parents[1] / "attention_quantized_paged_amd" / "csrc"
# scalar mnemonics that do not write SCC
SCC_SAFE = {"s_mov_b32", "s_nop", "s_waitcnt", "s_getreg_b32"}


def _asm_strings(text):
    for m in re.finditer(r"asm\s+volatile\s*\(((?:\s*\"(?:[^\"\\]|\\.)*\"\s*)+)", text):
        yield "".join(re.findall(r"\"((?:[^\"\\]|\\.)*)\"", m.group(1)))


def test_inline_asm_leaves_scc_alone():
    found = set()
    for f in sorted(list(CSRC.glob("*.hip")) + list(CSRC.glob("*.h"))):
        for body in _asm_strings(f.read_text()):
            for mn in re.findall(r"\b(s_[a-z0-9_]+)", body):
                found.add((f.name, mn))
    bad = sorted(x for x in found if x[1] not in SCC_SAFE)
    assert not bad, f"inline asm with scalar instructions that may write SCC: {bad}"
    assert found, "no inline asm found: the pattern no longer matches the sources"
