"""Each oracle mutant plants one plausible mistake (see the MUT() switches in
oracle/oracle.c); at least one pin must catch it.  CPU only."""
import pytest

import oracle_pins

MUTANTS = {
    1: "causal mask dropped",
    2: "causal limit off by one",
    3: "query head mapped to KV head h % H_kv",
    4: "softmax scale dropped",
    5: "LSE missing its max term",
    6: "averaging ignores the first averaged row",
    7: "averaging divides by the row count only",
    8: "top-K ties go to the higher position",
    9: "top-K output left in score order",
    10: "invalid draft positions clamped instead of ignored",
    11: "V gathered by position instead of slot",
    12: "pool layout read as [slots][d][H_kv]",
    13: "recent window shifted back one position (newest token dropped)",
    14: "stored positions past the context clamped to the last position",
    15: "one sink too many",
    16: "recallable index padded with position 0 instead of -1",
    17: "list coverage from exp(logit) without the LSE",
    18: "list coverage counts repeated entries once per repeat",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: f"m{m}")
def test_mutant_is_caught(mutant):
    from oracle import Oracle
    orc = Oracle(mutant=mutant)
    assert orc.lib.oracle_mutant_id() == mutant
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except Exception as e:  # an assertion or a shape error both count as caught
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"mutant {mutant} ({MUTANTS[mutant]}) passed every pin"
