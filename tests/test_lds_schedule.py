"""The LDS schedules of the query-side (four- and eight-wave), key-side and
shift kernels, replayed on the host for every instantiation the library
builds (tests/lds_model.py):
accesses in bounds, every byte read written before and visible to its reader,
no two waves touching a byte in one barrier phase with a write.  Planted
mistakes (a barrier removed, a buffer index frozen) must be caught."""
import pytest

from tests import lds_model as lm

QOUT = lm.qout_cases()
QOUT8 = lm.qout8_cases()
KSTATE = lm.kstate_cases()


@pytest.mark.parametrize("cfg", [c for c, _ in QOUT], ids=[n for _, n in QOUT])
def test_query_side_schedule(cfg):
    lm.qout_model(cfg)


@pytest.mark.parametrize("cfg", [c for c, _ in QOUT8], ids=[n for _, n in QOUT8])
def test_eight_wave_query_side_schedule(cfg):
    lm.qout8_model(cfg)


def test_eight_wave_query_side_covers_the_pages_example_shape():
    # d_h = 64, rank 64 (four 16-wide blocks), m = 256 (eight feature blocks)
    assert any(c.dh == 64 and c.r16 == 4 and c.fb == 8 for c, _ in QOUT8)


@pytest.mark.parametrize("cfg", [c for c, _ in KSTATE], ids=[n for _, n in KSTATE])
def test_key_side_schedule(cfg):
    lm.kstate_model(cfg)


@pytest.mark.parametrize("elem", lm.DTYPES)
@pytest.mark.parametrize("dh", lm.HEAD_DIMS)
@pytest.mark.parametrize("r16", lm.RANK_BLOCKS)
def test_shift_schedule(elem, dh, r16):
    lm.shift_model(elem, dh, r16)


def _first_caught(model, cases, mutation):
    for cfg, name in cases:
        try:
            model(cfg, mutate={mutation})
        except lm.Violation:
            return name
    return None


@pytest.mark.parametrize("mutation", ["no_kbuf_barrier", "no_kbuf1_barrier", "no_step_barrier", "ring_same_buffer",
                                      "kbuf_index_fixed", "no_z_wait"])
def test_model_catches_planted_query_side_mistakes(mutation):
    cases = QOUT
    if mutation == "no_kbuf1_barrier":
        cases = [(c, n) for c, n in QOUT if c.causal and c.derived()["kbuf"] == 1 and c.fb > 1]
    if mutation == "no_z_wait":
        cases = [(c, n) for c, n in QOUT if c.derived()["self_read"]]
    if not cases:
        pytest.skip(f"no instantiation exercises {mutation}")
    assert _first_caught(lm.qout_model, cases, mutation), f"{mutation} not caught"


@pytest.mark.parametrize("mutation", ["no_wait8", "no_m_barrier8", "kbuf8_index_fixed", "no_kbuf8_barrier",
                                      "no_exchange_barrier", "late8_after_barrier"])
def test_model_catches_planted_eight_wave_mistakes(mutation):
    assert _first_caught(lm.qout8_model, QOUT8, mutation), f"{mutation} not caught"


@pytest.mark.parametrize("mutation", ["tile_same_buffer", "no_tile_end_barrier", "no_m_wait"])
def test_model_catches_planted_key_side_mistakes(mutation):
    cases = [(c, n) for c, n in KSTATE if c.tiles > 1 or mutation == "no_m_wait"]
    if mutation == "no_tile_end_barrier":
        cases = [(c, n) for c, n in cases if c.derived()["nbuf"] == 1]
        if not cases:
            pytest.skip("every key-side instantiation double-buffers its tiles")
    assert _first_caught(lm.kstate_model, cases, mutation), f"{mutation} not caught"


def test_model_catches_shift_buffer_reuse():
    assert any(_raises(lambda: lm.shift_model(e, d, r, mutate={"shift_same_buffer"}))
               for e in lm.DTYPES for d in lm.HEAD_DIMS for r in (2, 4, 16))


def _raises(fn):
    try:
        fn()
    except lm.Violation:
        return True
    return False
