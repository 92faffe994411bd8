"""CPU tests of the pipeline-trace summary (head_attention_forward_fmha_amd.pipeline_trace)
on record streams built like the ping-pong kernel's."""

import numpy as np

from head_attention_forward_fmha_amd import pipeline_trace as pt


def _word(ev, t):
    return np.uint64((ev << 56) | t)


def _wave(n_tiles, mfma_first, detailed, t0=1000, mb=500, mw=120, vb=520, vw=100, head=300,
          tail=800, items=2):
    """Records of one wave over `items` work items of n_tiles tiles each, as the
    ping-pong kernel stamps them: item start, prologue, a slot start before each
    of the 2 * (n_tiles + 1) slots and one after the last barrier, the epilogue.
    The wave runs the MFMA phase in the first slot of each pair when mfma_first
    (group A), else the VALU phase first (group B)."""
    w, t = [], t0
    for _ in range(items):
        w.append(_word(pt.EV_ITEM, t))
        t += head
        for pair in range(n_tiles + 1):
            for half in range(2):
                w.append(_word(pt.EV_SLOT, t))
                if (half == 0) == mfma_first:
                    if detailed:
                        w.append(_word(pt.EV_QK_DONE, t + mb // 2))
                    w.append(_word(pt.EV_MFMA_DONE, t + mb))
                    if detailed:
                        w.append(_word(pt.EV_WAIT_DONE, t + mb + 1))
                    t += mb + mw
                else:
                    if detailed:
                        w.append(_word(pt.EV_COPY_ISSUED, t + 40))
                    w.append(_word(pt.EV_VALU_DONE, t + vb))
                    if detailed:
                        w.append(_word(pt.EV_WAIT_DONE, t + vb + 30))
                    t += vb + vw
        w.append(_word(pt.EV_SLOT, t))   # after the last barrier: the epilogue follows
        t += tail
    w.append(_word(pt.EV_ITEM, t))       # the next item starts
    return w


def _trace(detailed):
    tr = np.zeros((2, 8, 512), dtype=np.uint64)
    for wg in range(2):
        for wave in range(8):
            recs = _wave(5, wave < 4, detailed)
            tr[wg, wave, :len(recs)] = recs
    return tr


def test_decode_stops_at_zero_and_splits_event_and_time():
    recs = [_word(6, 10), _word(0, 15), _word(2, 40)]
    arr = np.zeros(8, dtype=np.uint64)
    arr[:3] = recs
    assert pt.decode_wave(arr) == [(6, 10), (0, 15), (2, 40)]


def test_coarse_summary_recovers_the_phase_times():
    s = pt.summarize(_trace(False), clock_ghz=2.0)
    m = s["mean_cycles"]
    assert s["waves"] == 16
    assert m["mfma_busy"] == 500 and m["mfma_wait"] == 120
    assert m["valu_busy"] == 520 and m["valu_wait"] == 100
    assert m["item_head"] == 300 and m["item_tail"] == 800
    assert s["period"] == 500 + 120 + 520 + 100
    assert abs(s["mfma_wait_p_share"] - 120 / 1240) < 1e-12
    assert s["period_ns"] == s["period"] / 2.0
    assert m["qk"] is None and m["softmax"] is None
    # per wave and item: 6 slot pairs of steady slots, then the epilogue
    assert s["count"]["item_tail"] == 16 * 2 and s["count"]["mfma_busy"] == 16 * 2 * 6


def test_detailed_summary_splits_the_phases():
    s = pt.summarize(_trace(True))
    m = s["mean_cycles"]
    assert m["qk"] == 250 and m["pv"] == 250
    assert m["copy"] == 40 and m["softmax"] == 480
    assert m["copy_wait"] == 30 and m["barrier"] == 70


def _trace_with(mb, mw, vb, vw):
    tr = np.zeros((2, 8, 512), dtype=np.uint64)
    for wg in range(2):
        for wave in range(8):
            recs = _wave(5, wave < 4, False, mb=mb, mw=mw, vb=vb, vw=vw)
            tr[wg, wave, :len(recs)] = recs
    return tr


def test_critical_path_names_the_later_phase():
    # every slot lasts 620 cycles; the VALU phase is done at 520, the MFMA phase at 500
    c = pt.critical_path(_trace_with(500, 120, 520, 100))
    assert c["slots"] == 2 * 2 * 2 * 6        # workgroups x items x slot pairs x 2
    assert c["mfma_last"] == 500 and c["valu_last"] == 520 and c["release"] == 620
    assert c["after_last_done"] == 100 and c["valu_share"] == 1.0
    # the MFMA phase is done later
    c = pt.critical_path(_trace_with(560, 60, 520, 100))
    assert c["mfma_last"] == 560 and c["after_last_done"] == 60 and c["valu_share"] == 0.0
    # the summary carries it
    assert pt.summarize(_trace_with(500, 120, 520, 100))["critical"]["valu_share"] == 1.0


def test_critical_path_of_an_empty_trace():
    assert pt.critical_path(np.zeros((1, 8, 16), dtype=np.uint64)) == {"slots": 0}
