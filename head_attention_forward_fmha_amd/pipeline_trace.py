"""Summary of a pipeline trace recorded by ``fwd_trace`` (fmha_fwd_trace).

The trace follows "Kernel Bottleneck Tuning (validated on FA4 FP4/FP8 PV,
GB300)", section 2 (trace the real pipeline, coarsely): per wave, the cycles of
each phase of the ping-pong kernel's slots. A slot is the stretch between two
workgroup barriers; a wave runs the MFMA phase (Q.K^T then P.V) or the VALU
phase (copies, mask and softmax, wait for its copies) in it, and the two groups
of four waves alternate. From the records:

  mfma_busy   slot start -> MFMA phase done (MFMA role)
  mfma_wait   MFMA phase done -> next slot: the matrix-core group idles at the
              barrier until the other group has P ready (the pages' "MMA wait P")
  valu_busy   slot start -> softmax done (VALU role)
  valu_wait   softmax done -> next slot (copy wait and barrier)
  period      cycles per 64-key tile step (an MFMA slot plus a VALU slot)
  qk, pv, copy, softmax, copy_wait, barrier   the detailed mode's split of the
              phases (longer than untraced: each stamp blocks interleaving)

The stretch from an item's start to its first slot (prologue copies) and from
its last barrier to the next item's start (epilogue) are reported apart
(item_head, item_tail); a wave's last epilogue has no end record.
"""

from __future__ import annotations

import numpy as np

EV_SLOT, EV_QK_DONE, EV_MFMA_DONE, EV_COPY_ISSUED, EV_VALU_DONE, EV_WAIT_DONE, EV_ITEM = range(7)
TIME_MASK = (1 << 56) - 1


def decode_wave(words) -> list:
    """One wave's records -> [(event, time)], up to the first zero word."""
    out = []
    for w in np.asarray(words, dtype=np.uint64):
        w = int(w)
        if w == 0:
            break
        out.append((w >> 56, w & TIME_MASK))
    return out


def _slots(events):
    """Split a wave's records into slots: (kind, start, end, {event: time}).

    kind is "mfma" or "valu" for slots inside an item, "item_tail" for the
    stretch from an item's last slot start (after its last barrier) to the next
    item's start (the epilogue), and "item_head" for an item's start up to its
    first slot.
    """
    slots = []
    i = 0
    n = len(events)
    while i < n:
        ev, t = events[i]
        if ev == EV_ITEM:
            j = i + 1
            while j < n and events[j][0] not in (EV_SLOT, EV_ITEM):
                j += 1
            if j < n and events[j][0] == EV_SLOT:
                slots.append(("item_head", t, events[j][1], {}))
            i = j
            continue
        if ev == EV_SLOT:
            marks = {}
            j = i + 1
            while j < n and events[j][0] not in (EV_SLOT, EV_ITEM):
                marks[events[j][0]] = events[j][1]
                j += 1
            end = events[j][1] if j < n else None
            if end is not None:
                if events[j][0] == EV_ITEM:
                    kind = "item_tail"
                elif EV_MFMA_DONE in marks:
                    kind = "mfma"
                elif EV_VALU_DONE in marks:
                    kind = "valu"
                else:
                    kind = "other"
                slots.append((kind, t, end, marks))
            i = j
            continue
        i += 1
    return slots


def summarize(trace, clock_ghz: float | None = None) -> dict:
    """Summary of a trace array [workgroups, 8 waves, records] (uint64).

    Averages are over the recording waves' steady slots (inside items); all
    values are cycles of the shader clock unless noted.
    """
    trace = np.asarray(trace, dtype=np.uint64)
    acc = {k: [] for k in ("mfma_busy", "mfma_wait", "valu_busy", "valu_wait", "qk", "pv",
                           "copy", "softmax", "copy_wait", "barrier", "item_head", "item_tail")}
    waves = 0
    total = 0
    for wg in range(trace.shape[0]):
        for wave in range(trace.shape[1]):
            ev = decode_wave(trace[wg, wave])
            if len(ev) < 2:
                continue
            waves += 1
            total += ev[-1][1] - ev[0][1]
            for kind, start, end, m in _slots(ev):
                if kind == "mfma":
                    acc["mfma_busy"].append(m[EV_MFMA_DONE] - start)
                    acc["mfma_wait"].append(end - m[EV_MFMA_DONE])
                    if EV_QK_DONE in m:
                        acc["qk"].append(m[EV_QK_DONE] - start)
                        acc["pv"].append(m[EV_MFMA_DONE] - m[EV_QK_DONE])
                elif kind == "valu":
                    acc["valu_busy"].append(m[EV_VALU_DONE] - start)
                    acc["valu_wait"].append(end - m[EV_VALU_DONE])
                    if EV_COPY_ISSUED in m:
                        acc["copy"].append(m[EV_COPY_ISSUED] - start)
                        acc["softmax"].append(m[EV_VALU_DONE] - m[EV_COPY_ISSUED])
                    if EV_WAIT_DONE in m:
                        acc["copy_wait"].append(m[EV_WAIT_DONE] - m[EV_VALU_DONE])
                        acc["barrier"].append(end - m[EV_WAIT_DONE])
                elif kind in ("item_head", "item_tail"):
                    acc[kind].append(end - start)
    mean = {k: (float(np.mean(v)) if v else None) for k, v in acc.items()}
    counts = {k: len(v) for k, v in acc.items()}
    out = {"waves": waves, "cycles_per_wave": total / waves if waves else None,
           "mean_cycles": mean, "count": counts}
    if mean["mfma_busy"] is not None and mean["valu_busy"] is not None:
        mslot = mean["mfma_busy"] + mean["mfma_wait"]
        vslot = mean["valu_busy"] + mean["valu_wait"]
        out["period"] = mslot + vslot
        out["mfma_busy_share"] = mean["mfma_busy"] / out["period"]
        out["mfma_wait_p_share"] = mean["mfma_wait"] / out["period"]
        out["valu_busy_share"] = mean["valu_busy"] / out["period"]
        steady = sum(sum(acc[k]) for k in ("mfma_busy", "mfma_wait", "valu_busy", "valu_wait"))
        out["steady_share"] = steady / total if total else None
        if clock_ghz:
            out["period_ns"] = out["period"] / clock_ghz
    return out
