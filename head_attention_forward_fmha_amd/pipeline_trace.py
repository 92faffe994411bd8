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
    out["critical"] = critical_path(trace)
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


def critical_path(trace) -> dict:
    """Which phase ends each slot, from the stamps of all eight waves of a workgroup.

    Every wave of a workgroup passes the same barriers, so slot k of each wave
    is the same interval (coarse and detailed records both stamp every slot of
    every wave alike). Per steady slot with four MFMA-role and four VALU-role
    waves: t0 = the earliest slot start; mfma_last and valu_last = the latest
    phase-done stamp of each role, relative to t0; release = the latest slot end
    (the next barrier's release), relative to t0. The VALU role's done stamp is
    taken after its softmax and before it waits for its copies, so release -
    max(mfma_last, valu_last) holds that copy wait and the barrier itself.
    Returns the means and valu_share, the fraction of slots whose last phase
    to finish was a VALU phase.
    """
    trace = np.asarray(trace, dtype=np.uint64)
    m_last, v_last, rel, gap, v_crit = [], [], [], [], []
    for wg in range(trace.shape[0]):
        per_wave = [_slots(decode_wave(trace[wg, w])) for w in range(trace.shape[1])]
        if any(len(sl) == 0 for sl in per_wave):
            continue
        n = min(len(sl) for sl in per_wave)
        for k in range(n):
            slot = [sl[k] for sl in per_wave]
            if any(x[0] not in ("mfma", "valu") for x in slot):
                continue
            mf = [x for x in slot if x[0] == "mfma"]
            va = [x for x in slot if x[0] == "valu"]
            if len(mf) != 4 or len(va) != 4:
                continue
            t0 = min(x[1] for x in slot)
            ml = max(x[3][EV_MFMA_DONE] for x in mf) - t0
            vl = max(x[3][EV_VALU_DONE] for x in va) - t0
            r = max(x[2] for x in slot) - t0
            m_last.append(ml)
            v_last.append(vl)
            rel.append(r)
            gap.append(r - max(ml, vl))
            v_crit.append(1.0 if vl > ml else 0.0)
    if not rel:
        return {"slots": 0}
    return {"slots": len(rel), "mfma_last": float(np.mean(m_last)),
            "valu_last": float(np.mean(v_last)), "release": float(np.mean(rel)),
            "after_last_done": float(np.mean(gap)), "valu_share": float(np.mean(v_crit))}
