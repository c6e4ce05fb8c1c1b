"""Parity check of a quantized layer against the float64 oracle.

Test infrastructure (imported by the GPU tests and the smoke run).

The result of the sweep is unique given its inputs, except where a rounding
decision falls on a tie. The GPU keeps its working values in float32, so a
decision the oracle takes within a small distance of a rounding boundary can
go the other way on the GPU; the row then follows its own, equally valid,
continuation. The check therefore works row by row:

1. Start from the oracle's row.
2. Find the first decision where the tested row differs: a group's zero
   point (decided at the group's first column, before that column's code)
   or a code.
3. That decision must be one the oracle itself took within ``tie`` grid
   steps of a rounding boundary (its reported margin), and the tested value
   must be the integer on the other side of that boundary (one step away).
4. Re-run the oracle on that row with this decision flipped and every
   earlier flip kept (``rerun``), and continue from 2 with that continuation.

A row passes when, after at most ``max_flips_per_row`` such flips, its codes
and zero points equal the oracle continuation's exactly, its scales agree
within ``scale_rtol`` and its loss within ``row_loss_rtol``. So every code
mismatch against the matched oracle row is zero (within the required one
step), and every departure from the oracle's own row is explained by a
decision the oracle found at a near-tie. Besides, the share of rows that
needed any flip is bounded (``max_flip_rows``), the total loss is within 1%
of the oracle's, and the packed words are bit-exact for the tested codes.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Optional

import numpy as np

import oracle.gptq_oracle as O


class ParityError(AssertionError):
    pass


@dataclass
class LayerOutputs:
    """The tested side's outputs for the compared rows (numpy arrays)."""

    codes: np.ndarray  # [rows, d_col] uint8
    scales: np.ndarray  # [rows, n_groups]
    zeros: np.ndarray  # [rows, n_groups]
    packed: Optional[np.ndarray]  # [rows, words] uint32, or None
    row_loss: np.ndarray  # [rows]


ROW_KEYS = ("codes", "scales", "zeros", "row_loss", "code_margin", "zero_margin")


def _row(ref: dict, i: int) -> dict:
    return {k: np.asarray(ref[k])[i] for k in ROW_KEYS}


def rerun_for(W_rows, U, bits: int, group_size: int, block: int = 128, decide=np.float32, symmetric: bool = False):
    """A ``rerun`` callable: the oracle's sweep of compared row i alone, with
    the given flips (rows are independent given U)."""
    W_rows = np.asarray(W_rows)
    U = np.asarray(U, dtype=np.float64)

    def rerun(i, flips):
        return O.quantize_layer(W_rows[i : i + 1], U, bits, group_size, block, decide=decide, symmetric=symmetric,
                                flips=[(0, kind, idx) for kind, idx in flips])

    return rerun


def _first_decision(t_codes, t_zeros, r):
    """(kind, index, column) of the earliest decision where the tested row
    differs from reference row r, or None."""
    cm = np.flatnonzero(t_codes != r["codes"])
    zm = np.flatnonzero(t_zeros != r["zeros"])
    cand = []
    if zm.size:
        cand.append((int(zm[0]) * _group_width(r), 0, "zero", int(zm[0])))
    if cm.size:
        cand.append((int(cm[0]), 1, "code", int(cm[0])))
    if not cand:
        return None
    col, _, kind, idx = min(cand)
    return kind, idx, col


def _group_width(r):
    ng = r["zeros"].shape[0]
    d_col = r["codes"].shape[0]
    return d_col if ng == 1 else -(-d_col // ng)


def follow_row(t_codes, t_zeros, ref_row: dict, rerun: Callable, i: int, tie: float, max_flips: int):
    """Follow tested row i through oracle continuations (module docstring,
    steps 1-4). Returns (matched oracle row, list of flips)."""
    r = ref_row
    flips = []
    while True:
        d = _first_decision(t_codes, t_zeros, r)
        if d is None:
            return r, flips
        kind, idx, col = d
        if len(flips) >= max_flips:
            raise ParityError(f"row {i}: more than {max_flips} near-tie flips (next at {kind} {idx})")
        if kind == "code":
            margin = float(r["code_margin"][idx])
            step = int(t_codes[idx]) - int(r["codes"][idx])
        else:
            margin = float(r["zero_margin"][idx])
            step = int(t_zeros[idx]) - int(r["zeros"][idx])
        if not margin < tie:
            raise ParityError(
                f"row {i}: {kind} {idx} (column {col}) differs by {step} at a decision {margin:.3g} grid steps "
                f"from a rounding boundary (not a near-tie; tie = {tie})")
        if abs(step) != 1:
            raise ParityError(f"row {i}: {kind} {idx} differs by {step} steps at a near-tie")
        flips.append((kind, idx))
        r = _row(rerun(i, flips), 0)


def check_quant(t: LayerOutputs, ref: dict, bits: int, rerun: Callable, *, tie: float = 1e-3, max_flip_rows: float = 0.1,
                max_flips_per_row: int = 16, scale_rtol: float = 1e-3, row_loss_rtol: float = 1e-2,
                loss_rtol: float = 1e-2, label: str = "", log=print) -> dict:
    """Check the tested rows against the oracle (module docstring). Returns
    a summary: codes matching the oracle's own rows, rows that needed
    flips, flips in total, the largest code difference against the
    oracle's own rows, the match against the followed continuations, and
    ``matched``: the oracle rows each tested row was matched with (codes,
    scales, zeros, row_loss; all values the oracle computed)."""
    codes = np.asarray(t.codes)
    zeros = np.asarray(t.zeros).astype(np.int64)
    scales = np.asarray(t.scales, dtype=np.float64)
    row_loss = np.asarray(t.row_loss, dtype=np.float64)
    n_rows, d_col = codes.shape
    if ref["codes"].shape != codes.shape:
        raise ParityError(f"shape {codes.shape} against the oracle's {ref['codes'].shape}")
    if int(codes.max(initial=0)) > (1 << bits) - 1:
        raise ParityError("a code exceeds 2^bits - 1")
    if t.packed is not None and not np.array_equal(np.asarray(t.packed).view(np.uint32), O.pack(codes, bits)):
        raise ParityError("packed words differ from the bitstream of the tested codes")

    diff0 = codes.astype(np.int64) - ref["codes"].astype(np.int64)
    match0 = float(np.mean(diff0 == 0)) if diff0.size else 1.0
    flipped_rows, n_flips = 0, 0
    matched_equal = 0
    worst_scale = 0.0
    matched = {k: np.array(ref[k], copy=True) for k in ("codes", "scales", "zeros", "row_loss")}
    for i in range(n_rows):
        r, flips = follow_row(codes[i], zeros[i], _row(ref, i), rerun, i, tie, max_flips_per_row)
        for k in matched:
            matched[k][i] = r[k]
        if flips:
            flipped_rows += 1
            n_flips += len(flips)
        # full tolerance against the matched oracle row
        d = codes[i].astype(np.int64) - r["codes"].astype(np.int64)
        if np.any(np.abs(d) > 1):
            raise ParityError(f"row {i}: a code differs by more than one step from its oracle row")
        matched_equal += int(np.sum(d == 0))
        if not np.array_equal(zeros[i], r["zeros"].astype(np.int64)):
            raise ParityError(f"row {i}: zero points differ from the oracle row")
        rel = np.abs(scales[i] - r["scales"]) / np.abs(r["scales"])
        worst_scale = max(worst_scale, float(rel.max(initial=0.0)))
        if not np.all(rel <= scale_rtol):
            raise ParityError(f"row {i}: scale off by {float(rel.max()):.3g} relative")
        lr = float(r["row_loss"])
        if abs(row_loss[i] - lr) > row_loss_rtol * abs(lr) + 1e-30:
            raise ParityError(f"row {i}: row loss {row_loss[i]:.6g} against {lr:.6g}")
    match = matched_equal / max(codes.size, 1)
    if match < 0.999:
        raise ParityError(f"codes match the followed oracle rows on {match:.6f} of entries")
    if flipped_rows > max(1, max_flip_rows * n_rows):
        raise ParityError(f"{flipped_rows} of {n_rows} rows took a near-tie flip (bound {max_flip_rows:.3g})")
    lref = float(np.sum(ref["row_loss"]))
    lt = float(np.sum(row_loss))
    if abs(lt - lref) > loss_rtol * abs(lref) + 1e-30:
        raise ParityError(f"loss {lt:.6g} against the oracle's {lref:.6g}")
    summary = dict(rows=n_rows, match_oracle=match0, max_abs_diff_oracle=int(np.abs(diff0).max(initial=0)),
                   flipped_rows=flipped_rows, flips=n_flips, match_followed=match, worst_scale_rel=worst_scale,
                   loss=lt, loss_oracle=lref, matched=matched)
    if log:
        log(f"  parity{(' ' + label) if label else ''}: {n_rows} rows; codes equal to the oracle's own rows "
            f"{match0:.6f} (max |diff| {summary['max_abs_diff_oracle']}); rows followed through near-tie flips "
            f"{flipped_rows} ({n_flips} flips); equal to the followed rows {match:.6f}; worst scale rel "
            f"{worst_scale:.2e}; loss {lt:.6g} vs {lref:.6g}")
    return summary
