"""Helpers for the GPU parity tests: host<->device copies of bf16 bit
patterns, guarded output buffers (canary bytes around every output catch
out-of-bounds writes) and the GEMM acceptance gates."""
import json
import os
import sys

import numpy as np
import torch

CANARY = 0xA5
PAD = 256  # bytes of guard on each side (keeps 16-byte alignment)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(a_u16: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a_u16, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class Guarded:
    """An output tensor with canary bytes before and after it."""

    def __init__(self, shape, dtype):
        self.shape = tuple(shape)
        self.dtype = dtype
        n = int(np.prod(self.shape)) if len(self.shape) else 1
        esz = torch.tensor([], dtype=dtype).element_size()
        self.nbytes = n * esz
        self.buf = torch.full((self.nbytes + 2 * PAD,), CANARY, dtype=torch.uint8, device="cuda")
        self.t = self.buf[PAD:PAD + self.nbytes].view(dtype).view(self.shape)

    def check(self):
        b = self.buf.cpu().numpy()
        assert np.all(b[:PAD] == CANARY), "write before the start of an output buffer"
        assert np.all(b[PAD + self.nbytes:] == CANARY), "write past the end of an output buffer"

    def np(self):
        return self.t.cpu().numpy()


def bf16_half_ulp(f: np.ndarray) -> np.ndarray:
    """Half an ulp of bf16 at the magnitude of f (binary32 values)."""
    a = np.abs(f.astype(np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 8)


def gemm_gate(G: np.ndarray, F: np.ndarray, D: np.ndarray, bf16: bool, tol: float = 1e-3):
    """Strict gate: rel = |G - F| / max(|F|, D/64) <= tol (less half a bf16
    ulp of F for BF16 outputs).  For data the matrix unit sums exactly.
    Returns (ok, max_rel, n_floored)."""
    G = G.astype(np.float64)
    Fd = F.astype(np.float64)
    floor = np.maximum(np.abs(Fd), D / 64.0)
    err = np.abs(G - Fd)
    if bf16:
        err = np.maximum(err - bf16_half_ulp(F), 0.0)
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = np.where(floor > 0, err / floor, np.where(err == 0, 0.0, np.inf))
    return bool(np.all(rel <= tol)), float(np.max(rel)) if rel.size else 0.0, int(np.sum(np.abs(Fd) < D / 64.0))


def gate_stats(G: np.ndarray, ref: dict, bf16: bool, tol: float = 1e-3, h_of=None):
    """The GEMM gate on every element:
        rel = |G - F| / max(|F|, D/64) <= tol
    with F the oracle's FP32-accumulated result and D = sum |a^ b^| (the
    floor keeps cancelled outputs from inflating the ratio); for BF16
    outputs the error is taken less half a bf16 ulp (at the larger binade of
    |F| and |G|: within tol before the final rounding).

    h_of(idx) -> H for the elements idx (k x 2 array of indices): the
    oracle's bound on what the matrix unit's in-instruction alignment may
    drop (each product of a group of 8 that has bits below 2^(e_max - 13)
    loses less than that step; measured rule of every FP8 matrix
    instruction of gfx950).  When given, the elements above tol are
    checked again as rel_hw = max(|G - F| - H, 0) / max(|F|, D/64): the
    same gate with that allowance, equal to rel wherever H = 0.
    Returns a dict: max rel, count above tol, floored entries, normwise
    error ||G - F|| / ||F||, and (with h_of) max rel_hw over all elements."""
    G64 = G.astype(np.float64)
    F = ref["F"].astype(np.float64)
    D = ref["D"]
    floor = np.maximum(np.abs(F), D / 64.0)
    err = np.abs(G64 - F)
    if bf16:   # half an ulp at the larger binade of F and the rounded G
        err = np.maximum(err - bf16_half_ulp(np.maximum(np.abs(F), np.abs(G64))), 0.0)
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = np.where(floor > 0, err / floor, np.where(err == 0, 0.0, np.inf))
    nf = float(np.linalg.norm(F))
    over = rel > tol
    st = {"max_rel": float(np.max(rel)) if rel.size else 0.0,
          "n_over": int(np.sum(over)), "n": int(rel.size),
          "n_floored": int(np.sum(np.abs(F) < D / 64.0)),
          "normwise": float(np.linalg.norm(G64 - F) / nf) if nf > 0 else 0.0}
    if h_of is not None:
        rel_hw = rel.copy()
        idx = np.argwhere(over)
        if len(idx):
            H = np.asarray(h_of(idx), np.float64)
            e2 = np.maximum(err[over] - H, 0.0)
            with np.errstate(invalid="ignore", divide="ignore"):
                rel_hw[over] = np.where(floor[over] > 0, e2 / floor[over],
                                        np.where(e2 == 0, 0.0, np.inf))
        st["max_rel_hw"] = float(np.max(rel_hw)) if rel_hw.size else 0.0
    return st


def h_sampler(O, A, af, asc, sa, B, bf, bsc, sb, ms=None, ns=None):
    """h_of for gate_stats on the output block (ms x ns) of the GEMM A B^T:
    the oracle's H at the requested elements (one row at a time)."""
    M, N = A.shape[0], B.shape[0]
    ms = np.arange(M, dtype=np.int64) if ms is None else np.asarray(ms, np.int64)
    ns = np.arange(N, dtype=np.int64) if ns is None else np.asarray(ns, np.int64)

    def h_of(idx):
        out = np.empty(len(idx), np.float64)
        for i in np.unique(idx[:, 0]):
            sel = np.nonzero(idx[:, 0] == i)[0]
            r = O.gemm(A, af, asc, sa, B, bf, bsc, sb, ms=ms[i:i + 1], ns=ns[idx[sel, 1]],
                       want=("H",))
            out[sel] = r["H"][0]
        return out
    return h_of


def log_gate(label: str, st: dict):
    """Print a GATE line (and append it to $FP8LIN_GATE_LOG when set)."""
    say("GATE", label, " ".join(f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}"
                                for k, v in st.items()))
    path = os.environ.get("FP8LIN_GATE_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"label": label, **st}) + "\n")


def gemm_check(G: np.ndarray, ref: dict, K: int, bf16: bool, tol: float = 1e-3):
    """Gate for random 8-bit codes over the whole format range (not the
    layer's data): products of such codes span up to 2^50 within one group
    of 8, where the matrix unit's alignment drops the low bits of all but
    the largest (rule measured on gfx950: each loses less than 2^(e_max-13)).
    This departs from the GEMM gate of gate_stats, which every test on the
    layer's data (and on exactly summable codes) asserts; two conditions on
    every element:
      (1) |G - F| <= tol * D            (relative error against sum |a^ b^|,
                                         less half a bf16 ulp for BF16 out);
      (2) |G - E| <= H + gamma * D + u_out |G|: the unit's bound H,
          binary32 combination of the K/8 group sums (gamma_{K/8+3} with
          2^-23 per operation), and the output rounding.
    Returns (ok1, ok2, max componentwise rel, max ratio to the model bound)."""
    G = G.astype(np.float64)
    F = ref["F"].astype(np.float64)
    E, D, H = ref["E"], ref["D"], ref["H"]
    e1 = np.abs(G - F)
    if bf16:
        e1 = np.maximum(e1 - bf16_half_ulp(ref["F"]), 0.0)
    with np.errstate(invalid="ignore", divide="ignore"):
        r1 = np.where(D > 0, e1 / D, np.where(e1 == 0, 0.0, np.inf))
    j = K / 8 + 3
    gam = j * 2.0 ** -23 / (1 - j * 2.0 ** -23)
    bound = H + gam * D + (2.0 ** -8 if bf16 else 0.0) * np.abs(G)
    e2 = np.abs(G - E)
    with np.errstate(invalid="ignore", divide="ignore"):
        r2 = np.where(bound > 0, e2 / bound, np.where(e2 == 0, 0.0, np.inf))
    m1 = float(np.max(r1)) if r1.size else 0.0
    m2 = float(np.max(r2)) if r2.size else 0.0
    return m1 <= tol, m2 <= 1.0, m1, m2
