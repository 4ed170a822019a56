"""Run the HIP path and the fp64 oracle on the same seeded inputs."""

from __future__ import annotations

import numpy as np
import torch

import layer_rnn_forward_amd as R
from oracle import rnn_oracle as orc


def normwise(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.size == 0:
        return 0.0
    den = max(float(np.max(np.abs(b))), 1e-30)
    return float(np.max(np.abs(a - b)) / den)


def to_dev(a, dtype=torch.float32):
    if a is None:
        return None
    return torch.as_tensor(np.ascontiguousarray(a), dtype=torch.float64).to(dtype).to("cuda")


def run_gpu(mode, L, D, case, wtype="f32", sched=R.SCHED_AUTO, training=True, backward=True,
            pass_state=True, pass_grads=True, repeat=1, lengths=None, dropout=None):
    """Returns a dict of numpy results from the library (fp32 -> fp64).
    ``lengths``: per-row valid steps (list of ints) or None; ``dropout``:
    ``(p, seed)`` of inter-layer dropout or None."""
    x = case["x"]
    T, B, I = x.shape
    H = case["params"][0][0]["w_hh"].shape[1]
    h = R.rnn_create(mode, L, D, I, H, wtype)
    R.rnn_set_schedule(h, sched)
    if dropout is not None:
        R.rnn_set_dropout(h, *dropout)
    if lengths is not None:
        R.rnn_set_sequence_lengths(h, torch.as_tensor(lengths, dtype=torch.int32, device="cuda"))
    W = R.pack_weights(h, case["params"])
    ws = torch.empty(R.rnn_workspace_size(h, T, B, 1 if training else 0), dtype=torch.uint8,
                     device="cuda")
    xd = to_dev(x)
    h0 = to_dev(case["h0"]) if pass_state else None
    c0 = to_dev(case["c0"]) if (pass_state and mode == "lstm") else None
    y = torch.full((T, B, D * H), float("nan"), device="cuda")
    hy = torch.full((L * D, B, H), float("nan"), device="cuda")
    cy = torch.full((L * D, B, H), float("nan"), device="cuda") if mode == "lstm" else None
    out = {}
    for _ in range(repeat):
        if training:
            R.rnn_forward_training(h, T, B, xd, h0, c0, W, y, hy, cy, ws)
        else:
            R.rnn_forward_inference(h, T, B, xd, h0, c0, W, y, hy, cy, ws)
        torch.cuda.synchronize()
        assert R.rnn_device_status(h, ws) == 0
        out["y"] = y.double().cpu().numpy().copy()
        out["hy"] = hy.double().cpu().numpy().copy()
        if mode == "lstm":
            out["cy"] = cy.double().cpu().numpy().copy()
        if training and backward:
            dy = to_dev(case["dy"])
            dhy = to_dev(case["dhy"]) if pass_grads else None
            dcy = to_dev(case["dcy"]) if (pass_grads and mode == "lstm") else None
            dx = torch.full((T, B, I), float("nan"), device="cuda")
            dh0 = torch.full((L * D, B, H), float("nan"), device="cuda")
            dc0 = torch.full((L * D, B, H), float("nan"), device="cuda") if mode == "lstm" else None
            R.rnn_backward_data(h, T, B, y, dy, dhy, dcy, W, h0, c0, dx, dh0, dc0, ws)
            dW = torch.full((R.rnn_weights_size(h, 1) // 4,), float("nan"), device="cuda")
            R.rnn_backward_weights(h, T, B, xd, h0, y, ws, dW)
            torch.cuda.synchronize()
            assert R.rnn_device_status(h, ws) == 0
            out["dx"] = dx.double().cpu().numpy().copy()
            out["dh0"] = dh0.double().cpu().numpy().copy()
            if mode == "lstm":
                out["dc0"] = dc0.double().cpu().numpy().copy()
            out["dW"] = R.unpack_weights(h, dW, grad=1)
    R.rnn_destroy(h)
    return out


# library modes that are oracle GRU flavours
GRU_FLAVOURS = {"gru_tf": "tf", "gru_paper": "paper"}


def run_oracle(mode, L, D, case, backward=True, pass_state=True, pass_grads=True, lengths=None,
               dropout=None):
    variant = GRU_FLAVOURS.get(mode, "pytorch")
    mode = "gru" if mode in GRU_FLAVOURS else mode
    h0 = case["h0"] if pass_state else None
    c0 = case["c0"] if (pass_state and mode == "lstm") else None
    y, hy, cy, cache = orc.forward(mode, case["x"], case["params"], h0=h0, c0=c0, num_dirs=D,
                                   gru_variant=variant, keep=backward, lengths=lengths,
                                   dropout=dropout[0] if dropout else 0.0,
                                   dropout_seed=dropout[1] if dropout else 0)
    out = {"y": y, "hy": hy}
    if mode == "lstm":
        out["cy"] = cy
    if backward:
        dhy = case["dhy"] if pass_grads else None
        dcy = case["dcy"] if (pass_grads and mode == "lstm") else None
        dx, dh0, dc0, dp = orc.backward(mode, case["params"], cache, case["dy"], dhy=dhy, dcy=dcy,
                                        num_dirs=D)
        out["dx"] = dx
        out["dh0"] = dh0
        if mode == "lstm":
            out["dc0"] = dc0
        out["dW"] = dp
    return out


def elementwise(a, b, floor=1e-3):
    """Largest elementwise relative error max |a - b| / max(|b|, floor): a
    diagnostic next to the normwise gate (reported, never gated on)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), floor)))


def compare(g, o, mode, L, D, report=True):
    """Per-output normwise errors, {name: err} (the gate).  With ``report``
    the elementwise diagnostic of every output is printed as well."""
    errs, diag = {}, {}
    pairs = []
    for k in ("y", "hy", "cy", "dx", "dh0", "dc0"):
        if k in g and k in o:
            pairs.append((k, g[k], o[k]))
    if "dW" in g and "dW" in o:
        for l in range(L):
            for d in range(D):
                for n in ("w_ih", "w_hh", "b_ih", "b_hh"):
                    pairs.append((f"d{n}[{l},{d}]", g["dW"][l][d][n], o["dW"][l][d][n]))
    for k, a, b in pairs:
        errs[k] = normwise(a, b)
        diag[k] = elementwise(a, b)
    if report and diag:
        worst = max(diag, key=diag.get)
        print(f"elementwise max |g-o|/max(|o|,1e-3): worst {worst} {diag[worst]:.2e}; "
              f"normwise worst {max(errs.values()):.2e}", flush=True)
    return errs


FWD_KEYS = ("y", "hy", "cy")


def check(errs, tol_fwd, tol_bwd):
    bad = {k: v for k, v in errs.items()
           if not (v <= (tol_fwd if k in FWD_KEYS else tol_bwd))}
    assert not bad, f"parity failures: {bad}"
