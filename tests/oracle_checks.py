"""Checks that pin the fp64 oracle to things other than itself.

Each check takes the oracle *module* as an argument so that the mutation test
can run the same checks against deliberately broken copies of the oracle.
Every check returns the worst error it saw (a float); callers compare it with
a tolerance.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def zero_params(G, I, H, L=1, D=1):
    out = []
    for l in range(L):
        I_l = I if l == 0 else D * H
        out.append([{"w_ih": np.zeros((G * H, I_l)), "w_hh": np.zeros((G * H, H)),
                     "b_ih": np.zeros(G * H), "b_hh": np.zeros(G * H)} for _ in range(D)])
    return out


def rand_case(mode, L, D, T, B, I, H, seed, scale=0.6):
    """Small random case in fp64 (own generator; the oracle pins do not need
    the working-precision rounding of the GPU inputs)."""
    G = {"rnn_tanh": 1, "lstm": 4, "gru": 3}[mode]
    rng = np.random.default_rng(seed)
    params = []
    for l in range(L):
        I_l = I if l == 0 else D * H
        params.append([{"w_ih": rng.uniform(-scale, scale, (G * H, I_l)),
                        "w_hh": rng.uniform(-scale, scale, (G * H, H)),
                        "b_ih": rng.uniform(-scale, scale, G * H),
                        "b_hh": rng.uniform(-scale, scale, G * H)} for _ in range(D)])
    x = rng.normal(size=(T, B, I))
    h0 = rng.normal(size=(L * D, B, H)) * 0.5
    c0 = rng.normal(size=(L * D, B, H)) * 0.5 if mode == "lstm" else None
    dy = rng.normal(size=(T, B, D * H))
    dhy = rng.normal(size=(L * D, B, H))
    dcy = rng.normal(size=(L * D, B, H)) if mode == "lstm" else None
    return dict(params=params, x=x, h0=h0, c0=c0, dy=dy, dhy=dhy, dcy=dcy)


def normwise(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / den) if a.size else 0.0


# ---------------------------------------------------------------- GRU variants
def check_gru_worked_values(orc):
    """Worst absolute error against the hand-worked values of the three GRU
    flavours (golden fixture)."""
    spec = json.load(open(os.path.join(GOLDEN, "gru_variants_worked.json")))
    inp = spec["inputs"]
    worst = 0.0
    for case in spec["cases"]:
        b_iz = math.log(3.0) if case["b_iz"] == "ln3" else float(case["b_iz"])
        p = {"w_ih": np.zeros((3, 1)), "w_hh": np.zeros((3, 1)),
             "b_ih": np.array([inp["b_ir"], b_iz, inp["b_in"]]),
             "b_hh": np.array([inp["b_hr"], inp["b_hz"], inp["b_hn"]])}
        x = np.full((1, 1, 1), inp["x"])
        h0 = np.full((1, 1, 1), inp["h_prev"])
        for variant in ("pytorch", "tf", "paper"):
            y, hy, _, _ = orc.forward("gru", x, [[p]], h0=h0, gru_variant=variant)
            worst = max(worst, abs(float(y[0, 0, 0]) - case[variant]),
                        abs(float(hy[0, 0, 0]) - case[variant]))
    return worst


# ---------------------------------------------------------------- closed forms
def check_closed_forms(orc):
    spec = json.load(open(os.path.join(GOLDEN, "closed_forms.json")))
    worst = 0.0
    # GRU: b_in = 1, everything else 0, h0 = 0
    for T_s, val in spec["gru_constant_input"]["values"].items():
        T = int(T_s)
        p = zero_params(3, 2, 3)
        p[0][0]["b_ih"][6:9] = 1.0
        x = np.zeros((T, 2, 2))
        y, hy, _, _ = orc.forward("gru", x, p)
        worst = max(worst, float(np.max(np.abs(hy - val))))
        # the formula itself at every step, nonzero h0
        h0 = np.full((1, 2, 3), 0.3)
        y, hy, _, _ = orc.forward("gru", x, p, h0=h0)
        tb = math.tanh(1.0)
        for t in range(T):
            ref = tb + 2.0 ** -(t + 1) * (0.3 - tb)
            worst = max(worst, float(np.max(np.abs(y[t] - ref))))
    # LSTM: b_ih = 1, b_hh = 0, c0 = 0
    for T_s, val in spec["lstm_all_bias_one"]["values"].items():
        T = int(T_s)
        p = zero_params(4, 3, 2)
        p[0][0]["b_ih"][:] = 1.0
        x = np.zeros((T, 2, 3))
        y, hy, cy, _ = orc.forward("lstm", x, p)
        worst = max(worst, float(np.max(np.abs(hy - val))))
    for T_s, val in spec["lstm_zero_bias_c0_one"]["values"].items():
        T = int(T_s)
        p = zero_params(4, 3, 2)
        x = np.zeros((T, 1, 3))
        y, hy, cy, _ = orc.forward("lstm", x, p, c0=np.ones((1, 1, 2)))
        worst = max(worst, float(np.max(np.abs(hy - val))),
                    float(np.max(np.abs(cy - 2.0 ** -T))))
    # LSTM general constant-gate recurrence with distinct gate biases
    b = np.array([0.3, -0.7, 0.9, 0.2])
    p = zero_params(4, 1, 1)
    p[0][0]["b_ih"][:] = b
    T = 7
    c0 = 0.4
    y, hy, cy, _ = orc.forward("lstm", np.zeros((T, 1, 1)), p, c0=np.full((1, 1, 1), c0),
                               h0=np.full((1, 1, 1), -0.8))
    s = lambda a: 1.0 / (1.0 + math.exp(-a))
    i, f, g, o = s(b[0]), s(b[1]), math.tanh(b[2]), s(b[3])
    for t in range(T):
        n = t + 1
        c_ref = f ** n * c0 + i * g * (1 - f ** n) / (1 - f)
        worst = max(worst, abs(float(y[t, 0, 0]) - o * math.tanh(c_ref)))
    # vanilla: h_t = tanh(b_ih + b_hh) independent of h0
    p = zero_params(1, 2, 3)
    p[0][0]["b_ih"][:] = [0.1, -0.4, 2.0]
    p[0][0]["b_hh"][:] = [0.5, 0.3, -1.0]
    y, hy, _, _ = orc.forward("rnn_tanh", np.zeros((4, 2, 2)), p, h0=np.full((1, 2, 3), 0.7))
    ref = np.tanh(np.array([0.6, -0.1, 1.0]))
    worst = max(worst, float(np.max(np.abs(y - ref))))
    return worst


def check_bptt_closed_forms(orc):
    worst = 0.0
    # GRU, same weights as the forward closed form: only path is z*h -> dh0 = 2^-T g
    for T in (1, 3, 16):
        p = zero_params(3, 2, 3)
        p[0][0]["b_ih"][6:9] = 1.0
        x = np.zeros((T, 2, 2))
        _, _, _, cache = orc.forward("gru", x, p, keep=True)
        g = np.arange(1.0, 7.0).reshape(1, 2, 3)
        dx, dh0, _, _ = orc.backward("gru", p, cache, np.zeros((T, 2, 3)), dhy=g)
        worst = max(worst, float(np.max(np.abs(dh0 - 2.0 ** -T * g))))
        worst = max(worst, float(np.max(np.abs(dx))))
    # LSTM: dy = dhy = 0, dcy = g -> dc0 = sigmoid(b_f)^T g, dh0 = 0
    bf = 0.35
    for T in (1, 4, 9):
        p = zero_params(4, 2, 3)
        p[0][0]["b_ih"][3:6] = bf
        x = np.zeros((T, 2, 2))
        _, _, _, cache = orc.forward("lstm", x, p, c0=np.full((1, 2, 3), 0.2), keep=True)
        g = np.linspace(-1, 1, 6).reshape(1, 2, 3)
        dx, dh0, dc0, _ = orc.backward("lstm", p, cache, np.zeros((T, 2, 3)),
                                       dhy=np.zeros((1, 2, 3)), dcy=g)
        f = 1.0 / (1.0 + math.exp(-bf))
        worst = max(worst, float(np.max(np.abs(dc0 - f ** T * g))),
                    float(np.max(np.abs(dh0))))
    # vanilla: dh0 = 0 with zero recurrent weights
    p = zero_params(1, 2, 3)
    p[0][0]["b_ih"][:] = 0.4
    _, _, _, cache = orc.forward("rnn_tanh", np.zeros((5, 2, 2)), p, keep=True)
    rng = np.random.default_rng(0)
    _, dh0, _, _ = orc.backward("rnn_tanh", p, cache, rng.normal(size=(5, 2, 3)),
                                dhy=rng.normal(size=(1, 2, 3)))
    worst = max(worst, float(np.max(np.abs(dh0))))
    return worst


# ------------------------------------------------------------- torch.nn match
def _torch_module(mode, I, H, L, D):
    kw = dict(input_size=I, hidden_size=H, num_layers=L, bidirectional=(D == 2),
              dtype=torch.float64)
    if mode == "lstm":
        return torch.nn.LSTM(**kw)
    if mode == "gru":
        return torch.nn.GRU(**kw)
    return torch.nn.RNN(nonlinearity="tanh", **kw)


def check_against_torch(orc, mode, L, D, T=4, B=3, I=5, H=6, seed=11, lengths=None):
    """Normwise error of the oracle's forward outputs and all gradients
    against ``torch.nn`` in float64 on the CPU (same equations; PyTorch is
    the implementation the oneDNN issue names for the GRU flavour).  With
    ``lengths`` (all >= 1, torch's packed sequences reject empty rows) the
    torch module runs on ``pack_padded_sequence`` input and its output is
    padded back with zeros."""
    case = rand_case(mode, L, D, T, B, I, H, seed)
    params = case["params"]
    m = _torch_module(mode, I, H, L, D)
    with torch.no_grad():
        for l in range(L):
            for d in range(D):
                sfx = f"l{l}" + ("_reverse" if d == 1 else "")
                for name in ("w_ih", "w_hh", "b_ih", "b_hh"):
                    tname = {"w_ih": "weight_ih_", "w_hh": "weight_hh_",
                             "b_ih": "bias_ih_", "b_hh": "bias_hh_"}[name] + sfx
                    getattr(m, tname).copy_(torch.from_numpy(params[l][d][name]))
    x = torch.from_numpy(case["x"]).requires_grad_(True)
    h0 = torch.from_numpy(case["h0"]).requires_grad_(True)
    xin = x
    if lengths is not None:
        xin = torch.nn.utils.rnn.pack_padded_sequence(
            x, torch.as_tensor(lengths, dtype=torch.int64), enforce_sorted=False)
    if mode == "lstm":
        c0 = torch.from_numpy(case["c0"]).requires_grad_(True)
        out, (hn, cn) = m(xin, (h0, c0))
    else:
        out, hn = m(xin, h0)
    if lengths is not None:
        out, _ = torch.nn.utils.rnn.pad_packed_sequence(out, total_length=T)
    loss = (out * torch.from_numpy(case["dy"])).sum() + (hn * torch.from_numpy(case["dhy"])).sum()
    if mode == "lstm":
        loss = loss + (cn * torch.from_numpy(case["dcy"])).sum()
    loss.backward()

    y, hy, cy, cache = orc.forward(mode, case["x"], params, h0=case["h0"], c0=case["c0"],
                                   num_dirs=D, keep=True, lengths=lengths)
    errs = [normwise(y, out.detach().numpy()), normwise(hy, hn.detach().numpy())]
    if mode == "lstm":
        errs.append(normwise(cy, cn.detach().numpy()))
    dx, dh0, dc0, dparams = orc.backward(mode, params, cache, case["dy"], dhy=case["dhy"],
                                         dcy=case["dcy"], num_dirs=D)
    errs += [normwise(dx, x.grad.numpy()), normwise(dh0, h0.grad.numpy())]
    if mode == "lstm":
        errs.append(normwise(dc0, c0.grad.numpy()))
    for l in range(L):
        for d in range(D):
            sfx = f"l{l}" + ("_reverse" if d == 1 else "")
            for name, tname in (("w_ih", "weight_ih_"), ("w_hh", "weight_hh_"),
                                ("b_ih", "bias_ih_"), ("b_hh", "bias_hh_")):
                errs.append(normwise(dparams[l][d][name], getattr(m, tname + sfx).grad.numpy()))
    return max(errs)


def check_dropout_against_torch(orc, mode, L, D, p, seed, T=4, B=3, I=5, H=6, case_seed=23):
    """Normwise error of the oracle's training pass with inter-layer dropout
    against a composition of one-layer ``torch.nn`` modules (float64, CPU):
    layer ``l``'s input is the previous module's output times
    ``keep_l / (1 - p)``, with ``keep_l`` from ``orc.dropout_keep`` and the
    scaling done here; torch's autograd supplies every gradient."""
    case = rand_case(mode, L, D, T, B, I, H, case_seed)
    params = case["params"]
    x = torch.from_numpy(case["x"]).requires_grad_(True)
    h0 = torch.from_numpy(case["h0"]).requires_grad_(True)
    c0 = torch.from_numpy(case["c0"]).requires_grad_(True) if mode == "lstm" else None
    mods, hns, cns = [], [], []
    inp = x
    for l in range(L):
        I_l = I if l == 0 else D * H
        m = _torch_module(mode, I_l, H, 1, D)
        with torch.no_grad():
            for d in range(D):
                sfx = "l0" + ("_reverse" if d == 1 else "")
                for name, tname in (("w_ih", "weight_ih_"), ("w_hh", "weight_hh_"),
                                    ("b_ih", "bias_ih_"), ("b_hh", "bias_hh_")):
                    getattr(m, tname + sfx).copy_(torch.from_numpy(params[l][d][name]))
        if l > 0:
            keep = orc.dropout_keep(p, seed, l, tuple(inp.shape))
            scale = 1.0 / (1.0 - p) if p < 1.0 else 0.0
            inp = inp * torch.from_numpy(np.where(keep, scale, 0.0))
        if mode == "lstm":
            inp, (hn, cn) = m(inp, (h0[l * D:(l + 1) * D], c0[l * D:(l + 1) * D]))
            cns.append(cn)
        else:
            inp, hn = m(inp, h0[l * D:(l + 1) * D])
        hns.append(hn)
        mods.append(m)
    hn = torch.cat(hns, 0)
    loss = (inp * torch.from_numpy(case["dy"])).sum() + (hn * torch.from_numpy(case["dhy"])).sum()
    if mode == "lstm":
        cn = torch.cat(cns, 0)
        loss = loss + (cn * torch.from_numpy(case["dcy"])).sum()
    loss.backward()

    y, hy, cy, cache = orc.forward(mode, case["x"], params, h0=case["h0"], c0=case["c0"],
                                   num_dirs=D, keep=True, dropout=p, dropout_seed=seed)
    errs = [normwise(y, inp.detach().numpy()), normwise(hy, hn.detach().numpy())]
    if mode == "lstm":
        errs.append(normwise(cy, cn.detach().numpy()))
    dx, dh0, dc0, dparams = orc.backward(mode, params, cache, case["dy"], dhy=case["dhy"],
                                         dcy=case["dcy"], num_dirs=D)
    errs += [normwise(dx, x.grad.numpy()), normwise(dh0, h0.grad.numpy())]
    if mode == "lstm":
        errs.append(normwise(dc0, c0.grad.numpy()))
    for l in range(L):
        for d in range(D):
            sfx = "l0" + ("_reverse" if d == 1 else "")
            for name, tname in (("w_ih", "weight_ih_"), ("w_hh", "weight_hh_"),
                                ("b_ih", "bias_ih_"), ("b_hh", "bias_hh_")):
                errs.append(normwise(dparams[l][d][name], getattr(mods[l], tname + sfx).grad.numpy()))
    return max(errs)


# --------------------------------------------------------- finite differences
def _loss(orc, mode, case, D, lengths=None, gru_variant="pytorch", dropout=0.0, dropout_seed=0):
    y, hy, cy, _ = orc.forward(mode, case["x"], case["params"], h0=case["h0"], c0=case["c0"],
                               num_dirs=D, lengths=lengths, gru_variant=gru_variant,
                               dropout=dropout, dropout_seed=dropout_seed)
    v = float(np.sum(y * case["dy"]) + np.sum(hy * case["dhy"]))
    if mode == "lstm":
        v += float(np.sum(cy * case["dcy"]))
    return v


def check_finite_differences(orc, mode, L, D, T=3, B=2, I=3, H=4, seed=5, eps=1e-6,
                             lengths=None, gru_variant="pytorch", dropout=0.0, dropout_seed=0):
    """Worst normwise error of every analytic gradient against central
    differences of the scalar loss ``sum(y*dy) + sum(hy*dhy) + sum(cy*dcy)``
    (optionally with per-row sequence lengths, or another GRU flavour)."""
    case = rand_case(mode, L, D, T, B, I, H, seed)
    _, _, _, cache = orc.forward(mode, case["x"], case["params"], h0=case["h0"], c0=case["c0"],
                                 num_dirs=D, keep=True, lengths=lengths, gru_variant=gru_variant,
                                 dropout=dropout, dropout_seed=dropout_seed)
    dx, dh0, dc0, dparams = orc.backward(mode, case["params"], cache, case["dy"],
                                         dhy=case["dhy"], dcy=case["dcy"], num_dirs=D)

    def fd(arr):
        g = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = arr[idx]
            arr[idx] = old + eps
            lp = _loss(orc, mode, case, D, lengths, gru_variant, dropout, dropout_seed)
            arr[idx] = old - eps
            lm = _loss(orc, mode, case, D, lengths, gru_variant, dropout, dropout_seed)
            arr[idx] = old
            g[idx] = (lp - lm) / (2 * eps)
        return g

    errs = [normwise(dx, fd(case["x"])), normwise(dh0, fd(case["h0"]))]
    if mode == "lstm":
        errs.append(normwise(dc0, fd(case["c0"])))
    for l in range(L):
        for d in range(D):
            for name in ("w_ih", "w_hh", "b_ih", "b_hh"):
                errs.append(normwise(dparams[l][d][name], fd(case["params"][l][d][name])))
    return max(errs)


# ------------------------------------------------------------ packed batches
def check_packed_truncation(orc, mode, L, D, lengths, T=5, I=3, H=4, seed=17):
    """Worst normwise error between a batch with per-row lengths and, row by
    row, the plain (unmasked) pass over that row's sequence cut to its
    length: outputs, final states, dx, dh0, dc0 and the weight gradients
    (the batched gradient is the sum of the rows').  Rows of length 0 must
    return h0 / dhy unchanged and zeros elsewhere."""
    B = len(lengths)
    case = rand_case(mode, L, D, T, B, I, H, seed)
    P = case["params"]
    y, hy, cy, cache = orc.forward(mode, case["x"], P, h0=case["h0"], c0=case["c0"],
                                   num_dirs=D, keep=True, lengths=lengths)
    dx, dh0, dc0, dp = orc.backward(mode, P, cache, case["dy"], dhy=case["dhy"], dcy=case["dcy"],
                                    num_dirs=D)
    errs = []
    acc = [[{k: np.zeros_like(v) for k, v in P[l][d].items()} for d in range(D)] for l in range(L)]
    for b, n in enumerate(lengths):
        sl = slice(b, b + 1)
        st = lambda a: None if a is None else a[:, sl]
        if n == 0:
            errs += [float(np.max(np.abs(y[:, b]))), float(np.max(np.abs(dx[:, b]))),
                     normwise(hy[:, b], case["h0"][:, b]), normwise(dh0[:, b], case["dhy"][:, b])]
            if mode == "lstm":
                errs += [normwise(cy[:, b], case["c0"][:, b]), normwise(dc0[:, b], case["dcy"][:, b])]
            continue
        yr, hyr, cyr, cr = orc.forward(mode, case["x"][:n, sl], P, h0=st(case["h0"]), c0=st(case["c0"]),
                                       num_dirs=D, keep=True)
        dxr, dh0r, dc0r, dpr = orc.backward(mode, P, cr, case["dy"][:n, sl], dhy=st(case["dhy"]),
                                            dcy=st(case["dcy"]), num_dirs=D)
        errs += [normwise(y[:n, b], yr[:, 0]), float(np.max(np.abs(y[n:, b]), initial=0.0)),
                 normwise(hy[:, b], hyr[:, 0]), normwise(dx[:n, b], dxr[:, 0]),
                 float(np.max(np.abs(dx[n:, b]), initial=0.0)), normwise(dh0[:, b], dh0r[:, 0])]
        if mode == "lstm":
            errs += [normwise(cy[:, b], cyr[:, 0]), normwise(dc0[:, b], dc0r[:, 0])]
        for l in range(L):
            for d in range(D):
                for k in acc[l][d]:
                    acc[l][d][k] += dpr[l][d][k]
    for l in range(L):
        for d in range(D):
            for k in acc[l][d]:
                errs.append(normwise(dp[l][d][k], acc[l][d][k]))
    return max(errs)


# ---------------------------------------------------------------- dropout
# Random123 known-answer vectors of Philox4x32-10 and Philox4x64-10:
# (counter words, key words, output words)
PHILOX_KAT32 = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]
PHILOX_KAT64 = [((0, 0, 0, 0), (0, 0),
                 (0x16554D9ECA36314C, 0xDB20FE9D672D0FDC, 0xD7E772CEE186176B, 0x7E68B68AEC7BA23B))]


def philox_kat_failures(px):
    """Known-answer vectors missed by the scalar and the array generator."""
    bad = []
    for ctr, key, out in PHILOX_KAT32:
        if tuple(px.philox4(ctr, key, 32)) != out:
            bad.append(("scalar32", ctr))
        arr = px.philox4x32_array(*[np.array([c]) for c in ctr], *key)
        if tuple(int(a[0]) for a in arr) != out:
            bad.append(("array32", ctr))
    for ctr, key, out in PHILOX_KAT64:
        if tuple(px.philox4(ctr, key, 64)) != out:
            bad.append(("scalar64", ctr))
    return bad


def dropout_mask_failures(orc, px):
    """Properties of ``orc.dropout_keep`` that do not restate its code:
    keep fraction within 6 sigma of 1 - p, a different mask per layer and
    per seed (both seed words), dependence on the flat index only, nesting
    in p, the p = 0 / p = 1 ends, and single elements against the scalar
    generator ``px.philox4``."""
    bad = []
    for p in (0.1, 0.5, 0.9):
        k = orc.dropout_keep(p, 2024, 1, (50, 20, 64))
        if abs(k.sum() - k.size * (1 - p)) >= 6 * np.sqrt(k.size * p * (1 - p)):
            bad.append(("fraction", p))
    shape = (6, 5, 40)
    a = orc.dropout_keep(0.5, 99, 1, shape)
    if np.array_equal(a, orc.dropout_keep(0.5, 99, 2, shape)):
        bad.append("layer")
    if np.array_equal(a, orc.dropout_keep(0.5, 100, 1, shape)):
        bad.append("seed")
    if np.array_equal(a, orc.dropout_keep(0.5, 99 + (1 << 32), 1, shape)):
        bad.append("seed-high")
    if not np.array_equal(a.ravel(), orc.dropout_keep(0.5, 99, 1, (a.size, 1, 1)).ravel()):
        bad.append("flat")
    lo, hi = orc.dropout_keep(0.3, 99, 1, shape), orc.dropout_keep(0.6, 99, 1, shape)
    if not np.all(lo[hi]):
        bad.append("nested")
    if not orc.dropout_keep(0.0, 99, 1, shape).all() or orc.dropout_keep(1.0, 99, 1, shape).any():
        bad.append("ends")
    # element e = 4q + w takes word w at counter (q mod 2^32, q div 2^32, layer, 0)
    shape, p, layer = (7, 3, 10), 0.37, 2
    seed = (0xA5A5A5A5 << 32) | 0x01020304
    k = orc.dropout_keep(p, seed, layer, shape).ravel()
    thr = orc.dropout_threshold(p)
    for e in (0, 1, 2, 3, 4, 77, 150, k.size - 1):
        q, w = divmod(e, 4)
        word = px.philox4((q & 0xFFFFFFFF, q >> 32, layer, 0),
                          (seed & 0xFFFFFFFF, seed >> 32), 32)[w]
        if bool(k[e]) != (word >= thr):
            bad.append(("element", e))
    return bad
