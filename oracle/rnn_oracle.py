"""Plain fp64 implementation of the stacked RNN forward pass and its
backward-through-time (BPTT).

TEST INFRASTRUCTURE ONLY (see the package docstring).  Slow on purpose: one
time step at a time, one matrix product per term, no blocking, no fusion, no
hoisting of the input projection.  Every function here is pinned by the
tests in ``tests/test_oracle_*.py`` (hand-worked GRU values, zero-weight
closed forms, central finite differences, invariants, and ``torch.nn`` fp64
special cases); none is left unpinned.

Notation (per layer ``l`` and direction ``d``)
----------------------------------------------
* ``G`` gate blocks of width ``H`` each, in memory order
  ``rnn_tanh: [a]``, ``lstm: [i, f, g, o]``, ``gru: [r, z, n]``.
* ``gi_t = x_t W_ih^T + b_ih`` and ``gh_t = h_prev W_hh^T + b_hh``, both
  ``[B, G*H]`` -- the two ``F.linear`` calls of the PyTorch GRU snippet in
  oneDNN issue #218 "rnn training example?", applied to every cell type.
* ``h_prev`` is ``h_{t-1}`` for ``d = 0`` and ``h_{t+1}`` for ``d = 1``
  (direction 1 walks ``t = T-1 .. 0``); the first ``h_prev`` is
  ``h0[l*D + d]``.

Cell equations
--------------
* GRU, PyTorch/cuDNN flavour (the flavour the same issue says PyTorch and
  cuDNN share; equations listed under "PyTorch equations" and in the snippet):
  ``r = s(gi_r + gh_r)``, ``z = s(gi_z + gh_z)``,
  ``n = tanh(gi_n + r * gh_n)``, ``h = (1 - z) * n + z * h_prev``.
* GRU, TensorFlow flavour (listed as "Tensorflow" and as the flavour oneDNN
  first implemented): ``n = tanh(gi_n + (r * h_prev) W_hn^T + b_hn)``; ``h``
  as PyTorch.  The stray closing parenthesis printed in that line is read as
  a typo.
* GRU, original-paper flavour ("Note that in the paper"): ``n`` as
  TensorFlow, ``h = (1 - z) * h_prev + z * n``.
* LSTM (named on the MXNet "fused RNN operator" page, equations not printed):
  the standard two-bias form ``a = gi + gh`` split ``[i, f, g, o]``,
  ``i, f, o = s(.)``, ``g = tanh(.)``, ``c = f * c_prev + i * g``,
  ``h = o * tanh(c)``; no peepholes, no projection, no forget-bias offset.
* Vanilla RNN (named on the same page as "Vanilla RNN", equations not
  printed): ``h = tanh(gi + gh)``.

Stacking (Keras issue #3692, the ``CudnnLSTM(num_layers, ...)`` descriptor;
MXNet page, "5-layers ... with bi-direction"): the input of layer 0 is ``x``,
the input of layer ``l > 0`` is ``y_{l-1}``, the concatenation
``[h^(0) | h^(1)]`` along features; ``y_l[t, :, d*H:(d+1)*H] = h_t^(d)``;
``hy[l*D + d]`` (and ``cy``) is the last state produced: ``h_{T-1}`` for
``d = 0`` and ``h_0`` for ``d = 1`` (shapes ``(num_layers*num_directions,
batch, hidden)`` from the hx/cx/hy/cy question in oneDNN issue #218).

Variable-length (packed) batches (the packed-sequence question of oneDNN
issue #218 asks for them; the pages fix no semantics, so the plainest
reading -- the one PyTorch's packed sequences have -- is taken): row ``b``
has ``lengths[b]`` valid steps ``t < lengths[b]``; at the other steps its
state is carried unchanged (``h``, and ``c`` for LSTM) and its output is 0.
Direction 0 thus stops at ``t = lengths[b] - 1`` and direction 1 starts
there, so ``hy`` is the state after the last valid step of each direction.
In the backward pass such a step passes ``dh`` (and ``dc``) through
unchanged, ignores ``dy`` there, and contributes nothing to ``dx``, ``dW``
or ``db``.

Inter-layer dropout (the MKL-DNN issue thread asks whether dropout will
come as cuDNN has it; the pages fix no semantics, so the plainest reading,
cuDNN's and PyTorch's, is taken): in training, the input of every layer ``l >= 1`` is
``y_{l-1} * m_l`` with ``m_l = keep_l / (1 - p)`` (inverted dropout: kept
elements are scaled so the expectation is unchanged; ``m_l = 0`` for
``p = 1``); ``x`` itself, the recurrent state and the top layer's ``y`` are
never dropped.  The keep mask is drawn from Philox4x32-10
(:mod:`oracle.philox`) -- see :func:`dropout_multiplier`.  The backward pass
multiplies the gradient reaching ``y_{l-1}`` by the same ``m_l``, and
``dW_ih`` of layer ``l`` uses the dropped input.

Backward (the pages only say forward results are reused by the backward
pass, MXNet page "Operator Registration"; the chain rule below is derived by
hand and pinned by central finite differences): see :func:`backward`.
"""

from __future__ import annotations

import math

import numpy as np

from oracle.philox import philox4x32_array

MODES = ("rnn_tanh", "lstm", "gru")
GATES = {"rnn_tanh": 1, "lstm": 4, "gru": 3}
GRU_VARIANTS = ("pytorch", "tf", "paper")


def _sigmoid(a):
    # logistic function; exp overflow for very negative a gives 1/inf = 0,
    # which is the correct limit
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-a))


def _blocks(a, n):
    """Split the last axis of ``a`` into ``n`` equal gate blocks."""
    return np.split(a, n, axis=-1)


def cell_forward(mode, x_t, h_prev, c_prev, p, gru_variant="pytorch"):
    """One cell step.  Returns ``(h, c, saved)`` where ``saved`` holds what
    the backward pass needs for this step.

    ``x_t`` ``[B, I]``, ``h_prev``/``c_prev`` ``[B, H]`` (``c_prev`` ignored
    unless LSTM), ``p`` a dict with ``w_ih [G*H, I]``, ``w_hh [G*H, H]``,
    ``b_ih [G*H]``, ``b_hh [G*H]``.
    """
    gi = x_t @ p["w_ih"].T + p["b_ih"]
    if mode == "rnn_tanh":
        gh = h_prev @ p["w_hh"].T + p["b_hh"]
        h = np.tanh(gi + gh)
        return h, None, {"h": h}
    if mode == "lstm":
        gh = h_prev @ p["w_hh"].T + p["b_hh"]
        a_i, a_f, a_g, a_o = _blocks(gi + gh, 4)
        i = _sigmoid(a_i)
        f = _sigmoid(a_f)
        g = np.tanh(a_g)
        o = _sigmoid(a_o)
        c = f * c_prev + i * g
        h = o * np.tanh(c)
        return h, c, {"i": i, "f": f, "g": g, "o": o, "c": c, "c_prev": c_prev}
    if mode == "gru":
        H = h_prev.shape[1]
        gi_r, gi_z, gi_n = _blocks(gi, 3)
        w_hr, w_hz, w_hn = (p["w_hh"][k * H:(k + 1) * H] for k in range(3))
        b_hr, b_hz, b_hn = (p["b_hh"][k * H:(k + 1) * H] for k in range(3))
        r = _sigmoid(gi_r + h_prev @ w_hr.T + b_hr)
        z = _sigmoid(gi_z + h_prev @ w_hz.T + b_hz)
        if gru_variant == "pytorch":
            gh_n = h_prev @ w_hn.T + b_hn
            n = np.tanh(gi_n + r * gh_n)
            h = (1.0 - z) * n + z * h_prev
            return h, None, {"r": r, "z": z, "n": n, "gh_n": gh_n}
        if gru_variant in ("tf", "paper"):
            n = np.tanh(gi_n + (r * h_prev) @ w_hn.T + b_hn)
            if gru_variant == "tf":
                h = (1.0 - z) * n + z * h_prev
            else:
                h = (1.0 - z) * h_prev + z * n
            return h, None, {"r": r, "z": z, "n": n}
        raise ValueError(f"unknown GRU variant {gru_variant!r}")
    raise ValueError(f"unknown mode {mode!r}")


def _check_params(mode, params, num_layers, num_dirs, input_size, hidden):
    G = GATES[mode]
    assert len(params) == num_layers
    for l in range(num_layers):
        assert len(params[l]) == num_dirs
        I_l = input_size if l == 0 else num_dirs * hidden
        for d in range(num_dirs):
            p = params[l][d]
            assert p["w_ih"].shape == (G * hidden, I_l), (l, d, p["w_ih"].shape)
            assert p["w_hh"].shape == (G * hidden, hidden)
            assert p["b_ih"].shape == (G * hidden,)
            assert p["b_hh"].shape == (G * hidden,)


def _valid_rows(lengths, t, B):
    """``[B, 1]`` boolean mask of the rows for which step ``t`` is valid."""
    if lengths is None:
        return np.ones((B, 1), dtype=bool)
    return (t < np.asarray(lengths))[:, None]


def dropout_threshold(p):
    """Integer threshold of drop probability ``p``: an element is dropped
    when its 32-bit random word is below ``floor(p * 2**32)`` (exact in
    fp64: a power-of-two scaling), so ``p = 0`` drops nothing and ``p = 1``
    drops everything."""
    if not 0.0 <= p <= 1.0:
        raise ValueError(f"dropout probability {p} outside [0, 1]")
    return math.floor(p * 4294967296.0)


def dropout_keep(p, seed, layer, shape):
    """Keep mask (bool, ``shape`` = ``[T, B, C]``) of the input of layer
    ``layer`` in a training pass with seed ``seed`` (below 2**64).

    Element ``e`` (row-major flat index) takes word ``e mod 4`` of
    Philox4x32-10 applied to the counter ``(q mod 2**32, q div 2**32, layer,
    0)``, ``q = e div 4``, under the key ``(seed mod 2**32, seed div
    2**32)``; it is kept when that word is at least
    :func:`dropout_threshold`."""
    n = int(np.prod(shape))
    e = np.arange(n, dtype=np.uint64)
    q = e >> np.uint64(2)
    words = philox4x32_array(q & np.uint64(0xFFFFFFFF), q >> np.uint64(32),
                             np.full(n, layer, dtype=np.uint64), np.zeros(n, dtype=np.uint64),
                             seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    w = np.stack(words, axis=0)[(e & np.uint64(3)).astype(np.int64), np.arange(n)]
    return (w.astype(np.int64) >= dropout_threshold(p)).reshape(shape)


def dropout_multiplier(p, seed, layer, shape):
    """``keep / (1 - p)`` (0 where dropped; all 0 for ``p = 1``)."""
    k = dropout_keep(p, seed, layer, shape)
    return np.where(k, 1.0 / (1.0 - p) if p < 1.0 else 0.0, 0.0)


def forward(mode, x, params, h0=None, c0=None, num_dirs=1, gru_variant="pytorch",
            keep=False, lengths=None, dropout=0.0, dropout_seed=0):
    """Stacked, optionally bidirectional forward pass in fp64.

    ``x`` ``[T, B, I]`` (TNC, the layout named in the oneDNN issue's
    packed-sequence question); ``params[l][d]`` as in :func:`cell_forward`;
    ``h0``/``c0`` ``[L*D, B, H]`` or ``None`` (zeros).

    Returns ``(y, hy, cy, cache)``: ``y [T, B, D*H]`` of the top layer,
    ``hy``/``cy`` ``[L*D, B, H]`` (``cy`` is ``None`` unless LSTM) and, if
    ``keep``, the per-step intermediates the backward pass reuses (the MXNet
    page's "reserved workspace"), else ``None``.  ``lengths`` (``[B]`` ints
    in ``[0, T]``, or ``None`` for all ``T``) gives each row's number of
    valid steps (module docstring).  ``dropout`` > 0 makes this a training
    pass with inter-layer dropout of that probability, masks from
    ``dropout_seed`` (module docstring).
    """
    x = np.asarray(x, dtype=np.float64)
    T, B, I = x.shape
    L = len(params)
    D = num_dirs
    H = params[0][0]["w_hh"].shape[1]
    _check_params(mode, params, L, D, I, H)
    if mode != "gru" and gru_variant != "pytorch":
        raise ValueError("gru_variant only applies to mode 'gru'")
    h0 = np.zeros((L * D, B, H)) if h0 is None else np.asarray(h0, np.float64)
    if mode == "lstm":
        c0 = np.zeros((L * D, B, H)) if c0 is None else np.asarray(c0, np.float64)
    hy = np.zeros((L * D, B, H))
    cy = np.zeros((L * D, B, H)) if mode == "lstm" else None
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        assert lengths.shape == (B,) and np.all((lengths >= 0) & (lengths <= T)), lengths
    cache = ({"layer_inputs": [], "steps": {}, "gru_variant": gru_variant, "lengths": lengths,
              "dropout": {}} if keep else None)

    layer_in = x
    for l in range(L):
        if l > 0 and dropout > 0.0:
            m = dropout_multiplier(dropout, dropout_seed, l, layer_in.shape)
            layer_in = layer_in * m
            if keep:
                cache["dropout"][l] = m
        if keep:
            cache["layer_inputs"].append(layer_in)
        y_l = np.zeros((T, B, D * H))
        for d in range(D):
            p = params[l][d]
            h = h0[l * D + d]
            c = c0[l * D + d] if mode == "lstm" else None
            order = range(T) if d == 0 else range(T - 1, -1, -1)
            for t in order:
                h_prev, c_prev = h, c
                h, c, saved = cell_forward(mode, layer_in[t], h_prev, c, p, gru_variant)
                valid = _valid_rows(lengths, t, B)
                if lengths is not None:   # rows past their length keep their state
                    h = np.where(valid, h, h_prev)
                    if mode == "lstm":
                        c = np.where(valid, c, c_prev)
                y_l[t, :, d * H:(d + 1) * H] = np.where(valid, h, 0.0)
                if keep:
                    saved["valid"] = valid
                    saved["h_prev"] = h_prev
                    cache["steps"][(l, d, t)] = saved
            hy[l * D + d] = h
            if mode == "lstm":
                cy[l * D + d] = c
        layer_in = y_l
    return layer_in, hy, cy, cache


def backward(mode, params, cache, dy, dhy=None, dcy=None, num_dirs=1):
    """Backward through time for :func:`forward` (every GRU flavour).

    Gradients of the scalar ``sum(y*dy) + sum(hy*dhy) + sum(cy*dcy)``.
    Returns ``(dx, dh0, dc0, dparams)`` with ``dparams[l][d]`` holding
    ``w_ih, w_hh, b_ih, b_hh`` gradients (overwritten, not accumulated into
    anything the caller passed).

    Per layer from the top down, per direction, walking opposite to that
    direction's forward order, with ``dh = dhy[l*D+d]``, ``dc = dcy[l*D+d]``
    at the start, each step adds ``dY_l[t, :, d*H:(d+1)*H]`` to ``dh`` and
    then:

    * vanilla: ``da = dh * (1 - h^2)``; ``dG_i = dG_h = da``.
    * LSTM: ``tau = tanh(c)``; ``do = dh * tau``;
      ``dc += dh * o * (1 - tau^2)``; ``di = dc * g``; ``dg = dc * i``;
      ``df = dc * c_prev``;
      ``dG = [di*i(1-i), df*f(1-f), dg*(1-g^2), do*o(1-o)] = dG_i = dG_h``;
      the carry becomes ``dc * f``.
    * GRU: ``dn = dh * (1 - z)``; ``dz = dh * (h_prev - n)``;
      ``da_n = dn * (1 - n^2)``; ``da_r = da_n * gh_n * r(1-r)``;
      ``da_z = dz * z(1-z)``; ``dG_i = [da_r, da_z, da_n]``;
      ``dG_h = [da_r, da_z, da_n * r]``; plus the direct term ``dh * z``.
    * GRU, TensorFlow / original-paper flavours (``n`` reads ``(r * h_prev)
      W_hn^T``): ``dn = dh * (1 - z)``, ``dz = dh * (h_prev - n)``, direct
      ``dh * z`` (TensorFlow) or ``dn = dh * z``, ``dz = dh * (n - h_prev)``,
      direct ``dh * (1 - z)`` (paper); ``da_n = dn * (1 - n^2)``;
      ``d_rh = da_n W_hn`` (the gradient of ``r * h_prev``); ``dr = d_rh *
      h_prev``; ``da_r = dr * r(1-r)``; ``da_z = dz * z(1-z)``;
      ``dG_i = dG_h = [da_r, da_z, da_n]``, where the n block of ``W_hh``
      multiplies ``r * h_prev`` (so ``dW_hn = da_n^T (r * h_prev)``) and the
      direct term gains ``d_rh * r``.

    Then ``dh_prev = dG_h W_hh (+ dh*z for GRU)``, ``dX_l[t] += dG_i W_ih``,
    ``dW_ih += dG_i^T x_t``, ``dW_hh += dG_h^T h_prev``,
    ``db_ih += sum_b dG_i``, ``db_hh += sum_b dG_h``.  ``dX_l`` is
    ``dY_{l-1}``; ``dX_0`` is ``dx``.  For the rows of a step past their
    length (the forward's ``lengths``) ``dY`` is ignored, ``dG_i = dG_h = 0``
    and ``dh``, ``dc`` pass through unchanged.
    """
    if cache is None:
        raise ValueError("backward needs the cache of forward(..., keep=True)")
    variant = cache["gru_variant"]
    L = len(params)
    D = num_dirs
    dy = np.asarray(dy, np.float64)
    T, B, _ = dy.shape
    H = params[0][0]["w_hh"].shape[1]
    dhy = np.zeros((L * D, B, H)) if dhy is None else np.asarray(dhy, np.float64)
    if mode == "lstm":
        dcy = np.zeros((L * D, B, H)) if dcy is None else np.asarray(dcy, np.float64)
    dh0 = np.zeros((L * D, B, H))
    dc0 = np.zeros((L * D, B, H)) if mode == "lstm" else None
    dparams = [[None] * D for _ in range(L)]

    dY = dy
    for l in range(L - 1, -1, -1):
        layer_in = cache["layer_inputs"][l]
        dX = np.zeros_like(layer_in)
        for d in range(D):
            p = params[l][d]
            g = {k: np.zeros_like(v) for k, v in p.items()}
            dh = dhy[l * D + d].copy()
            dc = dcy[l * D + d].copy() if mode == "lstm" else None
            # reverse of the forward order of this direction
            order = range(T - 1, -1, -1) if d == 0 else range(T)
            for t in order:
                s = cache["steps"][(l, d, t)]
                h_prev = s["h_prev"]
                valid = s["valid"]
                dh_carried, dc_carried = dh, dc
                dh = dh + np.where(valid, dY[t, :, d * H:(d + 1) * H], 0.0)
                direct = 0.0
                if mode == "rnn_tanh":
                    da = dh * (1.0 - s["h"] ** 2)
                    dG_i = dG_h = da
                elif mode == "lstm":
                    i, f, gg, o, c = s["i"], s["f"], s["g"], s["o"], s["c"]
                    tau = np.tanh(c)
                    d_o = dh * tau
                    dc = dc + dh * o * (1.0 - tau ** 2)
                    d_i = dc * gg
                    d_g = dc * i
                    d_f = dc * s["c_prev"]
                    dG_i = dG_h = np.concatenate(
                        [d_i * i * (1.0 - i), d_f * f * (1.0 - f),
                         d_g * (1.0 - gg ** 2), d_o * o * (1.0 - o)], axis=1)
                    dc = dc * f
                elif variant in ("tf", "paper"):   # gru, n reads (r * h_prev) W_hn^T
                    r, z, n = s["r"], s["z"], s["n"]
                    if variant == "tf":
                        dn, dz, direct = dh * (1.0 - z), dh * (h_prev - n), dh * z
                    else:
                        dn, dz, direct = dh * z, dh * (n - h_prev), dh * (1.0 - z)
                    da_n = dn * (1.0 - n ** 2)
                    w_hn = p["w_hh"][2 * H:]
                    d_rh = da_n @ w_hn
                    da_r = d_rh * h_prev * r * (1.0 - r)
                    da_z = dz * z * (1.0 - z)
                    dG_i = dG_h = np.concatenate([da_r, da_z, da_n], axis=1)
                    direct = direct + d_rh * r
                else:  # gru, PyTorch/cuDNN flavour
                    r, z, n, gh_n = s["r"], s["z"], s["n"], s["gh_n"]
                    dn = dh * (1.0 - z)
                    dz = dh * (h_prev - n)
                    da_n = dn * (1.0 - n ** 2)
                    da_r = da_n * gh_n * r * (1.0 - r)
                    da_z = dz * z * (1.0 - z)
                    dG_i = np.concatenate([da_r, da_z, da_n], axis=1)
                    dG_h = np.concatenate([da_r, da_z, da_n * r], axis=1)
                    direct = dh * z
                if cache["lengths"] is not None:   # rows past their length
                    dG_i = np.where(valid, dG_i, 0.0)
                    dG_h = np.where(valid, dG_h, 0.0)
                    direct = np.where(valid, direct, dh_carried)
                    if mode == "lstm":
                        dc = np.where(valid, dc, dc_carried)
                dX[t] += dG_i @ p["w_ih"]
                g["w_ih"] += dG_i.T @ layer_in[t]
                g["b_ih"] += dG_i.sum(axis=0)
                g["b_hh"] += dG_h.sum(axis=0)
                if mode == "gru" and variant in ("tf", "paper"):
                    g["w_hh"][:2 * H] += dG_h[:, :2 * H].T @ h_prev
                    g["w_hh"][2 * H:] += dG_h[:, 2 * H:].T @ (s["r"] * h_prev)
                    dh = dG_h[:, :2 * H] @ p["w_hh"][:2 * H] + direct
                else:
                    g["w_hh"] += dG_h.T @ h_prev
                    dh = dG_h @ p["w_hh"] + direct
            dh0[l * D + d] = dh
            if mode == "lstm":
                dc0[l * D + d] = dc
            dparams[l][d] = g
        # the gradient of y_{l-1} passes the same dropout multiplier
        dY = dX * cache["dropout"][l] if l in cache["dropout"] else dX
    return dY, dh0, dc0, dparams


def forward_flops(mode, T, B, input_size, hidden, num_layers, num_dirs):
    """GEMM flops of one forward pass, ``2*M*N*K`` per product:
    ``sum_{l,d} 2*T*B*G*H*(I_l + H)``.  Pointwise work is not counted (the
    GFLOPS column of the cuDNN-5 optimisation table in Keras issue #3692
    gives no definition; this is the plain GEMM count)."""
    G = GATES[mode]
    tot = 0
    for l in range(num_layers):
        I_l = input_size if l == 0 else num_dirs * hidden
        tot += num_dirs * 2 * T * B * G * hidden * (I_l + hidden)
    return tot


def train_step_flops(mode, T, B, input_size, hidden, num_layers, num_dirs):
    """Forward + backward-data (dX at every layer, dh recurrence) +
    backward-weights (dW_ih, dW_hh): three times the forward count."""
    return 3 * forward_flops(mode, T, B, input_size, hidden, num_layers, num_dirs)
