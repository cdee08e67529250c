"""Brute-force KL in mpmath for tiny inputs (test infrastructure only).

An implementation of the distillation loss written independently of
``kd_oracle``: plain Python loops over positions, vocabulary, hidden size and
the K cached entries, evaluated with 50-digit mpmath arithmetic and no
max-shift tricks.  It follows the quantity itself -- for each unmasked position
the KL divergence of the renormalised top-K teacher distribution from the
student distribution at the same K token ids, summed over positions -- not the
rearranged ``negent - sum p z + s lse`` form the oracle uses.

With a temperature ``tau`` the teacher and student distributions are
softmaxes of ``a / tau`` and ``z / tau`` and the sum is multiplied by
``tau^2`` (the usual temperature-scaled distillation loss; the aihot.vn page,
section "Mô hình học sinh thu được", reports loss-choice ablations without
defining any); ``tau = 1`` is the plain loss.

Gradients come from central differences of that loss at 50 digits, so they pin
the closed-form gradient without using it (the pages only say a closed form
exists: aihot.vn page "Tối ưu hóa chi phí chưng cất tri thức…", section
"Mô hình học sinh thu được").
"""
from __future__ import annotations

import mpmath

DPS = 50


def _mp(x):
    return mpmath.mpf(float(x))


def loss(H, W, ids, logits, mask=None, tau=1):
    """Return ``(L, lse_list, row_loss_list)`` as mpmath numbers (``lse`` of
    ``z / tau``).

    ``H [n][d]``, ``W [v][d]``, ``ids [n][K]``, ``logits [n][K]`` are nested
    sequences of floats/ints (exact values), ``mask`` a sequence of 0/1 or None."""
    with mpmath.workdps(DPS):
        t = _mp(tau)
        n, d, v = len(H), len(H[0]), len(W)
        Hm = [[_mp(x) for x in row] for row in H]
        Wm = [[_mp(x) for x in row] for row in W]
        total = mpmath.mpf(0)
        lses, rls = [], []
        for i in range(n):
            z = []
            for j in range(v):
                acc = mpmath.mpf(0)
                for c in range(d):
                    acc += Hm[i][c] * Wm[j][c]
                z.append(acc / t)
            partition = mpmath.fsum(mpmath.exp(zj) for zj in z)
            lses.append(mpmath.log(partition))
            if mask is not None and not mask[i]:
                rls.append(mpmath.mpf(0))
                continue
            a = [_mp(x) / t for x in logits[i]]
            za = mpmath.fsum(mpmath.exp(x) for x in a)
            row = mpmath.mpf(0)
            for kk in range(len(a)):
                p = mpmath.exp(a[kk]) / za
                q = mpmath.exp(_z_at(z, ids[i][kk])) / partition
                if p != 0:
                    row += p * mpmath.log(p / q)
            row *= t * t
            rls.append(row)
            total += row
        return total, lses, rls


def grad_fd(H, W, ids, logits, mask=None, g=1.0, step="1e-20", tau=1):
    """Central-difference gradient of ``g * L`` w.r.t. every entry of H and W.

    Returns ``(dH, dW)`` as nested lists of mpmath numbers."""
    with mpmath.workdps(DPS):
        h = mpmath.mpf(step)
        gm = _mp(g)
        Hm = [[_mp(x) for x in row] for row in H]
        Wm = [[_mp(x) for x in row] for row in W]

        def L(Hx, Wx):
            with mpmath.workdps(DPS):
                return _loss_mp(Hx, Wx, ids, logits, mask, _mp(tau))

        dH = [[None] * len(Hm[0]) for _ in Hm]
        for i in range(len(Hm)):
            for c in range(len(Hm[0])):
                old = Hm[i][c]
                Hm[i][c] = old + h
                up = L(Hm, Wm)
                Hm[i][c] = old - h
                dn = L(Hm, Wm)
                Hm[i][c] = old
                dH[i][c] = gm * (up - dn) / (2 * h)
        dW = [[None] * len(Wm[0]) for _ in Wm]
        for j in range(len(Wm)):
            for c in range(len(Wm[0])):
                old = Wm[j][c]
                Wm[j][c] = old + h
                up = L(Hm, Wm)
                Wm[j][c] = old - h
                dn = L(Hm, Wm)
                Wm[j][c] = old
                dW[j][c] = gm * (up - dn) / (2 * h)
        return dH, dW


def _loss_mp(Hm, Wm, ids, logits, mask, t):
    """Same sum as ``loss`` on mpmath matrices (no widening)."""
    total = mpmath.mpf(0)
    for i in range(len(Hm)):
        if mask is not None and not mask[i]:
            continue
        z = [mpmath.fsum(Hm[i][c] * Wm[j][c] for c in range(len(Hm[i]))) / t for j in range(len(Wm))]
        partition = mpmath.fsum(mpmath.exp(zj) for zj in z)
        a = [_mp(x) / t for x in logits[i]]
        za = mpmath.fsum(mpmath.exp(x) for x in a)
        for kk in range(len(a)):
            p = mpmath.exp(a[kk]) / za
            q = mpmath.exp(_z_at(z, ids[i][kk])) / partition
            if p != 0:
                total += p * mpmath.log(p / q)
    return total * t * t


def _z_at(z, idx):
    """The (tempered) student logit of token ``idx``; an id outside the
    vocabulary matches no entry and its logit is taken as 0 (the reading for
    records that break the cache's contract)."""
    j = int(idx)
    return z[j] if 0 <= j < len(z) else mpmath.mpf(0)
