"""The oracle's pins must catch plausible mistakes (CPU).

Each case plants one mistake in a scratch copy of oracle/gdn_oracle.c (a dropped term, a wrong
sign or index, a transposed operand, a decay at the wrong place), builds that copy, and runs
the pin tests against it in a fresh process (GDN_ORACLE_SRC selects the copy).  The pins pass
on the real oracle (the rest of the suite), so a failing run here is the planted mistake being
caught.  A mistake that no pin caught would show as a passing run, and the case fails.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")

PINS_GDN = "tests/test_oracle_pins.py"
PINS_CAM = "tests/test_oracle_cam.py"
PINS_DHU = "tests/test_oracle_dhu.py"
PINS_CBWD = "tests/test_oracle_cam_bwd.py"
PINS_BBWD = "tests/test_oracle_bigdn_bwd.py"
PINS_PREPBWD = "tests/test_oracle_prep_bwd.py"
PINS_CPBWD = "tests/test_oracle_cam_prep_bwd.py"

# (name, pin file, text in gdn_oracle.c, replacement)
MUTATIONS = [
    ("missing beta", PINS_GDN, "d[c] = bt * (vt[c] - d[c]);", "d[c] = (vt[c] - d[c]);"),
    ("per-key gate sign", PINS_GDN, "if (gk) lam += gk[(long)t * sqk + r];",
     "if (gk) lam -= gk[(long)t * sqk + r];"),
    ("transposed read-out", PINS_GDN, "ot[c] += S[(size_t)r * V + c] * qt[r];",
     "ot[c] += S[(size_t)(c % K) * V + (r % V)] * qt[r];"),
    ("saved state after the decay", PINS_GDN,
     "    if (hch && (t % C) == 0)  /* state entering chunk t/C, before this token's decay */\n"
     "      memcpy(hch + (size_t)(t / C) * K * V, S, sizeof(double) * (size_t)K * V);", ""),
    ("k_scale on q", PINS_GDN, "qx = qx > 0.0 ? qx : 0.0;", "qx = (qx > 0.0 ? qx : 0.0) * k_scale;"),
    ("reverse decay index", PINS_GDN, "const double dcy = decay[(long)bh * F + fa];",
     "const double dcy = decay[(long)bh * F + f];"),
    ("transition: decay on columns", PINS_GDN,
     "      for (int c = 0; c < K; ++c) M[(size_t)r * K + c] *= a[r];",
     "      for (int c = 0; c < K; ++c) M[(size_t)r * K + c] *= a[c];"),
    ("transition: transposed rank-one update", PINS_GDN,
     "      for (int c = 0; c < K; ++c) M[(size_t)r * K + c] -= bt * kt[r] * w[c];",
     "      for (int c = 0; c < K; ++c) M[(size_t)r * K + c] -= bt * kt[c] * w[r];"),
    ("camera: transposed 4x4 matrix", PINS_CAM,
     "for (int j = 0; j < 4; ++j) acc += P[which][i * 4 + j] * xn[4 * g + j];",
     "for (int j = 0; j < 4; ++j) acc += P[which][j * 4 + i] * xn[4 * g + j];"),
    ("camera: RoPE without the pair swap", PINS_CAM,
     "y[Dh + r] = xn[Dh + r] * cosv[n * Dh + r] + xn[Dh + (r ^ 1)] * sinv[n * Dh + r];",
     "y[Dh + r] = xn[Dh + r] * cosv[n * Dh + r] + xn[Dh + r] * sinv[n * Dh + r];"),
    ("dhu: no decay on dv2's state term", PINS_DHU,
     "s += k[tk * K + r] * exp(gl[r] - gam[(size_t)i * K + r]) * dh[(size_t)r * V + c];",
     "s += k[tk * K + r] * dh[(size_t)r * V + c];"),
    ("dhu: sign of the w term", PINS_DHU,
     "dh[(size_t)r * V + c] += qr * do_[tk * V + c] - wr * dv2[tk * V + c];",
     "dh[(size_t)r * V + c] += qr * do_[tk * V + c] + wr * dv2[tk * V + c];"),
    ("backward inputs: w without beta", PINS_DHU,
     "w[TOK(r) * K + d] = br * exp(gam[(size_t)r * K + d]) * k[TOK(r) * K + d];",
     "w[TOK(r) * K + d] = exp(gam[(size_t)r * K + d]) * k[TOK(r) * K + d];"),
    ("backward inputs: P without its diagonal", PINS_DHU,
     "            for (int s = 0; s <= r; ++s) {\n              double p = 0.0;",
     "            for (int s = 0; s < r; ++s) {\n              double p = 0.0;"),
    ("BiGDN backward: dk_pos without the prediction term", PINS_BBWD,
     "dk_pos[base + t * D + r] = a[r] * bt * e1 - bt * ee * zp[r];",
     "dk_pos[base + t * D + r] = a[r] * bt * e1;"),
    ("BiGDN backward: dbeta without the z stream", PINS_BBWD,
     "dbeta[(long)bh * N + t] = db + ee * e1;", "dbeta[(long)bh * N + t] = db;"),
    ("BiGDN backward: decay gradient without the z stream's term", PINS_BBWD,
     "for (int r = 0; r < D; ++r) gd += dzp[r] * zs[(size_t)(it - 1) * D + r];", ";"),
    ("BiGDN backward: z gradient carried back without the decay", PINS_BBWD,
     "for (int r = 0; r < D; ++r) a[r] = g * dzp[r];", "for (int r = 0; r < D; ++r) a[r] = dzp[r];"),
    ("front-end backward: RoPE inverse with the token's own sine", PINS_PREPBWD,
     "drot[o + pd] * sinv[n * D + pd];", "drot[o + pd] * sinv[n * D + dd];"),
    ("front-end backward: RMSNorm without its correction term", PINS_PREPBWD,
     "out[which * C + c] = r * w[c] * g[which * C + c] - r * r * r / (double)C * x[c] * s;",
     "out[which * C + c] = r * w[c] * g[which * C + c];"),
    ("front-end backward: k without its scale", PINS_PREPBWD,
     "g[which * C + c] = xhat > 0.0 ? gp * (which ? k_scale : 1.0) : 0.0;",
     "g[which * C + c] = xhat > 0.0 ? gp : 0.0;"),
    ("merge backward: dden with one factor of 1 / (den + eps)", PINS_PREPBWD,
     "dden[(b * H + h) * N + n] = -acc * inv * inv;", "dden[(b * H + h) * N + n] = -acc * inv;"),
    ("camera prep backward: RoPE transpose with the token's own sine", PINS_CPBWD,
     "dy[Dh + (r ^ 1)] * sinv[n * Dh + (r ^ 1)];", "dy[Dh + (r ^ 1)] * sinv[n * Dh + r];"),
    ("camera prep backward: 4x4 block not transposed", PINS_CPBWD,
     "for (int i = 0; i < 4; ++i) acc += P[which][i * 4 + j] * dy[4 * gi + i];",
     "for (int i = 0; i < 4; ++i) acc += P[which][j * 4 + i] * dy[4 * gi + i];"),
    ("camera prep backward: inflation without its pre-norm term", PINS_CPBWD,
     "if (which == 1) gv = (gv + 2.0 * xn[1][d] * d_pre) * k_scale;",
     "if (which == 1) gv = gv * k_scale;"),
    ("camera prep backward: inflation's output term with one factor of y", PINS_CPBWD,
     "if (which == 1) dy[d] += 2.0 * y[d] * d_post;", "if (which == 1) dy[d] += 2.0 * d_post;"),
    ("camera backward: dv without beta", PINS_CBWD,
     "dv[base + (long)c * N + t] = bt * dd[c];", "dv[base + (long)c * N + t] = dd[c];"),
    ("camera backward: dk without the prediction term", PINS_CBWD,
     "acc += dS[(size_t)r * D + c] * d_[c] - sp[(size_t)r * D + c] * bt * dd[c];",
     "acc += dS[(size_t)r * D + c] * d_[c];"),
    ("camera backward: decay gradient against the decayed state", PINS_CBWD,
     "            const double* prev = St + (size_t)(it - 1) * DD;",
     "            const double* prev = Sp + (size_t)it * DD;"),
]


def _run_pins(src_path, pins):
    env = dict(os.environ, GDN_ORACLE_SRC=src_path, OMP_NUM_THREADS="4")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
           "-m", "not gpu", os.path.join(ROOT, pins)]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


@pytest.mark.parametrize("name,pins,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(tmp_path, name, pins, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation anchor of %r is not unique in gdn_oracle.c" % name
    dst = tmp_path / "gdn_oracle.c"
    dst.write_text(text.replace(old, new))
    res = _run_pins(str(dst), pins)
    assert res.returncode != 0, "no pin in %s caught the planted mistake %r:\n%s" % (
        pins, name, res.stdout[-2000:])


def test_unmutated_copy_passes(tmp_path):
    """Control: the same procedure on an unchanged copy passes every pin file."""
    dst = tmp_path / "gdn_oracle.c"
    shutil.copy(SRC, dst)
    for pins in (PINS_GDN, PINS_CAM, PINS_DHU, PINS_CBWD):
        res = _run_pins(str(dst), pins)
        assert res.returncode == 0, res.stdout[-2000:]
