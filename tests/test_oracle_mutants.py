"""Plant plausible mistakes in copies of the oracle; the pins must catch each one.

The mutants are made on the CPU from the oracle's source text; the real
oracle is untouched.  A mutant counts as caught when at least one pin fails
(an assertion or any other error).
"""

import os
import types

import pytest

import pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")

MUTANTS = {
    "scale dropped": ("                    s = scale * (qq @ kk[lo:hi].T)",
                      "                    s = (qq @ kk[lo:hi].T)"),
    "v used as k": ("                    s = scale * (qq @ kk[lo:hi].T)",
                    "                    s = scale * (qq @ vv[lo:hi].T)"),
    "split scale dropped": ("        s = scale * (qq @ kk[lo:hi].T)\n        m = s.max",
                            "        s = (qq @ kk[lo:hi].T)\n        m = s.max"),
    "causal direction flipped": ("vis &= j <= c", "vis &= j >= c"),
    "window exclusive": ("vis &= np.abs(c - j) <= window", "vis &= np.abs(c - j) < window"),
    "window one-sided": ("vis &= np.abs(c - j) <= window", "vis &= (c - j) <= window"),
    "causal top-left": ("\n    c = i + (Sk - Sq)\n", "\n    c = i\n"),
    "gqa by modulo": ("for h in range(g * G, (g + 1) * G):", "for h in range(g, Hq, Hkv):"),
    "query head from kv index": ("qq = _f64(q[b, h, rr])", "qq = _f64(q[b, g, rr])"),
    "lse misses max": ("lse = np.where(live, m_safe + np.log(", "lse = np.where(live, np.log("),
    "lse in log2": ("m_safe + np.log(np.where(live, l, 1.0)), NEG_INF)",
                    "m_safe + np.log2(np.where(live, l, 1.0)), NEG_INF)"),
    "no normalisation": ("o = np.where(live[:, None], o / np.where(live, l, 1.0)[:, None], 0.0)",
                         "o = np.where(live[:, None], o, 0.0)"),
    "exp sign": ("e = np.exp(s - m_safe[:, None])", "e = np.exp(m_safe[:, None] - s)"),
    "merge drops a factor": ("return M, l1 * f1 + l2 * f2,", "return M, l1 * f1 + l2,"),
    "merge max->min": ("M = np.maximum(m1, m2)", "M = np.minimum(m1, m2)"),
    "chunk length floored": ("    L = -(-Sk // num_splits)\n", "    L = Sk // num_splits if Sk >= num_splits else 1\n"),
    "chunk bound off by one": ("min((c + 1) * L, Sk)) for c in range(num_splits)]",
                               "min((c + 1) * L - 1, Sk)) for c in range(num_splits)]"),
    "online alpha inverted": ("alpha = np.where(np.isfinite(m), np.exp(m - m_ref), 0.0)",
                              "alpha = np.where(np.isfinite(m), np.exp(m_ref - m), 0.0)"),
    "online keeps stale max": ("                m = m_new\n", "                m = np.maximum(m, 0.0)\n"),
    "finish misses max": ("lse = np.where(live, m + np.log(np.where(live, l, 1.0)), NEG_INF)",
                          "lse = np.where(live, np.log(np.where(live, l, 1.0)), NEG_INF)"),
    "balanced tree drops odd leaf": ("            if len(parts) % 2:\n                nxt.append(parts[-1])\n",
                                     "            pass\n"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name!r} not unique/absent"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(name)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 -- any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
            break
    assert caught, f"no pin caught the mutant {name!r}"
