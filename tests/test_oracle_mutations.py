"""Plants plausible mistakes in a copy of the oracle (on the CPU) and requires
that at least one pin catches each of them.  A mistake no pin catches would
mean the oracle is not pinned against it."""
import sys
import types

import pytest

import oracle.dflash_oracle as O
import oracle_pins as P

MUTATIONS = {
    "rope sign": ("x1 * cos - x2 * sin, x2 * cos + x1 * sin", "x1 * cos + x2 * sin, x2 * cos - x1 * sin"),
    "rope pairing interleaved": ("x1, x2 = x[..., :half], x[..., half:]", "x1, x2 = x[..., 0::2], x[..., 1::2]"),
    "rope frequency": ("inv_freq = float(theta) ** (-2.0 * i / d)", "inv_freq = float(theta) ** (-1.0 * i / d)"),
    "attention no scale": ("/ np.sqrt(d)          # [Bq, T]", "/ 1.0"),
    "attention gqa modulo": ("g = h // group", "g = h % nkv"),
    "softmax over queries": ("s = s - s.max(axis=1, keepdims=True)\n        p = np.exp(s)\n        p = p / p.sum(axis=1, keepdims=True)",
                             "s = s - s.max(axis=0, keepdims=True)\n        p = np.exp(s)\n        p = p / p.sum(axis=0, keepdims=True)"),
    "rmsnorm eps outside": ("return x / np.sqrt(ms + eps) *", "return x / (np.sqrt(ms) + eps) *"),
    "rmsnorm sum not mean": ("ms = np.mean(x * x, axis=-1, keepdims=True)", "ms = np.sum(x * x, axis=-1, keepdims=True)"),
    "rmsnorm no gain": ("* np.asarray(gain, dtype=np.float64)", "* 1.0"),
    "silu sign": ("return x / (1.0 + np.exp(-x))", "return x / (1.0 + np.exp(x))"),
    "argmax last on ties": ("idx = np.argmax(logits, axis=-1)", "idx = logits.shape[-1] - 1 - np.argmax(logits[..., ::-1], axis=-1)"),
    "accept counts all matches": ("while n < B and draft[s, n] == tgt[s, n]:\n            n += 1",
                                  "n = int(np.sum(draft[s] == tgt[s, :B]))"),
    "bonus from last row": ("bonus[s] = tgt[s, n]", "bonus[s] = tgt[s, B]"),
    "linear reversed rows": ("out[..., r0:r0 + wc.shape[0]] = x @ wc.T", "out[..., r0:r0 + wc.shape[0]] = x @ wc[::-1].T"),
    "inject no rope": ("k = rope(k, pos, dims.rope_theta)", "pass"),
    "inject no norm": ("c = rms_norm(u, _get(weights, \"fc_norm\"), dims.rms_eps)", "c = u"),
    "inject v from k weights": ("v = linear(c, lw[\"wv\"]).reshape(n, nkv, d)", "v = linear(c, lw[\"wk\"]).reshape(n, nkv, d)"),
    "draft ignores block keys": ("keys = np.concatenate([cache.k[l, s, :, :C, :].transpose(1, 0, 2), ks], axis=0)\n            vals = np.concatenate([cache.v[l, s, :, :C, :].transpose(1, 0, 2), v[s]], axis=0)",
                                 "keys = cache.k[l, s, :, :C, :].transpose(1, 0, 2) if C else ks\n            vals = cache.v[l, s, :, :C, :].transpose(1, 0, 2) if C else v[s]"),
    "draft layer-0 cache everywhere": ("cache.k[l, s, :, :C, :]", "cache.k[0, s, :, :C, :]"),
    "draft block positions from 0": ("pos = np.arange(C, C + B) + pos_offset", "pos = np.arange(0, B) + pos_offset"),
    "draft no attention residual": ("h = h + linear(o, lw[\"wo\"])", "h = linear(o, lw[\"wo\"])"),
    "draft mlp gate/up swapped": ("act = silu(linear(a, lw[\"w_gate\"])) * linear(a, lw[\"w_up\"])",
                                  "act = silu(linear(a, lw[\"w_up\"])) * linear(a, lw[\"w_gate\"])"),
    "draft no final norm": ("z = rms_norm(h, _get(weights, \"final_norm\"), dims.rms_eps)", "z = h"),
    "anchor sees the whole context": ("np.array([p], dtype=np.int64))", "cache.length[s:s + 1].copy())"),
    "anchor one position late": ("view = OracleCache(cache.k[:, s:s + 1], cache.v[:, s:s + 1], np.array([p], dtype=np.int64))",
                                 "view = OracleCache(cache.k[:, s:s + 1], cache.v[:, s:s + 1], np.array([p + 1], dtype=np.int64))"),
    "gumbel sign": ("return -np.log(-np.log(u))", "return np.log(-np.log(u))"),
    "draft sample ignores temperature": ('tok, gaps = sample_categorical(dr["logits"] / float(temperature), u)',
                                         'tok, gaps = sample_categorical(dr["logits"], u)'),
    "accept ratio inverted": ("diff = (lp[j, d] - lq[j, d]) - np.log(float(u_accept[s, j]))",
                              "diff = (lq[j, d] - lp[j, d]) - np.log(float(u_accept[s, j]))"),
    "residual q minus p": ("w = np.maximum(0.0, np.exp(lp[j]) - np.exp(lq[j]))",
                           "w = np.maximum(0.0, np.exp(lq[j]) - np.exp(lp[j]))"),
    "residual without clipping": ("w = np.maximum(0.0, np.exp(lp[j]) - np.exp(lq[j]))", "w = np.exp(lp[j])"),
    "bonus from the last drafted row": ("logw = lp[B]", "logw = lp[B - 1]"),
    "target not causal": ("T = C + i + 1", "T = C + n"),
    "target sees one key ahead": ("T = C + i + 1", "T = min(C + i + 2, C + n)"),
    "target positions from 0": ("            pos = np.arange(C, C + n)\n            if parents is not None:",
                                "            pos = np.arange(0, n)\n            if parents is not None:"),
    "commit without the next token": ("cache.length += np.asarray(accept_len, dtype=np.int64) + 1",
                                      "cache.length += np.asarray(accept_len, dtype=np.int64)"),
    "features one layer late": ("feats = [resid[l] for l in feat_layers]",
                                "feats = [resid[min(l + 1, len(resid) - 1)] for l in feat_layers]"),
    "tree sibling not pushed": ("        if rk[-1] + 1 < K:                          # next sibling",
                                "        if False:                                   # next sibling"),
    "tree positions in slot order": ("                pos = C + depth", "                pos = C + np.arange(n)"),
    "tree mask without ancestors": ("            j = int(parent[j])", "            j = -1"),
    "tree accept follows the last match": ("        node = kids[0]", "        node = kids[-1]"),
    "tree commit keeps slot order": ("    rows = C + np.asarray(path, dtype=np.int64)", "    rows = C + np.arange(len(path))"),
    "inject wrong slot": ("cache.k[l, s, :, start:start + n, :] = k.transpose(1, 0, 2)",
                          "cache.k[l, s, :, start + 1:start + n + 1, :] = k.transpose(1, 0, 2)"),
}


def _mutant(old, new, tag):
    src = open(O.__file__).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    name = f"_oracle_mutant_{tag}"
    mod = types.ModuleType(name)
    mod.__file__ = O.__file__
    sys.modules[name] = mod
    try:
        exec(compile(src.replace(old, new), name, "exec"), mod.__dict__)
    except Exception:
        del sys.modules[name]
        raise
    return mod


@pytest.mark.parametrize("tag", sorted(MUTATIONS))
def test_planted_mistake_is_caught(tag, monkeypatch):
    old, new = MUTATIONS[tag]
    mod = _mutant(old, new, tag.replace(" ", "_").replace("/", "_").replace("-", "_"))
    monkeypatch.setattr(P, "O", mod)
    caught = []
    for check in P.ALL_CHECKS:
        try:
            check()
        except Exception as exc:  # AssertionError or a shape error: either way caught
            caught.append(check.__name__)
            break                 # one catching pin is enough
    assert caught, f"no pin catches the planted mistake '{tag}'"
