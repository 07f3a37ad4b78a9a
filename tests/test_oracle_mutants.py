"""Plant plausible mistakes in a copy of the oracle and check the pins catch
each one.  The copy is built from oracle/attention.py's source with one
textual change and executed as a throwaway module; the real oracle is never
modified.  Everything runs on the CPU.
"""

import importlib.util
import math
import os
import types

import numpy as np
import pytest

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "attention.py")

MUTANTS = {
    "causal_off_by_one": ("return j > np.asarray(row_idx)[:, None]",
                          "return j >= np.asarray(row_idx)[:, None]"),
    "causal_mask_transposed": ("return j > np.asarray(row_idx)[:, None]",
                               "return j < np.asarray(row_idx)[:, None]"),
    "scale_dropped": ("s = scale * (q[r] @ k.T)", "s = (q[r] @ k.T)"),
    "no_max_subtraction": ("e = np.exp(s - m_safe[:, None])                # exp(s - m); masked -> 0",
                           "e = np.exp(s)"),
    "lse_without_max": ("lse[c0:c0 + r.shape[0]][live] = m[live] + np.log(l[live])",
                        "lse[c0:c0 + r.shape[0]][live] = np.log(l[live])"),
    "lse_log2": ("lse[c0:c0 + r.shape[0]][live] = m[live] + np.log(l[live])",
                 "lse[c0:c0 + r.shape[0]][live] = m[live] + np.log2(l[live])"),
    "unnormalised": ("p[live] = e[live] / l[live, None]              # softmax weights",
                     "p[live] = e[live]"),
    "bwd_dv_not_transposed": ("dv = p.T @ do", "dv = p @ do"),
    "bwd_delta_sign": ("ds = p * (dp - D[:, None])", "ds = p * (dp + D[:, None])"),
    "bwd_delta_dropped": ("ds = p * (dp - D[:, None])", "ds = p * dp"),
    "bwd_dq_scale_dropped": ("dq = scale * (ds @ k)", "dq = (ds @ k)"),
    "bwd_dk_uses_k": ("dk = scale * (ds.T @ q)", "dk = scale * (ds.T @ k)"),
    "bwd_dp_wrong_operand": ("dp = do @ v.T", "dp = do @ q.T"),
    "bwd_mask_dropped": ("        s[_causal_mask(np.arange(n_q), n_k)] = -np.inf",
                         "        pass"),
    "block_mask_transposed": ("    return ~bm[qb][:, kb]", "    return ~bm.T[qb][:, kb]"),
    "block_rows_use_key_block_size": ("    qb = np.asarray(row_idx) // bq", "    qb = np.asarray(row_idx) // bk"),
    "decode_offset_dropped": ("causal=causal, causal_offset=n_k - n_q)", "causal=causal, causal_offset=0)"),
    "decode_offset_sign": ("causal=causal, causal_offset=n_k - n_q)", "causal=causal, causal_offset=n_q - n_k)"),
    "bwd_block_mask_dropped": ("        s[_block_masked(np.arange(n_q), n_k, block_mask, block)] = -np.inf",
                               "        pass"),
}


def _load_mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _load_real():
    spec = importlib.util.spec_from_file_location("oracle_real_copy", SRC)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _brute(q, k, v, scale, causal):
    out, lses = [], []
    for i in range(len(q)):
        sc = [(j, scale * sum(a * b for a, b in zip(q[i], k[j])))
              for j in range(len(k)) if not (causal and j > i)]
        m = max(s for _, s in sc)
        tot = sum(math.exp(s - m) for _, s in sc)
        out.append([sum(math.exp(s - m) / tot * v[j][c] for j, s in sc)
                    for c in range(len(v[0]))])
        lses.append(m + math.log(tot))
    return np.array(out), np.array(lses)


def _battery(mod):
    """Return the list of pin checks that fail for module `mod`."""
    failed = []
    rng = np.random.default_rng(5)
    # Brute force, both mask modes.
    for causal in (False, True):
        q, k, v = (rng.standard_normal((6, 3)) for _ in range(3))
        try:
            o, lse = mod.attention_forward_head(q, k, v, scale=0.6, causal=causal)
            bo, bl = _brute(q.tolist(), k.tolist(), v.tolist(), 0.6, causal)
            if not (np.allclose(o, bo, atol=1e-12) and np.allclose(lse, bl, atol=1e-12)):
                failed.append(f"brute_{causal}")
        except Exception:
            failed.append(f"brute_{causal}_raised")
    # Worked example through the embedding.
    s = np.array([2.0, 1.0, 3.0, 0.0])
    q = np.zeros((4, 4)); q[0, 0] = 1
    k = np.zeros((4, 4)); k[:, 0] = s
    o, lse = mod.attention_forward_head(q, k, np.eye(4), scale=1.0)
    if not (np.allclose(o[0], [0.2369, 0.0871, 0.6439, 0.0321], atol=5e-5)
            and abs(lse[0] - (3 + math.log(1.5530))) < 1e-4):
        failed.append("worked_example")
    # Key shift with a large offset.
    q, k, v = (rng.standard_normal((8, 4)) for _ in range(3))
    c = rng.standard_normal(4) * 400
    with np.errstate(all="ignore"):
        o1, l1 = mod.attention_forward_head(q, k, v)
        o2, l2 = mod.attention_forward_head(q, k + c, v)
    if not (np.all(np.isfinite(o2)) and np.allclose(o1, o2, atol=1e-10)
            and np.allclose(l2 - l1, q @ c / 2.0, atol=1e-8)):
        failed.append("key_shift")
    # Backward against torch autograd.
    for causal in (False, True):
        q, k, v, do = (rng.standard_normal((7, 4)) for _ in range(4))
        dq, dk, dv, _ = mod.attention_backward_head(q, k, v, do, scale=0.7, causal=causal)
        tq, tk, tv = (torch.from_numpy(x[None, None]).requires_grad_() for x in (q, k, v))
        to = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, is_causal=causal, scale=0.7)
        to.backward(torch.from_numpy(do[None, None]))
        if not (np.allclose(dq, tq.grad[0, 0].numpy(), atol=1e-12)
                and np.allclose(dk, tk.grad[0, 0].numpy(), atol=1e-12)
                and np.allclose(dv, tv.grad[0, 0].numpy(), atol=1e-12)):
            failed.append(f"autograd_{causal}")
    # Block mask (non-square blocks, non-symmetric mask): forward against
    # scalar loops, backward against torch autograd with the element mask.
    n, bq, bk = 9, 2, 3
    mask = np.array([[1, 0, 1], [0, 1, 0], [1, 1, 0], [0, 0, 1], [1, 0, 0]], dtype=np.uint8)
    allowed = mask[np.arange(n)[:, None] // bq, np.arange(n)[None, :] // bk] != 0
    q, k, v, do = (rng.standard_normal((n, 3)) for _ in range(4))
    try:
        o, lse = mod.attention_forward_head(q, k, v, scale=0.6, block_mask=mask, block=(bq, bk))
        bo = np.zeros((n, 3)); bl = np.zeros(n)
        for i in range(n):
            js = [j for j in range(n) if allowed[i, j]]
            sc = [0.6 * sum(a * b for a, b in zip(q[i], k[j])) for j in js]
            m = max(sc); tot = sum(math.exp(x - m) for x in sc)
            bo[i] = sum(math.exp(x - m) / tot * v[j] for x, j in zip(sc, js))
            bl[i] = m + math.log(tot)
        if not (np.allclose(o, bo, atol=1e-12) and np.allclose(lse, bl, atol=1e-12)):
            failed.append("block_brute")
        dq, dk, dv, _ = mod.attention_backward_head(q, k, v, do, scale=0.6, block_mask=mask, block=(bq, bk))
        tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
        to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(allowed),
                                                              scale=0.6)
        to.backward(torch.from_numpy(do))
        if not (np.allclose(dq, tq.grad.numpy(), atol=1e-12) and np.allclose(dk, tk.grad.numpy(), atol=1e-12)
                and np.allclose(dv, tv.grad.numpy(), atol=1e-12)):
            failed.append("block_autograd")
    except Exception:
        failed.append("block_raised")
    # Decoding: the last queries against the whole cache equal the last rows
    # of the full causal attention (scalar loops).
    nq, nk = 3, 8
    q, k, v = (rng.standard_normal((nk, 3)) for _ in range(3))
    o, lse = mod.attention_decode_head(q[nk - nq:], k, v, scale=0.6, causal=True)
    bo, bl = _brute(q.tolist(), k.tolist(), v.tolist(), 0.6, True)
    if not (np.allclose(o, bo[nk - nq:], atol=1e-12) and np.allclose(lse, bl[nk - nq:], atol=1e-12)):
        failed.append("decode_brute")
    return failed


def test_real_oracle_passes_battery():
    assert _battery(_load_real()) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    failed = _battery(_load_mutant(old, new))
    assert failed, f"mutant {name} passed every pin"
