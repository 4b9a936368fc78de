"""Planted mistakes in the oracle must each fail one of its pins (CPU only).

Each case swaps one oracle function for a copy with one plausible mistake (a
dropped term, a wrong sign, index or operand, a missing temperature, a wrong
rounding step, too short a candidate list) and runs the pins that guard it;
at least one of them has to fail.  The real oracle is restored after each case
(``monkeypatch``), and nothing here is used by the library or the GPU tests.
"""
import numpy as np
import pytest

from oracle import pkm_oracle as O
from tests import test_oracle_pins as pins


# ---------------------------------------------------------------------------
# mutated copies of oracle functions
# ---------------------------------------------------------------------------
def bn_backward_dropped_xhat_term(dq, xhat, gamma, var, eps):
    dbeta = dq.sum(axis=0)
    dgamma = (dq * xhat).sum(axis=0)
    dq_pre = gamma / np.sqrt(var + eps) * (dq - dq.mean(axis=0))
    return dq_pre, dgamma, dbeta


def bn_forward_unbiased(q_pre, gamma, beta, eps):
    mean = q_pre.mean(axis=0)
    var = ((q_pre - mean) ** 2).sum(axis=0) / max(1, q_pre.shape[0] - 1)
    xhat = (q_pre - mean) / np.sqrt(var + eps)
    return gamma * xhat + beta, mean, var, xhat


def softmax_backward_sign(w, dw, tau):
    return w * ((w * dw).sum(axis=-1, keepdims=True) - dw) / tau


def softmax_backward_times_tau(w, dw, tau):
    return w * (dw - (w * dw).sum(axis=-1, keepdims=True)) * tau


def softmax_backward_no_tau(w, dw, tau):
    return w * (dw - (w * dw).sum(axis=-1, keepdims=True))


def softmax_no_tau(s, tau):
    z = s - s.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def split_heads_swapped(q, heads, dq):
    T = q.shape[0]
    qh = q.reshape(T, heads, dq)
    return qh[:, :, dq // 2:], qh[:, :, : dq // 2]


def project_transposed(x, Wq):
    return x @ Wq


def candidates_wrong_row(i1, v1, i2, v2, n_keys2):
    # the second half taken as the major index
    sc = v1[..., :, None] + v2[..., None, :]
    rows = i2[..., None, :].astype(np.int64) * n_keys2 + i1[..., :, None].astype(np.int64)
    shp = sc.shape[:-2] + (sc.shape[-2] * sc.shape[-1],)
    return sc.reshape(shp), rows.reshape(shp)


def topk_highest_index_first(s, k):
    n = s.shape[-1]
    order = (n - 1 - np.argsort(-s[..., ::-1], axis=-1, kind="stable"))[..., :k]
    return order, np.take_along_axis(s, order, axis=-1)


def round_to_bf16_wrong_step(v):
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    step = np.ldexp(1.0, np.maximum(e - 7, -133))
    return np.rint(v / step) * step


def round_to_bf16_truncate(v):
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    step = np.ldexp(1.0, np.maximum(e - 8, -133))
    return np.trunc(v / step) * step


_real_lookup = O.lookup


def lookup_short_k1_list(cfg, q, C, Cp, keep_tables=False, score="dot"):
    """The near-tie list built from the k per-half candidates instead of k + 1."""
    out = _real_lookup(cfg, q, C, Cp, keep_tables, score)
    sc, rw = O.candidates(out["sub_idx1"], out["sub_val1"], out["sub_idx2"], out["sub_val2"], cfg.n_keys2)
    kk = min(cfg.topk + 1, sc.shape[-1])
    out["rows_k1"], out["scores_k1"] = O.select_topk(sc, rw, kk)
    return out


def gather_sum_first_head_only(rows, w, V, v_dtype, chunk=256):
    return O.__dict__["_gather_real"](rows[:, :1], w[:, :1], V, v_dtype, chunk)


def value_grad_dense_no_weight(rows, w, dY, y_dtype, n_rows):
    T = rows.shape[0]
    per_tok = rows.size // T
    dV = np.zeros((n_rows, dY.shape[1]), dtype=np.float64)
    dYf = O.decode(dY, y_dtype)
    flat = rows.reshape(-1)
    np.add.at(dV, flat, dYf[np.arange(flat.size) // per_tok])
    return dV


def subkey_backward_dC_from_q2(cfg, rows, ds, q, C, Cp):
    dq, dC, dCp = _real_subkey_backward(cfg, rows, ds, q, C, Cp)
    T, h, k = rows.shape
    half = cfg.dq // 2
    q1, q2 = O.split_heads(q, h, cfg.dq)
    i = rows // cfg.n_keys2
    hh = np.broadcast_to(np.arange(h)[None, :, None], i.shape)
    dC = np.zeros_like(C)
    np.add.at(dC, (hh.reshape(-1), i.reshape(-1)), (ds[..., None] * q2[:, :, None, :]).reshape(-1, half))
    return dq, dC, dCp


_real_subkey_backward = O.subkey_backward


def adam_no_bias_correction(V_rows, m_rows, v_rows, g, lr, beta1, beta2, eps, step, v_dtype):
    g = np.asarray(g, dtype=np.float64)
    m1 = beta1 * np.asarray(m_rows, dtype=np.float64) + (1.0 - beta1) * g
    v1 = beta2 * np.asarray(v_rows, dtype=np.float64) + (1.0 - beta2) * g * g
    V1 = O.decode(V_rows, v_dtype) - lr * m1 / (np.sqrt(v1) + eps)
    return O.round_to_storage(V1, v_dtype), m1, v1


def e4m3_decode_subnormal_step(codes):
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -7, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode_ties_away(x):
    finite = np.array([c for c in range(256) if not np.isnan(O.e4m3_decode(np.array([c]))[0])], dtype=np.int64)
    vals = O.e4m3_decode(finite)
    pos = finite[(vals >= 0) & ~((vals == 0) & (finite == 0x80))]
    pv = O.e4m3_decode(pos)
    order = np.argsort(pv)
    pos, pv = pos[order], pv[order]
    a = np.minimum(np.abs(np.asarray(x, dtype=np.float64)), O.E4M3_MAX)
    i = np.clip(np.searchsorted(pv, a), 1, len(pv) - 1)
    take_hi = (pv[i] - a) <= (a - pv[i - 1])                         # a tie goes up, not to the even code
    code = np.where(a == 0, 0, np.where(take_hi, pos[i], pos[i - 1]))
    neg = np.signbit(np.asarray(x, dtype=np.float64)) & (code != 0)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize_rows_fp8_fnuz_max(V, v_dtype):
    # the row maximum mapped to 240 (the largest value of the other e4m3 variant) instead of 448
    Vf = O.decode(V, v_dtype).astype(np.float32)
    mx = np.abs(Vf).max(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        scale = np.where(mx > 0, mx / np.float32(240), np.float32(0)).astype(np.float32)
        inv = np.where(mx > 0, np.float32(240) / mx, np.float32(0)).astype(np.float32)
    return scale, O.e4m3_encode((Vf * inv[:, None]).astype(np.float32))


def idw_scores_squared_distance(q1, q2, C, Cp):
    def idw(qh, K):
        d2 = ((qh[:, :, None, :] - K[None, :, :, :]) ** 2).sum(-1)
        return -np.log(np.maximum(d2, O.IDW_FLOOR))
    return idw(q1, C), idw(q2, Cp)


def idw_scores_plus_log(q1, q2, C, Cp):
    s1, s2 = _real_idw(q1, q2, C, Cp)
    return -s1, -s2


_real_idw = O.subkey_scores_idw
_real_fwpkm = O.fwpkm_chunk


def fwpkm_chunk_ascent(cfg, q, C, Cp, V, target, lr, dense=True):
    return _real_fwpkm(cfg, q, C, Cp, V, target, -lr, dense)


def fwpkm_chunk_read_after_write(cfg, q, C, Cp, V, target, lr, dense=True):
    y, Vn, sel = _real_fwpkm(cfg, q, C, Cp, V, target, lr, True)
    y = O.round_to_storage(O.gather_sum(sel["rows"], sel["w"], Vn, O.F64), cfg.dtype)
    return y, Vn, sel


_real_diagnostics = O.diagnostics


def diagnostics_entropy_log2(rows, w, n_keys, n_keys2):
    hc, hcp, used, ent = _real_diagnostics(rows, w, n_keys, n_keys2)
    return hc, hcp, used, ent / np.log(2.0)


def diagnostics_first_index_by_n_keys(rows, w, n_keys, n_keys2):
    hc, hcp, used, ent = _real_diagnostics(rows, w, n_keys, n_keys2)
    for hh in range(rows.shape[1]):
        r = rows[:, hh, :].reshape(-1).astype(np.int64)
        hc[hh] = np.bincount(np.minimum(r // n_keys, n_keys - 1), minlength=n_keys)[:n_keys]
    return hc, hcp, used, ent


_real_weight_grad = O.weight_grad


def weight_grad_tokens_reversed(rows, dY, V, dtype, chunk=256):
    return _real_weight_grad(rows, dY[::-1], V, dtype, chunk)



_real_adam_rows = O.adam_rows_state_step


def _adam_rows_variant(touched, slot, M, Vm, n_used, capacity, V_rows, g, lr, beta1, beta2, eps, step, v_dtype,
                       descending=False, fresh_from_pool=False, count_granted_only=False):
    touched = np.asarray(touched, dtype=np.int64)
    slot = np.array(slot, dtype=np.int64)
    M = np.array(M, dtype=np.float64)
    Vm = np.array(Vm, dtype=np.float64)
    new = slot[touched] == -1
    rank = np.cumsum(new) - 1
    if descending:
        rank = new.sum() - 1 - rank
    s_new = n_used + rank
    granted = new & (s_new < capacity)
    slot[touched[granted]] = s_new[granted]
    stepped = ~new | granted
    out = O.decode(V_rows, v_dtype).copy()
    s = slot[touched[stepped]]
    fresh = np.zeros_like(new[stepped]) if fresh_from_pool else new[stepped]
    m0 = np.where(fresh[:, None], 0.0, M[s])
    v0 = np.where(fresh[:, None], 0.0, Vm[s])
    V1, m1, v1 = O.sparse_adam_rows(np.asarray(V_rows)[stepped], m0, v0, np.asarray(g)[stepped], lr, beta1, beta2,
                                    eps, step, v_dtype)
    out[stepped] = V1
    M[s] = m1
    Vm[s] = v1
    return out, slot, M, Vm, int(n_used + (granted.sum() if count_granted_only else new.sum())), stepped


def adam_rows_descending(*a):
    return _adam_rows_variant(*a, descending=True)


def adam_rows_fresh_from_pool(*a):
    return _adam_rows_variant(*a, fresh_from_pool=True)


def adam_rows_count_granted_only(*a):
    return _adam_rows_variant(*a, count_granted_only=True)

# ---------------------------------------------------------------------------
# the pins each mistake must trip (functions of tests/test_oracle_pins.py)
# ---------------------------------------------------------------------------
def _fd_all():
    for bn, tau in ((False, 1.0), (True, 1.0), (False, 0.37), (True, 0.37)):
        pins.test_gradients_by_finite_differences(bn, tau)


def _selection_pins():
    pins.test_brute_force_matches_python_loops_integer_ties()
    for seed in range(40):
        pins.test_product_key_selection_is_exact_topk(seed)
    pins.test_selection_integer_ties_small_brute()


def _k1_pins():
    for seed in range(40):
        pins.test_top_k_plus_one_list_is_exact(seed)


def _idw_pins():
    pins.test_idw_scores_closed_forms()
    for seed in range(3):
        pins.test_idw_product_key_selection_is_exact_topk(seed)


def _bf16_pins():
    pins.test_round_to_bf16_special_values()
    pins.test_round_to_bf16_matches_torch_cast()


MUTATIONS = {
    "bn backward: dropped xhat term": ("batchnorm_backward", bn_backward_dropped_xhat_term,
                                        [_fd_all, pins.test_backward_invariants]),
    "bn forward: unbiased variance": ("batchnorm_forward", bn_forward_unbiased,
                                      [pins.test_batchnorm_closed_form_and_torch]),
    "softmax backward: sign": ("softmax_backward", softmax_backward_sign, [_fd_all]),
    "softmax backward: times tau": ("softmax_backward", softmax_backward_times_tau, [_fd_all]),
    "softmax backward: tau dropped": ("softmax_backward", softmax_backward_no_tau, [_fd_all]),
    "softmax: tau dropped": ("softmax", softmax_no_tau, [pins.test_softmax_closed_forms]),
    "halves swapped": ("split_heads", split_heads_swapped, [_selection_pins]),
    "projection transposed": ("project", project_transposed, [pins.test_project_permutation_and_scaling]),
    "row formula": ("candidates", candidates_wrong_row, [_selection_pins]),
    "tie order": ("topk_sorted", topk_highest_index_first, [pins.test_topk_sorted_against_python_sort]),
    "bf16 step": ("round_to_bf16", round_to_bf16_wrong_step, [_bf16_pins]),
    "bf16 truncation": ("round_to_bf16", round_to_bf16_truncate, [_bf16_pins]),
    "top-(k+1) from k candidates per half": ("lookup", lookup_short_k1_list, [_k1_pins]),
    "gather: one head": ("gather_sum", gather_sum_first_head_only, [pins.test_gather_k1_is_row_copy_and_heads_add,
                                                                   lambda: pins.test_gather_sum_dense_identity("f32")]),
    "dV: weight dropped": ("value_grad_dense", value_grad_dense_no_weight,
                           [pins.test_value_grad_dense_identity_and_conservation]),
    "dC from the second half's query": ("subkey_backward", subkey_backward_dC_from_q2, [_fd_all]),
    "Adam: no bias correction": ("sparse_adam_rows", adam_no_bias_correction,
                                 [pins.test_sparse_adam_all_rows_touched_matches_dense_adam]),
    "e4m3 decode: subnormal step": ("e4m3_decode", e4m3_decode_subnormal_step,
                                    [pins.test_e4m3_decode_matches_torch_float8_on_every_code]),
    "e4m3 encode: ties away from zero": ("e4m3_encode", e4m3_encode_ties_away,
                                         [pins.test_e4m3_encode_matches_torch_cast_including_ties]),
    "fp8 rows: maximum 240": ("quantize_rows_fp8", quantize_rows_fp8_fnuz_max,
                              [pins.test_quantize_rows_fp8_closed_forms_and_error_bound]),
    "IDW: log of the squared distance": ("subkey_scores_idw", idw_scores_squared_distance,
                                         [pins.test_idw_scores_closed_forms]),
    "IDW: sign": ("subkey_scores_idw", idw_scores_plus_log, [_idw_pins]),
    "FwPKM write: ascent": ("fwpkm_chunk", fwpkm_chunk_ascent,
                            [pins.test_fwpkm_chunk_write_is_the_gradient_step_of_the_reconstruction_loss]),
    "FwPKM: read after the write": ("fwpkm_chunk", fwpkm_chunk_read_after_write,
                                    [pins.test_fwpkm_chunk_write_is_the_gradient_step_of_the_reconstruction_loss]),
    "entropy in bits": ("diagnostics", diagnostics_entropy_log2,
                        [pins.test_diagnostics_against_python_loops, pins.test_diagnostics_entropy_closed_forms]),
    "hits of C: row // |C|": ("diagnostics", diagnostics_first_index_by_n_keys,
                              [pins.test_diagnostics_against_python_loops]),
    "dw: tokens reversed": ("weight_grad", weight_grad_tokens_reversed, [_fd_all]),
    "row state: slots in descending row order": ("adam_rows_state_step", adam_rows_descending,
                                                 [pins.test_adam_rows_state_slot_rule_worked_example]),
    "row state: a fresh row reads the pool": ("adam_rows_state_step", adam_rows_fresh_from_pool,
                                              [pins.test_adam_rows_state_matches_torch_sparse_adam]),
    "row state: refused rows not counted": ("adam_rows_state_step", adam_rows_count_granted_only,
                                            [pins.test_adam_rows_state_slot_rule_worked_example]),
}


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_planted_mistake_fails_a_pin(name, monkeypatch):
    attr, bad, checks = MUTATIONS[name]
    if attr == "gather_sum":
        monkeypatch.setitem(O.__dict__, "_gather_real", O.gather_sum)
    monkeypatch.setattr(O, attr, bad)
    failed = []
    for check in checks:
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            failed.append(getattr(check, "__name__", "check"))
    assert failed, f"planted mistake '{name}' passed every pin"


def test_unmutated_oracle_passes_the_same_pins():
    # the harness itself: with the real oracle every check above passes
    for _, (_, _, checks) in MUTATIONS.items():
        for check in checks:
            check()
