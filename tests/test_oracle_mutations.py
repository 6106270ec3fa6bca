"""Plant plausible mistakes into the CPU oracle and check that a pin catches each.

Each mutation rewrites one substring of one oracle function's source, execs
the result in the oracle module's namespace and patches it in.  The test fails
if the substring is missing (so the list tracks the oracle) or if no pin in the
chosen group fails on the mutated oracle.  Mutations live only on the CPU.
"""

import inspect
import textwrap

import pytest

import pins
from oracle import attnres_oracle as orc

FWD = pins.ALL_FORWARD_PINS
BWD = pins.ALL_BACKWARD_PINS
FBWD = pins.ALL_FULL_BACKWARD_PINS

MUTATIONS = [
    ("rms_sum_not_mean", "rms_normalise",
     "np.mean(v * v, axis=-1, keepdims=True)", "np.sum(v * v, axis=-1, keepdims=True)", FWD),
    ("sum_normalised_sources", "depth_read",
     'h = np.einsum("thn,nthk->thk", alpha, Vh)', 'h = np.einsum("thn,nthk->thk", alpha, Kh)', FWD),
    ("score_scaled_by_sqrt_d", "depth_read",
     'scores = np.einsum("nthk,hk->thn", Kh, wh)', 'scores = np.einsum("nthk,hk->thn", Kh, wh) / np.sqrt(d)', FWD),
    ("query_heads_strided", "depth_read",
     "wh = _f64(w).reshape(H, dh)", "wh = _f64(w).reshape(dh, H).T", FWD),
    ("gain_ignored", "depth_read",
     "K = rms_normalise(V, eps) * _f64(g)[None, None, :]", "K = rms_normalise(V, eps)", FWD),
    ("first_sublayer_reads_a_partial", "block_sources",
     "if i == 1:", "if i == 0:", FWD),
    ("partial_index_off_by_one", "block_sources",
     "_f64(partials)[i - 2]", "_f64(partials)[max(i - 3, 0)]", FWD),
    ("full_prefix_one_too_long", "full_fwd",
     "n_j = n_src - n_dst + j + 1", "n_j = min(n_src, n_src - n_dst + j + 2)", FWD),
    ("merge_sign_error", "block_phase2_merge",
     "b = np.exp(s_p - m)[..., None]", "b = np.exp(m - s_p)[..., None]", FWD),
    ("fused_update_ignores_previous_partial", "block_phase2_merge_update",
     "partial = f if partial_prev is None else _f64(partial_prev) + f", "partial = f", FWD),
    ("fused_update_rms_without_mean", "block_phase2_merge_update",
     "np.mean(h * h, axis=-1)", "np.sum(h * h, axis=-1)", FWD),
    ("lse_drops_max", "block_phase1",
     "lse[l] = (m + np.log(", "lse[l] = (0.0 + np.log(", FWD),
    ("bwd_drops_norm_path", "block_bwd",
     "- X * r[..., None] * cs.T[..., None] / d)", ")", BWD),
    ("bwd_c_without_centering", "block_bwd",
     "c = alpha * (a - np.sum(alpha * a, axis=-1, keepdims=True))", "c = alpha * a", BWD),
    ("bwd_dw_uses_w", "block_bwd",
     "dw[j] = _gain_row(gain, j, d) * Z[j]", "dw[j] = w[j] * Z[j]", BWD),
    ("bwd_partial_grad_from_wrong_source", "block_bwd",
     "d_partials[i_sub - 2] += grad[N]", "d_partials[i_sub - 2] += grad[0]", BWD),
    ("bwd_query_path_without_r", "block_bwd",
     "+ r[..., None] * np.einsum(\"tkn,k->ntk\", c_full, q)", "+ np.einsum(\"tkn,k->ntk\", c_full, q)", BWD),
    ("full_bwd_prefix_one_too_long", "full_bwd",
     "n = n_src - n_dst + j + 1", "n = min(n_src, n_src - n_dst + j + 2)", FBWD),
    ("full_bwd_drops_norm_path", "full_bwd",
     "- X * r[..., None] * cs.T[..., None] / d)", ")", FBWD),
    ("full_bwd_c_without_centering", "full_bwd",
     "c = alpha * (a - np.sum(alpha * a, axis=-1, keepdims=True))", "c = alpha * a", FBWD),
    ("full_bwd_dgain_uses_gain", "full_bwd",
     "dg_rows[j] = w[j] * Z[j]", "dg_rows[j] = _gain_row(gain, j, d) * Z[j]", FBWD),
    ("full_bwd_value_path_from_wrong_destination", "full_bwd",
     "np.einsum(\"tkn,tk->ntk\", alpha_full, dout[j])", "np.einsum(\"tkn,tk->ntk\", alpha_full, dout[0])", FBWD),
]


def _mutated(fn_name: str, old: str, new: str):
    src = textwrap.dedent(inspect.getsource(getattr(orc, fn_name)))
    assert old in src, f"mutation target not found in {fn_name}: {old!r}"
    ns = dict(vars(orc))
    exec(compile(src.replace(old, new, 1), f"<mutant {fn_name}>", "exec"), ns)
    return ns[fn_name]


@pytest.mark.parametrize("name,fn_name,old,new,group", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(monkeypatch, name, fn_name, old, new, group):
    monkeypatch.setattr(orc, fn_name, _mutated(fn_name, old, new))
    caught = []
    for pin in group:
        try:
            pin()
        except Exception as exc:  # AssertionError or a shape error both count as caught
            caught.append((getattr(pin, "__name__", "pin"), type(exc).__name__))
            break
    assert caught, f"no pin caught mutation {name}"
