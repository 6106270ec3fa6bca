"""The MSAR oracle against its pins, and planted mistakes that a pin must catch
(the same mechanism as test_oracle_mutations.py, on the MSAR module)."""

import inspect
import textwrap

import pytest

import pins_msar
from oracle import msar_oracle as mso

PINS = pins_msar.ALL_MSAR_PINS


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_msar_pin(pin):
    pin()


MUTATIONS = [
    ("taps_reversed", "msar_expand",
     "out[r, k:] += conv[off + k] * v[:T - k]", "out[r, k:] += conv[off + K - 1 - k] * v[:T - k]"),
    ("convolution_looks_ahead", "msar_expand",
     "out[r, k:] += conv[off + k] * v[:T - k]", "out[r, :T - k] += conv[off + k] * v[k:]"),
    ("kernel_sizes_reversed", "msar_expand",
     "K, off = MSAR_KERNEL_SIZES[r - 1], MSAR_TAP_OFFSETS[r - 1]",
     "K, off = MSAR_KERNEL_SIZES[3 - r], MSAR_TAP_OFFSETS[r - 1]"),
    ("values_are_normalised_keys", "msar_fwd",
     'Z[j, r] = np.einsum("it,itc->tc", a, vals)', 'Z[j, r] = np.einsum("it,itc->tc", a, keys)'),
    ("values_are_raw_sources", "msar_fwd",
     'Z[j, r] = np.einsum("it,itc->tc", a, vals)', 'Z[j, r] = np.einsum("it,itc->tc", a, streams[:n, 0])'),
    ("one_query_for_all_streams", "msar_fwd",
     'np.einsum("itc,c->it", keys, w[j, r])', 'np.einsum("itc,c->it", keys, w[j, 0])'),
    ("mixer_without_rmsnorm", "msar_fwd",
     "sigmoid(rms_normalise(flat, eps) @ P[j])", "sigmoid(flat @ P[j])"),
    ("flatten_interleaves_streams", "msar_fwd",
     "flat = np.concatenate([Z[j, r] for r in range(MSAR_STREAMS)], axis=-1)",
     "flat = np.stack([Z[j, r] for r in range(MSAR_STREAMS)], axis=-1).reshape(T, -1)"),
    ("mixer_weights_are_a_softmax", "msar_fwd",
     "beta[j] = sigmoid(rms_normalise(flat, eps) @ P[j])",
     "beta[j] = np.exp(rms_normalise(flat, eps) @ P[j]); beta[j] /= beta[j].sum(-1, keepdims=True)"),
    ("prefix_one_too_long", "msar_fwd",
     "n = n_src - n_dst + j + 1", "n = min(n_src, n_src - n_dst + j + 2)"),
    ("phase1_lse_drops_max", "block_msar_phase1",
     "lse[i, r] = m + np.log(l)", "lse[i, r] = np.log(l)"),
    ("phase2_merge_sign_error", "block_msar_phase2",
     "b = np.exp(sp - m)[:, None]", "b = np.exp(m - sp)[:, None]"),
    ("phase2_merges_raw_partial", "block_msar_phase2",
     "Z[r] = (a * o_i[r] + b * xp[r]) / (a + b)", "Z[r] = (a * o_i[r] + b * xp[0]) / (a + b)"),
    ("phase1_sublayer1_mixer_from_wrong_state", "block_msar_phase1",
     "return _mixer(o[0], P1, eps), o[1:], lse[1:]", "return _mixer(o[1], P1, eps), o[1:], lse[1:]"),
]


def _mutated(fn_name, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(mso, fn_name)))
    assert old in src, f"mutation target not found in {fn_name}: {old!r}"
    ns = dict(vars(mso))
    exec(compile(src.replace(old, new, 1), f"<mutant {fn_name}>", "exec"), ns)
    return ns[fn_name]


@pytest.mark.parametrize("name,fn_name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_msar_mutation_is_caught(monkeypatch, name, fn_name, old, new):
    monkeypatch.setattr(mso, fn_name, _mutated(fn_name, old, new))
    for pin in PINS:
        try:
            pin()
        except Exception:
            return
    pytest.fail(f"no pin caught mutation {name}")
