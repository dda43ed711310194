"""Planted mistakes: each mutant of the oracle's source (a dropped term, a wrong
sign or index, a swapped operand) must make at least one pin test fail.  The
mutations are applied to the oracle on the CPU only."""
import inspect
import types

import pytest

import oracle
import oracle.attention as attention_src
import oracle.context as context_src
import oracle.generate as generate_src
import oracle.mamba as mamba_src
import oracle.sampling as sampling_src
import oracle.sublayer as sublayer_src
import oracle.unmask as unmask_src

from . import test_oracle_attention as TA
from . import test_oracle_context as TC
from . import test_oracle_generate as TG
from . import test_oracle_mamba as TM
from . import test_oracle_sampling as TS
from . import test_oracle_sublayer as TL
from . import test_oracle_unmask as TU

ATTN_PINS = [TA.test_p1_empty_context_is_library_attention,
             TA.test_p2_concat_block_causal_equivalence,
             TA.test_p3_rows_sum_to_one, TA.test_p4_single_key_returns_value,
             TA.test_p5_equal_keys_give_mean_value,
             lambda: TA.test_p6_planted_key_weight(3.0),
             TA.test_p7_adaln_special_cases, TA.test_p8_permutations,
             TA.test_p9_gqa_is_repeated_mha, TA.test_brute_force_tiny,
             TA.test_timestep_embedding_special_values, TA.test_adaln_single_pins]

UNMASK_PINS = [TU.test_u1_exact_half_and_inclusive_threshold,
               lambda: TU.test_u2_planted_logit_closed_form(1024),
               TU.test_u3_one_commit_rule, TU.test_u4_lowest_id_on_ties,
               lambda: TU.test_u5_u8_loop_invariants(0), TU.test_u6_monotone_in_gamma,
               lambda: TU.test_u7_temperature_closed_form(0.1),
               TU.test_mask_id_prediction_commits, TU.test_nothing_masked_is_a_noop,
               lambda: TU.test_u9_brute_force(1)]

ATTN_MUTANTS = [
    ("g = h // group", "g = h % Hkv"),                          # wrong GQA head map
    ("@ keys.T / np.sqrt(d)", "@ keys.T"),                      # dropped 1/sqrt(d)
    ("(1.0 + _f64(scale)", "(_f64(scale)"),                     # dropped the 1 in (1+scale)
    ("q = q + _f64(shift)", "q = q - _f64(shift)"),             # wrong sign of shift
    ("kc[st:st + n, g, :], kb[b, :, g, :]", "kc[st:st + n, g, :]"),   # dropped block keys
    ("o = o + _f64(residual)[b, :, h, :]", "o = o"),            # dropped residual
    ("mx[:, 0] + np.log(z[:, 0])\n            if gate", "np.log(z[:, 0])\n            if gate"),  # lse without max
    ("[np.cos(args), np.sin(args)]", "[np.sin(args), np.cos(args)]"),  # swapped sinusoid halves
    ("silu = e / (1.0 + np.exp(-e))", "silu = e"),              # dropped SiLU
    ("u[None, :, :, :] + table[:, :, None, :]", "u[None, :, :, :] + 0 * table[:, :, None, :]"),
    ("u.reshape(e.shape[0], 3, width).transpose(1, 0, 2)",
     "u.reshape(e.shape[0], width, 3).transpose(2, 0, 1)"),     # interleaved chunks
]

CONTEXT_PINS = [TC.test_c1_empty_context_is_library_causal_attention,
                TC.test_c2_dense_mask_with_one_block_per_token,
                TC.test_c3_row_equals_single_token_decode,
                TC.test_c4_last_row_bidirectional_first_row_value,
                TC.test_c5_causality_and_context_permutation, TC.test_c6_brute_force_tiny,
                TC.test_k1_append_regions_and_length_rule, TC.test_k2_grown_context_feeds_next_block]

CONTEXT_MUTANTS = [
    ("kb[b, :s + 1, g, :]], axis=0)", "kb[b, :, g, :]], axis=0)"),     # no causal mask
    ("kb[b, :s + 1, g, :]], axis=0)", "kb[b, :s + 2, g, :]], axis=0)"),  # off by one
    ("vb[b, :s + 1, g, :]], axis=0)", "vb[b, :s + 1, g, :]][::-1], axis=0)"),  # misaligned V
    ("keys = np.concatenate([kc[st:st + n, g, :], ", "keys = np.concatenate([kc[st:st + n, 0, :], "),
    ("/ np.sqrt(d)            # [n + s + 1]", "           # [n + s + 1]"),  # dropped 1/sqrt(d)
    ("o = o + _f64(residual)[b, s, h, :]", "o = o"),                      # dropped residual
    ("kc[st + n:st + n + S] = kb[b]", "kc[st + n - 1:st + n - 1 + S] = kb[b]"),  # overwrites context
    ("if n + S > int(ctx_end[b]) - st:", "if n + S > int(ctx_end[b]):"),  # room test ignores start
    ("if n[b] + block_size <= int(ctx_end[b]) - int(ctx_start[b]):",
     "if n[b] < int(ctx_end[b]) - int(ctx_start[b]):"),                  # length rule without S
]

SAMPLING_PINS = [TS.test_s1_philox_known_answers, TS.test_s2_uniform_map, TS.test_s3_gumbel_moments,
                 TS.test_s4_sampling_follows_softmax, TS.test_s5_confidence_closed_forms,
                 TS.test_s6_counter_fields, TS.test_s7_sampled_unmask_commit_rule]

SAMPLING_MUTANTS = [
    ("_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)",
     "_M0, _M1 = np.uint64(0xCD9E8D57), np.uint64(0xD2511F53)"),        # swapped multipliers
    ("        if r:\n            k0 = (k0 + _W0) & _MASK32", "        if False:\n            k0 = (k0 + _W0) & _MASK32"),
    ("c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0", "c0, c1, c2, c3 = hi0 ^ c1 ^ k0, lo1, hi1 ^ c3 ^ k1, lo0"),
    ("for r in range(10):", "for r in range(7):"),                      # too few rounds
    ("(2.0 * (w >> np.uint64(9)).astype(np.float64) + 1.0) / 16777216.0",
     "(w >> np.uint64(8)).astype(np.float64) / 16777216.0"),            # u may be 0
    ("return -np.log(-np.log(u))", "return -np.log(u)"),                # exponential, not Gumbel
    ("key = x + tau * g", "key = x + g"),                               # noise not scaled by tau
    ("return pred, math.exp((x[pred] - m) / tau) / z, margin", "return pred, 1.0 / z, margin"),  # greedy p
    ("pred = int(np.flatnonzero(key == best)[0])", "pred = int(np.argmax(x))"),  # no sampling
]

GENERATE_PINS = [TG.test_g1_eos_stop, TG.test_g2_cache_contents,
                 TG.test_g3_next_block_sees_committed_block, TG.test_g4_last_step_commits_the_rest,
                 TG.test_g5_room_stop, TG.test_g6_sampling_small_temperature_is_argmax]

GENERATE_MUTANTS = [
    ("if eos_token_id is not None and np.any(tok[b] == eos_token_id):", "if False:"),  # no EOS stop
    ("            elif not appended[b]:", "            elif False:"),                   # no room stop
    ("max_steps=steps,\n", "max_steps=S,\n"),                                     # steps ignored
    ("finish_block=True)", "finish_block=False)"),                                 # blocks left unfinished
    ("sample=None if seed is None else (seed, blk)", "sample=None if seed is None else (seed, 0)"),
    ("lens, appended = ctx_advance(S, ctx_start, ctx_end, lens, act_u8)",
     "_, appended = ctx_advance(S, ctx_start, ctx_end, lens, act_u8)"),              # lengths never grow
    ("            kc[layer], vc[layer], _ = kv_append(", "            _, _, _ = kv_append("),  # no append
]

MAMBA_PINS = [TM.test_m1_scan_equals_dual_form, TM.test_m2_seeded_block_equals_scan_of_concatenation,
              TM.test_m3_conv_against_numpy, TM.test_m4_closed_forms, TM.test_m5_brute_force_tiny,
              TM.test_m6_causal_in_block]

MAMBA_MUTANTS = [
    ("g = h // (H // G)\n            st = _f64(ssm_state[b, h]).copy()",
     "g = h % G\n            st = _f64(ssm_state[b, h]).copy()"),             # wrong group map
    ("y[b, s, h] = st @ Cm[s, g] + _f64(D)[h] * x[s, h]", "y[b, s, h] = st @ Cm[s, g]"),  # no skip
    ("dt = softplus(_f64(dt_raw[b]) + _f64(dt_bias)[None, :])          # [S, H]",
     "dt = softplus(_f64(dt_raw[b]))          # [S, H]"),                      # dt bias dropped
    ("out[s] = (u[s:s + W] * w.T).sum(axis=0) + b", "out[s] = (u[s:s + W][::-1] * w.T).sum(axis=0) + b"),
    ("st = np.exp(dt[s, h] * A[h]) * st + dt[s, h] * np.outer(x[s, h], Bm[s, g])",
     "st = np.exp(A[h]) * st + dt[s, h] * np.outer(x[s, h], Bm[s, g])"),      # decay without dt
    ("st = np.exp(dt[s, h] * A[h]) * st + dt[s, h] * np.outer(x[s, h], Bm[s, g])",
     "st = np.exp(dt[s, h] * A[h]) * st + np.outer(x[s, h], Bm[s, g])"),      # input without dt
    ("st = _f64(ssm_state[b, h]).copy()", "st = 0.0 * _f64(ssm_state[b, h])"),  # seed ignored
    ("u = np.concatenate([cs.T, xbc], axis=0)", "u = np.concatenate([0 * cs.T, xbc], axis=0)"),  # conv seed ignored
    ("return silu(out), u[S:].T.copy()", "return out, u[S:].T.copy()"),      # SiLU dropped
    ("A = -np.exp(_f64(A_log))\n    y = np.empty((Bn, S, H, P))\n    new_conv",
     "A = np.exp(_f64(A_log))\n    y = np.empty((Bn, S, H, P))\n    new_conv"),  # growing state
]

SUBLAYER_PINS = [TL.test_l1_layer_norm_is_library_layer_norm,
                 TL.test_l2_l3_layer_norm_closed_form_and_invariants,
                 TL.test_m1_modulation_special_cases, TL.test_linear_and_split_brute_force,
                 TL.test_s1_gate_and_inactive_special_cases,
                 TL.test_s2_selection_weights_reduce_to_block_attention,
                 TL.test_s3_brute_force_tiny, TL.test_s4_block_permutation]

SUBLAYER_MUTANTS = [
    ("var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)",
     "var = ((x - mu) ** 2).sum(axis=-1, keepdims=True) / (x.shape[-1] - 1)"),   # sample variance
    ("return (x - mu) / np.sqrt(var + eps)", "return (x - mu) / np.sqrt(var)"),  # eps dropped
    ("(1.0 + _f64(scale)[:, None, :])", "_f64(scale)[:, None, :]"),              # dropped the 1
    ("+ _f64(shift)[:, None, :]", "- _f64(shift)[:, None, :]"),                  # wrong sign of shift
    ("k = qkv[..., nq:nq + nk]", "k = qkv[..., nq + nk:]"),                       # k takes v's columns
    ("return _f64(x) @ _f64(w).T", "return _f64(x) @ _f64(w)[:, ::-1].T"),       # reversed input order
    ("return _f64(x) + _f64(gate)[:, None, :] * _f64(y)", "return _f64(x) + _f64(y)"),  # no gate
    ("y = linear(o.reshape(B, S, n_q_heads * head_dim), w_o)",
     "y = linear(o.transpose(0, 1, 3, 2).reshape(B, S, n_q_heads * head_dim), w_o)"),  # head/channel order
    ("o, _ = block_attn(q, k, v, k_ctx, v_ctx, ctx_start, ctx_len, active=active)",
     "o, _ = block_attn(q, k, v, k_ctx, v_ctx, ctx_start, 0 * np.asarray(ctx_len), active=active)"),
]

UNMASK_MUTANTS = [
    ("conf[b, s] >= g or", "conf[b, s] > g or"),                # exclusive threshold
    ("np.flatnonzero(x == m)[0]", "np.flatnonzero(x == m)[-1]"),  # highest id on ties
    ("/ float(temperature)", ""),                               # ignored temperature
    ("top = min(s for s", "top = max(s for s"),                 # highest slot on ties
    ("tok[b, s] = mask_token_id", "pass"),                      # no re-mask
    ("chosen = [top]", "chosen = []"),                          # no one-commit rule
    ("n_m.astype(np.float64) / S", "1.0 - n_m.astype(np.float64) / S"),
]


def _mutant(module, old, new):
    src = inspect.getsource(module)
    assert old in src, old
    mod = types.ModuleType(module.__name__ + "_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new, 1), module.__name__ + "_mutant", "exec"), mod.__dict__)
    return mod


def _caught(pins):
    for pin in pins:
        try:
            pin()
        except Exception:
            return True
    return False


@pytest.mark.parametrize("old,new", ATTN_MUTANTS)
def test_attention_mutant_is_caught(monkeypatch, old, new):
    mod = _mutant(attention_src, old, new)
    for name in ("timestep_embedding", "adaln_single", "modulate_q", "block_attn",
                 "dense_block_causal_attn"):
        monkeypatch.setattr(oracle, name, getattr(mod, name))
    assert _caught(ATTN_PINS)


@pytest.mark.parametrize("old,new", CONTEXT_MUTANTS)
def test_context_mutant_is_caught(monkeypatch, old, new):
    mod = _mutant(context_src, old, new)
    for name in ("ctx_block_attn", "kv_append", "ctx_advance"):
        monkeypatch.setattr(oracle, name, getattr(mod, name))
    assert _caught(CONTEXT_PINS)


@pytest.mark.parametrize("old,new", SAMPLING_MUTANTS)
def test_sampling_mutant_is_caught(monkeypatch, old, new):
    mod = _mutant(sampling_src, old, new)
    for name in ("philox4x32_10", "uniform_words", "gumbel_noise", "row_sample"):
        monkeypatch.setattr(sampling_src, name, getattr(mod, name))
        monkeypatch.setattr(oracle, name, getattr(mod, name))
    import oracle.unmask as um
    monkeypatch.setattr(um, "row_sample", mod.row_sample)
    assert _caught(SAMPLING_PINS)


@pytest.mark.parametrize("old,new", GENERATE_MUTANTS)
def test_generate_mutant_is_caught(monkeypatch, old, new):
    mod = _mutant(generate_src, old, new)
    monkeypatch.setattr(oracle, "generate", mod.generate)
    assert _caught(GENERATE_PINS)


@pytest.mark.parametrize("old,new", MAMBA_MUTANTS)
def test_mamba_mutant_is_caught(monkeypatch, old, new):
    mod = _mutant(mamba_src, old, new)
    for name in ("softplus", "silu", "causal_conv", "mamba_block_scan"):
        monkeypatch.setattr(mamba_src, name, getattr(mod, name))
    assert _caught(MAMBA_PINS)


@pytest.mark.parametrize("old,new", SUBLAYER_MUTANTS)
def test_sublayer_mutant_is_caught(monkeypatch, old, new):
    mod = _mutant(sublayer_src, old, new)
    for name in ("layer_norm", "ln_modulate", "linear", "split_qkv", "gate_residual",
                 "adaln_attn_sublayer"):
        monkeypatch.setattr(sublayer_src, name, getattr(mod, name))
    assert _caught(SUBLAYER_PINS)


@pytest.mark.parametrize("old,new", UNMASK_MUTANTS)
def test_unmask_mutant_is_caught(monkeypatch, old, new):
    mod = _mutant(unmask_src, old, new)
    for name in ("row_confidence", "confidence_unmask", "denoise_block"):
        monkeypatch.setattr(oracle, name, getattr(mod, name))
    assert _caught(UNMASK_PINS + [_loop_timestep_pin])


def _loop_timestep_pin():
    """The loop's timestep is the masked fraction: with adaLN weights that map
    the embedding's first channel straight into the gate, the first step's
    gate equals SiLU(cos(1000 * n_masked / S)) (the embedding at frequency 1)."""
    import math

    import numpy as np
    B, S, Hq, d = 1, 4, 1, 2
    W = Hq * d
    w = np.zeros((256, 3 * W))
    w[0, 2 * W:3 * W] = 1.0                       # gate <- SiLU(emb[0])
    masked = np.array([[1, 1, 1, 0]], np.uint8)
    q = np.zeros((B, S, Hq, d))
    kv = np.ones((B, S, Hq, d))
    ctx = np.zeros((1, 1, d))
    lg = np.zeros((B, S, 4))
    lg[..., 0] = 50.0
    r = oracle.denoise_block(lambda k, l: (q, kv, kv), lambda k: lg, [ctx], [ctx],
                             np.zeros(B, np.int64), np.zeros(B, np.int32),
                             np.full((B, S), 3), masked, 0.8, 1.0, 3, max_steps=1,
                             ada_w=w, ada_bias=np.zeros(3 * W),
                             ada_table=np.zeros((1, 3, W)))
    e0 = math.cos(1000.0 * 3 / 4)
    gate = e0 / (1 + math.exp(-e0))
    out = r["outputs"][0][0][0]
    assert np.allclose(out[0, 0, 0], gate * 1.0, atol=1e-12)


def test_loop_timestep_is_masked_fraction():
    _loop_timestep_pin()
