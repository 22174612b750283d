"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case swaps one oracle function for a copy with a plausible bug (a dropped term, a wrong
sign, index or scale, a transposed role) and runs the pin tests; at least one must fail.
The oracle itself is restored after every case.
"""

import numpy as np
import pytest

from oracle import attention as A
from oracle import spec_verify as S
import tests.test_oracle_attention as TA
import tests.test_oracle_kv8 as TK
import tests.test_oracle_fp8 as TF
import tests.test_oracle_kv_cache as TC
import tests.test_oracle_logits_verify as TL
from oracle import logits_verify as LV
from oracle import kv_cache as KC
import tests.test_oracle_spec_verify as TS
import tests.test_oracle_tree as TT
import tests.test_oracle_tree_verify as TV
from oracle import tree_verify as TVO

GOLDEN = TA.os.path.join(TA.os.path.dirname(TA.os.path.abspath(TA.__file__)), "golden")

ATTN_PINS = [
    lambda: TA.test_golden_worked_cases(GOLDEN),
    TA.test_single_key_returns_its_value_exactly,
    TA.test_equal_keys_give_the_mean_of_visible_values,
    lambda: TA.test_matches_torch_sdpa_fp64(5, 40, 4, 4, 32),
    lambda: TA.test_matches_torch_sdpa_fp64(5, 77, 32, 8, 128),
    TA.test_matches_torch_sdpa_with_explicit_scale_and_large_scores,
    TA.test_verify_rows_equal_sequential_decodes,
    lambda: TA.test_block_table_permutation_gives_contiguous_result_bit_exact(16),
    TA.test_physical_slot_translation_by_hand,
]


def _seq_variant(scale_fn=None, visible_fn=None, head_fn=None, row_fn=None, tree_fn=None):
    def attention_sequence(q_seq, k_seq, v_seq, scale=None, heads=None, rows=None, tree_mask=None):
        Q, Hq, D = q_seq.shape
        L, Hkv, _ = k_seq.shape
        if Hq % Hkv or not 1 <= Q <= L:
            raise ValueError("bad shape")
        G = Hq // Hkv
        if scale is None:
            scale = scale_fn(D) if scale_fn else 1.0 / np.sqrt(D)
        out = np.full((Q, Hq, D), np.nan)
        for i in (range(Q) if rows is None else rows):
            if tree_mask is None:
                vis = visible_fn(L, Q, i) if visible_fn else L - Q + i + 1
                sel = slice(0, max(1, min(L, vis)))
            else:
                sel = tree_fn(L, Q, i, tree_mask) if tree_fn else A.visible_keys(L, Q, i, tree_mask)
            for h in (range(Hq) if heads is None else heads):
                g = head_fn(h, G, Hkv) if head_fn else h // G
                f = row_fn or A.attend_row
                out[i, h] = f(q_seq[i, h], k_seq[sel, g], v_seq[sel, g], scale)
        return out
    return attention_sequence


def _row_no_shift(q, k, v, scale):
    w = np.exp(scale * (k @ q))
    return (w @ v) / w.sum()


def _row_no_normalise(q, k, v, scale):
    z = scale * (k @ q)
    return np.exp(z - z.max()) @ v


def _row_keys_for_values(q, k, v, scale):
    z = scale * (k @ q)
    w = np.exp(z - z.max())
    return (w @ k) / w.sum()


def _slots_swapped(table_row, n_tokens, block_size):
    j = np.arange(n_tokens)
    blocks = np.asarray(table_row)[j // block_size].astype(np.int64)
    return blocks + (j % block_size) * block_size


ATTN_MUTANTS = {
    "scale 1/D": ("attention_sequence", _seq_variant(scale_fn=lambda D: 1.0 / D)),
    "no scale": ("attention_sequence", _seq_variant(scale_fn=lambda D: 1.0)),
    "causal limit one short": ("attention_sequence", _seq_variant(visible_fn=lambda L, Q, i: L - Q + i)),
    "causal from the wrong end": ("attention_sequence", _seq_variant(visible_fn=lambda L, Q, i: L - i)),
    "gqa h % Hkv": ("attention_sequence", _seq_variant(head_fn=lambda h, G, Hkv: h % Hkv)),
    "no max shift": ("attend_row", _row_no_shift),
    "no normalisation": ("attend_row", _row_no_normalise),
    "keys used as values": ("attend_row", _row_keys_for_values),
    "slot = block + row * bs": ("physical_slots", _slots_swapped),
}


KV8_PINS = [
    lambda: TK.test_dequantize_matches_torch_per_channel_affine(0),
    lambda: TK.test_u8_attention_equals_bf16_attention_on_exact_values(
        dict(ctx_lens=[1, 17, 40, 64], q_lens=[1, 1, 1, 1], Hq=8, Hkv=2, D=64, bs=16)),
    lambda: TK.test_u8_attention_equals_bf16_attention_on_exact_values(
        dict(ctx_lens=[100, 31], q_lens=[1, 8], Hq=6, Hkv=3, D=16, bs=32)),
    TK.test_u8_block_placement_invariance,
]


def _deq_plus_zero(codes, scale, zero_point):
    c = np.asarray(codes).astype(np.float64)
    return np.asarray(scale, np.float64)[..., None] * (c + np.asarray(zero_point, np.float64)[..., None])


def _deq_no_zero(codes, scale, zero_point):
    return np.asarray(scale, np.float64)[..., None] * np.asarray(codes).astype(np.float64)


def _gather_u8_variant(k_cols=(0, 1), v_cols=(2, 3), transpose=True):
    def gather_sequence_kv_u8(codes, kv_scales, table_row, n_tokens):
        sc = np.asarray(kv_scales)
        sc = np.transpose(sc, (0, 2, 1, 3)) if transpose else sc
        s = A.gather_sequence_kv(sc, table_row, n_tokens)
        kc = A.gather_sequence_kv(codes[0], table_row, n_tokens)
        vc = A.gather_sequence_kv(codes[1], table_row, n_tokens)
        return (A.dequantize_u8(kc, s[..., k_cols[0]], s[..., k_cols[1]]),
                A.dequantize_u8(vc, s[..., v_cols[0]], s[..., v_cols[1]]))
    return gather_sequence_kv_u8


KV8_MUTANTS = {
    "zero point added": ("dequantize_u8", _deq_plus_zero),
    "zero point dropped": ("dequantize_u8", _deq_no_zero),
    "K scales used for V": ("gather_sequence_kv_u8", _gather_u8_variant(v_cols=(0, 1))),
    "scale and zero swapped": ("gather_sequence_kv_u8", _gather_u8_variant(k_cols=(1, 0))),
    "scale layout not transposed": ("gather_sequence_kv_u8", _gather_u8_variant(transpose=False)),
}


TREE_PINS = [
    lambda: TT.test_chain_mask_is_the_causal_verify(5),
    lambda: TT.test_each_node_equals_the_causal_verify_of_its_path(0),
    lambda: TT.test_each_node_equals_the_causal_verify_of_its_path(1),
    TT.test_single_node_tree_is_a_decode_row,
]


def _tree_nodes(L, Q, i, tree_mask, shift=0, self_bit=True):
    m = int(tree_mask[i])
    if not self_bit:
        m &= ~(1 << i)
    return [j for j in range(Q) if (m >> (j + shift)) & 1]


TREE_MUTANTS = {
    "tree: node does not see itself": lambda L, Q, i, tm: np.concatenate(
        [np.arange(L - Q), L - Q + np.array(_tree_nodes(L, Q, i, tm, self_bit=False), dtype=np.int64)]).astype(np.int64),
    "tree: prefix dropped": lambda L, Q, i, tm: (L - Q + np.array(_tree_nodes(L, Q, i, tm), dtype=np.int64)),
    "tree: mask bits off by one": lambda L, Q, i, tm: np.concatenate(
        [np.arange(L - Q), L - Q + np.array(_tree_nodes(L, Q, i, tm, shift=1), dtype=np.int64)]).astype(np.int64),
}


TREE_VERIFY_PINS = [
    lambda: TV.test_golden_worked_cases(GOLDEN),
    lambda: [TV.test_chain_tree_is_the_chain_verifier(s) for s in range(6)],
    lambda: TV.test_root_only_is_numpy_inverse_cdf(0),
    TV.test_lossless_monte_carlo_on_a_two_level_tree,
]


def _tree_verify_variant(update="normalised", q_of="parent", order=1, final="current", final_u=0):
    def tree_verify_sequence(p_rows, q_rows, parents, tokens, uniforms):
        p_rows = np.asarray(p_rows, dtype=np.float64)
        q_rows = np.asarray(q_rows, dtype=np.float64)
        N, V = p_rows.shape
        kids = TVO.tree_children(parents)
        ids, path = [], []
        u, p_cur = 0, p_rows[0]
        while True:
            accepted = None
            for c in kids[u][::order]:
                x = int(tokens[c])
                inside = 0 <= x < V
                qrow = q_rows[u] if q_of == "parent" else q_rows[c]
                P = p_cur[x] if inside else 0.0
                Qx = qrow[x] if inside else 0.0
                if S.accept_draft(P, Qx, uniforms[c]):
                    accepted = c
                    break
                if update == "normalised":
                    p_cur = TVO.residual(p_cur, qrow)
                elif update == "raw":
                    p_cur = np.maximum(0.0, p_cur - qrow)
            if accepted is None:
                row = p_cur if final == "current" else p_rows[u]
                y = S.sample_inverse_cdf(row, uniforms[final_u])
                ids.append(max(y, 0))
                break
            path.append(accepted)
            ids.append(int(tokens[accepted]))
            u, p_cur = accepted, p_rows[accepted]
        out = np.full(N, -1, dtype=np.int64)
        out[:len(ids)] = ids
        nodes = np.full(N, -1, dtype=np.int64)
        nodes[:len(path)] = path
        return out, nodes, len(path)
    return tree_verify_sequence


TREE_VERIFY_MUTANTS = {
    "no residual after a rejection": _tree_verify_variant(update="none"),
    "residual not normalised": _tree_verify_variant(update="raw"),
    "residual against the child's q row": _tree_verify_variant(q_of="child"),
    "children tested in reverse order": _tree_verify_variant(order=-1),
    "final draw ignores the residual": _tree_verify_variant(final="fresh"),
    "final draw uses the last node's uniform": _tree_verify_variant(final_u=-1),
}


KV_CACHE_PINS = [
    lambda: TC.test_quantiser_equals_torch_per_channel_minmax(0),
    TC.test_append_writes_exactly_the_new_positions,
    TC.test_append_u8_quantises_each_row_and_touches_nothing_else,
    TC.test_chain_commit_only_shortens,
    lambda: TC.test_tree_commit_then_decode_equals_tree_attention_of_the_last_node("bf16"),
    lambda: TC.test_tree_commit_then_decode_equals_tree_attention_of_the_last_node("u8"),
]


def _quantize_variant(clamp_lo=True, eps=True, levels=255, zero_round=np.rint, divide=False, neg_lo=False):
    def quantize_rows_u8(x):
        x = np.asarray(x, dtype=np.float32)
        lo = x.min(axis=-1)
        if clamp_lo:
            lo = np.minimum(lo, np.float32(0))
        hi = np.maximum(x.max(axis=-1), np.float32(0))
        scale = ((hi - lo) / np.float32(levels)).astype(np.float32)
        if eps:
            scale = np.maximum(scale, KC.FP32_EPS).astype(np.float32)
        num = -lo if neg_lo else np.float32(0) - lo
        zero = np.clip(zero_round(num / scale), 0, 255).astype(np.float32)
        if divide:
            y = x / scale[..., None]
        else:
            y = x * (np.float32(1) / scale).astype(np.float32)[..., None]
        codes = np.clip(np.rint(y) + zero[..., None], 0, 255).astype(np.uint8)
        return codes, scale, zero
    return quantize_rows_u8


def _new_slots_variant(offset=True):
    def _new_slots(table_row, L, Q, bs):
        start = L - Q if offset else 0
        return A.physical_slots(table_row, L, bs)[start:start + Q]
    return _new_slots


def _commit_variant(src_shift=0, dst_start=1, move_scales=True, keep_root=1, gather_first=True):
    def kv_commit_tree(pool, block_tables, ctx_lens, q_lens, path, n_accepted, kv_scales=None):
        pool = np.array(pool, copy=True)
        scales = None if kv_scales is None else np.array(kv_scales, copy=True)
        NB, bs = pool.shape[1], pool.shape[2]
        flat = pool.reshape(2, NB * bs, *pool.shape[3:])
        for s in range(len(ctx_lens)):
            L, Q, n = int(ctx_lens[s]), int(q_lens[s]), int(n_accepted[s])
            slots = A.physical_slots(block_tables[s], L, bs)
            src = slots[L - Q + src_shift + np.asarray(path[s][:n], dtype=np.int64)]
            dst = slots[L - Q + dst_start + np.arange(n)]
            if gather_first:
                flat[:, dst] = flat[:, src].copy()
            else:
                for a, b in zip(src, dst):
                    flat[:, b] = flat[:, a]
            if scales is not None and move_scales:
                scales[dst // bs, :, dst % bs] = scales[src // bs, :, src % bs].copy()
        L2 = (np.asarray(ctx_lens) - np.asarray(q_lens) + keep_root + np.asarray(n_accepted)).astype(np.int64)
        return pool, scales, L2
    return kv_commit_tree


KV_CACHE_MUTANTS = {
    "quantiser: lower end not clamped to 0": ("quantize_rows_u8", _quantize_variant(clamp_lo=False)),
    "quantiser: 256 levels": ("quantize_rows_u8", _quantize_variant(levels=256)),
    "quantiser: zero point floored": ("quantize_rows_u8", _quantize_variant(zero_round=np.floor)),
    "quantiser: no eps floor on the scale": ("quantize_rows_u8", _quantize_variant(eps=False)),
    "quantiser: divides instead of multiplying by 1/scale": ("quantize_rows_u8", _quantize_variant(divide=True)),
    "quantiser: zero point -0 for rows without negatives": ("quantize_rows_u8", _quantize_variant(neg_lo=True)),
    "append: written from position 0": ("_new_slots", _new_slots_variant(offset=False)),
    "commit: source node off by one": ("kv_commit_tree", _commit_variant(src_shift=-1)),
    "commit: overwrites the root": ("kv_commit_tree", _commit_variant(dst_start=0)),
    "commit: scales left behind": ("kv_commit_tree", _commit_variant(move_scales=False)),
    "commit: root not kept in the length": ("kv_commit_tree", _commit_variant(keep_root=0)),
}


LOGITS_PINS = [
    lambda: TL.test_golden_worked_cases(GOLDEN),
    lambda: TL.test_tempered_softmax_is_scipy(0.37),
    lambda: TL.test_positive_temperature_is_the_probability_verifier(0),
    TL.test_shift_and_scale_invariance,
    TL.test_zero_temperature_is_exact_matching,
    TL.test_small_temperature_approaches_greedy,
    TL.test_lossless_first_token_at_temperature,
]


def _softmax_variant(use_T="divide", shift=True, axis=-1):
    def tempered_softmax(z, T):
        z = np.asarray(z, dtype=np.float64)
        y = {"divide": z / float(T), "multiply": z * float(T), "ignore": z}[use_T]
        if shift:
            y = y - y.max(axis=axis, keepdims=True)
        with np.errstate(over="ignore", invalid="ignore"):
            e = np.exp(y)
            return e / e.sum(axis=axis, keepdims=True)
    return tempered_softmax


def _greedy_variant(last=False):
    def greedy_rows(z):
        z = np.asarray(z)
        out = np.zeros(z.shape, dtype=np.float64)
        idx = z.shape[-1] - 1 - np.argmax(z[..., ::-1], axis=-1) if last else np.argmax(z, axis=-1)
        np.put_along_axis(out, idx[..., None], 1.0, axis=-1)
        return out
    return greedy_rows


def _distributions_variant(draft_tempered=True, zero_as_one=False):
    def distributions(zp, zq, T):
        if T == 0.0:
            if zero_as_one:
                return LV.tempered_softmax(zp, 1.0), LV.tempered_softmax(zq, 1.0)
            return LV.greedy_rows(zp), LV.greedy_rows(zq)
        return LV.tempered_softmax(zp, T), LV.tempered_softmax(zq, T if draft_tempered else 1.0)
    return distributions


LOGITS_MUTANTS = {
    "temperature ignored": ("tempered_softmax", _softmax_variant(use_T="ignore")),
    "temperature multiplies the logits": ("tempered_softmax", _softmax_variant(use_T="multiply")),
    "no max shift before exp": ("tempered_softmax", _softmax_variant(shift=False)),
    "softmax over the draft positions": ("tempered_softmax", _softmax_variant(axis=0)),
    "greedy ties to the largest id": ("greedy_rows", _greedy_variant(last=True)),
    "draft rows not tempered": ("distributions", _distributions_variant(draft_tempered=False)),
    "temperature 0 sampled as temperature 1": ("distributions", _distributions_variant(zero_as_one=True)),
}

def _any_pin_fails(pins):
    for pin in pins:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            return True
    return False


@pytest.mark.parametrize("name", sorted(ATTN_MUTANTS))
def test_attention_mutant_is_caught(name, monkeypatch):
    attr, fn = ATTN_MUTANTS[name]
    monkeypatch.setattr(A, attr, fn)
    assert _any_pin_fails(ATTN_PINS), f"no attention pin caught: {name}"


@pytest.mark.parametrize("name", sorted(TREE_MUTANTS))
def test_tree_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(A, "attention_sequence", _seq_variant(tree_fn=TREE_MUTANTS[name]))
    assert _any_pin_fails(TREE_PINS), f"no tree pin caught: {name}"


@pytest.mark.parametrize("name", sorted(TREE_VERIFY_MUTANTS))
def test_tree_verify_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(TVO, "tree_verify_sequence", TREE_VERIFY_MUTANTS[name])
    assert _any_pin_fails(TREE_VERIFY_PINS), f"no tree-verification pin caught: {name}"


@pytest.mark.parametrize("name", sorted(KV8_MUTANTS))
def test_kv8_mutant_is_caught(name, monkeypatch):
    attr, fn = KV8_MUTANTS[name]
    monkeypatch.setattr(A, attr, fn)
    assert _any_pin_fails(KV8_PINS), f"no 8-bit KV pin caught: {name}"


FP8_PINS = [
    TF.test_e4m3_decode_matches_torch_on_every_code,
    lambda: [TF.test_e4m3_hand_worked_codes(c, v) for c, v in ((0x3C, 1.5), (0x07, 7 * 2.0 ** -9), (0xB8, -1.0))],
    TF.test_dequantize_fp8_scale_and_zero,
    lambda: TF.test_fp8_attention_equals_bf16_attention_on_exact_values(
        dict(ctx_lens=[1, 17, 40, 64], q_lens=[1, 1, 1, 1], Hq=8, Hkv=2, D=64, bs=16)),
]


def _e4m3_variant(bias=7, subnormals=True, mant_div=8.0, signed=True):
    def e4m3_to_f64(codes):
        c = np.asarray(codes).astype(np.int64)
        sign = np.where(c & 0x80, -1.0, 1.0) if signed else np.ones(c.shape)
        e = (c >> 3) & 0xF
        m = (c & 0x7).astype(np.float64)
        normal = (1.0 + m / mant_div) * np.exp2(e.astype(np.float64) - bias)
        mag = np.where(e == 0, m * 2.0 ** -9, normal) if subnormals else normal
        return np.where((e == 0xF) & (c & 0x7 == 0x7), np.nan, sign * mag)
    return e4m3_to_f64


def _dequant_fp8_variant(zero_sign=-1.0, use_scale=True):
    def dequantize_fp8(codes, scale, zero_point):
        x = A.e4m3_to_f64(codes)
        s = np.asarray(scale, np.float64)[..., None] if use_scale else 1.0
        return s * (x + zero_sign * np.asarray(zero_point, np.float64)[..., None])
    return dequantize_fp8


FP8_MUTANTS = {
    "exponent bias 8 (the FNUZ format)": ("e4m3_to_f64", _e4m3_variant(bias=8)),
    "subnormals decoded as normals": ("e4m3_to_f64", _e4m3_variant(subnormals=False)),
    "mantissa read as four bits": ("e4m3_to_f64", _e4m3_variant(mant_div=16.0)),
    "sign bit ignored": ("e4m3_to_f64", _e4m3_variant(signed=False)),
    "zero point added": ("dequantize_fp8", _dequant_fp8_variant(zero_sign=1.0)),
    "scale not applied": ("dequantize_fp8", _dequant_fp8_variant(use_scale=False)),
}


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_fp8_mutant_is_caught(name, monkeypatch):
    attr, fn = FP8_MUTANTS[name]
    monkeypatch.setattr(A, attr, fn)
    assert _any_pin_fails(FP8_PINS), f"no FP8 KV pin caught: {name}"


SPEC_PINS = [
    lambda: TS.test_golden_worked_cases(GOLDEN),
    TS.test_p_equal_q_accepts_every_draft,
    TS.test_zero_target_probability_is_always_rejected,
    TS.test_temperature_zero_reduces_to_exact_matching,
    TS.test_k_zero_is_numpy_inverse_cdf,
    TS.test_out_of_range_draft_is_rejected,
    TS.test_emitted_distribution_exact_by_stratified_enumeration,
]


def _verify_variant(accept=None, residual=None, bonus_row=None, keep_going=False, pad=-1):
    def verify_sequence(p_rows, q_rows, drafts, uniforms):
        p_rows = np.asarray(p_rows, dtype=np.float64)
        q_rows = np.asarray(q_rows, dtype=np.float64)
        k = len(drafts)
        V = p_rows.shape[1]
        out = np.full(k + 1, pad, dtype=np.int64)
        n = k
        for i in range(k):
            x = int(drafts[i])
            inside = 0 <= x < V
            P = p_rows[i, x] if inside else 0.0
            Qx = q_rows[i, x] if inside else 0.0
            ok = accept(P, Qx, uniforms[i]) if accept else S.accept_draft(P, Qx, uniforms[i])
            if ok:
                out[i] = x
            elif n == k:
                n = i
                if not keep_going:
                    break
        if n < k:
            w = residual(p_rows[n], q_rows[n]) if residual else np.maximum(0.0, p_rows[n] - q_rows[n])
        else:
            w = p_rows[bonus_row(k)] if bonus_row else p_rows[k]
        y = S.sample_inverse_cdf(w, uniforms[k])
        if y < 0:
            y = S.sample_inverse_cdf(p_rows[n], uniforms[k])
        out[n] = max(y, 0)
        return out, n
    return verify_sequence


def _cdf_descending(w, u):
    w = np.asarray(w, dtype=np.float64)[::-1]
    cum = np.cumsum(w)
    if not cum[-1] > 0:
        return -1
    return int(w.size - 1 - np.nonzero(cum > u * cum[-1])[0][0])


def _cdf_u_not_scaled(w, u):
    cum = np.cumsum(np.asarray(w, dtype=np.float64))
    if not cum[-1] > 0:
        return -1
    above = np.nonzero(cum > u)[0]
    return int(above[0]) if above.size else int(np.nonzero(np.asarray(w) > 0)[0][-1])


SPEC_MUTANTS = {
    "inverted ratio": ("verify_sequence", _verify_variant(accept=lambda P, Q, r: Q > 0 and r * P <= Q)),
    "accept ignores ratio": ("verify_sequence", _verify_variant(accept=lambda P, Q, r: P > 0)),
    "residual q - p": ("verify_sequence", _verify_variant(residual=lambda p, q: np.maximum(0.0, q - p))),
    "residual without clamp": ("verify_sequence", _verify_variant(residual=lambda p, q: np.abs(p - q))),
    "residual is p": ("verify_sequence", _verify_variant(residual=lambda p, q: p)),
    "bonus from row k-1": ("verify_sequence", _verify_variant(bonus_row=lambda k: max(k - 1, 0))),
    "keeps checking after a rejection": ("verify_sequence", _verify_variant(keep_going=True)),
    "pads with 0": ("verify_sequence", _verify_variant(pad=0)),
    "cdf in descending id": ("sample_inverse_cdf", _cdf_descending),
    "u not scaled by Z": ("sample_inverse_cdf", _cdf_u_not_scaled),
}


@pytest.mark.parametrize("name", sorted(KV_CACHE_MUTANTS))
def test_kv_cache_mutant_is_caught(name, monkeypatch):
    attr, fn = KV_CACHE_MUTANTS[name]
    monkeypatch.setattr(KC, attr, fn)
    assert _any_pin_fails(KV_CACHE_PINS), f"no KV-cache pin caught: {name}"


@pytest.mark.parametrize("name", sorted(LOGITS_MUTANTS))
def test_logits_verify_mutant_is_caught(name, monkeypatch):
    attr, fn = LOGITS_MUTANTS[name]
    monkeypatch.setattr(LV, attr, fn)
    assert _any_pin_fails(LOGITS_PINS), f"no logits-verification pin caught: {name}"


@pytest.mark.parametrize("name", sorted(SPEC_MUTANTS))
def test_spec_verify_mutant_is_caught(name, monkeypatch):
    attr, fn = SPEC_MUTANTS[name]
    monkeypatch.setattr(S, attr, fn)
    assert _any_pin_fails(SPEC_PINS), f"no spec_verify pin caught: {name}"


def test_unmodified_wrappers_pass_every_pin(monkeypatch):
    """Controls: the mutant scaffolding without a planted mistake passes all pins, so a caught
    mutant is caught for its mistake and not for the scaffolding."""
    monkeypatch.setattr(A, "attention_sequence", _seq_variant())
    monkeypatch.setattr(S, "verify_sequence", _verify_variant())
    monkeypatch.setattr(A, "gather_sequence_kv_u8", _gather_u8_variant())
    assert not _any_pin_fails(ATTN_PINS)
    assert not _any_pin_fails(SPEC_PINS)
    assert not _any_pin_fails(KV8_PINS)
    assert not _any_pin_fails(TREE_PINS)
    monkeypatch.setattr(TVO, "tree_verify_sequence", _tree_verify_variant())
    assert not _any_pin_fails(TREE_VERIFY_PINS)
    monkeypatch.setattr(KC, "quantize_rows_u8", _quantize_variant())
    monkeypatch.setattr(KC, "_new_slots", _new_slots_variant())
    monkeypatch.setattr(KC, "kv_commit_tree", _commit_variant())
    assert not _any_pin_fails(KV_CACHE_PINS)
    monkeypatch.setattr(LV, "tempered_softmax", _softmax_variant())
    monkeypatch.setattr(LV, "greedy_rows", _greedy_variant())
    monkeypatch.setattr(LV, "distributions", _distributions_variant())
    assert not _any_pin_fails(LOGITS_PINS)
    monkeypatch.setattr(A, "e4m3_to_f64", _e4m3_variant())
    monkeypatch.setattr(A, "dequantize_fp8", _dequant_fp8_variant())
    assert not _any_pin_fails(FP8_PINS)
