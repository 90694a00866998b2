"""Plant plausible mistakes in copies of the oracle source and require the pins
to catch each one. The mistakes are made in temporary copies on the CPU; the
oracle in the tree is never modified. Every mutant stays in bounds (no planted
mistake changes which memory is touched beyond the buffers' extents)."""
import os
import shutil

import pytest

import oracle
import pins

# (name, original text, planted text); the original must occur exactly once.
MUTANTS = [
    ("drop_dt_in_input", "sp[n] * dA + v * Bg[n] * xs", "sp[n] * dA + Bg[n] * xs"),
    ("drop_x_in_input", "sp[n] * dA + v * Bg[n] * xs", "sp[n] * dA + v * Bg[n]"),
    ("drop_decay", "sp[n] * dA + v * Bg[n] * xs", "sp[n] + v * Bg[n] * xs"),
    ("decay_sign", "exp(pb->A[h] * v)", "exp(-pb->A[h] * v)"),
    ("decay_uses_raw_dt", "exp(pb->A[h] * v)", "exp(pb->A[h] * (pb->dt_per_dim ? pb->dt[xi] : pb->dt[row * H + h]))"),
    ("C_swapped_for_B", "acc += sp[n] * Cg[n];", "acc += sp[n] * Bg[n];"),
    ("output_from_old_state",
     "sp[n] = sp[n] * dA + v * Bg[n] * xs;\n                acc += sp[n] * Cg[n];",
     "acc += sp[n] * Cg[n];\n                sp[n] = sp[n] * dA + v * Bg[n] * xs;"),
    ("group_modulo", "const int64_t g = h / heads_per_group;", "const int64_t g = h % pb->ngroups;"),
    ("D_without_x", "y += pb->D[h] * xs;", "y += pb->D[h];"),
    ("gate_without_z", "y *= zz * sigmoid(zz);", "y *= sigmoid(zz);"),
    ("gate_sign", "y *= zz * sigmoid(zz);", "y *= zz * sigmoid(-zz);"),
    ("D_after_gate",
     "if (pb->D) y += pb->D[h] * xs;\n            if (pb->z) {\n                const double zz = pb->z[xi];\n                y *= zz * sigmoid(zz);\n            }",
     "if (pb->z) {\n                const double zz = pb->z[xi];\n                y *= zz * sigmoid(zz);\n            }\n            if (pb->D) y += pb->D[h] * xs;"),
    ("softplus_branch", "if (v > 0.0) return v + log1p(exp(-v));", "if (v > 0.0) return log1p(exp(-v));"),
    ("bias_after_softplus",
     "if (pb->dt_bias) v += pb->dt_bias[h];\n            if (pb->dt_softplus) v = softplus(v);",
     "if (pb->dt_softplus) v = softplus(v);\n            if (pb->dt_bias) v += pb->dt_bias[h];"),
    ("bias_ignored", "if (pb->dt_bias) v += pb->dt_bias[h];", ""),
    ("dt_head_index", "pb->dt[row * H + h]", "pb->dt[h]"),
    ("accepted_entry_k", "(k - 1) * src_step_stride", "(k - 1 + (k < steps)) * src_step_stride"),
    ("accepted_ignored", "r = src_table[b * src_seq_stride + (k - 1) * src_step_stride];",
     "r = src_table[b * src_seq_stride];"),
    ("pad_read_not_skipped", "if (!slot_valid(r, pad_slot_id, nslots)) continue;\n        memcpy(s, state_in + r * slot_elems, (size_t)slot_elems * sizeof(double));\n        step_token(&pb, s, b, out);",
     "memcpy(s, state_in + (slot_valid(r, pad_slot_id, nslots) ? r : 0) * slot_elems, (size_t)slot_elems * sizeof(double));\n        step_token(&pb, s, b, out);"),
    ("disable_ignored_one_token", "if (!disable_state_update && slot_valid(w, pad_slot_id, nslots))",
     "if (slot_valid(w, pad_slot_id, nslots))"),
    ("dst_ignored_one_token", "const int64_t w = dst ? dst[b] : r;", "const int64_t w = r;"),
    ("packed_writes_read_slot", "w = t < steps ? dst_table[b * dst_seq_stride + t * dst_step_stride]\n                              : pad_slot_id;",
     "w = r;"),
    ("packed_state_not_chained",
     "step_token(&pb, s, begin + t, out);",
     "memcpy(s, state_in + r * slot_elems, (size_t)slot_elems * sizeof(double));\n            step_token(&pb, s, begin + t, out);"),
    ("sr_row_base_ignored", "    row += rd->row_base;", "    (void)0;"),
    ("valid_upper_bound", "slot >= 0 && slot < nslots", "slot >= 0 && slot <= nslots - 2"),
    ("pad_id_ignored", "return slot != pad_slot_id && slot >= 0", "return slot >= 0"),
    ("ring_window_off_by_one", "if (counted + 1 > logical_window) {", "if (counted + 1 >= logical_window) {"),
    ("ring_no_modulo", "ring_start[s] = (ring_start[s] + counted) % ring_buffer_len;\n            prev_num_accepted[s] = 1;",
     "ring_start[s] = ring_start[s] + counted;\n            prev_num_accepted[s] = 1;"),
    ("ring_restart_at_zero", "prev_num_accepted[s] = 1;", "prev_num_accepted[s] = 0;"),
    ("ring_reset_keeps_query_len", "            prev_query_len[s] = 0;\n            continue;", "            continue;"),
    ("commit_no_window_keeps_count", "if (window == 0) {\n            prev_num_accepted[s] = 0;", "if (window == 0) {\n            prev_num_accepted[s] = counted;"),
    ("commit_tests_accepted", "} else if (counted + window > logical_window) {", "} else if (counted + accepted > logical_window) {"),
    ("commit_checkpoint_keeps_count", "            prev_num_accepted[s] = accepted;\n        } else {", "            prev_num_accepted[s] = counted;\n        } else {"),
    ("commit_start_by_window", "ring_start[s] = (ring_start[s] + counted) % ring_buffer_len;\n            prev_num_accepted[s] = accepted;",
     "ring_start[s] = (ring_start[s] + window) % ring_buffer_len;\n            prev_num_accepted[s] = accepted;"),
    ("commit_window_from_accepted", "prev_query_len[s] = query_start_loc[i + 1] - query_start_loc[i];", "prev_query_len[s] = num_accepted[i];"),
    ("sr_strict_threshold", "((U - 1.0) + frac >= 0.0 ? 1.0 : 0.0)", "((U - 1.0) + frac > 0.0 ? 1.0 : 0.0)"),
    ("sr_threshold_frac", "((U - 1.0) + frac >= 0.0 ? 1.0 : 0.0)", "(U >= frac ? 1.0 : 0.0)"),
    ("sr_random_bits", "const int kbits = format == 1 ? 24 : 16;", "const int kbits = format == 1 ? 16 : 16;"),
    ("sr_exponent_off_by_one", "    e -= 1;                                          /* a in [2^e, 2^(e+1)) */\n", ""),
    ("sr_f16_subnormal_spacing", "const int emin = format == 1 ? -14 : -126;", "const int emin = format == 1 ? -15 : -126;"),
    ("sr_no_overflow", "    if (r > maxfin) r = INFINITY;\n", ""),
    ("philox_multiplier_swap", "const uint64_t p0 = (uint64_t)M0 * c0;", "const uint64_t p0 = (uint64_t)M1 * c0;"),
    ("philox_no_key_bump", "            k0 += W0;\n            k1 += W1;\n", "            k1 += W1;\n"),
    ("philox_key_words_swapped", "const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;", "const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k1;"),
    ("sr_counter_element", "const uint32_t ctr[4] = {(uint32_t)(e / group),", "const uint32_t ctr[4] = {(uint32_t)(e),"),
    ("sr_word_index", "w = words[e % 4];", "w = words[0];"),
    ("sr_bf16_half_swapped", "(e % 2) ? (word >> 16) : (word & 0xFFFFu)", "(e % 2) ? (word & 0xFFFFu) : (word >> 16)"),
    ("sr_bf16_group", "const int64_t group = bf16 ? 8 : 4;", "const int64_t group = 4;"),
    ("sr_row_of_token", "store_state(state_out + w * slot_elems, s, slot_elems, begin + t, rounding);", "store_state(state_out + w * slot_elems, s, slot_elems, begin, rounding);"),
    ("ssd_no_clamp", "        u = fmin(fmax(u, dt_min), dt_max);\n", ""),
    ("ssd_clamp_before_softplus",
     "if (pb->dt_softplus) u = softplus(u);\n        u = fmin(fmax(u, dt_min), dt_max);",
     "u = fmin(fmax(u, dt_min), dt_max);\n        if (pb->dt_softplus) u = softplus(u);"),
    ("ssd_clamp_upper_only", "u = fmin(fmax(u, dt_min), dt_max);", "u = fmin(u, dt_max);"),
    ("ssd_decay_uses_raw_dt", "exp(pb->A[h] * u)", "exp(pb->A[h] * pb->dt[t * H + h])"),
    ("ssd_group_modulo", "const int64_t grp = h / ratio;", "const int64_t grp = h % pb->ngroups;"),
    ("ssd_D_per_dim_index", "pb->D[h * P + p]", "pb->D[p]"),
    ("ssd_gate_dropped", "            if (pb->z) y *= pb->z[i] * sigmoid(pb->z[i]);\n", ""),
    ("ssd_every_chunk_opens", "if (c == 0 || seq_idx[c] != seq_idx[c - 1]) {", "{"),
    ("ssd_initial_state_by_order",
     "memcpy(s, initial_states + seq_idx[c] * elems,",
     "memcpy(s, initial_states + (c == 0 ? 0 : seq_idx[c - 1] + 1) * elems,"),
    ("ssd_state_before_chunk",
     "        for (int64_t t = cu_chunk_seqlens[c]; t < cu_chunk_seqlens[c + 1]; ++t)\n            ssd_step_token(&pb, D_per_dim, dt_min, dt_max, s, t, out);\n        memcpy(chunk_states + c * elems, s, (size_t)elems * sizeof(double));",
     "        memcpy(chunk_states + c * elems, s, (size_t)elems * sizeof(double));\n        for (int64_t t = cu_chunk_seqlens[c]; t < cu_chunk_seqlens[c + 1]; ++t)\n            ssd_step_token(&pb, D_per_dim, dt_min, dt_max, s, t, out);"),
    ("ssd_final_from_run_end",
     "memcpy(final_states + b * elems, chunk_states + last_chunk_indices[b] * elems,",
     "memcpy(final_states + b * elems, chunk_states + (b + 1 < batch ? last_chunk_indices[b + 1] - 1 : nchunks - 1) * elems,"),
    ("ssd_output_from_old_state",
     "st[n] = st[n] * decay + u * Bt[n] * xv;\n                dot += st[n] * Ct[n];",
     "dot += st[n] * Ct[n];\n                st[n] = st[n] * decay + u * Bt[n] * xv;"),
    ("ring_position_not_strided", "const int64_t s = slots[i * slot_stride];\n        if (!slot_valid(s, pad_slot_id, num_states)) continue;\n        if (reset)",
     "const int64_t s = slots[i];\n        if (!slot_valid(s, pad_slot_id, num_states)) continue;\n        if (reset)"),
]


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


def _build_mutant(workdir, name, old, new):
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"{name}: anchor occurs {src.count(old)} times"
    d = workdir / name
    d.mkdir()
    shutil.copy(os.path.join(oracle.HERE, "ssu_oracle.h"), d / "ssu_oracle.h")
    (d / "ssu_oracle.c").write_text(src.replace(old, new))
    lib = str(d / f"libssu_oracle_{name}.so")
    oracle.build(str(d / "ssu_oracle.c"), lib)
    return oracle.Oracle(lib)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(workdir, name, old, new):
    mutant = _build_mutant(workdir, name, old, new)
    caught = []
    for pin in pins.ALL:
        try:
            pin(mutant)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name!r}"
