"""Plant a plausible mistake in a copy of the oracle and check that the pins
catch it (a dropped term, a wrong index, sign or rounding rule, a transposed
operand, a reordered reduction). Runs on the CPU; the real oracle is never
modified. Each mutant is chosen so that it stays in bounds (no crash)."""
import pytest

import oracle
import pins

MUTANTS = [
    # number formats
    ("e4m3 truncates instead of rounding",
     "double m = nearbyint((2.0 * fr - 1.0) * 8.0);", "double m = floor((2.0 * fr - 1.0) * 8.0);"),
    ("e4m3 subnormal rounding truncates",
     "double m = nearbyint(a * 512.0);", "double m = floor(a * 512.0);"),
    ("e4m3 mantissa carry ignored",
     "    if (m == 8.0) {\n        m = 0.0;\n        efield += 1;\n    }", "    if (m == 8.0) m = 7.0;"),
    ("e4m3 exponent bias off by one", "int efield = (ex - 1) + 7;", "int efield = (ex - 1) + 8;"),
    ("e4m3 loses the sign", "uint8_t sign = signbit(v) ? 0x80 : 0x00;", "uint8_t sign = 0x00;"),
    ("bf16 ties away from zero",
     "return ((lo >> 16) & 1u) ? (uint16_t)(hi >> 16) : (uint16_t)(lo >> 16);",
     "return (uint16_t)(hi >> 16);"),
    ("bf16 truncates", "if (d_lo < d_hi) return (uint16_t)(lo >> 16);",
     "if (d_lo < 1e300) return (uint16_t)(lo >> 16);"),
    # layout
    ("stable rank counts twice", "            fill[e] += 1;\n", "            fill[e] += 2;\n"),
    ("rank is inclusive", "rank_in_expert[(size_t)t * k + j] = fill[e];",
     "rank_in_expert[(size_t)t * k + j] = fill[e] + 1;"),
    ("expert -> rank map transposed",
     "is_token_in_rank[(size_t)t * R + e / experts_per_rank] = 1;",
     "is_token_in_rank[(size_t)t * R + e % R] = 1;"),
    ("expert offsets inclusive", "            expert_off[e] = off;\n            off += recv_cnt[e];",
     "            off += recv_cnt[e];\n            expert_off[e] = off - recv_cnt[e] + (recv_cnt[e] > 0);"),
    ("source offsets skip the current rank",
     "            src_expert_off[(size_t)s * E + e] = expert_off[e] + before;\n            before += cnt_se[(size_t)s * E + e];",
     "            before += cnt_se[(size_t)s * E + e];\n            src_expert_off[(size_t)s * E + e] = expert_off[e] + before;"),
    ("source offsets expert-relative", "            src_expert_off[(size_t)s * E + e] = expert_off[e] + before;",
     "            src_expert_off[(size_t)s * E + e] = before;"),
    ("per-rank token count counts slots",
     "cnt_sd[(size_t)s * R + d] += is_token_in_rank[(size_t)t * R + d];",
     "cnt_sd[(size_t)s * R + d] += 2 * is_token_in_rank[(size_t)t * R + d];"),
    ("repeated experts not detected", "        if (row[jj] == e) {", "        if (row[jj] == e && 0) {"),
    ("bad ids not flagged", "        *status |= ORACLE_ST_BAD_EXPERT;\n        return 0;", "        return 0;"),
    ("capacity compares with >", "if ((long long)off > cap_rows) status |= ORACLE_ST_CAPACITY;",
     "if ((long long)off > cap_rows + 1) status |= ORACLE_ST_CAPACITY;"),
    ("positions keep the row at cap", "            if (local >= cap_rows) {", "            if (local > cap_rows) {"),
    ("positions ignore the rank base",
     "long long p = (long long)(e / experts_per_rank) * cap_rows + local;",
     "long long p = (long long)(e / experts_per_rank) * cap_rows + local - (local > 0);"),
    # dispatch / quantization
    ("amax without abs", "float v = fabsf(bf16_to_float(x_row[g * 128 + i]));",
     "float v = bf16_to_float(x_row[g * 128 + i]);"),
    ("scale inverted", "float scale = a / 448.0f;", "float scale = 448.0f / a;"),
    ("quantize ignores the scale", "float prod = bf16_to_float(x_row[g * 128 + i]) * inv;",
     "float prod = bf16_to_float(x_row[g * 128 + i]) * 448.0f;"),
    ("quantize reads the next group", "float prod = bf16_to_float(x_row[g * 128 + i]) * inv;",
     "float prod = bf16_to_float(x_row[((g + 1) % G) * 128 + i]) * inv;"),
    ("recv_w takes the first slot's weight", "if (recv_w && topk_w) recv_w[p] = topk_w[(size_t)t * k + j];",
     "if (recv_w && topk_w) recv_w[p] = topk_w[(size_t)t * k];"),
    # combine / backward
    ("combine unfused", "for (int i = 0; i < H; ++i) a[i] = fmaf(wt, bf16_to_float(r[i]), a[i]);",
     "for (int i = 0; i < H; ++i) a[i] = wt * bf16_to_float(r[i]) + a[i];"),
    ("combine reversed slot order",
     "        for (int j = 0; j < k; ++j) {\n            int32_t p = pos[(size_t)t * k + j];\n            if (p < 0) continue;\n            float wt",
     "        for (int j = k - 1; j >= 0; --j) {\n            int32_t p = pos[(size_t)t * k + j];\n            if (p < 0) continue;\n            float wt"),
    ("combine uses slot 0's weight", "float wt = w ? w[(size_t)t * k + j] : 1.0f;",
     "float wt = w ? w[(size_t)t * k] : 1.0f;"),
    ("combine drops the last slot",
     "        for (int j = 0; j < k; ++j) {\n            int32_t p = pos[(size_t)t * k + j];\n            if (p < 0) continue;\n            float wt",
     "        for (int j = 0; j < k - 1; ++j) {\n            int32_t p = pos[(size_t)t * k + j];\n            if (p < 0) continue;\n            float wt"),
    # low-latency receive layout
    ("low-latency rows counted over all sources",
     "long long p = (long long)e * region + (long long)s * tpr + recv_count[e * R + s];",
     "long long p = (long long)e * region + (long long)s * tpr + recv_count[e * R] * (s == 0);"),
    ("low-latency region stride per source wrong",
     "long long p = (long long)e * region + (long long)s * tpr + recv_count[e * R + s];",
     "long long p = (long long)e * region + (long long)s * (tpr - 1) + recv_count[e * R + s];"),
    ("low-latency source of a token off by one", "        int s = t / tpr;\n        for (int j = 0; j < k; ++j) {\n            pos[(size_t)t * k + j] = -1;",
     "        int s = (t + 1) / tpr % R;\n        for (int j = 0; j < k; ++j) {\n            pos[(size_t)t * k + j] = -1;"),
    # rank-deduplicated exchange
    ("dedup leader by expert instead of rank",
     "if (slot_is_valid(row, jj, E, &ignore) && row[jj] / experts_per_rank == d) leader = 0;",
     "if (slot_is_valid(row, jj, E, &ignore) && row[jj] == row[j]) leader = 0;"),
    ("dedup rank is inclusive", "rank_in_rank[(size_t)t * k + j] = fill[d];",
     "rank_in_rank[(size_t)t * k + j] = fill[d] + 1;"),
    ("dedup local expert keeps the rank base",
     "recv_topk_idx[(size_t)p * k + jj] = here ? row[jj] - d * experts_per_rank : -1;",
     "recv_topk_idx[(size_t)p * k + jj] = here ? row[jj] : -1;"),
    ("dedup weights of other ranks' slots kept",
     "recv_topk_w[(size_t)p * k + jj] = here ? topk_w[(size_t)t * k + jj] : 0.0f;",
     "recv_topk_w[(size_t)p * k + jj] = topk_w[(size_t)t * k + jj];"),
    ("dedup positions keep the row at cap", "if (r < 0 || (long long)r >= cap_rows) {",
     "if (r < 0 || (long long)r > cap_rows) {"),
    # expert-side pre-reduction
    ("prereduce drops the last slot", "        for (int slot = 0; slot < k; ++slot) {",
     "        for (int slot = 0; slot < k - 1; ++slot) {"),
    ("prereduce reversed slot order", "        for (int slot = 0; slot < k; ++slot) {",
     "        for (int slot = k - 1; slot >= 0; --slot) {"),
    ("prereduce ignores the weights", "float weight = recv_topk_w ? recv_topk_w[r * k + slot] : 1.0f;",
     "float weight = 1.0f;"),
    ("prereduce reads the next slot's output",
     "const uint16_t *out = expert_out + ((size_t)r * k + slot) * (size_t)H;",
     "const uint16_t *out = expert_out + ((size_t)r * k + (slot + 1) % k) * (size_t)H;"),
    ("prereduce unfused", "for (int i = 0; i < H; ++i) s[i] = fmaf(weight, bf16_to_float(out[i]), s[i]);",
     "for (int i = 0; i < H; ++i) s[i] = s[i] + weight * bf16_to_float(out[i]);"),
    ("prereduce writes unused rows", "if (d >= R || local >= (long long)token_rows[d]) continue; /* not a used row */",
     "if (d >= R) continue;"),
    ("prereduce rank from the range-relative row", "        long long d = p / cap_rows;",
     "        long long d = (p - row_lo) / cap_rows;"),
    ("combine_backward copies the wrong token",
     "memcpy(grad_rows + (size_t)p * H, grad_y + (size_t)t * H, sizeof(uint16_t) * (size_t)H);",
     "memcpy(grad_rows + (size_t)p * H, grad_y + (size_t)((t + 1) % T) * H, sizeof(uint16_t) * (size_t)H);"),
]


@pytest.fixture(scope="module")
def source():
    return oracle.source_text()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(source, tmp_path, name, old, new):
    assert source.count(old) == 1, f"mutation site not unique/present: {name}"
    orc = oracle.build_variant(source.replace(old, new), str(tmp_path))
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake: {name}"
