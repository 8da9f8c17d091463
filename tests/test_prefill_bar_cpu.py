"""Why the prefill parity test applies the whole-output bar only where every
row sees many keys (CPU only, oracle only).

In MHA-mode prefill a query row that sees one cached key outputs W_UV c of
that key, ~15x larger than rows that average hundreds of keys.  The bf16
rounding of such a row alone (2^-9 of its values) then exceeds 2e-2 of the
RMS taken over all rows, so no bf16 implementation can meet a whole-output
bar there, while the same rounding stays under the per-row bar (2e-2 of the
row's own RMS).  On long contexts, where every row averages over a thousand
keys, the rounding also stays under the whole-output bar."""
import numpy as np

from mla_inputs import CONFIGS
from mla_inputs.prefill import generate_prefill
from oracle.prefill import mha_prefill


def _bf16_round(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _ratios(pi):
    c = pi.cfg
    ref = mha_prefill(pi.q, pi.q_lens, pi.c_kv, pi.c_kv_scale, pi.k_rope, pi.block_table,
                      pi.seq_lens, pi.W_UK, pi.W_UV, c.sm_scale, c.page_size, q_tag=c.q_dtype,
                      cache_tag=c.cache_dtype, rope_tag=c.rope_dtype, weight_tag=c.weight_dtype)
    mask = ~np.isnan(ref)
    r = np.where(mask, ref, 0.0)
    err = np.abs(_bf16_round(r) - r)
    rows = mask.all(axis=-1)
    row_rms = np.sqrt(np.mean(r * r, axis=-1))
    per_row = np.max(np.where(rows, err.max(axis=-1) / np.where(rows, row_rms, 1.0), 0.0))
    whole = err.max() / np.sqrt(np.mean(ref[mask] ** 2))
    return per_row, whole


def test_one_key_rows_make_the_whole_output_bar_unreachable():
    cfg = CONFIGS["dsv3_ragged_32k"].replace(heads=4, batch=4, seed=5200, out_dtype="bf16")
    pi = generate_prefill(cfg, 160, seq_lens=[1, 70, 200, 333], q_lens=[1, 70, 64, 150])
    per_row, whole = _ratios(pi)
    assert per_row < 2e-2            # the per-row bar holds above the rounding
    assert whole > 2e-2              # the whole-output bar is below it


def test_long_context_rows_keep_the_whole_output_bar_reachable():
    cfg = CONFIGS["dsv3_ragged_32k"].replace(heads=2, batch=1, seed=5207, out_dtype="bf16")
    pi = generate_prefill(cfg, 64, seq_lens=[1500], q_lens=[64])
    per_row, whole = _ratios(pi)
    assert whole < 2e-2              # output rounding alone leaves room under the bar
