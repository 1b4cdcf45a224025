"""Print the error of each storage plan of ``precision_plan.PLANS`` on the
seeded workloads: max |Y_plan - Y| / RMS(Y) against the fp64 oracle.

TEST INFRASTRUCTURE ONLY (a script beside the emulator it runs).

    python -m oracle.precision_table [WORKLOAD ...]

Sizes evaluated (fp64 on the host; minutes for all of them):
  d512/h8/b2/t128 and d512/h8/b16/t1024: every batch element and row;
  d1024/h16/b8/t4096: batch elements 0 and 1, every row;
  padded cross d512/h8/b32: batch elements 0..7, every row;
  d4096/h32/b1/t8192: rows 0..255 and 256 rows spaced evenly over the
  sequence; the maximum is taken over all of them, the RMS over the evenly
  spaced ones only (the first rows' outputs are many times the tensor RMS,
  so including them would overstate it).
"""

from __future__ import annotations

import sys
import time

import numpy as np

from mha_inputs import WORKLOADS, as_float64_numpy, make_inputs
from oracle import mha_oracle
from oracle.precision_plan import PLANS, emulate, max_abs_over_rms

SUBSETS = {
    "self_fp32_d512_h8_b2_t128": (None, None),
    "causal_bf16_d512_h8_b16_t1024": (None, None),
    "causal_bf16_d1024_h16_b8_t4096": (2, None),
    "cross_pad_bf16_d512_h8_b32_tq512_tk2048": (8, None),
    "causal_bf16_d4096_h32_b1_t8192": (
        None, np.concatenate([np.arange(256), np.linspace(0, 8191, 256).astype(np.int64)])),
}
# evenly spaced rows (positions in the sampled list) that estimate the RMS
RMS_ROWS = {"causal_bf16_d4096_h32_b1_t8192": np.arange(256, 512)}


def table(names):
    f = as_float64_numpy
    print("| workload | rows | " + " | ".join(PLANS) + " |")
    print("|---|---|" + "---|" * len(PLANS))
    for name in names:
        w = WORKLOADS[name]
        nb, rows = SUBSETS[name]
        inp = make_inputs(w, seed=0)
        B = w.B if nb is None else nb
        mask = inp["key_padding_mask"]
        args = (f(inp["x_q"][:B]), f(inp["w_qkv"]), f(inp["b_qkv"]), f(inp["w_o"]),
                f(inp["b_o"]), w.h)
        kw = dict(x_kv=None if inp["x_kv"] is None else f(inp["x_kv"][:B]), causal=w.causal,
                  key_padding_mask=None if mask is None else mask[:B].numpy())
        t0 = time.time()
        if rows is None:
            ref = mha_oracle.mha_forward_blocked(*args, **kw)
        else:
            got = mha_oracle.mha_forward_rows(*args, {b: rows for b in range(B)}, **kw)
            ref = np.stack([got[b] for b in range(B)])
        rms = None
        if name in RMS_ROWS:
            sub = ref[:, RMS_ROWS[name]]
            rms = float(np.sqrt(np.mean(sub[~np.isnan(sub)] ** 2)))
        errs = []
        for plan in PLANS.values():
            y = emulate(plan, *args, rows=rows, **kw)
            errs.append(max_abs_over_rms(y, ref, rms))
        what = "all" if rows is None else f"{len(rows)} sampled"
        print(f"| {name} (B={B}) | {what} | " + " | ".join(f"{e:.2e}" for e in errs)
              + f" |   <!-- {time.time() - t0:.0f} s -->", flush=True)


if __name__ == "__main__":
    table(sys.argv[1:] or list(SUBSETS))
