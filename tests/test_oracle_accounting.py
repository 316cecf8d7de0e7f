"""Pins for oracle.accounting: every number below is printed on a source page.

The fixtures in tests/golden/ name the page and section of each row.

Pages cited by short name:
  L3.2              "L3.2 显存优化与 ZeRO" (yulong.wang)
  Illustrated ZeRO  "图解分布式训练（八）—— ZeRO 学习" (llm.jiangnianmeng.cn)
  ZeRO paper notes  "ZeRO:" paper notes (puzhiyuan.github.io)
"""

import csv
import math
import os

import pytest

from oracle import accounting

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name), newline="") as f:
        lines = [ln for ln in f if ln.strip() and not ln.lstrip().startswith("#")]
    return [[c.strip() for c in row] for row in csv.reader(lines)]


@pytest.mark.parametrize("row", _rows("pages_model_states.csv"), ids=lambda r: f"{r[0]}-{r[1]}-s{r[2]}-k{r[3]}")
def test_printed_model_states(row):
    psi, nd, stage, k, printed, decimals = float(row[0]), int(row[1]), int(row[2]), int(row[3]), \
        float(row[4]), int(row[5])
    gb = accounting.model_state_bytes(psi, nd, stage, k) / 1e9
    assert round(gb, decimals) == pytest.approx(printed, abs=1e-9), row[6]


@pytest.mark.parametrize("row", _rows("pages_max_model.csv"), ids=lambda r: f"{r[0]}GB-{r[1]}-s{r[2]}")
def test_printed_max_model(row):
    mem, nd, stage, printed, rel = float(row[0]) * 1e9, float(row[1]), int(row[2]), float(row[3]), \
        float(row[4])
    nd = math.inf if nd == math.inf else int(nd)
    billions = accounting.max_params(mem, nd, stage) / 1e9
    assert billions == pytest.approx(printed, rel=rel), row[5]
    assert billions >= printed * (1 - 1e-12), row[5]      # the printed model fits


def test_optimizer_share_is_three_quarters():
    # Illustrated distributed training (8) ZeRO §五: optimizer states are about
    # 75% of model states (12 of 16 bytes per parameter).
    psi = 1.0
    opt = accounting.model_state_bytes(psi, 1, 0) - accounting.model_state_bytes(psi, 1, 0, k=0)
    assert opt / accounting.model_state_bytes(psi, 1, 0) == pytest.approx(0.75)


def test_reduction_factors():
    # Illustrated ZeRO §6.1 table and ZeRO paper notes 0x05 §5.1-5.3: ZeRO-1
    # saves 4x, ZeRO-2 8x (limits as Nd grows), ZeRO-3 saves Nd x (64x at 64).
    base = accounting.model_state_bytes(1.0, 1, 0)
    # max_params(1 byte) is the reciprocal of the limiting bytes per parameter.
    assert base * accounting.max_params(1.0, math.inf, 1) == pytest.approx(4.0)
    assert base * accounting.max_params(1.0, math.inf, 2) == pytest.approx(8.0)
    assert base / accounting.model_state_bytes(1.0, 64, 3) == pytest.approx(64.0)
    big = 1 << 40
    assert base / accounting.model_state_bytes(1.0, big, 1) == pytest.approx(4.0, rel=1e-9)
    assert base / accounting.model_state_bytes(1.0, big, 2) == pytest.approx(8.0, rel=1e-9)


def test_comm_volume_four_cards():
    # CMU 11-868 Lecture 18 notes §3.1: counts per card in units of psi carry a
    # factor 3/4 on 4 cards; without it DP, ZeRO-1 and ZeRO-2 send 2 psi and
    # ZeRO-3 sends 3 psi, i.e. 1.5x (L3.2 §2.3; ZeRO paper notes 0x07).
    for stage in (0, 1, 2):
        assert accounting.comm_volume(1.0, 4, stage) == pytest.approx(1.5)
        assert accounting.comm_volume(1.0, 4, stage) / 0.75 == pytest.approx(2.0)
    assert accounting.comm_volume(1.0, 4, 3) == pytest.approx(2.25)
    assert accounting.comm_volume(1.0, 4, 3) / accounting.comm_volume(1.0, 4, 1) == pytest.approx(1.5)


def test_one_rank_sends_nothing():
    for stage in range(4):
        assert accounting.comm_volume(123.0, 1, stage) == 0.0


def test_invalid_stage():
    with pytest.raises(ValueError):
        accounting.model_state_bytes(1.0, 4, 5)
