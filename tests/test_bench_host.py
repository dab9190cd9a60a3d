"""Host-side pieces of bench.py (CPU only): the one-GPU refusal, the algorithmic byte counts the
roofline is priced on, and the counter summary's source-hash check."""
import importlib.util
import os
import subprocess
import sys

import pytest

from fft_long_convolution_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""   # no JSON line


def test_headline_algorithmic_bytes(bench):
    # u, q, v in and y out (4 x 16*768*4096 bf16), the spectrum's Hermitian half
    # 768*4097 complex bf16, and D
    spec = wl.WORKLOADS["hyena_gated_bf16_b16_h768_n4096"]
    act = 16 * 768 * 4096 * 2
    assert bench.algorithmic_bytes(spec) == 4 * act + 768 * 4097 * 4 + 768 * 2 == 415_240_704


def test_gradient_algorithmic_bytes(bench):
    # dy, u, q, v in; du, dq, dv out; the spectrum's half and D in; dk, dD out in fp32
    spec = wl.WORKLOADS["hyena_gated_bf16_b16_h768_n4096"]
    act = 16 * 768 * 4096 * 2
    want = 7 * act + 768 * 4097 * 4 + 768 * 2 + 768 * 4097 * 4
    assert bench.backward_bytes(spec) == want == 729_816_576


def test_long_and_state_space_algorithmic_bytes(bench):
    # ungated: u in, y out, the spectrum (none for the state-space filter: it is its modes), D
    vl = wl.WORKLOADS["very_long_bf16_b1_h64_n2097152"]
    assert bench.algorithmic_bytes(vl) == 2 * 64 * 2 ** 21 * 2 + 64 * (2 ** 21 + 1) * 4 + 64 * 2
    ssm = wl.WORKLOADS["ssm_bf16_b1_h64_n2097152_ns64"]
    assert bench.algorithmic_bytes(ssm) == 2 * 64 * 2 ** 21 * 2 + 64 * 2 == 536_871_040


def test_counter_summary_is_used_only_for_the_sources_it_was_taken_on(bench, monkeypatch):
    name = "hyena_gated_bf16_b16_h768_n4096"
    with open(os.path.join(ROOT, bench.COUNTER_FILES[name])) as f:
        recorded = [l.split(":", 1)[1].strip() for l in f if l.startswith("source_sha256:")][0]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: recorded)
    cur = bench.counter_summary(name)
    assert int(cur["traffic_bytes_per_launch"]) > bench.algorithmic_bytes(wl.WORKLOADS[name])
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 64)
    assert bench.counter_summary(name) == {}
