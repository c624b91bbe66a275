"""The host scheduler (csrc/pa_sched.cpp) under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

The scheduler source is compiled on its own with the host compiler and both
sanitizers into a test-only shared library; a child Python process (the
sanitizer runtime preloaded) binds the package's scheduler wrapper to that
library instead of libpa.so and runs the scheduler parity tests against the
oracle scheduler (every step of three seeded traces compared, plus the
whole block-pool state every few steps).  Any invalid access, use after
free or undefined operation aborts the child, and the test fails with its
report.  Leak detection is off in that child (the interpreter itself keeps
memory until exit); `test_sched_driver_no_leaks` covers leaks with a small
C++ driver of the scheduler's C ABI instead.
"""

import os
import subprocess

import pytest

import sched_build
from sched_build import CXX

pytestmark = pytest.mark.skipif(CXX is None, reason="needs the host C++ compiler")

SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer"]


def _runtime(name):
    out = subprocess.run([CXX, f"-print-file-name={name}"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _build(tmp_path, extra_sources=(), shared=True):
    out = tmp_path / ("libpa_sched_san.so" if shared else "sched_driver")
    return sched_build.build(out, SAN_FLAGS, extra_sources, shared)


def test_sched_parity_under_sanitizers(tmp_path):
    lib = _build(tmp_path)
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("sanitizer runtimes not found")
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = sched_build.run_parity_child(lib, tmp_path, env)
    # the report's first lines name the fault and the scheduler's frames
    tail = r.stdout[-1500:] + "\n" + r.stderr[:3000]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr, tail
    assert "runtime error" not in r.stderr, tail


DRIVER = r"""
// Drives the scheduler's C ABI through a synthetic serving trace (prefix
// hits, chunked prefill, preemption under a small pool, forks) and destroys
// it; under the sanitizers any leak, invalid access or undefined operation
// ends the process with a report.
#include <stdint.h>
#include <stdio.h>
#include <vector>
#include "pa_sched.h"

int main() {
  pa_sched_config cfg{};
  cfg.num_blocks = 48;
  cfg.block_size = 16;
  cfg.max_num_batched_tokens = 96;
  cfg.max_num_seqs = 8;
  cfg.max_model_len = 512;
  cfg.long_prefill_token_threshold = 0;
  cfg.enable_chunked_prefill = 1;
  cfg.enable_prefix_caching = 1;
  pa_sched* s = nullptr;
  if (pa_sched_create(&cfg, &s) != 0) return 2;
  const int cap_tok = cfg.max_num_batched_tokens, cap_seq = cfg.max_num_seqs;
  const int stride = (cfg.max_model_len + 15) / 16;
  std::vector<int64_t> ids(cap_seq), pre(cap_seq + 16), fin(cap_seq + 16);
  std::vector<int32_t> qsl(cap_seq + 1), nc(cap_seq), sl(cap_seq), bt(cap_seq * stride),
      tok(cap_tok), cp(2 * cap_seq * stride), sampled(cap_seq);
  uint32_t x = 12345;
  auto rnd = [&]() { x = x * 1664525u + 1013904223u; return x >> 8; };
  int64_t next_id = 0;
  for (int step = 0; step < 400; ++step) {
    if (step < 200 && rnd() % 3 == 0) {
      std::vector<int32_t> prompt(20 + rnd() % 150);
      const int sys_len = (rnd() % 2) ? 48 : 0;  // a shared system prompt
      for (size_t i = 0; i < prompt.size(); ++i)
        prompt[i] = (int)i < sys_len ? 7 + (int)i : (int)(rnd() % 1000);
      if (pa_sched_add_request(s, next_id++, prompt.data(), (int)prompt.size(),
                               1 + rnd() % 40) != 0)
        return 3;
    }
    if (step % 17 == 5 && next_id > 0)
      pa_sched_fork(s, (int64_t)(rnd() % next_id), 1000000 + step, 1 + rnd() % 10);
    pa_sched_step st{};
    st.request_ids = ids.data();
    st.query_start_loc = qsl.data();
    st.num_computed = nc.data();
    st.seq_lens = sl.data();
    st.block_table = bt.data();
    st.token_ids = tok.data();
    st.copy_pairs = cp.data();
    st.preempted_ids = pre.data();
    st.block_table_stride = stride;
    if (pa_sched_schedule(s, &st) != 0) return 4;
    for (int i = 0; i < st.num_seqs; ++i) sampled[i] = (int32_t)(rnd() % 1000);
    int32_t nfin = 0;
    if (pa_sched_update(s, sampled.data(), st.num_seqs, fin.data(), &nfin) != 0) return 5;
  }
  pa_sched_destroy(s);
  printf("driver ok\n");
  return 0;
}
"""


def test_sched_driver_no_leaks(tmp_path):
    src = tmp_path / "driver.cpp"
    src.write_text(DRIVER)
    exe = _build(tmp_path, [str(src)], shared=False)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "driver ok" in r.stdout, r.stdout[-1500:] + r.stderr[:3000]
