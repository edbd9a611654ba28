"""bench.py's mapping from rocprofv3 kernel names (mangled, demangled, or half-demangled
as the profiler prints them) to the library's launch names, which the HBM-counter
ingestion and the roofline lookup rely on.  Host logic only."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


CASES = [
    ("_ZN3kda13kda_bwd_chunkIDF16bDF16bLi128ELi128ELb0ELi0EEEvNS_4ArgsE", "kda_bwd_chunk"),
    ("_ZN3kda13kda_bwd_chunkIDF16bfLi128ELi128ELb1ELi1EEEvNS_4ArgsE", "kda_bwd_chunk_steep"),
    ("_ZN3kda13kda_bwd_chunkIffLi64ELi64ELb0ELi1EEEvNS_4ArgsE", "kda_bwd_chunk"),   # fp32: every chunk-head
    ("_ZN3kda13kda_state_revIDF16bLi128ELi128ELi64ELb0EEEvNS_4ArgsE", "kda_state_bwd_revpass"),
    ("_ZN3kda13kda_state_revIDF16bLi128ELi128ELi64ELb1EEEvNS_4ArgsE", "kda_seg_rev_local"),
    ("void kda::kda_prep8<128, 128, true, false, false, 0>(kda::Args)", "kda_prep_save"),
    ("void kda::kda_prep8<128, 128, true, false, false, 1>(kda::Args)", "kda_prep_steep"),
    ("void kda::kda_prep8<128, 128, false, true, true, 0>(kda::Args)", "kda_prep"),
    ("void kda::kda_state<bool _Accum, bLi128ELi128ELi6 (ELb1), true, 1, 0, true>(kda::Args)", "kda_state_fwd_save"),
    ("void kda::kda_state<bool _Accum, bLi128ELi128ELi6 (ELb0), false, 1, 2, false>(kda::Args)",
     "kda_seg_local_transfer"),
    ("void kda::kda_state<bool _Accum, bLi128ELi128ELi6 (ELb1), false, 1, 0, false>(kda::Args)", "kda_state_fwd"),
    ("void kda::kda_state<bool _Accum, bLi128ELi128ELi6 (ELb0), true, 1, 0, true>(kda::Args)",
     "kda_state_bwd_fwdpass"),
    ("kda::kda_grad_absmax(bool _Accum const*, float const*, unsigned long, float*)", "kda_grad_absmax"),
    ("kda::kda_grad_scale(float const*, int, float*)", "kda_grad_scale"),
    ("void kda::kda_segment_scan<128, 128>(kda::Args)", "kda_seg_scan"),
    ("kda::kda_chunk_map(int const*, int, int, kda::ChunkInfo*, int*, int, int*)", "kda_chunk_map"),
    ("__amd_rocclr_copyBuffer", None),
]


@pytest.mark.parametrize("name,short", CASES)
def test_kernel_names(bench, name, short):
    assert bench._short_name(name) == short


def test_template_argument_parsing(bench):
    half = "void kda::kda_state<bool _Accum, bLi128ELi128ELi6 (ELb1), true, 1, 2, false>(kda::Args)"
    assert bench._bools(half) == [True, True, False]
    assert bench._ints(half) == [128, 128, 1, 2]
    assert bench._bools("_ZN3kda3fooILb0ELb1EEEv") == [False, True]
    assert bench._ints("void kda::kda_prep8<64, 128, true, false, false, 1>(kda::Args)") == [64, 128, 1]
