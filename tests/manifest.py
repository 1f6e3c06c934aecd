"""Determinism manifest: every accumulating entry point of the library, with the
tests that show its deterministic route bit-identical from run to run (under
concurrent load), equal to the CPU oracle bit for bit, and its atomic arm close
to it and varying (so that the replay check could fail). The GDN gate page
(Megatron-LM PR #8244, pre-checks) registers its ordered reduction in such a
manifest; test_manifest.py checks that every entry point declared in
include/detgrad.h is listed and that every listed test exists.

Each entry: the C entry point -> {"cite": page and part, "replay": tests,
"parity": tests, "atomic": tests or None when the call has no atomic arm,
"graph": the test that captures the call into a HIP graph and replays it}.
Tests are "file::function".
"""

MANIFEST = {
    "det_colsum": {
        "cite": "Megatron-LM PR #8244 (GDN gate), description",
        "replay": ["test_gpu_colsum.py::test_replay_under_load_and_atomic_arm"],
        "parity": ["test_gpu_colsum.py::test_train_shape_all_cfgs_with_tail", "test_gpu_colsum.py::test_detmath_bitwise",
                   "test_gpu_detmath_exhaustive.py::test_every_float32_input"],
        "atomic": ["test_gpu_colsum.py::test_replay_under_load_and_atomic_arm"],
        "graph": ["test_gpu_graph.py::test_colsum_and_da"],
    },
    "det_colsum_da": {
        "cite": "Megatron-LM PR #8244 (GDN gate), BF16/FP32 tests; elementwise da of the same gate",
        "replay": ["test_gpu_colsum.py::test_da_output"],
        "parity": ["test_gpu_colsum.py::test_da_output"],
        "atomic": ["test_gpu_colsum.py::test_da_output"],
        "graph": ["test_gpu_graph.py::test_colsum_and_da"],
    },
    "det_colsum_noalloc": {
        "cite": "the callers that cannot allocate (no page)",
        "replay": ["test_zz_no_alloc.py::test_noalloc_matches_the_workspace_call_twice_then_smaller"],
        "parity": ["test_zz_no_alloc.py::test_noalloc_matches_the_workspace_call_twice_then_smaller"],
        "atomic": None,
        "graph": ["test_gpu_graph.py::test_colsum_noalloc"],
    },
    "det_index_add": {
        "cite": "Megatron-LM PR #7441 (DSv4), source 3 and its fix",
        "replay": ["test_gpu_index_add.py::test_replay_under_load_and_atomic_arm"],
        "parity": ["test_gpu_index_add.py::test_parity_small", "test_gpu_index_add.py::test_full_size_parity",
                   "test_gpu_index_add.py::test_f32_sources"],
        "atomic": ["test_gpu_index_add.py::test_replay_under_load_and_atomic_arm"],
        "graph": ["test_gpu_graph.py::test_index_add"],
    },
    "det_indexer_dk": {
        "cite": "Megatron-LM PR #7441 (DSv4), source 3 fix: the clipped-KL indexer gradient",
        "replay": ["test_gpu_indexer_dk.py::test_replay_under_load_and_atomic_arm"],
        "parity": ["test_gpu_indexer_dk.py::test_parity_small", "test_gpu_indexer_dk.py::test_full_size_parity",
                   "test_gpu_indexer_dk.py::test_equals_index_add_of_the_explicit_source_rows"],
        "atomic": ["test_gpu_indexer_dk.py::test_replay_under_load_and_atomic_arm"],
        "graph": ["test_gpu_graph.py::test_indexer_dk"],
    },
    "det_grouped_dprob": {
        "cite": "cudnn-frontend PR #521, first commit (deterministic dprob)",
        "replay": ["test_gpu_dprob.py::test_replay_under_load_and_atomic_arm"],
        "parity": ["test_gpu_dprob.py::test_full_size_parity_and_non_default_stream"],
        "atomic": ["test_gpu_dprob.py::test_replay_under_load_and_atomic_arm"],
        "graph": ["test_gpu_graph.py::test_dprob"],
    },
    "det_grouped_dbias": {
        "cite": "cudnn-frontend PR #521, the commit that extends the flag to dbias",
        "replay": ["test_gpu_dbias.py::test_replay_under_load_and_atomic_arm"],
        "parity": ["test_gpu_dbias.py::test_full_size_parity_and_non_default_stream"],
        "atomic": ["test_gpu_dbias.py::test_replay_under_load_and_atomic_arm"],
        "graph": ["test_gpu_graph.py::test_dbias"],
    },
    "det_grouped_wgrad_acc": {
        "cite": "FlashInfer PR #8602 and #8924 (deterministic accumulate into main_grad)",
        "replay": ["test_gpu_wgrad.py::test_full_size_replay_under_load_and_varying_atomic_arm",
                   "test_gpu_wgrad.py::test_replay_under_load_and_atomic_arm"],
        "parity": ["test_gpu_wgrad.py::test_full_size_default_kernel_bitwise_vs_oracle",
                   "test_gpu_wgrad.py::test_bitwise_vs_oracle", "test_gpu_mfma_model.py::test_single_instructions_match_the_model"],
        "atomic": ["test_gpu_wgrad.py::test_full_size_replay_under_load_and_varying_atomic_arm"],
        "graph": ["test_gpu_graph.py::test_wgrad"],
    },
    "det_grouped_wgrad_acc_bf16": {
        "cite": "FlashInfer PR #8924, Design and numerics (bf16 dW added in bf16)",
        "replay": ["test_gpu_wgrad.py::test_bf16_main_grad_full_size_replay"],
        "parity": ["test_gpu_wgrad.py::test_bf16_main_grad_bitwise_vs_oracle"],
        "atomic": None,
        "graph": ["test_gpu_graph.py::test_wgrad"],
    },
    "det_topk_canonicalize": {
        "cite": "Megatron-LM PR #7441 (DSv4), source 1 and its fix",
        "replay": ["test_gpu_topk.py::test_replay_under_load"],
        "parity": ["test_gpu_topk.py::test_full_size_and_slot_order_invariance", "test_gpu_topk.py::test_parity"],
        "atomic": None,
        "graph": ["test_gpu_graph.py::test_topk"],
    },
}

# declared functions that are sizes, set-up or diagnostics rather than accumulating entry points
NOT_ENTRY_POINTS = {"det_abi_version", "det_last_error", "det_workspace_init", "det_index_add_bad_ids",
                    "det_colsum_select_cfg", "det_detmath_eval", "det_mfma_eval", "det_mfma_rate"}
