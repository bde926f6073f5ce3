"""Plain CPU oracle of the block-diffusion (DFlash) draft head's propose pass.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or call anything in this package. The HIP library
never uses it and shares no code with it.

It is written from three documentation pages, cited by title and section:

* "Struct BlockDiffusionDraftHead" in spark_model::layers::dflash_head
  (atlas-docs), called [Head/atlas] below;
* "Struct BlockDiffusionDraftHead" in metrale_model_arch::dflash_head
  (docs.metrale.ai, a later revision), called [Head/metrale];
* "Trait DraftProposer" in spark_model::speculative (atlas-docs), called
  [DraftProposer].

The pages describe the head's fields and API but print no layer equations, so
the layer internals (RMSNorm, Q/K/V projections, rotate-half RoPE, GQA
attention without a mask, o_proj, SwiGLU MLP) follow the plain textbook forms;
each such reading is stated in the docstring of the function that takes it.

Modules:

* ``numerics`` - bf16 widening and the OCP FP8 E4M3FN codec;
* ``dflash``   - vectorised float64 numpy definition of the whole path;
* ``brute``    - explicit-loop float64 twin for tiny shapes (pins ``dflash``).

Parity status per function is stated in each docstring. The composition of
the whole forward at full geometry is "parity unpinned" beyond the per-step
pins, because the pages print no worked example.
"""
